"""The streaming-ceiling kernels (ar_stream_ceiling) do the work they are
timed for: every destination holds the exclusive or of every source, in
every configuration the bench searches."""

import pytest
import torch

from all_reduce_reduction_rank_amd import stream_ceiling

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("reads,writes", [(1, 1), (2, 1), (3, 2), (8, 1), (0, 2), (1, 0)])
def test_streams_hold_the_xor_of_the_sources(reads, writes):
    g = torch.Generator(device="cuda")
    g.manual_seed(reads * 10 + writes)
    n = (1 << 20) + 16 * 77  # bytes: several grids of vectors and a ragged end
    src = [torch.randint(0, 2 ** 31, (n // 4,), generator=g, device="cuda", dtype=torch.int32) for _ in range(reads)]
    want = torch.zeros(n // 4, dtype=torch.int32, device="cuda")
    for s in src:
        want ^= s
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for nt_l in (False, True):
        for nt_s in (False, True):
            for unroll in (4, 8, 16):
                for per_cu in (1, 0):
                    dst = [torch.full((n // 4,), -1, dtype=torch.int32, device="cuda") for _ in range(writes)]
                    stream_ceiling(src, dst, sink, nt_l, nt_s, unroll, per_cu)
                    torch.cuda.synchronize()
                    for d in dst:
                        if reads:
                            assert torch.equal(d, want), (reads, writes, nt_l, nt_s, unroll, per_cu)
                        else:  # values made from the vector index: every vector written
                            assert not torch.any(d.view(-1, 4)[:, 3] != 1)
    if writes == 0:
        assert int(sink.item()) in (0, 0x9E3779B9 - 2 ** 32)
