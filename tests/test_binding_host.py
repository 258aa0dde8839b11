"""Host-side argument checks of the Python binding (no GPU).

The C ABI takes bare device pointers, so a rank tensor shorter than the call
implies would let a kernel read or write past it.  The binding checks every
tensor's element count (and the fused call's shapes) before it builds the
pointer arrays; these tests drive a communicator object that never reached
the device and expect the error before anything else is touched.
"""

import ctypes

import pytest
import torch

from all_reduce_reduction_rank_amd.binding import Comm


def _comm(n):
    c = Comm.__new__(Comm)  # no device: the checks must fire before any library call
    c.nranks, c.device, c._h = n, 0, ctypes.c_void_p()
    return c


def _t(k, dtype=torch.float32):
    return torch.zeros(k, dtype=dtype)


def test_allreduce_needs_equal_counts():
    c = _comm(4)
    send = [_t(100) for _ in range(4)]
    with pytest.raises(ValueError, match="send\\[2\\] holds 99"):
        c.allreduce(send[:2] + [_t(99)] + send[3:], [_t(100) for _ in range(4)])
    with pytest.raises(ValueError, match="recv\\[3\\] holds 50"):
        c.allreduce(send, [_t(100)] * 3 + [_t(50)])


def test_reduce_scatter_send_is_n_times_recv():
    c = _comm(4)
    recv = [_t(10) for _ in range(4)]
    with pytest.raises(ValueError, match="send\\[0\\] holds 39 elements; the call needs 40"):
        c.reduce_scatter([_t(39)] + [_t(40)] * 3, recv)
    with pytest.raises(ValueError, match="recv\\[1\\] holds 9"):
        c.reduce_scatter([_t(40)] * 4, [_t(10), _t(9), _t(10), _t(10)])


def test_allgather_recv_is_n_times_send():
    c = _comm(8)
    with pytest.raises(ValueError, match="recv\\[7\\] holds 79 elements; the call needs 80"):
        c.allgather([_t(10)] * 8, [_t(80)] * 7 + [_t(79)])
    with pytest.raises(ValueError, match="send\\[4\\] holds 11"):
        c.allgather([_t(10)] * 4 + [_t(11)] + [_t(10)] * 3, [_t(80)] * 8)


def test_matching_sizes_reach_the_device_checks():
    # With the right sizes the next check (device tensors) is the one that fires.
    c = _comm(2)
    with pytest.raises(ValueError, match="device tensors"):
        c.allreduce([_t(16), _t(16)], [_t(16), _t(16)])


def test_fused_rmsnorm_shapes():
    c = _comm(2)
    send = [torch.zeros(4, 64) for _ in range(2)]
    w = torch.zeros(64)
    with pytest.raises(ValueError, match="out\\[1\\] has shape \\(4, 32\\)"):
        c.allreduce_rmsnorm(send, [torch.zeros(4, 64), torch.zeros(4, 32)], w)
    with pytest.raises(ValueError, match="residual\\[0\\] has shape \\(256,\\)"):
        c.allreduce_rmsnorm(send, [torch.zeros(4, 64)] * 2, w, residual=[torch.zeros(256), torch.zeros(4, 64)])
    with pytest.raises(ValueError, match="send\\[1\\] has shape \\(3, 64\\)"):
        c.allreduce_rmsnorm([torch.zeros(4, 64), torch.zeros(3, 64)], [torch.zeros(4, 64)] * 2, w)


def test_mixed_dtypes_and_counts_of_buffers_are_refused():
    c = _comm(2)
    with pytest.raises(TypeError, match="share one dtype"):
        c.allreduce([_t(16), _t(16, torch.bfloat16)], [_t(16), _t(16)])
    with pytest.raises(ValueError, match="need 2 rank buffers, got 3"):
        c.allreduce([_t(16)] * 3, [_t(16)] * 3)
    with pytest.raises(TypeError, match="unsupported tensor dtype"):
        c.allreduce([_t(16, torch.float64)] * 2, [_t(16, torch.float64)] * 2)


def test_fast_marshalling_accepts_only_buffers_every_check_passes():
    # _marshal is the per-call fast path; it must refuse whatever the named
    # checks refuse.  CPU tensors report device -1, which stands in for the
    # communicator's device here.
    from all_reduce_reduction_rank_amd.binding import _marshal

    ok = [_t(32) for _ in range(4)]
    arr = _marshal(ok, 4, torch.float32, 32, -1)
    assert [arr[i] for i in range(4)] == [t.data_ptr() for t in ok]
    assert _marshal(ok, 3, torch.float32, 32, -1) is None  # count of buffers
    assert _marshal(ok, 4, torch.bfloat16, 32, -1) is None  # dtype
    assert _marshal(ok, 4, torch.float32, 33, -1) is None  # elements
    assert _marshal(ok, 4, torch.float32, 32, 0) is None  # device
    strided = torch.zeros(64)[::2]
    assert strided.numel() == 32 and not strided.is_contiguous()
    assert _marshal(ok[:3] + [strided], 4, torch.float32, 32, -1) is None  # layout


def test_fused_fast_path_accepts_only_buffers_every_check_passes():
    # The fused call's one-pass check (_rmsnorm_buffers) must refuse what
    # the named checks refuse; CPU tensors (device -1) stand in for device ones.
    c = _comm(2)
    c.device = -1
    send = [torch.zeros(4, 64) for _ in range(2)]
    out = [torch.zeros(4, 64) for _ in range(2)]
    w = torch.zeros(64)
    got = c._rmsnorm_buffers(send, out, w, None)
    assert got is not None and got[:3] == ("f32", 4, 64) and got[5] is None
    assert [got[3][i] for i in range(2)] == [t.data_ptr() for t in send]
    assert c._rmsnorm_buffers(send, [torch.zeros(4, 64), torch.zeros(64, 4)], w, None) is None  # shape
    assert c._rmsnorm_buffers(send, out, torch.zeros(32), None) is None  # weight length
    assert c._rmsnorm_buffers(send, out, w, [torch.zeros(4, 64)]) is None  # residual count
    assert c._rmsnorm_buffers(send, out, w.to(torch.bfloat16), None) is None  # weight dtype
    strided = torch.zeros(64, 4).T
    assert strided.shape == (4, 64) and not strided.is_contiguous()
    assert c._rmsnorm_buffers(send, [strided, out[1]], w, None) is None  # layout
    c.device = 0
    assert c._rmsnorm_buffers(send, out, w, None) is None  # not on the communicator's device
