"""Structure of the compiled gfx950 kernels (CPU only: compiles to assembly).

Regression guard for a hang: when thread 0's ticket fetch (top of the
persistent task loop) and a thread-0-only store (end of a task) sat in one
lane-divergent region around the loop's back edge, the compiler split the
loop by lane.  Lanes 1..63 then re-ran the task on a stale ticket at the
barrier while lane 0 waited for them outside: an endless loop.  The kernels
now keep every barrier of a task in the same loop as the ticket fetch.
Also checks that no kernel spills vector registers to scratch memory, and
that consumers order their payload loads after their flag loads.
"""

import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "all_reduce_reduction_rank_amd", "csrc", "kernels.hip")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("isa") / "kernels.s"
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-S", "--cuda-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", str(out), SRC]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        pytest.fail(res.stderr)
    return out.read_text()


def _kernels(text):
    return list(re.finditer(r"^(_ZN2ar17collective_kernel\w+):(.*?)^\.Lfunc_end", text, re.S | re.M))


def _colocated_kernels(text):
    return list(re.finditer(r"^(_ZN2ar16colocated_kernel\w+):(.*?)^\.Lfunc_end", text, re.S | re.M))


def _colocated_twoshot_kernels(text):
    return list(re.finditer(r"^(_ZN2ar24colocated_twoshot_kernel\w+):(.*?)^\.Lfunc_end", text, re.S | re.M))


def _colocated_twoshot_ll_kernels(text):
    return list(re.finditer(r"^(_ZN2ar27colocated_twoshot_ll_kernel\w+):(.*?)^\.Lfunc_end", text, re.S | re.M))


def _protocol(name):
    """Protocol of a kernel: collective_kernel<DT, PROTO, KIND>,
    colocated_kernel<DT, PROTO, PASSES>; colocated_twoshot_kernel<DT, PASSES,
    WORDS> is LL128 only."""
    if "colocated_twoshot_kernel" in name:
        return 2
    return int(re.match(r"_ZN2ar\d+\w+?_kernelILi\dELi(\d)E", name).group(1))


def test_every_kernel_compiled(asm):
    # 3 payload types x (3 protocols x 5 schedules + the Simple tree + 1 copy kernel)
    assert len(_kernels(asm)) == 51
    # small one-shots, one workgroup per (tile, rank): 3 payload types x
    # {LL one pass, LL up to 8 passes, LL128 one pass, LL128 up to 2 passes}
    assert len(_colocated_kernels(asm)) == 12
    # small LL128 two-shots: {1, 2 passes} x {fp32, int32, bf16 by words}
    # and bf16 by elements in one pass
    assert len(_colocated_twoshot_kernels(asm)) == 7
    # small LL two-shots: rounds of {4, 8} words a thread x {fp32, int32,
    # bf16 by words, bf16 by halves}
    assert len(_colocated_twoshot_ll_kernels(asm)) == 8


def _label_of(line):
    m = re.match(r"^\.(LBB\w+):", line)
    return m.group(1) if m else None


def test_ticket_fetch_and_barriers_share_one_loop(asm):
    # The fetch must run once per iteration of the loop that holds the first
    # barrier after it: either inside that loop, or in a block that the loop's
    # back edge branches to and that falls through into the loop header (the
    # layout the compiler picks when the first iteration skips the fetch).
    for m in _kernels(asm):
        name, body = m.group(1), m.group(2)
        header = label = None
        fetch_loop = fetch_label = barrier_loop = None
        branches = []  # (loop of the branching block, target label)
        for line in body.split("\n"):
            lab = _label_of(line)
            if lab:
                label = lab
                header = None
            if line.startswith(".LBB") or line.startswith("; %bb"):
                h = re.search(r"Header=BB(\w+) Depth=(\d)", line)
                if h:
                    header = h.groups()
                elif "Loop Header" in line:
                    header = (line.split(":")[0][4:], re.search(r"Depth=(\d)", line).group(1))
                elif line.startswith("; %bb"):
                    header = None
            br = re.search(r"s_(?:c)?branch\w* \.(LBB\w+)$", line)
            if br:
                branches.append((header, br.group(1)))
            if fetch_loop is None and fetch_label is None and \
                    re.search(r"global_atomic_add v\d+, v(?:\d+|\[\d+:\d+\]), v\d+, (?:s\[\d+:\d+\]|off) sc0$", line):
                fetch_loop, fetch_label = header, label
            elif (fetch_loop or fetch_label) and barrier_loop is None and "s_barrier" in line:
                barrier_loop = header
        assert fetch_label is not None or fetch_loop is not None, name
        assert barrier_loop is not None, name
        if fetch_loop is not None:
            assert barrier_loop == fetch_loop, f"{name}: first barrier in loop {barrier_loop}, fetch in {fetch_loop}"
        else:
            assert (barrier_loop, fetch_label) in branches, \
                f"{name}: fetch block {fetch_label} is not re-entered from loop {barrier_loop}"


def _blocks_by_loop(body):
    """Map each line to the innermost loop header of its basic block."""
    header, out = None, []
    for line in body.split("\n"):
        if line.startswith(".LBB"):
            h = re.search(r"Header=BB(\w+) Depth=(\d)", line)
            if h:
                header = h.groups()
            elif "Loop Header" in line:
                header = (line.split(":")[0][4:], re.search(r"Depth=(\d)", line).group(1))
        out.append((header, line))
    return out


def test_flag_raise_stays_in_its_task_loop(asm):
    # A signal (the flag's atomic max) must sit in a loop that also holds a
    # barrier -- the task's own iteration -- not be deferred to an outer
    # loop behind the next ticket fetch.
    seen = 0
    for m in _kernels(asm):
        lines = _blocks_by_loop(m.group(2))
        barrier_loops = {h for h, l in lines if "s_barrier" in l}
        for h, l in lines:
            if "global_atomic_umax_x2" in l:
                seen += 1
                assert h in barrier_loops, f"{m.group(1)}: signal in loop {h} without a barrier"
    assert seen >= 9  # ring, two-shot, one-shot-in-place signals of the Simple kernels


def test_no_spills_to_memory(asm):
    spills = re.findall(r"\.vgpr_spill_count:\s+(\d+)", asm)
    assert spills and all(int(x) == 0 for x in spills)
    assert not re.search(r"^\s+scratch_(load|store)", asm, re.M)


def test_fused_rmsnorm_kernel_keeps_its_row_in_registers(tmp_path):
    out = tmp_path / "rmsnorm.s"
    src = os.path.join(ROOT, "all_reduce_reduction_rank_amd", "csrc", "rmsnorm.hip")
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "-S", "--cuda-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", str(out), src]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    text = out.read_text()
    spills = re.findall(r"\.vgpr_spill_count:\s+(\d+)", text)
    assert len(spills) == 4 and all(int(x) == 0 for x in spills)  # {bf16, fp32} x {one row, rows}
    assert not re.search(r"^\s+scratch_(load|store)", text, re.M)


# ------------------------------------------------------------------ ordering
# A consumer reads a flag with a relaxed device-scope load and then the
# payload the flag publishes with device-scope (sc1) loads; no acquire fence
# sits between them.  That is correct only while every payload load issues
# after the flag value has come back: the producer's payload stores were
# complete device-wide before its flag store, and sc1 loads read the
# coherence point, not a stale cache.  The check: in the Simple and LL128
# kernels, no 16-byte sc1 load (payload) issues while an 8-byte sc1 load (a
# flag; LL128's flag word, Simple's flag array) is still in flight.  Loads
# in flight are tracked in file order and kept across labels and branches,
# which is stricter than any single execution path.  LL needs no such order:
# its flag and payload arrive in one 8-byte load.
_LOAD = re.compile(r"^\s+(?:global|buffer)_load_(\w+)\s")
_WAIT = re.compile(r"s_waitcnt\s.*vmcnt\((\d+)\)")
_SC1 = re.compile(r"\ssc1(?:\s|$)")


def _payload_over_flag(body):
    """(payload loads checked, payload loads issued while a flag load was in flight)."""
    pending, checked, bad = [], 0, []
    for line in body.split("\n"):
        w = _WAIT.search(line)
        if w:
            keep = int(w.group(1))
            pending = pending[len(pending) - keep:] if keep else []
            continue
        m = _LOAD.match(line)
        if m:
            sc1 = _SC1.search(line) is not None
            if m.group(1) == "dwordx4" and sc1:
                checked += 1
                if "flag" in pending:
                    bad.append(line.strip())
            # flags: 8-byte device-scope loads, and the 4-byte ones of the
            # LL128 two-shot's low-half flag polls (buffer loads; control
            # words such as the abort word load through global_load)
            is_flag = sc1 and (m.group(1) == "dwordx2" or (m.group(1) == "dword" and line.lstrip().startswith("buffer_")))
            pending.append("flag" if is_flag else "data")
        elif re.match(r"^\s+(?:global|buffer)_(?:store|atomic)", line):
            pending.append("data")  # stores and atomics count in vmcnt too
    return checked, bad


def test_the_order_check_sees_a_payload_load_over_a_flag():
    flag = "\tglobal_load_dwordx2 v[2:3], v1, s[4:5] sc1"
    data = "\tglobal_load_dword v6, v1, s[8:9]"
    payload = "\tbuffer_load_dwordx4 v[8:11], v1, s[12:15], 0 offen sc1"
    plain = "\tbuffer_load_dwordx4 v[8:11], v1, s[12:15], 0 offen"
    assert _payload_over_flag("\n".join([flag, payload]))[1]
    assert not _payload_over_flag("\n".join([flag, "\ts_waitcnt vmcnt(0)", payload]))[1]
    assert not _payload_over_flag("\n".join([flag, data, "\ts_waitcnt vmcnt(1)", payload]))[1]
    assert _payload_over_flag("\n".join([data, flag, "\ts_waitcnt vmcnt(1)", payload]))[1]
    assert _payload_over_flag("\n".join([flag, ".LBB0_1:", "\ts_cbranch_scc1 .LBB0_2", payload]))[1]
    assert not _payload_over_flag("\n".join([flag, plain]))[1]
    assert _payload_over_flag("\n".join([flag, payload, plain])) == (1, [payload.strip()])
    low = "\tbuffer_load_dword v4, v1, s[16:19], 0 offen offset:120 sc1"
    ctl = "\tglobal_load_dword v5, v1, s[8:9] sc1"
    assert _payload_over_flag("\n".join([low, payload]))[1]
    assert not _payload_over_flag("\n".join([low, "\ts_waitcnt vmcnt(0)", payload]))[1]
    assert not _payload_over_flag("\n".join([ctl, payload]))[1]


def test_payload_loads_wait_for_their_flags(asm):
    checked = 0
    for m in _kernels(asm) + _colocated_kernels(asm) + _colocated_twoshot_kernels(asm):
        name = m.group(1)
        proto = _protocol(name)
        if proto == 1:  # LL
            continue
        n, bad = _payload_over_flag(m.group(2))
        checked += n
        assert not bad, f"{name}: payload loads issued over a flag load: {bad[:3]}"
    # The pattern must keep matching the code: a renamed instruction would
    # otherwise pass vacuously.
    assert checked >= 300, checked
