"""Python binding of libar.so: argument marshalling only.

Every step of a collective runs in the library's HIP kernels; PyTorch only
supplies device memory (tensors) and the stream.  The entry points keep the
C names (``include/ar.h``):

    comm = Comm(nranks, max_bytes_per_rank, max_line_bytes_per_rank)
    comm.allreduce(send, recv, algo="ring", proto="simple", chunk_bytes=0)   # or "auto"
    comm.reduce_scatter(send, recv, ...)
    comm.allgather(send, recv, ...)
    plan_bytes(nranks, op, count, dtype, algo, proto, ...)
    select(nranks, op, count, dtype, algo="auto", proto="auto", max_line_bytes_per_rank=0)

``send`` / ``recv`` are lists of N contiguous CUDA (HIP) tensors on the
communicator's device.  If the library is missing it is built once with hipcc;
if that fails every call raises -- there is no CPU fallback.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# AR_LIBRARY points at another build of the same library (measurements only).
LIB_PATH = os.environ.get("AR_LIBRARY") or os.path.join(HERE, "libar.so")

OPS = {"allreduce": 0, "reduce_scatter": 1, "allgather": 2}
ALGOS = {"oneshot": 0, "twoshot": 1, "ring": 2, "tree": 3}
PROTOS = {"simple": 0, "ll": 1, "ll128": 2}
ALGO_AUTO, PROTO_AUTO = 4, 3  # AR_ALGO_AUTO / AR_PROTO_AUTO: the library picks (ar_select)
DTYPES = {"f32": 0, "bf16": 1, "i32": 2}
ESIZE = {"f32": 4, "bf16": 2, "i32": 4}

STATUS = {
    0: "AR_OK", 1: "AR_ERR_INVALID", 2: "AR_ERR_UNSUPPORTED", 3: "AR_ERR_NOMEM",
    4: "AR_ERR_TOO_LARGE", 5: "AR_ERR_HIP", 6: "AR_ERR_TIMEOUT", 7: "AR_ERR_BROKEN",
}

# Every symbol include/ar.h declares.
SYMBOLS = (
    "ar_comm_create", "ar_comm_destroy", "ar_comm_check", "ar_comm_reset",
    "ar_comm_workspace_bytes", "ar_comm_set_max_workgroups", "ar_allreduce", "ar_allreduce_rmsnorm", "ar_reduce_scatter", "ar_allgather",
    "ar_plan_bytes", "ar_select", "ar_debug_inject", "ar_debug_state", "ar_status_string",
    "ar_allreduce_noalloc", "ar_debug_calls", "ar_stream_ceiling",
)


class CallRecord(ctypes.Structure):
    """ar_call_record (include/ar.h)."""
    _fields_ = [("seq", ctypes.c_uint64), ("op", ctypes.c_int32), ("algo", ctypes.c_int32),
                ("proto", ctypes.c_int32), ("dtype", ctypes.c_int32), ("nranks", ctypes.c_int32),
                ("in_place", ctypes.c_int32), ("grid", ctypes.c_uint32), ("batch", ctypes.c_uint32),
                ("counter_free", ctypes.c_uint32), ("by_die", ctypes.c_uint32), ("count", ctypes.c_uint64),
                ("ntasks", ctypes.c_uint64), ("tile_bytes", ctypes.c_uint64)]


class ARError(RuntimeError):
    def __init__(self, status, what=""):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_lib().ar_status_string(status).decode()})")


_LIB = None


def _declare(lib):
    P, S, I, U64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_uint64
    PP = ctypes.POINTER(ctypes.c_void_p)
    lib.ar_comm_create.argtypes = [I, S, S, ctypes.POINTER(P)]
    lib.ar_comm_destroy.argtypes = [P]
    lib.ar_comm_check.argtypes = [P, P, ctypes.POINTER(I), ctypes.POINTER(I)]
    lib.ar_comm_reset.argtypes = [P, P]
    lib.ar_comm_workspace_bytes.argtypes = [P]
    lib.ar_comm_workspace_bytes.restype = S
    lib.ar_comm_set_max_workgroups.argtypes = [P, ctypes.c_uint]
    lib.ar_allreduce_rmsnorm.argtypes = [P, PP, PP, PP, P, S, S, ctypes.c_float, I, P]
    for name in ("ar_allreduce", "ar_reduce_scatter", "ar_allgather"):
        getattr(lib, name).argtypes = [P, PP, PP, S, I, I, I, S, P]
    lib.ar_allreduce_noalloc.argtypes = [I, PP, PP, S, I, I, I, S, P]
    lib.ar_debug_calls.argtypes = [P, ctypes.POINTER(CallRecord), I, ctypes.POINTER(I)]
    lib.ar_stream_ceiling.argtypes = [I, PP, I, PP, S, P, I, I, I, P]
    lib.ar_plan_bytes.argtypes = [I, I, S, I, I, I, S, I, ctypes.POINTER(U64), ctypes.POINTER(U64),
                                  ctypes.POINTER(U64), ctypes.POINTER(U64)]
    lib.ar_select.argtypes = [I, I, S, I, I, I, S, ctypes.POINTER(I), ctypes.POINTER(I),
                              ctypes.POINTER(ctypes.c_double)]
    lib.ar_debug_inject.argtypes = [P, I, I, U64]
    lib.ar_debug_state.argtypes = [P, P, ctypes.POINTER(U64), I]
    lib.ar_status_string.argtypes = [I]
    lib.ar_status_string.restype = ctypes.c_char_p
    for name in SYMBOLS:
        if name not in ("ar_comm_workspace_bytes", "ar_status_string"):
            getattr(lib, name).restype = I
    return lib


def _lib():
    """Load libar.so (building it first if it is not there)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            from .build import build
            build()
        _LIB = _declare(ctypes.CDLL(LIB_PATH))
    return _LIB


def library():
    return _lib()


def _check(status, what):
    if status != 0:
        raise ARError(status, what)


def _algo(name):
    return ALGO_AUTO if name == "auto" else ALGOS[name]


def _proto(name):
    return PROTO_AUTO if name == "auto" else PROTOS[name]


_TORCH = None
_DT_NAMES = None  # torch dtype -> "f32" / "bf16" / "i32"


def _torch():
    global _TORCH, _DT_NAMES
    if _TORCH is None:
        import torch

        _DT_NAMES = {torch.float32: "f32", torch.bfloat16: "bf16", torch.int32: "i32"}
        _TORCH = torch
    return _TORCH


def _dtype_name(t):
    _torch()
    name = _DT_NAMES.get(t.dtype)
    if name is None:
        raise TypeError(f"unsupported tensor dtype {t.dtype}")
    return name


def _ptrs(tensors, nranks, device):
    if len(tensors) != nranks:
        raise ValueError(f"need {nranks} rank buffers, got {len(tensors)}")
    for t in tensors:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("rank buffers must be contiguous device tensors")
        if t.device.index != device:
            raise ValueError("rank buffers must live on the communicator's device")
    return (ctypes.c_void_p * nranks)(*[t.data_ptr() for t in tensors])


def _sizes(tensors, want, what):
    for i, t in enumerate(tensors):
        if t.numel() != want:
            raise ValueError(f"{what}[{i}] holds {t.numel()} elements; the call needs {want}")


def _marshal(tensors, nranks, dtype, want, device):
    """Pointer array of `nranks` rank tensors that all pass the checks keeping
    a kernel inside them (dtype, element count, device, contiguity), in one
    pass of cheap attribute reads; None if any fails (then `_rank_buffers`
    names the failure).  Small calls are bound by this host work."""
    if len(tensors) != nranks:
        return None
    ptrs = []
    for t in tensors:
        if t.dtype is not dtype or t.numel() != want or t.get_device() != device or not t.is_contiguous():
            return None
        ptrs.append(t.data_ptr())
    return (ctypes.c_void_p * nranks)(*ptrs)


def _rank_buffers(send, recv, nranks, device, n_send, n_recv):
    """(dtype name, send pointers, recv pointers) of a call, or the first
    failed check as an exception: dtypes, then element counts, then device
    and layout."""
    dt = _dtype_name(send[0])
    dtype = send[0].dtype
    s = _marshal(send, nranks, dtype, n_send, device)
    r = _marshal(recv, nranks, dtype, n_recv, device)
    if s is not None and r is not None:
        return dt, s, r
    for t in list(send) + list(recv):
        if _dtype_name(t) != dt:
            raise TypeError("all rank buffers must share one dtype")
    _sizes(send, n_send, "send")
    _sizes(recv, n_recv, "recv")
    _ptrs(send, nranks, device)
    _ptrs(recv, nranks, device)
    raise ValueError("rank buffers failed the device check")  # not reached: _ptrs names the failure


def _stream_handle(stream, device=None):
    torch = _torch()
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    if device is not None:  # the raw handle without building a Stream object
        return ctypes.c_void_p(torch._C._cuda_getCurrentRawStream(device))
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


class Comm:
    """N simulated ranks on the current device with a workspace allocated once."""

    def __init__(self, nranks: int, max_bytes_per_rank: int, max_line_bytes_per_rank: int = 0):
        import torch

        self.nranks = nranks
        self.device = torch.cuda.current_device()
        self._h = ctypes.c_void_p()
        _check(_lib().ar_comm_create(nranks, max_bytes_per_rank, max_line_bytes_per_rank,
                                     ctypes.byref(self._h)), "ar_comm_create")

    def close(self):
        if self._h:
            _check(_lib().ar_comm_destroy(self._h), "ar_comm_destroy")
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            if self._h:
                _lib().ar_comm_destroy(self._h)
        except Exception:
            pass

    @property
    def workspace_bytes(self) -> int:
        return _lib().ar_comm_workspace_bytes(self._h)

    def set_max_workgroups(self, max_workgroups: int):
        """Workgroup budget of later calls (0: the default, up to 3 per CU)."""
        _check(_lib().ar_comm_set_max_workgroups(self._h, max_workgroups), "ar_comm_set_max_workgroups")

    def _call(self, name, send, recv, count, algo, proto, chunk_bytes, stream, n_send, n_recv):
        """n_send / n_recv: the elements every send / recv buffer must hold.
        The C ABI sees only pointers, so a shorter tensor would let the kernel
        read or write past it: sizes are checked here, before any launch."""
        dt, s, r = _rank_buffers(send, recv, self.nranks, self.device, n_send, n_recv)
        status = getattr(_lib(), name)(self._h, s, r, count, DTYPES[dt], _algo(algo), _proto(proto),
                                       chunk_bytes, _stream_handle(stream, self.device))
        _check(status, name)

    def allreduce_rmsnorm(self, send, out, weight, eps=1e-6, residual=None, stream=None):
        """out[r] = RMSNorm(sum of send[0..N-1] (+ residual[r])) * weight, row by row.

        send / out / residual: N contiguous [rows, hidden] device tensors
        (residual updated in place, or None); weight: [hidden]."""
        fast = self._rmsnorm_buffers(send, out, weight, residual)
        if fast is not None:  # every check passed in one cheap pass
            dt, rows, hidden, s, o, res = fast
            status = _lib().ar_allreduce_rmsnorm(self._h, s, o, res, ctypes.c_void_p(weight.data_ptr()), rows,
                                                 hidden, float(eps), DTYPES[dt], _stream_handle(stream, self.device))
            _check(status, "ar_allreduce_rmsnorm")
            return out
        dt = _dtype_name(send[0])
        for t in list(send) + list(out) + list(residual or []) + [weight]:
            if _dtype_name(t) != dt:
                raise TypeError("all buffers must share one dtype")
        if send[0].dim() != 2:
            raise ValueError("rank buffers must be [rows, hidden]")
        rows, hidden = send[0].shape
        for what, ts in (("send", send), ("out", out), ("residual", residual or [])):
            for i, t in enumerate(ts):
                if tuple(t.shape) != (rows, hidden):
                    raise ValueError(f"{what}[{i}] has shape {tuple(t.shape)}; the call needs {(rows, hidden)}")
        if weight.numel() != hidden or not weight.is_contiguous() or not weight.is_cuda:
            raise ValueError("weight must be a contiguous device vector of `hidden` elements")
        s, o = _ptrs(send, self.nranks, self.device), _ptrs(out, self.nranks, self.device)
        res = _ptrs(residual, self.nranks, self.device) if residual is not None else None
        status = _lib().ar_allreduce_rmsnorm(self._h, s, o, res, ctypes.c_void_p(weight.data_ptr()), rows, hidden,
                                             float(eps), DTYPES[dt], _stream_handle(stream))
        _check(status, "ar_allreduce_rmsnorm")
        return out

    def _rmsnorm_buffers(self, send, out, weight, residual):
        """(dtype name, rows, hidden, pointer arrays) of a fused call whose
        buffers all pass its checks (one dtype, [rows, hidden] contiguous
        on the communicator's device, weight [hidden]), else None."""
        _torch()
        dt = _DT_NAMES.get(send[0].dtype)
        if dt is None or send[0].dim() != 2:
            return None
        dtype, shape = send[0].dtype, send[0].shape
        rows, hidden = shape
        n, dev = self.nranks, self.device
        ptrs = []
        for ts in (send, out) + ((residual,) if residual is not None else ()):
            if len(ts) != n:
                return None
            p = []
            for t in ts:
                if t.dtype is not dtype or t.shape != shape or t.get_device() != dev or not t.is_contiguous():
                    return None
                p.append(t.data_ptr())
            ptrs.append((ctypes.c_void_p * n)(*p))
        if (weight.dtype is not dtype or weight.numel() != hidden or weight.get_device() != dev
                or not weight.is_contiguous()):
            return None
        return dt, rows, hidden, ptrs[0], ptrs[1], ptrs[2] if residual is not None else None

    def allreduce(self, send, recv=None, algo="ring", proto="simple", chunk_bytes=0, stream=None):
        """recv[r] = sum of send[0..N-1]; recv=None runs in place."""
        recv = send if recv is None else recv
        count = send[0].numel()
        self._call("ar_allreduce", send, recv, count, algo, proto, chunk_bytes, stream, count, count)
        return recv

    def reduce_scatter(self, send, recv, algo="ring", proto="simple", chunk_bytes=0, stream=None):
        """send[i] holds N*recvcount elements; recv[r] receives slice r of the sum."""
        count = recv[0].numel()
        self._call("ar_reduce_scatter", send, recv, count, algo, proto, chunk_bytes, stream, self.nranks * count,
                   count)
        return recv

    def allgather(self, send, recv, algo="ring", proto="simple", chunk_bytes=0, stream=None):
        """recv[r] = send[0] | send[1] | ... | send[N-1]."""
        count = send[0].numel()
        self._call("ar_allgather", send, recv, count, algo, proto, chunk_bytes, stream, count,
                   self.nranks * count)
        return recv

    def check(self, stream=None):
        """Synchronize and return (status name, rank, step) of a latched error."""
        rank, step = ctypes.c_int(-1), ctypes.c_int(-1)
        st = _lib().ar_comm_check(self._h, _stream_handle(stream), ctypes.byref(rank), ctypes.byref(step))
        return STATUS.get(st, st), rank.value, step.value

    def reset(self, stream=None):
        _check(_lib().ar_comm_reset(self._h, _stream_handle(stream)), "ar_comm_reset")

    def debug_state(self, stream=None):
        """Device control block: see ar_debug_state in include/ar.h."""
        out = (ctypes.c_uint64 * 10)()
        _check(_lib().ar_debug_state(self._h, _stream_handle(stream), out, 10), "ar_debug_state")
        keys = ("timeouts", "flag_index", "seen", "awaited", "epoch_then", "tasks_done", "calls", "ticket",
                "done", "abort")
        return dict(zip(keys, list(out)))

    def debug_calls(self, max_calls=16):
        """The communicator's most recent calls (ar_debug_calls), oldest first."""
        recs = (CallRecord * max_calls)()
        n = ctypes.c_int()
        _check(_lib().ar_debug_calls(self._h, recs, max_calls, ctypes.byref(n)), "ar_debug_calls")
        names = ({v: k for k, v in OPS.items()}, {v: k for k, v in ALGOS.items()}, {v: k for k, v in PROTOS.items()},
                 {v: k for k, v in DTYPES.items()})
        out = []
        for r in recs[:n.value]:
            d = {f: getattr(r, f) for f, _ in CallRecord._fields_}
            d["op"], d["algo"], d["proto"], d["dtype"] = (names[0][r.op], names[1][r.algo], names[2][r.proto],
                                                          names[3][r.dtype])
            out.append(d)
        return out

    def inject(self, rank: int, step: int, timeout_us: int = 0):
        _check(_lib().ar_debug_inject(self._h, rank, step, timeout_us), "ar_debug_inject")


def allreduce_noalloc(send, recv=None, algo="ring", proto="simple", chunk_bytes=0, stream=None):
    """ar_allreduce_noalloc: recv[r] = sum of send[0..N-1] with N = len(send),
    on the current device, with no communicator and no device allocation
    (Simple only, at most 1 GiB per rank).  recv=None runs in place."""
    import torch

    recv = send if recv is None else recv
    n = len(send)
    count = send[0].numel()
    dev = torch.cuda.current_device()
    dt, s, r = _rank_buffers(send, recv, n, dev, count, count)
    _check(_lib().ar_allreduce_noalloc(n, s, r, count, DTYPES[dt], _algo(algo), _proto(proto), chunk_bytes,
                                       _stream_handle(stream, dev)), "ar_allreduce_noalloc")
    return recv


def stream_ceiling(src, dst, sink=None, nt_loads=False, nt_stores=False, unroll=8, wg_per_cu=0, stream=None):
    """ar_stream_ceiling: one streaming pass reading every tensor of `src`
    and writing every tensor of `dst` (all contiguous device tensors of the
    same byte size; a measurement aid), plain or non-temporal."""
    tensors = list(src) + list(dst)
    nbytes = tensors[0].numel() * tensors[0].element_size()
    for t in tensors:
        if not t.is_cuda or not t.is_contiguous() or t.numel() * t.element_size() != nbytes:
            raise ValueError("streams must be contiguous device tensors of one byte size")
    s = (ctypes.c_void_p * max(1, len(src)))(*[t.data_ptr() for t in src])
    d = (ctypes.c_void_p * max(1, len(dst)))(*[t.data_ptr() for t in dst])
    _check(_lib().ar_stream_ceiling(len(src), s, len(dst), d, nbytes,
                                    ctypes.c_void_p(sink.data_ptr() if sink is not None else 0),
                                    int(nt_loads) | 2 * int(nt_stores), unroll, wg_per_cu, _stream_handle(stream)),
           "ar_stream_ceiling")


def select(nranks, op, count, dtype, algo="auto", proto="auto", max_line_bytes_per_rank=0):
    """The library's choice for a call: (algo, proto, predicted_us)."""
    a, p, t = ctypes.c_int(), ctypes.c_int(), ctypes.c_double()
    _check(_lib().ar_select(nranks, OPS[op], count, DTYPES[dtype], _algo(algo), _proto(proto),
                            max_line_bytes_per_rank, ctypes.byref(a), ctypes.byref(p), ctypes.byref(t)),
           "ar_select")
    names_a = {v: k for k, v in ALGOS.items()}
    names_p = {v: k for k, v in PROTOS.items()}
    return names_a[a.value], names_p[p.value], t.value


def plan_bytes(nranks, op, count, dtype, algo, proto, chunk_bytes=0, in_place=False):
    """Host-side byte accounting of one call (no GPU needed)."""
    rd, wr, nt = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
    link = (ctypes.c_uint64 * nranks)()
    _check(_lib().ar_plan_bytes(nranks, OPS[op], count, DTYPES[dtype], ALGOS[algo], PROTOS[proto],
                                chunk_bytes, int(in_place), ctypes.byref(rd), ctypes.byref(wr), link,
                                ctypes.byref(nt)), "ar_plan_bytes")
    return {"read": rd.value, "write": wr.value, "hbm": rd.value + wr.value,
            "link": list(link), "ntasks": nt.value}
