"""MI355X all-reduce family: one-shot, two-shot and ring all-reduce,
reduce-scatter and all-gather over N simulated rank buffers on one GPU, with
Simple, LL and LL128 transports.  The work runs in hand-written HIP kernels
(libar.so, C ABI in include/ar.h); ``binding`` marshals arguments to it."""

from .binding import (ALGOS, DTYPES, OPS, PROTOS, ARError, Comm, allreduce_noalloc, library,  # noqa: F401
                      plan_bytes, select, stream_ceiling)
