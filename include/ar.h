/*
 * ar.h -- C ABI of the MI355X all-reduce family library (libar.so).
 *
 * One GPU holds N simulated rank buffers in its HBM.  Each call runs every
 * rank's program of one collective in a single HIP kernel on the caller's
 * stream; rank programs exchange data only through device memory, guarded by
 * flags (Simple) or by flag-carrying lines (LL, LL128).
 *
 * The operations, algorithms and protocols follow these pages:
 *   [Q]  "NCCL collectives, ring all-reduce & launching TP/PP", section
 *        "Direct answer" -- all-reduce sums a tensor every rank holds and every
 *        rank ends with the result; all-gather concatenates the shards;
 *        reduce-scatter sums and each rank keeps its slice; ring all-reduce is
 *        a reduce-scatter followed by an all-gather.
 *   [H]  "Collective communication: NCCL's algorithms and protocols, and
 *        custom all-reduce" -- section "Algorithms" (ring, one-shot,
 *        two-shot), section "Protocols" (LL: 8-byte lines with a 4-byte flag;
 *        LL128: 128-byte lines with an 8-byte flag; Simple: block, fence,
 *        flag), exercise 3 (a pre-registered buffer allocated once caps the
 *        largest message and keeps addresses fixed for graph capture).
 *   [P]  llama.cpp pull request "Add nccl support for tensor parrallel",
 *        overview -- a communicator is created once per group of ranks and
 *        per-tensor collective calls are then made on it.
 *
 * Conventions shared by every entry point:
 *   - Buffers: `sendbufs` / `recvbufs` are HOST arrays of N DEVICE pointers
 *     (N = the communicator's rank count), all on the communicator's device,
 *     each 16-byte aligned.  The arrays are read during the call only; the
 *     caller owns every rank buffer, which must stay alive until the stream
 *     reaches the call.  Element type and count are given per call.
 *   - Streams: `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *     asynchronous and ordered on that stream; a communicator must be used on
 *     one stream at a time (flags are tagged with a device-resident call
 *     counter, so calls and HIP-graph replays never need a reset).
 *   - A call with count 0 does nothing and returns AR_OK (pointers unused).
 *   - Errors: argument errors return at once and launch nothing.  A device
 *     wait that exceeds the communicator's time limit stops the call, latches
 *     AR_ERR_TIMEOUT in device memory and makes later calls no-ops until
 *     ar_comm_reset; ar_comm_check reports it.  The exception: a call that
 *     cannot wait (Simple one-shot out of place, direct reduce-scatter or
 *     all-gather, small enough that one grid covers all its tiles) still
 *     runs in full.  Once ar_comm_check has seen the error, every call
 *     returns AR_ERR_BROKEN until ar_comm_reset.  Nothing is printed unless
 *     the environment variable AR_DEBUG is set (see ar_debug_calls).
 *   - Measurement overrides, read once per process from the environment;
 *     they change how work is cut and ordered, never a result:
 *     AR_TILE_KB (Simple tile), AR_LINE_TILE_KB (LL / LL128 tile payload;
 *     LL128 rounds it down to whole 3840-byte wave passes), AR_BATCH (tickets
 *     per counter fetch, 1..16), AR_WG_PER_CU (resident workgroups per CU a
 *     call's grid may take, 1..16, at most what fits),
 *     AR_LAG (receiver groups behind their senders), AR_RING_WINDOW and
 *     AR_RING_SKEW (ring ticket order), AR_ONESHOT_FOLD_MIB (largest N*S of
 *     a one-shot that loads every term of a pass at once), AR_COLOC_TILE_KB
 *     (largest tile of a Simple two-shot run one workgroup per tile and
 *     rank; 0: never).
 */
#ifndef AR_H
#define AR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AR_OK = 0,
  AR_ERR_INVALID = 1,     /* bad argument: N, pointer, alignment, enum, aliasing */
  AR_ERR_UNSUPPORTED = 2, /* combination not provided */
  AR_ERR_NOMEM = 3,       /* workspace allocation failed */
  AR_ERR_TOO_LARGE = 4,   /* message exceeds the communicator's capacity */
  AR_ERR_HIP = 5,         /* a HIP runtime call failed */
  AR_ERR_TIMEOUT = 6,     /* a rank program waited past the time limit */
  AR_ERR_BROKEN = 7       /* communicator holds a latched device error */
} ar_status;

/* Payload types; the reduction is always SUM ([Q] "Direct answer").
 * AR_F32: IEEE binary32 adds, round to nearest even, no flush to zero.
 * AR_BF16: bf16 storage, each add done in fp32, rounded to bf16 (nearest
 *          even) where the value is stored or put on the wire.
 * AR_I32: two's-complement adds that wrap. */
typedef enum { AR_F32 = 0, AR_BF16 = 1, AR_I32 = 2 } ar_dtype;

/* [H] "Algorithms".  For reduce-scatter and all-gather, ONESHOT and TWOSHOT
 * both name the direct schedule (one exchange: every rank reads its slices
 * straight from every rank).  AR_TREE: the double binary tree, all-reduce
 * with AR_SIMPLE only (other combinations return AR_ERR_UNSUPPORTED): half h
 * of the buffer (the N=2 block split) is reduced up tree h and its sum sent
 * back down; both trees are complete binary trees in heap layout, tree 0
 * holding rank p at position p and tree 1 rank N-1-p; a node adds its own
 * input, then its left and right children's partials, and sends its partial
 * up in the payload type.  AR_ALGO_AUTO: the library picks (ar_select). */
typedef enum { AR_ONESHOT = 0, AR_TWOSHOT = 1, AR_RING = 2, AR_TREE = 3, AR_ALGO_AUTO = 4 } ar_algo;

/* [H] "Protocols".  AR_PROTO_AUTO: the library picks (ar_select). */
typedef enum { AR_SIMPLE = 0, AR_LL = 1, AR_LL128 = 2, AR_PROTO_AUTO = 3 } ar_proto;

typedef enum { AR_OP_ALLREDUCE = 0, AR_OP_REDUCE_SCATTER = 1, AR_OP_ALLGATHER = 2 } ar_op;

typedef struct ar_comm* ar_comm_t;
typedef void* ar_stream_t; /* a hipStream_t */

/* Create a communicator of `nranks` (1..8) simulated ranks on the current HIP
 * device ([P] overview; [H] exercise 3).  It allocates, once, the workspace
 * every later call uses: flags, a device call counter, an error record,
 * staging for ring reduce-scatter partials sized for buffers of up to
 * `max_bytes_per_rank`, and LL and LL128 line staging (one region per
 * protocol, so that no line slot ever holds another protocol's bytes where
 * its flag goes) sized for payloads of up to `max_line_bytes_per_rank` per
 * rank (0: LL / LL128 calls are refused).
 * The per-rank cap applies to the largest buffer of a call: count*esize for
 * all-reduce, nranks*recvcount*esize (input) for reduce-scatter,
 * nranks*sendcount*esize (output) for all-gather.
 * On success *out owns the workspace; release it with ar_comm_destroy.
 * Errors: AR_ERR_INVALID (nranks out of range, out == NULL), AR_ERR_NOMEM,
 * AR_ERR_HIP. */
ar_status ar_comm_create(int nranks, size_t max_bytes_per_rank,
                         size_t max_line_bytes_per_rank, ar_comm_t* out);

/* Free the workspace.  The caller must have synchronized every stream that
 * used the communicator.  Errors: AR_ERR_INVALID (NULL), AR_ERR_HIP. */
ar_status ar_comm_destroy(ar_comm_t comm);

/* Synchronize `stream` and report any latched device error.  On
 * AR_ERR_TIMEOUT, *err_rank / *err_step (either may be NULL) receive the
 * rank program and step of the earliest blocked wait.  Steps: ring -- step s
 * of a block's chain (reduce steps first, run by the receiving rank); two-shot
 * -- 0 = a rank sums its own block, 1 = it gathers the others; one-shot in
 * place -- 0 = a rank has read every input tile, 1 = it writes its output.
 * Returns AR_OK when no error is latched. */
ar_status ar_comm_check(ar_comm_t comm, ar_stream_t stream, int* err_rank, int* err_step);

/* Clear a latched device error so the communicator can be used again
 * (stream-ordered; no buffers are touched: flags are tagged per call). */
ar_status ar_comm_reset(ar_comm_t comm, ar_stream_t stream);

/* Device workspace bytes owned by the communicator. */
size_t ar_comm_workspace_bytes(ar_comm_t comm);

/* All-reduce (SUM) of `count` elements per rank ([Q] "Direct answer";
 * [H] "Algorithms").  recvbufs[r] receives the sum of sendbufs[0..N-1].
 *   ONESHOT: rank r reads all N inputs and sums them in rank order 0..N-1.
 *   TWOSHOT: rank j sums block j of every rank (same order), then every rank
 *            reads the N block sums back.
 *   RING:    N-1 reduce steps then N-1 copy steps; block j's sum starts at
 *            rank j+1 and ends at rank j; bf16 partials are rounded per hop.
 * Blocks: B = ceil(count/N) rounded up to a 16-byte vector; block j holds
 * elements [jB, min((j+1)B, count)).  The ring walks each block in chunks of
 * `chunk_bytes` (0 = 512 KiB; LL128 rounds it down to a multiple of 240
 * bytes), which never changes the result.
 * In place (sendbufs[r] == recvbufs[r] for every r) is allowed; otherwise
 * send and receive buffers must not overlap.
 * Errors: AR_ERR_INVALID, AR_ERR_TOO_LARGE, AR_ERR_BROKEN (latched device
 * error), AR_ERR_HIP (launch failure). */
ar_status ar_allreduce(ar_comm_t comm, const void* const* sendbufs, void* const* recvbufs,
                       size_t count, ar_dtype dtype, ar_algo algo, ar_proto proto,
                       size_t chunk_bytes, ar_stream_t stream);

/* All-reduce with a fused RMSNorm epilogue ([H] "Source code": the fused
 * all-reduce + RMSNorm kernel that follows tensor parallelism's all-reduce).
 * Each rank buffer is a row-major [rows, hidden] matrix of `dtype` (AR_F32
 * or AR_BF16; AR_I32 returns AR_ERR_UNSUPPORTED).  For every rank r, row i:
 *   a = the one-shot all-reduce of row i (ascending rank order, fp32
 *       accumulate, rounded to dtype once: the same bits ar_allreduce gives);
 *   h = a + residualbufs[r][i] in fp32 (h = a when residualbufs is NULL);
 *   residualbufs[r][i] <- h rounded to dtype (in place);
 *   outbufs[r][i] = h * (1 / sqrt(mean(h*h) + eps)) * weight, in fp32,
 *       rounded once to dtype.
 * `weight`: one DEVICE vector of `hidden` dtype elements shared by all ranks.
 * `residualbufs`: NULL, or a HOST array of N DEVICE pointers (rows*hidden
 * each).  hidden*esize must be a multiple of 16 and hidden <= 12288; every
 * pointer 16-byte aligned; outputs and residuals must not overlap any other
 * buffer of the call (out of place only).  rows*hidden*esize must fit the
 * communicator's max_bytes_per_rank.  No device waits: one kernel, each
 * workgroup normalizing one (row, rank) at a time.  rows or hidden 0:
 * AR_OK, nothing done.
 * Errors: AR_ERR_INVALID, AR_ERR_UNSUPPORTED, AR_ERR_TOO_LARGE,
 * AR_ERR_BROKEN, AR_ERR_HIP. */
ar_status ar_allreduce_rmsnorm(ar_comm_t comm, const void* const* sendbufs, void* const* outbufs,
                               void* const* residualbufs, const void* weight, size_t rows, size_t hidden,
                               float eps, ar_dtype dtype, ar_stream_t stream);

/* Reduce-scatter (SUM): sendbufs[i] holds N*recvcount elements; recvbufs[r]
 * (recvcount elements) receives sum_i sendbufs[i][r*recvcount ...]
 * ([Q] "Direct answer").  ONESHOT/TWOSHOT: direct, rank r sums in rank order;
 * RING: the reduce half of the ring (slice j's sum starts at rank j+1, ends
 * at rank j).  Out of place only (AR_ERR_INVALID otherwise). */
ar_status ar_reduce_scatter(ar_comm_t comm, const void* const* sendbufs, void* const* recvbufs,
                            size_t recvcount, ar_dtype dtype, ar_algo algo, ar_proto proto,
                            size_t chunk_bytes, ar_stream_t stream);

/* All-gather: sendbufs[j] holds `sendcount` elements; every recvbufs[r]
 * (N*sendcount elements) receives sendbufs[0] | ... | sendbufs[N-1]
 * ([Q] "Direct answer").  ONESHOT/TWOSHOT: direct; RING: the copy half of
 * the ring.  Out of place only. */
ar_status ar_allgather(ar_comm_t comm, const void* const* sendbufs, void* const* recvbufs,
                       size_t sendcount, ar_dtype dtype, ar_algo algo, ar_proto proto,
                       size_t chunk_bytes, ar_stream_t stream);

/* Workgroup budget of the communicator's calls (NCCL's channel count): each
 * call's kernel runs at most `max_workgroups` workgroups of 256 threads
 * (0, the default: up to 3 per CU, which measured fastest), leaving CUs to
 * kernels running concurrently on other streams ([H] "Protocols", the
 * paragraph on channels: each channel runs as one block, so communication
 * occupies SMs that compute could use; "Common environment variables and
 * debugging": the channel count sets both bandwidth and the SMs used).
 * Any budget is deadlock-free (every ticket is taken by a running
 * workgroup); an in-place one-shot call still gets at least N.  Results do
 * not depend on it.  Takes effect for calls issued afterwards.  Errors:
 * AR_ERR_INVALID (null comm). */
ar_status ar_comm_set_max_workgroups(ar_comm_t comm, unsigned max_workgroups);

/* Host-only choice of algorithm and protocol ([H] "Algorithms": the latency
 * plus bytes-over-bandwidth model, t = alpha + S / beta, decides which
 * algorithm and protocol win at which message size).  alpha and beta are
 * fitted per (operation, N, element size, algorithm, protocol) to a
 * message-size sweep measured on MI355X, separately for calls whose inputs
 * and outputs fit in the 256 MB MALL (2 N S <= 256 MiB) and for larger ones;
 * S = bytes per rank (the larger of a rank's send and receive buffers).
 * Rank counts between the measured ones (2, 4, 8) interpolate linearly.
 * `algo` / `proto` may each be a fixed value (kept) or AUTO (chosen).  LL
 * and LL128 are candidates only when S <= max_line_bytes_per_rank (the
 * communicator's line capacity; 0 = none) and N > 1.  The calls resolve
 * AUTO the same way with their communicator's capacity.  Fills
 * chosen_algo / chosen_proto (required) and predicted_us (may be NULL; a
 * negative value means no fit covered the choice).  `count` has the same
 * meaning as in the call for `op`.  Errors: AR_ERR_INVALID. */
ar_status ar_select(int nranks, ar_op op, size_t count, ar_dtype dtype, ar_algo algo, ar_proto proto,
                    size_t max_line_bytes_per_rank, ar_algo* chosen_algo, ar_proto* chosen_proto,
                    double* predicted_us);

/* Host-only accounting of one call's schedule (no device work; works
 * without a GPU).  `count` has the same meaning as in the call for `op`.
 * Fills (any pointer may be NULL):
 *   hbm_read / hbm_write -- device-memory bytes all N rank programs load /
 *       store (payload and lines; flags excluded), summed over tasks;
 *   link_bytes -- array of nranks: payload bytes each rank receives from its
 *       peers ([H] "Algorithms": ring 2(N-1)/N S, one-shot (N-1) S, two-shot
 *       2(N-1)/N S);
 *   ntasks -- tasks in the call's kernel.
 * Errors: AR_ERR_INVALID. */
ar_status ar_plan_bytes(int nranks, ar_op op, size_t count, ar_dtype dtype, ar_algo algo,
                        ar_proto proto, size_t chunk_bytes, int in_place,
                        uint64_t* hbm_read, uint64_t* hbm_write, uint64_t* link_bytes,
                        uint64_t* ntasks);

/* Test hook: from the next call on, the rank program `rank` withholds what
 * it sends at step `step` -- with Simple the signal after that step, with LL
 * the lines it writes (payload and flag are one 8-byte store), with LL128
 * the flag word of every line it writes -- and waits give up after
 * `timeout_us` microseconds (0 keeps the default of 5 s).  rank = -1 clears
 * the injection.  Steps of the line protocols: ring -- step 0 puts a block on
 * the wire, step s >= 1 receives what step s-1 wrote (the last step writes
 * nothing); two-shot -- 0 a rank sends its slices, 1 an owner sums and
 * publishes its block, 2 a rank receives the sums; one-shot, direct
 * reduce-scatter and all-gather -- 0 sends, 1 receives.  Used to exercise
 * the timeout path from the host. */
ar_status ar_debug_inject(ar_comm_t comm, int rank, int step, uint64_t timeout_us);

/* Test hook: synchronize `stream` and copy up to n (<= 10) words of the
 * communicator's device control block into out: [0] timed-out waits,
 * [1] flag index, [2] value seen and [3] value awaited by the first of them,
 * [4] the call counter then, [5] tasks finished (all calls), [6] calls
 * completed, [7] ticket counter, [8] finished workgroups, [9] abort word.
 * Calls that cannot wait and run without the ticket counter (see Errors
 * above) add to neither [5] nor [6]. */
ar_status ar_debug_state(ar_comm_t comm, ar_stream_t stream, uint64_t* out, int n);

/* The all-reduce of ar_allreduce without a communicator, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It allocates nothing (no hipMalloc,
 * no hipFree, no allocating library routine); its kernels keep their control
 * block and flags in a fixed 8 MiB device array built into the library, one
 * copy per GPU, held until the process ends.
 * Arguments and results are those of ar_allreduce on a communicator of
 * `nranks` ranks (same schedules, same kernels, the same bits), with the
 * current HIP device as the device, these limits:
 *   - proto AR_SIMPLE or AR_PROTO_AUTO (which then picks Simple): AR_LL and
 *     AR_LL128 return AR_ERR_UNSUPPORTED (their line staging grows with the
 *     message);
 *   - count*esize at most 1 GiB per rank (AR_ERR_TOO_LARGE beyond);
 *   - no workgroup budget, no environment overrides.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (on two streams, or a graph replay beside another call) race and must be
 * ordered by the caller.  The first call on a device clears the array (one
 * small kernel on `stream`, ahead of the collective); every call's kernel
 * leaves its counters and error record cleared for the next.  A wait that
 * passes the 5 s limit (which no correct call reaches: one kernel runs every
 * rank program, in an order that cannot deadlock) makes that call give up
 * with its outputs undefined; no later call reports it.
 * Errors (returned at once, nothing launched): AR_ERR_INVALID,
 * AR_ERR_UNSUPPORTED, AR_ERR_TOO_LARGE; AR_ERR_HIP if the device array
 * cannot be reached or a launch fails. */
ar_status ar_allreduce_noalloc(int nranks, const void* const* sendbufs, void* const* recvbufs,
                               size_t count, ar_dtype dtype, ar_algo algo, ar_proto proto,
                               size_t chunk_bytes, ar_stream_t stream);

/* One entry of a communicator's call log (ar_debug_calls): the schedule a
 * call launched, with AUTO choices resolved. */
typedef struct {
  uint64_t seq;          /* 1 for the communicator's first launched call, then 2, 3, ... */
  int32_t op;            /* ar_op */
  int32_t algo, proto;   /* ar_algo, ar_proto (never AUTO) */
  int32_t dtype;         /* ar_dtype */
  int32_t nranks, in_place;
  uint32_t grid;         /* workgroups launched */
  uint32_t batch;        /* tickets a workgroup takes per fetch */
  uint32_t counter_free; /* 1: the call ran without the ticket counter */
  uint32_t by_die;       /* N > 0: the N rank programs reading a tile ran on one die (XCD) */
  uint64_t count;        /* the call's count argument */
  uint64_t ntasks;       /* tasks of the call's kernel */
  uint64_t tile_bytes;   /* payload bytes per task tile */
} ar_call_record;

/* Test and debug hook ([H] "Common environment variables and debugging":
 * the library reports the schedules it built, and a flight recorder keeps
 * the recent collectives so that a hang can be traced to the call a rank
 * missed).  The communicator logs the last 16 calls it launched; this copies
 * the most recent min(max, 16) of them, oldest first, into out and sets
 * *n_out to how many.  With the environment variable AR_DEBUG set, each call
 * also prints its record to stderr when it launches, and ar_comm_check
 * prints the timeout diagnostics and the log when it finds a latched error.
 * Host only, no synchronization.  Errors: AR_ERR_INVALID. */
ar_status ar_debug_calls(ar_comm_t comm, ar_call_record* out, int max, int* n_out);

/* Measurement aid, not a collective: a streaming kernel that reads `nread`
 * (0..8) source buffers and writes `nwrite` (0..2) destination buffers of
 * `bytes` each (a multiple of 16, at most 2 GiB), 16-byte vectors; `flags`
 * bit 0 makes the loads and bit 1 the stores non-temporal (plain
 * otherwise); `unroll` (4, 8 or 16) vectors per thread per source in flight
 * (with more than two sources, about 2*unroll loads per thread in all);
 * `wg_per_cu` caps the workgroups per CU (0: every one that fits).
 * Timed on buffers larger than the 256 MB MALL it gives the practical HBM
 * bandwidth of this GPU for that mix of reads and writes, the ceiling that a
 * collective with the same mix can be held against ([H] "Reading
 * nccl-tests": bus bandwidth is compared with the hardware's own).  Each
 * destination receives the exclusive or of the sources (with no source,
 * values made from the vector index).  `sink`: a device word written only to
 * keep the loads of a read-only run (nwrite 0) alive; NULL otherwise allowed.
 * Errors: AR_ERR_INVALID (counts, alignment, null pointers, flags, unroll),
 * AR_ERR_HIP. */
ar_status ar_stream_ceiling(int nread, const void* const* src, int nwrite, void* const* dst, size_t bytes,
                            void* sink, int flags, int unroll, int wg_per_cu, ar_stream_t stream);

/* Static description of a status code. */
const char* ar_status_string(ar_status status);

#ifdef __cplusplus
}
#endif

#endif /* AR_H */
