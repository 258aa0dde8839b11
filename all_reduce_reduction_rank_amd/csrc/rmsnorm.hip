// rmsnorm.hip -- all-reduce with a fused RMSNorm epilogue (one-shot, Simple).
//
// "Collective communication: NCCL's algorithms and protocols, and custom
// all-reduce", section "Source code", names the fused all-reduce + RMSNorm
// kernel (FlashInfer, integrated by SGLang) as the operation that follows
// tensor parallelism's all-reduce; fusing it saves writing the sum and
// reading it back.  For every rank r and row i of a [rows, hidden] buffer:
//
//   a = sum of row i over the N ranks, ascending rank order, fp32
//       accumulate, rounded to the payload type (the one-shot all-reduce)
//   h = a + residual[r][i]  (fp32 add; h = a without a residual)
//   residual[r][i] <- h rounded to the payload type
//   out[r][i] = h * (1 / sqrt(mean(h^2) + eps)) * weight, rounded once
//
// One workgroup runs one (row, rank) item at a time: the one-shot sum needs
// no flags (every input is ready when the kernel starts), and the row's h
// values wait in registers between the two passes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"
#include "plan.hpp"
#include "rmsnorm.hpp"

namespace ar {

// The E = 16/esize elements of a 16-byte payload vector as floats.
template <int DT>
struct VecF {
  static constexpr int E = DT == DT_BF16 ? 8 : 4;
  float v[E];
  __device__ __forceinline__ static VecF load(const uint4& x) {
    VecF r;
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == DT_BF16) {
        r.v[2 * i] = __uint_as_float(w[i] << 16);
        r.v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      } else {
        r.v[i] = __uint_as_float(w[i]);
      }
    }
    return r;
  }
  __device__ __forceinline__ uint4 store() const {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (DT == DT_BF16) w[i] = bf16_round(v[2 * i]) | (bf16_round(v[2 * i + 1]) << 16);
      else w[i] = __float_as_uint(v[i]);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// EARLY_W: the weights' loads go out with the inputs' (the weights do not
// depend on the sum), so a row costs one round trip to memory, not two.
// Chosen when every workgroup runs one row at most (decode): there latency
// is all.  With several rows per workgroup (prefill) the extra registers and
// loads in flight measured 3 % slower, and at fp32 (twice the vectors per
// row) they would cut residency from 3 to 2 workgroups per CU.
// T: threads per workgroup.  A decode call has only N items (one row per
// rank), so it runs 1024 threads per row: a row of up to 1024 vectors is
// one pass, its loads one round trip.  With 256 threads the same row took
// three passes, each waiting for its own loads.
// The residual is read with the inputs and written back in the output pass,
// so no store sits between the first pass's loads.
template <int DT, bool EARLY_W, int T>
__global__ __launch_bounds__(T) void rmsnorm_kernel(RmsArgs a) {
  constexpr int E = VecF<DT>::E;
  // vectors of a row each thread holds at most: the row's h stays in
  // registers (48 floats per thread at the largest hidden size and T = 256)
  constexpr int VPT = (int)((RMS_MAX_HIDDEN / E + T - 1) / T);
  constexpr uint64_t es = DT == DT_BF16 ? 2 : 4;
  __shared__ float s_part[T / 64];
  const uint64_t nvec = a.hidden / E;
  const uint64_t items = a.rows * (uint64_t)a.nranks;
  const int n = a.nranks;
  // Items (row, rank) = row * N + rank, gridDim.x at a time; by die, the
  // N items of a row (which read the same N input rows) run on one die.
  const uint64_t first = a.by_die ? die_ticket(blockIdx.x, a.by_die) : blockIdx.x;
  for (uint64_t item = first; item < items; item += gridDim.x) {
    const uint64_t row = item / (uint64_t)n;
    const int r = (int)(item % (uint64_t)n);
    const uint64_t base = row * a.hidden * es;
    char* res = a.res[r];
    VecF<DT> h[VPT];
    uint4 wv[EARLY_W ? VPT : 1];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const uint64_t v = threadIdx.x + (uint64_t)i * T;
      if (v < nvec) {
        const uint64_t off = base + v * 16;
        if constexpr (EARLY_W) wv[i] = ld16(a.weight + v * 16);
        // all N loads in flight (and the residual's), then the sum in
        // ascending rank order; the N rank programs of a row re-read the
        // same inputs, so these stay cached
        uint4 x[MAX_RANKS];
#pragma unroll
        for (int j = 0; j < MAX_RANKS; ++j)
          if (j < n) x[j] = ld16(a.in[j] + off);
        const uint4 q = res ? ld16(res + off) : make_uint4(0, 0, 0, 0);
        Vec<DT> acc = Vec<DT>::widen(x[0]);
#pragma unroll
        for (int j = 1; j < MAX_RANKS; ++j)
          if (j < n) acc.add(Vec<DT>::widen(x[j]));
        h[i] = VecF<DT>::load(acc.narrow());  // the all-reduce result, rounded
        if (res) {
          const VecF<DT> qf = VecF<DT>::load(q);
#pragma unroll
          for (int e = 0; e < E; ++e) h[i].v[e] = h[i].v[e] + qf.v[e];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) ss = ss + h[i].v[e] * h[i].v[e];
      }
    }
    // sum of squares over the workgroup: within each wave, then across waves
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = s_part[0];
#pragma unroll
    for (int w = 1; w < T / 64; ++w) tot += s_part[w];
    const float inv = 1.0f / sqrtf(tot / (float)a.hidden + a.eps);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const uint64_t v = threadIdx.x + (uint64_t)i * T;
      if (v < nvec) {
        const VecF<DT> w = VecF<DT>::load(EARLY_W ? wv[EARLY_W ? i : 0] : ld16(a.weight + v * 16));
        if (res) st16(res + base + v * 16, h[i].store());  // residual <- h, rounded
        VecF<DT> o;
#pragma unroll
        for (int e = 0; e < E; ++e) o.v[e] = (h[i].v[e] * inv) * w.v[e];
        st16_hint<true>(a.out[r] + base + v * 16, o.store());
      }
    }
    __syncthreads();  // s_part is reused by the next item
  }
}

hipError_t launch_rmsnorm(const RmsArgs& a, int dtype, int device, hipStream_t stream, uint32_t max_workgroups) {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) cus = 1;
  const uint64_t items = a.rows * (uint64_t)a.nranks;
  uint64_t grid = umin(items, 3ull * (uint64_t)cus);
  if (max_workgroups) grid = umin(grid, (uint64_t)max_workgroups);
  if (grid < 1) grid = 1;
  const bool one_row = items <= grid;
  // Like the one-shot: once the N inputs exceed one die's L2, the N items
  // of a row run on one die, with a grid of whole 8 N blocks so that each
  // stride of gridDim.x items is one permutation of them.
  RmsArgs b = a;
  b.by_die = 0;
  const uint64_t n = (uint64_t)a.nranks, es = dtype == DT_BF16 ? 2 : 4;
  if (!one_row && oneshot_by_die(n, a.rows * a.hidden * es) && grid >= XCDS * n) {
    grid = grid / (XCDS * n) * (XCDS * n);
    b.by_die = (uint32_t)n;
  }
  const dim3 g((unsigned)grid);
  if (dtype == DT_BF16) {
    if (one_row) hipLaunchKernelGGL((rmsnorm_kernel<DT_BF16, true, 1024>), g, dim3(1024), 0, stream, b);
    else hipLaunchKernelGGL((rmsnorm_kernel<DT_BF16, false, WG_THREADS>), g, dim3(WG_THREADS), 0, stream, b);
  } else {
    if (one_row) hipLaunchKernelGGL((rmsnorm_kernel<DT_F32, true, 1024>), g, dim3(1024), 0, stream, b);
    else hipLaunchKernelGGL((rmsnorm_kernel<DT_F32, false, WG_THREADS>), g, dim3(WG_THREADS), 0, stream, b);
  }
  return hipGetLastError();
}

}  // namespace ar
