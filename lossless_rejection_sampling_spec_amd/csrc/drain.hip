// drain.hip -- the steps after a verify (see include/specverify.h):
//   spec_verify_drain       commit n = a + 1 tokens per OK request into a packed
//                           array and give back the unused verify slots;
//   spec_verify_accounting  the acceptance counters, a per-request moving average
//                           of the acceptance rate and the next lookahead.
// Both are one workgroup of 1,024 threads (a batch holds at most 1,024
// requests), one request per thread: a few kilobytes of reads and writes,
// latency-bound, so the block scan and reductions go through LDS in wave order.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "specverify.h"

namespace svd {

constexpr int NT = 1024;          // threads per workgroup = requests per call at most
constexpr int NW = NT / 64;

// Inclusive sum over the workgroup in thread order (waves by DPP-free shuffles,
// then the wave totals in wave order).
template <typename T>
__device__ __forceinline__ T block_scan_incl(T x, T* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const T y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  T carry = 0;
  for (int i = 0; i < w; ++i) carry += wsum[i];
  return x + carry;
}

// A request's rows [cu0, cu1) inside the token buffer, with k = cu1 - cu0 - 1 >= 0.
__device__ __forceinline__ bool rows_inside(int cu0, int cu1, int total_rows) {
  return cu0 >= 0 && cu0 < cu1 && cu1 <= total_rows;
}

__global__ __launch_bounds__(NT) void k_drain(const int32_t* __restrict__ cu,
                                              const int32_t* __restrict__ accepted,
                                              const int32_t* __restrict__ status,
                                              const int32_t* __restrict__ tokens, int batch,
                                              int total_rows, int32_t* __restrict__ committed,
                                              int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ rollback) {
  __shared__ int wsum[NW];
  const int b = threadIdx.x;
  int n = 0, give = 0, cu0 = 0;
  if (b < batch) {
    cu0 = cu[b];
    const int cu1 = cu[b + 1];
    const int st = status[b];
    if (st != SV_ROW_BAD_K && rows_inside(cu0, cu1, total_rows)) {
      const int k = cu1 - cu0 - 1;
      const int a = accepted[b];
      if (st == SV_ROW_OK && a >= 0 && a <= k) n = a + 1;
      give = k + 1 - n;
    }
  }
  const int incl = block_scan_incl<int>(n, wsum);
  const int off = incl - n;
  if (b < batch) {
    offsets[b] = off;
    rollback[b] = give;
    if (b == batch - 1) offsets[batch] = incl;
    for (int i = 0; i < n; ++i)
      if (off + i < total_rows) committed[off + i] = tokens[cu0 + i];
  }
}

__global__ __launch_bounds__(NT) void k_accounting(const int32_t* __restrict__ cu,
                                                   const int32_t* __restrict__ accepted,
                                                   const int32_t* __restrict__ status, int batch,
                                                   const float* ema_in, float* ema_out, float beta,
                                                   float threshold, int k_low, int k_high,
                                                   int32_t* __restrict__ k_next,
                                                   int64_t* __restrict__ counters) {
  __shared__ long long wsum[NW][4];
  const int b = threadIdx.x;
  long long c[4] = {0, 0, 0, 0};
  if (b < batch) {
    const int k = cu[b + 1] - cu[b] - 1;
    const int a = accepted[b];
    float e = ema_in[b];
    if (status[b] == SV_ROW_OK && k >= 0 && a >= 0 && a <= k) {
      c[0] = a + 1;
      c[1] = k;
      c[2] = a;
      c[3] = 1;
      if (k > 0) {
        // the float32 state's own precision, in this order (no contraction)
        const float r = __fdiv_rn((float)a, (float)k);
        e = __fadd_rn(e, __fmul_rn(beta, __fsub_rn(r, e)));
      }
    }
    ema_out[b] = e;
    k_next[b] = (e < threshold) ? k_low : k_high;
  }
  // counters: wave sums by shuffles, then the waves in order by thread 0
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    long long x = c[f];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x += __shfl_xor(x, d, 64);
    if (lane == 0) wsum[w][f] = x;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      long long t = 0;
      for (int i = 0; i < NW; ++i) t += wsum[i][f];
      counters[f] += t;
    }
  }
}

}  // namespace svd

using namespace svd;

extern "C" {

int spec_verify_drain(const int32_t* cu_seqlens, const int32_t* accepted, const int32_t* status,
                      const int32_t* out_tokens, int batch, int total_rows, int32_t* committed,
                      int32_t* commit_offsets, int32_t* rollback, void* stream) {
  if (!cu_seqlens || !accepted || !status || !out_tokens || !committed || !commit_offsets ||
      !rollback)
    return SV_ERR_NULL;
  if (batch < 1 || batch > NT || total_rows < batch) return SV_ERR_SHAPE;
  hipLaunchKernelGGL(k_drain, dim3(1), dim3(NT), 0, (hipStream_t)stream, cu_seqlens, accepted,
                     status, out_tokens, batch, total_rows, committed, commit_offsets, rollback);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

int spec_verify_accounting(const int32_t* cu_seqlens, const int32_t* accepted,
                           const int32_t* status, int batch, const float* ema_in, float* ema_out,
                           float beta, float threshold, int k_low, int k_high, int32_t* k_next,
                           int64_t* counters, void* stream) {
  if (!cu_seqlens || !accepted || !status || !ema_in || !ema_out || !k_next || !counters)
    return SV_ERR_NULL;
  if (batch < 1 || batch > NT || !(beta >= 0.f && beta <= 1.f) || !(threshold == threshold) ||
      k_low < 0 || k_low > 63 || k_high < 0 || k_high > 63)
    return SV_ERR_SHAPE;
  hipLaunchKernelGGL(k_accounting, dim3(1), dim3(NT), 0, (hipStream_t)stream, cu_seqlens,
                     accepted, status, batch, ema_in, ema_out, beta, threshold, k_low, k_high,
                     k_next, counters);
  return hipGetLastError() == hipSuccess ? SV_OK : SV_ERR_LAUNCH;
}

}  // extern "C"
