// Dispatch (gather routed rows) and combine (router-weighted scatter back to
// token order).  Paper summary page, "D.1 Implementation details": dispatch
// feeds the first expert GEMM and scatter/combine follows the second;
// "D.3 End-to-end serving benchmark": token combination and output layout
// stay outside the expert kernel.  All three kernels are HBM copies with
// 16-byte loads and stores.
#include "common.hpp"

namespace moesq {

constexpr int DISPATCH_THREADS = 256;
// A work unit is one row and a slice of its 16-byte columns: 64 * COPY_UNROLL
// columns for the copies (each lane has COPY_UNROLL loads in flight before
// its first store), 64 for the combine (each lane has up to COMBINE_BATCH
// rows in flight).  Units are assigned round-robin over the wavefronts, so
// that short batches (a few rows) still spread over the chip and every lane
// keeps several loads in flight: one dependent load per lane at a time
// leaves a copy latency-bound well below the HBM rate.
constexpr int COPY_UNROLL = 4;
constexpr int COMBINE_BATCH = 8;

// dst row i = src row row_of(i), or zero where row_of(i) < 0.
template <typename RowOf>
__device__ __forceinline__ void gather_rows(const uint4 *__restrict__ src,
                                            uint4 *__restrict__ dst, int rows, int n16,
                                            RowOf row_of) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * DISPATCH_THREADS + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * DISPATCH_THREADS) >> 6;
  const int S = (n16 + 64 * COPY_UNROLL - 1) / (64 * COPY_UNROLL);
  const long long units = (long long)rows * S;
  for (long long u = wave; u < units; u += nwaves) {
    const int i = (int)(u / S), s = (int)(u - (long long)i * S);
    const int r = row_of(i);
    const uint4 *sp = src + (size_t)(r < 0 ? 0 : r) * n16;
    uint4 v[COPY_UNROLL];
#pragma unroll
    for (int h = 0; h < COPY_UNROLL; ++h) {
      const int c = (s * COPY_UNROLL + h) * 64 + lane;
      v[h] = (r >= 0 && c < n16) ? sp[c] : make_uint4(0, 0, 0, 0);
    }
    uint4 *dp = dst + (size_t)i * n16;
#pragma unroll
    for (int h = 0; h < COPY_UNROLL; ++h) {
      const int c = (s * COPY_UNROLL + h) * 64 + lane;
      if (c < n16) dp[c] = v[h];
    }
  }
}

// x_routed[r] = x[perm[r] / k]; rows with perm[r] outside [0, M) are zero.
__global__ __launch_bounds__(DISPATCH_THREADS) void permute_kernel(
    const uint4 *__restrict__ x, const int32_t *__restrict__ perm, int M, int k, int K8,
    uint4 *__restrict__ xr) {
  gather_rows(x, xr, M, K8, [&](int r) {
    const int src = perm[r];
    return (src >= 0 && src < M) ? src / k : -1;
  });
}

// out[i] = y[inv_perm[i]] (flat order); invalid entries give zero rows.
__global__ __launch_bounds__(DISPATCH_THREADS) void unpermute_kernel(
    const uint4 *__restrict__ y, const int32_t *__restrict__ inv_perm, int M, int N8,
    uint4 *__restrict__ out) {
  gather_rows(y, out, M, N8, [&](int i) {
    const int r = inv_perm[i];
    return (r >= 0 && r < M) ? r : -1;
  });
}

// out[t] = bf16(sum_j w[t*k+j] * y[inv_perm[t*k+j]]), fp32 accumulation in j
// order (rows with inv_perm outside [0, M) are skipped).  The k rows of a
// token are read in batches of COMBINE_BATCH, all loads of a batch issued
// before the first multiply-add.
__global__ __launch_bounds__(DISPATCH_THREADS) void combine_kernel(
    const uint4 *__restrict__ y, const int32_t *__restrict__ inv_perm,
    const float *__restrict__ w, int T, int k, int M, int N8, uint4 *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * DISPATCH_THREADS + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * DISPATCH_THREADS) >> 6;
  const int S = (N8 + 63) >> 6;
  const long long units = (long long)T * S;
  for (long long u = wave; u < units; u += nwaves) {
    const int t = (int)(u / S), s = (int)(u - (long long)t * S);
    const int c = s * 64 + lane;
    const bool cv = c < N8;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int j0 = 0; j0 < k; j0 += COMBINE_BATCH) {
      int r[COMBINE_BATCH];
      float wj[COMBINE_BATCH];
      uint4 v[COMBINE_BATCH];
#pragma unroll
      for (int jj = 0; jj < COMBINE_BATCH; ++jj) {
        const int j = j0 + jj;
        r[jj] = -1;
        wj[jj] = 0.f;
        if (j < k) {
          const int q = inv_perm[(size_t)t * k + j];
          r[jj] = (q >= 0 && q < M) ? q : -1;
          wj[jj] = w[(size_t)t * k + j];
        }
      }
#pragma unroll
      for (int jj = 0; jj < COMBINE_BATCH; ++jj)
        v[jj] = (r[jj] >= 0 && cv) ? y[(size_t)r[jj] * N8 + c] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int jj = 0; jj < COMBINE_BATCH; ++jj) {
        if (r[jj] < 0) continue;
        const uint32_t q[4] = {v[jj].x, v[jj].y, v[jj].z, v[jj].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc[2 * h] = fmaf(wj[jj], bf16_lo(q[h]), acc[2 * h]);
          acc[2 * h + 1] = fmaf(wj[jj], bf16_hi(q[h]), acc[2 * h + 1]);
        }
      }
    }
    if (cv)
      out[(size_t)t * N8 + c] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                           pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  }
}

// Blocks for `units` work units (one wavefront each), capped at 32 blocks
// per CU.
static int units_grid(long long units) {
  const long long waves_per_block = DISPATCH_THREADS / 64;
  long long blocks = (units + waves_per_block - 1) / waves_per_block;
  const long long cap = (long long)device_cu_count() * 32;
  if (blocks > cap) blocks = cap;
  return (int)(blocks < 1 ? 1 : blocks);
}
static long long copy_units(long long rows, int n16) {
  return rows * ((n16 + 64 * COPY_UNROLL - 1) / (64 * COPY_UNROLL));
}

}  // namespace moesq

using namespace moesq;

extern "C" moesq_status_t moesq_permute(const uint16_t *x, const int32_t *perm, int32_t T,
                                        int32_t k, int32_t K, uint16_t *x_routed,
                                        hipStream_t stream) {
  clear_error();
  if (T < 0 || k < 1) return fail(MOESQ_ERR_SHAPE, "moesq_permute: need T >= 0, k >= 1");
  if (K <= 0 || K % 8) return fail(MOESQ_ERR_SHAPE, "moesq_permute: K must be a positive multiple of 8");
  const long long M = (long long)T * k;
  if (M >= (1ll << 31)) return fail(MOESQ_ERR_SHAPE, "moesq_permute: T*k must be < 2^31");
  if (M == 0) return MOESQ_OK;
  if (!x || !perm || !x_routed) return fail(MOESQ_ERR_NULL, "moesq_permute: NULL pointer");
  hipLaunchKernelGGL(permute_kernel, dim3(units_grid(copy_units(M, K / 8))), dim3(DISPATCH_THREADS), 0, stream,
                     (const uint4 *)x, perm, (int)M, k, K / 8, (uint4 *)x_routed);
  return launch_status("moesq_permute");
}

extern "C" moesq_status_t moesq_unpermute(const uint16_t *y, const int32_t *inv_perm,
                                          const float *topk_weights, int32_t T, int32_t k,
                                          int32_t N, uint16_t *out, hipStream_t stream) {
  clear_error();
  if (T < 0 || k < 1) return fail(MOESQ_ERR_SHAPE, "moesq_unpermute: need T >= 0, k >= 1");
  if (N <= 0 || N % 8) return fail(MOESQ_ERR_SHAPE, "moesq_unpermute: N must be a positive multiple of 8");
  const long long M = (long long)T * k;
  if (M >= (1ll << 31)) return fail(MOESQ_ERR_SHAPE, "moesq_unpermute: T*k must be < 2^31");
  if (M == 0) return MOESQ_OK;
  if (!y || !inv_perm || !out) return fail(MOESQ_ERR_NULL, "moesq_unpermute: NULL pointer");
  if (topk_weights) {
    hipLaunchKernelGGL(combine_kernel, dim3(units_grid((long long)T * ((N / 8 + 63) / 64))), dim3(DISPATCH_THREADS), 0, stream,
                       (const uint4 *)y, inv_perm, topk_weights, T, k, (int)M, N / 8,
                       (uint4 *)out);
  } else {
    hipLaunchKernelGGL(unpermute_kernel, dim3(units_grid(copy_units(M, N / 8))), dim3(DISPATCH_THREADS), 0, stream,
                       (const uint4 *)y, inv_perm, (int)M, N / 8, (uint4 *)out);
  }
  return launch_status("moesq_unpermute");
}
