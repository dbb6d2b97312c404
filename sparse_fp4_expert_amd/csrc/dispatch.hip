// Dispatch (gather routed rows) and combine (router-weighted scatter back to
// token order).  Paper summary page, "D.1 Implementation details": dispatch
// feeds the first expert GEMM and scatter/combine follows the second;
// "D.3 End-to-end serving benchmark": token combination and output layout
// stay outside the expert kernel.  Both kernels are HBM copies: one
// wavefront per row, 16-byte loads and stores, rows assigned round-robin.
#include "common.hpp"

namespace moesq {

constexpr int DISPATCH_THREADS = 256;

// x_routed[r] = x[perm[r] / k]; rows with perm[r] outside [0, M) are zero.
__global__ __launch_bounds__(DISPATCH_THREADS) void permute_kernel(
    const uint4 *__restrict__ x, const int32_t *__restrict__ perm, int M, int k, int K8,
    uint4 *__restrict__ xr) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * DISPATCH_THREADS + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * DISPATCH_THREADS) >> 6;
  for (int r = wave; r < M; r += nwaves) {
    const int src = perm[r];
    const bool ok = src >= 0 && src < M;
    const uint4 *s = x + (size_t)(ok ? src / k : 0) * K8;
    uint4 *d = xr + (size_t)r * K8;
    for (int c = lane; c < K8; c += 64) d[c] = ok ? s[c] : make_uint4(0, 0, 0, 0);
  }
}

// out[t] = bf16(sum_j w[t*k+j] * y[inv_perm[t*k+j]]), fp32 accumulation in j order.
__global__ __launch_bounds__(DISPATCH_THREADS) void combine_kernel(
    const uint4 *__restrict__ y, const int32_t *__restrict__ inv_perm,
    const float *__restrict__ w, int T, int k, int M, int N8, uint4 *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * DISPATCH_THREADS + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * DISPATCH_THREADS) >> 6;
  for (int t = wave; t < T; t += nwaves) {
    for (int c = lane; c < N8; c += 64) {
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int j = 0; j < k; ++j) {
        const int r = inv_perm[t * k + j];
        if (r < 0 || r >= M) continue;
        const float wj = w[t * k + j];
        const uint4 v = y[(size_t)r * N8 + c];
        const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          acc[2 * h] = fmaf(wj, bf16_lo(q[h]), acc[2 * h]);
          acc[2 * h + 1] = fmaf(wj, bf16_hi(q[h]), acc[2 * h + 1]);
        }
      }
      out[(size_t)t * N8 + c] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                           pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    }
  }
}

// out[i] = y[inv_perm[i]] (flat order); invalid entries give zero rows.
__global__ __launch_bounds__(DISPATCH_THREADS) void unpermute_kernel(
    const uint4 *__restrict__ y, const int32_t *__restrict__ inv_perm, int M, int N8,
    uint4 *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * DISPATCH_THREADS + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * DISPATCH_THREADS) >> 6;
  for (int i = wave; i < M; i += nwaves) {
    const int r = inv_perm[i];
    const bool ok = r >= 0 && r < M;
    const uint4 *s = y + (size_t)(ok ? r : 0) * N8;
    uint4 *d = out + (size_t)i * N8;
    for (int c = lane; c < N8; c += 64) d[c] = ok ? s[c] : make_uint4(0, 0, 0, 0);
  }
}

static int rows_grid(long long rows) {
  const long long waves_per_block = DISPATCH_THREADS / 64;
  long long blocks = (rows + waves_per_block - 1) / waves_per_block;
  const long long cap = (long long)device_cu_count() * 32;
  if (blocks > cap) blocks = cap;
  return (int)(blocks < 1 ? 1 : blocks);
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
  hipLaunchKernelGGL(permute_kernel, dim3(rows_grid(M)), dim3(DISPATCH_THREADS), 0, stream,
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
    hipLaunchKernelGGL(combine_kernel, dim3(rows_grid(T)), dim3(DISPATCH_THREADS), 0, stream,
                       (const uint4 *)y, inv_perm, topk_weights, T, k, (int)M, N / 8,
                       (uint4 *)out);
  } else {
    hipLaunchKernelGGL(unpermute_kernel, dim3(rows_grid(M)), dim3(DISPATCH_THREADS), 0, stream,
                       (const uint4 *)y, inv_perm, (int)M, N / 8, (uint4 *)out);
  }
  return launch_status("moesq_unpermute");
}
