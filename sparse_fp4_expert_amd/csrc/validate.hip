// Debug check of the caller contracts the hot-path kernels rely on without
// checking them: routed ids in range, consistent expert offsets, exactly four
// kept positions per 4:8 group (the format keeps four values of every eight,
// paper summary page, "A Sparse-quantized representation"; for the paired
// layouts, one of the six pair patterns per group), and block scales that
// are non-negative finite E4M3 codes.  Each check counts its violations
// in a small device array; the call synchronises and reports the counts.
#include <string>

#include "common.hpp"

namespace moesq {

enum { V_IDS = 0, V_OFFSETS = 1, V_MASKS = 2, V_SCALES = 3, V_GSCALE = 4, V_COUNT = 5 };

__device__ __forceinline__ void count_add(unsigned long long *cnt, int slot, unsigned long long v) {
  // one atomic per wave
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  if ((threadIdx.x & 63) == 0 && v) atomicAdd(&cnt[slot], v);
}

__global__ void check_ids_kernel(const int32_t *ids, long long n, int E, unsigned long long *cnt) {
  unsigned long long bad = 0;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    bad += (ids[i] < 0 || ids[i] >= E);
  count_add(cnt, V_IDS, bad);
}

// offsets[0] == 0, offsets[e] <= offsets[e+1], offsets[E] == M
__global__ void check_offsets_kernel(const int32_t *off, int E, long long M, unsigned long long *cnt) {
  unsigned long long bad = 0;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e <= E; e += gridDim.x * blockDim.x) {
    if (e == 0) bad += off[0] != 0;
    if (e < E) bad += off[e] > off[e + 1];
    if (e == E) bad += (long long)off[E] != M;
  }
  count_add(cnt, V_OFFSETS, bad);
}

// Every byte of `p` through a per-byte predicate; 16-byte loads where the
// buffer allows them.
template <int SLOT, typename Pred>
__global__ void check_bytes_kernel(const uint8_t *p, long long n, Pred pred, unsigned long long *cnt) {
  unsigned long long bad = 0;
  const long long stride = (long long)gridDim.x * blockDim.x;
  const long long t0 = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  const bool vec = ((reinterpret_cast<uintptr_t>(p) & 15) == 0);
  const long long nv = vec ? n / 16 : 0;
  for (long long i = t0; i < nv; i += stride) {
    const uint4 v = reinterpret_cast<const uint4 *>(p)[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) bad += pred((w[j] >> (8 * b)) & 0xffu);
  }
  for (long long i = nv * 16 + t0; i < n; i += stride) bad += pred(p[i]);
  count_add(cnt, SLOT, bad);
}

struct MaskNotFour {
  __device__ bool operator()(uint32_t m) const { return __builtin_popcount(m) != 4; }
};
// canonical paired: both pattern indices of the byte in [0, 6)
struct PatternBad {
  __device__ bool operator()(uint32_t b) const { return (b & 15u) > 5u || (b >> 4) > 5u; }
};
// paired tiled: both nibbles are window positions i | j << 2 with i < j,
// i.e. one of 4, 8, 9, 12, 13, 14 (bits of 0x7310)
struct WindowBad {
  __device__ bool operator()(uint32_t b) const {
    return !((0x7310u >> (b & 15u)) & 1u) || !((0x7310u >> (b >> 4)) & 1u);
  }
};
// sign bit set, or the NaN code 0x7F
struct ScaleBad {
  __device__ bool operator()(uint32_t s) const { return (s & 0x80u) || s == 0x7fu; }
};

__global__ void check_gscale_kernel(const float *g, int E, unsigned long long *cnt) {
  unsigned long long bad = 0;
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < E; e += gridDim.x * blockDim.x)
    bad += !(__builtin_isfinite(g[e]) && g[e] >= 0.f);
  count_add(cnt, V_GSCALE, bad);
}

static unsigned grid_for(long long n, int threads) {
  long long b = (n + threads - 1) / threads;
  const long long cap = (long long)device_cu_count() * 16;
  if (b > cap) b = cap;
  return (unsigned)(b < 1 ? 1 : b);
}

}  // namespace moesq

using namespace moesq;

extern "C" moesq_status_t moesq_validate(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E,
                                         const int32_t *expert_offsets,
                                         const moesq_weights_t *w, uint64_t *counts,
                                         hipStream_t stream) {
  clear_error();
  if (topk_ids || expert_offsets) {
    if (E < 1 || E > MOESQ_MAX_EXPERTS)
      return fail(MOESQ_ERR_SHAPE, "moesq_validate: E must be in [1, " +
                                       std::to_string(MOESQ_MAX_EXPERTS) + "]");
    if (T < 0 || k < 1) return fail(MOESQ_ERR_SHAPE, "moesq_validate: need T >= 0 and k >= 1");
  }
  if (w) {
    if (w->layout < MOESQ_LAYOUT_CANONICAL || w->layout > MOESQ_LAYOUT_PAIRED_TILED)
      return fail(MOESQ_ERR_LAYOUT, "moesq_validate: unknown weight layout");
    if (w->E < 1 || w->N < 1 || w->K < 32 || w->K % 32)
      return fail(MOESQ_ERR_SHAPE, "moesq_validate: bad weight shape");
    if (!w->masks || !w->scales || !w->global_scale)
      return fail(MOESQ_ERR_NULL, "moesq_validate: NULL weight buffer");
  }
  unsigned long long *cnt = nullptr;
  if (hipMalloc(&cnt, V_COUNT * sizeof(unsigned long long)) != hipSuccess)
    return fail(MOESQ_ERR_HIP, "moesq_validate: hipMalloc of the counters failed");
  unsigned long long host[V_COUNT] = {0};
  moesq_status_t st = MOESQ_OK;
  hipError_t e = hipMemcpyAsync(cnt, host, sizeof host, hipMemcpyHostToDevice, stream);
  const long long M = (long long)T * k;
  if (e == hipSuccess && topk_ids && M > 0)
    hipLaunchKernelGGL(check_ids_kernel, dim3(grid_for(M, 256)), dim3(256), 0, stream, topk_ids, M,
                       E, cnt);
  if (e == hipSuccess && expert_offsets)
    hipLaunchKernelGGL(check_offsets_kernel, dim3(grid_for(E + 1, 256)), dim3(256), 0, stream,
                       expert_offsets, E, M, cnt);
  if (e == hipSuccess && w) {
    const long long groups = (long long)w->E * w->N * (w->K / 8);
    const long long blocks = (long long)w->E * w->N * (w->K / 32);
    if (w->layout == MOESQ_LAYOUT_PAIRED)
      hipLaunchKernelGGL((check_bytes_kernel<V_MASKS, PatternBad>), dim3(grid_for(groups / 32 + 1, 256)),
                         dim3(256), 0, stream, w->masks, groups / 2, PatternBad{}, cnt);
    else if (w->layout == MOESQ_LAYOUT_PAIRED_TILED)
      hipLaunchKernelGGL((check_bytes_kernel<V_MASKS, WindowBad>), dim3(grid_for(groups / 32 + 1, 256)),
                         dim3(256), 0, stream, w->masks, groups / 2, WindowBad{}, cnt);
    else
      hipLaunchKernelGGL((check_bytes_kernel<V_MASKS, MaskNotFour>), dim3(grid_for(groups / 16 + 1, 256)),
                         dim3(256), 0, stream, w->masks, groups, MaskNotFour{}, cnt);
    hipLaunchKernelGGL((check_bytes_kernel<V_SCALES, ScaleBad>), dim3(grid_for(blocks / 16 + 1, 256)),
                       dim3(256), 0, stream, w->scales, blocks, ScaleBad{}, cnt);
    hipLaunchKernelGGL(check_gscale_kernel, dim3(grid_for(w->E, 256)), dim3(256), 0, stream,
                       w->global_scale, w->E, cnt);
  }
  if (e == hipSuccess) e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpyAsync(host, cnt, sizeof host, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  (void)hipFree(cnt);
  if (e != hipSuccess) return fail(MOESQ_ERR_HIP, std::string("moesq_validate: ") + hipGetErrorString(e));
  if (counts)
    for (int i = 0; i < V_COUNT; ++i) counts[i] = host[i];
  static const char *names[V_COUNT] = {"ids outside [0, E)", "offset violations",
                                       "masks or pattern bytes outside the format",
                                       "scale bytes negative or NaN", "non-finite global scales"};
  std::string msg;
  for (int i = 0; i < V_COUNT; ++i)
    if (host[i]) msg += (msg.empty() ? "" : "; ") + std::to_string(host[i]) + " " + names[i];
  if (!msg.empty()) st = fail(MOESQ_ERR_ARG, "moesq_validate: " + msg);
  return st;
}
