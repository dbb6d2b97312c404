// NVFP4 activation quantization for the W4A4 expert GEMM.
//
// Paper summary page, "D.1 Implementation details": the serving integration
// quantizes the activations for the first expert GEMM, in 32-element scale
// blocks; "3.4 Implementation details": weights and quantized activations are
// packed in corresponding scale blocks (here the same 32-position K blocks as
// the weights' E4M3 scales).  Each row is quantized on its own, in fp32 and in
// this order (the second-level scale is one fp32 per row):
//   g     = amax_row / 2688        (2688 = 6 * 448; g = 1 for a zero row)
//   s_b   = E4M3(amax_b / (6 g))   nearest, ties to even, saturating at 448
//   q     = E2M1(x / (E4M3(s_b) g)) nearest, ties to even, saturating at 6
// Layout: codes [T][K/2] (position 2i in the low nibble of byte i), scales
// [T][K/32], row_scale [T].
//
// One wave per row: a first pass finds the row maximum, a second pass
// reloads each 32-position block (the row is still in L2), finds its
// maximum, its scale and its 32 codes.  The kernel is a stream over the
// tokens: 2K bytes read and K/2 + K/32 + 4 written per row.
#include "common.hpp"
#include "encode.hpp"

namespace moesq {

constexpr int AQ_WAVES = 4;
constexpr int AQ_THREADS = AQ_WAVES * 64;

__device__ __forceinline__ float absmax8(uint4 v, float m) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = fmaxf(m, fabsf(bf16_lo(w[i])));
    m = fmaxf(m, fabsf(bf16_hi(w[i])));
  }
  return m;
}

__global__ __launch_bounds__(AQ_THREADS) void act_quant_kernel(const uint4 *__restrict__ x, int T,
                                                               int K, uint4 *__restrict__ codes,
                                                               uint8_t *__restrict__ scales,
                                                               float *__restrict__ row_scale) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * AQ_WAVES + (threadIdx.x >> 6);
  if (row >= T) return;   // the whole wave leaves together
  const int nb = K / 32;
  const uint4 *xr = x + (size_t)row * (size_t)(K / 8);   // four 16-byte units per block
  float amax = 0.0f;
  for (int b = lane; b < nb; b += 64) {
    uint4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = xr[4 * b + i];
#pragma unroll
    for (int i = 0; i < 4; ++i) amax = absmax8(v[i], amax);
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
  const float g = amax > 0.0f ? __fdiv_rn(amax, 2688.0f) : 1.0f;
  const float six_g = 6.0f * g;
  for (int b = lane; b < nb; b += 64) {
    uint4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = xr[4 * b + i];
    float bmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) bmax = absmax8(v[i], bmax);
    const uint32_t sc = e4m3_encode(__fdiv_rn(bmax, six_g));
    const float sg = e4m3_to_f32(sc) * g;
    uint32_t out[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
      uint32_t c = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float lo = bf16_lo(w[j]), hi = bf16_hi(w[j]);
        const uint32_t clo = sg > 0.0f ? e2m1_encode(__fdiv_rn(lo, sg)) : 0u;
        const uint32_t chi = sg > 0.0f ? e2m1_encode(__fdiv_rn(hi, sg)) : 0u;
        c |= (clo | (chi << 4)) << (8 * j);
      }
      out[i] = c;
    }
    codes[(size_t)row * nb + b] = make_uint4(out[0], out[1], out[2], out[3]);
    scales[(size_t)row * nb + b] = (uint8_t)sc;
  }
  if (lane == 0) row_scale[row] = g;
}

}  // namespace moesq

using namespace moesq;

extern "C" moesq_status_t moesq_quantize_activations(const uint16_t *x, int32_t T, int32_t K,
                                                     uint8_t *codes, uint8_t *scales,
                                                     float *row_scale, hipStream_t stream) {
  static const char *who = "moesq_quantize_activations";
  clear_error();
  if (T < 0) return fail(MOESQ_ERR_SHAPE, std::string(who) + ": T must be >= 0");
  if (K < 32 || K % 32) return fail(MOESQ_ERR_SHAPE, std::string(who) + ": K must be a positive multiple of 32");
  if (T == 0) return MOESQ_OK;
  if (!x || !codes || !scales || !row_scale)
    return fail(MOESQ_ERR_NULL, std::string(who) + ": NULL buffer");
  if (((uintptr_t)x | (uintptr_t)codes) & 15)
    return fail(MOESQ_ERR_ARG, std::string(who) + ": x and codes must be 16-byte aligned");
  const unsigned grid = (unsigned)((T + AQ_WAVES - 1) / AQ_WAVES);
  hipLaunchKernelGGL(act_quant_kernel, dim3(grid), dim3(AQ_THREADS), 0, stream,
                     reinterpret_cast<const uint4 *>(x), (int)T, (int)K,
                     reinterpret_cast<uint4 *>(codes), scales, row_scale);
  return launch_status(who);
}
