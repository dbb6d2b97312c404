// Compression of dense fp32 experts into the 4:8 / E2M1 / E4M3 layout, and a
// decode-to-dense kernel that exercises the GEMM's in-register decoder.
//
// Paper summary page, "3.4 Implementation details": after the scales are
// recomputed, the packer stores the FP4 (E2M1) codes, the sparsity metadata
// and one unsigned E4M3 scale for every block of 32 logical weights.  "A Sparse-quantized representation": 4 of every 8 weights are
// kept, the 16 kept values of a 32-weight block share the scale, and zero is
// on the grid.  The support here is the hard top-4 by magnitude.
//
// Steps (one expert matrix at a time, every decision in fp32):
//   zero      amax[e] = 0
//   amax      amax[e] = max |w| over the expert (atomicMax on the fp32 bits,
//             exact and order-free for non-negative values)
//   finalize  g[e] = amax / 2688 (= 6*448), or 1 when amax == 0
//   quantize  one thread per group of 8; four neighbouring lanes form a
//             32-weight block and share its maximum through lane shuffles
#include "common.hpp"
#include "encode.hpp"

namespace moesq {

constexpr int PACK_THREADS = 256;

__global__ void fill_u32_kernel(uint32_t *p, int n, uint32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

__global__ __launch_bounds__(PACK_THREADS) void amax_kernel(const float4 *__restrict__ dense,
                                                            long long per_expert4,
                                                            uint32_t *amax_bits) {
  const int e = blockIdx.y;
  const float4 *src = dense + (long long)e * per_expert4;
  uint32_t m = 0;
  for (long long i = (long long)blockIdx.x * PACK_THREADS + threadIdx.x; i < per_expert4;
       i += (long long)gridDim.x * PACK_THREADS) {
    const float4 v = src[i];
    m = max(m, __float_as_uint(fabsf(v.x)));
    m = max(m, __float_as_uint(fabsf(v.y)));
    m = max(m, __float_as_uint(fabsf(v.z)));
    m = max(m, __float_as_uint(fabsf(v.w)));
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 64));
  if ((threadIdx.x & 63) == 0 && m) atomicMax(amax_bits + e, m);
}

__global__ void finalize_g_kernel(uint32_t *bits, int E) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= E) return;
  const float amax = __uint_as_float(bits[e]);
  const float g = amax > 0.0f ? __fdiv_rn(amax, 2688.0f) : 1.0f;
  bits[e] = __float_as_uint(g);
}

__global__ __launch_bounds__(PACK_THREADS) void quantize_kernel(
    const float4 *__restrict__ dense, long long total_groups, long long groups_per_expert,
    const float *__restrict__ gscale, uint16_t *__restrict__ values, uint8_t *__restrict__ masks,
    uint8_t *__restrict__ scales) {
  const long long G = (long long)blockIdx.x * PACK_THREADS + threadIdx.x;
  const bool valid = G < total_groups;
  float w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float g = 1.0f;
  if (valid) {
    const float4 lo = dense[2 * G], hi = dense[2 * G + 1];
    w[0] = lo.x; w[1] = lo.y; w[2] = lo.z; w[3] = lo.w;
    w[4] = hi.x; w[5] = hi.y; w[6] = hi.z; w[7] = hi.w;
    g = gscale[G / groups_per_expert];
  }
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = fabsf(w[i]);
  // support: position i is kept iff fewer than 4 positions beat it
  uint32_t mask = 0;
  float gmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int beat = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) beat += (a[j] > a[i]) || (a[j] == a[i] && j < i);
    if (beat < 4) mask |= 1u << i;
    gmax = fmaxf(gmax, a[i]);
  }
  // block maximum over the 4 groups of this 32-weight block
  float bmax = fmaxf(gmax, __shfl_xor(gmax, 1, 64));
  bmax = fmaxf(bmax, __shfl_xor(bmax, 2, 64));
  const float six_g = 6.0f * g;
  const uint32_t sc = e4m3_encode(__fdiv_rn(bmax, six_g));
  const float sg = e4m3_to_f32(sc) * g;
  uint32_t codes = 0;
  int j = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if ((mask >> i) & 1u) {
      const float q = sg > 0.0f ? __fdiv_rn(w[i], sg) : 0.0f;
      codes |= e2m1_encode(q) << (4 * j);
      ++j;
    }
  }
  if (valid) {
    values[G] = (uint16_t)codes;
    masks[G] = (uint8_t)mask;
    if ((G & 3) == 0) scales[G >> 2] = (uint8_t)sc;
  }
}

// Canonical -> tiled: one thread per (expert, 32-row block, 64-position
// segment, row), in tiled order, moving the row's 16 value, 8 mask and 2
// scale bytes of that segment.
__global__ __launch_bounds__(PACK_THREADS) void tile_kernel(
    const uint8_t *__restrict__ sv, const uint8_t *__restrict__ sm, const uint8_t *__restrict__ ss,
    int E, int N, int K, uint8_t *__restrict__ dv, uint8_t *__restrict__ dm,
    uint8_t *__restrict__ ds) {
  const long long t = (long long)blockIdx.x * PACK_THREADS + threadIdx.x;
  const int J = K / 64, NB = N / 32;
  const long long total = (long long)E * NB * J * 32;
  if (t >= total) return;
  const int r = (int)(t & 31);
  const long long u = t >> 5;                 // (e*NB + b)*J + j
  const int j = (int)(u % J);
  const long long eb = u / J;                 // e*NB + b
  const long long row = (eb / NB) * N + (eb % NB) * 32 + r;   // e*N + n
  const uint4 v = *reinterpret_cast<const uint4 *>(sv + row * (K / 4) + j * 16);
  const uint2 m = *reinterpret_cast<const uint2 *>(sm + row * (K / 8) + j * 8);
  const uint16_t s = *reinterpret_cast<const uint16_t *>(ss + row * (K / 32) + j * 2);
  *reinterpret_cast<uint4 *>(dv + t * 16) = v;
  *reinterpret_cast<uint2 *>(dm + t * 8) = m;
  *reinterpret_cast<uint16_t *>(ds + t * 2) = s;
}

// dense[n][8g .. 8g+8) = decoded group g of row n of one expert (bf16, no
// global scale), from either layout.
__global__ __launch_bounds__(PACK_THREADS) void decode_kernel(
    const uint8_t *__restrict__ values, const uint8_t *__restrict__ masks,
    const uint8_t *__restrict__ scales, int N, int K, int tiled, uint4 *__restrict__ dense) {
  __shared__ uint4 lut[256];
  build_group_lut(lut);
  __syncthreads();
  const long long G = (long long)blockIdx.x * PACK_THREADS + threadIdx.x;
  const long long groups = (long long)N * K / 8;
  if (G >= groups) return;
  long long vo, mo, so;
  if (tiled) {
    const int n = (int)(G / (K / 8)), g = (int)(G % (K / 8));
    const long long seg = ((long long)(n / 32) * (K / 64) + g / 8) * 32 + (n % 32);
    vo = seg * 16 + (g % 8) * 2;
    mo = seg * 8 + (g % 8);
    so = seg * 2 + (g % 8) / 4;
  } else {
    vo = G * 2;
    mo = G;
    so = G >> 2;
  }
  const uint32_t v = *reinterpret_cast<const uint16_t *>(values + vo);
  // the GEMM's scale conversion (hardware OCP E4M3), so both agree on any byte
  const float s = __builtin_amdgcn_cvt_f32_fp8(scales[so], 0);
  dense[G] = decode_group<0>(masks[mo], v, s, lut);
}

// ---- paired 4:8 ("Blackwell paired 4:8 NVFP4": two of the four position
// pairs (2i, 2i+1) of a group are kept).  The pair sums decide in fp32; pair
// i is kept iff fewer than two pairs beat it (a larger sum, or an equal sum
// at a lower index), which always keeps exactly two.  Returns the keep-mask
// and the pattern index of the kept couple (lexicographic numbering).
__device__ __forceinline__ uint32_t paired_pick(const float (&a)[8], uint32_t &pidx) {
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = a[2 * i] + a[2 * i + 1];
  uint32_t kept = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int beat = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) beat += (s[j] > s[i]) || (s[j] == s[i] && j < i);
    if (beat < 2) kept |= 1u << i;
  }
  const uint32_t i0 = __builtin_ctz(kept), i1 = 31u - __builtin_clz(kept);
  pidx = i0 == 0 ? i1 - 1 : (i0 == 1 ? i1 + 1 : 5u);
  return (3u << (2 * i0)) | (3u << (2 * i1));
}

// Largest kept |w| of each expert (the paired support can drop the largest
// weight of a group, so the plain maximum is not the one the scales use).
__global__ __launch_bounds__(PACK_THREADS) void amax_paired_kernel(const float4 *__restrict__ dense,
                                                                   long long groups_per_expert,
                                                                   uint32_t *amax_bits) {
  const int e = blockIdx.y;
  const float4 *src = dense + (long long)e * groups_per_expert * 2;
  uint32_t m = 0;
  for (long long i = (long long)blockIdx.x * PACK_THREADS + threadIdx.x; i < groups_per_expert;
       i += (long long)gridDim.x * PACK_THREADS) {
    const float4 lo = src[2 * i], hi = src[2 * i + 1];
    const float a[8] = {fabsf(lo.x), fabsf(lo.y), fabsf(lo.z), fabsf(lo.w),
                        fabsf(hi.x), fabsf(hi.y), fabsf(hi.z), fabsf(hi.w)};
    uint32_t p;
    const uint32_t mask = paired_pick(a, p);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((mask >> j) & 1u) m = max(m, __float_as_uint(a[j]));
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, d, 64));
  if ((threadIdx.x & 63) == 0 && m) atomicMax(amax_bits + e, m);
}

// One thread per group, as quantize_kernel; neighbouring lanes (groups 2u,
// 2u+1) combine their pattern indices into one byte.
__global__ __launch_bounds__(PACK_THREADS) void quantize_paired_kernel(
    const float4 *__restrict__ dense, long long total_groups, long long groups_per_expert,
    const float *__restrict__ gscale, uint16_t *__restrict__ values, uint8_t *__restrict__ patterns,
    uint8_t *__restrict__ scales) {
  const long long G = (long long)blockIdx.x * PACK_THREADS + threadIdx.x;
  const bool valid = G < total_groups;
  float w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  float g = 1.0f;
  if (valid) {
    const float4 lo = dense[2 * G], hi = dense[2 * G + 1];
    w[0] = lo.x; w[1] = lo.y; w[2] = lo.z; w[3] = lo.w;
    w[4] = hi.x; w[5] = hi.y; w[6] = hi.z; w[7] = hi.w;
    g = gscale[G / groups_per_expert];
  }
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = fabsf(w[i]);
  uint32_t pidx;
  const uint32_t mask = paired_pick(a, pidx);
  float gmax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if ((mask >> i) & 1u) gmax = fmaxf(gmax, a[i]);
  float bmax = fmaxf(gmax, __shfl_xor(gmax, 1, 64));
  bmax = fmaxf(bmax, __shfl_xor(bmax, 2, 64));
  const float six_g = 6.0f * g;
  const uint32_t sc = e4m3_encode(__fdiv_rn(bmax, six_g));
  const float sg = e4m3_to_f32(sc) * g;
  uint32_t codes = 0;
  int j = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if ((mask >> i) & 1u) {
      const float q = sg > 0.0f ? __fdiv_rn(w[i], sg) : 0.0f;
      codes |= e2m1_encode(q) << (4 * j);
      ++j;
    }
  }
  const uint32_t p_odd = (uint32_t)__shfl_xor((int)pidx, 1, 64);
  if (valid) {
    values[G] = (uint16_t)codes;
    if ((G & 1) == 0) patterns[G >> 1] = (uint8_t)(pidx | (p_odd << 4));
    if ((G & 3) == 0) scales[G >> 2] = (uint8_t)sc;
  }
}

// A unit (groups 2u, 2u+1) of the canonical paired layout -- its four value
// bytes and its pattern byte -- in the window order of the tiled layout:
// codes G v0, G v2, G' v0, G' v2, G v1, G v3, G' v1, G' v3 and window
// positions w(G) | w(G') << 4.
__device__ __forceinline__ void paired_unit_from_canonical(uint32_t v4, uint32_t pbyte,
                                                           uint32_t &vu, uint32_t &wu) {
  const uint32_t g0 = v4 & 0xffu, g1 = (v4 >> 8) & 0xffu, h0 = (v4 >> 16) & 0xffu, h1 = v4 >> 24;
  vu = (g0 & 15u) | (g1 & 15u) << 4 | (h0 & 15u) << 8 | (h1 & 15u) << 12 | (g0 >> 4) << 16 |
       (g1 >> 4) << 20 | (h0 >> 4) << 24 | (h1 >> 4) << 28;
  wu = paired_window_index(pbyte & 15u) | paired_window_index(pbyte >> 4) << 4;
}

// Canonical paired -> paired tiled, one thread per (expert, 32-row block,
// segment, row) as tile_kernel.
__global__ __launch_bounds__(PACK_THREADS) void tile_paired_kernel(
    const uint8_t *__restrict__ sv, const uint8_t *__restrict__ sp, const uint8_t *__restrict__ ss,
    int E, int N, int K, uint8_t *__restrict__ dv, uint8_t *__restrict__ dp,
    uint8_t *__restrict__ ds) {
  const long long t = (long long)blockIdx.x * PACK_THREADS + threadIdx.x;
  const int J = K / 64, NB = N / 32;
  const long long total = (long long)E * NB * J * 32;
  if (t >= total) return;
  const int r = (int)(t & 31);
  const long long u = t >> 5;
  const int j = (int)(u % J);
  const long long eb = u / J;
  const long long row = (eb / NB) * N + (eb % NB) * 32 + r;
  const uint4 v = *reinterpret_cast<const uint4 *>(sv + row * (K / 4) + j * 16);
  const uint32_t p = *reinterpret_cast<const uint32_t *>(sp + row * (K / 16) + j * 4);
  const uint16_t s = *reinterpret_cast<const uint16_t *>(ss + row * (K / 32) + j * 2);
  const uint32_t vin[4] = {v.x, v.y, v.z, v.w};
  uint32_t vo[4], wo = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t wu;
    paired_unit_from_canonical(vin[k], (p >> (8 * k)) & 0xffu, vo[k], wu);
    wo |= wu << (8 * k);
  }
  *reinterpret_cast<uint4 *>(dv + t * 16) = make_uint4(vo[0], vo[1], vo[2], vo[3]);
  *reinterpret_cast<uint32_t *>(dp + t * 4) = wo;
  *reinterpret_cast<uint16_t *>(ds + t * 2) = s;
}

// dense[n][16u .. 16u+16) = decoded unit u of row n of one paired expert
// (bf16, no global scale), from either paired layout, through the GEMM's
// unit decoder; the slots are then placed at their positions.
__global__ __launch_bounds__(PACK_THREADS) void decode_paired_kernel(
    const uint8_t *__restrict__ values, const uint8_t *__restrict__ patterns,
    const uint8_t *__restrict__ scales, int N, int K, int tiled, uint4 *__restrict__ dense) {
  const long long U = (long long)blockIdx.x * PACK_THREADS + threadIdx.x;
  const long long units = (long long)N * K / 16;
  if (U >= units) return;
  uint32_t vu, wu, sb;
  if (tiled) {
    const int n = (int)(U / (K / 16)), uu = (int)(U % (K / 16));
    const long long seg = ((long long)(n / 32) * (K / 64) + uu / 4) * 32 + (n % 32);
    vu = *reinterpret_cast<const uint32_t *>(values + seg * 16 + (uu % 4) * 4);
    wu = patterns[seg * 4 + (uu % 4)];
    sb = scales[seg * 2 + (uu % 4) / 2];
  } else {
    paired_unit_from_canonical(*reinterpret_cast<const uint32_t *>(values + U * 4), patterns[U], vu,
                               wu);
    sb = scales[U >> 1];
  }
  const uint4 d = decode_paired_unit(vu, __builtin_amdgcn_cvt_f32_fp8(sb, 0));
  const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
  auto slot = [&](int i) { return (dw[i >> 1] >> (16 * (i & 1))) & 0xffffu; };
  uint32_t out[8] = {0, 0, 0, 0, 0, 0, 0, 0};     // 16 bf16, two per dword
  auto put = [&](int pos, uint32_t b) { out[pos >> 1] |= b << (16 * (pos & 1)); };
#pragma unroll
  for (int h = 0; h < 2; ++h) {                  // G (h = 0) and G' (h = 1)
    const uint32_t w = (wu >> (4 * h)) & 15u, i = w & 3u, j = w >> 2;
    const int base = 8 * h;
    put(base + 2 * i, slot(2 * h));              // v0
    put(base + 2 * j, slot(2 * h + 1));          // v2
    put(base + 2 * i + 1, slot(4 + 2 * h));      // v1
    put(base + 2 * j + 1, slot(4 + 2 * h + 1));  // v3
  }
  dense[2 * U] = make_uint4(out[0], out[1], out[2], out[3]);
  dense[2 * U + 1] = make_uint4(out[4], out[5], out[6], out[7]);
}

}  // namespace moesq

using namespace moesq;

extern "C" moesq_status_t moesq_pack_weights(const float *dense, int32_t E, int32_t N, int32_t K,
                                             uint8_t *values, uint8_t *masks, uint8_t *scales,
                                             float *global_scale, hipStream_t stream) {
  clear_error();
  if (E < 1 || E > 65535 || N < 1 || K < 32 || K % 32)
    return fail(MOESQ_ERR_SHAPE,
                "moesq_pack_weights: need 1 <= E <= 65535, N >= 1, K a positive multiple of 32");
  if (!dense || !values || !masks || !scales || !global_scale)
    return fail(MOESQ_ERR_NULL, "moesq_pack_weights: NULL pointer");
  const long long per_expert = (long long)N * K;
  uint32_t *bits = reinterpret_cast<uint32_t *>(global_scale);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((E + 255) / 256), dim3(256), 0, stream, bits, E, 0u);
  long long bx = (per_expert / 4 + PACK_THREADS * 16 - 1) / (PACK_THREADS * 16);
  if (bx > 1024) bx = 1024;
  hipLaunchKernelGGL(amax_kernel, dim3((unsigned)bx, E), dim3(PACK_THREADS), 0, stream,
                     (const float4 *)dense, per_expert / 4, bits);
  hipLaunchKernelGGL(finalize_g_kernel, dim3((E + 255) / 256), dim3(256), 0, stream, bits, E);
  const long long groups = (long long)E * per_expert / 8;
  const long long blocks = (groups + PACK_THREADS - 1) / PACK_THREADS;
  if (blocks >= (1ll << 31)) return fail(MOESQ_ERR_SHAPE, "moesq_pack_weights: too many groups");
  hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)blocks), dim3(PACK_THREADS), 0, stream,
                     (const float4 *)dense, groups, per_expert / 8, global_scale,
                     (uint16_t *)values, masks, scales);
  return launch_status("moesq_pack_weights");
}

extern "C" moesq_status_t moesq_pack_weights_paired(const float *dense, int32_t E, int32_t N,
                                                    int32_t K, uint8_t *values, uint8_t *patterns,
                                                    uint8_t *scales, float *global_scale,
                                                    hipStream_t stream) {
  clear_error();
  if (E < 1 || E > 65535 || N < 1 || K < 32 || K % 32)
    return fail(MOESQ_ERR_SHAPE,
                "moesq_pack_weights_paired: need 1 <= E <= 65535, N >= 1, K a positive multiple of 32");
  if (!dense || !values || !patterns || !scales || !global_scale)
    return fail(MOESQ_ERR_NULL, "moesq_pack_weights_paired: NULL pointer");
  const long long per_expert = (long long)N * K;
  uint32_t *bits = reinterpret_cast<uint32_t *>(global_scale);
  hipLaunchKernelGGL(fill_u32_kernel, dim3((E + 255) / 256), dim3(256), 0, stream, bits, E, 0u);
  long long bx = (per_expert / 8 + PACK_THREADS * 8 - 1) / (PACK_THREADS * 8);
  if (bx > 1024) bx = 1024;
  hipLaunchKernelGGL(amax_paired_kernel, dim3((unsigned)bx, E), dim3(PACK_THREADS), 0, stream,
                     (const float4 *)dense, per_expert / 8, bits);
  hipLaunchKernelGGL(finalize_g_kernel, dim3((E + 255) / 256), dim3(256), 0, stream, bits, E);
  const long long groups = (long long)E * per_expert / 8;
  const long long blocks = (groups + PACK_THREADS - 1) / PACK_THREADS;
  if (blocks >= (1ll << 31))
    return fail(MOESQ_ERR_SHAPE, "moesq_pack_weights_paired: too many groups");
  hipLaunchKernelGGL(quantize_paired_kernel, dim3((unsigned)blocks), dim3(PACK_THREADS), 0, stream,
                     (const float4 *)dense, groups, per_expert / 8, global_scale,
                     (uint16_t *)values, patterns, scales);
  return launch_status("moesq_pack_weights_paired");
}

extern "C" moesq_status_t moesq_tile_weights(const moesq_weights_t *src, uint8_t *values,
                                             uint8_t *masks, uint8_t *scales, hipStream_t stream) {
  clear_error();
  if (!src || !values || !masks || !scales)
    return fail(MOESQ_ERR_NULL, "moesq_tile_weights: NULL pointer");
  if (src->layout != MOESQ_LAYOUT_CANONICAL && src->layout != MOESQ_LAYOUT_PAIRED)
    return fail(MOESQ_ERR_LAYOUT, "moesq_tile_weights: source must be canonical or paired");
  if (!src->values || !src->masks || !src->scales)
    return fail(MOESQ_ERR_NULL, "moesq_tile_weights: NULL weight buffer");
  if (src->E < 1 || src->N < 32 || src->N % 32 || src->K < 64 || src->K % 64)
    return fail(MOESQ_ERR_SHAPE, "moesq_tile_weights: need E >= 1, N % 32 == 0, K % 64 == 0");
  const long long total = (long long)src->E * (src->N / 32) * (src->K / 64) * 32;
  const long long blocks = (total + PACK_THREADS - 1) / PACK_THREADS;
  if (blocks >= (1ll << 31)) return fail(MOESQ_ERR_SHAPE, "moesq_tile_weights: too large");
  if (src->layout == MOESQ_LAYOUT_PAIRED)
    hipLaunchKernelGGL(tile_paired_kernel, dim3((unsigned)blocks), dim3(PACK_THREADS), 0, stream,
                       src->values, src->masks, src->scales, src->E, src->N, src->K, values, masks,
                       scales);
  else
    hipLaunchKernelGGL(tile_kernel, dim3((unsigned)blocks), dim3(PACK_THREADS), 0, stream,
                       src->values, src->masks, src->scales, src->E, src->N, src->K, values, masks,
                       scales);
  return launch_status("moesq_tile_weights");
}

extern "C" moesq_status_t moesq_decode_weights(const moesq_weights_t *w, int32_t expert,
                                               uint16_t *dense, hipStream_t stream) {
  clear_error();
  if (!w || !dense) return fail(MOESQ_ERR_NULL, "moesq_decode_weights: NULL pointer");
  if (w->layout < MOESQ_LAYOUT_CANONICAL || w->layout > MOESQ_LAYOUT_PAIRED_TILED)
    return fail(MOESQ_ERR_LAYOUT, "moesq_decode_weights: unknown layout");
  if (!w->values || !w->masks || !w->scales)
    return fail(MOESQ_ERR_NULL, "moesq_decode_weights: NULL weight buffer");
  if (w->E < 1 || w->N < 1 || w->K < 32 || w->K % 32)
    return fail(MOESQ_ERR_SHAPE, "moesq_decode_weights: bad E/N/K");
  const bool tiled = w->layout == MOESQ_LAYOUT_TILED || w->layout == MOESQ_LAYOUT_PAIRED_TILED;
  if (tiled && (w->N % 32 || w->K % 64))
    return fail(MOESQ_ERR_SHAPE, "moesq_decode_weights: tiled layout needs N % 32 == 0, K % 64 == 0");
  if (expert < 0 || expert >= w->E)
    return fail(MOESQ_ERR_ARG, "moesq_decode_weights: expert out of range");
  const long long groups = (long long)w->N * w->K / 8;
  const long long g0 = (long long)expert * groups;
  if (w->layout == MOESQ_LAYOUT_PAIRED || w->layout == MOESQ_LAYOUT_PAIRED_TILED) {
    const long long units = groups / 2;
    hipLaunchKernelGGL(decode_paired_kernel,
                       dim3((unsigned)((units + PACK_THREADS - 1) / PACK_THREADS)),
                       dim3(PACK_THREADS), 0, stream, w->values + g0 * 2, w->masks + g0 / 2,
                       w->scales + g0 / 4, w->N, w->K, (int)tiled, (uint4 *)dense);
    return launch_status("moesq_decode_weights");
  }
  hipLaunchKernelGGL(decode_kernel, dim3((unsigned)((groups + PACK_THREADS - 1) / PACK_THREADS)),
                     dim3(PACK_THREADS), 0, stream, w->values + g0 * 2, w->masks + g0,
                     w->scales + g0 / 4, w->N, w->K, (int)tiled, (uint4 *)dense);
  return launch_status("moesq_decode_weights");
}
