// Shared host/device helpers of libmoesq: status handling, bf16 rounding,
// the E4M3 block-scale decode and the in-register 4:8 group decoder.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "moesq.h"

namespace moesq {

// ------------------------------------------------------------------ host side

// Records the detail of the last error of the calling thread.
moesq_status_t fail(moesq_status_t st, const std::string &msg);
// Checks a kernel launch; returns MOESQ_OK or MOESQ_ERR_HIP with the detail.
moesq_status_t launch_status(const char *what);
// Compute units of the current device (cached per device).
int device_cu_count();
// Clears the thread's last-error detail (start of every entry point).
void clear_error();

// ------------------------------------------------------------------ device side

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_bits_rne(lo) | (bf16_bits_rne(hi) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// E4M3 code (sign ignored) -> fp32, exact; used by the packer on the codes it
// has just encoded (never 0x7F or negative).  Exponent field 0 is subnormal
// (m * 2^-9).  The decoders use the hardware conversion instead.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float sub = (float)m * 0.001953125f;                       // m * 2^-9
  float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
  return e ? nrm : sub;
}

// Byte selectors of one 4:8 group for v_perm_b32.  With the group's kept
// values as bf16 in P0 = {b1:b0} and P1 = {b3:b2} (kept value j occupies
// bytes 2j and 2j+1 of the 8-byte {P1:P0}), output dword d holds the bf16 of
// positions 2d (low half) and 2d+1 (high half): selector bytes 2j, 2j+1 for
// a kept position carrying kept value j, 0x0C (yields 0x00) for a cleared one.
// Masks with more than four bits set decode their first four only.
__host__ __device__ inline uint32_t group_selector(uint32_t mask, int d) {
  uint32_t sel = 0;
  for (int h = 0; h < 2; ++h) {
    int p = 2 * d + h;
    uint32_t lo = 0x0c, hi = 0x0c;
    if ((mask >> p) & 1u) {
      uint32_t below = mask & ((1u << p) - 1u);
      uint32_t j = __builtin_popcount(below);
      if (j < 4) { lo = 2 * j; hi = 2 * j + 1; }
    }
    sel |= (lo | (hi << 8)) << (16 * h);
  }
  return sel;
}

// Fills a 256-entry selector table (one uint4 per mask byte) in LDS.
// Call with all threads of the block, then __syncthreads().
__device__ __forceinline__ void build_group_lut(uint4 *lut) {
  for (int m = threadIdx.x; m < 256; m += blockDim.x)
    lut[m] = make_uint4(group_selector(m, 0), group_selector(m, 1), group_selector(m, 2),
                        group_selector(m, 3));
}

// Decodes one 4:8 group to 8 bf16 (4 dwords, position 0 in the low half of
// dword 0).  `vw` holds the group's two value bytes at byte offset BYTE
// (0 or 2): byte BYTE = kept values 0,1 (low nibble first), byte BYTE+1 =
// kept values 2,3.  `scale` is the block scale in fp32.  Every decoded value
// E2M1 * E4M3 has at most 6 significant bits, so the fp32 product is exact
// and its upper 16 bits are the exact bf16.
template <int BYTE>
__device__ __forceinline__ uint4 decode_group(uint32_t mask8, uint32_t vw, float scale,
                                              const uint4 *lut) {
  f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(vw, 1.0f, BYTE);
  f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(vw, 1.0f, BYTE + 1);
  uint32_t u0 = __float_as_uint(a[0] * scale), u1 = __float_as_uint(a[1] * scale);
  uint32_t u2 = __float_as_uint(b[0] * scale), u3 = __float_as_uint(b[1] * scale);
  uint32_t p0 = __builtin_amdgcn_perm(u1, u0, 0x07060302u);  // {hi16(u1) : hi16(u0)}
  uint32_t p1 = __builtin_amdgcn_perm(u3, u2, 0x07060302u);
  uint4 s = lut[mask8];
  return make_uint4(__builtin_amdgcn_perm(p1, p0, s.x), __builtin_amdgcn_perm(p1, p0, s.y),
                    __builtin_amdgcn_perm(p1, p0, s.z), __builtin_amdgcn_perm(p1, p0, s.w));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

// ---- paired 4:8 ("Blackwell paired 4:8 NVFP4": two of the four position
// pairs of a group of eight are kept, six patterns).
//
// Reordering a group's positions as (0,2,4,6 | 1,3,5,7) turns every paired
// pattern into 2:4 on both halves with the same two indices: kept pairs
// i < j put one value at slots i and j of the even half and one at slots i
// and j of the odd half.  The sparse MFMA of gfx950 takes exactly that: per
// window of four dense K positions two compressed values and two 2-bit
// positions.  A "unit" is two neighbouring groups G, G' (16 positions) read
// as the four windows [G even, G' even, G odd, G' odd].

// 2-bit window positions i | j << 2 of canonical pattern index p (pairs in
// lexicographic order (0,1) (0,2) (0,3) (1,2) (1,3) (2,3)); 0 for p > 5.
__host__ __device__ inline uint32_t paired_window_index(uint32_t p) {
  constexpr uint32_t t = 4u | 8u << 4 | 12u << 8 | 9u << 12 | 13u << 16 | 14u << 20;
  return p < 6 ? (t >> (4 * p)) & 15u : 0u;
}

// Decodes a unit's eight compressed E2M1 codes (nibble i = compressed slot
// i) times the block scale to bf16, slot order (slot 0 in the low half of
// dword 0); exact, as in decode_group.
__device__ __forceinline__ uint4 decode_paired_unit(uint32_t v, float scale) {
  const f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 0);
  const f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 1);
  const f32x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 2);
  const f32x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(v, 1.0f, 3);
  auto hi2 = [&](float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi * scale), __float_as_uint(lo * scale),
                                 0x07060302u);
  };
  return make_uint4(hi2(a[0], a[1]), hi2(b[0], b[1]), hi2(c[0], c[1]), hi2(d[0], d[1]));
}

// x * sigmoid(x) with the hardware reciprocal (about 1 ulp): the result is
// rounded to bf16, 2^16 times coarser, so the IEEE division (a dozen
// instructions per element of the epilogue) buys nothing.
__device__ __forceinline__ float silu_f32(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

}  // namespace moesq
