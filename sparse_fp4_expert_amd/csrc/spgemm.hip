// Grouped 4:8 sparse-FP4 expert GEMM for gfx950.
//
// Paper summary page, "3.4 Implementation details": grouped execution runs
// every routing-dependent expert problem within one launch, with the sparse
// weights as the first MMA operand.  Here the weights stay compressed in HBM
// (13/32 byte per logical weight) and are decoded in registers straight into
// the A operand of v_mfma_f32_16x16x32_bf16: the decoded values E2M1*E4M3
// are exact in bf16, so only the fp32 accumulation and the final bf16
// rounding round.  Routed tokens are the B operand, staged through LDS.
//
// Work decomposition.  An item is (expert e, token tile of up to BM routed
// rows, row tile of BN weight rows).  Every workgroup reads the expert
// offsets into LDS, forms the per-expert item counts and their prefix, and
// walks items blockIdx.x, blockIdx.x + gridDim.x, ...; so the grid never
// depends on the routing, which only the device knows.  Token tiles are
// trimmed to whole 16-row MFMA fragments, so an expert with few rows costs
// few MFMAs and mostly streams its weights.
//
// K order inside a chunk of KC = 128.  The contraction order is free as long
// as both operands agree, so lane group q = lane/16 owns the 32 K positions
// [k0 + 32q, k0 + 32q + 32): one scale block, four groups of 8, 8 value
// bytes, 4 mask bytes and one scale byte, each a single load.  At k-step s
// (0..3) the A fragment of a lane is group s of its block, which is exactly
// the 8 consecutive bf16 the MFMA expects per lane, and the B fragment is the
// same 8 K positions of the lane's token, read from LDS.
#include <algorithm>

#include "common.hpp"

namespace moesq {

struct SpgemmArgs {
  const uint16_t *x;
  const int32_t *offsets;
  const uint8_t *values;
  const uint8_t *masks;
  const uint8_t *scales;
  const float *gscale;
  uint16_t *y;
  int M, E, N, K;
  int swiglu;
  int row_tiles;
};

constexpr int KC = 128;

template <int WAVES, int RF, int TF>
__global__ __launch_bounds__(WAVES * 64) void spgemm_kernel(SpgemmArgs a) {
  constexpr int THREADS = WAVES * 64;
  constexpr int BM = TF * 16;
  constexpr int BN = WAVES * RF * 16;
  constexpr int PITCH = KC + 8;  // bf16 elements per LDS token row (+16 B breaks bank aliasing)
  static_assert(RF % 2 == 0, "SwiGLU pairs gate and up fragments");

  __shared__ uint4 lut[256];
  __shared__ int s_lo[MOESQ_MAX_EXPERTS + 1];
  __shared__ int s_item[MOESQ_MAX_EXPERTS + 1];
  __shared__ __attribute__((aligned(16))) uint16_t tok[BM * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int E = a.E, N = a.N, K = a.K, M = a.M;

  build_group_lut(lut);
  // clamped expert ranges: rows [s_lo[e], s_lo[e+1]) with 0 <= lo <= hi <= M
  for (int e = tid; e <= E; e += THREADS) {
    int o = a.offsets[e];
    s_lo[e] = min(max(o, 0), M);
  }
  __syncthreads();
  if (wave == 0) {
    // items per expert, exclusive prefix by one wave
    const int per = (E + 63) / 64;
    const int e0 = min(E, lane * per), e1 = min(E, e0 + per);
    int sum = 0;
    for (int e = e0; e < e1; ++e) {
      const int rows = max(0, s_lo[e + 1] - s_lo[e]);
      sum += (rows + BM - 1) / BM * a.row_tiles;
    }
    int incl = sum;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(incl, d, 64);
      if (lane >= d) incl += t;
    }
    int run = incl - sum;
    for (int e = e0; e < e1; ++e) {
      s_item[e] = run;
      const int rows = max(0, s_lo[e + 1] - s_lo[e]);
      run += (rows + BM - 1) / BM * a.row_tiles;
    }
    if (lane == 63) s_item[E] = incl;
  }
  __syncthreads();
  const int total = s_item[E];

  const int q = lane >> 4;      // lane group: K block inside the chunk
  const int r16 = lane & 15;    // row inside an A fragment / token inside a B fragment
  const int half = N >> 1;
  const size_t vrow = (size_t)(K >> 2), mrow = (size_t)(K >> 3), srow = (size_t)(K >> 5);

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    // expert of this item: the largest e with s_item[e] <= item
    int lo = 0, hi = E;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_item[mid] <= item) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int local = item - s_item[e];
    const int tt = local / a.row_tiles, rt = local - tt * a.row_tiles;
    const int e_lo = s_lo[e], e_hi = max(e_lo, s_lo[e + 1]);
    const int tok0 = e_lo + tt * BM;
    const int ntok = min(BM, e_hi - tok0);
    const int nft = (ntok + 15) >> 4;

    // weight rows of this lane, one per fragment
    int frow[RF];
    bool fval[RF];
#pragma unroll
    for (int f = 0; f < RF; ++f) {
      if (a.swiglu) {
        const int hf = f % (RF / 2);
        const int gate0 = rt * (BN / 2) + (wave * (RF / 2) + hf) * 16;
        fval[f] = gate0 < half;
        frow[f] = (f < RF / 2 ? gate0 : half + gate0) + r16;
      } else {
        const int r0 = rt * BN + (wave * RF + f) * 16;
        fval[f] = r0 < N;
        frow[f] = r0 + r16;
      }
    }

    f32x4_t acc[RF][TF];
#pragma unroll
    for (int f = 0; f < RF; ++f)
#pragma unroll
      for (int t = 0; t < TF; ++t) acc[f][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < K; k0 += KC) {
      // compressed weights of this lane's K block, one load each
      const int kb = k0 + 32 * q;
      uint2 vv[RF];
      uint32_t mm[RF];
      float ss[RF];
#pragma unroll
      for (int f = 0; f < RF; ++f) {
        vv[f] = make_uint2(0, 0);
        mm[f] = 0;
        ss[f] = 0.f;
        if (fval[f] && kb < K) {
          const size_t row = (size_t)e * N + frow[f];
          vv[f] = *reinterpret_cast<const uint2 *>(a.values + row * vrow + (kb >> 2));
          mm[f] = *reinterpret_cast<const uint32_t *>(a.masks + row * mrow + (kb >> 3));
          ss[f] = e4m3_to_f32(a.scales[row * srow + (kb >> 5)]);
        }
      }
      // routed tokens of this chunk -> LDS (zero outside the tile and K)
      __syncthreads();
      for (int u = tid; u < BM * (KC / 8); u += THREADS) {
        const int row = u / (KC / 8), c8 = u % (KC / 8);
        const int kk = k0 + c8 * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (row < ntok && kk < K)
          v = *reinterpret_cast<const uint4 *>(a.x + (size_t)(tok0 + row) * K + kk);
        *reinterpret_cast<uint4 *>(&tok[row * PITCH + c8 * 8]) = v;
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint4 A[RF];
#pragma unroll
        for (int f = 0; f < RF; ++f) {
          const uint32_t m8 = (mm[f] >> (8 * s)) & 0xffu;
          const uint32_t vw = (s < 2) ? vv[f].x : vv[f].y;
          A[f] = (s & 1) ? decode_group<2>(m8, vw, ss[f], lut) : decode_group<0>(m8, vw, ss[f], lut);
        }
#pragma unroll
        for (int t = 0; t < TF; ++t) {
          if (t < nft) {
            const uint4 B = *reinterpret_cast<const uint4 *>(
                &tok[(t * 16 + r16) * PITCH + 32 * q + 8 * s]);
#pragma unroll
            for (int f = 0; f < RF; ++f)
              acc[f][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(A[f]), as_bf16x8(B),
                                                                  acc[f][t], 0, 0, 0);
          }
        }
      }
    }

    // epilogue: lane holds rows 4q..4q+3 of each fragment for token r16
    const float g = a.gscale[e];
#pragma unroll
    for (int t = 0; t < TF; ++t) {
      const int trow = t * 16 + r16;
      if (t >= nft || trow >= ntok) continue;
      const size_t out_r = (size_t)(tok0 + trow);
      if (!a.swiglu) {
#pragma unroll
        for (int f = 0; f < RF; ++f) {
          if (!fval[f]) continue;
          const int n0 = frow[f] - r16 + 4 * q;
          const f32x4_t c = acc[f][t];
          uint2 o;
          o.x = pack_bf16x2(g * c[0], g * c[1]);
          o.y = pack_bf16x2(g * c[2], g * c[3]);
          *reinterpret_cast<uint2 *>(a.y + out_r * N + n0) = o;
        }
      } else {
#pragma unroll
        for (int f = 0; f < RF / 2; ++f) {
          if (!fval[f]) continue;
          const int c0 = frow[f] - r16 + 4 * q;
          const f32x4_t gt = acc[f][t], up = acc[f + RF / 2][t];
          float h[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) h[i] = silu_f32(g * gt[i]) * (g * up[i]);
          uint2 o;
          o.x = pack_bf16x2(h[0], h[1]);
          o.y = pack_bf16x2(h[2], h[3]);
          *reinterpret_cast<uint2 *>(a.y + out_r * half + c0) = o;
        }
      }
    }
  }
}

template <int WAVES, int RF, int TF>
static moesq_status_t launch_spgemm(const SpgemmArgs &base, hipStream_t stream) {
  constexpr int BM = TF * 16, BN = WAVES * RF * 16;
  SpgemmArgs a = base;
  a.row_tiles = a.swiglu ? (a.N / 2 + BN / 2 - 1) / (BN / 2) : (a.N + BN - 1) / BN;
  // upper bound of the item count: every expert may hold one partial tile
  const long long tiles = (long long)a.M / BM + std::min(a.E, a.M);
  long long grid = tiles * a.row_tiles;
  const long long cap = (long long)device_cu_count() * 4;
  if (grid > cap) grid = cap;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL((spgemm_kernel<WAVES, RF, TF>), dim3((unsigned)grid), dim3(WAVES * 64), 0,
                     stream, a);
  return launch_status("moesq_grouped_spgemm");
}

static moesq_status_t check_weights(const moesq_weights_t *w, const char *who) {
  if (!w) return fail(MOESQ_ERR_NULL, std::string(who) + ": weight descriptor is NULL");
  if (w->layout != MOESQ_LAYOUT_CANONICAL)
    return fail(MOESQ_ERR_LAYOUT, std::string(who) + ": unknown weight layout");
  if (!w->values || !w->masks || !w->scales || !w->global_scale)
    return fail(MOESQ_ERR_NULL, std::string(who) + ": NULL weight buffer");
  if (w->E < 1 || w->E > MOESQ_MAX_EXPERTS)
    return fail(MOESQ_ERR_SHAPE, std::string(who) + ": E must be in [1, " +
                                     std::to_string(MOESQ_MAX_EXPERTS) + "]");
  if (w->N < 16 || w->N % 16) return fail(MOESQ_ERR_SHAPE, std::string(who) + ": N must be a positive multiple of 16");
  if (w->K < 32 || w->K % 32) return fail(MOESQ_ERR_SHAPE, std::string(who) + ": K must be a positive multiple of 32");
  return MOESQ_OK;
}

}  // namespace moesq

using namespace moesq;

extern "C" size_t moesq_spgemm_workspace_bytes(int32_t, const moesq_weights_t *) { return 0; }

extern "C" moesq_status_t moesq_grouped_spgemm(const uint16_t *x_routed,
                                               const int32_t *expert_offsets, int32_t M,
                                               const moesq_weights_t *w, int32_t epilogue,
                                               uint16_t *y, void *ws, size_t ws_bytes,
                                               hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  clear_error();
  moesq_status_t st = check_weights(w, "moesq_grouped_spgemm");
  if (st != MOESQ_OK) return st;
  if (epilogue != MOESQ_EPI_NONE && epilogue != MOESQ_EPI_SWIGLU)
    return fail(MOESQ_ERR_ARG, "moesq_grouped_spgemm: unknown epilogue");
  if (epilogue == MOESQ_EPI_SWIGLU && w->N % 32)
    return fail(MOESQ_ERR_SHAPE, "moesq_grouped_spgemm: SwiGLU needs N % 32 == 0");
  if (M < 0) return fail(MOESQ_ERR_SHAPE, "moesq_grouped_spgemm: M must be >= 0");
  if (!expert_offsets) return fail(MOESQ_ERR_NULL, "moesq_grouped_spgemm: expert_offsets is NULL");
  if (M == 0) return MOESQ_OK;
  if (!x_routed || !y) return fail(MOESQ_ERR_NULL, "moesq_grouped_spgemm: NULL x_routed or y");
  SpgemmArgs a{};
  a.x = x_routed;
  a.offsets = expert_offsets;
  a.values = w->values;
  a.masks = w->masks;
  a.scales = w->scales;
  a.gscale = w->global_scale;
  a.y = y;
  a.M = M;
  a.E = w->E;
  a.N = w->N;
  a.K = w->K;
  a.swiglu = epilogue == MOESQ_EPI_SWIGLU;
  return launch_spgemm<4, 4, 4>(a, stream);
}
