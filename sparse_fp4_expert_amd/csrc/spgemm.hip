// Grouped 4:8 sparse-FP4 expert GEMM for gfx950.
//
// Paper summary page, "3.4 Implementation details": grouped execution runs
// every routing-dependent expert problem within one launch, with the sparse
// weights as the first MMA operand (here: one launch per tiling, each over
// the experts of its size range; see the tile choice at the end).  The
// weights stay compressed in HBM
// (13/32 byte per logical weight) and are decoded in registers straight into
// the A operand of a bf16 MFMA (v_mfma_f32_16x16x32_bf16 or
// v_mfma_f32_32x32x16_bf16): the decoded values E2M1*E4M3 are exact in bf16,
// so only the fp32 accumulation and the final bf16 rounding round.  Routed
// tokens are the B operand, staged through LDS by direct global->LDS loads.
//
// Work decomposition.  An item is (expert e, token tile of up to BM routed
// rows, row tile of BN weight rows).  Every workgroup reads the expert
// offsets, forms the item list in LDS -- all whole token tiles first, then
// the partial ones by descending size, so that rounds of workgroups take
// the costly items first -- and walks the items with a grid-sized stride,
// so the grid never depends on the routing, which only the device knows.  Token tiles are trimmed to whole
// MFMA fragments, so an expert with few rows costs few MFMAs and mostly
// streams its weights.
//
// K order.  The contraction order is free as long as both operands agree.
// An MFMA of shape MS x MS x (8*LG) gives lane group q = lane / MS (LG = 64/MS
// groups) eight consecutive K positions.  Inside a chunk of KC positions,
// lane group q owns the KQ = KC/LG positions [k0 + KQ*q, k0 + KQ*q + KQ):
// whole scale blocks, so its values, masks and scales are one load each, and
// k-step s hands it the 4:8 group s of that range -- exactly one decoded
// group per lane -- while the B fragment holds the same 8 positions of the
// lane's token.
#include <algorithm>
#include <climits>
#include <type_traits>

#include "common.hpp"
#include "route_dev.hpp"

namespace moesq {

struct SpgemmArgs {
  const uint16_t *x;        // routed rows [M][K], or tokens [T][K] with `perm`
  const int32_t *perm;      // NULL, or gather: routed row r reads token perm[r] / k
  int T, k;                 // token rows of x and experts per token (gather only)
  const int32_t *offsets;
  const uint8_t *values;
  const uint8_t *masks;
  const uint8_t *scales;
  const float *gscale;
  uint16_t *y;
  int M, E, N, K;
  int row_tiles;
  int rows_lo, rows_hi;     // this launch takes the experts with rows_lo < rows <= rows_hi
  // fused routing (decode batches): the flat top-k ids [M]; every workgroup
  // builds the plan in LDS, workgroup 0 also stores it
  const int32_t *ids;
  int32_t *route_offsets, *route_perm, *route_inv;
  int flat;   // store result row r at y[perm[r]] (flat order) instead of y[r]
  // NVFP4 activations (W4A4): codes [rows][K/2], E4M3 scales [rows][K/32] and
  // the fp32 row scales of the token rows (rows = T with a gather, else M)
  const uint8_t *aq_codes;
  const uint8_t *aq_scales;
  const float *aq_g;
};

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int MS>
struct Mfma;
template <>
struct Mfma<16> {
  using C = f32x4_t;
  static constexpr int NC = 4;
  static __device__ __forceinline__ C run(uint4 a, uint4 b, C c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
  }
};
template <>
struct Mfma<32> {
  using C = f32x16_t;
  static constexpr int NC = 16;
  static __device__ __forceinline__ C run(uint4 a, uint4 b, C c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
  }
};

// Compressed weights of one lane for one K chunk: for each of its RF
// fragment rows, the KQ positions of its lane group.
template <int RF, int KQ>
struct WChunk {
  static constexpr int VD = KQ / 16;   // value dwords (8 nibbles each)
  static constexpr int MD = KQ / 32;   // mask dwords (4 groups each)
  uint32_t v[RF][VD];
  uint32_t m[RF][MD];
  uint32_t s[RF];                      // KQ/32 scale bytes
};

// vb/mb/sb: the expert's value/mask/scale bases; fv/fm/fs: byte offsets of
// each fragment's first row (uniform); vo/mo/so: this lane's offsets inside
// a fragment (its row and lane group); kv/km/ks: offsets of the chunk.
// ok[f]: the lane's first scale block lies inside K; the two-block range
// loads only its first block when `whole` is false (K ends in the middle of
// the range).
template <int RF>
__device__ __forceinline__ void load_wchunk(WChunk<RF, 64> &w, const uint8_t *vb,
                                            const uint8_t *mb, const uint8_t *sb,
                                            const uint32_t (&fv)[RF], const uint32_t (&fm)[RF],
                                            const uint32_t (&fs)[RF], uint32_t vo, uint32_t mo,
                                            uint32_t so, const bool (&ok)[RF], bool whole,
                                            uint32_t kv, uint32_t km, uint32_t ks) {
#pragma unroll
  for (int f = 0; f < RF; ++f) {
    if (!ok[f]) {
#pragma unroll
      for (int i = 0; i < 4; ++i) w.v[f][i] = 0;
#pragma unroll
      for (int i = 0; i < 2; ++i) w.m[f][i] = 0;
      w.s[f] = 0;
      continue;
    }
    const uint8_t *pv = vb + (fv[f] + vo + kv);
    const uint8_t *pm = mb + (fm[f] + mo + km);
    const uint8_t *ps = sb + (fs[f] + so + ks);
    if (!whole) {
      const uint2 v = *reinterpret_cast<const uint2 *>(pv);
      w.v[f][0] = v.x;
      w.v[f][1] = v.y;
      w.v[f][2] = 0;
      w.v[f][3] = 0;
      w.m[f][0] = *reinterpret_cast<const uint32_t *>(pm);
      w.m[f][1] = 0;
      w.s[f] = *ps;
    } else {
      const uint4 v = *reinterpret_cast<const uint4 *>(pv);
      w.v[f][0] = v.x;
      w.v[f][1] = v.y;
      w.v[f][2] = v.z;
      w.v[f][3] = v.w;
      const uint2 m = *reinterpret_cast<const uint2 *>(pm);
      w.m[f][0] = m.x;
      w.m[f][1] = m.y;
      w.s[f] = *reinterpret_cast<const uint16_t *>(ps);
    }
  }
}

// Tiled layout: a lane group's 64 positions of one fragment are 16 value
// bytes, 8 mask bytes and 2 scale bytes at offsets lo, lo/2, lo/8 past the
// fragment's segment-row start fv/fm/fs inside the expert's arrays.  Buffer
// loads take lo in a VGPR and the fragment offset in an SGPR.
template <int RF>
__device__ __forceinline__ void load_wchunk_tiled(WChunk<RF, 64> &w, __amdgpu_buffer_rsrc_t vr,
                                                  __amdgpu_buffer_rsrc_t mr, __amdgpu_buffer_rsrc_t sr,
                                                  const uint32_t (&fv)[RF], const uint32_t (&fm)[RF],
                                                  const uint32_t (&fs)[RF], uint32_t lo) {
#pragma unroll
  for (int f = 0; f < RF; ++f) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(vr, lo, fv[f], 0);
    const u32x2_t m = __builtin_amdgcn_raw_buffer_load_b64(mr, lo >> 1, fm[f], 0);
    w.v[f][0] = v[0];
    w.v[f][1] = v[1];
    w.v[f][2] = v[2];
    w.v[f][3] = v[3];
    w.m[f][0] = m[0];
    w.m[f][1] = m[1];
    w.s[f] = __builtin_amdgcn_raw_buffer_load_b16(sr, lo >> 3, fs[f], 0);
  }
}

template <int RF, int KQ>
__device__ __forceinline__ void decode_step(uint4 (&A)[RF], const WChunk<RF, KQ> &w,
                                            const float (&sf)[RF][KQ / 32], const uint4 *lut,
                                            int s) {
#pragma unroll
  for (int f = 0; f < RF; ++f) {
    const uint32_t m8 = (w.m[f][s >> 2] >> (8 * (s & 3))) & 0xffu;
    const uint32_t vw = w.v[f][s >> 1];
    A[f] = (s & 1) ? decode_group<2>(m8, vw, sf[f][s >> 2], lut)
                   : decode_group<0>(m8, vw, sf[f][s >> 2], lut);
  }
}

// Decode + MFMA over one K chunk staged in `tk`: token T's 16-byte unit c of
// the chunk sits at element T*KC + 8*(c ^ (T % UPR)), so the MS lanes of a
// lane group read MS different columns.  The A fragments of k-step s+1 are
// decoded while the MFMAs of step s run.  (A scheduling barrier per step,
// which kept the compiler from moving work across steps, measured 0.5-1 %
// slower on the prefill and decode workloads.)  FULL: all TF token
// fragments hold routed rows.
template <int MS, int RF, int TF, int KC, bool FULL>
__device__ __forceinline__ void mma_chunk(typename Mfma<MS>::C (&acc)[RF][TF],
                                          const uint16_t *tk, const WChunk<RF, KC * MS / 64> &w,
                                          const uint4 *lut, int nft, int q, int rl) {
  constexpr int KQ = KC * MS / 64;
  constexpr int S = KQ / 8;
  constexpr int UPR = KC / 8;
  static_assert(KQ == 64, "a lane group covers two scale blocks per chunk");
  // block scales: the hardware E4M3 (OCP) conversion is exact
  float sf[RF][2];
#pragma unroll
  for (int f = 0; f < RF; ++f) {
    const f32x2_t p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.s[f], 1.0f, false);
    sf[f][0] = p[0];
    sf[f][1] = p[1];
  }
  const uint16_t *brow = tk + rl * KC;
  const int cbase = (KQ / 8) * q;
  uint4 A[2][RF];
  decode_step<RF, KQ>(A[0], w, sf, lut, 0);
#pragma unroll
  for (int s = 0; s < S; ++s) {
    uint4 B[TF];
#pragma unroll
    for (int t = 0; t < TF; ++t)
      if (FULL || t < nft)
        B[t] = *reinterpret_cast<const uint4 *>(
            brow + t * MS * KC + (((cbase + s) ^ ((t * MS + rl) & (UPR - 1))) << 3));
    if (s + 1 < S) decode_step<RF, KQ>(A[(s + 1) & 1], w, sf, lut, s + 1);
#pragma unroll
    for (int t = 0; t < TF; ++t)
      if (FULL || t < nft)
#pragma unroll
        for (int f = 0; f < RF; ++f) acc[f][t] = Mfma<MS>::run(A[s & 1][f], B[t], acc[f][t]);
  }
}

// ---- paired 4:8 weights on the sparse MFMA (v_smfmac_f32_16x16x64_bf16,
// v_smfmac_f32_32x32x32_bf16).  Lane l holds A row l % MS and eight
// compressed bf16 for the dense K range [16q, 16q+16), q = l / MS: one unit
// (two groups as the windows [G even, G' even, G odd, G' odd]) with its
// 2-bit window positions in the index operand.  B lane l holds token
// l % MS: elements 0..7 are dense K 8q..8q+7 and elements 8..15 dense K
// 8q+32..8q+39 (16x16x64) or 8q+16..8q+23 (32x32x32), i.e. the even or odd
// half of a unit of lane group q >> 1 and of lane group (q >> 1) + LG/2.
// The accumulator layout is that of the dense MFMA of the same shape.
template <int MS>
struct Smfmac;
template <>
struct Smfmac<16> {
  using C = f32x4_t;
  static __device__ __forceinline__ C run(uint4 a, bf16x16_t b, C c, int idx) {
    return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(as_bf16x8(a), b, c, idx, 0, 0);
  }
};
template <>
struct Smfmac<32> {
  using C = f32x16_t;
  static __device__ __forceinline__ C run(uint4 a, bf16x16_t b, C c, int idx) {
    return __builtin_amdgcn_smfmac_f32_32x32x32_bf16(as_bf16x8(a), b, c, idx, 0, 0);
  }
};

// Paired tiled weights of one lane for one K chunk: per fragment, its lane
// group's 64-position segment -- four units of eight codes, four window
// bytes, two scale bytes.
template <int RF>
struct PChunk {
  uint32_t v[RF][4];
  uint32_t w[RF];
  uint32_t s[RF];
};

template <int RF>
__device__ __forceinline__ void load_pchunk(PChunk<RF> &c, __amdgpu_buffer_rsrc_t vr,
                                            __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr,
                                            const uint32_t (&fv)[RF], const uint32_t (&fw)[RF],
                                            const uint32_t (&fs)[RF], uint32_t lo) {
#pragma unroll
  for (int f = 0; f < RF; ++f) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(vr, lo, fv[f], 0);
    c.v[f][0] = v[0];
    c.v[f][1] = v[1];
    c.v[f][2] = v[2];
    c.v[f][3] = v[3];
    c.w[f] = __builtin_amdgcn_raw_buffer_load_b32(wr, lo >> 2, fw[f], 0);
    c.s[f] = __builtin_amdgcn_raw_buffer_load_b16(sr, lo >> 3, fs[f], 0);
  }
}

// Sparse MFMAs over one chunk staged in `tk`: a token row of the chunk holds
// KC/16 units of 32 bytes, [8 even-position bf16 | 8 odd-position bf16],
// whose 16-byte halves h sit at slot (2u + h) ^ (row % (KC/8)).  Step s
// takes unit s of every lane group's segment; the A operands of step s+1
// are decoded while the sparse MFMAs of step s run.
template <int MS, int RF, int TF, int KC, bool FULL>
__device__ __forceinline__ void mma_chunk_paired(typename Smfmac<MS>::C (&acc)[RF][TF],
                                                 const uint16_t *tk, const PChunk<RF> &w, int nft,
                                                 int q, int rl) {
  constexpr int LG = 64 / MS;
  constexpr int SLOTS = KC / 8;
  float sf[RF][2];
#pragma unroll
  for (int f = 0; f < RF; ++f) {
    const f32x2_t p = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w.s[f], 1.0f, false);
    sf[f][0] = p[0];
    sf[f][1] = p[1];
  }
  const int half = q & 1, ulo = 4 * (q >> 1), uhi = 4 * ((q >> 1) + LG / 2);
  uint4 A[2][RF];
  int I[2][RF];
  auto dec = [&](uint4 (&a)[RF], int (&ix)[RF], int s) {
#pragma unroll
    for (int f = 0; f < RF; ++f) {
      a[f] = decode_paired_unit(w.v[f][s], sf[f][s >> 1]);
      // window byte s into bytes 0 and 1: the same positions for both halves
      ix[f] = (int)__builtin_amdgcn_perm(w.w[f], w.w[f], 0x0c0c0000u | (uint32_t)(s << 8) | (uint32_t)s);
    }
  };
  auto load_b = [&](int t, int s) {
    const int row = t * MS + rl;
    const uint16_t *br = tk + row * KC;
    const int sw = row & (SLOTS - 1);
    const uint4 lo = *reinterpret_cast<const uint4 *>(br + 8 * ((2 * (ulo + s) + half) ^ sw));
    const uint4 hi = *reinterpret_cast<const uint4 *>(br + 8 * ((2 * (uhi + s) + half) ^ sw));
    struct { uint4 l, h; } lh = {lo, hi};
    return __builtin_bit_cast(bf16x16_t, lh);
  };
  dec(A[0], I[0], 0);
  // token fragments one ahead: two B operands (16 VGPRs) live, not TF.  The
  // 32-row tile also carries the lookahead across steps (the last fragment
  // of step s loads the first of step s+1); on the 16-row tile that costs
  // spills.
  constexpr bool ACROSS = MS == 32;
  bf16x16_t B = load_b(0, 0);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (!ACROSS && s > 0) B = load_b(0, s);
    if (s + 1 < 4) dec(A[(s + 1) & 1], I[(s + 1) & 1], s + 1);
#pragma unroll
    for (int t = 0; t < TF; ++t) {
      if (!FULL && t >= nft) break;
      bf16x16_t Bn = B;
      if (t + 1 < TF && (FULL || t + 1 < nft))
        Bn = load_b(t + 1, s);
      else if (ACROSS && s + 1 < 4)
        Bn = load_b(0, s + 1);
#pragma unroll
      for (int f = 0; f < RF; ++f)
        acc[f][t] = Smfmac<MS>::run(A[s & 1][f], B, acc[f][t], I[s & 1][f]);
      B = Bn;
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// LDS pointer / 32-bit LDS address of a __shared__ object (device only: the
// address space does not exist on the host).
__device__ __forceinline__ __attribute__((address_space(3))) void *lds_ptr(void *p) {
  return (__attribute__((address_space(3))) void *)p;
}
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}
// SIZE bytes per lane from a buffer to LDS at lds + SIZE * lane.
template <int SIZE>
__device__ __forceinline__ void buffer_to_lds(__amdgpu_buffer_rsrc_t r, void *lds, uint32_t voff,
                                              uint32_t soff) {
  static_assert(SIZE == 16 || SIZE == 4 || SIZE == 2, "LDS DMA of 2, 4 or 16 bytes per lane");
  if constexpr (SIZE == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(lds), 16, voff, soff, 0, 0);
  else if constexpr (SIZE == 4)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(lds), 4, voff, soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_ptr(lds), 2, voff, soff, 0, 0);
}

// Weight formats of the kernel.
enum { FMT_CANONICAL = 0, FMT_TILED = 1, FMT_PAIRED = 2 };

// Dynamic LDS of the item schedule for E experts: prefix [E+1] and row
// counts [E] as int, partial-tile experts [E] as uint16, rounded to 16 bytes.
__host__ __device__ inline size_t spgemm_sched_bytes(int E) {
  return ((size_t)(2 * E + 1) * 4 + (size_t)E * 2 + 15) & ~(size_t)15;
}

template <int WAVES, int MS, int RF, int TF, int KC, bool SWIGLU, int FMT, bool ROUTE = false,
          bool ACT4 = false>
__global__ __launch_bounds__(WAVES * 64)
// 16-row tiles stream weights: at most 128 VGPRs, so that four 4-wave
// workgroups share a CU.  32-row tiles hold 128 accumulators per lane.
__attribute__((amdgpu_waves_per_eu(MS == 16 ? 4 : 1, MS == 16 ? 4 : 2))) void spgemm_kernel(
    SpgemmArgs a) {
  constexpr bool TILED = FMT != FMT_CANONICAL;
  constexpr bool PAIRED = FMT == FMT_PAIRED;
  using MF = Mfma<MS>;
  constexpr int LG = 64 / MS;          // lane groups
  constexpr int BM = TF * MS;          // tokens per tile
  constexpr int BN = WAVES * RF * MS;  // weight rows per tile
  constexpr int KQ = KC / LG;          // K positions per lane group per chunk
  constexpr int UPR = KC / 8;          // 16-byte units per token row of a chunk
  constexpr int NBLK = BM * KC * 2 / 1024;  // 1 KB direct-to-LDS loads per chunk
  constexpr int BPW = NBLK / WAVES;    // ... per wave
  static_assert(NBLK % WAVES == 0, "token tile must split evenly over the waves");
  static_assert(64 % UPR == 0, "a 1 KB load covers whole token rows");
  static_assert(RF % 2 == 0, "SwiGLU pairs gate and up fragments");
  static_assert(KQ == 64, "a lane group covers one 64-position segment (two scale blocks) per chunk");

  __shared__ uint4 lut[PAIRED ? 1 : 256];   // 4:8 selector table (paired needs none)
  // Item order (contraction tiles): every expert's whole token tiles first
  // (expert order), then the partial tiles (at most one per expert) by
  // descending fragment count.  Workgroups take items in fixed rounds, so
  // putting the costly items first and the cheap ones last balances the
  // rounds (longest job first).  Streaming tiles: see STREAM below.
  // The three per-expert arrays sit in dynamic LDS sized for the launch's
  // E (spgemm_sched_bytes), so that a small expert count leaves room for
  // more workgroups per CU.
  extern __shared__ __attribute__((aligned(16))) int s_dyn[];
  __shared__ int s_npart;
  __shared__ __attribute__((aligned(1024))) uint16_t tkA[BM * KC];
  __shared__ __attribute__((aligned(1024))) uint16_t tkB[BM * KC];
  // Contraction tile on paired weights: the weights of chunk c + 2 stream
  // into a three-slot LDS ring by direct-to-LDS buffer loads while chunk c
  // computes, so each weight load has two chunks of compute to land in; the
  // tokens stay one chunk ahead.  (The sparse MFMA halves the compute per
  // chunk, which one chunk of prefetch no longer covers.  The 4:8 tile keeps
  // its weights in registers: its decode already loads LDS with the
  // selector table, and measured slower with the ring.)  Per slot, wave and
  // fragment: the 64 lanes' 16 value bytes, their mask (8) or window (4)
  // bytes and 2 scale bytes, in lane order.
  constexpr bool RING = PAIRED && MS == 32;
  // (a 2-byte direct-to-LDS load fills a 4-byte slot per lane)
  constexpr int RV = 64 * 16, RM = 64 * (PAIRED ? 4 : 8), RS = 64 * 4;
  constexpr int RFB = RV + RM + RS;                 // bytes per fragment
  constexpr int RSLOT = WAVES * RF * RFB;           // bytes per slot
  constexpr int RING_LOADS = RF * (PAIRED ? 3 : 4); // buffer loads per wave per slot
  __shared__ __attribute__((aligned(16))) uint8_t wring[RING ? 3 * RSLOT : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = a.E, N = a.N, K = a.K, M = a.M;
  int *const s_full = s_dyn;                  // [E+1] item prefix of the whole tiles
  int *const s_cnt = s_dyn + E + 1;           // [E] routed rows per expert
  uint16_t *const s_part = reinterpret_cast<uint16_t *>(s_dyn + 2 * E + 1);
                                              // [E] experts with a partial tile, costly first

  if constexpr (!PAIRED) build_group_lut(lut);
  // Fused routing (decode batches): the routing plan of the M flat ids
  // (offsets and gather permutation), built in LDS after the schedule
  // arrays, exactly as moesq_route builds it (stable counting sort);
  // workgroup 0 also stores it for the combine.
  int *const s_roff = s_dyn + spgemm_sched_bytes(E) / 4;   // [E+1]
  int *const s_rperm = s_roff + E + 1;                      // [M]
  // expert row ranges straight from the offsets (clamped to [0, M]); only
  // the item prefix is kept in LDS
  auto off_at = [&](int e) {
    return min(max(ROUTE ? s_roff[e] : a.offsets[e], 0), M);
  };
  auto perm_at = [&](int r) { return ROUTE ? s_rperm[r] : a.perm[r]; };
  // Streaming tiles (16-row fragments) cost about the same whatever their
  // row count (the weight decode dominates), so every token tile of an
  // expert, partial or not, goes in the prefix in expert order, with the
  // token tiles of one row tile next to each other: they read the same
  // weights at the same time on one XCD, and the second read hits L2.
  constexpr bool STREAM = MS == 16;
  auto tiles_of = [&](int e) { return STREAM ? (s_cnt[e] + BM - 1) / BM : s_cnt[e] / BM; };
  if constexpr (ROUTE) {
    // Every wave takes a contiguous segment of at most 64 * J ids (M is at
    // most MOESQ_FUSED_ROUTE_MAX_ROWS, checked on the host) and counts it
    // per expert into its own row of `cw` (the token buffer, unused until
    // the first item); one scan over the experts then gives the offsets,
    // the item prefix and each wave's first routed row per expert, and each
    // wave scatters its segment.  Segments in wave order and ids in lane
    // order within a wave keep the sort stable.
    static_assert(!ROUTE || (STREAM && WAVES * MOESQ_MAX_EXPERTS <= BM * KC),
                  "fused routing runs on the streaming tile; per-wave counts fit its token buffer");
    constexpr int NT = WAVES * 64;
    constexpr int J = (MOESQ_FUSED_ROUTE_MAX_ROWS + NT - 1) / NT;
    constexpr int EP = (MOESQ_MAX_EXPERTS + NT - 1) / NT;   // experts per thread in the scan
    __shared__ int s_wtot[2 * WAVES];
    uint16_t *const cw = tkA;                               // [WAVES][E]
    uint16_t *const mine = cw + wave * E;
    const uint64_t lt = lanes_below(lane);
    const int nbits = id_bits(E);
    const int seg = 64 * ((M + NT - 1) / NT);
    const int beg = min(M, wave * seg), len = min(M, beg + seg) - beg;
    int idv[J];
    wave_load_ids(a.ids, beg, len, E, lane, idv);
    for (int i = tid; i < WAVES * E; i += NT) cw[i] = 0;
    __syncthreads();
    wave_count_regs(idv, len, nbits, lt, mine);
    __syncthreads();
    // experts [tid * EP, tid * EP + EP) of this thread, in expert order
    int cin[EP], rows_l = 0, tiles_l = 0;
#pragma unroll
    for (int q = 0; q < EP; ++q) {
      const int e = tid * EP + q;
      int c = 0;
      if (e < E)
        for (int w = 0; w < WAVES; ++w) c += cw[w * E + e];
      cin[q] = c;
      rows_l += c;
      const int ci = (c > a.rows_lo && c <= a.rows_hi) ? c : 0;
      tiles_l += (ci + BM - 1) / BM;
    }
    const int rincl = wave_incl_scan(rows_l, lane), tincl = wave_incl_scan(tiles_l, lane);
    if (lane == 63) {
      s_wtot[wave] = rincl;
      s_wtot[WAVES + wave] = tincl;
    }
    __syncthreads();
    int rrun = rincl - rows_l, trun = tincl - tiles_l, rtot = 0, ttot = 0;
    for (int w = 0; w < WAVES; ++w) {
      if (w < wave) {
        rrun += s_wtot[w];
        trun += s_wtot[WAVES + w];
      }
      rtot += s_wtot[w];
      ttot += s_wtot[WAVES + w];
    }
#pragma unroll
    for (int q = 0; q < EP; ++q) {
      const int e = tid * EP + q;
      if (e >= E) break;
      const int c = cin[q];
      const int ci = (c > a.rows_lo && c <= a.rows_hi) ? c : 0;
      s_roff[e] = rrun;
      s_cnt[e] = ci;
      s_full[e] = trun * a.row_tiles;
      trun += (ci + BM - 1) / BM;
      int r = rrun;   // each wave's first routed row of expert e
      for (int w = 0; w < WAVES; ++w) {
        const int t = cw[w * E + e];
        cw[w * E + e] = (uint16_t)r;
        r += t;
      }
      rrun += c;
    }
    if (tid == 0) {
      s_roff[E] = rtot;
      s_full[E] = ttot * a.row_tiles;
      s_npart = 0;
    }
    __syncthreads();
    wave_scatter_regs(idv, beg, len, nbits, lt, lane, mine, s_rperm,
                      blockIdx.x == 0 ? a.route_inv : nullptr);
    __syncthreads();
    if (blockIdx.x == 0) {
      for (int e = tid; e <= E; e += NT) a.route_offsets[e] = s_roff[e];
      for (int r = tid; r < rtot; r += NT) a.route_perm[r] = s_rperm[r];
    }
  } else {
    // routed rows per expert; experts outside this launch's row range count
    // as empty (another launch of the same call takes them)
    for (int e = tid; e < E; e += WAVES * 64) {
      const int c = max(0, off_at(e + 1) - off_at(e));
      s_cnt[e] = (c > a.rows_lo && c <= a.rows_hi) ? c : 0;
    }
    __syncthreads();
    if (wave == 0) {
      // by one wave: prefix of the whole tiles, then the partial tiles
      // bucketed by fragment count (TF down to 1), experts ascending within
      // a bucket
      const int per = (E + 63) / 64;
      const int e0 = min(E, lane * per), e1 = min(E, e0 + per);
      int sum = 0;
      for (int e = e0; e < e1; ++e) sum += tiles_of(e);
      const int incl = wave_incl_scan(sum, lane);
      int run = incl - sum;
      for (int e = e0; e < e1; ++e) {
        s_full[e] = run * a.row_tiles;
        run += tiles_of(e);
      }
      if (lane == 63) s_full[E] = incl * a.row_tiles;
      int base = 0;
      for (int c = STREAM ? 0 : TF; c >= 1; --c) {
        auto cls = [&](int e) {
          const int rem = s_cnt[e] % BM;
          return rem > 0 && (rem + MS - 1) / MS == c;
        };
        int cnt = 0;
        for (int e = e0; e < e1; ++e) cnt += cls(e);
        const int ci = wave_incl_scan(cnt, lane);
        int pos = base + ci - cnt;
        for (int e = e0; e < e1; ++e)
          if (cls(e)) s_part[pos++] = e;
        base += __shfl(ci, 63, 64);
      }
      if (lane == 0) s_npart = base;
    }
  }
  __syncthreads();
  const int nfull = s_full[E];
  const int total = nfull + s_npart * a.row_tiles;

  const int q = lane / MS;     // lane group: K range [k0 + KQ*q, +KQ) of a chunk
  const int rl = lane % MS;    // A-fragment row / B-fragment token of this lane
  const int half = N >> 1;
  const size_t vrow = (size_t)(K >> 2), mrow = (size_t)(K >> 3), srow = (size_t)(K >> 5);
  const int nk = (K + KC - 1) / KC;
  // this lane's offsets inside a fragment: canonical rows are K/4, K/8, K/32
  // bytes long; tiled segments hold 32 rows of 16, 8, 2 bytes
  const uint32_t vo = TILED ? q * 512u + rl * 16u : (uint32_t)rl * (uint32_t)vrow + (KQ / 4) * q;
  const uint32_t mo = TILED ? q * 256u + rl * 8u : (uint32_t)rl * (uint32_t)mrow + (KQ / 8) * q;
  const uint32_t so = TILED ? q * 64u + rl * 2u : (uint32_t)rl * (uint32_t)srow + (KQ / 32) * q;
  const uint32_t segs = (uint32_t)(K >> 6);

  // Items of one round of workgroups are spread XCD-major: the grid is a
  // multiple of 8 and workgroup b runs on XCD b % 8.  A round's n items are
  // cut into 8 runs of ceil(n/8) consecutive items, one run per XCD, so
  // consecutive items (the row tiles of one token tile) share an XCD's L2
  // and a short last round still uses every XCD.
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7, wg_in_xcd = blockIdx.x >> 3;

  for (int base = 0; base < total; base += G) {
    const int n_round = min(G, total - base);
    const int per = (n_round + 7) >> 3;
    if (wg_in_xcd >= per || xcd * per + wg_in_xcd >= n_round) break;   // no item in the last round
    const int item = base + xcd * per + wg_in_xcd;
    int e, tt, rt;
    if (item < nfull) {
      int lo = 0, hi = E;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_full[mid] <= item) lo = mid; else hi = mid - 1;
      }
      e = lo;
      const int local = item - s_full[e];
      if constexpr (STREAM) {
        const int ntt = tiles_of(e);
        rt = local / ntt;
        tt = local - rt * ntt;
      } else {
        tt = local / a.row_tiles;
        rt = local - tt * a.row_tiles;
      }
    } else {
      const int j = (item - nfull) / a.row_tiles;
      rt = item - nfull - j * a.row_tiles;
      e = s_part[j];
      tt = s_cnt[e] / BM;   // the last, partial tile
    }
    const int e_lo = off_at(e), e_hi = max(e_lo, off_at(e + 1));
    const int tok0 = e_lo + tt * BM;
    const int ntok = min(BM, e_hi - tok0);
    const int nft = (ntok + MS - 1) / MS;

    // first weight row of each fragment (uniform); SwiGLU pairs gate
    // fragment f with up fragment f + RF/2, N/2 rows further
    int frow[RF];
    bool fval[RF];
#pragma unroll
    for (int f = 0; f < RF; ++f) {
      if constexpr (SWIGLU) {
        const int gate0 = rt * (BN / 2) + (wave * (RF / 2) + f % (RF / 2)) * MS;
        fval[f] = gate0 < half;
        frow[f] = f < RF / 2 ? gate0 : half + gate0;
      } else {
        frow[f] = rt * BN + (wave * RF + f) * MS;
        fval[f] = frow[f] < N;
      }
    }
    const size_t erow = (size_t)e * N;
    const uint8_t *vb = a.values + erow * vrow, *mb = a.masks + erow * (PAIRED ? mrow / 2 : mrow),
                  *sb = a.scales + erow * srow;
    const uint32_t ebytes = (uint32_t)(vrow * (size_t)N);   // value bytes of one expert
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc((void *)vb, 0, (int)ebytes, 0x20000);
    // mask bytes: half the value bytes; paired window bytes: a quarter
    const __amdgpu_buffer_rsrc_t mr =
        __builtin_amdgcn_make_buffer_rsrc((void *)mb, 0, (int)(ebytes >> (PAIRED ? 2 : 1)), 0x20000);
    const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc((void *)sb, 0, (int)(ebytes >> 3), 0x20000);
    // token rows: T rows with a gather, else the M routed rows (under 4 GiB:
    // checked on the host)
    const uint32_t xbytes = (uint32_t)((size_t)((ROUTE || a.perm) ? a.T : a.M) * (size_t)K * 2u);
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void *)a.x, 0, (int)xbytes, 0x20000);
    uint32_t fv[RF], fm[RF], fs[RF];
#pragma unroll
    for (int f = 0; f < RF; ++f) {
      const uint32_t r = fval[f] ? (uint32_t)frow[f] : 0u;
      if constexpr (TILED) {
        const uint32_t blk = (r >> 5) * segs, rin = r & 31u;
        fv[f] = blk * 512u + rin * 16u;
        fm[f] = PAIRED ? blk * 128u + rin * 4u : blk * 256u + rin * 8u;
        fs[f] = blk * 64u + rin * 2u;
      } else {
        fv[f] = r * (uint32_t)vrow;
        fm[f] = r * (uint32_t)mrow;
        fs[f] = r * (uint32_t)srow;
      }
    }
    // chunk offsets: canonical advances k/4, k/8, k/32 bytes; tiled advances
    // one 64-position segment (512, 256, 64 bytes) per 64 positions
    auto koff = [&](int k0, uint32_t &kv, uint32_t &km, uint32_t &ks) {
      if constexpr (TILED) {
        kv = (uint32_t)k0 * 8u;
        km = (uint32_t)k0 * 4u;
        ks = (uint32_t)k0;
      } else {
        kv = (uint32_t)k0 >> 2;
        km = (uint32_t)k0 >> 3;
        ks = (uint32_t)k0 >> 5;
      }
    };

    // tiled: this lane's segment of the chunk at k0, clamped into K
    auto tlo = [&](int k0) {
      const uint32_t seg = min((uint32_t)(k0 >> 6) + (uint32_t)q, segs - 1u);
      return seg * 512u + (uint32_t)rl * 16u;
    };
    auto wok = [&](int k0, bool (&ok)[RF]) {
#pragma unroll
      for (int f = 0; f < RF; ++f) ok[f] = fval[f] && (k0 + KQ * q < K);
      return k0 + KQ * q + KQ <= K;
    };
    auto load_w = [&](WChunk<RF, KQ> &w, int k0) {
      if constexpr (TILED) {
        load_wchunk_tiled(w, vr, mr, sr, fv, fm, fs, tlo(k0));
      } else {
        bool ok[RF];
        const bool whole = wok(k0, ok);
        uint32_t kv, km, ks;
        koff(k0, kv, km, ks);
        load_wchunk(w, vb, mb, sb, fv, fm, fs, vo, mo, so, ok, whole, kv, km, ks);
      }
    };
    auto ring_load = [&](int slot, int k0) {
      const uint32_t lo = tlo(k0);
      uint8_t *base = wring + slot * RSLOT + wave * (RF * RFB);
#pragma unroll
      for (int f = 0; f < RF; ++f) {
        uint8_t *fb = base + f * RFB;
        buffer_to_lds<16>(vr, fb, lo, fv[f]);
        if constexpr (PAIRED) {
          buffer_to_lds<4>(mr, fb + RV, lo >> 2, fm[f]);
        } else {
          buffer_to_lds<4>(mr, fb + RV, lo >> 1, fm[f]);
          buffer_to_lds<4>(mr, fb + RV + 256, (lo >> 1) + 4, fm[f]);
        }
        buffer_to_lds<2>(sr, fb + RV + RM, lo >> 3, fs[f]);
      }
    };
    // The item's first weight chunk is issued before the gather offsets
    // below (a dependent load), so that the two latencies overlap.  The
    // previous item ended on a barrier: the ring slots and registers are free.
    using FirstChunk = std::conditional_t<PAIRED, PChunk<RF>, WChunk<RF, KQ>>;
    FirstChunk w0;
    if constexpr (RING) {
      ring_load(0, 0);
      if (nk > 1) ring_load(1, KC);
    } else if constexpr (PAIRED) {
      load_pchunk(w0, vr, mr, sr, fv, fm, fs, tlo(0));
    } else {
      load_w(w0, 0);
    }

    // Token tile of a chunk: each 1 KB direct-to-LDS load of this wave
    // covers 64/UPR token rows; lane L fetches unit (L % UPR) ^ (row % UPR)
    // of its row, so that it lands in the swizzled slot mma_chunk reads.
    // Rows past the tile repeat the last routed row and positions past K
    // repeat the last 8; their products only reach unstored outputs or meet
    // zero weights.
    // Source row of each token-tile row this lane loads: the routed row, or
    // with a gather permutation the token perm[routed row] / k (dispatch
    // fused into the GEMM; an out-of-range entry reads token 0 and its
    // output row is written as zero, as a zero routed row would give).
    const int nrows = nft * MS;
    // element offsets from x (under 2^31: checked on the host), so that the
    // loads take x as a scalar base and a 32-bit lane offset
    uint32_t srow[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      srow[j] = 0;
      if constexpr (!ACT4) {
        const int r = tok0 + min((wave * BPW + j) * (64 / UPR) + lane / UPR, ntok - 1);
        int src = r;
        if (ROUTE || a.perm) {
          const int pi = perm_at(r);
          src = (pi >= 0 && pi < a.T * a.k) ? pi / a.k : 0;
        }
        srow[j] = (uint32_t)src * (uint32_t)K;
      }
    }
    // NVFP4 activations (W4A4): each chunk, thread tid stages one 32-position
    // block (16 code bytes and its E4M3 scale) of token-tile row a_tr: the
    // loads go to registers while the previous chunk computes, then the
    // block is decoded exactly to bf16 (E2M1 * E4M3 has at most six
    // significant bits) and written into the tile layout the MFMA loop
    // reads; the row's fp32 scale is applied in the epilogue.  Rows past the
    // routed ones repeat the last routed row, blocks past K are zero.
    constexpr int BPR = KC / 32;                      // blocks per row of a chunk
    static_assert(!ACT4 || BM * BPR <= WAVES * 64, "one activation block per thread and chunk");
    const int a_tr = tid / BPR, a_jb = tid - (tid / BPR) * BPR;
    const bool a_on = ACT4 && tid < BM * BPR && a_tr < nrows;
    const uint32_t nbk = (uint32_t)(K >> 5);
    uint32_t a_vo = 0, a_so = 0;
    if constexpr (ACT4) {
      int src = tok0 + min(a_tr, ntok - 1);
      if (ROUTE || a.perm) {
        const int pi = perm_at(src);
        src = (pi >= 0 && pi < a.T * a.k) ? pi / a.k : 0;
      }
      a_vo = (uint32_t)src * (uint32_t)(K >> 1) + (uint32_t)a_jb * 16u;
      a_so = (uint32_t)src * nbk + (uint32_t)a_jb;
    }
    const uint32_t arows = ACT4 ? (uint32_t)((ROUTE || a.perm) ? a.T : a.M) : 0u;
    const __amdgpu_buffer_rsrc_t acr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.aq_codes, 0, (int)(arows * (uint32_t)(K >> 1)), 0x20000);
    const __amdgpu_buffer_rsrc_t asr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)a.aq_scales, 0, (int)(arows * nbk), 0x20000);
    struct AReg {
      u32x4_t c;
      uint32_t s;
    };
    auto act_load = [&](AReg &r, int k0) {
      const uint32_t kb = (uint32_t)(k0 >> 5) + (uint32_t)a_jb;
      if (a_on && kb < nbk) {
        r.c = __builtin_amdgcn_raw_buffer_load_b128(acr, a_vo, (uint32_t)k0 >> 1, 0);
        r.s = __builtin_amdgcn_raw_buffer_load_b8(asr, a_so, (uint32_t)k0 >> 5, 0);
      } else {
        r.c = u32x4_t{0u, 0u, 0u, 0u};
        r.s = 0u;
      }
    };
    // Decode and LDS writes (asm: the writes must not wait for direct-to-LDS
    // weight loads still in flight; the caller waits for them before its
    // barrier).  4:8 weights: unit c of a row at slot c ^ (row % UPR), dword d
    // of a unit = positions 2d, 2d+1.  Paired weights: a 16-position unit u
    // (groups G, G') as its even half [G 0 2 4 6 | G' 0 2 4 6] at slot
    // (2u) ^ (row % UPR) and its odd half at slot (2u + 1) ^ (row % UPR).
    auto act_store = [&](uint16_t *buf, const AReg &r) {
      if (!a_on) return;
      const float sc = __builtin_amdgcn_cvt_f32_fp8(r.s, 0);
      const uint32_t rowb = lds_addr(buf + a_tr * KC);
      const uint32_t sw = (uint32_t)(a_tr & (UPR - 1));
      auto up = [&](float v) { return __float_as_uint(v * sc); };
      auto pk = [&](float lo, float hi) { return __builtin_amdgcn_perm(up(hi), up(lo), 0x07060302u); };
      auto wr = [&](uint32_t slot, uint32_t d0, uint32_t d1, uint32_t d2, uint32_t d3) {
        const u32x4_t v = {d0, d1, d2, d3};
        asm volatile("ds_write_b128 %0, %1" ::"v"(rowb + 16u * (slot ^ sw)), "v"(v) : "memory");
      };
      if constexpr (!PAIRED) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.c[i], 1.0f, 0);
          const f32x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.c[i], 1.0f, 1);
          const f32x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.c[i], 1.0f, 2);
          const f32x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(r.c[i], 1.0f, 3);
          wr(4u * (uint32_t)a_jb + (uint32_t)i, pk(p0[0], p0[1]), pk(p1[0], p1[1]),
             pk(p2[0], p2[1]), pk(p3[0], p3[1]));
        }
      } else {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const uint32_t G = r.c[2 * m], H = r.c[2 * m + 1];
          const f32x2_t g0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(G, 1.0f, 0);
          const f32x2_t g1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(G, 1.0f, 1);
          const f32x2_t g2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(G, 1.0f, 2);
          const f32x2_t g3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(G, 1.0f, 3);
          const f32x2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(H, 1.0f, 0);
          const f32x2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(H, 1.0f, 1);
          const f32x2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(H, 1.0f, 2);
          const f32x2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(H, 1.0f, 3);
          const uint32_t u = 2u * (uint32_t)a_jb + (uint32_t)m;
          wr(2u * u, pk(g0[0], g1[0]), pk(g2[0], g3[0]), pk(h0[0], h1[0]), pk(h2[0], h3[0]));
          wr(2u * u + 1u, pk(g0[1], g1[1]), pk(g2[1], g3[1]), pk(h0[1], h1[1]), pk(h2[1], h3[1]));
        }
      }
    };
    // 4:8 weights: the token loads are buffer loads to LDS.  The byte offset
    // of the lane's row and 16-byte unit is fixed for the item (VGPR), the
    // chunk's K offset is uniform (SGPR), so a whole chunk costs no vector
    // addressing (prefill-1t gate/up -1.6 %, prefill-30b -3 %, decode-1t
    // gate/up -3 %); a chunk that runs past K clamps each lane's unit to the
    // row's last 8 positions.  Paired weights keep the global form (2 %
    // faster there).
    uint32_t tvo[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int row = (wave * BPW + j) * (64 / UPR) + lane / UPR;
      tvo[j] = (srow[j] + (uint32_t)(((lane % UPR) ^ (row % UPR)) * 8)) * 2u;
    }
    auto load_tok = [&](uint16_t *buf, int k0) {
      const bool whole = k0 + KC <= K;
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        if ((wave * BPW + j) * (64 / UPR) >= nrows) break;   // fragment never read
        uint16_t *dst = buf + (wave * BPW + j) * 512;
        if (!PAIRED && whole) {
          buffer_to_lds<16>(xr, dst, tvo[j], (uint32_t)k0 * 2u);
          continue;
        }
        const int row = (wave * BPW + j) * (64 / UPR) + lane / UPR;
        const int c = (lane % UPR) ^ (row % UPR);
        const int kk = min(k0 + c * 8, K - 8);
        if constexpr (!PAIRED) {
          buffer_to_lds<16>(xr, dst, (srow[j] + (uint32_t)kk) * 2u, 0u);
        } else {
          __builtin_amdgcn_global_load_lds(
              (__attribute__((address_space(1))) void *)(a.x + (srow[j] + (uint32_t)kk)),
              (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
        }
      }
    };
    // Paired weights: the sparse MFMA contracts each 16-position unit in the
    // order [even positions | odd positions].  The direct-to-LDS loads above
    // move whole dwords (position pairs), so once this wave's loads have
    // landed (vmcnt(0): the count is per wave) every lane rewrites its own
    // 16-byte slot in place: the slot pair (P, P^1) of a unit holds its two
    // groups G, G' and becomes its even half and its odd half.  Lane L's
    // slot P = L % UPR holds logical unit-half h = (P ^ row) & 1, the same
    // for every 1 KB block of the lane, since a block starts at an even row
    // and covers 64 / UPR rows.  Both slots are read before either is
    // written: LDS instructions of one wave run in order.  The batched path
    // (four blocks per wave) leaves its writes in flight: every caller waits
    // (lgkmcnt(0), in asm,
    // which the compiler cannot drop as it can a fence's wait for LDS work it
    // does not know of) before its barrier.
    const int split_h = ((lane % UPR) ^ (lane / UPR)) & 1;
    const uint32_t split_sel = split_h ? 0x07060302u : 0x05040100u;
    auto split_tok = [&](uint16_t *buf) {
      if constexpr (BPW == 4) {
        if ((wave * BPW + BPW - 1) * (64 / UPR) < nrows) {
          // all four blocks loaded: every read first (one wait), then the
          // perms, then every write (block j sits 1 KB after block j-1); the
          // caller waits for the writes before its barrier.  One wait per
          // chunk instead of two per block: paired prefill-1t -1.4 % (gate/up)
          // and -2 % (down), prefill-30b -5 %.
          const uint32_t blk = lds_addr(buf + (wave * BPW) * 512);
          const uint32_t a_own = blk + 16u * lane, a_nbr = blk + 16u * (lane ^ 1);
          u32x4_t x0, y0, x1, y1, x2, y2, x3, y3;
          asm volatile(
              "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\t"
              "ds_read_b128 %2, %8 offset:1024\n\tds_read_b128 %3, %9 offset:1024\n\t"
              "ds_read_b128 %4, %8 offset:2048\n\tds_read_b128 %5, %9 offset:2048\n\t"
              "ds_read_b128 %6, %8 offset:3072\n\tds_read_b128 %7, %9 offset:3072\n\t"
              "s_waitcnt lgkmcnt(0)"
              : "=&v"(x0), "=&v"(y0), "=&v"(x1), "=&v"(y1), "=&v"(x2), "=&v"(y2), "=&v"(x3),
                "=&v"(y3)
              : "v"(a_own), "v"(a_nbr)
              : "memory");
          auto pk = [&](const u32x4_t &v) {
            u32x2_t r;
            r[0] = __builtin_amdgcn_perm(v[1], v[0], split_sel);
            r[1] = __builtin_amdgcn_perm(v[3], v[2], split_sel);
            return r;
          };
          const u32x2_t o0 = pk(x0), n0 = pk(y0), o1 = pk(x1), n1 = pk(y1), o2 = pk(x2),
                        n2 = pk(y2), o3 = pk(x3), n3 = pk(y3);
          const uint32_t w_own = a_own + 8u * split_h, w_nbr = a_own + 8u * (split_h ^ 1);
          asm volatile(
              "ds_write_b64 %0, %2\n\tds_write_b64 %1, %3\n\t"
              "ds_write_b64 %0, %4 offset:1024\n\tds_write_b64 %1, %5 offset:1024\n\t"
              "ds_write_b64 %0, %6 offset:2048\n\tds_write_b64 %1, %7 offset:2048\n\t"
              "ds_write_b64 %0, %8 offset:3072\n\tds_write_b64 %1, %9 offset:3072"
              :
              : "v"(w_own), "v"(w_nbr), "v"(o0), "v"(n0), "v"(o1), "v"(n1), "v"(o2), "v"(n2),
                "v"(o3), "v"(n3)
              : "memory");
          return;
        }
      }
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        if ((wave * BPW + j) * (64 / UPR) >= nrows) break;   // block never loaded
        // LDS accesses in asm with their own waits: the waitcnt pass cannot
        // tell this buffer from the weight ring still streaming in, and
        // would wait for the ring's loads (vmcnt) before these writes
        const uint32_t blk = lds_addr(buf + (wave * BPW + j) * 512);
        const uint32_t a_own = blk + 16u * lane, a_nbr = blk + 16u * (lane ^ 1);
        u32x4_t x, y;
        asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                     : "=&v"(x), "=&v"(y) : "v"(a_own), "v"(a_nbr) : "memory");
        // own group: dwords p0 p1; the neighbour's: p2 p3; G goes first
        u32x2_t own, nbr;
        own[0] = __builtin_amdgcn_perm(x[1], x[0], split_sel);
        own[1] = __builtin_amdgcn_perm(x[3], x[2], split_sel);
        nbr[0] = __builtin_amdgcn_perm(y[1], y[0], split_sel);
        nbr[1] = __builtin_amdgcn_perm(y[3], y[2], split_sel);
        asm volatile("ds_write_b64 %0, %1\n\tds_write_b64 %2, %3\n\ts_waitcnt lgkmcnt(0)"
                     :: "v"(a_own + 8u * split_h), "v"(own), "v"(a_own + 8u * (split_h ^ 1)), "v"(nbr)
                     : "memory");
      }
    };

    // One K loop + epilogue per path: full token tiles run without any
    // per-fragment test, partial tiles skip the empty fragments.  The
    // accumulators live inside each path, so they are never merged.
    auto run_item = [&](auto full_tag, auto nf_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
      constexpr int NF = decltype(nf_tag)::value;   // token fragments computed
      typename MF::C acc[RF][NF];
  #pragma unroll
      for (int f = 0; f < RF; ++f)
  #pragma unroll
        for (int t = 0; t < NF; ++t)
  #pragma unroll
          for (int i = 0; i < MF::NC; ++i) acc[f][t][i] = 0.f;

      if constexpr (RING) {
        // The ring is read with one asm block per fragment that waits for its
        // own reads (lgkmcnt): the waitcnt pass would otherwise make every
        // read of the ring wait for the slot still streaming in (vmcnt).
        const uint32_t ring0 = lds_addr(wring) + (uint32_t)(wave * (RF * RFB));
        using WC = std::conditional_t<PAIRED, PChunk<RF>, WChunk<RF, KQ>>;
        auto ring_read = [&](WC &w, int slot) {
          if constexpr (PAIRED && RF == 2) {
            // both fragments in one block with one wait (fragment 1 sits RFB
            // bytes after fragment 0)
            const uint32_t fb = ring0 + (uint32_t)(slot * RSLOT);
            const uint32_t av = fb + lane * 16, am = fb + RV + lane * 4, as = fb + RV + RM + lane * 4;
            u32x4_t v0, v1;
            uint32_t m0, m1, s0, s1;
            asm volatile("ds_read_b128 %0, %6\n\tds_read_b32 %1, %7\n\tds_read_u16 %2, %8\n\t"
                         "ds_read_b128 %3, %6 offset:%9\n\tds_read_b32 %4, %7 offset:%9\n\t"
                         "ds_read_u16 %5, %8 offset:%9\n\ts_waitcnt lgkmcnt(0)"
                         : "=&v"(v0), "=&v"(m0), "=&v"(s0), "=&v"(v1), "=&v"(m1), "=&v"(s1)
                         : "v"(av), "v"(am), "v"(as), "n"(RFB)
                         : "memory");
            w.w[0] = m0;
            w.w[1] = m1;
            w.s[0] = s0;
            w.s[1] = s1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              w.v[0][i] = v0[i];
              w.v[1][i] = v1[i];
            }
            return;
          }
#pragma unroll
          for (int f = 0; f < RF; ++f) {
            const uint32_t fb = ring0 + (uint32_t)(slot * RSLOT + f * RFB);
            const uint32_t av = fb + lane * 16, am = fb + RV + lane * 4, as = fb + RV + RM + lane * 4;
            u32x4_t v;
            uint32_t m0, m1 = 0, sc;
            if constexpr (PAIRED) {
              asm volatile("ds_read_b128 %0, %3\n\tds_read_b32 %1, %4\n\tds_read_u16 %2, %5\n\t"
                           "s_waitcnt lgkmcnt(0)"
                           : "=&v"(v), "=&v"(m0), "=&v"(sc) : "v"(av), "v"(am), "v"(as) : "memory");
              w.w[f] = m0;
            } else {
              asm volatile("ds_read_b128 %0, %4\n\tds_read_b32 %1, %5\n\t"
                           "ds_read_b32 %2, %5 offset:256\n\tds_read_u16 %3, %6\n\t"
                           "s_waitcnt lgkmcnt(0)"
                           : "=&v"(v), "=&v"(m0), "=&v"(m1), "=&v"(sc)
                           : "v"(av), "v"(am), "v"(as) : "memory");
              w.m[f][0] = m0;
              w.m[f][1] = m1;
            }
            w.v[f][0] = v[0];
            w.v[f][1] = v[1];
            w.v[f][2] = v[2];
            w.v[f][3] = v[3];
            w.s[f] = sc;
          }
        };
        AReg ar;
        if constexpr (ACT4) {
          act_load(ar, 0);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          act_store(tkA, ar);
        } else {
          load_tok(tkA, 0);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          if constexpr (PAIRED) split_tok(tkA);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        // One chunk: tokens of c + 1 and weights of c + 2 are issued in that
        // order, so waiting for all but the last RING_LOADS loads lands the
        // tokens (and, being older, the weights of c + 1) and leaves the
        // weights of c + 2 in flight.  A bare barrier: every LDS write this
        // chunk makes (split, ring) is covered by the explicit waits.
        auto chunk = [&](int c, int slot, const uint16_t *cur, uint16_t *nxt) {
          if (c + 1 < nk) {
            if constexpr (ACT4) act_load(ar, (c + 1) * KC);
            else load_tok(nxt, (c + 1) * KC);
          }
          if (c + 2 < nk) ring_load(slot == 0 ? 2 : slot - 1, (c + 2) * KC);
          WC wc;
          ring_read(wc, slot);
          if ((c + 1) * KC > K) {
            // segments past K were clamped to the last one: clear their
            // masks (4:8) or codes (paired)
            const bool ok = (uint32_t)((c * KC) >> 6) + (uint32_t)q < segs;
#pragma unroll
            for (int f = 0; f < RF; ++f) {
              if constexpr (PAIRED) {
#pragma unroll
                for (int i = 0; i < 4; ++i) wc.v[f][i] = ok ? wc.v[f][i] : 0u;
              } else {
#pragma unroll
                for (int i = 0; i < WChunk<RF, KQ>::MD; ++i) wc.m[f][i] = ok ? wc.m[f][i] : 0u;
              }
            }
          }
          if constexpr (PAIRED)
            mma_chunk_paired<MS, RF, NF, KC, FULL>(acc, cur, wc, nft, q, rl);
          else
            mma_chunk<MS, RF, NF, KC, FULL>(acc, cur, wc, lut, nft, q, rl);
          if (c + 2 < nk)
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(RING_LOADS) : "memory");
          else
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          if (c + 1 < nk) {
            if constexpr (ACT4) act_store(nxt, ar);
            else if constexpr (PAIRED) split_tok(nxt);
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          __builtin_amdgcn_s_barrier();
        };
        // slots cycle 0,1,2 and token buffers A,B: unrolled over the chunk
        // pair, the slot advances at run time
        int slot = 0;
        for (int c = 0; c < nk; c += 2) {
          chunk(c, slot, tkA, tkB);
          slot = slot == 2 ? 0 : slot + 1;
          if (c + 1 < nk) {
            chunk(c + 1, slot, tkB, tkA);
            slot = slot == 2 ? 0 : slot + 1;
          }
        }
      } else if constexpr (PAIRED) {
        PChunk<RF> wA = w0, wB;
        AReg ar;
        if constexpr (ACT4) {
          act_load(ar, 0);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          act_store(tkA, ar);
        } else {
          load_tok(tkA, 0);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          split_tok(tkA);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the split's writes
        __syncthreads();
        auto chunk = [&](int c, const uint16_t *cur, uint16_t *nxt, PChunk<RF> &wc,
                         PChunk<RF> &wn) {
          if (c + 1 < nk) {
            load_pchunk(wn, vr, mr, sr, fv, fm, fs, tlo((c + 1) * KC));
            if constexpr (ACT4) act_load(ar, (c + 1) * KC);
            else load_tok(nxt, (c + 1) * KC);
          }
          if ((c + 1) * KC > K) {
            // segments past K were clamped to the last one: zero their codes
            const bool ok = (uint32_t)((c * KC) >> 6) + (uint32_t)q < segs;
#pragma unroll
            for (int f = 0; f < RF; ++f)
#pragma unroll
              for (int i = 0; i < 4; ++i) wc.v[f][i] = ok ? wc.v[f][i] : 0u;
          }
          mma_chunk_paired<MS, RF, NF, KC, FULL>(acc, cur, wc, nft, q, rl);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          if (c + 1 < nk) {
            if constexpr (ACT4) act_store(nxt, ar);
            else split_tok(nxt);
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the split's writes
          __syncthreads();
        };
        for (int c = 0; c < nk; c += 2) {
          chunk(c, tkA, tkB, wA, wB);
          if (c + 1 < nk) chunk(c + 1, tkB, tkA, wB, wA);
        }
      } else {
        WChunk<RF, KQ> wA = w0, wB;
        AReg ar;
        if constexpr (ACT4) {
          act_load(ar, 0);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          act_store(tkA, ar);
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        } else {
          load_tok(tkA, 0);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        __syncthreads();
        // One chunk: prefetch chunk c + 1 into (nxt, wn), compute chunk c from
        // (cur, wc).  The two token buffers are distinct LDS objects, so the
        // reads of `cur` need not wait for the direct-to-LDS loads into `nxt`.
        auto chunk = [&](int c, const uint16_t *cur, uint16_t *nxt, WChunk<RF, KQ> &wc,
                         WChunk<RF, KQ> &wn) {
          if (c + 1 < nk) {
            load_w(wn, (c + 1) * KC);
            if constexpr (ACT4) act_load(ar, (c + 1) * KC);
            else load_tok(nxt, (c + 1) * KC);
          }
          if constexpr (TILED) {
            if ((c + 1) * KC > K) {
              // segments past K were clamped to the last one: clear their masks
              const bool ok = (uint32_t)((c * KC) >> 6) + (uint32_t)q < segs;
  #pragma unroll
              for (int f = 0; f < RF; ++f)
  #pragma unroll
                for (int i = 0; i < WChunk<RF, KQ>::MD; ++i) wc.m[f][i] = ok ? wc.m[f][i] : 0u;
            }
          }
          mma_chunk<MS, RF, NF, KC, FULL>(acc, cur, wc, lut, nft, q, rl);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          if constexpr (ACT4) {
            if (c + 1 < nk) act_store(nxt, ar);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          }
          __syncthreads();
        };
        for (int c = 0; c < nk; c += 2) {
          chunk(c, tkA, tkB, wA, wB);
          if (c + 1 < nk) chunk(c + 1, tkB, tkA, wB, wA);
        }

      }

      // Epilogue.  Accumulator element r of a lane holds weight row
      // (r/4)*4*LG + 4q + r%4 of its fragment for token rl of its token
      // fragment: four consecutive rows per group of four, one 8-byte store.
      const float ge = a.gscale[e];
  #pragma unroll
      for (int t = 0; t < NF; ++t) {
        const int trow = t * MS + rl;
        if (trow >= ntok) continue;
        size_t out_r = (size_t)(tok0 + trow);
        bool keep = true;
        int src = (int)out_r;   // the token row of the activations
        if (ROUTE || a.perm) {
          const int pi = perm_at((int)out_r);
          keep = pi >= 0 && pi < a.T * a.k;
          src = keep ? pi / a.k : 0;
          if (a.flat) {   // scatter to the flat position; no destination: no store
            if (!keep) continue;
            out_r = (size_t)pi;
          }
        }
        // W4A4: the activation row's fp32 scale joins the expert's
        const float g = ACT4 ? ge * a.aq_g[src] : ge;
  #pragma unroll
        for (int r4 = 0; r4 < MF::NC / 4; ++r4) {
          const int roff = r4 * 4 * LG + 4 * q;
          if constexpr (!SWIGLU) {
  #pragma unroll
            for (int f = 0; f < RF; ++f) {
              if (!fval[f]) continue;
              const typename MF::C &c = acc[f][t];
              uint2 o;
              o.x = keep ? pack_bf16x2(g * c[4 * r4 + 0], g * c[4 * r4 + 1]) : 0u;
              o.y = keep ? pack_bf16x2(g * c[4 * r4 + 2], g * c[4 * r4 + 3]) : 0u;
              *reinterpret_cast<uint2 *>(a.y + out_r * N + (frow[f] + roff)) = o;
            }
          } else {
  #pragma unroll
            for (int f = 0; f < RF / 2; ++f) {
              if (!fval[f]) continue;
              const typename MF::C &gt = acc[f][t], &up = acc[f + RF / 2][t];
              float h[4];
  #pragma unroll
              for (int i = 0; i < 4; ++i) h[i] = silu_f32(g * gt[4 * r4 + i]) * (g * up[4 * r4 + i]);
              uint2 o;
              o.x = keep ? pack_bf16x2(h[0], h[1]) : 0u;
              o.y = keep ? pack_bf16x2(h[2], h[3]) : 0u;
              *reinterpret_cast<uint2 *>(a.y + out_r * half + (frow[f] + roff)) = o;
            }
          }
        }
      }
    };
    // The contraction tiles take partial token tiles on a K loop of their
    // own per fragment count (per-fragment branches inside one loop made
    // the ring tile's accumulators spill, and cost the 4:8 tile 1-3 %); the
    // streaming tiles test the fragments at run time.
    using std::integral_constant;
    if constexpr (RING || MS == 32) {
      if (nft <= 1)
        run_item(std::true_type{}, integral_constant<int, 1>{});
      else if (nft == 2)
        run_item(std::true_type{}, integral_constant<int, (TF < 2 ? TF : 2)>{});
      else if (nft == 3)
        run_item(std::true_type{}, integral_constant<int, (TF < 3 ? TF : 3)>{});
      else
        run_item(std::true_type{}, integral_constant<int, TF>{});
    } else if (nft == TF) {
      run_item(std::true_type{}, integral_constant<int, TF>{});
    } else {
      run_item(std::false_type{}, integral_constant<int, TF>{});
    }
  }
}

template <int WAVES, int MS, int RF, int TF, int KC, bool SWIGLU, int FMT, bool ROUTE = false,
          bool ACT4 = false>
static moesq_status_t launch_one(SpgemmArgs a, hipStream_t stream) {
  constexpr int BM = TF * MS, BN = WAVES * RF * MS;
  auto kern = spgemm_kernel<WAVES, MS, RF, TF, KC, SWIGLU, FMT, ROUTE, ACT4>;
  a.row_tiles = SWIGLU ? (a.N / 2 + BN / 2 - 1) / (BN / 2) : (a.N + BN - 1) / BN;
  // schedule arrays, then with fused routing its offsets and permutation
  const size_t dyn = spgemm_sched_bytes(a.E) + (ROUTE ? (size_t)(a.E + 1 + a.M) * 4 : 0);
  // upper bound of the item count: every expert may hold one partial tile
  const long long items = ((long long)a.M / BM + std::min(a.E, a.M)) * a.row_tiles;
  // workgroups per CU for this dynamic LDS size (cached per device and size)
  static thread_local int occ_dev = -1, occ = 1;
  static thread_local size_t occ_dyn = 0;
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (occ_dev != dev || occ_dyn != dyn) {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, kern, WAVES * 64, dyn) != hipSuccess ||
        o < 1)
      o = 1;
    occ = o;
    occ_dev = dev;
    occ_dyn = dyn;
  }
  long long grid = (long long)device_cu_count() * occ;
  if (grid > items) grid = items;
  grid = (grid + 7) & ~7ll;          // XCD-major item spreading needs a multiple of 8
  if (grid < 8) grid = 8;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(WAVES * 64), dyn, stream, a);
  return launch_status("moesq_grouped_spgemm");
}

// Tile choice.  The streaming tile: 16x16x32 MFMAs on 32 weight rows per
// wave, 256-position chunks.  The contraction tile: 32x32x16 MFMAs on 64
// weight rows x 128 tokens per wave, two waves per SIMD, so that every
// decoded weight feeds 4 MFMAs of 32 tokens.  A sweep over active experts x
// rows per expert puts their crossover between 32 and 64 rows per expert.
// Up to 4 rows per expert on average (decode batches) one launch runs the
// streaming tile with one 16-token fragment in 4-wave workgroups of 128
// weight rows (four per CU): such batches have few (expert, row tile)
// items, and items half as large spread them more evenly over the CUs
// (30B-class decode -17 %); an expert with more rows takes several token
// tiles.  Larger GEMMs (at least ~5e11 multiply-adds) make three launches
// that split the experts by their own row counts, which only the device
// knows: experts of up to 16 rows on the one-fragment streaming tile, up
// to 32 on the 8-wave streaming tile with two fragments (32 tokens), larger
// ones on the contraction tile
// (trillion-class prefill: gate/up -1 to -3 % on 4:8 weights, -8 % on
// paired ones).
// Shorter ones (30B-class prefill, 1e11) lose more to the second launch
// than they gain (+5 to 8 %) and make one launch, the streaming tile up to
// 32 rows per expert on average, else the contraction tile.  Fragments are whole: the 32-row tile needs the output
// rows (N, or N/2 under SwiGLU) to be a multiple of 32, else one launch of
// the streaming tile takes every expert.
// Paired weights take the same tiles on the sparse MFMA (16x16x64 and
// 32x32x32): the same token and weight-row counts per wave, each step
// contracting twice the dense K.
template <int FMT, bool ACT4 = false>
static moesq_status_t launch_layout(SpgemmArgs a, bool swiglu, hipStream_t stream) {
  const int out_rows = swiglu ? a.N / 2 : a.N;
  a.rows_lo = 0;
  a.rows_hi = INT_MAX;
  // decode batches: one launch of the one-fragment streaming tile
  if ((long long)a.M <= 4ll * a.E)
    return swiglu ? launch_one<4, 16, 2, 1, 256, true, FMT, false, ACT4>(a, stream)
                  : launch_one<4, 16, 2, 1, 256, false, FMT, false, ACT4>(a, stream);
  if (out_rows % 32 != 0)   // the 32-row tile needs whole 32-row fragments
    return swiglu ? launch_one<8, 16, 2, 2, 256, true, FMT, false, ACT4>(a, stream)
                  : launch_one<8, 16, 2, 2, 256, false, FMT, false, ACT4>(a, stream);
  // A GEMM under ~5e11 multiply-adds is too short to pay for a second
  // launch: one launch, its tile from the average rows per expert.
  if ((double)a.M * a.N * a.K < 5.5e11) {
    if ((long long)a.M <= 32ll * a.E)
      return swiglu ? launch_one<8, 16, 2, 2, 256, true, FMT, false, ACT4>(a, stream)
                    : launch_one<8, 16, 2, 2, 256, false, FMT, false, ACT4>(a, stream);
    return swiglu ? launch_one<8, 32, 2, 4, 128, true, FMT, false, ACT4>(a, stream)
                  : launch_one<8, 32, 2, 4, 128, false, FMT, false, ACT4>(a, stream);
  }
  // otherwise launches split by each expert's own row count (read on the
  // device): up to 16 rows the one-fragment streaming tile, up to 32 the
  // two-fragment one, above that the contraction tile
  a.rows_hi = 16;
  moesq_status_t st = swiglu ? launch_one<4, 16, 2, 1, 256, true, FMT, false, ACT4>(a, stream)
                             : launch_one<4, 16, 2, 1, 256, false, FMT, false, ACT4>(a, stream);
  if (st != MOESQ_OK) return st;
  a.rows_lo = 16;
  a.rows_hi = 32;
  st = swiglu ? launch_one<8, 16, 2, 2, 256, true, FMT, false, ACT4>(a, stream)
              : launch_one<8, 16, 2, 2, 256, false, FMT, false, ACT4>(a, stream);
  if (st != MOESQ_OK) return st;
  a.rows_lo = 32;
  a.rows_hi = INT_MAX;
  return swiglu ? launch_one<8, 32, 2, 4, 128, true, FMT, false, ACT4>(a, stream)
                : launch_one<8, 32, 2, 4, 128, false, FMT, false, ACT4>(a, stream);
}

static moesq_status_t launch_spgemm(const SpgemmArgs &a, bool swiglu, int layout,
                                    hipStream_t stream, bool act4 = false) {
  if (act4) {
    switch (layout) {
      case MOESQ_LAYOUT_TILED: return launch_layout<FMT_TILED, true>(a, swiglu, stream);
      case MOESQ_LAYOUT_PAIRED_TILED: return launch_layout<FMT_PAIRED, true>(a, swiglu, stream);
      default: return launch_layout<FMT_CANONICAL, true>(a, swiglu, stream);
    }
  }
  switch (layout) {
    case MOESQ_LAYOUT_TILED: return launch_layout<FMT_TILED>(a, swiglu, stream);
    case MOESQ_LAYOUT_PAIRED_TILED: return launch_layout<FMT_PAIRED>(a, swiglu, stream);
    default: return launch_layout<FMT_CANONICAL>(a, swiglu, stream);
  }
}

static moesq_status_t check_weights(const moesq_weights_t *w, const char *who) {
  if (!w) return fail(MOESQ_ERR_NULL, std::string(who) + ": weight descriptor is NULL");
  if (w->layout == MOESQ_LAYOUT_PAIRED)
    return fail(MOESQ_ERR_LAYOUT, std::string(who) +
                                      ": paired weights must be tiled first (moesq_tile_weights)");
  if (w->layout != MOESQ_LAYOUT_CANONICAL && w->layout != MOESQ_LAYOUT_TILED &&
      w->layout != MOESQ_LAYOUT_PAIRED_TILED)
    return fail(MOESQ_ERR_LAYOUT, std::string(who) + ": unknown weight layout");
  if (w->layout != MOESQ_LAYOUT_CANONICAL && (w->N % 32 || w->K % 64))
    return fail(MOESQ_ERR_SHAPE, std::string(who) + ": tiled layout needs N % 32 == 0, K % 64 == 0");
  if (!w->values || !w->masks || !w->scales || !w->global_scale)
    return fail(MOESQ_ERR_NULL, std::string(who) + ": NULL weight buffer");
  if (w->E < 1 || w->E > MOESQ_MAX_EXPERTS)
    return fail(MOESQ_ERR_SHAPE, std::string(who) + ": E must be in [1, " +
                                     std::to_string(MOESQ_MAX_EXPERTS) + "]");
  if (w->N < 16 || w->N % 16)
    return fail(MOESQ_ERR_SHAPE, std::string(who) + ": N must be a positive multiple of 16");
  if (w->K < 32 || w->K % 32)
    return fail(MOESQ_ERR_SHAPE, std::string(who) + ": K must be a positive multiple of 32");
  if ((long long)w->N * w->K / 4 > 0x7fffffffll)
    return fail(MOESQ_ERR_SHAPE, std::string(who) + ": one expert's value array must stay under 2 GiB");
  return MOESQ_OK;
}

}  // namespace moesq

using namespace moesq;

extern "C" size_t moesq_spgemm_workspace_bytes(int32_t, const moesq_weights_t *) { return 0; }

static moesq_status_t spgemm_entry(const char *who, const uint16_t *x, const int32_t *perm, int32_t T,
                                   int32_t k, const int32_t *expert_offsets, int32_t M,
                                   const moesq_weights_t *w, int32_t epilogue, uint16_t *y,
                                   hipStream_t stream, const moesq_act4_t *xq = nullptr) {
  clear_error();
  moesq_status_t st = check_weights(w, who);
  if (st != MOESQ_OK) return st;
  const bool flat = (epilogue & MOESQ_OUT_FLAT) != 0;
  epilogue &= ~MOESQ_OUT_FLAT;
  if (epilogue != MOESQ_EPI_NONE && epilogue != MOESQ_EPI_SWIGLU)
    return fail(MOESQ_ERR_ARG, std::string(who) + ": unknown epilogue");
  if (flat && !perm)
    return fail(MOESQ_ERR_ARG, std::string(who) + ": MOESQ_OUT_FLAT needs the gather permutation");
  if (epilogue == MOESQ_EPI_SWIGLU && w->N % 32)
    return fail(MOESQ_ERR_SHAPE, std::string(who) + ": SwiGLU needs N % 32 == 0");
  if (M < 0) return fail(MOESQ_ERR_SHAPE, std::string(who) + ": M must be >= 0");
  if (!expert_offsets) return fail(MOESQ_ERR_NULL, std::string(who) + ": expert_offsets is NULL");
  if (M == 0) return MOESQ_OK;
  if ((!x && !xq) || !y) return fail(MOESQ_ERR_NULL, std::string(who) + ": NULL input or output rows");
  // token rows are addressed by 32-bit element offsets
  if ((long long)(perm ? T : M) * w->K > 0x7fffffffll)
    return fail(MOESQ_ERR_SHAPE, std::string(who) + ": rows of x times K must stay under 2^31");
  if (xq) {
    if (!xq->codes || !xq->scales || !xq->row_scale)
      return fail(MOESQ_ERR_NULL, std::string(who) + ": NULL activation codes, scales or row scales");
    if (xq->K != w->K)
      return fail(MOESQ_ERR_SHAPE, std::string(who) + ": activation K differs from the weights' K");
    if (xq->rows != (perm ? T : M))
      return fail(MOESQ_ERR_SHAPE, std::string(who) + ": activation rows must be T with a gather "
                                                      "permutation, else M");
  }
  SpgemmArgs a{};
  a.x = x;
  a.perm = perm;
  a.T = T;
  a.k = k;
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
  a.flat = flat;
  if (xq) {
    a.aq_codes = xq->codes;
    a.aq_scales = xq->scales;
    a.aq_g = xq->row_scale;
  }
  return launch_spgemm(a, epilogue == MOESQ_EPI_SWIGLU, w->layout, stream, xq != nullptr);
}

extern "C" moesq_status_t moesq_grouped_spgemm(const uint16_t *x_routed,
                                               const int32_t *expert_offsets, int32_t M,
                                               const moesq_weights_t *w, int32_t epilogue,
                                               uint16_t *y, void *ws, size_t ws_bytes,
                                               hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  return spgemm_entry("moesq_grouped_spgemm", x_routed, nullptr, 0, 1, expert_offsets, M, w,
                      epilogue, y, stream);
}

// Fused routing + dispatch + grouped GEMM of a decode batch.
template <int FMT>
static moesq_status_t launch_routed(const SpgemmArgs &a, bool swiglu, hipStream_t stream) {
  return swiglu ? launch_one<4, 16, 2, 1, 256, true, FMT, true>(a, stream)
                : launch_one<4, 16, 2, 1, 256, false, FMT, true>(a, stream);
}

extern "C" moesq_status_t moesq_route_grouped_spgemm(const int32_t *topk_ids, const uint16_t *x,
                                                     int32_t T, int32_t k,
                                                     const moesq_weights_t *w, int32_t epilogue,
                                                     uint16_t *y, int32_t *expert_offsets,
                                                     int32_t *perm, int32_t *inv_perm,
                                                     hipStream_t stream) {
  static const char *who = "moesq_route_grouped_spgemm";
  clear_error();
  moesq_status_t st = check_weights(w, who);
  if (st != MOESQ_OK) return st;
  if (T < 0 || k < 1 || (long long)T * k > 0x7fffffffll)
    return fail(MOESQ_ERR_SHAPE, std::string(who) + ": need T >= 0, k >= 1, T*k < 2^31");
  if (k > w->E) return fail(MOESQ_ERR_SHAPE, std::string(who) + ": need k <= E");
  const int32_t epi = epilogue & ~MOESQ_OUT_FLAT;
  if (epi != MOESQ_EPI_NONE && epi != MOESQ_EPI_SWIGLU)
    return fail(MOESQ_ERR_ARG, std::string(who) + ": unknown epilogue");
  if (epi == MOESQ_EPI_SWIGLU && w->N % 32)
    return fail(MOESQ_ERR_SHAPE, std::string(who) + ": SwiGLU needs N % 32 == 0");
  if (!expert_offsets) return fail(MOESQ_ERR_NULL, std::string(who) + ": expert_offsets is NULL");
  const int M = T * k;
  if (M > 0 && (!topk_ids || !x || !y || !perm || !inv_perm))
    return fail(MOESQ_ERR_NULL,
                std::string(who) + ": NULL ids, tokens, output rows or routing output");
  if ((long long)T * w->K > 0x7fffffffll)
    return fail(MOESQ_ERR_SHAPE, std::string(who) + ": rows of x times K must stay under 2^31");
  if (M == 0 || M > MOESQ_FUSED_ROUTE_MAX_ROWS || (long long)M > 4ll * w->E) {
    // not a decode batch: the plan by moesq_route, then the gather GEMM
    st = moesq_route(topk_ids, T, k, w->E, expert_offsets, perm, inv_perm, nullptr, 0, stream);
    if (st != MOESQ_OK) return st;
    return moesq_grouped_spgemm_gather(x, perm, T, k, expert_offsets, w, epilogue, y, nullptr,
                                       0, stream);
  }
  SpgemmArgs a{};
  a.x = x;
  a.perm = nullptr;
  a.T = T;
  a.k = k;
  a.offsets = nullptr;
  a.values = w->values;
  a.masks = w->masks;
  a.scales = w->scales;
  a.gscale = w->global_scale;
  a.y = y;
  a.M = M;
  a.E = w->E;
  a.N = w->N;
  a.K = w->K;
  a.rows_lo = 0;
  a.rows_hi = INT_MAX;
  a.ids = topk_ids;
  a.route_offsets = expert_offsets;
  a.route_perm = perm;
  a.route_inv = inv_perm;
  a.flat = (epilogue & MOESQ_OUT_FLAT) != 0;
  const bool sw = epi == MOESQ_EPI_SWIGLU;
  switch (w->layout) {
    case MOESQ_LAYOUT_TILED: return launch_routed<FMT_TILED>(a, sw, stream);
    case MOESQ_LAYOUT_PAIRED_TILED: return launch_routed<FMT_PAIRED>(a, sw, stream);
    default: return launch_routed<FMT_CANONICAL>(a, sw, stream);
  }
}

extern "C" moesq_status_t moesq_grouped_spgemm_gather(const uint16_t *x, const int32_t *perm,
                                                      int32_t T, int32_t k,
                                                      const int32_t *expert_offsets,
                                                      const moesq_weights_t *w, int32_t epilogue,
                                                      uint16_t *y, void *ws, size_t ws_bytes,
                                                      hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  if (T < 0 || k < 1 || (long long)T * k > 0x7fffffffll)
    return fail(MOESQ_ERR_SHAPE, "moesq_grouped_spgemm_gather: need T >= 0, k >= 1, T*k < 2^31");
  if (T > 0 && !perm) return fail(MOESQ_ERR_NULL, "moesq_grouped_spgemm_gather: perm is NULL");
  return spgemm_entry("moesq_grouped_spgemm_gather", x, perm, T, k, expert_offsets, T * k, w,
                      epilogue, y, stream);
}

extern "C" moesq_status_t moesq_grouped_spgemm_act4(const moesq_act4_t *x, const int32_t *perm,
                                                    int32_t T, int32_t k,
                                                    const int32_t *expert_offsets, int32_t M,
                                                    const moesq_weights_t *w, int32_t epilogue,
                                                    uint16_t *y, hipStream_t stream) {
  static const char *who = "moesq_grouped_spgemm_act4";
  clear_error();
  if (!x) return fail(MOESQ_ERR_NULL, std::string(who) + ": activation descriptor is NULL");
  if (perm) {
    if (T < 0 || k < 1 || (long long)T * k > 0x7fffffffll)
      return fail(MOESQ_ERR_SHAPE, std::string(who) + ": need T >= 0, k >= 1, T*k < 2^31");
    if ((long long)T * k != M)
      return fail(MOESQ_ERR_SHAPE, std::string(who) + ": with a gather permutation M must be T*k");
  }
  return spgemm_entry(who, nullptr, perm, T, k, expert_offsets, M, w, epilogue, y, stream, x);
}
