/*
 * moesq.h -- C ABI of the grouped 4:8 sparse-FP4 expert GEMM library
 * (libmoesq.so, built for AMD Instinct MI355X / gfx950).
 *
 * Method: Hardware-Native Joint Sparse-Quantization for Trillion-Scale
 * Mixture-of-Experts (paper summary page).  The library runs the expert half
 * of a MoE layer whose expert weights are stored 4:8 semi-structured sparse
 * with E2M1 (FP4) values and E4M3 block scales:
 *
 *   route      expert offsets + stable gather permutation      ("3.4 Implementation details":
 *                                                               one launch covers every
 *                                                               routing-dependent expert problem)
 *   permute    dispatch: gather routed token rows               ("D.1 Implementation details")
 *   grouped_spgemm  Y = X_routed * W_e^T for every expert, the  ("3.4 Implementation details",
 *              weights decoded in registers, optional SwiGLU    "A Sparse-quantized representation",
 *              epilogue                                         "D.1 Implementation details")
 *   unpermute  combine: back to token order, optionally         ("D.1", "D.3 End-to-end serving
 *              weighted by the router                            benchmark")
 *   pack_weights  compress dense fp32 experts into the format   ("3.4 Implementation details":
 *                                                               FP4 codes, sparsity metadata,
 *                                                               a scale for each 32 weights)
 *
 * Conventions (every call):
 *   - Pointers are DEVICE pointers unless marked "host".  bf16 tensors are
 *     passed as uint16_t (raw bf16 bits).  All tensors are dense row-major.
 *   - The caller owns every buffer.  The library allocates and frees no
 *     device memory, never synchronises the stream, and enqueues all work on
 *     `stream` (0 = the null stream).  (Exception: the debug call
 *     moesq_validate.)
 *   - A call checks its arguments on the host first; on a bad argument it
 *     returns an error and launches nothing.  A failed launch returns
 *     MOESQ_ERR_HIP.  moesq_last_error() gives a detail string for the last
 *     error of the calling thread.
 *   - Kernels are memory-safe for any bytes in the inputs: out-of-range ids,
 *     offsets or permutation entries are clamped or skipped, never
 *     dereferenced.  Results for such inputs are unspecified.
 *   - Calls that share buffers and overlap on different streams race; calls
 *     on one stream run in order.
 */
#ifndef MOESQ_H
#define MOESQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOESQ_OK = 0,
  MOESQ_ERR_NULL = -1,      /* a required pointer is NULL                     */
  MOESQ_ERR_SHAPE = -2,     /* a size or count is outside the supported range  */
  MOESQ_ERR_WORKSPACE = -3, /* workspace missing or smaller than required      */
  MOESQ_ERR_LAYOUT = -4,    /* unknown weight layout                           */
  MOESQ_ERR_HIP = -5,       /* a HIP runtime call or kernel launch failed      */
  MOESQ_ERR_ARG = -6        /* any other invalid argument                      */
} moesq_status_t;

typedef enum {
  MOESQ_EPI_NONE = 0,   /* y[r][n] = bf16(g_e * acc[r][n])                              */
  MOESQ_EPI_SWIGLU = 1  /* y[r][c] = bf16(silu(g_e*acc[r][c]) * g_e*acc[r][c+N/2]), c<N/2 */
} moesq_epilogue_t;

/*
 * Output-order flag, OR-ed into the epilogue argument of
 * moesq_grouped_spgemm_gather and moesq_route_grouped_spgemm: result row r
 * (routed order) is stored at y[perm[r]], i.e. y comes out in flat order
 * t*k + j, the order moesq_unpermute without weights produces from the
 * routed rows -- the scatter after the expert GEMM fused into its epilogue
 * ("D.1 Implementation details": the serving kernels fuse dispatch and
 * scatter with the first expert GEMM).  Same values, bit for bit; rows r
 * whose perm[r] is outside [0, T*k) are not stored anywhere, so with a
 * valid routing (perm a permutation of [0, T*k)) every row of y is written
 * exactly once.  moesq_grouped_spgemm (no permutation) rejects the flag with
 * MOESQ_ERR_ARG.
 */
#define MOESQ_OUT_FLAT 0x100

#define MOESQ_LAYOUT_CANONICAL 0
#define MOESQ_LAYOUT_TILED 1
#define MOESQ_LAYOUT_PAIRED 2
#define MOESQ_LAYOUT_PAIRED_TILED 3

/* Limits of this build. */
#define MOESQ_MAX_EXPERTS 1024
/* Largest T*k that moesq_route_grouped_spgemm routes inside the GEMM launch. */
#define MOESQ_FUSED_ROUTE_MAX_ROWS 1024

/*
 * Compressed expert weights, canonical layout.  For expert e (0 <= e < E),
 * W_e is N x K (output features x contraction), K % 32 == 0.  Source of the
 * format: "A Sparse-quantized representation" (groups of eight keep four
 * values; 16 kept values share one scale; zero is on the grid) and "Storage
 * layout"; this library stores an unconstrained 8-bit mask per group, i.e.
 * 13/32 byte per logical weight.
 *
 *   values [E][N][K/4]  E2M1 codes, two per byte.  The four kept codes of a
 *                       group of 8 come in ascending K position; the lower
 *                       position sits in the low nibble.
 *   masks  [E][N][K/8]  bit i set <=> position 8*g+i of group g is kept.
 *                       Exactly four bits must be set (caller contract).
 *   scales [E][N][K/32] E4M3 block scale of positions [32b, 32b+32).
 *   global_scale [E]    fp32 scale of the whole expert matrix.
 *
 *   W_e[n][8g+i] = E2M1(code_j) * E4M3(scale_b) * global_scale[e] at the j-th
 *   set bit i of mask byte g, and 0 at cleared bits.
 *
 * The struct itself is a host object; its pointers are device pointers.
 * Buffers are read-only to the library except in moesq_pack_weights.
 */
typedef struct {
  const uint8_t *values;
  const uint8_t *masks;
  const uint8_t *scales;
  const float *global_scale;
  int32_t E, N, K;
  int32_t layout; /* MOESQ_LAYOUT_CANONICAL, _TILED, _PAIRED or _PAIRED_TILED */
} moesq_weights_t;

/*
 * MOESQ_LAYOUT_TILED: the same bytes as the canonical layout, permuted so
 * that the GEMM's loads are whole cache lines.  Needs N % 32 == 0 and
 * K % 64 == 0.  For expert e, row n = 32*b + r (0 <= r < 32) and segment
 * j = k/64 (64 logical weights = 8 groups = 2 scale blocks):
 *
 *   values [E][N/32][K/64][32][16]  the 16 value bytes of row n for k in [64j, 64j+64)
 *   masks  [E][N/32][K/64][32][8]   its 8 mask bytes
 *   scales [E][N/32][K/64][32][2]   its 2 scale bytes
 *
 * Inside a segment the byte order is the canonical one.  Sizes per array
 * equal the canonical sizes.
 */

/*
 * MOESQ_LAYOUT_PAIRED: the pages' paired 4:8 format ("A Sparse-quantized
 * representation": each group of eight keeps two of its four adjacent pairs,
 * six patterns; "Storage layout": per group its four kept FP4 codes and
 * the index of its pattern, per 32 weights one unsigned E4M3 scale, 2.75
 * bits per weight).  The `masks` pointer carries the pattern indices:
 *
 *   values [E][N][K/4]   as the canonical layout (four kept codes per group,
 *                        ascending position, lower one in the low nibble)
 *   masks  [E][N][K/16]  pattern index p of group g in byte g/2, the even
 *                        group in the low nibble.  p in [0, 6) numbers the
 *                        kept pair couples (0,1) (0,2) (0,3) (1,2) (1,3) (2,3),
 *                        pair i being positions 2i and 2i+1 (caller contract:
 *                        p < 6).
 *   scales, global_scale as the canonical layout.
 *
 * MOESQ_LAYOUT_PAIRED_TILED: the GEMM's layout of paired weights (N % 32 == 0,
 * K % 64 == 0), produced by moesq_tile_weights.  Segments as in
 * MOESQ_LAYOUT_TILED; a "unit" u (0..3) of a row's segment is its groups
 * G = 2u and G' = 2u+1, read as the windows [G even positions, G' even,
 * G odd, G' odd] (positions 0,2,4,6 / 1,3,5,7 of a group):
 *
 *   values [E][N/32][K/64][32][16]  dword u: eight E2M1 codes in nibbles 0..7
 *                                   = G v0, G v2, G' v0, G' v2, G v1, G v3,
 *                                   G' v1, G' v3 (v0..v3: the group's kept
 *                                   codes in ascending position)
 *   masks  [E][N/32][K/64][32][4]   byte u: w(G) | w(G') << 4, where
 *                                   w = i | j << 2 for kept pairs i < j
 *   scales [E][N/32][K/64][32][2]   as MOESQ_LAYOUT_TILED
 *
 * Array sizes equal those of MOESQ_LAYOUT_PAIRED.
 */

/*
 * Routing plan (stable counting sort of the flat top-k ids).
 *   topk_ids        [T*k] int32, flat index i = t*k + j; ids in [0, E).
 *   expert_offsets  [E+1] int32 out: offsets[e] = first routed row of expert e
 *                   (the number of valid ids below e); offsets[E] = T*k.
 *   perm            [T*k] int32 out: perm[r] = flat index i of routed row r;
 *                   rows are ordered by (expert, i), so the order is stable.
 *   inv_perm        [T*k] int32 out: inv_perm[perm[r]] = r.
 *   ws, ws_bytes    workspace; moesq_route_workspace_bytes() bytes (may be 0).
 * Limits: 1 <= E <= MOESQ_MAX_EXPERTS, 1 <= k <= E, T >= 0, T*k < 2^31.
 * Ids outside [0, E) are not routed: they get inv_perm = -1 and are left out
 * of the offsets (offsets[E] then counts only valid ids).
 * Results are bit-identical on every run.
 */
moesq_status_t moesq_route(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E,
                           int32_t *expert_offsets, int32_t *perm, int32_t *inv_perm,
                           void *ws, size_t ws_bytes, hipStream_t stream);
size_t moesq_route_workspace_bytes(int32_t T, int32_t k, int32_t E);

/*
 * moesq_route for callers that cannot allocate device memory: code under HIP
 * graph capture that must not call hipMalloc, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, results and limits as moesq_route,
 * bit for bit, without the workspace: when the ids need the block counts
 * (moesq_route_workspace_bytes(T, k, E) > 0) they go to a scratch array of
 * MOESQ_ROUTE_SCRATCH_BYTES that the library holds in device memory, one per
 * device, from the device's first call until the process ends.  The call
 * allocates nothing (no hipMalloc, no allocating library routine).
 *   Returns MOESQ_ERR_SHAPE, launching nothing, when the counts need more
 *   than MOESQ_ROUTE_SCRATCH_BYTES (for example E = 384 above about 1.4
 *   million ids, E = 1024 above 524,288 ids); moesq_route with a workspace
 *   takes those.
 * Every call on one device shares that device's scratch: calls that overlap
 * in time on one device (different streams, or graphs replayed
 * concurrently) race and give unspecified plans.  The scratch needs no
 * clearing: each call writes every count it reads.
 */
#define MOESQ_ROUTE_SCRATCH_BYTES ((size_t)4 << 20)
moesq_status_t moesq_route_noalloc(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E,
                                   int32_t *expert_offsets, int32_t *perm, int32_t *inv_perm,
                                   hipStream_t stream);

/*
 * Dispatch: x_routed[r][:] = x[perm[r] / k][:].
 *   x         [T][K] bf16;  perm [T*k] int32 (from moesq_route);
 *   x_routed  [T*k][K] bf16 out.  Rows with perm[r] outside [0, T*k) are zero.
 * Limits: K % 8 == 0, K > 0.
 */
moesq_status_t moesq_permute(const uint16_t *x, const int32_t *perm, int32_t T, int32_t k,
                             int32_t K, uint16_t *x_routed, hipStream_t stream);

/*
 * Grouped sparse GEMM over all experts in one call (one kernel launch, or
 * for large calls three: experts of up to 16, up to 32 and more rows on
 * different tilings, split on the device):
 *   for every expert e and routed row r in [offsets[e], offsets[e+1]):
 *     acc[r][n] = sum_k x_routed[r][k] * W~_e[n][k]   (fp32 accumulation, the
 *                 decoded bf16 weights W~ = E2M1*E4M3 are exact)
 *     epilogue NONE:   y[r][n] = bf16_rne(global_scale[e] * acc[r][n]),  y is [M][N]
 *     epilogue SWIGLU: y[r][c] = bf16_rne(silu(g*acc[r][c]) * g*acc[r][c+N/2]),
 *                      c < N/2, y is [M][N/2]  (gate = first half of W rows)
 *   x_routed        [M][K] bf16, expert-sorted rows (moesq_permute output)
 *   expert_offsets  [E+1] int32 (moesq_route output); offsets are clamped to [0, M]
 *   w               host pointer to the weight descriptor: layout CANONICAL,
 *                   TILED or PAIRED_TILED (paired weights run on the sparse
 *                   MFMA; the canonical paired layout is an exchange format
 *                   and returns MOESQ_ERR_LAYOUT: tile it first)
 *   ws, ws_bytes    workspace; moesq_spgemm_workspace_bytes() bytes (may be 0)
 * Rows of y outside every expert range are not written.
 * Limits: K % 32 == 0, N % 16 == 0 (SWIGLU: N % 32 == 0), E <= MOESQ_MAX_EXPERTS,
 *         M >= 0, N*K/4 < 2^31 (one expert's values under 2 GiB),
 *         M*K < 2^31 (x_routed under 4 GiB).
 */
moesq_status_t moesq_grouped_spgemm(const uint16_t *x_routed, const int32_t *expert_offsets,
                                    int32_t M, const moesq_weights_t *w, int32_t epilogue,
                                    uint16_t *y, void *ws, size_t ws_bytes, hipStream_t stream);
size_t moesq_spgemm_workspace_bytes(int32_t M, const moesq_weights_t *w);

/*
 * Dispatch fused into the grouped GEMM ("D.1 Implementation details": the
 * serving kernels fuse dispatch with the expert GEMM): the same result as
 * moesq_permute(x, perm, T, k, K, x_routed) followed by
 * moesq_grouped_spgemm(x_routed, expert_offsets, T*k, w, epilogue, y, ...),
 * without the routed copy of the tokens -- routed row r reads token
 * perm[r] / k of x directly.
 *   x        [T][K] bf16 tokens;  perm [T*k] int32 (moesq_route output)
 *   expert_offsets, w, epilogue, y, ws, ws_bytes: as moesq_grouped_spgemm,
 *   with M = T*k.  Rows r whose perm[r] is outside [0, T*k) come out zero.
 * Limits: those of moesq_grouped_spgemm, with T*K < 2^31 in place of M*K;
 *         T >= 0, k >= 1, T*k < 2^31.
 */
moesq_status_t moesq_grouped_spgemm_gather(const uint16_t *x, const int32_t *perm, int32_t T,
                                           int32_t k, const int32_t *expert_offsets,
                                           const moesq_weights_t *w, int32_t epilogue, uint16_t *y,
                                           void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Routing, dispatch and grouped GEMM of a decode batch in one launch: the
 * results of moesq_route(topk_ids, T, k, E, expert_offsets, perm, inv_perm,
 * ...) followed by moesq_grouped_spgemm_gather(x, perm, T, k, expert_offsets,
 * w, epilogue, y, ...), bit for bit.  Every workgroup of the GEMM builds the
 * routing plan of the T*k ids in LDS (the same stable counting sort) and
 * workgroup 0 stores it, so the plan is there for moesq_unpermute.  The
 * pages keep routing outside the expert kernel ("D.3 End-to-end serving
 * benchmark"); for decode batches the separate routing launch and its gap
 * cost as much as a fifth of a 30B-class step, hence this fused form.
 *   topk_ids [T*k] int32; x [T][K] bf16; w, epilogue, y as
 *   moesq_grouped_spgemm_gather; expert_offsets [E+1], perm [T*k],
 *   inv_perm [T*k] int32 out (as moesq_route; perm and inv_perm may be NULL
 *   when T*k == 0).
 * One launch when 0 < T*k <= MOESQ_FUSED_ROUTE_MAX_ROWS and T*k <= 4*E (a
 * decode batch); otherwise the call makes the two separate calls above
 * (moesq_route without workspace, then the gather GEMM).
 * Limits: those of moesq_route (1 <= k <= E) and of
 *         moesq_grouped_spgemm_gather.
 */
moesq_status_t moesq_route_grouped_spgemm(const int32_t *topk_ids, const uint16_t *x, int32_t T,
                                          int32_t k, const moesq_weights_t *w, int32_t epilogue,
                                          uint16_t *y, int32_t *expert_offsets, int32_t *perm,
                                          int32_t *inv_perm, hipStream_t stream);

/*
 * NVFP4 activations for the W4A4 expert GEMM ("D.1 Implementation details":
 * the serving integration quantizes the activations of the expert GEMM in
 * 32-element scale blocks; "3.4 Implementation details": weights and
 * quantized activations are packed in corresponding scale blocks; "B
 * Experimental setup", Compression scope: paired 4:8 NVFP4 W4A4 with
 * 32-element blocks).  Rows of K activations (K % 32 == 0):
 *
 *   codes     [rows][K/2]  E2M1 codes, two per byte, position 2i in the low nibble
 *   scales    [rows][K/32] E4M3 scale (sign 0) of positions [32b, 32b+32),
 *                          the same K blocks as the weights' scales
 *   row_scale [rows]       fp32 second-level scale of the row
 *
 *   x~[r][k] = E2M1(code) * E4M3(scale of k's block) * row_scale[r]
 *
 * The struct is a host object; its pointers are device pointers.
 */
typedef struct {
  const uint8_t *codes;
  const uint8_t *scales;
  const float *row_scale;
  int32_t rows, K;
} moesq_act4_t;

/*
 * Quantize bf16 activation rows to NVFP4 (the layout above), one row on its
 * own, every decision in fp32 with ties to the even code:
 *   row_scale[t] = amax_t / 2688 (2688 = 6*448; 1 for a zero row)
 *   scales[t][b] = E4M3(amax_b / (6 * row_scale[t])), saturating at 448
 *   code         = E2M1(x / (E4M3(scale) * row_scale[t])), saturating at 6;
 *                  0 where that product is 0; zero is +0
 *   x [T][K] bf16 in; codes [T][K/2], scales [T][K/32], row_scale [T] out.
 * Inputs must be finite.  x and codes 16-byte aligned (MOESQ_ERR_ARG).
 * Limits: K % 32 == 0, K > 0, T >= 0.
 */
moesq_status_t moesq_quantize_activations(const uint16_t *x, int32_t T, int32_t K,
                                          uint8_t *codes, uint8_t *scales, float *row_scale,
                                          hipStream_t stream);

/*
 * W4A4 grouped GEMM: moesq_grouped_spgemm (perm == NULL) or
 * moesq_grouped_spgemm_gather (perm != NULL) with NVFP4 activations instead
 * of bf16 ones:
 *   acc[r][n] = sum_k x~[src(r)][k] * W~_e[n][k]   (fp32 accumulation; the
 *               decoded bf16 operands E2M1*E4M3 are exact)
 *   y as moesq_grouped_spgemm with g = global_scale[e] * row_scale[src(r)]
 *   src(r) = perm[r] / k with a gather permutation (x->rows == T, M == T*k;
 *   the quantized tokens are gathered inside the GEMM, as moesq_permute would
 *   copy their bf16 rows), else r (x->rows == M: rows in routed order, such
 *   as the quantized SwiGLU output feeding the down projection).
 *   MOESQ_OUT_FLAT as for the gather call (needs perm).
 *   x: host descriptor, x->K == w->K.  Other arguments and limits as
 *   moesq_grouped_spgemm_gather / moesq_grouped_spgemm; rows of y outside
 *   every expert range are not written; perm entries outside [0, T*k) give
 *   zero rows.
 */
moesq_status_t moesq_grouped_spgemm_act4(const moesq_act4_t *x, const int32_t *perm, int32_t T,
                                         int32_t k, const int32_t *expert_offsets, int32_t M,
                                         const moesq_weights_t *w, int32_t epilogue, uint16_t *y,
                                         hipStream_t stream);

/*
 * Combine.
 *   topk_weights != NULL: out[t][:] = bf16_rne( sum_{j<k} w[t*k+j] * y[inv_perm[t*k+j]][:] ),
 *                         fp32 accumulation in j order; out is [T][N].
 *   topk_weights == NULL: out[i][:] = y[inv_perm[i]][:] for i < T*k (flat order); out is [T*k][N].
 *   y [T*k][N] bf16 (routed order), inv_perm [T*k] int32, topk_weights [T*k] fp32.
 * Entries of inv_perm outside [0, T*k) contribute zero.
 * Limits: N % 8 == 0, N > 0.
 */
moesq_status_t moesq_unpermute(const uint16_t *y, const int32_t *inv_perm,
                               const float *topk_weights, int32_t T, int32_t k, int32_t N,
                               uint16_t *out, hipStream_t stream);

/*
 * Compress dense fp32 experts into the canonical layout above
 * ("3.4 Implementation details": the scales are recomputed first, then the
 * FP4 codes, the sparsity masks and one scale per 32 weights are stored).
 * Per expert:
 *   support  keep the 4 largest |w| of every group of 8; equal |w| -> lower position
 *   g        = amax / 2688 in fp32 (2688 = 6*448), g = 1 if amax == 0
 *   s_b      = E4M3 round-to-nearest-even, saturating at 448, of amax_b / (6*g)
 *   q        = E2M1 round-to-nearest-even, saturating at 6, of w / (E4M3(s_b)*g);
 *              zero is encoded +0; q = 0 when E4M3(s_b)*g == 0
 *   dense [E][N][K] fp32 in; values/masks/scales/global_scale out (sizes above).
 * Dense inputs must be finite.  global_scale doubles as the scratch of the
 * per-expert maximum, so it must not alias the other buffers.
 * Limits: K % 32 == 0, N >= 1, E >= 1.
 */
moesq_status_t moesq_pack_weights(const float *dense, int32_t E, int32_t N, int32_t K,
                                  uint8_t *values, uint8_t *masks, uint8_t *scales,
                                  float *global_scale, hipStream_t stream);

/*
 * Compress dense fp32 experts into MOESQ_LAYOUT_PAIRED ("A Sparse-quantized
 * representation", Blackwell paired 4:8 NVFP4 and Storage layout).  As
 * moesq_pack_weights, except the support: in every group of 8 the two pairs
 * (2i, 2i+1) with the largest |w_2i| + |w_2i+1| (fp32 sum) are kept, equal
 * sums to the lower pair; amax and the block maxima run over kept weights.
 *   dense [E][N][K] fp32 in; values [E][N][K/4], patterns [E][N][K/16],
 *   scales [E][N][K/32], global_scale [E] out.
 * Limits: K % 32 == 0, N >= 1, 1 <= E <= 65535.
 */
moesq_status_t moesq_pack_weights_paired(const float *dense, int32_t E, int32_t N, int32_t K,
                                         uint8_t *values, uint8_t *patterns, uint8_t *scales,
                                         float *global_scale, hipStream_t stream);

/*
 * Re-lay canonical weights into MOESQ_LAYOUT_TILED (a pure byte permutation),
 * or MOESQ_LAYOUT_PAIRED weights into MOESQ_LAYOUT_PAIRED_TILED (codes
 * reordered into the window order, pattern indices re-encoded as window
 * positions; an index above 5 becomes positions (0, 0), of unspecified
 * effect).
 *   src: CANONICAL or PAIRED descriptor (host struct, device buffers).
 *   values, masks, scales: device outputs of the source sizes; they must not
 *   alias src.
 *   The global scales are not touched (share src->global_scale).
 * Limits: N % 32 == 0, K % 64 == 0.
 */
moesq_status_t moesq_tile_weights(const moesq_weights_t *src, uint8_t *values, uint8_t *masks,
                                  uint8_t *scales, hipStream_t stream);

/*
 * Decode one expert to dense bf16 WITHOUT the global scale (any layout):
 *   dense[n][k] = E2M1(code) * E4M3(scale) (exact in bf16) or 0.
 * Uses the same in-register decoder as moesq_grouped_spgemm; meant for
 * checking and debugging.  dense is [N][K] bf16.  0 <= expert < E.
 */
moesq_status_t moesq_decode_weights(const moesq_weights_t *w, int32_t expert, uint16_t *dense,
                                    hipStream_t stream);

/*
 * DEBUG check of the caller contracts that the kernels above rely on without
 * checking them ("A Sparse-quantized representation": four kept values per
 * group of eight, E4M3 block scales).  Unlike every other call it allocates a
 * small device buffer (40 bytes), enqueues its checks on `stream` and
 * SYNCHRONISES the stream; it is not for the hot path.  Each input may be NULL
 * (w too) to skip its checks.
 *   topk_ids [T*k]     every id in [0, E)
 *   expert_offsets [E+1] offsets[0] == 0, non-decreasing, offsets[E] == T*k
 *   w (host struct)    every mask byte has exactly four bits set (paired
 *                      layouts: every pattern nibble is an index in [0, 6),
 *                      or in the tiled layout valid window positions); every
 *                      scale byte is a non-negative finite E4M3 code (not
 *                      0x7F, sign bit clear); every global scale is finite
 *                      and >= 0.  Either layout (the checks are per byte).
 *   counts (host, may be NULL) [5] out: violations of the five checks, in
 *                      the order ids, offsets, masks, scales, global scales.
 * Returns MOESQ_OK when every check passes, MOESQ_ERR_ARG when one fails
 * (moesq_last_error() names the failed checks and their counts), and the
 * usual errors for bad sizes or a failed HIP call.
 * Limits: with ids or offsets, 1 <= E <= MOESQ_MAX_EXPERTS, T >= 0, k >= 1.
 */
moesq_status_t moesq_validate(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E,
                              const int32_t *expert_offsets, const moesq_weights_t *w,
                              uint64_t *counts, hipStream_t stream);

/*
 * moesq_stream_read — measurement utility, not a step of the MoE path.
 * Reads `bytes` of device memory at `buf` once, in 16-byte loads with eight
 * in flight per lane, and writes nothing of use: the rate it reaches is the
 * practical HBM read ceiling against which the decode GEMMs (weight streams)
 * are compared, beside the device's published pin rate.
 *   buf [bytes] device, 16-byte aligned; bytes a multiple of 16 (0 is a no-op)
 *   sink [1]   device uint32, written only in a case that cannot occur for
 *              ordinary data (keeps the loads from being dropped); caller-owned.
 * Returns MOESQ_ERR_NULL / MOESQ_ERR_ARG for bad arguments, MOESQ_ERR_HIP if
 * the launch fails.  Asynchronous on `stream`.
 */
moesq_status_t moesq_stream_read(const void *buf, size_t bytes, uint32_t *sink,
                                 hipStream_t stream);

/* Human-readable name of a status code (static string). */
const char *moesq_status_string(moesq_status_t st);
/* Detail of the last error returned on the calling thread ("" if none). */
const char *moesq_last_error(void);
/* Library version, major*10000 + minor*100 + patch. */
int32_t moesq_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOESQ_H */
