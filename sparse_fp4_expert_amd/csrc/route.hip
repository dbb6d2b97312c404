// Routing plan: expert offsets and the stable gather permutation.
//
// The grouped GEMM executes every routing-dependent expert problem in one
// launch (Hardware-Native Joint Sparse-Quantization for Trillion-Scale MoE,
// paper summary page, "3.4 Implementation details"), so the routed rows are
// grouped by expert first: a stable counting sort of the flat top-k ids.
//
// One workgroup of ROUTE_WAVES wavefronts.  Wave w owns the contiguous slice
// [w*C, (w+1)*C) of the flat ids and walks it 64 ids at a time.  Inside a
// batch, lanes holding the same expert find each other with one ballot per
// id bit (a wave-wide multi-split); the lowest such lane is the leader, and
// a lane's rank among its peers is the popcount of peers below it.
//   pass 1: per-wave expert histograms in LDS (leaders add their peer count)
//   scan:   per expert, exclusive prefix over waves; then exclusive prefix
//           over experts -> offsets
//   pass 2: same walk again; row = offset[e] + base[w][e] + running + rank
// Every step is in index order, so perm is the stable order and the result
// is bit-identical on every run (no atomics).
#include "common.hpp"

namespace moesq {

constexpr int ROUTE_WAVES = 8;
constexpr int ROUTE_THREADS = ROUTE_WAVES * 64;

__device__ __forceinline__ uint64_t peers_of(int e, int nbits, uint64_t active) {
  uint64_t peers = active;
#pragma unroll 1
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t bal = __ballot(bit);
    peers &= bit ? bal : ~bal;
  }
  return peers;
}

__global__ __launch_bounds__(ROUTE_THREADS) void route_kernel(const int32_t *__restrict__ ids,
                                                              int M, int E, int32_t *offsets,
                                                              int32_t *perm, int32_t *inv_perm) {
  __shared__ int cnt[ROUTE_WAVES][MOESQ_MAX_EXPERTS];
  __shared__ int off[MOESQ_MAX_EXPERTS + 1];
  __shared__ int wave_tot[ROUTE_WAVES];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int nbits = (E > 1) ? 32 - __clz(E - 1) : 0;

  for (int i = threadIdx.x; i < ROUTE_WAVES * MOESQ_MAX_EXPERTS; i += ROUTE_THREADS)
    (&cnt[0][0])[i] = 0;
  __syncthreads();

  const int chunk = ((M + ROUTE_WAVES - 1) / ROUTE_WAVES + 63) & ~63;
  const int beg = min(M, w * chunk), end = min(M, beg + chunk);

  // pass 1: histogram of this wave's slice
  for (int base = beg; base < end; base += 64) {
    const int i = base + lane;
    int e = -1;
    if (i < end) {
      e = ids[i];
      if (e < 0 || e >= E) e = -1;
    }
    const uint64_t active = __ballot(e >= 0);
    const uint64_t peers = peers_of(e, nbits, active);
    if (e >= 0 && (peers & lt_mask) == 0) cnt[w][e] += __popcll(peers);
  }
  __syncthreads();

  // per expert: exclusive prefix over waves, total in off[e]
  for (int e = threadIdx.x; e < E; e += ROUTE_THREADS) {
    int run = 0;
#pragma unroll
    for (int v = 0; v < ROUTE_WAVES; ++v) {
      const int c = cnt[v][e];
      cnt[v][e] = run;
      run += c;
    }
    off[e] = run;
  }
  __syncthreads();

  // exclusive prefix over experts: each wave scans a contiguous range of
  // experts lane-serially, then the wave totals are combined.
  {
    const int per_wave = (E + ROUTE_WAVES - 1) / ROUTE_WAVES;
    const int e0 = min(E, w * per_wave), e1 = min(E, e0 + per_wave);
    const int per_lane = (e1 - e0 + 63) / 64;
    const int l0 = min(e1, e0 + lane * per_lane), l1 = min(e1, l0 + per_lane);
    int s = 0;
    for (int e = l0; e < l1; ++e) s += off[e];
    // inclusive wave scan of lane sums
    int incl = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(incl, d, 64);
      if (lane >= d) incl += t;
    }
    if (lane == 63) wave_tot[w] = incl;
    __syncthreads();
    int wbase = 0;
    for (int v = 0; v < w; ++v) wbase += wave_tot[v];
    int run = wbase + incl - s;
    // rewrite off[] in place as exclusive prefix (each lane owns its range)
    for (int e = l0; e < l1; ++e) {
      const int c = off[e];
      off[e] = run;
      run += c;
    }
    if (threadIdx.x == 0) {
      int tot = 0;
      for (int v = 0; v < ROUTE_WAVES; ++v) tot += wave_tot[v];
      off[E] = tot;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += ROUTE_THREADS) offsets[e] = off[e];

  // pass 2: ranks and scatter
  for (int base = beg; base < end; base += 64) {
    const int i = base + lane;
    int e = -1;
    if (i < end) {
      e = ids[i];
      if (e < 0 || e >= E) e = -1;
    }
    const uint64_t active = __ballot(e >= 0);
    const uint64_t peers = peers_of(e, nbits, active);
    int row = -1;
    if (e >= 0) row = off[e] + cnt[w][e] + __popcll(peers & lt_mask);
    // all lanes have read cnt[w][e]; leaders now advance it
    __builtin_amdgcn_wave_barrier();
    if (e >= 0 && (peers & lt_mask) == 0) cnt[w][e] += __popcll(peers);
    if (i < end) {
      inv_perm[i] = row;
      if (row >= 0) perm[row] = i;
    }
  }
}

}  // namespace moesq

using namespace moesq;

extern "C" size_t moesq_route_workspace_bytes(int32_t, int32_t, int32_t) { return 0; }

extern "C" moesq_status_t moesq_route(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E,
                                      int32_t *expert_offsets, int32_t *perm, int32_t *inv_perm,
                                      void *ws, size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  clear_error();
  if (E < 1 || E > MOESQ_MAX_EXPERTS)
    return fail(MOESQ_ERR_SHAPE, "moesq_route: E must be in [1, " +
                                     std::to_string(MOESQ_MAX_EXPERTS) + "]");
  if (k < 1 || k > E) return fail(MOESQ_ERR_SHAPE, "moesq_route: k must be in [1, E]");
  if (T < 0) return fail(MOESQ_ERR_SHAPE, "moesq_route: T must be >= 0");
  const long long M = (long long)T * k;
  if (M >= (1ll << 31)) return fail(MOESQ_ERR_SHAPE, "moesq_route: T*k must be < 2^31");
  if (!expert_offsets) return fail(MOESQ_ERR_NULL, "moesq_route: expert_offsets is NULL");
  if (M > 0 && (!topk_ids || !perm || !inv_perm))
    return fail(MOESQ_ERR_NULL, "moesq_route: topk_ids, perm and inv_perm must be non-NULL");
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(ROUTE_THREADS), 0, stream, topk_ids, (int)M, E,
                     expert_offsets, perm, inv_perm);
  return launch_status("moesq_route");
}
