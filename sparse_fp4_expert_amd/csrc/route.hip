// Routing plan: expert offsets and the stable gather permutation.
//
// The grouped GEMM executes every routing-dependent expert problem in one
// launch (Hardware-Native Joint Sparse-Quantization for Trillion-Scale MoE,
// paper summary page, "3.4 Implementation details"), so the routed rows are
// grouped by expert first: a stable counting sort of the flat top-k ids.
//
// A wave owns a contiguous slice of the flat ids and walks it 64 ids at a
// time.  Inside a batch, lanes holding the same expert find each other with
// one ballot per id bit (a wave-wide multi-split); the lowest such lane is
// the leader, and a lane's rank among its peers is the popcount of peers
// below it.
//   pass 1: per-wave expert histograms in LDS (leaders add their peer count)
//   scan:   per expert, exclusive prefix over waves (and blocks); then
//           exclusive prefix over experts -> offsets
//   pass 2: same walk again; row = base[w][e] + running + rank
// Every step is in index order, so perm is the stable order and the result
// is bit-identical on every run (no atomics).
//
// Small inputs run all of it in one workgroup.  Large ones split the ids
// into blocks of ROUTE_BLOCK_IDS: a histogram kernel per block, one scan
// kernel over (block, expert) counts in the workspace, and a scatter kernel
// per block.
#include <mutex>
#include <string>

#include "common.hpp"
#include "route_dev.hpp"

namespace moesq {

constexpr int ROUTE_WAVES = 8;
constexpr int ROUTE_THREADS = ROUTE_WAVES * 64;

// Exclusive prefix of v[0..n) in place by the whole block; returns the total.
template <int THREADS>
__device__ int block_exclusive_scan(int *v, int n, int *wave_tot) {
  constexpr int WAVES = THREADS / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int per_wave = (n + WAVES - 1) / WAVES;
  const int e0 = min(n, w * per_wave), e1 = min(n, e0 + per_wave);
  const int per_lane = (e1 - e0 + 63) / 64;
  const int l0 = min(e1, e0 + lane * per_lane), l1 = min(e1, l0 + per_lane);
  int s = 0;
  for (int e = l0; e < l1; ++e) s += v[e];
  int incl = s;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(incl, d, 64);
    if (lane >= d) incl += t;
  }
  if (lane == 63) wave_tot[w] = incl;
  __syncthreads();
  int wbase = 0, tot = 0;
  for (int u = 0; u < WAVES; ++u) {
    if (u < w) wbase += wave_tot[u];
    tot += wave_tot[u];
  }
  int run = wbase + incl - s;
  for (int e = l0; e < l1; ++e) {
    const int c = v[e];
    v[e] = run;
    run += c;
  }
  __syncthreads();
  return tot;
}

// Whole plan in one workgroup.
__global__ __launch_bounds__(ROUTE_THREADS) void route_kernel(const int32_t *__restrict__ ids,
                                                              int M, int E, int32_t *offsets,
                                                              int32_t *perm, int32_t *inv_perm) {
  __shared__ int cnt[ROUTE_WAVES][MOESQ_MAX_EXPERTS];
  __shared__ int off[MOESQ_MAX_EXPERTS + 1];
  __shared__ int wave_tot[ROUTE_WAVES];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const uint64_t lt_mask = lanes_below(lane);
  const int nbits = id_bits(E);

  for (int i = threadIdx.x; i < ROUTE_WAVES * MOESQ_MAX_EXPERTS; i += ROUTE_THREADS)
    (&cnt[0][0])[i] = 0;
  __syncthreads();

  const int chunk = ((M + ROUTE_WAVES - 1) / ROUTE_WAVES + 63) & ~63;
  const int beg = min(M, w * chunk), end = min(M, beg + chunk);
  wave_count(ids, beg, end, E, nbits, lt_mask, lane, cnt[w]);
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
  const int total = block_exclusive_scan<ROUTE_THREADS>(off, E, wave_tot);
  if (threadIdx.x == 0) off[E] = total;
  for (int e = threadIdx.x; e < E; e += ROUTE_THREADS) {
#pragma unroll
    for (int v = 0; v < ROUTE_WAVES; ++v) cnt[v][e] += off[e];
  }
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += ROUTE_THREADS) offsets[e] = off[e];
  wave_scatter(ids, beg, end, E, nbits, lt_mask, lane, cnt[w], perm, inv_perm);
}

constexpr int RB_WAVES = 4;
constexpr int RB_THREADS = RB_WAVES * 64;
constexpr int ROUTE_BLOCK_IDS = 512;           // ids per block, 128 per wave

// Large inputs, step 1: counts[b][e] of block b.
__global__ __launch_bounds__(RB_THREADS) void route_hist_kernel(const int32_t *__restrict__ ids,
                                                                int M, int E, int *counts) {
  __shared__ int cnt[RB_WAVES][MOESQ_MAX_EXPERTS];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < RB_WAVES * E; i += RB_THREADS) cnt[i / E][i % E] = 0;
  __syncthreads();
  const int b0 = blockIdx.x * ROUTE_BLOCK_IDS;
  const int per = ROUTE_BLOCK_IDS / RB_WAVES;
  const int beg = min(M, b0 + w * per), end = min(M, beg + per);
  wave_count(ids, beg, end, E, id_bits(E), lanes_below(lane), lane, cnt[w]);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += RB_THREADS) {
    int c = 0;
#pragma unroll
    for (int v = 0; v < RB_WAVES; ++v) c += cnt[v][e];
    counts[(size_t)blockIdx.x * E + e] = c;
  }
}

// Step 2 (one workgroup): counts[b][e] -> number of ids of expert e in the
// blocks before b (the first routed row of block b's ids of expert e is
// offsets[e] plus that); offsets.
__global__ __launch_bounds__(ROUTE_THREADS) void route_scan_kernel(int *counts, int nb, int E,
                                                                   int32_t *offsets) {
  __shared__ int tot[MOESQ_MAX_EXPERTS + 1];
  __shared__ int wave_tot[ROUTE_WAVES];
  // the counts of SCAN_BATCH blocks are loaded before any is rewritten, so
  // that the loads of a batch overlap instead of one load-store round trip
  // per block
  constexpr int SCAN_BATCH = 8;
  for (int e = threadIdx.x; e < E; e += ROUTE_THREADS) {
    int run = 0;
    for (int b0 = 0; b0 < nb; b0 += SCAN_BATCH) {
      int c[SCAN_BATCH];
#pragma unroll
      for (int j = 0; j < SCAN_BATCH; ++j)
        c[j] = b0 + j < nb ? counts[(size_t)(b0 + j) * E + e] : 0;
#pragma unroll
      for (int j = 0; j < SCAN_BATCH; ++j) {
        if (b0 + j < nb) counts[(size_t)(b0 + j) * E + e] = run;
        run += c[j];
      }
    }
    tot[e] = run;
  }
  __syncthreads();
  const int total = block_exclusive_scan<ROUTE_THREADS>(tot, E, wave_tot);
  for (int e = threadIdx.x; e < E; e += ROUTE_THREADS) offsets[e] = tot[e];
  if (threadIdx.x == 0) offsets[E] = total;
}

// Step 3: ranks inside block b on top of its bases; perm and inv_perm.
__global__ __launch_bounds__(RB_THREADS) void route_scatter_kernel(
    const int32_t *__restrict__ ids, int M, int E, const int *bases, const int32_t *offsets,
    int32_t *perm, int32_t *inv_perm) {
  __shared__ int cnt[RB_WAVES][MOESQ_MAX_EXPERTS];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int nbits = id_bits(E);
  const uint64_t lt_mask = lanes_below(lane);
  for (int i = threadIdx.x; i < RB_WAVES * E; i += RB_THREADS) cnt[i / E][i % E] = 0;
  __syncthreads();
  const int b0 = blockIdx.x * ROUTE_BLOCK_IDS;
  const int per = ROUTE_BLOCK_IDS / RB_WAVES;
  const int beg = min(M, b0 + w * per), end = min(M, beg + per);
  wave_count(ids, beg, end, E, nbits, lt_mask, lane, cnt[w]);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += RB_THREADS) {
    int run = bases[(size_t)blockIdx.x * E + e] + offsets[e];
#pragma unroll
    for (int v = 0; v < RB_WAVES; ++v) {
      const int c = cnt[v][e];
      cnt[v][e] = run;
      run += c;
    }
  }
  __syncthreads();
  wave_scatter(ids, beg, end, E, nbits, lt_mask, lane, cnt[w], perm, inv_perm);
}

static long long route_blocks(long long M) { return (M + ROUTE_BLOCK_IDS - 1) / ROUTE_BLOCK_IDS; }

// Scratch of moesq_route_noalloc: the per-block expert counts live in this
// file-scope device array instead of a caller's workspace.  Each device that
// the library runs on holds its own copy until the process ends.  Host code
// never passes the array's name to a kernel (on the host it is a stand-in,
// not a device address): set-up takes each device's address once with
// hipGetSymbolAddress and the launches use that.
constexpr size_t ROUTE_SCRATCH_BYTES = MOESQ_ROUTE_SCRATCH_BYTES;
static __device__ __align__(256) int scratch[ROUTE_SCRATCH_BYTES / sizeof(int)];

constexpr int SCRATCH_MAX_DEVICES = 64;

// Address of this device's scratch, taken on the device's first call.
static moesq_status_t scratch_ptr(int **out) {
  static std::mutex mu;
  static int *ptr[SCRATCH_MAX_DEVICES] = {nullptr};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES)
    return fail(MOESQ_ERR_HIP, "moesq_route_noalloc: no current device");
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MOESQ_ERR_HIP, std::string("moesq_route_noalloc: hipGetSymbolAddress: ") +
                                     hipGetErrorString(e));
    ptr[dev] = static_cast<int *>(p);
  }
  *out = ptr[dev];
  return MOESQ_OK;
}

}  // namespace moesq

using namespace moesq;

// Inputs up to this many ids take the one-workgroup path.
constexpr long long ROUTE_SMALL = 4096;

extern "C" size_t moesq_route_workspace_bytes(int32_t T, int32_t k, int32_t E) {
  const long long M = (long long)T * k;
  if (T < 0 || k < 1 || E < 1 || M <= ROUTE_SMALL) return 0;
  return (size_t)(route_blocks(M) * E * sizeof(int));
}

// Host checks shared by both routing entry points.
static moesq_status_t route_check(const char *who, const int32_t *topk_ids, int32_t T, int32_t k,
                                  int32_t E, const int32_t *expert_offsets, const int32_t *perm,
                                  const int32_t *inv_perm) {
  const std::string w(who);
  if (E < 1 || E > MOESQ_MAX_EXPERTS)
    return fail(MOESQ_ERR_SHAPE, w + ": E must be in [1, " + std::to_string(MOESQ_MAX_EXPERTS) + "]");
  if (k < 1 || k > E) return fail(MOESQ_ERR_SHAPE, w + ": k must be in [1, E]");
  if (T < 0) return fail(MOESQ_ERR_SHAPE, w + ": T must be >= 0");
  if ((long long)T * k >= (1ll << 31)) return fail(MOESQ_ERR_SHAPE, w + ": T*k must be < 2^31");
  if (!expert_offsets) return fail(MOESQ_ERR_NULL, w + ": expert_offsets is NULL");
  if ((long long)T * k > 0 && (!topk_ids || !perm || !inv_perm))
    return fail(MOESQ_ERR_NULL, w + ": topk_ids, perm and inv_perm must be non-NULL");
  return MOESQ_OK;
}

// The routing launches: one workgroup without counts, else the three
// block kernels over `counts` (route_blocks(M) x E ints).
static moesq_status_t route_launch(const char *who, const int32_t *topk_ids, int M, int E,
                                   int32_t *expert_offsets, int32_t *perm, int32_t *inv_perm,
                                   int *counts, hipStream_t stream) {
  if (!counts) {
    // one workgroup: no workspace needed (slower for large inputs)
    hipLaunchKernelGGL(route_kernel, dim3(1), dim3(ROUTE_THREADS), 0, stream, topk_ids, M, E,
                       expert_offsets, perm, inv_perm);
    return launch_status(who);
  }
  const int nb = (int)route_blocks(M);
  hipLaunchKernelGGL(route_hist_kernel, dim3(nb), dim3(RB_THREADS), 0, stream, topk_ids, M, E,
                     counts);
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(ROUTE_THREADS), 0, stream, counts, nb, E,
                     expert_offsets);
  hipLaunchKernelGGL(route_scatter_kernel, dim3(nb), dim3(RB_THREADS), 0, stream, topk_ids, M, E,
                     counts, expert_offsets, perm, inv_perm);
  return launch_status(who);
}

extern "C" moesq_status_t moesq_route(const int32_t *topk_ids, int32_t T, int32_t k, int32_t E,
                                      int32_t *expert_offsets, int32_t *perm, int32_t *inv_perm,
                                      void *ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  moesq_status_t st =
      route_check("moesq_route", topk_ids, T, k, E, expert_offsets, perm, inv_perm);
  if (st != MOESQ_OK) return st;
  const size_t need = moesq_route_workspace_bytes(T, k, E);
  int *counts = (need == 0 || !ws || ws_bytes < need) ? nullptr : static_cast<int *>(ws);
  return route_launch("moesq_route", topk_ids, T * k, E, expert_offsets, perm, inv_perm, counts,
                      stream);
}

extern "C" moesq_status_t moesq_route_noalloc(const int32_t *topk_ids, int32_t T, int32_t k,
                                              int32_t E, int32_t *expert_offsets, int32_t *perm,
                                              int32_t *inv_perm, hipStream_t stream) {
  static const char *who = "moesq_route_noalloc";
  clear_error();
  moesq_status_t st = route_check(who, topk_ids, T, k, E, expert_offsets, perm, inv_perm);
  if (st != MOESQ_OK) return st;
  const size_t need = moesq_route_workspace_bytes(T, k, E);
  if (need > ROUTE_SCRATCH_BYTES)
    return fail(MOESQ_ERR_SHAPE, std::string(who) + ": the block counts need " +
                                     std::to_string(need) + " bytes, more than the " +
                                     std::to_string(ROUTE_SCRATCH_BYTES) +
                                     " bytes of the library's scratch; "
                                     "use moesq_route with a workspace");
  int *counts = nullptr;
  if (need > 0) {
    st = scratch_ptr(&counts);
    if (st != MOESQ_OK) return st;
  }
  return route_launch(who, topk_ids, T * k, E, expert_offsets, perm, inv_perm, counts, stream);
}
