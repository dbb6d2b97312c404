// Wave-level pieces of the routing plan (stable counting sort of the flat
// top-k ids), shared by the routing kernels and by the grouped GEMM's fused
// routing prologue.  See route.hip for the method.
#pragma once

#include "common.hpp"

namespace moesq {

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

// Histogram of ids[beg, end) into cnt[e] by one wave (leaders add).
__device__ __forceinline__ void wave_count(const int32_t *__restrict__ ids, int beg, int end,
                                           int E, int nbits, uint64_t lt_mask, int lane,
                                           int *cnt) {
  for (int base = beg; base < end; base += 64) {
    const int i = base + lane;
    int e = -1;
    if (i < end) {
      e = ids[i];
      if (e < 0 || e >= E) e = -1;
    }
    const uint64_t active = __ballot(e >= 0);
    const uint64_t peers = peers_of(e, nbits, active);
    if (e >= 0 && (peers & lt_mask) == 0) cnt[e] += __popcll(peers);
  }
}

// Ranks and scatter of ids[beg, end) by one wave; run[e] holds the next
// routed row of expert e for this wave and advances.  inv_perm may be NULL
// (not written).
__device__ __forceinline__ void wave_scatter(const int32_t *__restrict__ ids, int beg, int end,
                                             int E, int nbits, uint64_t lt_mask, int lane,
                                             int *run, int32_t *perm, int32_t *inv_perm) {
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
    if (e >= 0) row = run[e] + __popcll(peers & lt_mask);
    // all lanes have read run[e]; leaders now advance it
    __builtin_amdgcn_wave_barrier();
    if (e >= 0 && (peers & lt_mask) == 0) run[e] += __popcll(peers);
    if (i < end) {
      if (inv_perm) inv_perm[i] = row;
      if (row >= 0) perm[row] = i;
    }
  }
}

// The same two passes over a segment ids[base, base + n) that one wave
// holds in registers: lane l, slot j holds ids[base + 64 j + l] (-1 past
// the segment or out of range), all loaded at once, so that a short
// segment (n <= 64 * J) pays one load latency instead of one per 64 ids
// and pass.  `cnt` / `run` may be int or uint16_t (counts of at most 65535).
template <int J>
__device__ __forceinline__ void wave_load_ids(const int32_t *__restrict__ ids, int base, int n,
                                              int E, int lane, int (&v)[J]) {
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = 64 * j + lane;
    v[j] = i < n ? ids[base + i] : -1;
  }
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (v[j] < 0 || v[j] >= E) v[j] = -1;
}

template <int J, typename C>
__device__ __forceinline__ void wave_count_regs(const int (&v)[J], int n, int nbits,
                                                uint64_t lt_mask, C *cnt) {
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (64 * j < n) {   // uniform
      const int e = v[j];
      const uint64_t peers = peers_of(e, nbits, __ballot(e >= 0));
      if (e >= 0 && (peers & lt_mask) == 0) cnt[e] = (C)(cnt[e] + __popcll(peers));
    }
  }
}

template <int J, typename C>
__device__ __forceinline__ void wave_scatter_regs(const int (&v)[J], int base, int n, int nbits,
                                                  uint64_t lt_mask, int lane, C *run,
                                                  int32_t *perm, int32_t *inv_perm) {
#pragma unroll
  for (int j = 0; j < J; ++j) {
    if (64 * j < n) {   // uniform
      const int i = 64 * j + lane;
      const int e = v[j];
      const uint64_t peers = peers_of(e, nbits, __ballot(e >= 0));
      int row = -1;
      if (e >= 0) row = (int)run[e] + __popcll(peers & lt_mask);
      __builtin_amdgcn_wave_barrier();
      if (e >= 0 && (peers & lt_mask) == 0) run[e] = (C)(run[e] + __popcll(peers));
      if (i < n) {
        if (inv_perm) inv_perm[base + i] = row;
        if (row >= 0) perm[row] = base + i;
      }
    }
  }
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

__device__ __forceinline__ int id_bits(int E) { return (E > 1) ? 32 - __clz(E - 1) : 0; }
__device__ __forceinline__ uint64_t lanes_below(int lane) {
  return (lane == 0) ? 0ull : (~0ull >> (64 - lane));
}


}  // namespace moesq
