// Block-wide stable counting sort of (token, slot) pairs by expert group: the
// argsort of tokens by expert of the Sem-MoE notes (Key design 4).
//
// Pair p = t * kk + j has key = ids[p] - g_begin when that lies in
// [0, n_groups) (an expert this GPU holds); otherwise its key is n_groups and
// the pair is dropped.  The W waves of the block each own a contiguous
// segment of pairs and walk it 64 pairs at a time.  Inside a 64-pair chunk a
// lane finds the lanes holding the same key with one ballot per key bit, so
// its rank among equal keys is a popcount of the lower lanes; no atomics
// decide any order.
//   pass 1: per-wave, per-group counts (LDS integer atomics: order-free)
//   pass 2: group totals, exclusive scan -> offsets; per-wave bases
//   pass 3: same walk again, each pair written to offsets[g] + base + rank
// Segments, chunks and lanes are visited in ascending pair order, so the sort
// is stable.  Keys are staged in LDS first (one coalesced sweep) when they
// fit, so the passes never wait on global memory.
#pragma once

#include "common.hpp"

namespace moe {

__device__ __forceinline__ unsigned long long match_key(int key, bool active, int nbits) {
  unsigned long long m = __ballot(active);
  for (int b = 0; b < nbits; ++b) {
    const int bit = (key >> b) & 1;
    const unsigned long long bm = __ballot(bit);
    m &= bit ? bm : ~bm;
  }
  return m;
}

// kCoherent: ids were written by other blocks of the same launch (st_agent).
template <bool kCoherent>
__device__ __forceinline__ int pair_key(const int32_t* ids, int p, int g_begin, int n_groups) {
  const int g = (kCoherent ? ld_agent(ids + p) : ids[p]) - g_begin;
  return (g >= 0 && g < n_groups) ? g : n_groups;
}

template <bool kStaged, bool kCoherent>
__device__ __forceinline__ int sort_key(const uint16_t* s_key, const int32_t* ids, int p, int g_begin,
                                        int n_groups) {
  return kStaged ? static_cast<int>(s_key[p]) : pair_key<kCoherent>(ids, p, g_begin, n_groups);
}

// Pass 1 over this wave's segment [p_begin, p_end): LDS integer atomics
// (order-free, so the counts are exact and deterministic) keep the pass free
// of any dependency between chunks.
template <bool kStaged, bool kCoherent>
__device__ __forceinline__ void sort_histogram(const uint16_t* s_key, const int32_t* ids, int p_begin,
                                               int p_end, int g_begin, int n_groups, int* my_cnt) {
  for (int p = p_begin + lane_id(); p < p_end; p += WAVE) {
    const int key = sort_key<kStaged, kCoherent>(s_key, ids, p, g_begin, n_groups);
    if (key < n_groups) atomicAdd(my_cnt + key, 1);
  }
}

// Pass 3 over the segment: my_cnt[g] enters as the offset of group g's first
// pair of this wave and is advanced chunk by chunk.
template <bool kStaged, bool kCoherent>
__device__ __forceinline__ void sort_scatter(const uint16_t* s_key, const int32_t* ids, int p_begin,
                                             int p_end, int g_begin, int n_groups, const int* s_off,
                                             int* my_cnt, int32_t* sorted_pair, int32_t* pair_pos) {
  const int l = lane_id();
  const int nbits = 32 - __clz(n_groups);  // keys 0..n_groups
  const unsigned long long lt_mask = (1ull << l) - 1ull;
  for (int base = p_begin; base < p_end; base += WAVE) {
    const int p = base + l;
    const bool active = p < p_end;
    const int key = active ? sort_key<kStaged, kCoherent>(s_key, ids, p, g_begin, n_groups) : n_groups;
    const unsigned long long m = match_key(key, active, nbits);
    const int rank = __popcll(m & lt_mask);
    const bool kept = key < n_groups;
    // One LDS read of the running count per chunk; the leader of each key
    // writes the advanced count back after every lane has read it.
    const int run = kept ? my_cnt[key] : 0;
    const int pos = kept ? s_off[key] + run + rank : -1;
    if (kept) sorted_pair[pos] = p;
    if (active) pair_pos[p] = pos;
    __builtin_amdgcn_wave_barrier();
    if (kept && rank == 0) my_cnt[key] = run + __popcll(m);
  }
}

// LDS needs: s_cnt[W * MAX_GROUPS] ints, s_off[MAX_GROUPS] ints and, for N <= key_cap,
// s_key[key_cap] 16-bit keys.  Must be called by all W*64 threads of the block.
// key_cap < 0: the caller has already written all N keys (as pair_key maps
// them) to s_key, and ids is not read.
template <int W, bool kCoherent>
__device__ void block_counting_sort(const int32_t* __restrict__ ids, int N, int g_begin,
                                    int n_groups, int32_t* __restrict__ counts,
                                    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
                                    int32_t* __restrict__ pair_pos, int* s_cnt, int* s_off,
                                    uint16_t* s_key, int key_cap) {
  const int tid = threadIdx.x;
  const int wv = tid / WAVE;
  const int l = lane_id();
  const bool staged = key_cap < 0 || N <= key_cap;
  if (key_cap >= 0 && staged) {
    // Eight loads in flight per thread (clamped addresses, no branches) before any is used.
    constexpr int U = 8;
    for (int p0 = tid; p0 < N; p0 += U * W * WAVE) {
      int key[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        key[u] = pair_key<kCoherent>(ids, min(p0 + u * W * WAVE, N - 1), g_begin, n_groups);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (p0 + u * W * WAVE < N) s_key[p0 + u * W * WAVE] = static_cast<uint16_t>(key[u]);
    }
  }
  for (int i = tid; i < W * MAX_GROUPS; i += W * WAVE) s_cnt[i] = 0;
  __syncthreads();

  const int per_wave = (N + W - 1) / W;
  const int seg = ((per_wave + WAVE - 1) / WAVE) * WAVE;
  const int p_begin = wv * seg;
  const int p_end = min(N, p_begin + seg);
  int* my_cnt = s_cnt + wv * MAX_GROUPS;

  if (staged)
    sort_histogram<true, kCoherent>(s_key, ids, p_begin, p_end, g_begin, n_groups, my_cnt);
  else
    sort_histogram<false, kCoherent>(s_key, ids, p_begin, p_end, g_begin, n_groups, my_cnt);
  __syncthreads();

  // Per-group totals; s_cnt[w][g] becomes the count of group g in waves < w.
  for (int g = tid; g < n_groups; g += W * WAVE) {
    int run = 0;
    for (int w = 0; w < W; ++w) {
      const int c = s_cnt[w * MAX_GROUPS + g];
      s_cnt[w * MAX_GROUPS + g] = run;
      run += c;
    }
    s_off[g] = run;
  }
  __syncthreads();
  if (wv == 0) {
    int base = 0;
    for (int g0 = 0; g0 < n_groups; g0 += WAVE) {
      const int g = g0 + l;
      const int c = (g < n_groups) ? s_off[g] : 0;
      const int incl = wave_inclusive_scan(c);
      if (g < n_groups) {
        counts[g] = c;
        offsets[g] = base + incl - c;
        s_off[g] = base + incl - c;
      }
      base += __shfl(incl, WAVE - 1, WAVE);
    }
    if (l == 0) offsets[n_groups] = base;
  }
  __syncthreads();

  if (staged)
    sort_scatter<true, kCoherent>(s_key, ids, p_begin, p_end, g_begin, n_groups, s_off, my_cnt,
                                  sorted_pair, pair_pos);
  else
    sort_scatter<false, kCoherent>(s_key, ids, p_begin, p_end, g_begin, n_groups, s_off, my_cnt,
                                   sorted_pair, pair_pos);
}

}  // namespace moe
