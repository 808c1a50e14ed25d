// Expert counts, offsets and the stable permutation of (token, slot) pairs by
// expert group -- the argsort of tokens by expert that the Sem-MoE notes
// describe (Key design 4), written as a one-block counting sort.
//
// Pair p = t * kk + j has key = id - g_begin when that lies in
// [0, n_groups) (an expert this GPU holds), else it is dropped.  The 16 waves
// of the block each own a contiguous segment of pairs and walk it 64 pairs
// at a time.  Inside a 64-pair chunk every lane finds the lanes holding the
// same key with one ballot per key bit, so its rank among equal keys is a
// popcount of the lower lanes; no atomics decide any order.
//   pass 1: per-wave, per-group counts in LDS
//   pass 2: group totals, exclusive scan -> offsets; per-wave bases
//   pass 3: same walk again, each pair written to offsets[g] + base + rank
// Segments, chunks and lanes are visited in ascending pair order, so the sort
// is stable: the oracle's counting sort gives the same permutation bit for bit.
#include "common.hpp"
#include "moe_internal.h"

namespace moe {

constexpr int PERM_WAVES = 16;

__device__ __forceinline__ unsigned long long match_key(int key, bool active, int nbits) {
  unsigned long long m = __ballot(active);
  for (int b = 0; b < nbits; ++b) {
    const int bit = (key >> b) & 1;
    const unsigned long long bm = __ballot(bit);
    m &= bit ? bm : ~bm;
  }
  return m;
}

__global__ __launch_bounds__(PERM_WAVES * WAVE) void permute_kernel(
    const int32_t* __restrict__ ids, int N, int g_begin, int n_groups, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos) {
  __shared__ int s_cnt[PERM_WAVES * MAX_GROUPS];
  __shared__ int s_off[MAX_GROUPS];

  const int wv = threadIdx.x / WAVE;
  const int l = lane_id();
  for (int i = threadIdx.x; i < PERM_WAVES * MAX_GROUPS; i += blockDim.x) s_cnt[i] = 0;
  __syncthreads();

  const int nbits = 32 - __clz(n_groups);  // keys 0..n_groups (n_groups = dropped)
  const int per_wave = (N + PERM_WAVES - 1) / PERM_WAVES;
  const int seg = ((per_wave + WAVE - 1) / WAVE) * WAVE;
  const int p_begin = wv * seg;
  const int p_end = min(N, p_begin + seg);
  int* my_cnt = s_cnt + wv * MAX_GROUPS;
  const unsigned long long lt_mask = (1ull << l) - 1ull;

  for (int base = p_begin; base < p_end; base += WAVE) {
    const int p = base + l;
    const bool active = p < p_end;
    int key = n_groups;
    if (active) {
      const int g = ids[p] - g_begin;
      key = (g >= 0 && g < n_groups) ? g : n_groups;
    }
    const unsigned long long m = match_key(key, active, nbits);
    const int rank = __popcll(m & lt_mask);
    if (active && rank == 0 && key < n_groups) my_cnt[key] += __popcll(m);
  }
  __syncthreads();

  // Per-group totals; s_cnt[w][g] becomes the count of group g in waves < w.
  for (int g = threadIdx.x; g < n_groups; g += blockDim.x) {
    int run = 0;
    for (int w = 0; w < PERM_WAVES; ++w) {
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

  for (int base = p_begin; base < p_end; base += WAVE) {
    const int p = base + l;
    const bool active = p < p_end;
    int key = n_groups;
    if (active) {
      const int g = ids[p] - g_begin;
      key = (g >= 0 && g < n_groups) ? g : n_groups;
    }
    const unsigned long long m = match_key(key, active, nbits);
    const int rank = __popcll(m & lt_mask);
    if (active) {
      if (key < n_groups) {
        const int pos = s_off[key] + my_cnt[key] + rank;
        sorted_pair[pos] = p;
        pair_pos[p] = pos;
      } else {
        pair_pos[p] = -1;
      }
    }
    __builtin_amdgcn_wave_barrier();
    if (active && rank == 0 && key < n_groups) my_cnt[key] += __popcll(m);
  }
}

void launch_permute(const int32_t* ids, int T, int kk, int g_begin, int n_groups, int32_t* counts,
                    int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, hipStream_t s) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(PERM_WAVES * WAVE), 0, s, ids, T * kk, g_begin,
                     n_groups, counts, offsets, sorted_pair, pair_pos);
}

}  // namespace moe
