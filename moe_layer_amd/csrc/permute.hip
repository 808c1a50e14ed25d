// moe_permute on its own: expert counts, offsets and the stable permutation of
// (token, slot) pairs by expert group (the argsort of tokens by expert of the
// Sem-MoE notes, Key design 4).
//
// Up to PERM_ONE_BLOCK_MAX pairs: one block of 16 waves runs the counting sort
// of sort.hpp (the fused routing launch, route.hip, runs the same sort in its
// last block).  Above that, one block sorting everything is the bottleneck,
// so the pairs are cut into contiguous segments, one per block, and no block
// waits for another: each block
//   1. sweeps the whole id table (L2-resident: 4 bytes per pair) and counts,
//      per group, all pairs and the pairs before its segment (LDS integer
//      atomics: order-free, so exact and deterministic);
//   2. turns the totals into offsets (block 0 also writes counts and offsets)
//      and the segment's base per group = offset + pairs before it;
//   3. ranks its own pairs with the passes of sort.hpp (per-wave histograms,
//      ballot ranks in pair order) from that base.
// A pair's row is therefore (pairs of lower groups) + (pairs of its group
// before it), exactly as in the one-block sort.
//
// Every block's sweep reads the whole table, so that launch does work that
// grows with the square of the pair count.  Above PM_SWEEP_MAX pairs the same
// sort runs in three launches that read each id a fixed number of times:
//   count:   block b counts its segment's pairs per group and parks the counts
//            in pair_pos[p0_b + g] (its own segment, g < n_groups: every
//            segment holds at least PM_SEG >= MAX_GROUPS pairs);
//   columns: block g turns column g of those counts into the pairs of group g
//            in the segments before each one (in place) and writes counts[g];
//   scatter: block b reads its parked bases back into LDS, then ranks and
//            writes its pairs as above.  Its pair_pos slots are overwritten
//            only after the read, and no other block reads them.
// No scratch memory beyond the outputs and no waits between blocks.
#include <algorithm>

#include "common.hpp"
#include "moe_internal.h"
#include "sort.hpp"

namespace moe {

constexpr int PERM_WAVES = 16;
constexpr int PERM_KEY_CAP = 16384;
constexpr int PM_WAVES = 8;
constexpr int PM_THREADS = PM_WAVES * WAVE;
constexpr int PM_SEG = 1024;   // pairs per block
constexpr int PM_UNROLL = 8;   // id loads in flight per thread in the sweep
constexpr int PM_SWEEP_MAX = 65536;  // pairs up to which each block sweeps the whole table
constexpr int PL_BLOCKS_MAX = 2048;  // segments of the three-launch sort
constexpr int PL_COL_THREADS = 256;
constexpr int PL_COL_PER_THREAD = PL_BLOCKS_MAX / PL_COL_THREADS;
static_assert(PM_SEG >= MAX_GROUPS, "a segment must hold its block's per-group counts");

__global__ __launch_bounds__(PERM_WAVES * WAVE) void permute_kernel(
    const int32_t* __restrict__ ids, int N, int g_begin, int n_groups, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos) {
  __shared__ int s_cnt[PERM_WAVES * MAX_GROUPS];
  __shared__ int s_off[MAX_GROUPS];
  __shared__ uint16_t s_key[PERM_KEY_CAP];
  block_counting_sort<PERM_WAVES, false>(ids, N, g_begin, n_groups, counts, offsets, sorted_pair,
                                         pair_pos, s_cnt, s_off, s_key, PERM_KEY_CAP);
}

// The pairs of [p0, p1) given s_off[g] = row of group g's first pair in the
// segment: per-wave histograms, the count of each group in the waves before,
// then ballot ranks in pair order from the base.  s_cnt must be zero.
__device__ __forceinline__ void segment_sort(const int32_t* __restrict__ ids, int p0, int p1, int g_begin,
                                             int n_groups, const int* s_off, int* s_cnt,
                                             int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos) {
  const int tid = threadIdx.x;
  const int wv = tid / WAVE;
  const int per_wave = (p1 - p0 + PM_WAVES - 1) / PM_WAVES;
  const int seg = ((per_wave + WAVE - 1) / WAVE) * WAVE;
  const int w_begin = min(p1, p0 + wv * seg);
  const int w_end = min(p1, w_begin + seg);
  int* my_cnt = s_cnt + wv * MAX_GROUPS;
  sort_histogram<false, false>(nullptr, ids, w_begin, w_end, g_begin, n_groups, my_cnt);
  __syncthreads();
  for (int g = tid; g < n_groups; g += PM_THREADS) {
    int run = 0;
    for (int w = 0; w < PM_WAVES; ++w) {
      const int c = s_cnt[w * MAX_GROUPS + g];
      s_cnt[w * MAX_GROUPS + g] = run;
      run += c;
    }
  }
  __syncthreads();
  sort_scatter<false, false>(nullptr, ids, w_begin, w_end, g_begin, n_groups, s_off, my_cnt, sorted_pair,
                             pair_pos);
}

__global__ __launch_bounds__(PM_THREADS) void permute_multi_kernel(
    const int32_t* __restrict__ ids, int N, int g_begin, int n_groups, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos) {
  __shared__ int s_tot[MAX_GROUPS];
  __shared__ int s_bef[MAX_GROUPS];
  __shared__ int s_off[MAX_GROUPS];
  __shared__ int s_cnt[PM_WAVES * MAX_GROUPS];
  const int tid = threadIdx.x;
  const int wv = tid / WAVE;
  const int l = lane_id();
  const int p0 = blockIdx.x * PM_SEG;
  const int p1 = min(N, p0 + PM_SEG);

  for (int g = tid; g < n_groups; g += PM_THREADS) {
    s_tot[g] = 0;
    s_bef[g] = 0;
  }
  for (int i = tid; i < PM_WAVES * MAX_GROUPS; i += PM_THREADS) s_cnt[i] = 0;
  __syncthreads();

  // 1. every pair's group, counted; PM_UNROLL clamped loads in flight.
  for (int q0 = tid; q0 < N; q0 += PM_THREADS * PM_UNROLL) {
    int key[PM_UNROLL];
#pragma unroll
    for (int u = 0; u < PM_UNROLL; ++u)
      key[u] = pair_key<false>(ids, min(q0 + u * PM_THREADS, N - 1), g_begin, n_groups);
#pragma unroll
    for (int u = 0; u < PM_UNROLL; ++u) {
      const int p = q0 + u * PM_THREADS;
      if (p < N && key[u] < n_groups) {
        atomicAdd(&s_tot[key[u]], 1);
        if (p < p0) atomicAdd(&s_bef[key[u]], 1);
      }
    }
  }
  __syncthreads();

  // 2. offsets (exclusive scan of the totals) and this segment's base per group
  if (wv == 0) {
    int base = 0;
    for (int g0 = 0; g0 < n_groups; g0 += WAVE) {
      const int g = g0 + l;
      const int c = g < n_groups ? s_tot[g] : 0;
      const int incl = wave_inclusive_scan(c);
      if (g < n_groups) {
        const int off = base + incl - c;
        s_off[g] = off + s_bef[g];
        if (blockIdx.x == 0) {
          counts[g] = c;
          offsets[g] = off;
        }
      }
      base += __shfl(incl, WAVE - 1, WAVE);
    }
    if (blockIdx.x == 0 && l == 0) offsets[n_groups] = base;
  }
  __syncthreads();

  segment_sort(ids, p0, p1, g_begin, n_groups, s_off, s_cnt, sorted_pair, pair_pos);
}

// Three-launch sort, above PM_SWEEP_MAX pairs.  Segment b is [b*len, (b+1)*len),
// the last one running to N.
__device__ __forceinline__ void pl_segment(int N, int nb, int len, int b, int& p0, int& p1) {
  p0 = b * len;
  p1 = (b == nb - 1) ? N : p0 + len;
}

__global__ __launch_bounds__(PM_THREADS) void permute_count_kernel(const int32_t* __restrict__ ids, int N, int nb,
                                                                   int len, int g_begin, int n_groups,
                                                                   int32_t* __restrict__ pair_pos) {
  __shared__ int s_cnt[MAX_GROUPS];
  const int tid = threadIdx.x;
  int p0, p1;
  pl_segment(N, nb, len, blockIdx.x, p0, p1);
  for (int g = tid; g < n_groups; g += PM_THREADS) s_cnt[g] = 0;
  __syncthreads();
  for (int q0 = p0 + tid; q0 < p1; q0 += PM_THREADS * PM_UNROLL) {
    int key[PM_UNROLL];
#pragma unroll
    for (int u = 0; u < PM_UNROLL; ++u)
      key[u] = pair_key<false>(ids, min(q0 + u * PM_THREADS, p1 - 1), g_begin, n_groups);
#pragma unroll
    for (int u = 0; u < PM_UNROLL; ++u)
      if (q0 + u * PM_THREADS < p1 && key[u] < n_groups) atomicAdd(&s_cnt[key[u]], 1);
  }
  __syncthreads();
  for (int g = tid; g < n_groups; g += PM_THREADS) pair_pos[p0 + g] = s_cnt[g];
}

// Block g: exclusive scan of column g (one value per segment, nb <= PL_BLOCKS_MAX),
// written back in place; the column total is counts[g].
__global__ __launch_bounds__(PL_COL_THREADS) void permute_columns_kernel(int nb, int len,
                                                                         int32_t* __restrict__ counts,
                                                                         int32_t* __restrict__ pair_pos) {
  __shared__ int s_wave[PL_COL_THREADS / WAVE];
  const int g = blockIdx.x;
  const int tid = threadIdx.x;
  const int l = lane_id();
  const int wv = tid / WAVE;
  const int b0 = tid * PL_COL_PER_THREAD;
  int v[PL_COL_PER_THREAD];
  int sum = 0;
#pragma unroll
  for (int u = 0; u < PL_COL_PER_THREAD; ++u) {
    const int b = b0 + u;
    v[u] = b < nb ? pair_pos[static_cast<long long>(b) * len + g] : 0;
    sum += v[u];
  }
  const int incl = wave_inclusive_scan(sum);
  if (l == WAVE - 1) s_wave[wv] = incl;
  __syncthreads();
  int before = incl - sum;
  for (int w = 0; w < wv; ++w) before += s_wave[w];
#pragma unroll
  for (int u = 0; u < PL_COL_PER_THREAD; ++u) {
    const int b = b0 + u;
    if (b < nb) pair_pos[static_cast<long long>(b) * len + g] = before;
    before += v[u];
  }
  if (tid == PL_COL_THREADS - 1) counts[g] = before;
}

__global__ __launch_bounds__(PM_THREADS) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int N, int nb, int len, int g_begin, int n_groups,
    const int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
    int32_t* __restrict__ pair_pos) {
  __shared__ int s_off[MAX_GROUPS];
  __shared__ int s_cnt[PM_WAVES * MAX_GROUPS];
  const int tid = threadIdx.x;
  const int wv = tid / WAVE;
  const int l = lane_id();
  int p0, p1;
  pl_segment(N, nb, len, blockIdx.x, p0, p1);
  for (int g = tid; g < n_groups; g += PM_THREADS) s_off[g] = pair_pos[p0 + g];
  for (int i = tid; i < PM_WAVES * MAX_GROUPS; i += PM_THREADS) s_cnt[i] = 0;
  __syncthreads();
  if (wv == 0) {
    int base = 0;
    for (int g0 = 0; g0 < n_groups; g0 += WAVE) {
      const int g = g0 + l;
      const int c = g < n_groups ? counts[g] : 0;
      const int incl = wave_inclusive_scan(c);
      if (g < n_groups) {
        const int off = base + incl - c;
        s_off[g] += off;
        if (blockIdx.x == 0) offsets[g] = off;
      }
      base += __shfl(incl, WAVE - 1, WAVE);
    }
    if (blockIdx.x == 0 && l == 0) offsets[n_groups] = base;
  }
  __syncthreads();
  segment_sort(ids, p0, p1, g_begin, n_groups, s_off, s_cnt, sorted_pair, pair_pos);
}

bool permute_uses_blocks(int T, int kk) { return static_cast<long long>(T) * kk > PERM_ONE_BLOCK_MAX; }

void launch_permute(const int32_t* ids, int T, int kk, int g_begin, int n_groups, int32_t* counts,
                    int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, hipStream_t s) {
  const int N = T * kk;
  if (N > PM_SWEEP_MAX) {
    const int nb = std::min(N / PM_SEG, PL_BLOCKS_MAX);
    const int len = N / nb;   // >= PM_SEG, so every segment can park n_groups counts
    hipLaunchKernelGGL(permute_count_kernel, dim3(nb), dim3(PM_THREADS), 0, s, ids, N, nb, len, g_begin,
                       n_groups, pair_pos);
    hipLaunchKernelGGL(permute_columns_kernel, dim3(n_groups), dim3(PL_COL_THREADS), 0, s, nb, len, counts,
                       pair_pos);
    hipLaunchKernelGGL(permute_scatter_kernel, dim3(nb), dim3(PM_THREADS), 0, s, ids, N, nb, len, g_begin,
                       n_groups, counts, offsets, sorted_pair, pair_pos);
    return;
  }
  if (permute_uses_blocks(T, kk)) {
    hipLaunchKernelGGL(permute_multi_kernel, dim3((N + PM_SEG - 1) / PM_SEG), dim3(PM_THREADS), 0, s, ids, N,
                       g_begin, n_groups, counts, offsets, sorted_pair, pair_pos);
    return;
  }
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(PERM_WAVES * WAVE), 0, s, ids, N, g_begin,
                     n_groups, counts, offsets, sorted_pair, pair_pos);
}

}  // namespace moe
