// Request scheduling under data-parallel attention (Sem-MoE notes, online data
// scheduling): each request goes to the rank (cluster) its tokens are most
// affine to, S_r = argmax_j sum_{i in r} R_ij, and every E consecutive
// requests are spread over all E ranks.
//
// One launch, no block waits for another.  Block r counts request r's tokens
// per cluster (R given as the cluster of every vocabulary id; for E <= 8 in
// packed per-thread counters, else LDS atomics) into an LDS histogram,
// publishes the E counts with agent-scope stores and picks S_r with one
// wave-wide max.  The last block of each group of E consecutive
// requests to finish (an integer arrival counter, reset by that block) then
// runs the balancing greedy for the group: lane j stands for rank j, and for
// each request in arrival order the free lane with the largest count (ties to
// the lowest rank) takes it.  Token ids outside [0, vocab) and clusters
// outside [0, E) are not counted; request bounds are clamped into the token
// array, so every access stays inside the caller's buffers.
#include "common.hpp"
#include "moe_internal.h"

namespace moe {

constexpr int SCHED_THREADS = 256;
constexpr int SCHED_UNROLL = 16;
constexpr int SCHED_GROUP_LOADS = 8;   // a group's count rows loaded at once by the balancing wave

// Sum over the 64 lanes (all active) with DPP row shifts and broadcasts.
__device__ __forceinline__ int wave_total_i(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

// The largest (score, -rank) over the lanes where `ok`, as a rank; -1 if
// none.  All 64 lanes active; ties go to the lowest rank.  The key
// score * 64 + (63 - lane) fits 31 bits (scores < 2^25), and the max runs on
// DPP moves: row shifts by 1, 2, 4, 8, then lane 15 of a row into the next row
// and lane 31 into rows 2 and 3 (lanes moved in from nowhere bring -1);
// lane 63 ends with the maximum.
__device__ __forceinline__ int wave_best_rank(int score, bool ok) {
  int k = ok ? (score << 6) | (63 - lane_id()) : -1;
  k = max(k, __builtin_amdgcn_update_dpp(-1, k, 0x111, 0xf, 0xf, false));   // row_shr:1
  k = max(k, __builtin_amdgcn_update_dpp(-1, k, 0x112, 0xf, 0xf, false));   // row_shr:2
  k = max(k, __builtin_amdgcn_update_dpp(-1, k, 0x114, 0xf, 0xf, false));   // row_shr:4
  k = max(k, __builtin_amdgcn_update_dpp(-1, k, 0x118, 0xf, 0xf, false));   // row_shr:8
  k = max(k, __builtin_amdgcn_update_dpp(-1, k, 0x142, 0xa, 0xf, false));   // row_bcast:15
  k = max(k, __builtin_amdgcn_update_dpp(-1, k, 0x143, 0xc, 0xf, false));   // row_bcast:31
  const int best = __builtin_amdgcn_readlane(k, 63);
  return best < 0 ? -1 : 63 - (best & 63);
}

struct SchedArgs {
  const int32_t* tokens;
  const int32_t* offsets;
  const int32_t* cluster;
  int n_tokens, n_req, vocab, E;
  int32_t *scores, *affinity, *assigned;
  int* ctr;
};

template <bool kPacked>
__global__ __launch_bounds__(SCHED_THREADS) void schedule_kernel(SchedArgs a) {
  __shared__ int s_hist[MAX_SCHED_RANKS];
  __shared__ int s_grp[MAX_SCHED_RANKS * MAX_SCHED_RANKS];   // a group's counts (balancing)
  __shared__ int s_last;
  const int r = blockIdx.x;
  const int tid = threadIdx.x;
  const int l = lane_id();
  if (tid < a.E) s_hist[tid] = 0;
  __syncthreads();

  const int lo = min(max(a.offsets[r], 0), a.n_tokens);
  const int hi = min(max(a.offsets[r + 1], lo), a.n_tokens);
  // Sixteen token loads, then sixteen cluster loads, in flight per thread
  // (indexes clamped into the request, so all are unconditional).
  //   kPacked (E <= 8): each thread counts in 8-bit fields of one 64-bit word
  //   (at most 16 per step), summed over the wave with DPP and added to LDS
  //   once per wave; otherwise one LDS atomic add per token.
  unsigned long long packed = 0;
  int cnt[kPacked ? 8 : 1] = {};
  for (int p0 = lo + tid; p0 < hi; p0 += SCHED_THREADS * SCHED_UNROLL) {
    int t[SCHED_UNROLL], c[SCHED_UNROLL];
#pragma unroll
    for (int u = 0; u < SCHED_UNROLL; ++u) t[u] = a.tokens[min(p0 + u * SCHED_THREADS, hi - 1)];
#pragma unroll
    for (int u = 0; u < SCHED_UNROLL; ++u) {
      const bool in = p0 + u * SCHED_THREADS < hi && t[u] >= 0 && t[u] < a.vocab;
      c[u] = a.cluster[in ? t[u] : 0];
      if (!in) c[u] = -1;
    }
    packed = 0;
#pragma unroll
    for (int u = 0; u < SCHED_UNROLL; ++u) {
      const bool ok = c[u] >= 0 && c[u] < a.E;
      if (kPacked) {
        packed += ok ? 1ull << (8 * (c[u] & 7)) : 0ull;
      } else if (ok) {
        atomicAdd(s_hist + c[u], 1);
      }
    }
    if (kPacked) {
#pragma unroll
      for (int j = 0; j < 8; ++j) cnt[j] += static_cast<int>((packed >> (8 * j)) & 0xFFu);
    }
  }
  if (kPacked) {
    // every wave reaches this point (loop bounds differ per thread, not the
    // code after the loop)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (j >= a.E) break;
      const int tot = wave_total_i(cnt[j]);
      if (l == 0 && tot) atomicAdd(s_hist + j, tot);
    }
  }
  __syncthreads();

  const int g = r / a.E;
  const int g0 = g * a.E;
  const int gn = min(a.E, a.n_req - g0);
  if (tid < WAVE) {
    const int sc = l < a.E ? s_hist[l] : 0;
    if (l < a.E) st_agent(a.scores + static_cast<size_t>(r) * a.E + l, sc);
    const int best = wave_best_rank(sc, l < a.E);
    if (l == 0) a.affinity[r] = best;
  }
  if (!last_to_arrive(a.ctr + g, gn, &s_last)) return;

  // Balancing of group g: lane j = rank j.  The group's counts are loaded
  // first (all loads in flight), then the greedy runs from LDS.
  if (tid < WAVE) {
    for (int i0 = 0; i0 < gn; i0 += SCHED_GROUP_LOADS) {
      int v[SCHED_GROUP_LOADS];
#pragma unroll
      for (int u = 0; u < SCHED_GROUP_LOADS; ++u) {
        const int i = min(i0 + u, gn - 1);
        v[u] = l < a.E ? ld_agent(a.scores + static_cast<size_t>(g0 + i) * a.E + l) : 0;
      }
#pragma unroll
      for (int u = 0; u < SCHED_GROUP_LOADS; ++u)
        if (i0 + u < gn && l < a.E) s_grp[(i0 + u) * MAX_SCHED_RANKS + l] = v[u];
    }
    __builtin_amdgcn_wave_barrier();
    bool taken = false;
    for (int i = 0; i < gn; ++i) {
      const int sc = l < a.E ? s_grp[i * MAX_SCHED_RANKS + l] : 0;
      const int best = wave_best_rank(sc, l < a.E && !taken);
      if (l == best) taken = true;
      if (l == 0) a.assigned[g0 + i] = best;
    }
  }
}

size_t schedule_workspace_bytes(int n_req, int E) {
  if (n_req <= 0 || E < 1) return 0;
  const size_t groups = (static_cast<size_t>(n_req) + E - 1) / E;
  return (groups * sizeof(int) + 255) & ~static_cast<size_t>(255);
}

void launch_schedule(const int32_t* tokens, int n_tokens, const int32_t* offsets, int n_req,
                     const int32_t* cluster, int vocab, int E, int32_t* scores, int32_t* affinity,
                     int32_t* assigned, void* ws, hipStream_t s) {
  if (n_req <= 0) return;
  SchedArgs a{tokens, offsets, cluster, n_tokens, n_req, vocab, E, scores, affinity, assigned,
              static_cast<int*>(ws)};
  if (E <= 8)
    hipLaunchKernelGGL(schedule_kernel<true>, dim3(n_req), dim3(SCHED_THREADS), 0, s, a);
  else
    hipLaunchKernelGGL(schedule_kernel<false>, dim3(n_req), dim3(SCHED_THREADS), 0, s, a);
}

}  // namespace moe
