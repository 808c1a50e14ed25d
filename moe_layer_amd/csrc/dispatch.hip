// EP dispatch, send side: every routed (token, slot) pair goes to the rank that
// owns its expert (Moebius review, problem definition: in the EP layout tokens
// reach the expert's GPU by an all-to-all; Sem-MoE notes, motivation: one
// all-to-all out to the remote experts and one back).  One send row per pair,
// rows grouped by destination rank, ascending pair id within a rank; pairs of
// experts at or beyond P * E_local (shared experts) stay local.
//
// One launch, no block waits for another.  Block b owns tokens
// [b*TB, (b+1)*TB) and so a contiguous range of pairs.  A pair's send row is
//     (pairs of lower ranks) + (pairs of its rank before this block) + (its
//     rank among this block's pairs of that rank)
// and every block computes the first two terms itself, from a sweep of the
// whole routing table (T*kk ids, a few KB to some 100 KB, served by L2): in
// packed per-lane counters for large tables and up to 8 ranks, else with one
// LDS atomic add per id.  Then one wave ranks the block's own pairs in
// pair order (ballots, stable) and the block's waves copy its token rows:
// each row is read from HBM once and stored to every send row of that token.
// The first token slice is loaded before the sweep, so the HBM read overlaps
// the counting.
#include <algorithm>

#include "common.hpp"
#include "moe_internal.h"

namespace moe {

constexpr int DP_THREADS = 512;
constexpr int DP_WAVES = DP_THREADS / WAVE;
constexpr int DP_POS_CAP = 4096;   // pairs per block (LDS send rows)
constexpr int DP_ID_UNROLL = 8;    // 16-byte id loads in flight per lane in the sweep
constexpr int DP_PACKED_P = 8;     // ranks counted in packed per-lane fields ...
constexpr int DP_PACKED_MIN_N = 8192;  // ... for routing tables of this many ids or more

// Lanes of the wave holding the same key as this lane (among `active` lanes).
__device__ __forceinline__ unsigned long long same_key_lanes(int key, bool active, int nbits) {
  unsigned long long m = __ballot(active);
  for (int b = 0; b < nbits; ++b) {
    const int bit = (key >> b) & 1;
    const unsigned long long bm = __ballot(bit);
    m &= bit ? bm : ~bm;
  }
  return m;
}

struct DispatchArgs {
  const uint4* x;
  const int32_t* ids;
  int T, kk, E_local, e_shift, P, TB, C;
  int nt;   // non-temporal send stores (measured faster for send buffers up to 32 MiB)
  int32_t *counts, *offsets, *send_order, *pair_pos, *send_ids;
  uint4* send_x;
};

// Owning rank of an expert id, P when the pair is not sent (id < 0 or
// id >= P * E_local).  Branch-free: a negative id read as unsigned is at
// least 2^31, which divides to at least P.
template <bool kShift>
__device__ __forceinline__ int rank_key(int id, const DispatchArgs& a) {
  const unsigned u = static_cast<unsigned>(id);
  const unsigned r = kShift ? u >> a.e_shift : u / static_cast<unsigned>(a.E_local);
  return static_cast<int>(min(r, static_cast<unsigned>(a.P)));
}

// Packed count of one id: 1 in the 8-bit field of its rank (0 if not sent).
__device__ __forceinline__ unsigned long long packed_one(int key, int P) {
  return key < P ? 1ull << (8 * (key & 7)) : 0ull;
}

template <int NP>
__device__ __forceinline__ void widen_counts(unsigned long long pt, unsigned long long pb, int (&tot)[NP],
                                             int (&bef)[NP]) {
#pragma unroll
  for (int d = 0; d < NP; ++d) {
    tot[d] += static_cast<int>((pt >> (8 * d)) & 0xFFu);
    bef[d] += static_cast<int>((pb >> (8 * d)) & 0xFFu);
  }
}

// Sum over the 64 lanes (all active) with DPP lane moves, no LDS: inclusive
// prefix sums inside each row of 16 lanes (row shifts by 1, 2, 4, 8; lanes
// shifted in from outside the row add 0), then lane 15 of a row added to the
// next row and lane 31 to rows 2 and 3; lane 63 ends with the total.
__device__ __forceinline__ int wave_total(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return __builtin_amdgcn_readlane(v, 63);
}

// One copy item: U 64-lane vector columns of one token row.  Indexes past the
// row end are clamped to its last vector: those lanes load and store that
// vector again (same value, same place), so no access sits behind a branch.
template <int U>
__device__ __forceinline__ void load_item(const DispatchArgs& a, int tok, int slice, u32x4_t (&v)[U]) {
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.x) + static_cast<size_t>(tok) * a.C;
  const int c0 = slice * U * WAVE + lane_id();
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = src[min(c0 + u * WAVE, a.C - 1)];
}

// Store one item to the send rows of its token (pos[j] < 0: slot j not sent).
template <int U>
__device__ __forceinline__ void store_item(const DispatchArgs& a, const int* pos, int slice,
                                           const u32x4_t (&v)[U]) {
  const int c0 = slice * U * WAVE + lane_id();
  int c[U];
#pragma unroll
  for (int u = 0; u < U; ++u) c[u] = min(c0 + u * WAVE, a.C - 1);
  for (int j = 0; j < a.kk; ++j) {
    const int row = __builtin_amdgcn_readfirstlane(pos[j]);
    if (row < 0) continue;
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(a.send_x) + static_cast<size_t>(row) * a.C;
    if (a.nt) {
#pragma unroll
      for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], dst + c[u]);
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) dst[c[u]] = v[u];
    }
  }
}

template <int U, bool kPacked, bool kShift>
__global__ __launch_bounds__(DP_THREADS) void dispatch_kernel(DispatchArgs a) {
  __shared__ int s_tot[MAX_GROUPS];
  __shared__ int s_base[MAX_GROUPS];
  __shared__ int s_pos[DP_POS_CAP];
  const int tid = threadIdx.x;
  const int w = tid / WAVE;
  const int l = lane_id();
  const unsigned long long lower = (1ull << l) - 1ull;
  const int t0 = blockIdx.x * a.TB;
  const int tn = max(0, min(a.TB, a.T - t0));
  const int r0 = t0 * a.kk;
  const int nr = tn * a.kk;
  const int N = a.T * a.kk;
  const int S = ((a.C + WAVE - 1) / WAVE + U - 1) / U;   // copy items per token
  const int n_items = tn * S;

  // Wave 0's first 64 own ids and every wave's first copy item are loaded
  // before the sweep, so their latency hides behind it.
  const int id0 = (w == 0 && l < nr) ? a.ids[r0 + l] : -1;
  u32x4_t v[U];
  if (w < n_items) load_item<U>(a, t0 + w / S, w % S, v);

  for (int i = tid; i < a.P; i += DP_THREADS) {
    s_tot[i] = 0;
    s_base[i] = 0;
  }
  __syncthreads();

  // Sweep: per-rank totals, and per-rank counts of the pairs before this
  // block's.  Counts are order-free integer sums.  Loads are clamped into the
  // table, so all of them are unconditional, and eight are in flight.
  //   kPacked (P <= 8, large tables): four ids per lane per 16-byte load;
  //   wave w takes the 256-id spans w, w + 8, ...; a lane counts in 8-bit
  //   fields of one 64-bit word per quantity (at most 32 ids per step, so no
  //   field overflows), widened into 32-bit counters after every step and
  //   summed over the wave at the end.  Whether a span lies before this
  //   block's pairs is decided per span; only the span that straddles the
  //   block start tests each id.  The N % 4 ids after the last whole vector
  //   are counted by wave 0.
  //   otherwise (small tables, or more ranks): one id per lane, wave w takes
  //   the 64-id groups w, w + 8, ..., one LDS atomic add per id.
  int tot[kPacked ? DP_PACKED_P : 1] = {}, bef[kPacked ? DP_PACKED_P : 1] = {};
  if (kPacked) {
    const int nfull = N / 4;
    const int4* ids4 = reinterpret_cast<const int4*>(a.ids);
    for (int q0 = w * WAVE; q0 < nfull; q0 += DP_WAVES * WAVE * DP_ID_UNROLL) {
      int4 c[DP_ID_UNROLL];
#pragma unroll
      for (int u = 0; u < DP_ID_UNROLL; ++u) c[u] = ids4[min(q0 + u * DP_WAVES * WAVE + l, nfull - 1)];
      unsigned long long pt = 0, pb = 0;
#pragma unroll
      for (int u = 0; u < DP_ID_UNROLL; ++u) {
        const int qb = q0 + u * DP_WAVES * WAVE;   // the span's first vector (wave-uniform)
        const bool valid = qb + l < nfull;
        const int e[4] = {c[u].x, c[u].y, c[u].z, c[u].w};
        int k[4];
        unsigned long long st = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          k[j] = valid ? rank_key<kShift>(e[j], a) : a.P;
          st += packed_one(k[j], a.P);
        }
        pt += st;
        if (4 * (qb + WAVE) <= r0) {
          pb += st;
        } else if (4 * qb < r0) {
#pragma unroll
          for (int j = 0; j < 4; ++j) pb += 4 * (qb + l) + j < r0 ? packed_one(k[j], a.P) : 0ull;
        }
      }
      widen_counts(pt, pb, tot, bef);
    }
    if (w == 0 && (N & 3)) {
      const int p = 4 * nfull + l;
      const int key = p < N ? rank_key<kShift>(a.ids[min(p, N - 1)], a) : a.P;
      const unsigned long long st = packed_one(key, a.P);
      widen_counts(st, p < r0 ? st : 0ull, tot, bef);
    }
#pragma unroll
    for (int d = 0; d < DP_PACKED_P; ++d) {
      if (d >= a.P) break;
      const int t = wave_total(tot[d]);
      const int b = wave_total(bef[d]);
      if (l == 0) {
        atomicAdd(s_tot + d, t);
        if (b) atomicAdd(s_base + d, b);
      }
    }
  } else {
    for (int g0 = w; g0 * WAVE < N; g0 += DP_WAVES * DP_ID_UNROLL) {
      int id[DP_ID_UNROLL];
#pragma unroll
      for (int u = 0; u < DP_ID_UNROLL; ++u) id[u] = a.ids[min((g0 + u * DP_WAVES) * WAVE + l, N - 1)];
#pragma unroll
      for (int u = 0; u < DP_ID_UNROLL; ++u) {
        const int p = (g0 + u * DP_WAVES) * WAVE + l;
        const int key = p < N ? rank_key<kShift>(id[u], a) : a.P;
        if (key < a.P) {
          atomicAdd(s_tot + key, 1);
          if (p < r0) atomicAdd(s_base + key, 1);
        }
      }
    }
  }
  __syncthreads();

  // Exclusive scan of the totals; s_base becomes this block's first send row
  // of each rank.  Block 0 publishes counts and offsets.
  if (w == 0) {
    int base = 0;
    for (int g0 = 0; g0 < a.P; g0 += WAVE) {
      const int g = g0 + l;
      const int c = g < a.P ? s_tot[g] : 0;
      const int incl = wave_inclusive_scan(c);
      if (g < a.P) {
        s_base[g] += base + incl - c;
        if (blockIdx.x == 0) {
          a.counts[g] = c;
          a.offsets[g] = base + incl - c;
        }
      }
      base += __shfl(incl, WAVE - 1, WAVE);
    }
    if (blockIdx.x == 0 && l == 0) a.offsets[a.P] = base;
  }
  __syncthreads();

  // Rank this block's pairs in pair order (stable): wave 0, 64 pairs a step.
  if (w == 0) {
    const int nbits = 32 - __clz(a.P);
    for (int i0 = 0; i0 < nr; i0 += WAVE) {
      const int i = i0 + l;
      const bool active = i < nr;
      const int p = r0 + i;
      const int id = i0 == 0 ? id0 : (active ? a.ids[p] : -1);
      const int key = rank_key<kShift>(id, a);
      const bool kept = key < a.P;
      const unsigned long long m = same_key_lanes(key, kept, nbits);
      const int run = kept ? s_base[key] : 0;
      const int pos = kept ? run + __popcll(m & lower) : -1;
      if (active) {
        a.pair_pos[p] = pos;
        s_pos[i] = pos;
      }
      if (kept) {
        a.send_order[pos] = p;
        a.send_ids[pos] = id;
      }
      __builtin_amdgcn_wave_barrier();
      if (kept && (m & lower) == 0) s_base[key] = run + __popcll(m);
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();

  // Copy: item it = (token it / S, slice it % S); the slice goes to every
  // send row of the token (row numbers are wave-uniform LDS reads).
  for (int it = w; it < n_items; it += DP_WAVES) {
    if (it != w) load_item<U>(a, t0 + it / S, it % S, v);
    store_item<U>(a, s_pos + (it / S) * a.kk, it % S, v);
  }
}

template <bool kPacked, bool kShift>
void launch_u(int U, int blocks, const DispatchArgs& a, hipStream_t s) {
  switch (U) {
    case 8: hipLaunchKernelGGL((dispatch_kernel<8, kPacked, kShift>), dim3(blocks), dim3(DP_THREADS), 0, s, a); break;
    case 4: hipLaunchKernelGGL((dispatch_kernel<4, kPacked, kShift>), dim3(blocks), dim3(DP_THREADS), 0, s, a); break;
    case 2: hipLaunchKernelGGL((dispatch_kernel<2, kPacked, kShift>), dim3(blocks), dim3(DP_THREADS), 0, s, a); break;
    default: hipLaunchKernelGGL((dispatch_kernel<1, kPacked, kShift>), dim3(blocks), dim3(DP_THREADS), 0, s, a); break;
  }
}

void launch_dispatch(int dtype, const void* x, const int32_t* ids, int T, int kk, int H, int E_local,
                     int P, int32_t* counts, int32_t* offsets, int32_t* send_order, int32_t* pair_pos,
                     void* send_x, int32_t* send_ids, hipStream_t s) {
  DispatchArgs a;
  a.x = static_cast<const uint4*>(x);
  a.ids = ids;
  a.T = T;
  a.kk = kk;
  a.E_local = E_local;
  a.e_shift = (E_local & (E_local - 1)) == 0 ? __builtin_ctz(static_cast<unsigned>(E_local)) : -1;
  a.P = P;
  a.C = static_cast<int>((static_cast<long long>(H) * (dtype == 1 ? 2 : 4)) / 16);
  a.counts = counts;
  a.offsets = offsets;
  a.send_order = send_order;
  a.pair_pos = pair_pos;
  a.send_ids = send_ids;
  a.send_x = static_cast<uint4*>(send_x);
  a.nt = static_cast<long long>(T) * kk * a.C * 16 <= (32LL << 20);
  // Tokens per block: one up to ~1000 tokens (a block per token), then enough
  // to keep the grid near 512 blocks so the id sweeps stay a small share of
  // the copy; at most DP_POS_CAP pairs per block.
  a.TB = std::max(1, std::min(T / 512, DP_POS_CAP / kk));
  const int blocks = T > 0 ? (T + a.TB - 1) / a.TB : 1;
  // Vector columns per copy item: spread one block's rows over its 8 waves.
  const int C64 = (a.C + WAVE - 1) / WAVE;
  const int want = (C64 * a.TB + DP_WAVES - 1) / DP_WAVES;
  const int U = want >= 8 ? 8 : want >= 4 ? 4 : want >= 2 ? 2 : 1;
  const bool shift = a.e_shift >= 0;
  if (P <= DP_PACKED_P && static_cast<long long>(T) * kk >= DP_PACKED_MIN_N) {
    if (shift) launch_u<true, true>(U, blocks, a, s);
    else launch_u<true, false>(U, blocks, a, s);
  } else {
    if (shift) launch_u<false, true>(U, blocks, a, s);
    else launch_u<false, false>(U, blocks, a, s);
  }
}

}  // namespace moe
