// Expert down-projection for short rows (bf16 storage, fp32 accumulate):
//   y_pair[r] = W2_g a[r]   from W2_g (H, I'), rows of I' * 2 <= 512 bytes
// (Moebius review, §3.1: W2 as (., H, I); in the TP view each rank holds an
// I/P slice, so its W2 rows are short -- 384 bytes for Qwen3-235B-A22B at
// P = 8.  Decode MoE GEMMs are memory-bound, §2.1 and Fig. 3.)
//
// With rows this short the wave-streaming kernel's 512-byte chunk loads use
// only part of each load (384 of 512 bytes at I' = 192), every work item is a
// single chunk step, and a wave keeps one 16-row tile in flight while it
// multiplies the previous one: its weight stream ran at three quarters of
// the rate of the long-row kernels, exactly the share of useful bytes.
//
// Here a 16-row weight tile is one contiguous block of 16 * I' * 2 bytes,
// fetched with I' * 2 / 64 loads of 1 KB (64 lanes x 16 bytes, all used).  A
// step is one tile of one pass (16 * NT token rows) over the whole K, so no
// step is ever split and there are no partial sums.  Steps are ordered group
// by group, pass by pass, tile by tile (all H / 16 tiles of a pass in a row),
// and the flattened sequence is cut into equal contiguous ranges, one per
// wave (an eighth of them per XCD, as in expert_gemm.hip).  A wave keeps its
// pass's token fragments in registers for the whole run of tiles and loads
// the next pass's fragments when its weight loads reach that pass; its
// weight loads run SH_RING - 1 tiles ahead of the tile it multiplies.  Loads
// past the end of the range re-read its last tile, so every step issues the
// same loads.  Each tile passes through the wave's private LDS tile into the
// 16x16x32 MFMA operand layout (lane l: row l % 16, bytes 16 * (l / 16) of
// each 64-byte K fragment).  Token rows past the pass repeat its last row and
// are never stored; every output element is written by exactly one lane.
// Groups taken by the LDS-tiled kernels (expert_tile.hip) get no steps, by
// the same rule as in the wave-streaming kernel.
#include "common.hpp"
#include "moe_internal.h"
#include "stream_ops.hpp"

namespace moe {

namespace {

constexpr int SH_WAVES = 4;  // waves per block (one block per CU)
constexpr int SH_RING = 4;   // weight tiles a wave holds: the one it multiplies and the next three
constexpr long long SH_KEEP_BYTES = 32LL << 20;  // weights of multi-pass groups read with the ordinary policy, at most (the chip's L2)

// One step of the sequence, decoded (wave-uniform): group, weight tile j,
// the group's first sorted row, and the pass's rows [t0, m_end).
struct SStep {
  int g, j, row0, t0, m_end;
};

template <int NT>
__device__ __forceinline__ SStep sh_decode(const XArgs& a, const int* s_istart, const int* s_off, int q) {
  int lo = 0, hi = a.n_groups;  // the last group with s_istart[lo] <= q holds step q
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (uni(s_istart[mid]) <= q) lo = mid;
    else hi = mid;
  }
  SStep d;
  d.g = lo;
  d.row0 = uni(s_off[lo]);
  const int m = uni(s_off[lo + 1]) - d.row0;
  const int ps = pass_rows<NT>(m);
  const int local = q - uni(s_istart[lo]);
  const int p = local / a.n_tiles;
  d.j = local - p * a.n_tiles;
  d.t0 = p * ps;
  d.m_end = min(m, d.t0 + ps);
  return d;
}

template <int KF>
constexpr int sh_pitch() { return KF * FRAG_BYTES + 16; }  // LDS row pitch of the transpose tile

// The stream of one wave, after the step table is built (NT token tiles per
// pass; KEEP: weights read with the ordinary policy instead of streamed).
template <int KF, int NT, bool KEEP>
__device__ __forceinline__ void short_body(const XArgs& a, const int* s_istart, const int* s_off, char* tile, int wv) {
  constexpr int RB = KF * FRAG_BYTES;  // bytes of a weight row and of an activation row
  constexpr int PITCH = sh_pitch<KF>();
  const int l = lane_id();
  const int lrow = l & 15;
  const int lq = l >> 4;

  const int Q = uni(s_istart[a.n_groups]);
  const int nblk = static_cast<int>(gridDim.x);
  const int W = min(nblk * SH_WAVES, Q);
  int w;
  if (nblk % 8 == 0) {
    const int xcd = blockIdx.x % 8;
    const int kx = wv * (nblk / 8) + blockIdx.x / 8;
    const int xlo = static_cast<int>(static_cast<long long>(W) * xcd / 8);
    if (kx >= static_cast<int>(static_cast<long long>(W) * (xcd + 1) / 8) - xlo) return;  // wave-uniform
    w = xlo + kx;
  } else {
    w = wv * nblk + blockIdx.x;
    if (w >= W) return;  // wave-uniform
  }
  const int q0 = static_cast<int>(static_cast<long long>(Q) * w / W);
  const int q1 = static_cast<int>(static_cast<long long>(Q) * (w + 1) / W);
  if (q0 >= q1) return;

  const char* wgt = reinterpret_cast<const char*>(a.w);
  const char* act = reinterpret_cast<const char*>(a.act);
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);

  // LDS byte offset of the 16 bytes this lane fetches with load i of a tile
  // (tile byte 1024 * i + 16 * l: row / RB, column % RB)
  int lds_w[KF];
#pragma unroll
  for (int i = 0; i < KF; ++i) {
    const int o = 1024 * i + 16 * l;
    lds_w[i] = (o / RB) * PITCH + o % RB;
  }
  auto wtile = [&](const SStep& d) -> const char* {
    return wgt + (static_cast<size_t>(d.g) * a.H + 16 * static_cast<size_t>(d.j)) * RB;
  };
  auto load_w = [&](const SStep& d, uint4 (&r)[KF]) {
    const char* b = wtile(d);
#pragma unroll
    for (int i = 0; i < KF; ++i) {
      if constexpr (KEEP) r[i] = ldg(b + 1024 * i, static_cast<uint32_t>(16 * l));
      else r[i] = ldg_nt(b + 1024 * i, static_cast<uint32_t>(16 * l));
    }
  };
  auto load_x = [&](const SStep& d, uint4 (&x)[NT][KF]) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      const int r = d.row0 + min(d.t0 + tt * 16 + lrow, d.m_end - 1);
      const uint32_t off = static_cast<uint32_t>(r) * RB + 16 * lq;
#pragma unroll
      for (int f = 0; f < KF; ++f) x[tt][f] = ldg(act + FRAG_BYTES * f, off);
    }
  };

  // With up to four token tiles the next pass's fragments are loaded ahead
  // into a second set (xn); eight tiles leave no room for it, and those passes
  // load theirs in place when the pass starts (once every H / 16 steps).
  constexpr bool XN = NT <= 4;
  SStep cur = sh_decode<NT>(a, s_istart, s_off, q0);  // the step being multiplied
  SStep ld = cur;                                     // the next step to load
  int lqs = q0;
  uint4 xc[NT][KF], xn[XN ? NT : 1][KF];
  load_x(cur, xc);
#pragma unroll
  for (int tt = 0; tt < (XN ? NT : 1); ++tt)
#pragma unroll
    for (int f = 0; f < KF; ++f) xn[tt][f] = make_uint4(0u, 0u, 0u, 0u);  // written before it is read
  // Move `ld` to the next step; past the range it stays on the last one.  On
  // entering a new pass, that pass's token fragments go to xn (a range
  // crosses into a new pass at most once every H / 16 >= SH_RING steps).
  auto advance_load = [&]() {
    if (lqs + 1 < q1) {
      ++lqs;
      if (++ld.j == a.n_tiles) {
        ld = sh_decode<NT>(a, s_istart, s_off, lqs);
        if constexpr (XN) load_x(ld, xn);
      }
    }
  };
  uint4 wr[SH_RING][KF];
#pragma unroll
  for (int b = 0; b < SH_RING - 1; ++b) {
    load_w(ld, wr[b]);
    advance_load();
  }

  int cq = q0;
  // Step b of a trip: load tile cq + SH_RING - 1 into slot (b + SH_RING - 1) %
  // SH_RING, then multiply slot b (loaded SH_RING - 1 steps ago) and store.
#define SH_STEP(B)                                                                              \
  {                                                                                             \
    load_w(ld, wr[(B + SH_RING - 1) % SH_RING]);                                                \
    advance_load();                                                                             \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    _Pragma("unroll") for (int i = 0; i < KF; ++i) *reinterpret_cast<uint4*>(tile + lds_w[i]) = wr[B][i]; \
    uint4 wt[KF];                                                                               \
    _Pragma("unroll") for (int f = 0; f < KF; ++f)                                              \
      wt[f] = *reinterpret_cast<const uint4*>(tile + lrow * PITCH + FRAG_BYTES * f + 16 * lq);  \
    const int nrows = cur.m_end - cur.t0;                                                       \
    _Pragma("unroll") for (int tt = 0; tt < NT; ++tt) {                                         \
      if (tt == 0 || 16 * tt < nrows) {                                                         \
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};                                                     \
        _Pragma("unroll") for (int f = 0; f < KF; ++f) acc = Elem<uint16_t>::mma(wt[f], xc[tt][f], acc); \
        const int tr = cur.t0 + tt * 16 + lrow;                                                 \
        if (tr < cur.m_end)                                                                     \
          Elem<uint16_t>::store4(out + static_cast<size_t>(cur.row0 + tr) * a.H + 16 * cur.j + 4 * lq, \
                                 acc[0], acc[1], acc[2], acc[3]);                               \
      }                                                                                         \
    }                                                                                           \
    if (++cq >= q1) break;                                                                      \
    if (++cur.j == a.n_tiles) {                                                                 \
      cur = sh_decode<NT>(a, s_istart, s_off, cq);                                              \
      if constexpr (XN) {                                                                       \
        _Pragma("unroll") for (int tt = 0; tt < (XN ? NT : 1); ++tt)                            \
          _Pragma("unroll") for (int f = 0; f < KF; ++f) xc[tt][f] = xn[tt][f];                 \
      } else {                                                                                  \
        load_x(cur, xc);                                                                        \
      }                                                                                         \
    }                                                                                           \
  }
  static_assert(SH_RING == 4, "the trip below is unrolled for four slots");
  while (true) {
    SH_STEP(0)
    SH_STEP(1)
    SH_STEP(2)
    SH_STEP(3)
  }
#undef SH_STEP
}

template <int KF, int NT>
__global__ __launch_bounds__(SH_WAVES * WAVE) void expert_short_kernel(XArgs a) {
  __shared__ int s_istart[MAX_GROUPS + 1];
  __shared__ int s_off[MAX_GROUPS + 1];
  __shared__ int s_ntx, s_multi[2];
  __shared__ __attribute__((aligned(16))) char s_wt[SH_WAVES][16 * sh_pitch<KF>()];

  const int wv = uni(threadIdx.x / WAVE);
  const int l = lane_id();
  // steps per group: its passes x H / 16 tiles (none for groups the tile
  // kernels take); a kernel built for four token tiles runs two when no
  // group holds more than 32 rows
  item_prefix<NT>(a.offsets, a.n_groups, a.n_tiles, a.tile_nt, a.tile_min, a.tile_m_min, s_istart, s_off, &s_ntx);
  if (wv == SH_WAVES - 1) {
    // groups with more than one pass, for passes of 16 * NT rows and (the
    // body a four-tile kernel may run instead) of 32
    int n0 = 0, n1 = 0;
    for (int g = l; g < a.n_groups; g += WAVE) {
      const int m = a.offsets[g + 1] - a.offsets[g];
      n0 += m > pass_rows<NT>(m);
      n1 += m > pass_rows<2>(m);
    }
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) {
      n0 += __shfl_xor(n0, d, WAVE);
      n1 += __shfl_xor(n1, d, WAVE);
    }
    if (l == 0) {
      s_multi[0] = n0;
      s_multi[1] = n1;
    }
  }
  __syncthreads();  // the only barrier; waves are independent from here on
  // When the groups with several passes hold at most SH_KEEP_BYTES of weights
  // (a few hot experts), every weight tile is read with the ordinary policy:
  // the passes of a group run side by side on one XCD (the waves' ranges are
  // contiguous), so the later ones find the tiles in L2.  Qwen3-235B TP share
  // under Zipf routing: B = 64 21.0 -> 19.5 us, B = 256 44.1 -> 34.8, B = 2048
  // 120.8 -> 114.0.  With more such groups (uniform routing, B = 2048: about
  // 64 of 1.5 MB) the temporal loads crowd L2 and the launch got slower (110
  // -> 124 us), so those launches stream, as do launches of one pass per
  // group.
  const bool four = NT == 4 && uni(s_ntx) == 4;
  const long long group_bytes = static_cast<long long>(a.n_tiles) * 16 * KF * FRAG_BYTES;
  const int n_multi = uni(NT == 4 && !four ? s_multi[1] : s_multi[0]);
  const bool keep = n_multi > 0 && n_multi * group_bytes <= SH_KEEP_BYTES;
  if constexpr (NT == 4) {
    if (four) {
      if (keep) short_body<KF, 4, true>(a, s_istart, s_off, s_wt[wv], wv);
      else short_body<KF, 4, false>(a, s_istart, s_off, s_wt[wv], wv);
    } else {
      if (keep) short_body<KF, 2, true>(a, s_istart, s_off, s_wt[wv], wv);
      else short_body<KF, 2, false>(a, s_istart, s_off, s_wt[wv], wv);
    }
  } else {
    if (keep) short_body<KF, NT, true>(a, s_istart, s_off, s_wt[wv], wv);
    else short_body<KF, NT, false>(a, s_istart, s_off, s_wt[wv], wv);
  }
}

template <int KF>
void launch_kf(const XArgs& a, int nt, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(device_cu_count())), block(SH_WAVES * WAVE);
  if (nt >= 8) hipLaunchKernelGGL((expert_short_kernel<KF, 8>), grid, block, 0, s, a);
  else if (nt >= 4) hipLaunchKernelGGL((expert_short_kernel<KF, 4>), grid, block, 0, s, a);
  else if (nt == 2) hipLaunchKernelGGL((expert_short_kernel<KF, 2>), grid, block, 0, s, a);
  else hipLaunchKernelGGL((expert_short_kernel<KF, 1>), grid, block, 0, s, a);
}

}  // namespace

bool expert_short_down_ok(int dtype, int H, int I) {
  const int rb = I * 2;
  return dtype == 1 && rb % FRAG_BYTES == 0 && rb >= FRAG_BYTES && rb <= 8 * FRAG_BYTES && H % 16 == 0 &&
         H / 16 >= SH_RING;
}

void launch_expert_down_short(const XArgs& a, int nt, hipStream_t s) {
  switch (a.I_loc * 2 / FRAG_BYTES) {
    case 1: launch_kf<1>(a, nt, s); break;
    case 2: launch_kf<2>(a, nt, s); break;
    case 3: launch_kf<3>(a, nt, s); break;
    case 4: launch_kf<4>(a, nt, s); break;
    case 5: launch_kf<5>(a, nt, s); break;
    case 6: launch_kf<6>(a, nt, s); break;
    case 7: launch_kf<7>(a, nt, s); break;
    default: launch_kf<8>(a, nt, s); break;
  }
}

}  // namespace moe
