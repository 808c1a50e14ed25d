// EP -> TP local permute of expert weights (Moebius review, §3.1 weight
// resharding and Fig. 4: before the exchange, each rank packs the bytes bound
// for each peer into one contiguous block per destination).
//
// Source (this rank's E_local whole experts):
//   W13 (E_local, 2I, H), W2 (E_local, H, I)
// Destination block q (peer q's TP slice S_q = [q I/P, (q+1) I/P) of them):
//   dst13[q] (E_local, 2I/P, H): rows S_q of the gate half, then rows S_q of
//                                the up half, of every local expert
//   dst2[q]  (E_local, H, I/P):  columns S_q of every W2 row
// Two launches, each with exactly the blocks that fit on the chip at once:
//   W13: each source row lands whole as one destination row; waves copy 4 KB
//        units (16 bytes per lane, four per lane in flight, the next unit's
//        loads issued before this unit's stores) in destination order, so the
//        writes in flight fill one block front to back;
//   W2:  each source row splits into P segments of I/P columns; a wave copies
//        a few whole consecutive rows per step, with lanes assigned by
//        destination so that every store instruction writes 1 KB of one or two
//        blocks.
// Every byte is read once and written once (non-temporal: streamed); the copy
// is exact.
#include "common.hpp"
#include "moe_internal.h"

namespace moe {

constexpr int RP_WAVES = 4;                 // waves per block
constexpr int RP_U = 4;                     // 16-byte chunks per lane per W13 step (4 KB per wave)
constexpr int RP_STEP = RP_U * WAVE;        // chunks per wave per step

struct RepackArgs {
  const char* w13;
  const char* w2;
  PeerPtrs d13;
  PeerPtrs d2;
  long long rows13;    // E_local * 2I source rows of W13
  long long rows2;     // E_local * H source rows of W2
  int row13;           // chunks per W13 row (H * elem / 16)
  int row2;            // chunks per W2 row (I * elem / 16)
  int I;               // rows per half of W13
  int Ip;              // I / P
  int seg2;            // chunks per W2 segment (Ip * elem / 16)
  int P;               // destination blocks
};

// W2 rows of at most 4 KB: a wave copies RW = 12/J consecutive rows per step
// (J = 16-byte chunks per lane per row), so every step moves about 12 KB of
// contiguous source with all loads issued before the stores; which block and
// column a lane's chunk j lands in is the same for every row.
template <int J>
__device__ __forceinline__ void repack_w2_rows(const RepackArgs& a, long long w0, long long nw, int l) {
  constexpr int RW = 12 / J;
  char* dbase[J];
  int dcol[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int c = j * WAVE + l;
    const int q = c < a.row2 ? c / a.seg2 : 0;
    dbase[j] = static_cast<char*>(a.d2.p[q]);
    dcol[j] = c - q * a.seg2;
  }
  for (long long r0 = w0 * RW; r0 < a.rows2; r0 += nw * RW) {
    u32x4_t v[RW][J];
#pragma unroll
    for (int rr = 0; rr < RW; ++rr)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int c = j * WAVE + l;
        if (r0 + rr < a.rows2 && c < a.row2)
          v[rr][j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(a.w2 + ((r0 + rr) * a.row2 + c) * 16));
      }
#pragma unroll
    for (int rr = 0; rr < RW; ++rr)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int c = j * WAVE + l;
        if (r0 + rr < a.rows2 && c < a.row2)
          __builtin_nontemporal_store(v[rr][j], reinterpret_cast<u32x4_t*>(dbase[j] + ((r0 + rr) * a.seg2 + dcol[j]) * 16));
      }
  }
}

// W2 rows that tile 768 chunks exactly (RW = 768 / row2 rows per step, e.g.
// four 3 KB rows): a wave step reads RW whole consecutive rows (12 KB of
// contiguous source) and writes, for each of the P blocks, its RW segments,
// which are contiguous there (RW * seg2 chunks).  The lanes are assigned by
// destination: slot k of lane l carries chunk d = 64k + l of the blocks'
// pieces laid end to end, so each store instruction writes 1 KB of at most
// two blocks, and the loads gather the matching chunks from the 12 KB region
// the step reads whole anyway.  The mapping is the same for every step.
__device__ __forceinline__ void repack_w2_blocks(const RepackArgs& a, long long w0, long long nw, int l) {
  constexpr int KS = 12;
  const int RW = KS * WAVE / a.row2;
  const int piece = RW * a.seg2;  // chunks each block receives per step
  uint32_t soff[KS];              // byte offset of the source chunk in the step's region
  char* dbase[KS];
  int dch[KS];                    // destination chunk within the block's piece
  int drow[KS];                   // source row of the slot within the step
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const int d = k * WAVE + l;
    const int q = d / piece;
    const int i = d - q * piece;
    const int rr = i / a.seg2;
    const int col = i - rr * a.seg2;
    soff[k] = static_cast<uint32_t>(rr * a.row2 + q * a.seg2 + col) * 16;
    dbase[k] = static_cast<char*>(a.d2.p[q]);
    dch[k] = i;
    drow[k] = rr;
  }
  for (long long r0 = w0 * RW; r0 < a.rows2; r0 += nw * RW) {
    const char* src = a.w2 + r0 * a.row2 * 16;
    u32x4_t v[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k)
      if (r0 + drow[k] < a.rows2) v[k] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + soff[k]));
#pragma unroll
    for (int k = 0; k < KS; ++k)
      if (r0 + drow[k] < a.rows2)
        __builtin_nontemporal_store(v[k], reinterpret_cast<u32x4_t*>(dbase[k] + (r0 * a.seg2 + dch[k]) * 16));
  }
}

// W13 part.  A unit's destination row is wave-uniform.
__global__ __launch_bounds__(RP_WAVES * WAVE) void repack13_kernel(RepackArgs a) {
  const int l = lane_id();
  const long long nw = static_cast<long long>(gridDim.x) * RP_WAVES;
  const long long w0 = static_cast<long long>(blockIdx.x) * RP_WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  // ---- W13: row (e, half, i) -> block q = i / Ip, row e*2Ip + half*Ip + i%Ip,
  // copied in units of half a row or less (RP_STEP chunks), two units in
  // flight: the next unit's loads are issued before this unit's stores.
  const int upr = (a.row13 + RP_STEP - 1) / RP_STEP;  // units per row
  const int units13 = static_cast<int>(a.rows13) * upr;
  // Units run in destination order (block q, then its rows), so the writes
  // of the waves in flight fill one block front to back.
  const int rows_per_block = static_cast<int>(a.rows13) / a.P;  // E_local * 2Ip
  auto unit = [&](int u, const char*& src, char*& dst, int& c0) {
    const int dr = u / upr;                 // destination row over all blocks
    c0 = (u - dr * upr) * RP_STEP;
    const int q = dr / rows_per_block;
    const int d = dr - q * rows_per_block;  // row in block q: (e, half, j)
    const int e = d / (2 * a.Ip);
    const int rem = d - e * 2 * a.Ip;
    const int half = rem >= a.Ip;
    const int j = rem - half * a.Ip;
    const int r = e * 2 * a.I + half * a.I + q * a.Ip + j;
    src = a.w13 + static_cast<long long>(r) * a.row13 * 16;
    dst = static_cast<char*>(a.d13.p[q]) + static_cast<long long>(d) * a.row13 * 16;
  };
  auto load = [&](const char* src, int c0, u32x4_t (&v)[RP_U]) {
#pragma unroll
    for (int u = 0; u < RP_U; ++u) {
      const int c = c0 + u * WAVE + l;
      if (c < a.row13) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + c * 16));
    }
  };
  auto store = [&](char* dst, int c0, const u32x4_t (&v)[RP_U]) {
#pragma unroll
    for (int u = 0; u < RP_U; ++u) {
      const int c = c0 + u * WAVE + l;
      if (c < a.row13) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4_t*>(dst + c * 16));
    }
  };
  int u = static_cast<int>(w0);
  if (u >= units13) return;
  const int step = static_cast<int>(nw);
  const char *sa, *sb;
  char *da, *db;
  int ca, cb;
  u32x4_t va[RP_U], vb[RP_U];
  unit(u, sa, da, ca);
  load(sa, ca, va);
  while (true) {
    if (u + step < units13) {
      unit(u + step, sb, db, cb);
      load(sb, cb, vb);
    }
    store(da, ca, va);
    u += step;
    if (u >= units13) break;
    if (u + step < units13) {
      unit(u + step, sa, da, ca);
      load(sa, ca, va);
    }
    store(db, cb, vb);
    u += step;
    if (u >= units13) break;
  }
}

// W2 part: PATH 0 = destination-ordered whole-row steps (768 % row2 == 0),
// 1..4 = J chunks per lane per row, several rows per step; 5 = row by row.
template <int PATH>
__global__ __launch_bounds__(RP_WAVES * WAVE) void repack2_kernel(RepackArgs a) {
  const int l = lane_id();
  const long long nw = static_cast<long long>(gridDim.x) * RP_WAVES;
  const long long w0 = static_cast<long long>(blockIdx.x) * RP_WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  // row r, chunk c -> block q = c / seg2, offset r*seg2 + c%seg2
  if constexpr (PATH == 0) {
    repack_w2_blocks(a, w0, nw, l);
  } else if constexpr (PATH >= 1 && PATH <= 4) {
    repack_w2_rows<PATH>(a, w0, nw, l);
  } else {
    for (int c0 = 0; c0 < a.row2; c0 += RP_STEP) {
      // row by row: which segment (and where in it) a lane's chunk of a step
      // lands is the same for every row, so it is worked out once per lane
      char* dbase[RP_U];
      int dcol[RP_U];
#pragma unroll
      for (int u = 0; u < RP_U; ++u) {
        const int c = c0 + u * WAVE + l;
        const int q = c < a.row2 ? c / a.seg2 : 0;
        dbase[u] = static_cast<char*>(a.d2.p[q]);
        dcol[u] = c - q * a.seg2;
      }
      for (long long r = w0; r < a.rows2; r += nw) {
        const char* src = a.w2 + r * a.row2 * 16;
        u32x4_t v[RP_U];
#pragma unroll
        for (int u = 0; u < RP_U; ++u) {
          const int c = c0 + u * WAVE + l;
          if (c < a.row2) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + c * 16));
        }
#pragma unroll
        for (int u = 0; u < RP_U; ++u) {
          const int c = c0 + u * WAVE + l;
          if (c < a.row2)
            __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4_t*>(dbase[u] + (r * a.seg2 + dcol[u]) * 16));
        }
      }
    }
  }
}

template <int PATH>
static void launch_repack2(const RepackArgs& a, hipStream_t s) {
  static int per_cu = 0;
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&repack2_kernel<PATH>),
                                                     RP_WAVES * WAVE, 0) != hipSuccess || n < 1)
      n = 1;
    per_cu = n;
  }
  long long g = static_cast<long long>(device_cu_count()) * per_cu;
  if (g > (a.rows2 + RP_WAVES - 1) / RP_WAVES) g = (a.rows2 + RP_WAVES - 1) / RP_WAVES;
  hipLaunchKernelGGL(repack2_kernel<PATH>, dim3(static_cast<unsigned>(g > 0 ? g : 1)), dim3(RP_WAVES * WAVE), 0, s, a);
}

bool repack_fits(int E_local, int H, int I, int dtype) {
  const long long row13 = static_cast<long long>(H) * (dtype == 1 ? 2 : 4) / 16;
  const long long units = static_cast<long long>(E_local) * 2 * I * ((row13 + RP_STEP - 1) / RP_STEP);
  return units < (1LL << 31);
}

void launch_repack_ep_to_tp(int dtype, const void* w13, const void* w2, int E_local, int H, int I,
                            int P, const PeerPtrs& d13, const PeerPtrs& d2, hipStream_t s) {
  const int eb = dtype == 1 ? 2 : 4;
  RepackArgs a{};
  a.w13 = static_cast<const char*>(w13);
  a.w2 = static_cast<const char*>(w2);
  a.d13 = d13;
  a.d2 = d2;
  a.row13 = H * eb / 16;
  a.row2 = I * eb / 16;
  a.rows13 = static_cast<long long>(E_local) * 2 * I;
  a.rows2 = static_cast<long long>(E_local) * H;
  a.I = I;
  a.Ip = I / P;
  a.seg2 = a.Ip * eb / 16;
  a.P = P;
  // Each part is its own launch with exactly the blocks that fit on the chip
  // at once (so every wave's share is equal and no block waits for a second
  // round), never more than its work needs.
  static int per_cu13 = 0;
  if (per_cu13 == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&repack13_kernel),
                                                     RP_WAVES * WAVE, 0) != hipSuccess || n < 1)
      n = 1;
    per_cu13 = n;
  }
  const long long units13 = a.rows13 * ((a.row13 + RP_STEP - 1) / RP_STEP);
  long long g13 = static_cast<long long>(device_cu_count()) * per_cu13;
  if (g13 > (units13 + RP_WAVES - 1) / RP_WAVES) g13 = (units13 + RP_WAVES - 1) / RP_WAVES;
  hipLaunchKernelGGL(repack13_kernel, dim3(static_cast<unsigned>(g13 > 0 ? g13 : 1)), dim3(RP_WAVES * WAVE), 0, s, a);
  if ((12 * WAVE) % a.row2 == 0) {
    launch_repack2<0>(a, s);
    return;
  }
  switch ((a.row2 + WAVE - 1) / WAVE) {
    case 1: launch_repack2<1>(a, s); break;
    case 2: launch_repack2<2>(a, s); break;
    case 3: launch_repack2<3>(a, s); break;
    case 4: launch_repack2<4>(a, s); break;
    default: launch_repack2<5>(a, s); break;
  }
}

}  // namespace moe
