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
// The TP -> EP direction (moe_repack_tp_to_ep) is the exact inverse: the P
// blocks received from the peers are gathered back into whole experts.  Both
// directions share the kernels below (INV selects which side is read).
//
// Two launches, each with exactly the blocks that fit on the chip at once:
//   W13: each expert row is one block row; waves copy 4 KB units (16 bytes
//        per lane, four per lane in flight, the next unit's loads issued
//        before this unit's stores) in the order of the side being written,
//        so the writes in flight fill one tensor front to back;
//   W2:  each expert row is P block segments of I/P columns; a wave copies a
//        few whole consecutive expert rows per step, with lanes assigned by
//        block position so that every block-side access instruction covers
//        1 KB of one or two blocks.
// Every byte is read once and written once (non-temporal: streamed); the copy
// is exact.
#include "common.hpp"
#include "moe_internal.h"

namespace moe {

constexpr int RP_WAVES = 4;                 // waves per block
constexpr int RP_U = 4;                     // 16-byte chunks per lane per W13 step (4 KB per wave)
constexpr int RP_STEP = RP_U * WAVE;        // chunks per wave per step

// Copy direction helpers: e = expert-side address, b = block-side address.
template <bool INV>
__device__ __forceinline__ u32x4_t rp_load(const char* e, const char* b) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(INV ? b : e));
}
template <bool INV>
__device__ __forceinline__ void rp_store(char* e, char* b, u32x4_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(INV ? e : b));
}

struct RepackArgs {
  char* w13;           // expert side: (E_local, 2I, H)
  char* w2;            // expert side: (E_local, H, I)
  PeerPtrs d13;        // block side: P x (E_local, 2I/P, H)
  PeerPtrs d2;         // block side: P x (E_local, H, I/P)
  long long rows13;    // E_local * 2I expert rows of W13
  long long rows2;     // E_local * H expert rows of W2
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
template <bool INV, int J>
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
          v[rr][j] = rp_load<INV>(a.w2 + ((r0 + rr) * a.row2 + c) * 16, dbase[j] + ((r0 + rr) * a.seg2 + dcol[j]) * 16);
      }
#pragma unroll
    for (int rr = 0; rr < RW; ++rr)
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const int c = j * WAVE + l;
        if (r0 + rr < a.rows2 && c < a.row2)
          rp_store<INV>(a.w2 + ((r0 + rr) * a.row2 + c) * 16, dbase[j] + ((r0 + rr) * a.seg2 + dcol[j]) * 16, v[rr][j]);
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
template <bool INV>
__device__ __forceinline__ void repack_w2_blocks(const RepackArgs& a, long long w0, long long nw, int l) {
  constexpr int KS = 12;
  const int RW = KS * WAVE / a.row2;
  const int piece = RW * a.seg2;  // chunks of each block per step
  uint32_t soff[KS];              // byte offset of the slot's chunk in the step's expert-side region
  char* dbase[KS];
  int dch[KS];                    // the slot's chunk within the block's piece
  int drow[KS];                   // expert row of the slot within the step
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
    char* ereg = a.w2 + r0 * a.row2 * 16;
    u32x4_t v[KS];
#pragma unroll
    for (int k = 0; k < KS; ++k)
      if (r0 + drow[k] < a.rows2) v[k] = rp_load<INV>(ereg + soff[k], dbase[k] + (r0 * a.seg2 + dch[k]) * 16);
#pragma unroll
    for (int k = 0; k < KS; ++k)
      if (r0 + drow[k] < a.rows2) rp_store<INV>(ereg + soff[k], dbase[k] + (r0 * a.seg2 + dch[k]) * 16, v[k]);
  }
}

// W13 part.  A unit's rows on both sides are wave-uniform.
template <bool INV>
__global__ __launch_bounds__(RP_WAVES * WAVE) void repack13_kernel(RepackArgs a) {
  const int l = lane_id();
  const long long nw = static_cast<long long>(gridDim.x) * RP_WAVES;
  const long long w0 = static_cast<long long>(blockIdx.x) * RP_WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  // Expert row (e, half, i) <-> block q = i / Ip, row e*2Ip + half*Ip + i%Ip,
  // copied in units of half a row or less (RP_STEP chunks).
  const int upr = (a.row13 + RP_STEP - 1) / RP_STEP;  // units per row
  const int units13 = static_cast<int>(a.rows13) * upr;
  const int rows_per_block = static_cast<int>(a.rows13) / a.P;  // E_local * 2Ip
  // Unit u in the written side's order: blocks (q, then its rows) when
  // packing, expert rows when unpacking.
  auto unit = [&](int u, char*& e_ptr, char*& b_ptr, int& c0) {
    const int wr = u / upr;
    c0 = (u - wr * upr) * RP_STEP;
    int r, q, d;
    if (!INV) {
      q = wr / rows_per_block;
      d = wr - q * rows_per_block;
      const int e = d / (2 * a.Ip);
      const int rem = d - e * 2 * a.Ip;
      const int half = rem >= a.Ip;
      r = e * 2 * a.I + half * a.I + q * a.Ip + (rem - half * a.Ip);
    } else {
      r = wr;
      const int e = r / (2 * a.I);
      const int i2 = r - e * 2 * a.I;
      const int half = i2 >= a.I;
      const int i = i2 - half * a.I;
      q = i / a.Ip;
      d = e * 2 * a.Ip + half * a.Ip + (i - q * a.Ip);
    }
    e_ptr = a.w13 + static_cast<long long>(r) * a.row13 * 16;
    b_ptr = static_cast<char*>(a.d13.p[q]) + static_cast<long long>(d) * a.row13 * 16;
  };
  auto load = [&](char* e_ptr, char* b_ptr, int c0, u32x4_t (&v)[RP_U]) {
#pragma unroll
    for (int u = 0; u < RP_U; ++u) {
      const int c = c0 + u * WAVE + l;
      if (c < a.row13) v[u] = rp_load<INV>(e_ptr + c * 16, b_ptr + c * 16);
    }
  };
  auto store = [&](char* e_ptr, char* b_ptr, int c0, const u32x4_t (&v)[RP_U]) {
#pragma unroll
    for (int u = 0; u < RP_U; ++u) {
      const int c = c0 + u * WAVE + l;
      if (c < a.row13) rp_store<INV>(e_ptr + c * 16, b_ptr + c * 16, v[u]);
    }
  };
  // two units in flight: the next unit's loads are issued before this one's stores
  int u = static_cast<int>(w0);
  if (u >= units13) return;
  const int step = static_cast<int>(nw);
  char *ea, *ba, *eb, *bb;
  int ca, cb;
  u32x4_t va[RP_U], vb[RP_U];
  unit(u, ea, ba, ca);
  load(ea, ba, ca, va);
  while (true) {
    if (u + step < units13) {
      unit(u + step, eb, bb, cb);
      load(eb, bb, cb, vb);
    }
    store(ea, ba, ca, va);
    u += step;
    if (u >= units13) break;
    if (u + step < units13) {
      unit(u + step, ea, ba, ca);
      load(ea, ba, ca, va);
    }
    store(eb, bb, cb, vb);
    u += step;
    if (u >= units13) break;
  }
}

// W2 part: PATH 0 = whole-row steps with block-ordered lanes (768 % row2
// == 0), 1..4 = J chunks per lane per row, several rows per step; 5 = row by
// row.  Expert row r, chunk c <-> block q = c / seg2, offset r*seg2 + c%seg2.
template <bool INV, int PATH>
__global__ __launch_bounds__(RP_WAVES * WAVE) void repack2_kernel(RepackArgs a) {
  const int l = lane_id();
  const long long nw = static_cast<long long>(gridDim.x) * RP_WAVES;
  const long long w0 = static_cast<long long>(blockIdx.x) * RP_WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  if constexpr (PATH == 0) {
    repack_w2_blocks<INV>(a, w0, nw, l);
  } else if constexpr (PATH >= 1 && PATH <= 4) {
    repack_w2_rows<INV, PATH>(a, w0, nw, l);
  } else {
    for (int c0 = 0; c0 < a.row2; c0 += RP_STEP) {
      // row by row: which segment (and where in it) a lane's chunk of a step
      // lies in is the same for every row, so it is worked out once per lane
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
        char* erow = a.w2 + r * a.row2 * 16;
        u32x4_t v[RP_U];
#pragma unroll
        for (int u = 0; u < RP_U; ++u) {
          const int c = c0 + u * WAVE + l;
          if (c < a.row2) v[u] = rp_load<INV>(erow + c * 16, dbase[u] + (r * a.seg2 + dcol[u]) * 16);
        }
#pragma unroll
        for (int u = 0; u < RP_U; ++u) {
          const int c = c0 + u * WAVE + l;
          if (c < a.row2) rp_store<INV>(erow + c * 16, dbase[u] + (r * a.seg2 + dcol[u]) * 16, v[u]);
        }
      }
    }
  }
}

template <typename K>
static int rp_per_cu(K kernel) {
  return kernel_blocks_per_cu(reinterpret_cast<const void*>(kernel), RP_WAVES * WAVE);
}

template <bool INV, int PATH>
static void launch_repack2(const RepackArgs& a, hipStream_t s) {
  static const int per_cu = rp_per_cu(&repack2_kernel<INV, PATH>);
  long long g = static_cast<long long>(device_cu_count()) * per_cu;
  if (g > (a.rows2 + RP_WAVES - 1) / RP_WAVES) g = (a.rows2 + RP_WAVES - 1) / RP_WAVES;
  hipLaunchKernelGGL((repack2_kernel<INV, PATH>), dim3(static_cast<unsigned>(g > 0 ? g : 1)), dim3(RP_WAVES * WAVE), 0,
                     s, a);
}

bool repack_fits(int E_local, int H, int I, int dtype) {
  const long long row13 = static_cast<long long>(H) * (dtype == 1 ? 2 : 4) / 16;
  const long long units = static_cast<long long>(E_local) * 2 * I * ((row13 + RP_STEP - 1) / RP_STEP);
  return units < (1LL << 31);
}

// Each part is its own launch with exactly the blocks that fit on the chip
// at once (so every wave's share is equal and no block waits for a second
// round), never more than its work needs.
template <bool INV>
static void launch_repack(int dtype, void* w13, void* w2, int E_local, int H, int I, int P, const PeerPtrs& d13,
                          const PeerPtrs& d2, hipStream_t s) {
  const int eb = dtype == 1 ? 2 : 4;
  RepackArgs a{};
  a.w13 = static_cast<char*>(w13);
  a.w2 = static_cast<char*>(w2);
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
  static const int per_cu13 = rp_per_cu(&repack13_kernel<INV>);
  const long long units13 = a.rows13 * ((a.row13 + RP_STEP - 1) / RP_STEP);
  long long g13 = static_cast<long long>(device_cu_count()) * per_cu13;
  if (g13 > (units13 + RP_WAVES - 1) / RP_WAVES) g13 = (units13 + RP_WAVES - 1) / RP_WAVES;
  hipLaunchKernelGGL(repack13_kernel<INV>, dim3(static_cast<unsigned>(g13 > 0 ? g13 : 1)), dim3(RP_WAVES * WAVE), 0, s,
                     a);
  if ((12 * WAVE) % a.row2 == 0) {
    launch_repack2<INV, 0>(a, s);
    return;
  }
  switch ((a.row2 + WAVE - 1) / WAVE) {
    case 1: launch_repack2<INV, 1>(a, s); break;
    case 2: launch_repack2<INV, 2>(a, s); break;
    case 3: launch_repack2<INV, 3>(a, s); break;
    case 4: launch_repack2<INV, 4>(a, s); break;
    default: launch_repack2<INV, 5>(a, s); break;
  }
}

void launch_repack_ep_to_tp(int dtype, const void* w13, const void* w2, int E_local, int H, int I,
                            int P, const PeerPtrs& d13, const PeerPtrs& d2, hipStream_t s) {
  launch_repack<false>(dtype, const_cast<void*>(w13), const_cast<void*>(w2), E_local, H, I, P, d13, d2, s);
}

void launch_repack_tp_to_ep(int dtype, const PeerPtrs& s13, const PeerPtrs& s2, int E_local, int H, int I, int P,
                            void* w13, void* w2, hipStream_t s) {
  launch_repack<true>(dtype, w13, w2, E_local, H, I, P, s13, s2, s);
}

}  // namespace moe
