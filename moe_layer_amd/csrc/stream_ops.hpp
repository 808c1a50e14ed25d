// Device pieces shared by the expert grouped-GEMM kernels that stream weights
// through registers (expert_gemm.hip: one wave per range of chunks;
// expert_coop.hip: one block per work item): the argument block, the item
// table, per-item weight and token addressing, the 512-byte chunk loads, the
// per-wave LDS transpose into the 16x16 MFMA operand layout and the MFMA
// steps.  The conventions are described where they are used.
#pragma once

#include "common.hpp"
#include "moe_internal.h"

namespace moe {

constexpr int CHUNK_FRAGS = 8;                          // 64-byte fragments per chunk
constexpr int CHUNK_BYTES = CHUNK_FRAGS * FRAG_BYTES;   // 512

enum XMode { XMODE_UP = 0, XMODE_DOWN = 1 };

struct XArgs {
  const void* act;         // up: x (T, H); down: a (n_pairs, I')
  const int* sorted_pair;  // up: pair id of each sorted row
  const int* offsets;      // (n_groups + 1) sorted-row offsets per group
  const void* w;           // up: w13 (G, 2I', H); down: w2 (G, H, I')
  void* out;               // up: a (n_pairs, I'); down: y_pair (n_pairs, H)
  int n_groups;
  int kk;
  int K;                   // contraction length in elements (up: H, down: I')
  int I_loc;
  int H;
  int kfrag_total;         // K * elem / 64
  int n_tiles;             // 16-row weight tiles per group
  int n_quads;             // items per pass: ceil(n_tiles / SUB) (SUB = weight tiles per item)
  int nck;                 // 512-byte chunks per item
  int waves;               // waves launched
  int tile_nt;             // > 0: the tile kernel ran first with this many weight tiles per group ...
  int tile_min;            // ... and took the groups above tile_m_min rows if they made this many tiles
  int tile_m_min;
  int* ctr;                // per-item arrival counters (zero between calls)
  float* part;             // per-wave partial tiles: [wave][2][SUB][NT][64 lanes][4]
  int sub;                 // block-cooperative kernel: weight tiles per item (runtime)
  int halve;               // wave-streaming kernel: the grid holds two blocks per CU (a multiple of 16 blocks)
};

// Token rows per pass of a group with m rows: 16, or 16*NT when the kernel
// holds NT token tiles and the group has more than 16 rows.
template <int NT>
__device__ __forceinline__ int pass_rows(int m) {
  return (NT > 1 && m > 16) ? 16 * NT : 16;
}

// Wave 0: s_off[g] = offsets[g]; s_istart[g] = items of the groups before g
// (passes x quads each); s_istart[n_groups] = total items; *s_ntx = token
// tiles of the pass (a kernel built for four runs two when every group it
// takes holds 32 rows or fewer: four cost more per chunk than they save).
template <int NT>
__device__ __forceinline__ void item_prefix(const int* __restrict__ offsets, int n_groups, int n_quads,
                                            int tile_nt, int tile_min, int tile_m_min, int* s_istart, int* s_off,
                                            int* s_ntx) {
  if (threadIdx.x >= WAVE) return;
  const int l = lane_id();
  // The tile kernel's decision, by the same formula: when it takes every
  // group, none is left here.
  int m_max = 0x7fffffff;
  if (tile_nt > 0 && tile_take_all(offsets, n_groups, tile_m_min, tile_min, TILE_ROWS, tile_nt)) m_max = -1;
  int ntx = NT;
  if (NT == 4) {
    int big = 0;
    for (int g = l; g < n_groups; g += WAVE) {
      const int m = offsets[g + 1] - offsets[g];
      big |= (m > 32 && m <= m_max) ? 1 : 0;
    }
    ntx = __any(big) ? 4 : 2;
  }
  int base = 0;
  for (int g0 = 0; g0 <= n_groups; g0 += WAVE) {
    const int g = g0 + l;
    if (g <= n_groups) s_off[g] = offsets[g];
    int v = 0;
    if (g < n_groups) {
      const int m = offsets[g + 1] - offsets[g];
      const int ps = (ntx > 1 && m > 16) ? 16 * ntx : 16;  // pass_rows of the kernel body that runs
      if (m <= m_max) v = (m + ps - 1) / ps * n_quads;
    }
    const int incl = wave_inclusive_scan(v);
    if (g < n_groups) s_istart[g] = base + incl - v;
    base += __shfl(incl, WAVE - 1, WAVE);
  }
  if (l == 0) {
    s_istart[n_groups] = base;
    *s_ntx = ntx;
  }
}

// Loads from a wave-uniform base (kept in SGPRs) plus a 32-bit lane offset:
// the compiler emits global_load with a scalar base and folds constant
// offsets into the instruction, so no per-lane 64-bit address arithmetic is
// spent per load.
__device__ __forceinline__ uint4 ldg_nt(const char* base, uint32_t off) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(base + off));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ldg(const char* base, uint32_t off) {
  return *reinterpret_cast<const uint4*>(base + off);
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int NT>
struct WItem {
  int row0, m_end, t0, n0; // group's first sorted row, end of this pass's rows, pass start, first weight row
  int n_sub;               // tiles of the item inside the matrix (1..SUB)
  const char* wbase;       // the item's first weight row (wave-uniform)
  uint32_t sub_bytes;      // byte distance between consecutive tiles of the item
  int keep;                // the tile has later passes: weights read with the temporal policy
  uint32_t woff[4];        // lane: row 4j + lq of a tile, + 16*lrow, relative to the tile's base
  uint32_t xoff[NT];       // lane: its token's activation row, + 16*lq, relative to the activations
};

// Weight side of an item: group, row window and the lane's 4 row offsets
// (needs only the item table, so the first weight loads can be issued before
// any token index is known).  `item` is wave-uniform.
template <typename T, int MODE, int NT, int SUB>
__device__ __forceinline__ void witem_weights(const XArgs& a, const int* s_istart, const int* s_off,
                                              int item, int lrow, int lq, uint32_t row_bytes,
                                              WItem<NT>& it, int sub = SUB) {
  int lo = 0, hi = a.n_groups;  // s_istart[lo] <= item < s_istart[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (uni(s_istart[mid]) <= item) lo = mid;
    else hi = mid;
  }
  it.row0 = uni(s_off[lo]);
  const int m = uni(s_off[lo + 1]) - it.row0;
  const int ps = pass_rows<NT>(m);
  const int np = (m + ps - 1) / ps;
  it.keep = np > 1;   // later passes over the same tiles follow
  const int local = item - uni(s_istart[lo]);
  const int nq = local / np;
  it.t0 = (local - nq * np) * ps;
  it.m_end = min(m, it.t0 + ps);
  it.n_sub = min(sub, a.n_tiles - nq * sub);
  // Tile s of the quad, row i (0..15): for up, gate row n0 + 8s + i (i < 8)
  // or up row I' + n0 + 8s + i - 8; for down, W2 row n0 + 16s + i.  I' is a
  // multiple of 8 and H of 16, so every tile is whole.
  size_t first_row;
  if (MODE == XMODE_UP) {
    it.n0 = nq * sub * 8;
    first_row = static_cast<size_t>(lo) * (2 * a.I_loc) + it.n0;
    it.sub_bytes = 8 * row_bytes;
  } else {
    it.n0 = nq * sub * 16;
    first_row = static_cast<size_t>(lo) * a.H + it.n0;
    it.sub_bytes = 16 * row_bytes;
  }
  it.wbase = reinterpret_cast<const char*>(a.w) + first_row * row_bytes;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * j + lq;
    const int rel = (MODE == XMODE_UP) ? (i < 8 ? i : a.I_loc + i - 8) : i;
    it.woff[j] = static_cast<uint32_t>(rel) * row_bytes + 16 * lrow;
  }
}

// Token side: the activation row of this lane's token in each 16-row tile.
template <typename T, int MODE, int NT>
__device__ __forceinline__ void witem_tokens(const XArgs& a, int lrow, int lq, uint32_t row_bytes,
                                             WItem<NT>& it) {
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int r = it.row0 + min(it.t0 + tt * 16 + lrow, it.m_end - 1);
    const int tok = (MODE == XMODE_UP) ? a.sorted_pair[r] / a.kk : r;
    it.xoff[tt] = static_cast<uint32_t>(tok) * row_bytes + 16 * lq;
  }
}
// The same in two steps: fetch the rows' pair ids, then form the offsets.
template <typename T, int MODE, int NT>
__device__ __forceinline__ void witem_token_ids(const XArgs& a, int lrow, const WItem<NT>& it, int (&raw)[NT]) {
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int r = it.row0 + min(it.t0 + tt * 16 + lrow, it.m_end - 1);
    raw[tt] = (MODE == XMODE_UP) ? a.sorted_pair[r] : r;
  }
}
template <typename T, int MODE, int NT>
__device__ __forceinline__ void witem_token_offsets(const XArgs& a, int lq, uint32_t row_bytes, const int (&raw)[NT],
                                                    WItem<NT>& it) {
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int tok = (MODE == XMODE_UP) ? raw[tt] / a.kk : raw[tt];
    it.xoff[tt] = static_cast<uint32_t>(tok) * row_bytes + 16 * lq;
  }
}

template <typename T, int MODE, int NT, int SUB>
__device__ __forceinline__ void witem_setup(const XArgs& a, const int* s_istart, const int* s_off,
                                            int item, int lrow, int lq, uint32_t row_bytes,
                                            WItem<NT>& it) {
  witem_weights<T, MODE, NT, SUB>(a, s_istart, s_off, item, lrow, lq, row_bytes, it);
  witem_tokens<T, MODE, NT>(a, lrow, lq, row_bytes, it);
}

// Base of tile s (aliased to tile 0 past the matrix) of an item, at chunk c.
template <int NT>
__device__ __forceinline__ const char* tile_chunk(const WItem<NT>& it, int s, int c) {
  return it.wbase + (s < it.n_sub ? s : 0) * it.sub_bytes + c * CHUNK_BYTES;
}

// Weight bytes of one tile-chunk in the load layout: register i holds row
// 4*(i%4) + l/16, bytes 256*(i/4) + 16*(l%16) of the chunk.  Non-temporal:
// streamed once.  The loaded registers are not touched until use, so the
// loads stay in flight.  When the chunk is the partial last one of K (valid
// < 512 bytes), lanes past the end re-read the chunk's first bytes of their
// row (finite data that meets zero token fragments).
__device__ __forceinline__ void wload_part(const char* cbase, const uint32_t (&woff)[4], int valid,
                                           int lrow, uint4 (&w)[CHUNK_FRAGS]) {
#pragma unroll
  for (int i = 0; i < CHUNK_FRAGS; ++i) {
    const int col = 256 * (i / 4) + 16 * lrow;
    w[i] = ldg_nt(cbase, woff[i % 4] + (col < valid ? 256 * (i / 4) : -16 * lrow));
  }
}
// The same loads with the ordinary (temporal) policy when `keep`: the lines
// stay in L2 for later passes over the same tile.
__device__ __forceinline__ void wload_full_keep(const char* cbase, const uint32_t (&woff)[4], uint4 (&w)[CHUNK_FRAGS],
                                                bool keep) {
  if (keep) {
#pragma unroll
    for (int i = 0; i < CHUNK_FRAGS; ++i) w[i] = ldg(cbase + 256 * (i / 4), woff[i % 4]);
  } else {
#pragma unroll
    for (int i = 0; i < CHUNK_FRAGS; ++i) w[i] = ldg_nt(cbase + 256 * (i / 4), woff[i % 4]);
  }
}
__device__ __forceinline__ void wload_full(const char* cbase, const uint32_t (&woff)[4], uint4 (&w)[CHUNK_FRAGS]) {
#pragma unroll
  for (int i = 0; i < CHUNK_FRAGS; ++i) w[i] = ldg_nt(cbase + 256 * (i / 4), woff[i % 4]);
}
// The partial-chunk loads with the ordinary (temporal) policy when `keep`.
__device__ __forceinline__ void wload_part_keep(const char* cbase, const uint32_t (&woff)[4], int valid,
                                                int lrow, uint4 (&w)[CHUNK_FRAGS], bool keep) {
  if (keep) {
#pragma unroll
    for (int i = 0; i < CHUNK_FRAGS; ++i) {
      const int col = 256 * (i / 4) + 16 * lrow;
      w[i] = ldg(cbase, woff[i % 4] + (col < valid ? 256 * (i / 4) : -16 * lrow));
    }
  } else {
    wload_part(cbase, woff, valid, lrow, w);
  }
}
// One load sequence for full and partial chunks (the partial form gives the
// full form's addresses when valid >= 512).  Loads behind a branch land in
// different registers on the two paths; the join then copies registers and
// the copies wait for the loads, draining the stream at every sub-step.
__device__ __forceinline__ void wload(const char* cbase, const uint32_t (&woff)[4], int valid, int lrow,
                                      uint4 (&w)[CHUNK_FRAGS]) {
  wload_part(cbase, woff, valid, lrow, w);
}

// Token fragments of one chunk for every tile (cx = activations + chunk offset).
template <int NT>
__device__ __forceinline__ void xload_full(const char* cx, const uint32_t (&xoff)[NT], int nrows,
                                           uint4 (&x)[NT][CHUNK_FRAGS]) {
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
    if (tt == 0 || 16 * tt < nrows) {
#pragma unroll
      for (int f = 0; f < CHUNK_FRAGS; ++f) x[tt][f] = ldg(cx + FRAG_BYTES * f, xoff[tt]);
    }
}
// Partial chunk: fragments past the end of K re-read a valid one; wmma_part
// zeroes them at use.
template <int NT>
__device__ __forceinline__ void xload_part(const char* cx, const uint32_t (&xoff)[NT], int nf, int nrows,
                                           uint4 (&x)[NT][CHUNK_FRAGS]) {
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
    if (tt == 0 || 16 * tt < nrows) {
#pragma unroll
      for (int f = 0; f < CHUNK_FRAGS; ++f) x[tt][f] = ldg(cx, xoff[tt] + FRAG_BYTES * min(f, nf - 1));
    }
}

constexpr int WT_ROW = CHUNK_BYTES + 16;  // padded row of the wave's LDS tile

// Load layout -> MFMA operand layout through the wave's own LDS tile
// (16 rows x WT_ROW bytes).  Reads after writes within one wave are ordered.
__device__ __forceinline__ void wtranspose(const uint4 (&w)[CHUNK_FRAGS], char* tile, int lrow,
                                           int lq, uint4 (&wt)[CHUNK_FRAGS]) {
#pragma unroll
  for (int i = 0; i < CHUNK_FRAGS; ++i)
    *reinterpret_cast<uint4*>(tile + (4 * (i % 4) + lq) * WT_ROW + 256 * (i / 4) + 16 * lrow) = w[i];
#pragma unroll
  for (int f = 0; f < CHUNK_FRAGS; ++f)
    wt[f] = *reinterpret_cast<const uint4*>(tile + lrow * WT_ROW + FRAG_BYTES * f + 16 * lq);
}

// Token tiles wholly past the pass's rows (nrows of them hold real rows) are
// skipped: a uniform branch around MFMAs only, no loads.  Rows past the end
// inside a tile repeat a real row and are never stored.
template <typename T, int NT>
__device__ __forceinline__ void wmma_full(const uint4 (&w)[CHUNK_FRAGS], const uint4 (&x)[NT][CHUNK_FRAGS],
                                          int nrows, f32x4_t (&acc)[NT]) {
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    if (tt == 0 || 16 * tt < nrows) {
#pragma unroll
      for (int f = 0; f < CHUNK_FRAGS; ++f) acc[tt] = Elem<T>::mma(w[f], x[tt][f], acc[tt]);
    }
  }
}
// Fragments f >= nf lie past the end of K: their token side is zeroed here,
// so they add exactly nothing whatever the weight side holds.
template <typename T, int NT>
__device__ __forceinline__ void wmma_part(const uint4 (&w)[CHUNK_FRAGS], const uint4 (&x)[NT][CHUNK_FRAGS],
                                          int nf, int nrows, f32x4_t (&acc)[NT]) {
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    if (tt == 0 || 16 * tt < nrows) {
#pragma unroll
      for (int f = 0; f < CHUNK_FRAGS; ++f) acc[tt] = Elem<T>::mma(w[f], keep_or_zero(f < nf, x[tt][f]), acc[tt]);
    }
  }
}

// Block-cooperative expert up-projection for decode-sized groups (expert_coop.hip):
// weight tiles per item for nck 512-byte chunks of K (0: not handled), and the
// launch (bf16; a's shape fields set as for the wave-streaming kernel).  It
// needs no workspace.
int expert_coop_sub(int nck);
void launch_expert_coop_up(XArgs a, hipStream_t s);
// Down-projection for W2 rows of at most 512 bytes (expert_short.hip):
// whether it takes these shapes, and the launch (a's shape and tile-rule
// fields set as for the wave-streaming kernel; NT = 1 or 2 token tiles per
// pass).  It needs no workspace.
bool expert_short_down_ok(int dtype, int H, int I);
void launch_expert_down_short(const XArgs& a, int nt, hipStream_t s);

}  // namespace moe
