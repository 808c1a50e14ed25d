// Expert grouped GEMMs for groups that hold many token rows (bf16 storage,
// fp32 accumulate):
//   up   : a[r]      = silu(W1_g x_t) * (W3_g x_t)   from W13_g (2I', H)
//   down : y_pair[r] = W2_g a[r]                      from W2_g  (H, I')
// (Moebius review, §3.1 gives W13 as (., 2I, H) and W2 as (., H, I).)
//
// The wave-streaming kernel reads a group's weights once per pass of 16-32
// token rows; a group with more rows than one pass holds goes here instead,
// where a block of four waves multiplies a tile of 128 weight rows by a tile
// of 128 token rows over the whole K, so every weight byte is fetched once
// per 128 tokens and the token side is shared by the four waves through LDS.
//
// Tile = (group g, weight tile n, token tile m).  Weight rows of a tile:
//   up   : 64 gate rows n0 .. n0+63 and the 64 matching up rows I'+n0 .., so
//          silu(gate)*up is formed in registers and `a` is written once;
//   down : 128 rows of W2 = 128 output features.
// K is walked in stages of 128 bytes per row: the 256 threads fetch a
// stage's 128 weight rows and 128 token rows (each load instruction takes
// 128 contiguous bytes from each of 8 rows), two stages ahead in registers,
// and write it to one of two LDS buffers; the waves then read MFMA operands
// back (16x16x32 bf16: lane l reads row l%16, 16 bytes at 16*(l/16) of each
// 64-byte K half).  The 16-byte chunks of a row are XOR-swizzled by row so
// that both the stores and the operand reads spread over all LDS banks.  One
// barrier per stage: the buffer a stage is written to was last read two
// stages before.
//
// Wave w computes token rows 64*(w&1) .. +63 of the tile against weight rows
// (down) 64*(w>>1) .. +63, or (up) gate rows 32*(w>>1) .. +31 with their up
// rows: 4 x 4 MFMA tiles, 64 fp32 accumulators per lane.
//
// Token rows past the group's count repeat its last row and weight rows
// past the matrix repeat its last row: both are multiplied and never
// stored.  Bytes of a stage past the end of K are zero on both sides.
// Tiles are listed group by group, weight tile by weight tile, token tile
// fastest; the grid is the blocks that fit on the chip at once, and the
// blocks on one XCD (the hardware deals blocks to the 8 XCDs in turn) walk
// one contiguous stretch of that list, so the token tiles that share a
// weight tile run side by side on one L2 and a group's token rows stay on
// one or two XCDs.  Every output element is written by exactly one lane.
#include <type_traits>

#include "common.hpp"
#include "moe_internal.h"

namespace moe {

constexpr int TL_M = TILE_ROWS;                // token rows per tile
constexpr int TL_N = 128;                      // weight rows per tile
static_assert(TL_N == 128, "expert_tile_nt assumes 128 weight rows (64 up columns) per tile");
constexpr int TL_KB = 128;                     // K bytes per stage and row
constexpr int TL_THREADS = 256;
constexpr int TL_WBYTES = TL_N * TL_KB;        // weight part of a stage
constexpr int TL_STAGE = (TL_M + TL_N) * TL_KB;
constexpr int TL_LD = 4;                       // rows each thread fetches per operand per stage
constexpr int TL_XCD = 8;
constexpr int TL_MIN_ST = 8;                   // stages per block at least
constexpr int TL_MAX_GRID = 512;               // blocks of a launch at most
constexpr int TL_PART_FLOATS = TL_M * TL_N;    // fp32 partial tile
constexpr int TL_MAX_PIECES = 2;               // pieces a leftover tile is cut into at most
constexpr int TL_PIECE_ST = 16;                // stages per piece of a leftover tile at least

enum TMode { TMODE_UP = 0, TMODE_DOWN = 1 };

struct TArgs {
  const void* act;         // up: x (T, H); down: a (n_pairs, I')
  const int* sorted_pair;  // up: pair id of each sorted row
  const int* offsets;      // (n_groups + 1) sorted-row offsets
  const void* w;           // up: w13 (G, 2I', H); down: w2 (G, H, I')
  void* out;               // up: a (n_pairs, I'); down: y_pair (n_pairs, H)
  int n_groups;
  int kk;
  int K;                   // contraction length (elements)
  int I_loc;
  int H;
  int n_nt;                // weight tiles per group
  int m_min;               // hot-group row threshold of tile_take_all (-1: every group) ...
  int min_tiles;           // ... and the tiles all groups must make
  int* ctr;                // per-tile arrival counters of split tiles (zero between calls)
  int* claim;              // the launch's claim counter, then an exit counter (zero between calls)
  float* part;             // two fp32 partial tiles per block
  int max_pieces;          // leftover tiles are cut into at most this many pieces along K
};

// Byte offset of 16-byte chunk c (0..7) of row r inside an operand region.
// A 128-bit LDS access is served 16 lanes per cycle -- lanes 8k..8k+7 with
// lanes 32+8k..32+8k+7 -- from 64 four-byte banks, i.e. 16 slots of 16 bytes
// at address mod 256 (two rows of 128 bytes).  The XOR key (bits 1 and 2 of
// the row) makes both access patterns use 16 different slots per cycle:
//   operand reads: lanes 8k.. read rows r0..r0+7 at chunk c, lanes 32+8k..
//     the same rows at chunk c^2; even rows take keys {0,1,4,5}, so c^key
//     and c^2^key cover all 8 slots of their half, and odd rows the other half;
//   stage writes: lanes 8k.. write a whole even row, lanes 32+8k.. a whole
//     odd row (tl_wrow), one half each.
// The key depends on r % 16 only, so rows 16 apart differ by a constant.
__device__ __forceinline__ int tl_swz(int r, int c) {
  return r * TL_KB + ((c ^ (((r >> 1) & 1) | (((r >> 2) & 1) << 2))) << 4);
}

// Row (0..31, then +32, +64, +96) whose chunk `tid & 7` thread tid fetches
// and stores: a wave covers 8 consecutive rows, lanes 8k..8k+7 an even row
// and lanes 32+8k.. the next odd row.
__device__ __forceinline__ int tl_wrow(int tid) {
  const int l = tid & 63;
  return 8 * (tid >> 6) + 2 * ((l >> 3) & 3) + (l >> 5);
}

__device__ __forceinline__ int tl_uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Wave 0: s_off[g] = offsets[g]; s_tstart[g] = tiles of the groups before g.
// The kernel takes every group or none, by tile_take_all (the wave-streaming
// kernel evaluates the same rule and takes the rest).
__device__ __forceinline__ void tile_prefix(const TArgs& a, int* s_tstart, int* s_off) {
  if (threadIdx.x >= WAVE) return;
  const int l = lane_id();
  const bool all = tile_take_all(a.offsets, a.n_groups, a.m_min, a.min_tiles, TL_M, a.n_nt);
  int base = 0;
  for (int g0 = 0; g0 <= a.n_groups; g0 += WAVE) {
    const int g = g0 + l;
    if (g <= a.n_groups) s_off[g] = a.offsets[g];
    int v = 0;
    if (g < a.n_groups && all) {
      const int m = a.offsets[g + 1] - a.offsets[g];
      v = (m + TL_M - 1) / TL_M * a.n_nt;
    }
    const int incl = wave_inclusive_scan(v);
    if (g < a.n_groups) s_tstart[g] = base + incl - v;
    base += __shfl(incl, WAVE - 1, WAVE);
  }
  if (l == 0) s_tstart[a.n_groups] = base;
}

__device__ __forceinline__ uint4 tl_ldg_nt(const char* base, uint32_t off) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(base + off));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 tl_ldg(const char* base, uint32_t off) {
  return *reinterpret_cast<const uint4*>(base + off);
}

// Block that owns stage q when Q stages are cut into W ranges [Q*w/W, Q*(w+1)/W).
__device__ __forceinline__ int tl_owner(long long q, long long Q, int W) {
  return static_cast<int>(((q + 1) * W - 1) / Q);
}

// Partial slot of block v's piece of tile t: slot 0 if v's range starts in
// tile t, else slot 1 (a range holds at most two split pieces: its first
// and its last).
__device__ __forceinline__ float* tl_slot(float* part, int v, int t, int nst, long long Q, int W) {
  const long long qv = Q * v / W;
  const int which = (qv / nst == t) ? 0 : 1;
  return part + (static_cast<size_t>(v) * 2 + which) * TL_PART_FLOATS;
}

template <int MODE>
__global__ __launch_bounds__(TL_THREADS, 2) void expert_tile_kernel(TArgs a) {
  __shared__ int s_tstart[MAX_GROUPS + 1];
  __shared__ int s_off[MAX_GROUPS + 1];
  __shared__ __attribute__((aligned(16))) char s_st[2][TL_STAGE];

  const int tid = threadIdx.x;
  const int l = lane_id();
  const int wv = tl_uni(tid / WAVE);
  const int lr = l & 15;
  const int lq = l >> 4;
  const int wm = wv & 1;   // token half of the tile
  const int wn = wv >> 1;  // weight half of the tile

  __shared__ int s_flag;
  __shared__ int s_claim;

  tile_prefix(a, s_tstart, s_off);
  __syncthreads();
  const int total = tl_uni(s_tstart[a.n_groups]);
  const uint32_t row_bytes = static_cast<uint32_t>(a.K) * 2;
  const int kbytes = a.K * 2;
  const int nst = (kbytes + TL_KB - 1) / TL_KB;

  // Few tiles (under half a tile per block): stream-K -- the tiles' stages,
  // Q in all, are cut into W equal contiguous ranges, one per block (at
  // least TL_MIN_ST stages each), and a tile whose stages fall into several
  // ranges is split along K: each of those blocks stores its fp32 partial,
  // and the last to arrive sums them in K order.  Logical block w runs on
  // XCD w / (W/8), so neighbouring ranges share an L2.
  const long long Q = static_cast<long long>(total) * nst;
  int W = min(static_cast<int>(gridDim.x), TL_MAX_GRID) / TL_XCD * TL_XCD;
  if (Q < static_cast<long long>(W) * TL_MIN_ST) W = max(TL_XCD, static_cast<int>(Q / TL_MIN_ST) / TL_XCD * TL_XCD);
  const int per = W / TL_XCD;
  if (static_cast<int>(blockIdx.x) / TL_XCD >= per || Q == 0) return;  // block-uniform
  const int w = (blockIdx.x % TL_XCD) * per + blockIdx.x / TL_XCD;
  // With at least half a tile per block no tile is split (a split costs a
  // partial tile's store and reload and a pipeline refill, more than the
  // finer balance gains): XCD x takes the x-th eighth of the tile list and
  // its blocks deal those tiles out in turn, so the token tiles that share
  // a weight tile run side by side and read it from HBM once.  When an
  // eighth holds only a few tiles more than its blocks (at most a quarter
  // more), each block starts on one of its first tiles and the few left go
  // to whichever blocks finish first, so tiles that run long do not leave
  // the launch waiting on a fixed block's second tile.  Each leftover tile is
  // cut along K into S <= TL_MAX_PIECES pieces of at least TL_PIECE_ST
  // stages, S chosen so that all pieces of an eighth could run at once on its
  // blocks.  The pieces of all eighths form one list (eighth by eighth, tile
  // by tile, in K order) handed out by one counter, so a block of an XCD that
  // finishes early also takes pieces of the other XCDs' leftovers (one
  // counter per eighth left EP B = 2048 up 9 us longer); the last piece of a
  // tile to finish sums the pieces' partials in K order.  The leftover then
  // costs about a piece's time after the first tiles instead of a tile's.
  // (More or shorter pieces measured slower: each adds a partial tile's store
  // and reload and a pipeline refill.)
  // With more left over, dealing them out keeps the token tiles of a weight
  // tile together, which measured faster; with none, the claims and their
  // contended counters would only add time.
  const bool whole = 2 * static_cast<long long>(total) >= W;
  const int surplus = (total + TL_XCD - 1) / TL_XCD - per;   // tiles of the largest eighth beyond one per block
  const bool claim = whole && surplus > 0 && 4 * surplus <= per;
  const int n_pc = claim ? max(1, min(min(per / max(surplus, 1), nst / TL_PIECE_ST), a.max_pieces)) : 1;
  const int t_lo = static_cast<int>(static_cast<long long>(total) * (blockIdx.x % TL_XCD) / TL_XCD);
  const int t_hi = static_cast<int>(static_cast<long long>(total) * (blockIdx.x % TL_XCD + 1) / TL_XCD);
  const int t_first = t_lo + static_cast<int>(blockIdx.x / TL_XCD);
  const long long q0 = whole ? static_cast<long long>(t_first) * nst : Q * w / W;
  const long long q1 = whole ? static_cast<long long>(t_hi) * nst : Q * (w + 1) / W;
  const int lc = tid & 7;        // 16-byte chunk of a stage row this thread fetches
  const int lrow = tl_wrow(tid); // first row it fetches; then +32, +64, +96
  const char* act = reinterpret_cast<const char*>(a.act);

  // LDS offsets of the four rows this thread stores (same for both operands)
  int sw[TL_LD];
#pragma unroll
  for (int i = 0; i < TL_LD; ++i) sw[i] = tl_swz(lrow + 32 * i, lc);

  // claimable pieces: the tiles of each eighth beyond one per block, n_pc each
  const int n_claims = claim ? (total - W) * n_pc : 0;
  long long q = q0;
  int c = -1;   // claim of the current unit (claiming launches; -1: the block's first tile)
  for (;;) {
    // ---- this block's piece of tile t: stages [sb, se) (block-uniform)
    int t, sb, se;
    int pj = 0;  // piece of a claimed leftover tile
    if (claim) {
      if (c < 0) {
        t = t_first;   // < t_lo + per <= t_hi
        sb = 0;
        se = nst;
      } else {
        if (c >= n_claims) break;
        // the eighth whose leftover pieces hold claim c (block-uniform)
        int base = 0, x = 0, nx = 0;
        for (; x < TL_XCD - 1; ++x) {
          nx = (static_cast<int>(static_cast<long long>(total) * (x + 1) / TL_XCD) -
                static_cast<int>(static_cast<long long>(total) * x / TL_XCD) - per) * n_pc;
          if (c < base + nx) break;
          base += nx;
        }
        const int u = (c - base) / n_pc;
        pj = c - base - u * n_pc;
        t = static_cast<int>(static_cast<long long>(total) * x / TL_XCD) + per + u;
        sb = pj * nst / n_pc;
        se = (pj + 1) * nst / n_pc;
      }
    } else {
      if (q >= q1) break;
      t = static_cast<int>(q / nst);
      sb = static_cast<int>(q - static_cast<long long>(t) * nst);
      se = static_cast<int>(min(static_cast<long long>(nst), q1 - static_cast<long long>(t) * nst));
      q = static_cast<long long>(whole ? t + per : t + 1) * nst;
    }
    int lo = 0, hi = a.n_groups;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tl_uni(s_tstart[mid]) <= t) lo = mid;
      else hi = mid;
    }
    const int g = lo;
    const int row0 = tl_uni(s_off[g]);
    const int m = tl_uni(s_off[g + 1]) - row0;
    const int n_mt = (m + TL_M - 1) / TL_M;
    const int local = t - tl_uni(s_tstart[g]);
    const int nt = local / n_mt;
    const int mt = local - nt * n_mt;
    const int m0 = mt * TL_M;

    // ---- this thread's weight and token rows (byte offsets of chunk lc)
    const char* wbase;
    uint32_t woff[TL_LD], xoff[TL_LD];
    if (MODE == TMODE_UP) {
      wbase = reinterpret_cast<const char*>(a.w) + static_cast<size_t>(g) * 2 * a.I_loc * row_bytes;
#pragma unroll
      for (int i = 0; i < TL_LD; ++i) {
        const int r = lrow + 32 * i;
        const int n = min(nt * 64 + (r & 63), a.I_loc - 1);
        woff[i] = static_cast<uint32_t>(n + (r >= 64 ? a.I_loc : 0)) * row_bytes + 16 * lc;
      }
    } else {
      wbase = reinterpret_cast<const char*>(a.w) + static_cast<size_t>(g) * a.H * row_bytes;
#pragma unroll
      for (int i = 0; i < TL_LD; ++i) {
        const int n = min(nt * TL_N + lrow + 32 * i, a.H - 1);
        woff[i] = static_cast<uint32_t>(n) * row_bytes + 16 * lc;
      }
    }
#pragma unroll
    for (int i = 0; i < TL_LD; ++i) {
      const int r = row0 + min(m0 + lrow + 32 * i, m - 1);
      const int tok = (MODE == TMODE_UP) ? a.sorted_pair[r] / a.kk : r;
      xoff[i] = static_cast<uint32_t>(tok) * row_bytes + 16 * lc;
    }

    // ---- K loop: stage s is fetched two stages ahead into registers
    // (a chunk past the end of K re-reads the row's last valid 64 bytes;
    // lstore zeroes it)
    // A group with more than one token tile reads each weight tile once per
    // token tile; those tiles run side by side on one XCD, so their weights
    // are read with the ordinary policy and the later reads find them in L2.
    // Every other weight tile is streamed once, non-temporally.
    const bool keep = n_mt > 1;
    auto gload = [&](auto keep_tag, int s, uint4 (&R)[2 * TL_LD]) {
      const int delta = min(0, kbytes - 16 - s * TL_KB - 16 * lc) & ~63;
      const char* wb = wbase + s * TL_KB;
      const char* xb = act + s * TL_KB;
      if constexpr (decltype(keep_tag)::value) {
#pragma unroll
        for (int i = 0; i < TL_LD; ++i) R[i] = tl_ldg(wb, woff[i] + delta);
      } else {
#pragma unroll
        for (int i = 0; i < TL_LD; ++i) R[i] = tl_ldg_nt(wb, woff[i] + delta);
      }
#pragma unroll
      for (int i = 0; i < TL_LD; ++i) R[TL_LD + i] = tl_ldg(xb, xoff[i] + delta);
    };
    auto lstore = [&](int s, const uint4 (&R)[2 * TL_LD], char* buf) {
      const bool ok = s * TL_KB + 16 * lc < kbytes;  // chunk inside K
#pragma unroll
      for (int i = 0; i < TL_LD; ++i) *reinterpret_cast<uint4*>(buf + sw[i]) = keep_or_zero(ok, R[i]);
#pragma unroll
      for (int i = 0; i < TL_LD; ++i)
        *reinterpret_cast<uint4*>(buf + TL_WBYTES + sw[i]) = keep_or_zero(ok, R[TL_LD + i]);
    };

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // operand rows of this wave inside the tile
    int arow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (MODE == TMODE_UP) arow[i] = (i < 2 ? 0 : 64) + 32 * wn + 16 * (i & 1) + lr;
      else arow[i] = 64 * wn + 16 * i + lr;
    }
    auto compute = [&](const char* buf) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 4 * h + lq;
        uint4 A[4], B[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) A[i] = *reinterpret_cast<const uint4*>(buf + tl_swz(arow[i], c));
#pragma unroll
        for (int j = 0; j < 4; ++j)
          B[j] = *reinterpret_cast<const uint4*>(buf + TL_WBYTES + tl_swz(64 * wm + 16 * j + lr, c));
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = Elem<uint16_t>::mma(A[i], B[j], acc[i][j]);
      }
    };

    // Three register stages: while stage s is multiplied out of LDS, stages
    // s+1 and s+2 are in flight and s+3 is issued.  LDS holds two stages
    // (stage s in buffer s & 1).  Each trip takes three stages with no exit
    // in between and unconditional stores (a stage past the range is stored
    // and never read), so every path into the loop header leaves the same
    // loads outstanding and the compiler's wait counts stay exact.
    // The load policy is a template parameter of the K loop, fixed per tile:
    // with a branch around the weight loads inside the loop the compiler
    // cannot tell which loads are outstanding, and its wait before each
    // stage's store would drain the next stage's loads as well (one stage
    // in flight instead of two).
    auto kloop = [&](auto keep_tag) {
      uint4 R0[2 * TL_LD], R1[2 * TL_LD], R2[2 * TL_LD];
      gload(keep_tag, sb, R0);
      gload(keep_tag, min(sb + 1, se - 1), R1);
      gload(keep_tag, min(sb + 2, se - 1), R2);
      lstore(sb, R0, s_st[sb & 1]);
      __syncthreads();
      int s = sb;
      for (; s + 2 < se; s += 3) {
        char* b0 = s_st[s & 1];
        char* b1 = s_st[(s + 1) & 1];
        gload(keep_tag, min(s + 3, se - 1), R0);
        __builtin_amdgcn_sched_barrier(0);
        compute(b0);                     // stage s
        __builtin_amdgcn_sched_barrier(0);
        lstore(s + 1, R1, b1);
        __syncthreads();
        gload(keep_tag, min(s + 4, se - 1), R1);
        __builtin_amdgcn_sched_barrier(0);
        compute(b1);                     // stage s+1
        __builtin_amdgcn_sched_barrier(0);
        lstore(s + 2, R2, b0);
        __syncthreads();
        gload(keep_tag, min(s + 5, se - 1), R2);
        __builtin_amdgcn_sched_barrier(0);
        compute(b0);                     // stage s+2
        __builtin_amdgcn_sched_barrier(0);
        lstore(s + 3, R0, b1);
        __syncthreads();
      }
      // at most two stages are left: s in LDS, s+1 in R1
      if (s < se) {
        compute(s_st[s & 1]);
        if (s + 1 < se) {
          lstore(s + 1, R1, s_st[(s + 1) & 1]);
          __syncthreads();
          compute(s_st[(s + 1) & 1]);
        }
      }
    };
    if (keep) kloop(std::true_type{});
    else kloop(std::false_type{});

    // ---- split tile: store this piece's partial; the last piece of the tile
    // to arrive sums all of them in K order into acc.  Only the 16-row token
    // tiles that hold rows of the group are kept.  Stream-K pieces belong to
    // blocks wa..wb (two partial slots per block); a claimed piece has the
    // slot of its claim number (< W), so piece pj of a tile is pj slots after
    // the tile's first.
    bool epilogue = true;
    if (sb != 0 || se != nst) {
      int wa, wb;
      float* mine;
      if (claim) {
        wa = c - pj;
        wb = wa + n_pc - 1;
        mine = a.part + static_cast<size_t>(c) * TL_PART_FLOATS;
      } else {
        const long long qa = static_cast<long long>(t) * nst;
        wa = tl_owner(qa, Q, W);
        wb = tl_owner(qa + nst - 1, Q, W);
        mine = tl_slot(a.part, w, t, nst, Q, W);
      }
      const int l_rows = m - m0 - 64 * wm;   // valid token rows of this wave's half
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (16 * j < l_rows) {
            uint64_t* p = reinterpret_cast<uint64_t*>(mine + ((i * 4 + j) * TL_THREADS + tid) * 4);
            st_agent(p, (static_cast<uint64_t>(__float_as_uint(acc[i][j][1])) << 32) | __float_as_uint(acc[i][j][0]));
            st_agent(p + 1, (static_cast<uint64_t>(__float_as_uint(acc[i][j][3])) << 32) | __float_as_uint(acc[i][j][2]));
          }
      epilogue = last_to_arrive(a.ctr + t, wb - wa + 1, &s_flag);  // block-uniform
      for (int v = wa; epilogue && v <= wb; ++v) {
        const float* src = claim ? a.part + static_cast<size_t>(v) * TL_PART_FLOATS : tl_slot(a.part, v, t, nst, Q, W);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (16 * j < l_rows) {
              const uint64_t* p = reinterpret_cast<const uint64_t*>(src + ((i * 4 + j) * TL_THREADS + tid) * 4);
              const uint64_t lo2 = ld_agent(p);
              const uint64_t hi2 = ld_agent(p + 1);
              const f32x4_t pv = {__uint_as_float(static_cast<uint32_t>(lo2)), __uint_as_float(static_cast<uint32_t>(lo2 >> 32)),
                                  __uint_as_float(static_cast<uint32_t>(hi2)), __uint_as_float(static_cast<uint32_t>(hi2 >> 32))};
              acc[i][j] = (v == wa) ? pv : acc[i][j] + pv;
            }
      }
    }

    // ---- epilogue: acc[i][j][r] = D[weight row 4*lq + r of tile i][token row lr of tile j]
    if (epilogue && MODE == TMODE_UP) {
      uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int n = nt * 64 + 32 * wn + 16 * i + 4 * lq;
        if (n < a.I_loc) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int tr = m0 + 64 * wm + 16 * j + lr;
            if (tr < m) {
              float o[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float gt = acc[i][j][r];
                o[r] = gt / (1.0f + __expf(-gt)) * acc[i + 2][j][r];
              }
              Elem<uint16_t>::store4(out + static_cast<size_t>(row0 + tr) * a.I_loc + n, o[0], o[1], o[2], o[3]);
            }
          }
        }
      }
    } else if (epilogue) {
      uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = nt * TL_N + 64 * wn + 16 * i + 4 * lq;
        if (n < a.H) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int tr = m0 + 64 * wm + 16 * j + lr;
            if (tr < m)
              Elem<uint16_t>::store4(out + static_cast<size_t>(row0 + tr) * a.H + n, acc[i][j][0], acc[i][j][1],
                                     acc[i][j][2], acc[i][j][3]);
          }
        }
      }
    }
    // the next tile's first stage goes to s_st[0], which the last stage may have used
    __syncthreads();
    if (claim) {
      // the next piece, or past the end of the list when none is left
      if (tid == 0) s_claim = atomicAdd(a.claim, 1);
      __syncthreads();
      c = s_claim;
    }
  }
  // Every block of a claiming launch arrives here after its last claim; the
  // last one clears the claim counter for the next call.
  if (claim && last_to_arrive(a.claim + 1, W, &s_flag) && tid == 0) a.claim[0] = 0;
}

// ---------------------------------------------------------------- host side

template <int MODE>
static int tile_resident_blocks() {
  static const int per_cu =
      kernel_blocks_per_cu(reinterpret_cast<const void*>(&expert_tile_kernel<MODE>), TL_THREADS);
  return device_cu_count() * per_cu;
}

// Tiles of one launch at most: groups with more than m_min rows number at
// most pairs / (m_min + 1) (and at most n_groups), and hold at most
// pairs / 128 + that many token tiles.  The kernels may take every
// non-empty group, so the counters are sized with m_min = 0.
static long long tile_bound(int T, int kk, int n_groups, int m_min, int n_nt) {
  const long long pairs = static_cast<long long>(T) * kk;
  long long big = pairs / (m_min + 1);
  if (big > n_groups) big = n_groups;
  return (pairs / TL_M + big) * n_nt;
}

// Split-tile counters (one per tile at most), then the claim counters.
static long long tl_split_ctrs(int T, int kk, int n_groups, int H, int I) {
  long long n = tile_bound(T, kk, n_groups, 0, expert_tile_nt(true, H, I));
  const long long d = tile_bound(T, kk, n_groups, 0, expert_tile_nt(false, H, I));
  return d > n ? d : n;
}
static size_t tl_ctr_bytes(int T, int kk, int n_groups, int H, int I) {
  const long long n = tl_split_ctrs(T, kk, n_groups, H, I) + 2;
  return (static_cast<size_t>(n) * sizeof(int) + 255) & ~static_cast<size_t>(255);
}

// The grid is every block that fits on the chip at once (a multiple of the
// XCD count, at most TL_MAX_GRID); the tile path takes the groups only when
// they make at least a third of a tile per compute unit (fewer tiles leave
// most of the chip idle, and the wave-streaming kernel does better).  When
// the wave-streaming kernel takes 64-row passes (m_min is TILE_M_MIN_WIDE) it
// needs a tile per compute unit.
static int tile_min_tiles(int m_min) {
  return m_min >= TILE_M_MIN_WIDE ? device_cu_count() : (device_cu_count() + 2) / 3;
}

template <int MODE>
static void tile_launch(TArgs a, int T, void* ws, hipStream_t s) {
  int grid = tile_resident_blocks<MODE>();
  if (grid > TL_MAX_GRID) grid = TL_MAX_GRID;
  grid = grid / TL_XCD * TL_XCD;
  if (grid < TL_XCD) grid = TL_XCD;
  a.min_tiles = a.m_min < 0 ? 0 : tile_min_tiles(a.m_min);
  a.ctr = static_cast<int*>(ws);
  a.claim = a.ctr + tl_split_ctrs(T, a.kk, a.n_groups, a.H, a.I_loc);
  a.part = reinterpret_cast<float*>(static_cast<char*>(ws) + tl_ctr_bytes(T, a.kk, a.n_groups, a.H, a.I_loc));
  a.max_pieces = TL_MAX_PIECES;
  hipLaunchKernelGGL(expert_tile_kernel<MODE>, dim3(static_cast<unsigned>(grid)), dim3(TL_THREADS), 0, s, a);
}

bool expert_tile_used(int T, int dtype) { return dtype == 1 && T > TILE_T_MIN; }

int expert_tile_min_tiles(int m_min) { return tile_min_tiles(m_min < TILE_M_MIN ? TILE_M_MIN : m_min); }

size_t expert_tile_workspace_bytes(int T, int kk, int n_groups, int H, int I, int dtype) {
  if (!expert_tile_used(T, dtype)) return 0;
  return tl_ctr_bytes(T, kk, n_groups, H, I) + static_cast<size_t>(TL_MAX_GRID) * 2 * TL_PART_FLOATS * sizeof(float);
}

void launch_expert_up_tiles(const void* x, const int32_t* sorted_pair, const int32_t* offsets, int n_groups,
                            int T, int kk, const void* w13, int H, int I, void* A, int m_min, void* ws,
                            hipStream_t s) {
  TArgs a{};
  a.act = x;
  a.sorted_pair = sorted_pair;
  a.offsets = offsets;
  a.w = w13;
  a.out = A;
  a.n_groups = n_groups;
  a.kk = kk;
  a.K = H;
  a.I_loc = I;
  a.H = H;
  a.n_nt = expert_tile_nt(true, H, I);
  a.m_min = m_min < 0 ? -1 : (m_min < TILE_M_MIN ? TILE_M_MIN : m_min);
  tile_launch<TMODE_UP>(a, T, ws, s);
}

void launch_expert_down_tiles(const void* A, const int32_t* offsets, int n_groups, int T, int kk,
                              const void* w2, int H, int I, void* y_pair, int m_min, void* ws, hipStream_t s) {
  TArgs a{};
  a.act = A;
  a.offsets = offsets;
  a.w = w2;
  a.out = y_pair;
  a.n_groups = n_groups;
  a.kk = kk;
  a.K = I;
  a.I_loc = I;
  a.H = H;
  a.n_nt = expert_tile_nt(false, H, I);
  a.m_min = m_min < 0 ? -1 : (m_min < TILE_M_MIN ? TILE_M_MIN : m_min);
  tile_launch<TMODE_DOWN>(a, T, ws, s);
}

}  // namespace moe
