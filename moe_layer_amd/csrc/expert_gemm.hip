// Expert grouped GEMMs (bf16 or fp32 storage, fp32 accumulate):
//   up   : a[r]      = silu(W1_g x_t) * (W3_g x_t)   from W13_g (2I', H)
//   down : y_pair[r] = W2_g a[r]                      from W2_g  (H, I')
// for every sorted pair row r of expert group g (Moebius review, §3.1 gives
// W13 as (., 2I, H) and W2 as (., H, I); the gate-then-up row order is this
// library's layout contract).
//
// Decode-shaped problems are HBM-bound: every weight byte must stream from
// HBM exactly once while the token side (a few to a few dozen rows per
// expert) is small and stays in L2.  At larger batches (bf16, T > 256) the
// groups with many rows may have been taken by the LDS-tiled kernels
// (expert_tile.hip) launched just before; this kernel re-derives that
// decision from the same counts and skips exactly those groups.
//
// Work item = (group g, SUB adjacent weight tiles (1 or 4, per launch), pass
// of 16 token rows -- 16*NT in the kernels holding NT = 2 or 4 token tiles
// when the group has more than 16) over the full K.  A kernel built for four
// token tiles also holds the two-tile body and runs it when no group it takes
// has more than 32 rows (the first wave decides when it builds the item
// table).  A weight tile is 16 rows:
//   up   : 8 gate rows and the matching 8 up rows, so SiLU(gate)*up is
//          formed in registers;
//   down : 16 rows of W2 = 16 output features.
// K is walked in 512-byte chunks; for each chunk the wave loads the token
// fragments once and multiplies them against the chunk of each of the item's
// tiles in turn, so with four tiles every token byte fetched serves four
// times as many weight bytes (with a few dozen tokens per expert their rows
// no longer fit L1, and these L2 reads otherwise crowd out the weight
// stream); four tiles also keep very short rows (small K) from making items
// too small.  With few tokens, one tile keeps items fine-grained.  A group's
// items run tile-major, so the passes over one set of tiles are adjacent.
// Tiles of the last item past the matrix alias tile 0 (read, never stored),
// so every step issues the same loads.
//
// Balance.  With every CU streaming, one CU moves only ~1/256 of the chip's
// HBM bandwidth, so the launch lasts as long as its most loaded CU.  The
// grid is therefore exactly the waves that fit on the chip at once, and the
// flattened sequence of (item, chunk) is cut into equal contiguous ranges,
// one per wave (an eighth of them per XCD, see the kernel; a partly used
// grid still covers every CU).  An item whose chunks fall into several waves' ranges is
// split along K: each of those waves stores its fp32 partial tiles, and the
// last of them to arrive (an integer counter per item; nobody waits) adds the
// partials in K order and runs the epilogue.  Only a range's first and last
// items can be split; the first one's partial stays in registers and both are
// handed over when the range's stream has ended, because the arrival count
// must wait for the partial's stores, and in mid-stream that wait would also
// wait for every weight load in flight.  The sum order depends only on the
// shapes and the grid, so results are reproducible.  Waves are otherwise
// independent: nothing synchronises them after start-up, so a slow load only
// ever stalls its own wave.
//
// Weights are read DRAM-friendly: each load instruction takes 256 contiguous
// bytes from each of 4 rows (non-temporal, streamed once), double-buffered in
// registers so the next tile-chunk is in flight while the current one is
// multiplied.  The wave passes each 16 rows x 512 B through a private LDS
// tile (rows padded by 16 B) to read them back in the 16x16 MFMA operand
// layout (lane l: row l%16, bytes 16*(l/16) of each 64-byte fragment); only
// the wave itself touches that tile, so no barrier is needed.  Token
// fragments of a chunk come from L2 just before use and are issued ahead of
// the next weight load, so waiting for them (loads retire in order) never
// waits for the weights in flight.  All addresses are a wave-uniform base
// plus a 32-bit lane offset (scalar-base loads, constant offsets folded into
// the instructions).  The stream runs across item boundaries, and the next
// item's token-row indices are fetched one item ahead (at start-up, before
// the first weight chunk, so forming them does not wait for it).
//
// Every load sits on the straight-line path: the next chunk's base is chosen
// with scalar selects, and K that is a whole number of 512-byte chunks gets
// its own instantiation without the partial-chunk masks.  A load issued on
// one side of a branch lands in other registers than on the other side; the
// join then copies them, and the copy waits for the load -- and, loads
// retiring in order, for all the weight loads issued before it.  Token rows past the
// group's count repeat a real row and are never stored; fragments past the
// end of K are zero on both sides.  Every output element is written by
// exactly one lane.
#include <algorithm>

#include "common.hpp"
#include "moe_internal.h"
#include "stream_ops.hpp"

namespace moe {


constexpr int XW_WAVES = 4;                             // waves per block (independent)
constexpr int SUB_MAX = 4;                              // weight tiles per item at most
constexpr int MIN_CPW = 2;                              // chunks per wave at least (bounds split items)
constexpr int MAX_WAVES = 2048;                         // waves of one launch at most
constexpr int NT_MAX = 4;
constexpr int COOP_T_MAX = 128;                         // batches the block-cooperative kernel takes

// acc[s][tt][r] = D[4*lq + r][lrow] of tile s: weight row 4*lq+r of the
// tile's 16, token row tt*16+lrow.  Tiles past the matrix are not stored.
template <typename T, int MODE, int NT, int SUB>
__device__ __forceinline__ void wstore(const XArgs& a, const WItem<NT>& it, f32x4_t (&acc)[SUB][NT],
                                       int lrow, int lq) {
#pragma unroll
  for (int s = 0; s < SUB; ++s) {
    if (s < it.n_sub) {
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const int tr = it.t0 + tt * 16 + lrow;
        if (MODE == XMODE_UP) {
          float up[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) up[r] = __shfl_xor(acc[s][tt][r], 32, WAVE);
          const int n = it.n0 + 8 * s + 4 * lq;
          if (lq < 2 && tr < it.m_end) {
            float o[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float gt = acc[s][tt][r];
              o[r] = gt / (1.0f + __expf(-gt)) * up[r];
            }
            T* dst = reinterpret_cast<T*>(a.out) + static_cast<size_t>(it.row0 + tr) * a.I_loc + n;
            Elem<T>::store4(dst, o[0], o[1], o[2], o[3]);
          }
        } else {
          const int n = it.n0 + 16 * s + 4 * lq;
          if (tr < it.m_end) {
            T* dst = reinterpret_cast<T*>(a.out) + static_cast<size_t>(it.row0 + tr) * a.H + n;
            Elem<T>::store4(dst, acc[s][tt][0], acc[s][tt][1], acc[s][tt][2], acc[s][tt][3]);
          }
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[s][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
}

// Wave that owns chunk q when Q chunks are cut into W ranges [Q*w/W, Q*(w+1)/W).
__device__ __forceinline__ int chunk_owner(long long q, long long Q, int W) {
  return static_cast<int>(((q + 1) * W - 1) / Q);
}

// A wave's partial of an item goes to slot 0 if the item is the first one its
// range touches, else to slot 1 (a range has at most two split items).
__device__ __forceinline__ float* part_slot(const XArgs& a, int tiles, int w, int item, long long Q, int W) {
  const long long q0 = Q * w / W;
  const int which = (q0 / a.nck == item) ? 0 : 1;
  return a.part + (static_cast<size_t>(w) * 2 + which) * tiles * WAVE * 4;
}

// Store this wave's partial of a split item (agent scope, no wait).
template <typename T, int MODE, int NT, int SUB>
__device__ __forceinline__ void split_publish(const XArgs& a, const f32x4_t (&acc)[SUB][NT], int item, int w, int W,
                                              long long Q) {
  const int l = lane_id();
  uint64_t* mine = reinterpret_cast<uint64_t*>(part_slot(a, SUB * NT, w, item, Q, W));
#pragma unroll
  for (int s = 0; s < SUB; ++s)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      uint64_t* p = mine + ((s * NT + tt) * WAVE + l) * 2;
      st_agent(p, (static_cast<uint64_t>(__float_as_uint(acc[s][tt][1])) << 32) | __float_as_uint(acc[s][tt][0]));
      st_agent(p + 1, (static_cast<uint64_t>(__float_as_uint(acc[s][tt][3])) << 32) | __float_as_uint(acc[s][tt][2]));
    }
}

// Arrivals counted for a split item so far, before this one, equals the
// number of other contributors: this wave is the last.
__device__ __forceinline__ int split_others(const XArgs& a, int item, long long Q, int W) {
  const long long qa = static_cast<long long>(item) * a.nck;
  return chunk_owner(qa + a.nck - 1, Q, W) - chunk_owner(qa, Q, W);
}

template <typename T, int MODE, int NT, int SUB>
__device__ __forceinline__ void split_reduce(const XArgs& a, const WItem<NT>& it, f32x4_t (&acc)[SUB][NT],
                                             int item, int w, int W, long long Q, int lrow, int lq, bool last) {
  const int l = lane_id();
  const long long qa = static_cast<long long>(item) * a.nck;
  const int wa = chunk_owner(qa, Q, W);
  const int wb = chunk_owner(qa + a.nck - 1, Q, W);
  if (last) {  // last to arrive (wave-uniform)
    if (l == 0) st_agent(a.ctr + item, 0);
    f32x4_t sum[SUB][NT];
    for (int v = wa; v <= wb; ++v) {
      if (v == w) {
#pragma unroll
        for (int s = 0; s < SUB; ++s)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) sum[s][tt] = (v == wa) ? acc[s][tt] : sum[s][tt] + acc[s][tt];
      } else {
        const uint64_t* src = reinterpret_cast<const uint64_t*>(part_slot(a, SUB * NT, v, item, Q, W));
#pragma unroll
        for (int s = 0; s < SUB; ++s)
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) {
            const uint64_t* p = src + ((s * NT + tt) * WAVE + l) * 2;
            const uint64_t lo = ld_agent(p);
            const uint64_t hi = ld_agent(p + 1);
            const f32x4_t pv = {__uint_as_float(static_cast<uint32_t>(lo)), __uint_as_float(static_cast<uint32_t>(lo >> 32)),
                                __uint_as_float(static_cast<uint32_t>(hi)), __uint_as_float(static_cast<uint32_t>(hi >> 32))};
            sum[s][tt] = (v == wa) ? pv : sum[s][tt] + pv;
          }
      }
    }
    wstore<T, MODE, NT, SUB>(a, it, sum, lrow, lq);
  }
#pragma unroll
  for (int s = 0; s < SUB; ++s)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[s][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
}

// The streaming part of the kernel, after the item table is built.
// KEEP: items whose tiles have later passes read their weights with the
// ordinary (temporal) policy, so the passes that follow (adjacent items,
// running at the same time on the same XCD) find them in L2; all other weights
// stream non-temporally.  Launches where every group fits one pass run the
// body without that choice.
// Blocks 0 .. nblk-1 of the grid take part.
template <typename T, int MODE, int NT, int SUB, bool FULLK, bool KEEP>
__device__ __forceinline__ void stream_body(const XArgs& a, const int* s_istart, const int* s_off, char* tile,
                                            int wv, int l, int lrow, int lq, int nblk) {
  const long long Q = static_cast<long long>(uni(s_istart[a.n_groups])) * a.nck;
  const int W = static_cast<int>(min(static_cast<long long>(nblk) * XW_WAVES, (Q + MIN_CPW - 1) / MIN_CPW));
  // Range index.  Blocks are dealt to the 8 XCDs in turn, so XCD x holds the
  // blocks b with b % 8 == x; it takes the contiguous ranges [x*W/8,
  // (x+1)*W/8), first one wave of each of its blocks, then the next.  Its
  // waves then work on neighbouring groups, whose token rows (and the
  // down-projection's `a` rows, re-read by every item of a group) stay in that
  // XCD's L2.  The assignment covers every range whenever the grid is a
  // multiple of 8 (always here; otherwise wave w takes range w).
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
  const long long q0 = Q * w / W;
  const long long q1 = Q * (w + 1) / W;
  if (q0 >= q1) return;

  const uint32_t row_bytes = static_cast<uint32_t>(a.K) * sizeof(T);
  const char* act = reinterpret_cast<const char*>(a.act);
  const int kbytes = a.kfrag_total * FRAG_BYTES;

  int item = static_cast<int>(q0 / a.nck);
  int cb = static_cast<int>(q0 - static_cast<long long>(item) * a.nck);   // first chunk of the item here
  int ce = static_cast<int>(min(static_cast<long long>(a.nck), q1 - static_cast<long long>(item) * a.nck));

  // The first weight chunk goes out before the token indices are fetched.
  WItem<NT> cur, nxt;
  witem_weights<T, MODE, NT, SUB>(a, s_istart, s_off, item, lrow, lq, row_bytes, cur);
  nxt = cur;
  uint4 w0[CHUNK_FRAGS], w1[CHUNK_FRAGS], x[NT][CHUNK_FRAGS];
  int c = cb;
  // Token ids first, then the first weight chunk: forming the token offsets
  // then waits only for the ids, not for the weight chunk behind them.
  int raw_c[NT], raw_n[NT];
  witem_token_ids<T, MODE, NT>(a, lrow, cur, raw_c);
  bool have_nxt = static_cast<long long>(item + 1) * a.nck < q1;
  if (have_nxt) {
    witem_weights<T, MODE, NT, SUB>(a, s_istart, s_off, item + 1, lrow, lq, row_bytes, nxt);
    witem_token_ids<T, MODE, NT>(a, lrow, nxt, raw_n);
  }
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (FULLK && KEEP)
    wload_full_keep(tile_chunk(cur, 0, c), cur.woff, w0, cur.keep);
  else if constexpr (FULLK)
    wload_full(tile_chunk(cur, 0, c), cur.woff, w0);
  else if constexpr (KEEP)
    wload_part_keep(tile_chunk(cur, 0, c), cur.woff, kbytes - c * CHUNK_BYTES, lrow, w0, cur.keep);
  else
    wload(tile_chunk(cur, 0, c), cur.woff, kbytes - c * CHUNK_BYTES, lrow, w0);
  __builtin_amdgcn_sched_barrier(0);
  witem_token_offsets<T, MODE, NT>(a, lq, row_bytes, raw_c, cur);
  if (have_nxt) witem_token_offsets<T, MODE, NT>(a, lq, row_bytes, raw_n, nxt);

  f32x4_t acc[SUB][NT];
#pragma unroll
  for (int s = 0; s < SUB; ++s)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[s][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Sub-step S of a chunk step: load the next tile-chunk into WN (tile S+1
  // of this chunk; after the last tile, tile 0 of the next chunk, of the next
  // item, or with no work left a harmless re-read), then multiply WC, the
  // chunk of tile S, with the chunk's token fragments.  Full chunks take the
  // plain paths; only a partial last chunk of K takes the masked ones, which
  // issue the same loads, so the outstanding-load count never depends on the
  // path.
#define XSUB(S, WC, WN)                                                                   \
  if constexpr (S < SUB) {                                                                \
    {                                                                                     \
      const char* nb;                                                                     \
      int nv;                                                                             \
      bool nk;                                                                            \
      if (S + 1 < SUB) {                                                                  \
        nb = tile_chunk(cur, S + 1, c);                                                   \
        nv = cvalid;                                                                      \
        nk = cur.keep;                                                                    \
      } else {                                                                            \
        const char* b_next = tile_chunk(cur, 0, c + 1);                                   \
        const char* b_item = tile_chunk(nxt, 0, 0);                                       \
        const char* b_same = tile_chunk(cur, 0, c);                                       \
        nb = !last ? b_next : (have_nxt ? b_item : b_same);                               \
        nv = !last ? cvalid - CHUNK_BYTES : (have_nxt ? kbytes : cvalid);                 \
        nk = (last && have_nxt) ? nxt.keep : cur.keep;                                    \
      }                                                                                   \
      if constexpr (FULLK && KEEP)                                                        \
        wload_full_keep(nb, cur.woff, WN, nk);                                            \
      else if constexpr (FULLK)                                                           \
        wload_full(nb, cur.woff, WN);                                                     \
      else if constexpr (KEEP)                                                            \
        wload_part_keep(nb, cur.woff, nv, lrow, WN, nk);                                  \
      else                                                                                \
        wload(nb, cur.woff, nv, lrow, WN);                                                \
    }                                                                                     \
    __builtin_amdgcn_sched_barrier(0);                                                    \
    uint4 wt[CHUNK_FRAGS];                                                                \
    wtranspose(WC, tile, lrow, lq, wt);                                                   \
    if (FULLK || cvalid >= CHUNK_BYTES)                                                   \
      wmma_full<T, NT>(wt, x, cur.m_end - cur.t0, acc[S]);                                \
    else                                                                                  \
      wmma_part<T, NT>(wt, x, cvalid / FRAG_BYTES, cur.m_end - cur.t0, acc[S]);           \
  }

  // One chunk step: the chunk's token fragments, then the SUB tiles (the
  // register buffers alternate, starting with WA); at the end of the item's
  // chunks in this range, finish it and move on (break when the range is
  // done).
#define CSTEP(WA, WB)                                                                     \
  {                                                                                       \
    const int cvalid = kbytes - c * CHUNK_BYTES; /* bytes of K left from this chunk on */ \
    if constexpr (FULLK)                                                                  \
      xload_full<NT>(act + c * CHUNK_BYTES, cur.xoff, cur.m_end - cur.t0, x);             \
    else                                                                                  \
      xload_part<NT>(act + c * CHUNK_BYTES, cur.xoff, cvalid / FRAG_BYTES, cur.m_end - cur.t0, x); \
    __builtin_amdgcn_sched_barrier(0); /* token loads stay ahead of the weight loads */   \
    const bool last = c + 1 >= ce;                                                        \
    XSUB(0, WA, WB)                                                                       \
    XSUB(1, WB, WA)                                                                       \
    XSUB(2, WA, WB)                                                                       \
    XSUB(3, WB, WA)                                                                       \
    if (!last) {                                                                          \
      ++c;                                                                                \
    } else {                                                                              \
      if (cb == 0 && ce == a.nck) {                                                       \
        wstore<T, MODE, NT, SUB>(a, cur, acc, lrow, lq);                                  \
      } else if (have_nxt) {                                                              \
        HOLD_STORE                                                                        \
      } else {                                                                            \
        break;                                                                            \
      }                                                                                   \
      if (!have_nxt) break;                                                               \
      ++item;                                                                             \
      cur = nxt;                                                                          \
      cb = 0;                                                                             \
      c = 0;                                                                              \
      ce = static_cast<int>(min(static_cast<long long>(a.nck), q1 - static_cast<long long>(item) * a.nck)); \
      have_nxt = static_cast<long long>(item + 1) * a.nck < q1;                           \
      if (have_nxt)                                                                       \
        witem_setup<T, MODE, NT, SUB>(a, s_istart, s_off, item + 1, lrow, lq, row_bytes, nxt); \
    }                                                                                     \
  }

  f32x4_t hold[SUB][NT];
  WItem<NT> hold_it = cur;
  int hold_item = -1;
#define HOLD_STORE                                                                        \
  {                                                                                       \
    _Pragma("unroll") for (int s_ = 0; s_ < SUB; ++s_)                                    \
      _Pragma("unroll") for (int t_ = 0; t_ < NT; ++t_) {                                 \
        hold[s_][t_] = acc[s_][t_];                                                       \
        acc[s_][t_] = f32x4_t{0.f, 0.f, 0.f, 0.f};                                        \
      }                                                                                   \
    hold_it = cur;                                                                        \
    hold_item = item;                                                                     \
  }
  static_assert(SUB == 1 || SUB == 2 || SUB == 4, "tiles per item");
  if constexpr (SUB % 2 == 0) {
    while (true) CSTEP(w0, w1)
  } else {
    while (true) {
      CSTEP(w0, w1)
      CSTEP(w1, w0)
    }
  }
#undef CSTEP
#undef XSUB
#undef HOLD_STORE
  {
    // Both split items of the range at once: partials, one wait, both counts.
    const bool h_ = hold_item >= 0;
    const bool e_ = !(cb == 0 && ce == a.nck);
    if (h_) split_publish<T, MODE, NT, SUB>(a, hold, hold_item, w, W, Q);
    if (e_) split_publish<T, MODE, NT, SUB>(a, acc, item, w, W, Q);
    __builtin_amdgcn_s_waitcnt(0);  // the partials are performed (agent scope) before the counts
    int o1 = 0, o2 = 0;
    if (lane_id() == 0) {
      if (h_) o1 = atomicAdd(a.ctr + hold_item, 1);
      if (e_) o2 = atomicAdd(a.ctr + item, 1);
    }
    o1 = __shfl(o1, 0, WAVE);
    o2 = __shfl(o2, 0, WAVE);
    if (h_) split_reduce<T, MODE, NT, SUB>(a, hold_it, hold, hold_item, w, W, Q, lrow, lq, o1 == split_others(a, hold_item, Q, W));
    if (e_) split_reduce<T, MODE, NT, SUB>(a, cur, acc, item, w, W, Q, lrow, lq, o2 == split_others(a, item, Q, W));
  }
}

template <typename T, int MODE, int NT, int SUB, bool FULLK>
__global__ __launch_bounds__(XW_WAVES * WAVE) void expert_wave_kernel(XArgs a) {
  __shared__ int s_istart[MAX_GROUPS + 1];
  __shared__ int s_off[MAX_GROUPS + 1];
  __shared__ int s_ntx, s_maxm;
  __shared__ __attribute__((aligned(16))) char s_wt[XW_WAVES][16 * WT_ROW];

  const int wv = uni(threadIdx.x / WAVE);
  const int l = lane_id();
  const int lrow = l & 15;
  const int lq = l >> 4;

  item_prefix<NT>(a.offsets, a.n_groups, a.n_quads, a.tile_nt, a.tile_min, a.tile_m_min, s_istart, s_off, &s_ntx);
  if constexpr (NT <= 2) {
    if (threadIdx.x < WAVE) {
      // largest group: more than one pass of 16 * NT rows means tiles with later passes
      int m = 0;
      for (int g = l; g < a.n_groups; g += WAVE) m = max(m, a.offsets[g + 1] - a.offsets[g]);
#pragma unroll
      for (int d = 1; d < WAVE; d <<= 1) m = max(m, __shfl_xor(m, d, WAVE));
      if (l == 0) s_maxm = m;
    }
  }
  __syncthreads();  // the only barrier; waves are independent from here on
  const int nblk = static_cast<int>(gridDim.x);
  if constexpr (NT == 4) {
    if (uni(s_ntx) == 4)
      stream_body<T, MODE, 4, SUB, FULLK, false>(a, s_istart, s_off, s_wt[wv], wv, l, lrow, lq, nblk);
    else
      stream_body<T, MODE, 2, SUB, FULLK, false>(a, s_istart, s_off, s_wt[wv], wv, l, lrow, lq, nblk);
  } else {
    if (uni(s_maxm) > 16 * NT) {
      stream_body<T, MODE, NT, SUB, FULLK, true>(a, s_istart, s_off, s_wt[wv], wv, l, lrow, lq, nblk);
    } else {
      // Every group in one pass and a grid of two blocks per CU: only the
      // first half of the grid (the blocks dispatched first, one per CU)
      // streams, provided each of its waves still gets three chunk steps.
      // With both, the waves of the block dispatched second ended 7 us after
      // those of the first (TP share, B = 64: medians 35.9 and 29.1 us), and
      // one block per CU gave the shorter launch.  Launches with later
      // passes, or with fewer steps, keep both: there, one block per CU was
      // slower.
      const long long q = static_cast<long long>(uni(s_istart[a.n_groups])) * a.nck;
      const int half = (a.halve && q >= 3LL * (nblk / 2) * XW_WAVES) ? nblk / 2 : nblk;
      if (static_cast<int>(blockIdx.x) < half)
        stream_body<T, MODE, NT, SUB, FULLK, false>(a, s_istart, s_off, s_wt[wv], wv, l, lrow, lq, half);
    }
  }
}

// ---------------------------------------------------------------- host side

static int elem_bytes_x(int dtype) { return dtype == 1 ? 2 : 4; }

// Token tiles from the mean rows per group (exact for the full and TP views;
// an over-estimate, by the rank count, for an EP share): two above 12, and
// from 64 tokens on already from 8 rows (groups of 8-16 rows vary enough that
// many need a second 16-row pass, which then re-reads the weights: Qwen3-30B
// T = 128 down 86.5 -> 76.8 us, T = 192 step 294 -> 248 us, TP Zipf B = 160
// 125 -> 108 us; at 4 rows two tiles cost 5 us, and below 64 tokens an EP
// share's estimate of 8 means about one row, where two tiles cost 8 us); four
// for batches of 384..767 tokens with more than 24 (groups of 33..64 rows then
// take one pass instead of two, or the LDS-tiled kernel, which is
// latency-bound with few tiles).  Four tiles need one wave per SIMD and
// compute more per chunk, so they lose wherever groups hold 32 rows or fewer.
static int pick_nt(int T, int kk, int n_groups) {
  const double mean = static_cast<double>(T) * kk / n_groups;
  if (T <= 16) return 1;
  if (T >= 384 && T < 768 && mean > 24.0) return 4;
  return (mean > 12.0 || (T >= 64 && mean > 7.0)) ? 2 : 1;
}

int expert_tile_m_min(int T, int kk, int n_groups) {
  return pick_nt(T, kk, n_groups) == 4 ? TILE_M_MIN_WIDE : TILE_M_MIN;
}

struct XShape {
  int n_tiles, kfrag_total, nck;
};

static XShape x_shape(int mode, int H, int I, int dtype) {
  XShape s{};
  const int K = mode == XMODE_UP ? H : I;
  s.n_tiles = mode == XMODE_UP ? I / 8 : H / 16;
  s.kfrag_total = K * elem_bytes_x(dtype) / FRAG_BYTES;
  s.nck = (s.kfrag_total + CHUNK_FRAGS - 1) / CHUNK_FRAGS;
  return s;
}

// Weight tiles per item: four when the token side is reused enough to matter
// (two token tiles) or when a tile alone is too small to be a work item
// (under 16 KB); else one.
static int pick_sub(int nt, int kfrag_total) {
  const long long tile_bytes = 16LL * kfrag_total * FRAG_BYTES;
  return (nt >= 2 || tile_bytes < 16384) ? 4 : 1;
}

// Items of one launch at most: sum over groups of ceil(m_g / 16) passes
// <= pairs / 16 + touched groups (NT = 1 is the largest count), each of
// n_tiles / sub items.
static long long max_items(const XShape& s, int sub, int T, int kk, int n_groups) {
  const long long pairs = static_cast<long long>(T) * kk;
  const long long touched = n_groups < pairs ? n_groups : pairs;
  return (pairs / 16 + touched) * ((s.n_tiles + sub - 1) / sub);
}

static size_t round256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// One layout serves both halves (a caller may use a single buffer for the up
// and the down launch in turn): counters for the larger item count of the
// two, then the partial slots for the larger wave count.
struct XWorkspace {
  size_t ctr_bytes, part_bytes;
};

static XWorkspace x_workspace(int T, int kk, int n_groups, int H, int I, int dtype) {
  XWorkspace w{};
  long long items = 0, waves = 0;
  for (int mode = XMODE_UP; mode <= XMODE_DOWN; ++mode) {
    const XShape s = x_shape(mode, H, I, dtype);
    const long long it = max_items(s, 1, T, kk, n_groups);  // the most items any choice of tiles gives
    long long wv = (it * s.nck + MIN_CPW - 1) / MIN_CPW;
    if (wv > MAX_WAVES) wv = MAX_WAVES;
    if (it > items) items = it;
    if (wv > waves) waves = wv;
  }
  w.ctr_bytes = round256(static_cast<size_t>(items) * sizeof(int));
  w.part_bytes = static_cast<size_t>(waves) * 2 * SUB_MAX * NT_MAX * WAVE * 4 * sizeof(float);
  return w;
}

bool expert_items_fit(int T, int kk, int n_groups, int H, int I, int dtype) {
  for (int mode = XMODE_UP; mode <= XMODE_DOWN; ++mode)
    if (max_items(x_shape(mode, H, I, dtype), 1, T, kk, n_groups) > 0x7fffffffLL) return false;
  // Lane offsets are 32-bit: a group's W13 slice, the activations and `a`
  // must each stay below 2 GiB.
  const long long e = elem_bytes_x(dtype);
  if (2LL * I * H * e >= (1LL << 31)) return false;
  if (static_cast<long long>(T) * H * e >= (1LL << 31)) return false;
  if (static_cast<long long>(T) * kk * I * e >= (1LL << 31)) return false;
  return true;
}

// Layout: the wave-streaming kernel's counters and partials, then (256-byte
// aligned) the tile kernels' region.
static size_t stream_workspace_bytes(int T, int kk, int n_groups, int H, int I, int dtype) {
  const XWorkspace w = x_workspace(T, kk, n_groups, H, I, dtype);
  return round256(w.ctr_bytes + w.part_bytes);
}

size_t expert_workspace_bytes(int T, int kk, int n_groups, int H, int I, int dtype) {
  if (T <= 0) return 0;
  return stream_workspace_bytes(T, kk, n_groups, H, I, dtype) + expert_tile_workspace_bytes(T, kk, n_groups, H, I, dtype);
}

template <typename T, int MODE, int NT, int SUB, bool FULLK>
static int resident_blocks() {
  // The streaming rate drops with more than two blocks of four waves per CU
  // (more concurrent row streams); kernels with two token tiles fit one.
  static const int per_cu = std::min(
      2, kernel_blocks_per_cu(reinterpret_cast<const void*>(&expert_wave_kernel<T, MODE, NT, SUB, FULLK>),
                              XW_WAVES * WAVE));
  long long g = static_cast<long long>(device_cu_count()) * per_cu;
  if (g * XW_WAVES > MAX_WAVES) g = MAX_WAVES / XW_WAVES;
  return static_cast<int>(g);
}

template <typename T, int MODE, int NT, int SUB, bool FULLK>
static void launch_k(XArgs a, hipStream_t s) {
  const int grid = resident_blocks<T, MODE, NT, SUB, FULLK>();
  a.waves = grid * XW_WAVES;
  a.halve = (grid == 2 * device_cu_count() && grid % 16 == 0) ? 1 : 0;
  a.n_quads = (a.n_tiles + SUB - 1) / SUB;
  hipLaunchKernelGGL((expert_wave_kernel<T, MODE, NT, SUB, FULLK>), dim3(grid), dim3(XW_WAVES * WAVE), 0, s, a);
}

// K a whole number of 512-byte chunks: no partial chunk, no masking.
template <typename T, int MODE, int NT, int SUB>
static void launch_t(XArgs a, hipStream_t s) {
  if (a.kfrag_total % CHUNK_FRAGS == 0)
    launch_k<T, MODE, NT, SUB, true>(a, s);
  else
    launch_k<T, MODE, NT, SUB, false>(a, s);
}

template <typename T, int MODE>
static void launch_tm(XArgs a, int nt, int sub, hipStream_t s) {
  if (nt == 4) launch_t<T, MODE, 4, 4>(a, s);
  else if (nt == 2) launch_t<T, MODE, 2, 4>(a, s);
  else if (sub == 4) launch_t<T, MODE, 1, 4>(a, s);
  else launch_t<T, MODE, 1, 1>(a, s);
}

// Token tiles per pass of the short-row down kernel, from the mean rows per
// group: it holds a pass's token fragments in registers and takes every
// group, so passes of 64 and 128 rows serve the larger batches.  Groups of
// about 64 rows take one 128-row pass rather than one or two of 64 (TP
// B = 1024: 84.5 -> 64.8 us); at 32 rows both are alike.
static int short_nt(int T, int kk, int n_groups) {
  const double mean = static_cast<double>(T) * kk / n_groups;
  if (T <= 16 || mean <= 12.0) return 1;
  if (mean <= 24.0) return 2;
  return mean <= 40.0 ? 4 : 8;
}

// Whether the down-projection of these shapes runs entirely in the short-row
// kernel (then no LDS-tiled launch precedes it).
static bool down_short(int dtype, int H, int I) { return expert_short_down_ok(dtype, H, I); }

template <int MODE>
static void launch_mode(int dtype, XArgs a, int T, int kk, void* ws, hipStream_t s) {
  const bool short_rows = MODE == XMODE_DOWN && down_short(dtype, a.H, a.I_loc);
  a.tile_nt = (expert_tile_used(T, dtype) && !short_rows) ? expert_tile_nt(MODE == XMODE_UP, a.H, a.I_loc) : 0;
  a.tile_m_min = expert_tile_m_min(T, kk, a.n_groups);
  a.tile_min = expert_tile_min_tiles(a.tile_m_min);
  const XShape sh = x_shape(MODE, a.H, a.I_loc, dtype);
  a.n_tiles = sh.n_tiles;
  a.kfrag_total = sh.kfrag_total;
  a.nck = sh.nck;
  a.ctr = static_cast<int*>(ws);
  a.part = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                    x_workspace(T, kk, a.n_groups, a.H, a.I_loc, dtype).ctr_bytes);
  // The up-projection of decode-sized batches (bf16, groups of a few rows):
  // the block-cooperative kernel (expert_coop.hip), which balances the
  // chunks of an item over a block's waves at run time.
  if (MODE == XMODE_UP && dtype == 1 && a.tile_nt == 0 && T <= COOP_T_MAX) {
    a.sub = expert_coop_sub(sh.nck);
    if (a.sub > 0) {
      launch_expert_coop_up(a, s);
      return;
    }
  }
  // Short W2 rows (the TP view's I / P slices): whole tiles per step.
  if (short_rows) {
    launch_expert_down_short(a, short_nt(T, kk, a.n_groups), s);
    return;
  }
  const int nt = pick_nt(T, kk, a.n_groups);
  const int sub = pick_sub(nt, sh.kfrag_total);
  if (dtype == 1)
    launch_tm<uint16_t, MODE>(a, nt, sub, s);
  else
    launch_tm<float, MODE>(a, nt, sub, s);
}

void launch_expert_up(int dtype, const void* x, const int32_t* sorted_pair, const int32_t* offsets,
                      int n_groups, int T, int kk, const void* w13, int H, int I, void* A, void* ws,
                      hipStream_t s) {
  XArgs a{};
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
  // From TILE_ONLY_T tokens on the LDS-tiled kernels take every group and
  // the wave-streaming launch (which would find nothing) is not made.
  const bool tiles = expert_tile_used(T, dtype);
  const bool tiles_only = tiles && T >= TILE_ONLY_T;
  if (tiles)
    launch_expert_up_tiles(x, sorted_pair, offsets, n_groups, T, kk, w13, H, I, A,
                           tiles_only ? -1 : expert_tile_m_min(T, kk, n_groups),
                           static_cast<char*>(ws) + stream_workspace_bytes(T, kk, n_groups, H, I, dtype), s);
  if (!tiles_only) launch_mode<XMODE_UP>(dtype, a, T, kk, ws, s);
}

void launch_expert_down(int dtype, const void* A, const int32_t* offsets, int n_groups, int T,
                        int kk, const void* w2, int H, int I, void* y_pair, void* ws, hipStream_t s) {
  XArgs a{};
  a.act = A;
  a.offsets = offsets;
  a.w = w2;
  a.out = y_pair;
  a.n_groups = n_groups;
  a.kk = kk;
  a.K = I;
  a.I_loc = I;
  a.H = H;
  const bool tiles = expert_tile_used(T, dtype) && !down_short(dtype, H, I);
  const bool tiles_only = tiles && T >= TILE_ONLY_T;
  if (tiles)
    launch_expert_down_tiles(A, offsets, n_groups, T, kk, w2, H, I, y_pair,
                             tiles_only ? -1 : expert_tile_m_min(T, kk, n_groups),
                             static_cast<char*>(ws) + stream_workspace_bytes(T, kk, n_groups, H, I, dtype), s);
  if (!tiles_only) launch_mode<XMODE_DOWN>(dtype, a, T, kk, ws, s);
}

}  // namespace moe
