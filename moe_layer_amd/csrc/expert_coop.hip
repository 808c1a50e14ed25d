// Expert up-projection for decode-sized groups, one block of eight waves per
// compute unit (bf16 storage, fp32 accumulation; the arithmetic is that of
// expert_gemm.hip, which runs every other case):
//   up : a[r] = silu(W1_g x_t) * (W3_g x_t)   from W13_g (2I', H)
// (The kernel also has the down mode, y_pair[r] = W2_g a[r]; the wave-streaming
// kernel measured faster there, so it is not launched.)
// (Moebius review, §3.1: W13 (., 2I, H); decode MoE GEMMs are memory-bound,
// §2.1 and Fig. 3, so every weight byte must stream once.)
//
// Work item = (group, `sub` adjacent 16-row weight tiles, pass of 16 token
// rows) over the full K, as in expert_gemm.hip.  An item is cut into
// units of one tile x one 512-byte chunk of K (16 rows x 512 B = 8 KB of
// weights), at most CO_UNITS_MAX per item; units are numbered tile-major, so
// the waves working on an item at the same time read neighbouring bytes of the
// same rows.
//
// Balance.  Items are split into 8 contiguous ranges, one per XCD (blocks are
// dealt to the XCDs in turn), and each XCD's blocks take its items in turn,
// so they work on neighbouring groups whose token rows stay in that XCD's
// L2.  Inside a block, the waves take units one at a time from a counter in
// LDS, so a wave that streams more slowly simply takes fewer units.  Each
// unit's fp32 partial tile goes to an LDS slot of its own (indexed by the
// unit, not by the wave), and the wave that completes an item's last unit adds
// the slots in unit order and runs the epilogue.  The result therefore depends
// only on the shapes -- not on which wave did what -- and nothing is summed
// through global memory or handed between blocks.  A ring of item slots in LDS
// lets the next item start while the last units of the previous one finish.
// (Taking items from shared queues instead, so that whole XCDs could balance,
// measured slower: every claim is a device-scope atomic round trip.)
//
// Waits.  The only wait is for a ring slot: before writing its partial, a
// wave waits until the item that held the slot before has run its epilogue,
// which the wave holding that item's last unit is bound to do (units are
// handed out in order, so that chain only leads back to earlier items).  It
// is also bounded by a spin limit.  Item decoding (group, rows, token rows) is
// published in LDS by the wave that starts the item two places earlier; a wave
// that finds no current entry decodes the item itself.
//
// Loads.  Weights: 256 contiguous bytes of each of 4 rows per load
// instruction, non-temporal, double-buffered in registers (the next unit's
// chunk is in flight while the current one is multiplied), passed through the
// wave's private LDS tile into the MFMA operand layout.  Token fragments come
// from L2; the next unit's are issued right after the current unit's MFMAs (and
// skipped when they are the same).
#include "common.hpp"
#include "moe_internal.h"
#include "stream_ops.hpp"

namespace moe {

namespace {

constexpr int CO_WAVES = 8;
constexpr int CO_THREADS = CO_WAVES * WAVE;
constexpr int CO_NT = 1;                      // token tiles per pass (passes of 16 rows)
constexpr int CO_UNITS_MAX = 16;              // units per item at most
constexpr int CO_PART_VECS = 4096;            // LDS partial ring: 4096 x 16 B = 64 KB
constexpr int CO_RING_MAX = 4;                // item slots in the ring at most
constexpr int CO_LOOK = 2;                    // items decoded ahead of the one being started
constexpr int CO_INFO = 8;                    // decoded items kept in LDS (a ring)
constexpr int CO_XCD = 8;
constexpr int ITEM_END = -1;
constexpr int SPIN_LIMIT = 1 << 22;

__device__ __forceinline__ int lds_load(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ int lds_add(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// Wait for this wave's LDS operations only, so outstanding global loads stay
// in flight; also a compiler barrier, so no memory access moves across it.
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Bounds of XCD x's item range [lo, hi).
__device__ __forceinline__ void xcd_range(int x, int n_items, int* lo, int* hi) {
  *lo = static_cast<int>(static_cast<long long>(n_items) * x / CO_XCD);
  *hi = static_cast<int>(static_cast<long long>(n_items) * (x + 1) / CO_XCD);
}
// One 16x16 output tile of an item (tile s, token tile tt): acc[r] = D[4*lq + r][lrow].
template <typename T, int MODE>
__device__ __forceinline__ void co_store(const XArgs& a, const WItem<CO_NT>& it, int s, int tt, f32x4_t acc,
                                         int lrow, int lq) {
  const int tr = it.t0 + tt * 16 + lrow;
  if (MODE == XMODE_UP) {
    float up[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) up[r] = __shfl_xor(acc[r], 32, WAVE);
    const int n = it.n0 + 8 * s + 4 * lq;
    if (lq < 2 && tr < it.m_end) {
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float gt = acc[r];
        o[r] = gt / (1.0f + __expf(-gt)) * up[r];
      }
      T* dst = reinterpret_cast<T*>(a.out) + static_cast<size_t>(it.row0 + tr) * a.I_loc + n;
      Elem<T>::store4(dst, o[0], o[1], o[2], o[3]);
    }
  } else {
    const int n = it.n0 + 16 * s + 4 * lq;
    if (tr < it.m_end) {
      T* dst = reinterpret_cast<T*>(a.out) + static_cast<size_t>(it.row0 + tr) * a.H + n;
      Elem<T>::store4(dst, acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

// An item decoded once: its group's first sorted row, the pass's rows
// [t0, m_end), the first weight row n0 of its tiles, the tiles inside the
// matrix, and the weight row its first tile starts at.  Wave-uniform.
struct CoItem {
  int tag, row0, m_end, t0, n0, n_sub, first_row;
  int pad;   // 1 when the item's tile has later passes (the weights are kept in L2)
};

template <int MODE>
__device__ __forceinline__ CoItem co_decode(const XArgs& a, const int* s_istart, const int* s_off, int item) {
  int lo = 0, hi = a.n_groups;  // s_istart[lo] <= item < s_istart[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (uni(s_istart[mid]) <= item) lo = mid;
    else hi = mid;
  }
  CoItem d;
  d.tag = item;
  d.row0 = uni(s_off[lo]);
  const int m = uni(s_off[lo + 1]) - d.row0;
  const int ps = pass_rows<CO_NT>(m);
  const int np = (m + ps - 1) / ps;
  d.pad = np > 1 ? 1 : 0;   // the tile has later passes
  const int local = item - uni(s_istart[lo]);
  const int nq = local / np;
  d.t0 = (local - nq * np) * ps;
  d.m_end = min(m, d.t0 + ps);
  d.n_sub = min(a.sub, a.n_tiles - nq * a.sub);
  if (MODE == XMODE_UP) {
    d.n0 = nq * a.sub * 8;
    d.first_row = lo * (2 * a.I_loc) + d.n0;
  } else {
    d.n0 = nq * a.sub * 16;
    d.first_row = lo * a.H + d.n0;
  }
  return d;
}

// Activation row of token row i (0 .. 16 * CO_NT - 1) of the item's pass
// (rows past the pass repeat its last row).
template <int MODE>
__device__ __forceinline__ int co_token_row(const XArgs& a, const CoItem& d, int i) {
  const int r = d.row0 + min(d.t0 + i, d.m_end - 1);
  return MODE == XMODE_UP ? a.sorted_pair[r] / a.kk : r;
}

}  // namespace

// LDS of one block, declared by the kernel and shared by both bodies.
struct CoShared {
  int* s_istart;
  int* s_off;
  int* s_next;
  int* s_maxm;
  int* s_done;
  int* s_fin;
  CoItem* s_info;
  int (*s_tok)[16 * CO_NT];
  char (*s_wt)[16 * WT_ROW];
  f32x4_t* s_part;
};

// KEEP: items whose tile has later passes read their weights with the
// ordinary (temporal) policy so that those passes, adjacent items on the same
// XCD, find them in L2; everything else streams them non-temporally.  A
// launch with no group above 16 rows has one pass per tile and runs the body
// without that choice.
template <typename T, int MODE, bool FULLK, bool KEEP>
__device__ __forceinline__ void coop_body(const XArgs& a, const CoShared& sh) {
  int* s_istart = sh.s_istart;
  int* s_off = sh.s_off;
  int& s_next = *sh.s_next;
  int* s_done = sh.s_done;
  int* s_fin = sh.s_fin;
  CoItem* s_info = sh.s_info;
  int (*s_tok)[16 * CO_NT] = sh.s_tok;
  char (*s_wt)[16 * WT_ROW] = sh.s_wt;
  f32x4_t* s_part = sh.s_part;
  const int wv = uni(threadIdx.x / WAVE);
  const int l = lane_id();
  const int lrow = l & 15;
  const int lq = l >> 4;
  const int nb = gridDim.x / CO_XCD;    // blocks per XCD (the grid is a multiple of 8)
  const int xcd = blockIdx.x % CO_XCD;
  const int jb = blockIdx.x / CO_XCD;
  const int n_items = s_istart[a.n_groups];
  const uint32_t row_bytes = static_cast<uint32_t>(a.K) * sizeof(T);
  const char* act = reinterpret_cast<const char*>(a.act);
  const int kbytes = a.kfrag_total * FRAG_BYTES;
  char* tile = s_wt[wv];
  const int ntx = CO_NT;                      // token tiles a partial slot holds
  const int U = a.nck * a.sub;                // units per item
  const int slot_vecs = U * ntx * WAVE;
  const int R = max(1, min(CO_RING_MAX, CO_PART_VECS / slot_vecs));
  const uint32_t sub_bytes = (MODE == XMODE_UP ? 8u : 16u) * row_bytes;
  uint32_t woff[4];  // lane: row 4j + lq of a tile, + 16 * lrow, from the tile's first row
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * j + lq;
    const int rel = (MODE == XMODE_UP) ? (i < 8 ? i : a.I_loc + i - 8) : i;
    woff[j] = static_cast<uint32_t>(rel) * row_bytes + 16 * lrow;
  }

  // Publish item k's decoded form (every lane of one wave calls this).
  auto publish = [&](int k, int item) {
    const CoItem d = co_decode<MODE>(a, s_istart, s_off, item);
    const int slot = k % CO_INFO;
    if (l == 0) lds_store(&s_info[slot].tag, -1);
    wait_lds();
    const int tok = l < 16 * CO_NT ? co_token_row<MODE>(a, d, l) : 0;
    if (l < 16 * CO_NT) s_tok[slot][l] = tok;
    if (l == 0) {
      CoItem e = d;
      e.tag = -1;
      s_info[slot] = e;
    }
    wait_lds();
    if (l == 0) lds_store(&s_info[slot].tag, k);
    wait_lds();
  };
  // An item's weight and token addressing for this lane, from the published
  // form when it is still there, else decoded here.
  auto load_item = [&](int k, int item, WItem<CO_NT>& it) {
    const int slot = k % CO_INFO;
    CoItem d = s_info[slot];
    int tok[CO_NT];
#pragma unroll
    for (int tt = 0; tt < CO_NT; ++tt) tok[tt] = s_tok[slot][tt * 16 + lrow];
    wait_lds();
    const int tag2 = lds_load(&s_info[slot].tag);
    if (uni(d.tag) != k || uni(tag2) != k) {
      d = co_decode<MODE>(a, s_istart, s_off, item);
#pragma unroll
      for (int tt = 0; tt < CO_NT; ++tt) tok[tt] = co_token_row<MODE>(a, d, tt * 16 + lrow);
    }
    it.row0 = uni(d.row0);
    it.m_end = uni(d.m_end);
    it.t0 = uni(d.t0);
    it.n0 = uni(d.n0);
    it.n_sub = uni(d.n_sub);
    it.sub_bytes = sub_bytes;
    it.keep = uni(d.pad);
    it.wbase = reinterpret_cast<const char*>(a.w) + static_cast<size_t>(uni(d.first_row)) * row_bytes;
#pragma unroll
    for (int j = 0; j < 4; ++j) it.woff[j] = woff[j];
#pragma unroll
    for (int tt = 0; tt < CO_NT; ++tt) it.xoff[tt] = static_cast<uint32_t>(tok[tt]) * row_bytes + 16 * lq;
  };

  // The block's items: its share of its XCD's range, in turn (local item k
  // is x_lo + jb + k * nb); n_own of them.
  int x_lo, x_hi;
  xcd_range(xcd, n_items, &x_lo, &x_hi);
  const int n_own = x_lo + jb < x_hi ? (x_hi - x_lo - jb + nb - 1) / nb : 0;
  auto item_of = [&](int k) -> int { return k < n_own ? x_lo + jb + k * nb : ITEM_END; };

  if (wv < CO_LOOK && wv < n_own) publish(wv, item_of(wv));  // the first items' decoded form
  if (threadIdx.x < CO_RING_MAX) s_fin[threadIdx.x] = static_cast<int>(threadIdx.x) - R;
  __syncthreads();

  auto next_unit = [&]() -> int {
    int v = 0;
    if (l == 0) v = lds_add(&s_next, 1);
    return uni(__shfl(v, 0, WAVE));
  };

  WItem<CO_NT> cur, nxt;
  int k = 0, u = 0, item = ITEM_END;
  {
    const int v = next_unit();
    k = v / U;
    u = v - k * U;
    item = item_of(k);
  }
  uint4 w0[CHUNK_FRAGS], w1[CHUNK_FRAGS], x[CO_NT][CHUNK_FRAGS];
  if (item != ITEM_END) {
    load_item(k, item, cur);
    const int s = u / a.nck, c = u - (u / a.nck) * a.nck;
    if constexpr (FULLK && KEEP) wload_full_keep(tile_chunk(cur, s, c), cur.woff, w0, cur.keep);
    else if constexpr (FULLK) wload_full(tile_chunk(cur, s, c), cur.woff, w0);
    else wload(tile_chunk(cur, s, c), cur.woff, kbytes - c * CHUNK_BYTES, lrow, w0);
    if constexpr (FULLK)
      xload_full<CO_NT>(act + c * CHUNK_BYTES, cur.xoff, cur.m_end - cur.t0, x);
    else
      xload_part<CO_NT>(act + c * CHUNK_BYTES, cur.xoff, (kbytes - c * CHUNK_BYTES) / FRAG_BYTES,
                        cur.m_end - cur.t0, x);
    if (u == 0 && k + CO_LOOK < n_own) publish(k + CO_LOOK, item_of(k + CO_LOOK));
  }

  // One unit: (k, u) of item `item` with its weights in WC; the next unit's
  // weights go to WN.
#define CO_STEP(WC, WN)                                                                         \
  {                                                                                             \
    const int s = u / a.nck;                                                                    \
    const int c = u - s * a.nck;                                                                \
    const int cvalid = kbytes - c * CHUNK_BYTES;                                                \
    const int nrows = cur.m_end - cur.t0;                                                       \
    const int v2 = next_unit();                                                                 \
    const int k2 = v2 / U;                                                                      \
    const int u2 = v2 - k2 * U;                                                                 \
    const int item2 = item_of(k2);                                                              \
    const bool more = item2 != ITEM_END;                                                        \
    if (more) {                                                                                 \
      if (k2 != k) load_item(k2, item2, nxt);                                                   \
      else nxt = cur;                                                                           \
      const int s2 = u2 / a.nck;                                                                \
      const int c2 = u2 - s2 * a.nck;                                                           \
      if constexpr (FULLK && KEEP)                                                              \
        wload_full_keep(tile_chunk(nxt, s2, c2), nxt.woff, WN, nxt.keep);                       \
      else if constexpr (FULLK)                                                                 \
        wload_full(tile_chunk(nxt, s2, c2), nxt.woff, WN);                                      \
      else                                                                                      \
        wload(tile_chunk(nxt, s2, c2), nxt.woff, kbytes - c2 * CHUNK_BYTES, lrow, WN);          \
    }                                                                                           \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    f32x4_t acc[CO_NT];                                                                         \
    _Pragma("unroll") for (int tt = 0; tt < CO_NT; ++tt) acc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f}; \
    {                                                                                           \
      uint4 wt[CHUNK_FRAGS];                                                                    \
      wtranspose(WC, tile, lrow, lq, wt);                                                       \
      if (FULLK || cvalid >= CHUNK_BYTES)                                                       \
        wmma_full<T, CO_NT>(wt, x, nrows, acc);                                                 \
      else                                                                                      \
        wmma_part<T, CO_NT>(wt, x, cvalid / FRAG_BYTES, nrows, acc);                            \
    }                                                                                           \
    /* the next unit's token fragments, unless they are the ones just used */                   \
    if (more) {                                                                                 \
      const int s2 = u2 / a.nck;                                                                \
      const int c2 = u2 - s2 * a.nck;                                                           \
      if (k2 != k || c2 != c) {                                                                 \
        if constexpr (FULLK)                                                                    \
          xload_full<CO_NT>(act + c2 * CHUNK_BYTES, nxt.xoff, nxt.m_end - nxt.t0, x);           \
        else                                                                                    \
          xload_part<CO_NT>(act + c2 * CHUNK_BYTES, nxt.xoff, (kbytes - c2 * CHUNK_BYTES) / FRAG_BYTES, \
                            nxt.m_end - nxt.t0, x);                                             \
      }                                                                                         \
    }                                                                                           \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    /* the item's ring slot must have been released by its previous holder */                   \
    const int r = k % R;                                                                        \
    for (int spin = 0; spin < SPIN_LIMIT && lds_load(&s_fin[r]) != k - R; ++spin)               \
      __builtin_amdgcn_s_sleep(2);                                                              \
    f32x4_t* slot = s_part + static_cast<size_t>(r) * slot_vecs;                                \
    _Pragma("unroll") for (int tt = 0; tt < CO_NT; ++tt)                                        \
      if (tt < ntx) slot[(u * ntx + tt) * WAVE + l] = acc[tt];                                  \
    wait_lds(); /* the partial is in LDS before the count says so */                            \
    int d = 0;                                                                                  \
    if (l == 0) d = lds_add(&s_done[r], 1);                                                     \
    d = uni(__shfl(d, 0, WAVE));                                                                \
    if (d == U - 1) {                                                                           \
      /* last unit of the item: add the slots in unit order, then the epilogue */               \
      for (int s3 = 0; s3 < cur.n_sub; ++s3) {                                                  \
        _Pragma("unroll") for (int tt = 0; tt < CO_NT; ++tt) {                                  \
          if (tt < ntx && 16 * tt < nrows) {                                                    \
            f32x4_t sum = slot[((s3 * a.nck) * ntx + tt) * WAVE + l];                           \
            for (int c3 = 1; c3 < a.nck; ++c3) sum += slot[((s3 * a.nck + c3) * ntx + tt) * WAVE + l]; \
            co_store<T, MODE>(a, cur, s3, tt, sum, lrow, lq);                                   \
          }                                                                                     \
        }                                                                                       \
      }                                                                                         \
      wait_lds(); /* the slots have been read before the ring slot is released */               \
      if (l == 0) {                                                                             \
        lds_store(&s_done[r], 0);                                                               \
        wait_lds();                                                                             \
        lds_store(&s_fin[r], k);                                                                \
      }                                                                                         \
    }                                                                                           \
    if (!more) break;                                                                           \
    if (u2 == 0 && k2 + CO_LOOK < n_own) publish(k2 + CO_LOOK, item_of(k2 + CO_LOOK));          \
    cur = nxt;                                                                                  \
    k = k2;                                                                                     \
    u = u2;                                                                                     \
    item = item2;                                                                               \
  }

  if (item != ITEM_END) {
    while (true) {
      CO_STEP(w0, w1)
      CO_STEP(w1, w0)
    }
  }
#undef CO_STEP
}

template <typename T, int MODE, bool FULLK>
__global__ __launch_bounds__(CO_THREADS) void expert_coop_kernel(XArgs a) {
  __shared__ int s_istart[MAX_GROUPS + 1];
  __shared__ int s_off[MAX_GROUPS + 1];
  __shared__ int s_ntx;
  __shared__ int s_next, s_maxm;
  __shared__ int s_done[CO_RING_MAX], s_fin[CO_RING_MAX];
  __shared__ __attribute__((aligned(16))) CoItem s_info[CO_INFO];
  __shared__ int s_tok[CO_INFO][16 * CO_NT];
  __shared__ __attribute__((aligned(16))) char s_wt[CO_WAVES][16 * WT_ROW];
  __shared__ f32x4_t s_part[CO_PART_VECS];
  const int l = lane_id();

  item_prefix<CO_NT>(a.offsets, a.n_groups, a.n_quads, a.tile_nt, a.tile_min, a.tile_m_min, s_istart, s_off,
                     &s_ntx);
  if (threadIdx.x < WAVE) {
    // largest group held here: more than 16 rows means tiles with later passes
    int m = 0;
    for (int g = l; g < a.n_groups; g += WAVE) m = max(m, a.offsets[g + 1] - a.offsets[g]);
#pragma unroll
    for (int d = 1; d < WAVE; d <<= 1) m = max(m, __shfl_xor(m, d, WAVE));
    if (l == 0) s_maxm = m;
  }
  if (threadIdx.x == 0) {
    s_next = 0;
    for (int r = 0; r < CO_RING_MAX; ++r) s_done[r] = 0;
  }
  if (threadIdx.x < CO_INFO) s_info[threadIdx.x].tag = -1;
  __syncthreads();
  const CoShared sh{s_istart, s_off, &s_next, &s_maxm, s_done, s_fin, s_info, s_tok, s_wt, s_part};
  if (uni(s_maxm) > 16)
    coop_body<T, MODE, FULLK, true>(a, sh);
  else
    coop_body<T, MODE, FULLK, false>(a, sh);
}

// ---------------------------------------------------------------- host side

namespace {

template <typename T, int MODE, bool FULLK>
void launch_co(const XArgs& a, hipStream_t s) {
  const int grid = (device_cu_count() + CO_XCD - 1) / CO_XCD * CO_XCD;
  hipLaunchKernelGGL((expert_coop_kernel<T, MODE, FULLK>), dim3(grid), dim3(CO_THREADS), 0, s, a);
}

}  // namespace

int expert_coop_sub(int nck) {
  if (nck < 1 || nck > CO_UNITS_MAX) return 0;
  return CO_UNITS_MAX / nck;
}

void launch_expert_coop_up(XArgs a, hipStream_t s) {
  a.n_quads = (a.n_tiles + a.sub - 1) / a.sub;
  if (a.kfrag_total % CHUNK_FRAGS == 0) launch_co<uint16_t, XMODE_UP, true>(a, s);
  else launch_co<uint16_t, XMODE_UP, false>(a, s);
}

}  // namespace moe
