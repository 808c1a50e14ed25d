// Routing in one launch: gate GEMM, softmax + top-k, and (optionally) the
// stable permutation of pairs by expert (Sem-MoE notes, Key design 1: the
// gate is top-k(softmax(W_g h + b_g)); Key design 4: the argsort of tokens by
// expert).
//
// Phase A -- gate GEMM.  logits[t, e] = sum_h x[t, h] W_g[e, h] + b[e] is cut
//   into units of 16 experts x 16 tokens x one K-slice; each wave computes a
//   unit with 16x16 MFMA tiles (lane l: expert/token row l%16, bytes
//   16*(l/16) of each 64-byte K fragment).  Both operands reach that layout
//   through the wave's own LDS tile: each load instruction takes 256
//   contiguous bytes of each of 4 rows (whole cache lines), and the tile,
//   XOR-swizzled by row, hands every lane its row's fragment without bank
//   conflicts.  (Loading the MFMA layout straight from memory, 64 bytes of
//   each of 16 rows per instruction, ran phase A two times slower.)  K is
//   split into KS slices (a power of two; trailing slices may be empty) so
//   that small batches still spread the gate matrix over many CUs.  With KS >= 8 a block's eight
//   waves take eight consecutive slices of one tile and the block sums them
//   in LDS (wave order), so only KS / 8 partial tiles go through memory;
//   with fewer slices each wave writes its own.  All blocks of one 16-token
//   tile share a counter.
// Phase B -- the block that completes a token tile's counter (the last one to
//   arrive; integer atomics, nobody waits) sums the KS partials of each of
//   the tile's logits in slice order, adds the bias and writes the logits
//   (to HBM and to LDS), then runs the top-k of each token, 32 lanes per
//   token: lane l holds experts l, l+32, ...; each of the k rounds reduces
//   the largest logit key over the lanes, then the lowest expert id holding
//   it -- "larger value first, then lower id", a total order, so every lane
//   sees the same winner and equal logits (-0.0 vs +0.0 included) go to the
//   lower id.
//   Selection is on the fp32 logits (the same set as on the softmax).
//   Weights: softmax over all E routed experts at the picks, optionally
//   renormalised over the k picks; shared experts E, E+1, ... follow with
//   weight 1.  All butterfly sums are commutative at every level, so every
//   lane holds the same bits.
// Phase C -- the block that completes the last token tile (second counter)
//   runs the stable counting sort of all T*kk pairs (sort.hpp).  A batch of
//   one token tile (T <= 16) needs no second counter: its phase-B block
//   writes the pair keys to LDS as it picks them and sorts from there.
// Counters live in the caller's workspace; each finishing block resets the
// counter it completed, so the workspace is zero again after every call.
// Everything one block hands to another (partial tiles, logits of the
// un-split case, top-k ids) is written and read with agent-scope relaxed
// accesses, which stay coherent across the XCDs' L2 caches; a fence would
// instead write back and invalidate the whole L2 of every arriving block.
#include <math.h>

#include <mutex>

#include "common.hpp"
#include "moe_internal.h"
#include "sort.hpp"

namespace moe {

constexpr int RT_WAVES = 8;
constexpr int RT_THREADS = RT_WAVES * WAVE;
constexpr int RT_CHUNK = 4;                // K fragments per inner step (256 bytes of each row)
constexpr int RT_TILE = 16 * RT_CHUNK * FRAG_BYTES;  // one operand's 16 rows of a step in LDS (4 KB)
constexpr int RT_MAX_KS = 16;              // K slices at most (a power of two)
constexpr int RT_KEY_CAP = 16 * MAX_E * 2; // 16-bit sort keys that fit the logit tile's LDS
constexpr int RT_UNROLL = 4;               // logits each thread reduces per pass of phase B
constexpr int N_XCD = 8;

struct RouteArgs {
  const void* x;
  const void* wg;
  const float* bias;       // nullable
  float* logits;           // (T, E)
  int32_t* ids;            // (T, kk)
  float* w;                // (T, kk)
  float* partial;          // (KS, T, E) when KS > 1
  int* ctr;                // n_tt + 1 counters
  // permutation outputs (null: routing only)
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_pair;
  int32_t* pair_pos;
  int g_begin, n_groups;
  int T, H, E, k, renorm, n_shared;
  int kfrag_total;         // H * elem / 64
  int kf;                  // fragments per slice
  int n_et;                // 16-expert tiles
  int n_tt;                // 16-token tiles
  int bpt;                 // blocks per token tile
};

// Phase-A staging.  A step covers 4 fragments (256 bytes, 16 chunks of 16
// bytes) of 16 rows.  Load instruction i, lane (lrow = l % 16, lq = l / 16):
// row 4i + lq, chunk lrow ^ (8 if lq >= 2), so each instruction reads 256
// contiguous bytes of 4 rows.  In LDS, chunk c of row r sits at slot
// c ^ swz(r) of the row's 256 bytes, swz(r) = bit 0 of r, plus bits 1-2 of r
// moved to bits 2-3.  Lanes 8k..8k+7 and 32+8k..32+8k+7 share an LDS cycle;
// with this map they touch 16 distinct 16-byte slots both when the rows are
// written and when lane (lrow, lq) reads chunk 4f + lq of row lrow (the
// operand of fragment f).
__device__ __forceinline__ int stage_swz(int r) { return (r & 1) | ((r & 6) << 1); }
__device__ __forceinline__ int stage_chunk(int lrow, int lq) { return lrow ^ ((lq & 2) << 2); }
__device__ __forceinline__ void stage_transpose(const uint4 (&v)[RT_CHUNK], char* tile, int lrow, int lq,
                                                uint4 (&t)[RT_CHUNK]) {
  const int c = stage_chunk(lrow, lq);
#pragma unroll
  for (int i = 0; i < RT_CHUNK; ++i) {
    const int r = 4 * i + lq;
    *reinterpret_cast<uint4*>(tile + r * 256 + 16 * (c ^ stage_swz(r))) = v[i];
  }
  const int sw = stage_swz(lrow);
#pragma unroll
  for (int f = 0; f < RT_CHUNK; ++f)
    t[f] = *reinterpret_cast<const uint4*>(tile + lrow * 256 + 16 * ((4 * f + lq) ^ sw));
}

// Top-k of one token by a group of 32 lanes (2 tokens per wave, 16 per block):
// lane r of the group holds experts r, r+32, r+64, ... as 32-bit keys, the
// order-preserving image of the fp32 logit (-0.0 and +0.0 map to one key; 0
// marks an empty or taken slot, so real keys are at least 1).  Each of the k
// rounds takes the lane maxima and reduces them over the group (DPP quad xor
// 1, quad xor 2, half-row mirror, row mirror, then the two 16-lane rows
// combined with v_permlane16_swap: every lane ends with the same value);
// among the experts holding that key the lowest id wins (a second, min
// reduction of ids), so equal logits go to the lower expert id.  Selection is
// on the fp32 logits, the same set as on the softmax.
constexpr int TK_LANES = 32;
constexpr int TK_MAXV = MAX_E / TK_LANES;

__device__ __forceinline__ uint32_t logit_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;  // -0.0 ties with +0.0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return u > 1u ? u : 1u;        // only a negative NaN maps below 1
}
__device__ __forceinline__ float key_logit(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(static_cast<int>(v), CTRL, 0xf, 0xf, false));
}
// The values of lanes i & ~16 and i | 16 (the two 16-lane rows of lane i's
// 32-lane half), in that order in every lane: v_permlane16_swap of a
// register with itself.
struct RowPair {
  uint32_t lo, hi;
};
__device__ __forceinline__ RowPair row_pair(uint32_t v) {
  const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return RowPair{p[0], p[1]};
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <-> 7 - i within 8
constexpr int DPP_MIRROR = 0x140;      // lane i <-> 15 - i within 16

__device__ __forceinline__ uint32_t group32_max(uint32_t v) {
  v = max(v, dpp32<DPP_XOR1>(v));
  v = max(v, dpp32<DPP_XOR2>(v));
  v = max(v, dpp32<DPP_HALF_MIRROR>(v));
  v = max(v, dpp32<DPP_MIRROR>(v));
  const RowPair p = row_pair(v);
  return max(p.lo, p.hi);
}
__device__ __forceinline__ uint32_t group32_min(uint32_t v) {
  v = min(v, dpp32<DPP_XOR1>(v));
  v = min(v, dpp32<DPP_XOR2>(v));
  v = min(v, dpp32<DPP_HALF_MIRROR>(v));
  v = min(v, dpp32<DPP_MIRROR>(v));
  const RowPair p = row_pair(v);
  return min(p.lo, p.hi);
}
// Every lane of the group gets the same bits: each DPP level adds two equal
// partial sums in either order (fp32 addition is commutative), and the last
// adds the two rows' sums in the same order in every lane.
__device__ __forceinline__ float group32_sum(float v) {
  v += __uint_as_float(dpp32<DPP_XOR1>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<DPP_XOR2>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<DPP_HALF_MIRROR>(__float_as_uint(v)));
  v += __uint_as_float(dpp32<DPP_MIRROR>(__float_as_uint(v)));
  const RowPair p = row_pair(__float_as_uint(v));
  return __uint_as_float(p.lo) + __uint_as_float(p.hi);
}

// lg: the token's E logits (LDS), E <= 32 * V.  All 32 lanes of the group
// call this.  Weights: softmax over all E routed experts at the picks,
// optionally renormalised over the k picks (the sum over all E then cancels
// and is not formed); shared experts E, E+1, ... follow with weight 1.  pk
// (LDS, nullable): the sort keys of the token's k + n_shared pairs (expert -
// g_begin when in [0, n_groups), else n_groups).
__device__ __forceinline__ uint16_t local_key(int id, int g_begin, int n_groups) {
  const int g = id - g_begin;
  return static_cast<uint16_t>((g >= 0 && g < n_groups) ? g : n_groups);
}
template <int V>
__device__ __forceinline__ void group_topk(const float* lg, int E, int k, int renorm, int n_shared,
                                           int32_t* ids, float* w, uint16_t* pk, int g_begin,
                                           int n_groups) {
  const int r = lane_id() & (TK_LANES - 1);
  uint32_t key[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int e = r + TK_LANES * j;
    key[j] = e < E ? logit_key(lg[e]) : 0u;
  }
  uint32_t pick = 0, top = 0;   // this lane's pick: round r; the first round's key
  int pick_id = 0;
  for (int round = 0; round < k; ++round) {
    uint32_t m = key[0];
#pragma unroll
    for (int j = 1; j < V; ++j) m = max(m, key[j]);
    const uint32_t best = group32_max(m);
    uint32_t cand = 0xffffffffu;  // this lane's lowest expert holding `best`
#pragma unroll
    for (int j = V - 1; j >= 0; --j) cand = key[j] == best ? static_cast<uint32_t>(r + TK_LANES * j) : cand;
    const uint32_t win = group32_min(cand);
#pragma unroll
    for (int j = 0; j < V; ++j) key[j] = static_cast<uint32_t>(r + TK_LANES * j) == win ? 0u : key[j];
    if (round == 0) top = best;
    if (r == round) {
      pick = best;
      pick_id = static_cast<int>(win);
    }
  }
  const float mx = key_logit(top);  // the largest logit
  const float p = (r < k) ? expf(key_logit(pick) - mx) : 0.f;
  float denom;
  if (renorm) {
    denom = group32_sum(p);
  } else {
    float s_all = 0.f;
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int e = r + TK_LANES * j;
      if (e < E) s_all += expf(lg[e] - mx);
    }
    denom = group32_sum(s_all);
  }
  if (r < k) {
    st_agent(ids + r, pick_id);
    w[r] = p / denom;
    if (pk) pk[r] = local_key(pick_id, g_begin, n_groups);
  }
  for (int sh = r; sh < n_shared; sh += TK_LANES) {
    st_agent(ids + k + sh, E + sh);
    w[k + sh] = 1.0f;
    if (pk) pk[k + sh] = local_key(E + sh, g_begin, n_groups);
  }
}

template <typename T, int KS>
__global__ __launch_bounds__(RT_THREADS) void route_kernel(RouteArgs a) {
  // Phase A's per-wave staging tiles share LDS with everything used after it.
  constexpr int LG_BYTES = 16 * MAX_E * 4;
  constexpr int CNT_BYTES = RT_WAVES * MAX_GROUPS * 4;
  constexpr int OFF_BYTES = MAX_GROUPS * 4;
  constexpr int PK_BYTES = 16 * MAX_KK * 2;
  constexpr int LATE_BYTES = LG_BYTES + CNT_BYTES + OFF_BYTES + PK_BYTES;
  constexpr int STAGE_BYTES = RT_WAVES * 2 * RT_TILE;
  __shared__ __align__(16) char s_raw[STAGE_BYTES > LATE_BYTES ? STAGE_BYTES : LATE_BYTES];
  __shared__ int s_last;              // hand-off flag
  // wave partials; the tile's logits; later the sort's 16-bit keys
  float* s_lg = reinterpret_cast<float*>(s_raw);
  int* s_cnt = reinterpret_cast<int*>(s_raw + LG_BYTES);
  int* s_off = reinterpret_cast<int*>(s_raw + LG_BYTES + CNT_BYTES);
  uint16_t* s_pk = reinterpret_cast<uint16_t*>(s_raw + LG_BYTES + CNT_BYTES + OFF_BYTES);  // keys of a single-tile batch

  // XCD-aware order: hardware deals blocks to the 8 XCDs round-robin, so
  // logical block b runs on XCD b / (grid / 8) and the blocks of one token
  // tile share an L2 (its activation rows are fetched from HBM once).
  const int per_xcd = gridDim.x / N_XCD;
  const int lb = (blockIdx.x % N_XCD) * per_xcd + blockIdx.x / N_XCD;
  if (lb >= a.n_tt * a.bpt) return;  // padding to a multiple of 8 blocks

  const int tid = threadIdx.x;
  const int wv = tid / WAVE;
  const int l = lane_id();
  const int lrow = l & 15;
  const int lq = l >> 4;
  const int tt = lb / a.bpt;
  const int unit = (lb % a.bpt) * RT_WAVES + wv;
  const size_t row_bytes = static_cast<size_t>(a.H) * sizeof(T);

  // ---------------- phase A: one 16x16 partial tile per wave.  With KS >= 8
  // the block's waves take 8 consecutive K slices of one expert tile and the
  // block sums them (wave order) in LDS: KS / 8 partial slices reach memory.
  constexpr bool kBlockSum = KS >= RT_WAVES;
  const int bi = lb % a.bpt;
  const int et_blk = bi % a.n_et;
  if (kBlockSum || unit < a.n_et * KS) {
    const int et = kBlockSum ? et_blk : unit % a.n_et;
    const int ks = kBlockSum ? (bi / a.n_et) * RT_WAVES + wv : unit / a.n_et;
    const int f_begin = ks * a.kf;
    const int f_end = min(a.kfrag_total, f_begin + a.kf);  // empty for trailing slices
    float b4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      b4[r] = (KS == 1 && a.bias) ? a.bias[min(et * 16 + 4 * lq + r, a.E - 1)] : 0.f;
    // The lane's rows in the load layout (row 4i + lq of the tile in load i)
    // and its chunk of each row's 256-byte step.
    const char* wp[RT_CHUNK];
    const char* xp[RT_CHUNK];
#pragma unroll
    for (int i = 0; i < RT_CHUNK; ++i) {
      wp[i] = reinterpret_cast<const char*>(a.wg) + static_cast<size_t>(min(et * 16 + 4 * i + lq, a.E - 1)) * row_bytes;
      xp[i] = reinterpret_cast<const char*>(a.x) + static_cast<size_t>(min(tt * 16 + 4 * i + lq, a.T - 1)) * row_bytes;
    }
    const int cbyte = 16 * stage_chunk(lrow, lq);
    char* wtile = s_raw + wv * 2 * RT_TILE;
    char* xtile = wtile + RT_TILE;
    // Two register buffers of RT_CHUNK fragments: the next step's loads are
    // in flight while the current one is transposed and multiplied.
    // Addresses are clamped into the slice, so every load is unconditional;
    // fragments past the slice end meet zero token fragments.
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    // Without block sums the waves of a block take 8 expert tiles of one K
    // slice, so when the expert tiles come in whole eights they all read the
    // same 16 token rows: waves 0-3 then load each step's token rows once
    // (row 4 * wave + lq per lane group) into a block-shared tile, double
    // buffered (the token halves of waves 0 and 1's own tiles), and every
    // wave reads its token fragments from there; one barrier per step.  The
    // buffer a step writes was last read two steps before, behind the
    // previous step's barrier.
    bool shared_x = false;
    if constexpr (!kBlockSum) shared_x = a.n_et % RT_WAVES == 0;
    if (f_begin < f_end && shared_x) {
      uint4 wa[RT_CHUNK], wb[RT_CHUNK], xa = make_uint4(0u, 0u, 0u, 0u), xb = xa;
      const int b_last = f_end * FRAG_BYTES - 16;
      const int xr = 4 * wv + lq;  // waves 0-3: the token row this lane group loads
      const char* xrow = reinterpret_cast<const char*>(a.x) + static_cast<size_t>(min(tt * 16 + xr, a.T - 1)) * row_bytes;
      const int xslot = xr * 256 + 16 * (stage_chunk(lrow, lq) ^ stage_swz(xr));
      char* sx0 = s_raw + RT_TILE;               // wave 0's token half
      char* sx1 = s_raw + 3 * RT_TILE;           // wave 1's token half
      auto load = [&](int f0, uint4 (&wf)[RT_CHUNK], uint4& xf) {
        const int b = min(f0 * FRAG_BYTES + cbyte, b_last);
#pragma unroll
        for (int i = 0; i < RT_CHUNK; ++i) wf[i] = ld16(wp[i] + b);
        if (wv < 4) xf = ld16(xrow + b);
      };
      auto mma = [&](int f0, const uint4 (&wf)[RT_CHUNK], const uint4& xf, char* sx) {
        if (wv < 4) *reinterpret_cast<uint4*>(sx + xslot) = xf;
        __syncthreads();
        uint4 wt[RT_CHUNK], xt[RT_CHUNK];
        stage_transpose(wf, wtile, lrow, lq, wt);
        const int sw = stage_swz(lrow);
#pragma unroll
        for (int f = 0; f < RT_CHUNK; ++f)
          xt[f] = *reinterpret_cast<const uint4*>(sx + lrow * 256 + 16 * ((4 * f + lq) ^ sw));
#pragma unroll
        for (int i = 0; i < RT_CHUNK; ++i) acc = Elem<T>::mma(wt[i], keep_or_zero(f0 + i < f_end, xt[i]), acc);
      };
      load(f_begin, wa, xa);
      for (int f0 = f_begin; f0 < f_end; f0 += 2 * RT_CHUNK) {
        load(f0 + RT_CHUNK, wb, xb);
        mma(f0, wa, xa, sx0);
        if (f0 + RT_CHUNK >= f_end) break;
        load(f0 + 2 * RT_CHUNK, wa, xa);
        mma(f0 + RT_CHUNK, wb, xb, sx1);
      }
    } else if (f_begin < f_end) {
      uint4 wa[RT_CHUNK], xa[RT_CHUNK], wb[RT_CHUNK], xb[RT_CHUNK];
      const int b_last = f_end * FRAG_BYTES - 16;
      auto load = [&](int f0, uint4 (&wf)[RT_CHUNK], uint4 (&xf)[RT_CHUNK]) {
        const int b = min(f0 * FRAG_BYTES + cbyte, b_last);
#pragma unroll
        for (int i = 0; i < RT_CHUNK; ++i) {
          wf[i] = ld16(wp[i] + b);
          xf[i] = ld16(xp[i] + b);
        }
      };
      auto mma = [&](int f0, const uint4 (&wf)[RT_CHUNK], const uint4 (&xf)[RT_CHUNK]) {
        uint4 wt[RT_CHUNK], xt[RT_CHUNK];
        stage_transpose(wf, wtile, lrow, lq, wt);
        stage_transpose(xf, xtile, lrow, lq, xt);
#pragma unroll
        for (int i = 0; i < RT_CHUNK; ++i) acc = Elem<T>::mma(wt[i], keep_or_zero(f0 + i < f_end, xt[i]), acc);
      };
      load(f_begin, wa, xa);
      for (int f0 = f_begin; f0 < f_end; f0 += 2 * RT_CHUNK) {
        load(f0 + RT_CHUNK, wb, xb);
        mma(f0, wa, xa);
        if (f0 + RT_CHUNK >= f_end) break;
        load(f0 + 2 * RT_CHUNK, wa, xa);
        mma(f0 + RT_CHUNK, wb, xb);
      }
    }
    // acc[r] = D[4*lq + r][lrow]: expert et*16 + 4*lq + r, token tt*16 + lrow.
    const int t = tt * 16 + lrow;
    if (kBlockSum) {
      __syncthreads();  // every wave is done with its staging tiles, which s_lg overlaps
      *reinterpret_cast<f32x4_t*>(s_lg + wv * 256 + 4 * l) = acc;
    } else if (t < a.T) {
      float* dst = (KS == 1) ? a.logits + static_cast<size_t>(t) * a.E
                             : a.partial + (static_cast<size_t>(ks) * a.T + t) * a.E;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int e = et * 16 + 4 * lq + r;
        if (e < a.E) st_agent(dst + e, acc[r] + b4[r]);
      }
    }
  }
  if (kBlockSum) {
    __syncthreads();
    if (tid < 256) {
      // element tid: lane tid / 4, register tid % 4 of every wave's tile
      float s = s_lg[tid];
#pragma unroll
      for (int w2 = 1; w2 < RT_WAVES; ++w2) s += s_lg[w2 * 256 + tid];
      const int li = tid >> 2;
      const int t = tt * 16 + (li & 15);
      const int e = et_blk * 16 + 4 * (li >> 4) + (tid & 3);
      if (t < a.T && e < a.E)
        st_agent(a.partial + (static_cast<size_t>(bi / a.n_et) * a.T + t) * a.E + e, s);
    }
  }

  // ---------------- hand-off: the last block of this token tile continues
  if (!last_to_arrive(a.ctr + tt, a.bpt, &s_last)) return;

  // ---------------- phase B1: the tile's logits into LDS (slice sums in slice order)
  const int t0 = tt * 16;
  const int n_tok = min(16, a.T - t0);
  const int n_lg = n_tok * a.E;
  const size_t slice = static_cast<size_t>(a.T) * a.E;
  const float* src = (KS == 1) ? a.logits : a.partial;
  constexpr int KSP = kBlockSum ? KS / RT_WAVES : KS;  // partial slices in memory
  for (int i0 = tid; i0 < n_lg; i0 += RT_THREADS * RT_UNROLL) {
    float part[RT_UNROLL][KSP];  // every load is issued before the first add
#pragma unroll
    for (int u = 0; u < RT_UNROLL; ++u) {
      const int i = min(i0 + u * RT_THREADS, n_lg - 1);
#pragma unroll
      for (int ks = 0; ks < KSP; ++ks) part[u][ks] = ld_agent(src + ks * slice + static_cast<size_t>(t0) * a.E + i);
    }
#pragma unroll
    for (int u = 0; u < RT_UNROLL; ++u) {
      const int i = i0 + u * RT_THREADS;
      if (i < n_lg) {
        float s = part[u][0];
#pragma unroll
        for (int ks = 1; ks < KSP; ++ks) s += part[u][ks];
        if (KS > 1) {
          s += a.bias ? a.bias[i % a.E] : 0.f;
          a.logits[static_cast<size_t>(t0) * a.E + i] = s;
        }
        s_lg[i] = s;
      }
    }
  }
  __syncthreads();

  // ---------------- phase B2: top-k of the tile's tokens, 32 lanes per token
  const int kk = a.k + a.n_shared;
  // A single token tile sorts in this block: its pair keys stay in LDS.
  const bool one_tile = a.n_tt == 1 && a.counts != nullptr;
  {
    const int j = tid / TK_LANES;  // group-uniform
    if (j < n_tok) {
      const size_t t = static_cast<size_t>(t0 + j);
      const float* lg = s_lg + j * a.E;
      int32_t* ids = a.ids + t * kk;
      float* w = a.w + t * kk;
      uint16_t* pk = one_tile ? s_pk + j * kk : nullptr;
      if (a.E <= 2 * TK_LANES) group_topk<2>(lg, a.E, a.k, a.renorm, a.n_shared, ids, w, pk, a.g_begin, a.n_groups);
      else if (a.E <= 4 * TK_LANES) group_topk<4>(lg, a.E, a.k, a.renorm, a.n_shared, ids, w, pk, a.g_begin, a.n_groups);
      else if (a.E <= 8 * TK_LANES) group_topk<8>(lg, a.E, a.k, a.renorm, a.n_shared, ids, w, pk, a.g_begin, a.n_groups);
      else group_topk<TK_MAXV>(lg, a.E, a.k, a.renorm, a.n_shared, ids, w, pk, a.g_begin, a.n_groups);
    }
  }
  if (a.counts == nullptr) return;  // routing only

  if (one_tile) {
    // the sort's first barrier orders the key writes before its passes
    block_counting_sort<RT_WAVES, true>(a.ids, a.T * kk, a.g_begin, a.n_groups, a.counts, a.offsets,
                                        a.sorted_pair, a.pair_pos, s_cnt, s_off, s_pk, -1);
    return;
  }

  // ---------------- hand-off: the block finishing the last tile sorts all pairs
  if (!last_to_arrive(a.ctr + a.n_tt, a.n_tt, &s_last)) return;

  // ---------------- phase C: stable counting sort of the T*kk pairs
  block_counting_sort<RT_WAVES, true>(a.ids, a.T * kk, a.g_begin, a.n_groups, a.counts, a.offsets,
                                      a.sorted_pair, a.pair_pos, s_cnt, s_off,
                                      reinterpret_cast<uint16_t*>(s_lg), RT_KEY_CAP);
}

// ---------------------------------------------------------------- host side

struct RoutePlan {
  int ks, kf, n_et, n_tt, bpt, grid;
  size_t ctr_bytes, partial_bytes;
};

static RoutePlan plan_route(int T, int H, int E, int dtype) {
  RoutePlan p{};
  const int kft = H * (dtype == 1 ? 2 : 4) / FRAG_BYTES;
  p.n_et = (E + 15) / 16;
  p.n_tt = (T + 15) / 16;
  // K slices (a power of two): enough wave units to spread the gate matrix
  // and the activations over the chip (~8 waves per CU), at least 8
  // fragments (512 bytes of each row) per slice.  (A target of 16 waves per
  // CU made the route call 1.9 us longer at T = 512 and 0.8 us at 2048; the
  // decode batches reach 16 slices under either target.)
  const long long tiles = static_cast<long long>(p.n_et) * p.n_tt;
  int ks = 1;
  while (ks < RT_MAX_KS && tiles * ks < 2048 && kft / (2 * ks) >= 8) ks *= 2;
  p.ks = ks;
  p.kf = (kft + ks - 1) / ks;
  p.bpt = (p.n_et * p.ks + RT_WAVES - 1) / RT_WAVES;
  p.grid = (p.n_tt * p.bpt + N_XCD - 1) / N_XCD * N_XCD;
  p.ctr_bytes = ((static_cast<size_t>(p.n_tt) + 1) * sizeof(int) + 255) & ~static_cast<size_t>(255);
  const int ksp = p.ks >= RT_WAVES ? p.ks / RT_WAVES : p.ks;  // partial slices in memory
  p.partial_bytes = p.ks > 1 ? static_cast<size_t>(ksp) * T * E * sizeof(float) : 0;
  return p;
}

bool route_fits(int T, int H, int E, int dtype) {
  if (T <= 0) return true;
  const long long n_tt = (static_cast<long long>(T) + 15) / 16;
  const long long n_et = (E + 15) / 16;
  // the fewest K slices any plan takes is 1: bpt >= ceil(n_et / 8); the most is RT_MAX_KS
  const long long bpt = (n_et * RT_MAX_KS + RT_WAVES - 1) / RT_WAVES;
  return n_tt * bpt + N_XCD <= 0x7fffffffLL && static_cast<long long>(H) * (dtype == 1 ? 2 : 4) / FRAG_BYTES > 0;
}

size_t route_workspace_bytes(int T, int H, int E, int dtype) {
  if (T <= 0) return 0;
  const RoutePlan p = plan_route(T, H, E, dtype);
  return p.ctr_bytes + p.partial_bytes;
}

template <typename T>
static void launch_route_t(const RoutePlan& p, const RouteArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(p.grid)), block(RT_THREADS);
  switch (p.ks) {
    case 1: hipLaunchKernelGGL((route_kernel<T, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((route_kernel<T, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((route_kernel<T, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((route_kernel<T, 8>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((route_kernel<T, 16>), grid, block, 0, s, a); break;
  }
}

// ---------------------------------------------------------------- allocation-free variant
//
// A fixed scratch region in device memory for callers that cannot allocate a
// workspace.  It is a file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  On the
// host its name is only a stand-in for that address, so host code never
// passes it to a kernel; it uses the per-device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current.  All calls on one GPU share its copy (calls that overlap in time
// race on it).
static __device__ __align__(256) char scratch[ROUTE_SCRATCH_BYTES];

namespace {

constexpr int SCRATCH_MAX_DEVICES = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[SCRATCH_MAX_DEVICES];

// The current device's copy of `scratch`, or nullptr with *err set.
void* scratch_address(hipError_t* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= SCRATCH_MAX_DEVICES) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot] {
    void* p = nullptr;
    slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (slot.err == hipSuccess && p == nullptr) slot.err = hipErrorInvalidSymbol;
    slot.ptr = slot.err == hipSuccess ? p : nullptr;
  });
  *err = slot.err;
  return slot.ptr;
}

__global__ void zero_ints_kernel(int* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

}  // namespace

int launch_route_permute_scratch(int dtype, const void* x, const void* wg, const float* bias, float* logits,
                                 int32_t* ids, float* w, int T, int H, int E, int k, int renorm,
                                 int n_shared, int g_begin, int n_groups, int32_t* counts, int32_t* offsets,
                                 int32_t* sorted_pair, int32_t* pair_pos, hipStream_t s) {
  hipError_t err = hipSuccess;
  void* ptr = scratch_address(&err);
  if (ptr == nullptr) return 1;
  // The counters must start at zero: a fill kernel (not a memset node, so
  // the call stays capturable in a graph) clears them on the stream first.
  const RoutePlan p = plan_route(T, H, E, dtype);
  const int n_ctr = p.n_tt + 1;
  hipLaunchKernelGGL(zero_ints_kernel, dim3((n_ctr + 255) / 256), dim3(256), 0, s, static_cast<int*>(ptr), n_ctr);
  launch_route(dtype, x, wg, bias, logits, ids, w, T, H, E, k, renorm, n_shared, ptr, g_begin, n_groups, counts,
               offsets, sorted_pair, pair_pos, s);
  return 0;
}

void launch_route(int dtype, const void* x, const void* wg, const float* bias, float* logits,
                  int32_t* ids, float* w, int T, int H, int E, int k, int renorm, int n_shared,
                  void* ws, int g_begin, int n_groups, int32_t* counts, int32_t* offsets,
                  int32_t* sorted_pair, int32_t* pair_pos, hipStream_t s) {
  // Many pairs: one block sorting them all would set the launch's end, so the
  // routing launch stops after the top-k and the multi-block permute follows.
  if (counts != nullptr && permute_uses_blocks(T, k + n_shared)) {
    launch_route(dtype, x, wg, bias, logits, ids, w, T, H, E, k, renorm, n_shared, ws, g_begin, n_groups,
                 nullptr, nullptr, nullptr, nullptr, s);
    launch_permute(ids, T, k + n_shared, g_begin, n_groups, counts, offsets, sorted_pair, pair_pos, s);
    return;
  }
  const RoutePlan p = plan_route(T, H, E, dtype);
  RouteArgs a{};
  a.x = x;
  a.wg = wg;
  a.bias = bias;
  a.logits = logits;
  a.ids = ids;
  a.w = w;
  a.ctr = static_cast<int*>(ws);
  a.partial = p.ks > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.ctr_bytes) : nullptr;
  a.counts = counts;
  a.offsets = offsets;
  a.sorted_pair = sorted_pair;
  a.pair_pos = pair_pos;
  a.g_begin = g_begin;
  a.n_groups = n_groups;
  a.T = T;
  a.H = H;
  a.E = E;
  a.k = k;
  a.renorm = renorm;
  a.n_shared = n_shared;
  a.kfrag_total = H * (dtype == 1 ? 2 : 4) / FRAG_BYTES;
  a.kf = p.kf;
  a.n_et = p.n_et;
  a.n_tt = p.n_tt;
  a.bpt = p.bpt;
  if (dtype == 1)
    launch_route_t<uint16_t>(p, a, s);
  else
    launch_route_t<float>(p, a, s);
}

}  // namespace moe
