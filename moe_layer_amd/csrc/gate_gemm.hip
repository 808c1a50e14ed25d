// Gate GEMM (bf16 or fp32 storage, fp32 accumulate) on the register-slab kernel.
//
// Work unit ("item"): one expert group g and one tile of 16 weight rows.
//   up   : rows are 8 gate rows (W1, W13 rows [n, n+8)) and the 8 matching up
//          rows (W3, W13 rows [I'+n, I'+n+8)), so SiLU(gate)*up is formed in
//          registers (Moebius review §3.1 gives W13 as (., 2I, H); the
//          gate-then-up row order is this library's layout contract).
//   down : rows are 16 rows of W2 (., H, I'), i.e. 16 output features.
//   gate : rows are 16 experts of the gate matrix (E, H) (Sem-MoE notes,
//          Key design 1: logits = W_g h + b).
// A block holds the item's weight rows as register-resident K-slabs: wave
// (ks, ns) keeps fragments [ks*kf, (ks+1)*kf) of n-tile ns, loaded once, and
// then streams the group's token rows through them 16 at a time.  Each weight
// byte is read from HBM exactly once per call however many tokens the group
// has; activations come from L2.  Waves that split K add their partial
// 16x16 tiles in LDS in a fixed order (no atomics), so results are
// bit-reproducible.
#include "common.hpp"
#include "moe_internal.h"

namespace moe {

constexpr int KF = 16;        // max fragments (x 64 B of K per row) held per wave
constexpr int BLOCK_MAX = 1024;

enum Mode { MODE_UP = 0, MODE_DOWN = 1, MODE_GATE = 2 };

struct GemmArgs {
  const void* act;         // up/gate: x (T, K); down: A (n_pairs, K)
  const int* sorted_pair;  // up: pair id of each sorted row
  const int* offsets;      // up/down: (n_groups + 1) row offsets
  const void* w;           // up: w13 (G, 2I', K); down: w2 (G, H, K); gate: wg (E, K)
  void* out;               // up: A (n_pairs, I'); down: y_pair (n_pairs, H); gate: logits (T, E)
  const float* bias;       // gate: (E) or null
  int n_groups;
  int kk;
  int K;                   // contraction length (elements)
  int I_loc;               // up: I'
  int n_rows;              // down: H; gate: E (rows of the weight matrix per group)
  int T;                   // gate: tokens
  int kfrag_total;         // K * elem / 64
  int kf;                  // fragments per wave
  int nw_k;                // waves splitting K
  int ns;                  // n-tiles per block
  int n_tiles;             // 16-row tiles per group, grouped by ns: items per group = n_tiles / ns
  int t_chunk;             // gate: tokens per item
};

template <typename T, int MODE>
__global__ __launch_bounds__(BLOCK_MAX) void grouped_gemm_kernel(GemmArgs a) {
  __shared__ int s_list[MAX_GROUPS];
  __shared__ int s_nlist;
  __shared__ f32x4_t s_red[MAX_KSPLIT][WAVE];

  const int wv = threadIdx.x / WAVE;
  const int ks = wv % a.nw_k;
  const int nsi = wv / a.nw_k;
  const int l = lane_id();
  const int lrow = l & 15;
  const int lq = l >> 4;
  const int items_per_group = a.n_tiles / a.ns;

  int n_items;
  if (MODE == MODE_GATE) {
    n_items = items_per_group * ((a.T + a.t_chunk - 1) / a.t_chunk);
  } else {
    touched_groups(a.offsets, a.n_groups, s_list, &s_nlist);
    __syncthreads();
    n_items = s_nlist * items_per_group;
  }

  const int f0 = ks * a.kf;
  const int nf = min(a.kf, a.kfrag_total - f0);
  const size_t row_bytes = static_cast<size_t>(a.K) * sizeof(T);
  const char* wbase = reinterpret_cast<const char*>(a.w);
  const char* abase = reinterpret_cast<const char*>(a.act);

  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    const int gi = item / items_per_group;
    const int nt = (item % items_per_group) * a.ns + nsi;
    int g = 0, row0 = 0, m = 0;
    if (MODE == MODE_GATE) {
      row0 = gi * a.t_chunk;
      m = min(a.t_chunk, a.T - row0);
    } else {
      g = s_list[gi];
      row0 = a.offsets[g];
      m = a.offsets[g + 1] - row0;
    }

    // This lane's weight row.
    size_t wrow;
    if (MODE == MODE_UP) {
      const int r = (lrow < 8) ? (nt * 8 + lrow) : (a.I_loc + nt * 8 + (lrow - 8));
      wrow = static_cast<size_t>(g) * (2 * a.I_loc) + r;
    } else if (MODE == MODE_DOWN) {
      wrow = static_cast<size_t>(g) * a.n_rows + nt * 16 + lrow;
    } else {
      wrow = min(nt * 16 + lrow, a.n_rows - 1);
    }
    const char* wp = wbase + wrow * row_bytes + static_cast<size_t>(f0) * FRAG_BYTES + lq * 16;
    uint4 wf[KF];
#pragma unroll
    for (int f = 0; f < KF; ++f)
      if (f < nf) wf[f] = ld16(wp + f * FRAG_BYTES);

    for (int mt = 0; mt < m; mt += 16) {
      const int r_in = mt + lrow;
      const int r_cl = (r_in < m) ? r_in : (m - 1);  // padded rows repeat a real row, never stored
      size_t arow;
      if (MODE == MODE_UP) arow = static_cast<size_t>(a.sorted_pair[row0 + r_cl] / a.kk);
      else arow = static_cast<size_t>(row0 + r_cl);
      const char* ap = abase + arow * row_bytes + static_cast<size_t>(f0) * FRAG_BYTES + lq * 16;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int f = 0; f < KF; ++f)
        if (f < nf) acc = Elem<T>::mma(wf[f], ld16(ap + f * FRAG_BYTES), acc);

      bool owner = true;
      if (a.nw_k > 1) {
        s_red[wv][l] = acc;
        __syncthreads();
        owner = (ks == 0);
        if (owner) {
          for (int v = 1; v < a.nw_k; ++v) acc += s_red[wv + v][l];
        }
        __syncthreads();
      }
      if (!owner) continue;

      // acc[r] = D[4*lq + r][lrow]: weight row 4*lq+r of the tile, token row lrow.
      const bool valid = r_in < m;
      if (MODE == MODE_UP) {
        float up[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) up[r] = __shfl_xor(acc[r], 32, WAVE);
        if (lq < 2 && valid) {
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float gt = acc[r];
            o[r] = gt / (1.0f + __expf(-gt)) * up[r];
          }
          T* dst = reinterpret_cast<T*>(a.out) + static_cast<size_t>(row0 + r_in) * a.I_loc + nt * 8 + 4 * lq;
          Elem<T>::store4(dst, o[0], o[1], o[2], o[3]);
        }
      } else if (MODE == MODE_DOWN) {
        if (valid) {
          T* dst = reinterpret_cast<T*>(a.out) + static_cast<size_t>(row0 + r_in) * a.n_rows + nt * 16 + 4 * lq;
          Elem<T>::store4(dst, acc[0], acc[1], acc[2], acc[3]);
        }
      } else {
        if (valid) {
          float* dst = reinterpret_cast<float*>(a.out) + static_cast<size_t>(row0 + r_in) * a.n_rows;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int e = nt * 16 + 4 * lq + r;
            if (e < a.n_rows) dst[e] = acc[r] + (a.bias ? a.bias[e] : 0.f);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- host side

static int g_cu_count[64];

int device_cu_count() {
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev < 0 || dev >= 64) dev = 0;
  if (g_cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_cu_count[dev] = n;
  }
  return g_cu_count[dev];
}

// Split K into nw_k waves of at most KF fragments each.
static void split_k(GemmArgs& a) {
  a.nw_k = (a.kfrag_total + KF - 1) / KF;
  a.kf = (a.kfrag_total + a.nw_k - 1) / a.nw_k;
  a.nw_k = (a.kfrag_total + a.kf - 1) / a.kf;
}

template <int MODE>
static void launch(int dtype, GemmArgs a, int max_items, hipStream_t s) {
  const int threads = a.nw_k * a.ns * WAVE;
  const int per_cu = (BLOCK_MAX * 2) / threads;  // aim for ~32 resident waves per CU
  int grid = device_cu_count() * (per_cu > 0 ? per_cu : 1);
  if (grid > max_items) grid = max_items;
  if (grid < 1) grid = 1;
  if (dtype == 1)
    hipLaunchKernelGGL((grouped_gemm_kernel<uint16_t, MODE>), dim3(grid), dim3(threads), 0, s, a);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<float, MODE>), dim3(grid), dim3(threads), 0, s, a);
}

static int elem_bytes(int dtype) { return dtype == 1 ? 2 : 4; }

void launch_gate_gemm(int dtype, const void* x, const void* wg, const float* bias, float* logits,
                      int T, int H, int E, hipStream_t s) {
  GemmArgs a{};
  a.act = x;
  a.w = wg;
  a.out = logits;
  a.bias = bias;
  a.K = H;
  a.n_rows = E;
  a.T = T;
  a.kfrag_total = H * elem_bytes(dtype) / FRAG_BYTES;
  split_k(a);
  a.n_tiles = (E + 15) / 16;
  a.ns = 1;
  // Enough items to spread the gate matrix and the tokens over the chip.
  const int want_items = 2 * device_cu_count();
  int chunks = (want_items + a.n_tiles - 1) / a.n_tiles;
  int t_chunk = (T + chunks - 1) / chunks;
  t_chunk = ((t_chunk + 15) / 16) * 16;
  if (t_chunk < 16) t_chunk = 16;
  a.t_chunk = t_chunk;
  const int n_items = a.n_tiles * ((T + t_chunk - 1) / t_chunk);
  launch<MODE_GATE>(dtype, a, n_items, s);
}

}  // namespace moe
