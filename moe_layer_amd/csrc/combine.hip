// Weighted combine: y[t] = sum over slots j = 0..kk-1, in slot order, of
// w[t, j] * y_pair[pos[t, j]], skipping slots whose pair this GPU does not hold
// (pos = -1).  Accumulation in fp32, one rounding to the output type.  In the
// EP view this is the rank's partial before the combine all-to-all; in the TP
// view it is the partial before the all-reduce (Moebius review, §2.1 and §3.1).
// After an EP dispatch the sender runs it on the rows that came back, with the
// dispatch's pair positions.  Without weights (w == nullptr) every weight is 1;
// with kk = 1 that is the receiver's un-permute of its expert outputs back to
// arrival order.  The first held slot initialises the sum, so one slot of
// weight 1 copies its row exactly (signed zeros included).
//
// Each thread owns one 16-byte vector of one token row; the slot positions and
// weights of that token are block-uniform (scalar loads).  Slots are taken
// eight at a time: their positions first, then all eight row loads, then the
// sums in slot order, so a token's rows arrive in one round trip.
#include "common.hpp"
#include "moe_internal.h"

namespace moe {

constexpr int COMBINE_THREADS = 256;

template <typename T>
__global__ __launch_bounds__(COMBINE_THREADS) void combine_kernel(const T* __restrict__ y_pair,
                                                                  const int32_t* __restrict__ pair_pos,
                                                                  const float* __restrict__ w, int kk,
                                                                  int H, int h_blocks, T* __restrict__ y) {
  constexpr int VEC = 16 / sizeof(T);
  const int t = blockIdx.x / h_blocks;
  const int h0 = ((blockIdx.x % h_blocks) * COMBINE_THREADS + threadIdx.x) * VEC;
  if (h0 >= H) return;
  constexpr int SLOTS = 8;
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
  bool first = true;
  const int32_t* pp = pair_pos + static_cast<size_t>(t) * kk;
  const float* pw = w ? w + static_cast<size_t>(t) * kk : nullptr;
  for (int j0 = 0; j0 < kk; j0 += SLOTS) {
    int pos[SLOTS];
    float wj[SLOTS];
#pragma unroll
    for (int u = 0; u < SLOTS; ++u) {
      pos[u] = j0 + u < kk ? pp[j0 + u] : -1;
      wj[u] = (pw && j0 + u < kk) ? pw[j0 + u] : 1.f;
    }
    uint4 v[SLOTS];
#pragma unroll
    for (int u = 0; u < SLOTS; ++u)
      v[u] = pos[u] >= 0 ? ld16(y_pair + static_cast<size_t>(pos[u]) * H + h0) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int u = 0; u < SLOTS; ++u) {
      if (pos[u] < 0) continue;
      const T* e = reinterpret_cast<const T*>(&v[u]);
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        const float term = wj[u] * Elem<T>::load(e + i);
        acc[i] = first ? term : acc[i] + term;
      }
      first = false;
    }
  }
  T* dst = y + static_cast<size_t>(t) * H + h0;
#pragma unroll
  for (int i = 0; i < VEC; i += 4) Elem<T>::store4(dst + i, acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
}

void launch_combine(int dtype, const void* y_pair, const int32_t* pair_pos, const float* w, int T,
                    int kk, int H, void* y, hipStream_t s) {
  const int vec = dtype == 1 ? 8 : 4;
  const int h_blocks = (H / vec + COMBINE_THREADS - 1) / COMBINE_THREADS;
  const dim3 grid(static_cast<unsigned>(h_blocks) * static_cast<unsigned>(T));
  if (dtype == 1)
    hipLaunchKernelGGL(combine_kernel<uint16_t>, grid, dim3(COMBINE_THREADS), 0, s,
                       static_cast<const uint16_t*>(y_pair), pair_pos, w, kk, H, h_blocks,
                       static_cast<uint16_t*>(y));
  else
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(COMBINE_THREADS), 0, s,
                       static_cast<const float*>(y_pair), pair_pos, w, kk, H, h_blocks,
                       static_cast<float*>(y));
}

}  // namespace moe
