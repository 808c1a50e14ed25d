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
// weights of that token are block-uniform.
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
  float acc[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) acc[i] = 0.f;
  bool first = true;
  for (int j = 0; j < kk; ++j) {
    const int pos = pair_pos[static_cast<size_t>(t) * kk + j];
    if (pos < 0) continue;
    const float wj = w ? w[static_cast<size_t>(t) * kk + j] : 1.f;
    const uint4 v = ld16(y_pair + static_cast<size_t>(pos) * H + h0);
    const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      const float term = wj * Elem<T>::load(e + i);
      acc[i] = first ? term : acc[i] + term;
    }
    first = false;
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
