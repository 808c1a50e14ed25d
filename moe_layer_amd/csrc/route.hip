// Softmax + top-k routing (Sem-MoE notes, Key design 1: top-k of the softmax
// of the gate logits).  One wavefront per token.
//
// Lane l holds logits of experts l, l+64, ... (up to 8).  Each of the k rounds
// takes every lane's best remaining (value, id) and reduces the wave with a
// xor-butterfly under the order "larger value first, then lower expert id";
// that order is total, so every lane ends with the same winner and equal
// logits (including -0.0 vs +0.0) always go to the lower id.  Lane j keeps the
// j-th pick.  Selection is on the fp32 logits, which picks the same set as
// the softmax.  The softmax weights use the row maximum (the first pick); the
// butterfly sums are commutative at every level, so every lane sees the same
// bits.  Shared experts follow the routed slots as ids E, E+1, ... with
// weight 1.
#include <math.h>

#include "common.hpp"
#include "moe_internal.h"

namespace moe {

constexpr int TOPK_WAVES = 4;
constexpr int MAX_PER_LANE = MAX_E / WAVE;

__global__ __launch_bounds__(TOPK_WAVES * WAVE) void topk_kernel(const float* __restrict__ logits,
                                                                  int T, int E, int k, int renorm,
                                                                  int n_shared,
                                                                  int32_t* __restrict__ ids,
                                                                  float* __restrict__ w) {
  const int t = blockIdx.x * TOPK_WAVES + threadIdx.x / WAVE;
  if (t >= T) return;  // whole wave leaves together
  const int l = lane_id();
  const int kk = k + n_shared;
  const float* row = logits + static_cast<size_t>(t) * E;

  float v[MAX_PER_LANE];
#pragma unroll
  for (int j = 0; j < MAX_PER_LANE; ++j) {
    const int e = l + WAVE * j;
    v[j] = (e < E) ? row[e] : -INFINITY;
  }
  unsigned taken = 0;  // bit j: expert l + 64 j already picked (or absent)
#pragma unroll
  for (int j = 0; j < MAX_PER_LANE; ++j)
    if (l + WAVE * j >= E) taken |= 1u << j;

  float my_v = -INFINITY;
  int my_e = -1;
  for (int round = 0; round < k; ++round) {
    float bv = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < MAX_PER_LANE; ++j) {
      const int e = l + WAVE * j;
      if (!((taken >> j) & 1u) && (be == 0x7fffffff || v[j] > bv)) {
        bv = v[j];
        be = e;
      }
    }
#pragma unroll
    for (int off = WAVE / 2; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, WAVE);
      const int oe = __shfl_xor(be, off, WAVE);
      if (oe != 0x7fffffff && (be == 0x7fffffff || ov > bv || (ov == bv && oe < be))) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & (WAVE - 1)) == l) taken |= 1u << (be / WAVE);
    if (l == round) {
      my_v = bv;
      my_e = be;
    }
  }

  const float mx = __shfl(my_v, 0, WAVE);
  float s_all = 0.f;
#pragma unroll
  for (int j = 0; j < MAX_PER_LANE; ++j)
    if (l + WAVE * j < E) s_all += expf(v[j] - mx);
  float p = (l < k) ? expf(my_v - mx) : 0.f;
  float s_sel = p;
#pragma unroll
  for (int off = WAVE / 2; off > 0; off >>= 1) {
    s_all += __shfl_xor(s_all, off, WAVE);
    s_sel += __shfl_xor(s_sel, off, WAVE);
  }
  const float denom = renorm ? s_sel : s_all;
  if (l < k) {
    ids[static_cast<size_t>(t) * kk + l] = my_e;
    w[static_cast<size_t>(t) * kk + l] = p / denom;
  } else if (l < kk) {
    ids[static_cast<size_t>(t) * kk + l] = E + (l - k);
    w[static_cast<size_t>(t) * kk + l] = 1.0f;
  }
}

void launch_topk(const float* logits, int T, int E, int k, int renorm, int n_shared, int32_t* ids,
                 float* w, hipStream_t s) {
  const int grid = (T + TOPK_WAVES - 1) / TOPK_WAVES;
  hipLaunchKernelGGL(topk_kernel, dim3(grid), dim3(TOPK_WAVES * WAVE), 0, s, logits, T, E, k,
                     renorm, n_shared, ids, w);
}

}  // namespace moe
