// moe_permute on its own: expert counts, offsets and the stable permutation of
// (token, slot) pairs by expert group in one block of 16 waves (the counting
// sort of sort.hpp).  The fused routing launch (route.hip) runs the same sort
// in its last block.
#include "common.hpp"
#include "moe_internal.h"
#include "sort.hpp"

namespace moe {

constexpr int PERM_WAVES = 16;
constexpr int PERM_KEY_CAP = 16384;

__global__ __launch_bounds__(PERM_WAVES * WAVE) void permute_kernel(
    const int32_t* __restrict__ ids, int N, int g_begin, int n_groups, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos) {
  __shared__ int s_cnt[PERM_WAVES * MAX_GROUPS];
  __shared__ int s_off[MAX_GROUPS];
  __shared__ uint16_t s_key[PERM_KEY_CAP];
  block_counting_sort<PERM_WAVES, false>(ids, N, g_begin, n_groups, counts, offsets, sorted_pair,
                                         pair_pos, s_cnt, s_off, s_key, PERM_KEY_CAP);
}

void launch_permute(const int32_t* ids, int T, int kk, int g_begin, int n_groups, int32_t* counts,
                    int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, hipStream_t s) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(PERM_WAVES * WAVE), 0, s, ids, T * kk, g_begin,
                     n_groups, counts, offsets, sorted_pair, pair_pos);
}

}  // namespace moe
