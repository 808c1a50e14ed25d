// EP -> TP local permute of expert weights (Moebius review, §3.1 weight
// resharding and Fig. 4: before the exchange, each rank packs the bytes bound
// for each peer into one contiguous block per destination).
//
// Source (this rank's E_local whole experts):
//   W13 (E_local, 2I, H), W2 (E_local, H, I)
// Destination block q (peer q's TP slice S_q = [q I/P, (q+1) I/P) of them):
//   dst13[q] (E_local, 2I/P, H): rows S_q of the gate half, then rows S_q of
//                                the up half, of every local expert
//   dst2[q]  (E_local, H, I/P):  columns S_q of every W2 row
// One launch walks both source tensors in address order, 16 bytes per lane:
// reads are fully coalesced, each W13 row lands as one contiguous row and
// each W2 row splits into P contiguous segments.  Every byte is read once and
// written once; the copy is exact.
#include "common.hpp"
#include "moe_internal.h"

namespace moe {

constexpr int REPACK_THREADS = 256;
constexpr int REPACK_UNROLL = 4;

struct RepackArgs {
  const char* w13;
  const char* w2;
  PeerPtrs d13;
  PeerPtrs d2;
  long long chunks13;  // 16-byte chunks in W13
  long long chunks2;   // 16-byte chunks in W2
  int row13;           // chunks per W13 row (H * elem / 16)
  int row2;            // chunks per W2 row (I * elem / 16)
  int I;               // rows per half of W13
  int Ip;              // I / P
  int seg2;            // chunks per W2 segment (Ip * elem / 16)
};

__device__ __forceinline__ char* repack_dst(const RepackArgs& a, long long c) {
  if (c < a.chunks13) {
    const long long row = c / a.row13;
    const int col = static_cast<int>(c - row * a.row13);
    const long long e = row / (2 * a.I);
    const int i2 = static_cast<int>(row - e * 2 * a.I);
    const int half = i2 / a.I;
    const int i = i2 - half * a.I;
    const int q = i / a.Ip;
    const long long drow = e * 2 * a.Ip + half * a.Ip + (i - q * a.Ip);
    return static_cast<char*>(a.d13.p[q]) + (drow * a.row13 + col) * 16;
  }
  c -= a.chunks13;
  const long long row = c / a.row2;  // (e, h) row of W2
  const int col = static_cast<int>(c - row * a.row2);
  const int q = col / a.seg2;
  return static_cast<char*>(a.d2.p[q]) + (row * a.seg2 + (col - q * a.seg2)) * 16;
}

__device__ __forceinline__ const char* repack_src(const RepackArgs& a, long long c) {
  return c < a.chunks13 ? a.w13 + c * 16 : a.w2 + (c - a.chunks13) * 16;
}

__global__ __launch_bounds__(REPACK_THREADS) void repack_kernel(RepackArgs a) {
  const long long total = a.chunks13 + a.chunks2;
  const long long stride = static_cast<long long>(gridDim.x) * REPACK_THREADS;
  long long c = static_cast<long long>(blockIdx.x) * REPACK_THREADS + threadIdx.x;
  for (; c < total; c += stride * REPACK_UNROLL) {
    u32x4_t v[REPACK_UNROLL];
#pragma unroll
    for (int u = 0; u < REPACK_UNROLL; ++u) {
      const long long cu = c + u * stride;
      if (cu < total) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(repack_src(a, cu)));
    }
#pragma unroll
    for (int u = 0; u < REPACK_UNROLL; ++u) {
      const long long cu = c + u * stride;
      if (cu < total) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4_t*>(repack_dst(a, cu)));
    }
  }
}

void launch_repack_ep_to_tp(int dtype, const void* w13, const void* w2, int E_local, int H, int I,
                            int P, const PeerPtrs& d13, const PeerPtrs& d2, hipStream_t s) {
  const int eb = dtype == 1 ? 2 : 4;
  RepackArgs a{};
  a.w13 = static_cast<const char*>(w13);
  a.w2 = static_cast<const char*>(w2);
  a.d13 = d13;
  a.d2 = d2;
  a.row13 = H * eb / 16;
  a.row2 = I * eb / 16;
  a.chunks13 = static_cast<long long>(E_local) * 2 * I * a.row13;
  a.chunks2 = static_cast<long long>(E_local) * H * a.row2;
  a.I = I;
  a.Ip = I / P;
  a.seg2 = a.Ip * eb / 16;
  const long long total = a.chunks13 + a.chunks2;
  long long want = (total + REPACK_THREADS * REPACK_UNROLL - 1) / (REPACK_THREADS * REPACK_UNROLL);
  const long long cap = static_cast<long long>(device_cu_count()) * 8;
  const int grid = static_cast<int>(want < cap ? (want > 0 ? want : 1) : cap);
  hipLaunchKernelGGL(repack_kernel, dim3(grid), dim3(REPACK_THREADS), 0, s, a);
}

}  // namespace moe
