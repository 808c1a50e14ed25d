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
// One launch walks both source tensors row by row (a wave per row, 16 bytes
// per lane): reads are fully coalesced, each W13 row lands as one contiguous
// row and each W2 row splits into P contiguous segments.  Every byte is read
// once and written once; the copy is exact.
#include "common.hpp"
#include "moe_internal.h"

namespace moe {

constexpr int RP_WAVES = 4;                 // waves per block
constexpr int RP_U = 8;                     // 16-byte chunks per lane per step
constexpr int RP_STEP = RP_U * WAVE;        // chunks per wave per step

struct RepackArgs {
  const char* w13;
  const char* w2;
  PeerPtrs d13;
  PeerPtrs d2;
  long long rows13;    // E_local * 2I source rows of W13
  long long rows2;     // E_local * H source rows of W2
  int row13;           // chunks per W13 row (H * elem / 16)
  int row2;            // chunks per W2 row (I * elem / 16)
  int I;               // rows per half of W13
  int Ip;              // I / P
  int seg2;            // chunks per W2 segment (Ip * elem / 16)
};

// One wave copies whole source rows, in address order, RP_U chunks per lane
// per step with all loads issued before the stores.  A W13 row has one
// wave-uniform destination row; a W2 row falls into P segments, and which
// segment (and where in it) a lane's chunk of a step lands is the same for
// every W2 row, so it is worked out once per lane.
__global__ __launch_bounds__(RP_WAVES * WAVE) void repack_kernel(RepackArgs a) {
  const int l = lane_id();
  const long long nw = static_cast<long long>(gridDim.x) * RP_WAVES;
  const long long w0 = static_cast<long long>(blockIdx.x) * RP_WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);

  // ---- W13: row (e, half, i) -> block q = i / Ip, row e*2Ip + half*Ip + i%Ip
  for (long long r = w0; r < a.rows13; r += nw) {
    const long long e = r / (2 * a.I);
    const int i2 = static_cast<int>(r - e * 2 * a.I);
    const int half = i2 >= a.I;
    const int i = i2 - half * a.I;
    const int q = i / a.Ip;
    const long long drow = e * 2 * a.Ip + half * a.Ip + (i - q * a.Ip);
    const char* src = a.w13 + r * a.row13 * 16;
    char* dst = static_cast<char*>(a.d13.p[q]) + drow * a.row13 * 16;
    for (int c0 = 0; c0 < a.row13; c0 += RP_STEP) {
      u32x4_t v[RP_U];
#pragma unroll
      for (int u = 0; u < RP_U; ++u) {
        const int c = c0 + u * WAVE + l;
        if (c < a.row13) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + c * 16));
      }
#pragma unroll
      for (int u = 0; u < RP_U; ++u) {
        const int c = c0 + u * WAVE + l;
        if (c < a.row13) __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4_t*>(dst + c * 16));
      }
    }
  }

  // ---- W2: row r, chunk c -> block q = c / seg2, offset r*seg2 + c%seg2
  for (int c0 = 0; c0 < a.row2; c0 += RP_STEP) {
    char* dbase[RP_U];
    int dcol[RP_U];
#pragma unroll
    for (int u = 0; u < RP_U; ++u) {
      const int c = c0 + u * WAVE + l;
      const int q = c < a.row2 ? c / a.seg2 : 0;
      dbase[u] = static_cast<char*>(a.d2.p[q]);
      dcol[u] = c - q * a.seg2;
    }
    for (long long r = w0; r < a.rows2; r += nw) {
      const char* src = a.w2 + r * a.row2 * 16;
      u32x4_t v[RP_U];
#pragma unroll
      for (int u = 0; u < RP_U; ++u) {
        const int c = c0 + u * WAVE + l;
        if (c < a.row2) v[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(src + c * 16));
      }
#pragma unroll
      for (int u = 0; u < RP_U; ++u) {
        const int c = c0 + u * WAVE + l;
        if (c < a.row2)
          __builtin_nontemporal_store(v[u], reinterpret_cast<u32x4_t*>(dbase[u] + (r * a.seg2 + dcol[u]) * 16));
      }
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
  a.rows13 = static_cast<long long>(E_local) * 2 * I;
  a.rows2 = static_cast<long long>(E_local) * H;
  a.I = I;
  a.Ip = I / P;
  a.seg2 = a.Ip * eb / 16;
  // Enough waves to keep every CU streaming, never more than there are rows.
  const long long rows = a.rows13 > a.rows2 ? a.rows13 : a.rows2;
  long long grid = static_cast<long long>(device_cu_count()) * 8;
  const long long need = (rows + RP_WAVES - 1) / RP_WAVES;
  if (grid > need) grid = need;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(repack_kernel, dim3(static_cast<unsigned>(grid)), dim3(RP_WAVES * WAVE), 0, s, a);
}

}  // namespace moe
