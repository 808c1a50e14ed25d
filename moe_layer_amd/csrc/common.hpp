// Device helpers shared by the MoE-layer kernels (gfx950 / CDNA4, wave64).
//
// Operand fragments.  Every contraction here has its K dimension contiguous
// in memory for both operands (weight rows and activation rows), so one lane
// loads one 16-byte chunk of a row straight into the register layout of a
// 16x16 MFMA: lane l holds row (l % 16), bytes [16*(l/16), 16*(l/16)+16) of a
// 64-byte K-chunk.  For bf16 that chunk is the 8 K-values the
// v_mfma_f32_16x16x32_bf16 operand wants from a lane; for fp32 it is four
// K-values consumed by four v_mfma_f32_16x16x4_f32 steps.  Both operands use
// the same byte->K mapping, so the K-sum is complete and exact in order-free
// terms.  The 16x16 fp32 result sits in lane l as rows 4*(l/16)+r, r = 0..3,
// column l % 16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int FRAG_BYTES = 64;  // bytes of K covered per row by one fragment step

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T>
struct Elem;

template <>
struct Elem<uint16_t> {  // bf16 storage
  static constexpr int bytes = 2;
  __device__ __forceinline__ static f32x4_t mma(uint4 a, uint4 b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ __forceinline__ static float load(const uint16_t* p) { return bf16_to_f32(*p); }
  // Store 4 consecutive values.
  __device__ __forceinline__ static void store4(uint16_t* p, float a, float b, float c, float d) {
    uint2 v;
    v.x = static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
    v.y = static_cast<uint32_t>(f32_to_bf16(c)) | (static_cast<uint32_t>(f32_to_bf16(d)) << 16);
    *reinterpret_cast<uint2*>(p) = v;
  }
};

template <>
struct Elem<float> {
  static constexpr int bytes = 4;
  __device__ __forceinline__ static f32x4_t mma(uint4 a, uint4 b, f32x4_t c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
  }
};

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// v if ok, else zeros; component-wise, so it stays a register select.
__device__ __forceinline__ uint4 keep_or_zero(bool ok, uint4 v) {
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

// Relaxed loads and stores at agent scope (global_load/store with sc1): they
// are coherent across the XCDs' separate L2 caches on their own, so data handed
// from one block to another inside a launch needs no whole-cache write-back or
// invalidate, only these accesses and a wait for the stores to complete.
template <typename V>
__device__ __forceinline__ V ld_agent(const V* p) {
  return __hip_atomic_load(const_cast<V*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ void st_agent(V* p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Arrival counter shared by the blocks of one launch: returns true, in every
// thread of the block, for the block that arrives n-th at *ctr, and that block
// resets the counter to zero.  Everything the arriving blocks stored with
// st_agent before the call is visible to ld_agent loads of the last block
// after it: each wave waits for its own stores to complete (vmcnt counts
// stores on gfx9) before the block barrier that precedes the atomic.
__device__ __forceinline__ bool last_to_arrive(int* ctr, int n, int* s_flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int old = atomicAdd(ctr, 1);
    const int last = old == n - 1;
    if (last) st_agent(ctr, 0);
    *s_flag = last;
  }
  __syncthreads();
  return *s_flag != 0;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

// Whether the LDS-tiled kernels take every group of the launch (else none),
// evaluated by one wave from the group sizes: the groups with more than m_min
// rows hold at least a quarter of all rows, and all groups together make at
// least min_tiles tiles of tile_rows token rows x n_nt weight tiles.  Under
// skewed routing the hot groups then read each weight tile once per 128
// rows, and the small groups ride along in the same launch instead of a
// second one (Qwen3-235B EP share, Zipf routing, step B = 512 208 -> 158 us,
// B = 1024 238 -> 177 us; TP share B = 1024 272 -> 201 us).  Under uniform
// routing at B = 512 (groups of 33-64 rows, m_min = 64) no group qualifies
// and the wave-streaming kernel's 64-row passes stay faster; from B = 1024
// every group holds more than 32 rows.  Lane-uniform result.
__device__ __forceinline__ bool tile_take_all(const int* __restrict__ offsets, int n_groups, int m_min,
                                              int min_tiles, int tile_rows, int n_nt) {
  int tiles = 0, rows = 0, hot = 0;
  for (int g = lane_id(); g < n_groups; g += WAVE) {
    const int m = offsets[g + 1] - offsets[g];
    tiles += (m + tile_rows - 1) / tile_rows * n_nt;
    rows += m;
    if (m > m_min) hot += m;
  }
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    tiles += __shfl_xor(tiles, d, WAVE);
    rows += __shfl_xor(rows, d, WAVE);
    hot += __shfl_xor(hot, d, WAVE);
  }
  return hot > 0 && 4LL * hot >= rows && tiles >= min_tiles;
}

// Inclusive prefix sum over the 64 lanes of a wave (Hillis-Steele with shuffles).
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    int o = __shfl_up(v, d, WAVE);
    if (l >= d) v += o;
  }
  return v;
}

// Build, in LDS, the list of expert groups that received at least one pair and
// the number of such groups.  Run by wave 0 of the block; `list` must hold
// n_groups entries.  The list is in ascending group order.
__device__ __forceinline__ void touched_groups(const int* __restrict__ offsets, int n_groups,
                                               int* list, int* n_list) {
  if (threadIdx.x >= WAVE) return;
  const int l = lane_id();
  int base = 0;
  for (int g0 = 0; g0 < n_groups; g0 += WAVE) {
    const int g = g0 + l;
    int used = 0;
    if (g < n_groups) used = (offsets[g + 1] - offsets[g]) > 0;
    const int incl = wave_inclusive_scan(used);
    if (used) list[base + incl - 1] = g;
    base += __shfl(incl, WAVE - 1, WAVE);
  }
  if (l == 0) *n_list = base;
}

}  // namespace moe
