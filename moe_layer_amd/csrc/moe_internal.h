// Internal launcher interface between the C-ABI layer (moe_api.hip) and the
// kernel files.  Every launcher assumes its arguments were validated by the
// C-ABI layer and only enqueues work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Limits shared by the host checks and the kernels.
constexpr int MAX_GROUPS = 512;   // expert groups per call (LDS tables)
constexpr int MAX_E = 512;        // routed experts in the gate (16 logits per top-k lane)
constexpr int MAX_K = 32;         // routed picks per token
constexpr int MAX_KK = 64;        // routed + shared slots per token
constexpr int MAX_P = 64;         // peers in a repack

// Compute units of the current device (queried on every call).
int device_cu_count();
// Blocks of `threads` threads of `kernel` resident on one compute unit (at
// least 1).  It depends only on the code object, so launchers keep it in a
// function-local constant: initialised once (thread-safely, as C++ does for
// such statics) and never written again.
int kernel_blocks_per_cu(const void* kernel, int threads);

// gate GEMM + softmax + top-k (+ renorm, + shared slots) in one launch, and,
// when `counts` is non-null, the stable permutation of the pairs as well.
// ws: route_workspace_bytes() bytes whose counter head is zero on entry (and
// is left zero).
size_t route_workspace_bytes(int T, int H, int E, int dtype);
// whether the launch grid of these sizes has a 32-bit block count
bool route_fits(int T, int H, int E, int dtype);
// The allocation-free routing: the workspace is a fixed device array of
// ROUTE_SCRATCH_BYTES per GPU (route.hip) whose counter head is cleared on
// the stream before the launch.  Needs route_workspace_bytes(T, H, E, dtype)
// <= ROUTE_SCRATCH_BYTES (checked by the caller).  Returns 0, or 1 when the
// array's device address could not be found (nothing was enqueued).
constexpr size_t ROUTE_SCRATCH_BYTES = size_t(16) << 20;
int launch_route_permute_scratch(int dtype, const void* x, const void* wg, const float* bias, float* logits,
                                 int32_t* ids, float* w, int T, int H, int E, int k, int renorm,
                                 int n_shared, int g_begin, int n_groups, int32_t* counts, int32_t* offsets,
                                 int32_t* sorted_pair, int32_t* pair_pos, hipStream_t s);
void launch_route(int dtype, const void* x, const void* wg, const float* bias, float* logits,
                  int32_t* ids, float* w, int T, int H, int E, int k, int renorm, int n_shared,
                  void* ws, int g_begin, int n_groups, int32_t* counts, int32_t* offsets,
                  int32_t* sorted_pair, int32_t* pair_pos, hipStream_t s);
// counts, offsets, stable permutation: one block up to PERM_ONE_BLOCK_MAX
// pairs, above that one block per segment of pairs (permute_uses_blocks)
constexpr long long PERM_ONE_BLOCK_MAX = 4096;
bool permute_uses_blocks(int T, int kk);
void launch_permute(const int32_t* ids, int T, int kk, int g_begin, int n_groups, int32_t* counts,
                    int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, hipStream_t s);
// EP dispatch: pairs by owning rank ids / E_local (< P), then the send rows
// send_x[i] = x[send_order[i] / kk] and send_ids[i] = ids[send_order[i]]
void launch_dispatch(int dtype, const void* x, const int32_t* ids, int T, int kk, int H, int E_local,
                     int P, int32_t* counts, int32_t* offsets, int32_t* send_order, int32_t* pair_pos,
                     void* send_x, int32_t* send_ids, hipStream_t s);
// expert GEMM workspace (one layout for the up and the down launch): split-item
// counters + per-wave partials
size_t expert_workspace_bytes(int T, int kk, int n_groups, int H, int I, int dtype);
// whether every work item of these sizes has a 32-bit index
bool expert_items_fit(int T, int kk, int n_groups, int H, int I, int dtype);
// expert up-projection with SiLU(gate)*up epilogue -> A (n_pairs, I)
void launch_expert_up(int dtype, const void* x, const int32_t* sorted_pair, const int32_t* offsets,
                      int n_groups, int T, int kk, const void* w13, int H, int I, void* a, void* ws,
                      hipStream_t s);
// expert down-projection -> y_pair (n_pairs, H)
void launch_expert_down(int dtype, const void* a, const int32_t* offsets, int n_groups, int T,
                        int kk, const void* w2, int H, int I, void* y_pair, void* ws, hipStream_t s);
// LDS-tiled expert kernels (expert_tile.hip) for groups holding many rows:
// for bf16 and T > TILE_T_MIN, launch_expert_up/down first launch them (the
// down-projection not for W2 rows of at most 512 bytes, which the short-row
// kernel of expert_short.hip takes whole).  They take every group of the
// launch when the groups with more than m_min sorted rows (TILE_M_MIN, or
// TILE_M_MIN_WIDE when the wave-streaming kernel holds four token tiles and
// takes up to 64 rows in one pass) hold at least a quarter of the rows, and
// all groups make at least expert_tile_min_tiles(m_min) tiles of TILE_ROWS
// token rows x (up: 64 intermediate columns; down: 128 output features);
// otherwise none, and the wave-streaming kernel takes every group.  Both
// kernels take this decision on the device, from the same counts and the
// same formula (tile_take_all in common.hpp).
constexpr int TILE_M_MIN = 32;
constexpr int TILE_M_MIN_WIDE = 64;
constexpr int TILE_T_MIN = 256;
// From this many tokens on the LDS-tiled kernels take every group (m_min =
// -1 forces tile_take_all) and no wave-streaming launch follows them: at
// these batches the rule above already hands them every group of the
// workloads measured here, and the streaming launch cost ~4.5 us for nothing.
constexpr int TILE_ONLY_T = 1024;
constexpr int TILE_ROWS = 128;
inline int expert_tile_nt(bool up, int H, int I) { return up ? (I + 63) / 64 : (H + 127) / 128; }
int expert_tile_min_tiles(int m_min);
// The row threshold of the LDS-tiled kernels for this launch (both kernels use it).
int expert_tile_m_min(int T, int kk, int n_groups);
bool expert_tile_used(int T, int dtype);
// Their workspace (split-tile counters, zero between calls, then fp32
// partial tiles) follows the wave-streaming kernel's in the expert workspace.
size_t expert_tile_workspace_bytes(int T, int kk, int n_groups, int H, int I, int dtype);
void launch_expert_up_tiles(const void* x, const int32_t* sorted_pair, const int32_t* offsets, int n_groups,
                            int T, int kk, const void* w13, int H, int I, void* a, int m_min, void* ws,
                            hipStream_t s);
void launch_expert_down_tiles(const void* a, const int32_t* offsets, int n_groups, int T, int kk,
                              const void* w2, int H, int I, void* y_pair, int m_min, void* ws, hipStream_t s);
// weighted combine -> y (T, H); w == nullptr: every weight 1
void launch_combine(int dtype, const void* y_pair, const int32_t* pair_pos, const float* w, int T,
                    int kk, int H, void* y, hipStream_t s);

// Attention-DP request scheduling: per-request cluster counts, argmax rank,
// and ranks balanced over groups of E consecutive requests (E <= 64).
constexpr int MAX_SCHED_RANKS = 64;
size_t schedule_workspace_bytes(int n_req, int E);
void launch_schedule(const int32_t* tokens, int n_tokens, const int32_t* offsets, int n_req,
                     const int32_t* cluster, int vocab, int E, int32_t* scores, int32_t* affinity,
                     int32_t* assigned, void* ws, hipStream_t s);

struct PeerPtrs {
  void* p[MAX_P];
};
// EP -> TP local permute of expert weights into P per-peer blocks (whether
// its 32-bit unit indexing covers these sizes)
bool repack_fits(int E_local, int H, int I, int dtype);
void launch_repack_ep_to_tp(int dtype, const void* w13, const void* w2, int E_local, int H, int I,
                            int P, const PeerPtrs& d13, const PeerPtrs& d2, hipStream_t s);
// TP -> EP: gather the P blocks back into whole experts (exact inverse)
void launch_repack_tp_to_ep(int dtype, const PeerPtrs& s13, const PeerPtrs& s2, int E_local, int H, int I, int P,
                            void* w13, void* w2, hipStream_t s);

}  // namespace moe
