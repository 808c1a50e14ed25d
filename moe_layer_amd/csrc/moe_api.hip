// The exported C ABI (declared in include/moe.h): host-side argument checks,
// then the launches.  Nothing here allocates, frees or synchronises.
#include "moe.h"
#include "moe_internal.h"

namespace moe {

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  return n;
}

int kernel_blocks_per_cu(const void* kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1) n = 1;
  return n;
}

}  // namespace moe

using namespace moe;

namespace {

constexpr int ABI_VERSION = 8;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
int elem_bytes(int dtype) { return dtype == MOE_DTYPE_BF16 ? 2 : 4; }
bool dtype_ok(int dtype) { return dtype == MOE_DTYPE_F32 || dtype == MOE_DTYPE_BF16; }

// A contraction length the fragment kernels take: whole 64-byte K fragments
// (rows of at most 1 MiB).
bool k_len_ok(int K, int dtype) {
  const long long b = static_cast<long long>(K) * elem_bytes(dtype);
  return b % 64 == 0 && b <= (1LL << 20);
}

int launched() { return hipGetLastError() == hipSuccess ? MOE_OK : MOE_EHIP; }

int check_gemm_shapes(int T, int kk, int n_groups, int H, int I, int dtype) {
  if (T < 0 || kk < 1 || kk > MAX_KK || n_groups < 1 || H < 1 || I < 1 || !dtype_ok(dtype))
    return MOE_EINVAL;
  if (n_groups > MAX_GROUPS) return MOE_EUNSUPPORTED;
  if (!k_len_ok(H, dtype) || H % 16 != 0) return MOE_EUNSUPPORTED;
  if (!k_len_ok(I, dtype) || I % 8 != 0) return MOE_EUNSUPPORTED;
  if (static_cast<long long>(T) * kk > (1LL << 30)) return MOE_EUNSUPPORTED;
  if (!expert_items_fit(T, kk, n_groups, H, I, dtype)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return ABI_VERSION; }

const char* moe_status_str(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK: success";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument (null or misaligned pointer, bad dimension)";
    case MOE_EUNSUPPORTED: return "MOE_EUNSUPPORTED: shape outside the kernels' tiling limits";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace missing or too small";
    case MOE_EHIP: return "MOE_EHIP: HIP kernel launch failed";
    default: return "unknown moe status";
  }
}

size_t moe_workspace_bytes(int op, int T, int kk, int n_groups, int H, int I, int dtype) {
  if (T <= 0 || kk <= 0 || n_groups <= 0 || H <= 0 || I <= 0 || !dtype_ok(dtype)) return 0;
  const size_t sk = expert_workspace_bytes(T, kk, n_groups, H, I, dtype);
  switch (op) {
    case MOE_OP_EXPERT_UP:
    case MOE_OP_EXPERT_DOWN: return sk;
    case MOE_OP_GROUPED_GEMM: {
      // a, then the region both halves use in turn (each leaves its counters zero)
      const size_t a = (static_cast<size_t>(T) * kk * I * elem_bytes(dtype) + 255) & ~static_cast<size_t>(255);
      return a + sk;
    }
    default: return 0;
  }
}

size_t moe_route_workspace_bytes(int T, int H, int E, int dtype) {
  if (T <= 0 || H <= 0 || E <= 0 || !dtype_ok(dtype)) return 0;
  return route_workspace_bytes(T, H, E, dtype);
}

namespace {

int check_route(const void* x, const void* w_gate, const float* gate_bias, int T, int H, int E, int k,
                int n_shared, int dtype, float* logits, int32_t* topk_ids, float* topk_w, void* ws,
                size_t ws_bytes) {
  if (T < 0 || H < 1 || E < 1 || k < 1 || n_shared < 0 || k > E || !dtype_ok(dtype)) return MOE_EINVAL;
  if (E > MAX_E || k > MAX_K || k + n_shared > MAX_KK || !k_len_ok(H, dtype)) return MOE_EUNSUPPORTED;
  // pair indices and the sort length are 32-bit; so is the launch grid
  if (static_cast<long long>(T) * (k + n_shared) > (1LL << 30) || !route_fits(T, H, E, dtype))
    return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w_gate || !logits || !topk_ids || !topk_w) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned4(logits) || !aligned4(topk_ids) ||
      !aligned4(topk_w) || (gate_bias && !aligned4(gate_bias)))
    return MOE_EINVAL;
  if (!ws || !aligned16(ws) || ws_bytes < route_workspace_bytes(T, H, E, dtype)) return MOE_EWORKSPACE;
  return MOE_OK;
}

}  // namespace

int moe_route(const void* x, const void* w_gate, const float* gate_bias, int T, int H, int E, int k,
              int renorm, int n_shared, int dtype, float* logits, int32_t* topk_ids, float* topk_w,
              void* ws, size_t ws_bytes, hipStream_t stream) {
  const int st = check_route(x, w_gate, gate_bias, T, H, E, k, n_shared, dtype, logits, topk_ids, topk_w,
                             ws, ws_bytes);
  if (st != MOE_OK || T == 0) return st;
  launch_route(dtype, x, w_gate, gate_bias, logits, topk_ids, topk_w, T, H, E, k, renorm ? 1 : 0,
               n_shared, ws, 0, 1, nullptr, nullptr, nullptr, nullptr, stream);
  return launched();
}

int moe_route_permute(const void* x, const void* w_gate, const float* gate_bias, int T, int H, int E,
                      int k, int renorm, int n_shared, int dtype, float* logits, int32_t* topk_ids,
                      float* topk_w, int g_begin, int n_groups, int32_t* counts, int32_t* offsets,
                      int32_t* sorted_pair, int32_t* pair_pos, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  int st = check_route(x, w_gate, gate_bias, T, H, E, k, n_shared, dtype, logits, topk_ids, topk_w, ws,
                       ws_bytes);
  if (st != MOE_OK) return st;
  if (g_begin < 0 || n_groups < 1) return MOE_EINVAL;
  if (n_groups > MAX_GROUPS) return MOE_EUNSUPPORTED;
  if (!counts || !offsets || !aligned4(counts) || !aligned4(offsets)) return MOE_EINVAL;
  if (T > 0 && (!sorted_pair || !pair_pos || !aligned4(sorted_pair) || !aligned4(pair_pos)))
    return MOE_EINVAL;
  if (T == 0) {
    // nothing is routed: the counts and offsets of an empty batch
    launch_permute(topk_ids, 0, k + n_shared, g_begin, n_groups, counts, offsets, sorted_pair,
                   pair_pos, stream);
    return launched();
  }
  launch_route(dtype, x, w_gate, gate_bias, logits, topk_ids, topk_w, T, H, E, k, renorm ? 1 : 0,
               n_shared, ws, g_begin, n_groups, counts, offsets, sorted_pair, pair_pos, stream);
  return launched();
}

int moe_route_permute_noalloc(const void* x, const void* w_gate, const float* gate_bias, int T, int H, int E,
                              int k, int renorm, int n_shared, int dtype, float* logits, int32_t* topk_ids,
                              float* topk_w, int g_begin, int n_groups, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_pair, int32_t* pair_pos, hipStream_t stream) {
  // The checks of moe_route_permute, with the fixed scratch standing in for
  // the workspace: its size limit is the scratch size (MOE_EWORKSPACE above).
  int st = check_route(x, w_gate, gate_bias, T, H, E, k, n_shared, dtype, logits, topk_ids, topk_w,
                       reinterpret_cast<void*>(256), ~size_t(0));
  if (st != MOE_OK) return st;
  if (T > 0 && route_workspace_bytes(T, H, E, dtype) > ROUTE_SCRATCH_BYTES) return MOE_EWORKSPACE;
  if (g_begin < 0 || n_groups < 1) return MOE_EINVAL;
  if (n_groups > MAX_GROUPS) return MOE_EUNSUPPORTED;
  if (!counts || !offsets || !aligned4(counts) || !aligned4(offsets)) return MOE_EINVAL;
  if (T > 0 && (!sorted_pair || !pair_pos || !aligned4(sorted_pair) || !aligned4(pair_pos)))
    return MOE_EINVAL;
  if (T == 0) {
    launch_permute(topk_ids, 0, k + n_shared, g_begin, n_groups, counts, offsets, sorted_pair,
                   pair_pos, stream);
    return launched();
  }
  if (launch_route_permute_scratch(dtype, x, w_gate, gate_bias, logits, topk_ids, topk_w, T, H, E, k,
                                   renorm ? 1 : 0, n_shared, g_begin, n_groups, counts, offsets, sorted_pair,
                                   pair_pos, stream) != 0)
    return MOE_EHIP;
  return launched();
}

int moe_permute(const int32_t* topk_ids, int T, int kk, int g_begin, int n_groups, int32_t* counts,
                int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, hipStream_t stream) {
  if (T < 0 || kk < 1 || kk > MAX_KK || g_begin < 0 || n_groups < 1) return MOE_EINVAL;
  if (n_groups > MAX_GROUPS || static_cast<long long>(T) * kk > (1LL << 30)) return MOE_EUNSUPPORTED;
  if (!counts || !offsets || !aligned4(counts) || !aligned4(offsets)) return MOE_EINVAL;
  if (T > 0 && (!topk_ids || !sorted_pair || !pair_pos || !aligned4(topk_ids) ||
                !aligned4(sorted_pair) || !aligned4(pair_pos)))
    return MOE_EINVAL;
  launch_permute(topk_ids, T, kk, g_begin, n_groups, counts, offsets, sorted_pair, pair_pos, stream);
  return launched();
}

int moe_expert_up(const void* x, const int32_t* sorted_pair, const int32_t* offsets, int T, int kk,
                  int n_groups, const void* w13, int H, int I, int dtype, void* a, void* ws,
                  size_t ws_bytes, hipStream_t stream) {
  const int st = check_gemm_shapes(T, kk, n_groups, H, I, dtype);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !sorted_pair || !offsets || !w13 || !a) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(w13) || !aligned16(a) || !aligned4(sorted_pair) || !aligned4(offsets))
    return MOE_EINVAL;
  if (!ws || !aligned16(ws) || ws_bytes < moe_workspace_bytes(MOE_OP_EXPERT_UP, T, kk, n_groups, H, I, dtype))
    return MOE_EWORKSPACE;
  launch_expert_up(dtype, x, sorted_pair, offsets, n_groups, T, kk, w13, H, I, a, ws, stream);
  return launched();
}

int moe_expert_down(const void* a, const int32_t* offsets, int T, int kk, int n_groups,
                    const void* w2, int H, int I, int dtype, void* y_pair, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  const int st = check_gemm_shapes(T, kk, n_groups, H, I, dtype);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!a || !offsets || !w2 || !y_pair) return MOE_EINVAL;
  if (!aligned16(a) || !aligned16(w2) || !aligned16(y_pair) || !aligned4(offsets)) return MOE_EINVAL;
  if (!ws || !aligned16(ws) ||
      ws_bytes < moe_workspace_bytes(MOE_OP_EXPERT_DOWN, T, kk, n_groups, H, I, dtype))
    return MOE_EWORKSPACE;
  launch_expert_down(dtype, a, offsets, n_groups, T, kk, w2, H, I, y_pair, ws, stream);
  return launched();
}

int moe_grouped_gemm(const void* x, const int32_t* sorted_pair, const int32_t* offsets, int T, int kk,
                     int n_groups, const void* w13, const void* w2, int H, int I, int dtype,
                     void* y_pair, void* ws, size_t ws_bytes, hipStream_t stream) {
  const int st = check_gemm_shapes(T, kk, n_groups, H, I, dtype);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  if (!x || !sorted_pair || !offsets || !w13 || !w2 || !y_pair) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(w13) || !aligned16(w2) || !aligned16(y_pair) ||
      !aligned4(sorted_pair) || !aligned4(offsets))
    return MOE_EINVAL;
  if (!ws || !aligned16(ws) || ws_bytes < moe_workspace_bytes(MOE_OP_GROUPED_GEMM, T, kk, n_groups, H, I, dtype))
    return MOE_EWORKSPACE;
  const size_t a_bytes = (static_cast<size_t>(T) * kk * I * elem_bytes(dtype) + 255) & ~static_cast<size_t>(255);
  void* sk = static_cast<char*>(ws) + a_bytes;
  launch_expert_up(dtype, x, sorted_pair, offsets, n_groups, T, kk, w13, H, I, ws, sk, stream);
  launch_expert_down(dtype, ws, offsets, n_groups, T, kk, w2, H, I, y_pair, sk, stream);
  return launched();
}

int moe_combine(const void* y_pair, const int32_t* pair_pos, const float* topk_w, int T, int kk, int H,
                int dtype, void* y, hipStream_t stream) {
  if (T < 0 || kk < 1 || kk > MAX_KK || H < 1 || !dtype_ok(dtype)) return MOE_EINVAL;
  if ((static_cast<long long>(H) * elem_bytes(dtype)) % 16 != 0) return MOE_EUNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y_pair || !pair_pos || !y) return MOE_EINVAL;
  if (!aligned16(y_pair) || !aligned16(y) || !aligned4(pair_pos) || (topk_w && !aligned4(topk_w)))
    return MOE_EINVAL;
  launch_combine(dtype, y_pair, pair_pos, topk_w, T, kk, H, y, stream);
  return launched();
}

size_t moe_schedule_workspace_bytes(int n_req, int E) { return schedule_workspace_bytes(n_req, E); }

int moe_schedule_requests(const int32_t* tokens, int n_tokens, const int32_t* req_offsets, int n_req,
                          const int32_t* cluster_of_token, int vocab, int E, int32_t* scores,
                          int32_t* affinity, int32_t* assigned, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  if (n_tokens < 0 || n_req < 0 || vocab < 1 || E < 1) return MOE_EINVAL;
  if (E > MAX_SCHED_RANKS || static_cast<long long>(n_req) * E > (1LL << 31) - 1) return MOE_EUNSUPPORTED;
  if (n_tokens >= (1 << 25)) return MOE_EUNSUPPORTED;   // counts must stay below 2^25
  if (n_req == 0) return MOE_OK;
  if (!req_offsets || !cluster_of_token || !scores || !affinity || !assigned || (n_tokens > 0 && !tokens))
    return MOE_EINVAL;
  if (!aligned4(req_offsets) || !aligned4(cluster_of_token) || !aligned4(scores) || !aligned4(affinity) ||
      !aligned4(assigned) || (tokens && !aligned4(tokens)))
    return MOE_EINVAL;
  if (!ws || !aligned4(ws) || ws_bytes < schedule_workspace_bytes(n_req, E)) return MOE_EWORKSPACE;
  launch_schedule(tokens, n_tokens, req_offsets, n_req, cluster_of_token, vocab, E, scores, affinity,
                  assigned, ws, stream);
  return launched();
}

int moe_dispatch(const void* x, const int32_t* topk_ids, int T, int kk, int H, int E_local, int P,
                 int dtype, int32_t* send_counts, int32_t* send_offsets, int32_t* send_order,
                 int32_t* pair_pos, void* send_x, int32_t* send_ids, hipStream_t stream) {
  if (T < 0 || kk < 1 || kk > MAX_KK || H < 1 || E_local < 1 || P < 1 || !dtype_ok(dtype))
    return MOE_EINVAL;
  if (P > MAX_GROUPS || static_cast<long long>(T) * kk > (1LL << 30)) return MOE_EUNSUPPORTED;
  if (static_cast<long long>(P) * E_local > (1LL << 31)) return MOE_EUNSUPPORTED;
  if ((static_cast<long long>(H) * elem_bytes(dtype)) % 16 != 0) return MOE_EUNSUPPORTED;
  if (static_cast<long long>(H) * elem_bytes(dtype) / 16 > (1LL << 30)) return MOE_EUNSUPPORTED;
  if (!send_counts || !send_offsets || !aligned4(send_counts) || !aligned4(send_offsets)) return MOE_EINVAL;
  if (T > 0 && (!x || !topk_ids || !send_order || !pair_pos || !send_x || !send_ids || !aligned16(x) ||
                !aligned16(send_x) || !aligned16(topk_ids) || !aligned4(send_order) ||
                !aligned4(pair_pos) || !aligned4(send_ids)))
    return MOE_EINVAL;
  launch_dispatch(dtype, x, topk_ids, T, kk, H, E_local, P, send_counts, send_offsets, send_order,
                  pair_pos, send_x, send_ids, stream);
  return launched();
}

namespace {

int check_repack(int E_local, int H, int I, int P, int dtype) {
  if (E_local < 1 || H < 1 || I < 1 || P < 1 || !dtype_ok(dtype)) return MOE_EINVAL;
  if (I % P != 0) return MOE_EINVAL;
  if (P > MAX_P) return MOE_EUNSUPPORTED;
  const int eb = elem_bytes(dtype);
  if ((static_cast<long long>(I / P) * eb) % 16 != 0 || (static_cast<long long>(H) * eb) % 16 != 0)
    return MOE_EUNSUPPORTED;
  if (!repack_fits(E_local, H, I, dtype)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

int gather_blocks(int P, void* const* p13, void* const* p2, PeerPtrs& b13, PeerPtrs& b2) {
  if (!p13 || !p2) return MOE_EINVAL;
  for (int q = 0; q < P; ++q) {
    if (!p13[q] || !p2[q] || !aligned16(p13[q]) || !aligned16(p2[q])) return MOE_EINVAL;
    b13.p[q] = p13[q];
    b2.p[q] = p2[q];
  }
  return MOE_OK;
}

}  // namespace

int moe_repack_ep_to_tp(const void* w13_ep, const void* w2_ep, int E_local, int H, int I, int P,
                        int dtype, void* const* dst13, void* const* dst2, hipStream_t stream) {
  int st = check_repack(E_local, H, I, P, dtype);
  if (st != MOE_OK) return st;
  if (!w13_ep || !w2_ep || !aligned16(w13_ep) || !aligned16(w2_ep)) return MOE_EINVAL;
  PeerPtrs d13{}, d2{};
  st = gather_blocks(P, dst13, dst2, d13, d2);
  if (st != MOE_OK) return st;
  launch_repack_ep_to_tp(dtype, w13_ep, w2_ep, E_local, H, I, P, d13, d2, stream);
  return launched();
}

int moe_repack_tp_to_ep(const void* const* src13, const void* const* src2, int E_local, int H, int I, int P,
                        int dtype, void* w13_ep, void* w2_ep, hipStream_t stream) {
  int st = check_repack(E_local, H, I, P, dtype);
  if (st != MOE_OK) return st;
  if (!w13_ep || !w2_ep || !aligned16(w13_ep) || !aligned16(w2_ep)) return MOE_EINVAL;
  PeerPtrs s13{}, s2{};
  st = gather_blocks(P, const_cast<void* const*>(src13), const_cast<void* const*>(src2), s13, s2);
  if (st != MOE_OK) return st;
  launch_repack_tp_to_ep(dtype, s13, s2, E_local, H, I, P, w13_ep, w2_ep, stream);
  return launched();
}

}  // extern "C"
