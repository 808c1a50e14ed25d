/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE-layer forward-pass library.
 *
 * One MoE layer on one GPU's share of the work, in the views of the Moebius
 * review (§2.1 and §3.1 weight resharding):
 *   full view : all E routed experts (+ shared experts) held whole;
 *   EP view   : this rank holds E/P whole experts, W13 (E/P, 2I, H), W2 (E/P, H, I);
 *   TP view   : this rank holds slice S_p of every expert, W13 (E, 2I/P, H),
 *               W2 (E, H, I/P); the output is the partial before the all-reduce.
 * The pass is: gate GEMM, softmax, top-k (moe_route); argsort of the
 * (token, slot) pairs by expert (moe_permute); the expert FFN
 * W2 (silu(W1 x) * W3 x) on every kept pair (moe_grouped_gemm); the weighted
 * sum per token (moe_combine).  moe_repack_ep_to_tp is the local-permute phase
 * of the EP->TP weight reshard.  moe_dispatch packs an EP rank's routed
 * token rows by destination rank (the all-to-all send layout); moe_combine
 * un-permutes and sums what comes back.
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns every
 *     buffer; the library never allocates or frees and only enqueues work on
 *     `stream` (no host synchronisation).  It keeps no data between calls:
 *     the compute-unit count is queried on every call, and each kernel's
 *     resident blocks per compute unit (a property of the code object) is a
 *     constant set once, thread-safely, on first use.  Calls are reentrant
 *     when they do not share a workspace, and graph-capturable.
 *   - dtype: MOE_DTYPE_F32 or MOE_DTYPE_BF16 is the storage type of activations
 *     and weights (bf16 = raw bfloat16 bits).  Accumulation is always fp32;
 *     bf16 results are rounded to nearest even.
 *   - Row-major, densely packed tensors; every tensor pointer 16-byte aligned.
 *   - Arguments are checked on the host before anything is enqueued.  On a
 *     non-zero return nothing was enqueued (MOE_EHIP: the launch itself failed)
 *     and outputs are unspecified.  Inputs must be finite.
 *   - T == 0 is valid: moe_permute still writes zero counts and offsets; the
 *     other calls do nothing.
 */
#ifndef MOE_LAYER_AMD_MOE_H
#define MOE_LAYER_AMD_MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = 1,        /* null / misaligned pointer, bad dimension, k > E, I % P != 0 ... */
  MOE_EUNSUPPORTED = 2,  /* shape outside the kernels' tiling limits (see each call) */
  MOE_EWORKSPACE = 3,    /* workspace missing or smaller than moe_workspace_bytes() */
  MOE_EHIP = 4           /* the HIP launch reported an error */
};

enum moe_dtype { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 };

enum moe_op { MOE_OP_ROUTE = 0, MOE_OP_PERMUTE = 1, MOE_OP_GROUPED_GEMM = 2, MOE_OP_COMBINE = 3,
              MOE_OP_REPACK = 4, MOE_OP_EXPERT_UP = 5, MOE_OP_EXPERT_DOWN = 6 };

/* Version of this ABI (incremented on any signature change). */
int moe_abi_version(void);

/* Human-readable text for a status code (static storage). */
const char* moe_status_str(int status);

/* Workspace bytes `op` needs for these sizes (0 if none).  The sizes depend
 * only on the arguments, not on the device.
 *   MOE_OP_EXPERT_UP / MOE_OP_EXPERT_DOWN: the expert GEMMs' split-item
 *     counters and per-wave fp32 partial tiles; both ops have the same size
 *     and layout, so one buffer serves the up and the down call in turn.
 *     Zero-fill the buffer before its first use; every completed call leaves
 *     the counters zero again, so the buffer serves any later call with
 *     sizes it was allocated for.
 *   MOE_OP_GROUPED_GEMM: the (T*kk, I) intermediate activations
 *     silu(W1 x) * W3 x in the storage dtype (256-byte aligned), followed by
 *     the region above (same zero-fill rule).
 * (Routing: moe_route_workspace_bytes.) */
size_t moe_workspace_bytes(int op, int T, int kk, int n_groups, int H, int I, int dtype);

/* Workspace bytes moe_route and moe_route_permute need for T tokens, hidden
 * size H and E routed experts (per-token-tile counters, then K-slice partial
 * logits).  The buffer must be zero-filled before its first use; every
 * completed call leaves its counter head zero again, so the same buffer can
 * be reused call after call.  Calls sharing one buffer must be ordered (one
 * stream, or synchronised streams). */
size_t moe_route_workspace_bytes(int T, int H, int E, int dtype);

/*
 * moe_route -- gate GEMM, softmax and top-k in one launch (Sem-MoE notes,
 * Key design 1: G(h) = top-k(softmax(W_g h + b_g))).
 *   x          (T, H) dtype          token activations
 *   w_gate     (E, H) dtype          gate matrix
 *   gate_bias  (E) fp32, nullable    added to the logits before softmax and top-k
 *   logits     (T, E) fp32 [out]     x . w_gate^T + b
 *   topk_ids   (T, k + n_shared) int32 [out]  routed ids in descending logit
 *              order, ties to the lower id; then shared experts E, E+1, ...
 *   topk_w     (T, k + n_shared) fp32 [out]   softmax over all E routed experts
 *              at the picked ids; if renorm != 0, divided by their sum over the
 *              k picks; shared slots weigh 1.
 *   ws         >= moe_route_workspace_bytes(T, H, E, dtype) bytes (see above)
 * Limits: 1 <= E <= 512; 1 <= k <= min(E, 32); k + n_shared <= 64;
 * T * (k + n_shared) <= 2^30; H * sizeof(dtype) a multiple of 64
 * (MOE_EUNSUPPORTED).
 */
int moe_route(const void* x, const void* w_gate, const float* gate_bias, int T, int H, int E, int k,
              int renorm, int n_shared, int dtype, float* logits, int32_t* topk_ids, float* topk_w,
              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_route_permute -- moe_route followed by moe_permute of its ids.  Up to
 * 4096 pairs (T*(k+n_shared)) this is one launch: the last block to finish
 * the routing sorts the pairs.  Above that the routing launch is followed by
 * moe_permute's own launches on the same stream.  Arguments and outputs are
 * those of the two calls; the same workspace rules as moe_route apply.
 */
int moe_route_permute(const void* x, const void* w_gate, const float* gate_bias, int T, int H, int E,
                      int k, int renorm, int n_shared, int dtype, float* logits, int32_t* topk_ids,
                      float* topk_w, int g_begin, int n_groups, int32_t* counts, int32_t* offsets,
                      int32_t* sorted_pair, int32_t* pair_pos, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/*
 * moe_route_permute_noalloc -- moe_route_permute without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  The
 * routing's scratch (per-token-tile counters, K-slice partial logits) is a
 * fixed 16 MiB device array inside the library, one copy per GPU, held until
 * the process ends; its address is looked up once per device.  Nothing is
 * allocated and no allocating routine is called.  Each call first clears the
 * counters it uses with a small fill kernel on `stream`, then runs the same
 * kernel as moe_route_permute, so its outputs are bit-identical to that
 * call's.  All calls on one GPU share the array: calls that overlap in time
 * (several streams or host threads) race on it and must be serialised by the
 * caller.  Arguments, outputs and limits are those of moe_route_permute;
 * shapes whose moe_route_workspace_bytes exceeds 16 MiB are rejected with
 * MOE_EWORKSPACE (every batch up to millions of tokens fits: the partial
 * logits never exceed about 8 MB), and a failed address lookup returns
 * MOE_EHIP with nothing enqueued.
 */
int moe_route_permute_noalloc(const void* x, const void* w_gate, const float* gate_bias, int T, int H, int E,
                              int k, int renorm, int n_shared, int dtype, float* logits, int32_t* topk_ids,
                              float* topk_w, int g_begin, int n_groups, int32_t* counts, int32_t* offsets,
                              int32_t* sorted_pair, int32_t* pair_pos, hipStream_t stream);

/*
 * moe_permute -- expert counts, offsets and the stable argsort of the
 * (token, slot) pairs by expert group (the token reorder of the Sem-MoE
 * notes, Key design 4).  Pair p = t*kk + j; its group is topk_ids[p] - g_begin
 * when that lies in [0, n_groups), otherwise the pair is not held here.
 *   topk_ids    (T, kk) int32
 *   counts      (n_groups) int32 [out]       pairs per group
 *   offsets     (n_groups + 1) int32 [out]   exclusive prefix sum; offsets[n_groups] = n_kept
 *   sorted_pair (T*kk) int32 [out]           first n_kept entries: pair ids in group
 *                                            order, ascending pair id within a group
 *   pair_pos    (T*kk) int32 [out]           row of each pair in sorted order, -1 if not held
 * Views: full / TP: g_begin = 0, n_groups = E + n_shared; EP rank r with
 * E_l = E/P local experts: g_begin = r*E_l, n_groups = E_l.
 * Limits: 1 <= kk <= 64; 1 <= n_groups <= 512.  Results are deterministic.
 * Above 65536 pairs the sort takes three launches and parks per-segment
 * group counts in pair_pos between them, so no output may overlap topk_ids
 * (true of every size) and pair_pos holds its final values only once the
 * call's work on `stream` has completed.
 */
int moe_permute(const int32_t* topk_ids, int T, int kk, int g_begin, int n_groups, int32_t* counts,
                int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, hipStream_t stream);

/*
 * moe_grouped_gemm -- the expert FFN on every held pair: for sorted row r of
 * group g (token t = sorted_pair[r] / kk)
 *     a[r]      = silu(W13[g][0:I] x_t) * (W13[g][I:2I] x_t),  silu(z) = z/(1+e^-z)
 *     y_pair[r] = W2[g] a[r]
 * (Moebius review, §3.1: W13 (., 2I, H) and W2 (., H, I); gate rows first.)
 *   x           (T, H) dtype
 *   sorted_pair, offsets   from moe_permute
 *   w13         (n_groups, 2I, H) dtype   I = this GPU's intermediate size (I/P in TP)
 *   w2          (n_groups, H, I) dtype
 *   y_pair      (T*kk, H) dtype [out]     first n_kept rows written.  Stored in
 *               the activation dtype, not fp32: each element is rounded once
 *               (RNE) from its fp32 sum.  In bf16 this adds at most 2^-9
 *               relative error per element before the combine; measured on
 *               the full-size workloads, the layer output y stays within
 *               rel-L2 3e-3 of the fp64 definition (bound: 5e-3), and it
 *               halves this intermediate's HBM write and read.
 *   ws          >= moe_workspace_bytes(MOE_OP_GROUPED_GEMM, ...) bytes, holds a
 *               and the split-item state; zero-filled before its first use
 * Limits: H * sizeof(dtype) and I * sizeof(dtype) multiples of 64; H % 16 == 0;
 * I % 8 == 0; n_groups <= 512.
 * a is rounded to dtype before the W2 product.
 */
int moe_grouped_gemm(const void* x, const int32_t* sorted_pair, const int32_t* offsets, int T, int kk,
                     int n_groups, const void* w13, const void* w2, int H, int I, int dtype,
                     void* y_pair, void* ws, size_t ws_bytes, hipStream_t stream);

/* The two halves of moe_grouped_gemm, for callers that keep `a` themselves.
 * moe_expert_up writes a (T*kk, I) dtype; moe_expert_down reads it.  Same
 * limits as moe_grouped_gemm.  ws: >= moe_workspace_bytes(MOE_OP_EXPERT_UP or
 * MOE_OP_EXPERT_DOWN, ...) bytes, 16-byte aligned, zero-filled before its
 * first use (each call leaves it reusable); calls sharing one ws must not
 * overlap in time.  Results are deterministic for given sizes on a given
 * device (the work split follows the number of compute units). */
int moe_expert_up(const void* x, const int32_t* sorted_pair, const int32_t* offsets, int T, int kk,
                  int n_groups, const void* w13, int H, int I, int dtype, void* a, void* ws,
                  size_t ws_bytes, hipStream_t stream);
int moe_expert_down(const void* a, const int32_t* offsets, int T, int kk, int n_groups,
                    const void* w2, int H, int I, int dtype, void* y_pair, void* ws, size_t ws_bytes,
                    hipStream_t stream);

/*
 * moe_combine -- y[t] = sum_{j=0..kk-1, in order, pair_pos[t*kk+j] >= 0}
 *                       topk_w[t*kk+j] * y_pair[pair_pos[t*kk+j]]
 * fp32 accumulation, one rounding to dtype; rows with no held pair are 0.
 * This is the EP rank's partial before the combine all-to-all, or the TP
 * rank's partial before the all-reduce (Moebius review, §2.1).  After
 * moe_dispatch it is the sender's sum of the rows that came back, with the
 * dispatch's pair_pos.
 *   y_pair (rows, H) dtype, every pair_pos entry < rows; pair_pos (T*kk)
 *   int32; topk_w (T*kk) fp32, or NULL for weight 1 on every slot (with
 *   kk = 1: the un-permute y[t] = y_pair[pair_pos[t]], an exact copy, which
 *   puts a receiver's expert outputs back in arrival order); y (T, H) dtype
 *   [out].   Limit: H * sizeof(dtype) a multiple of 16.
 */
int moe_combine(const void* y_pair, const int32_t* pair_pos, const float* topk_w, int T, int kk, int H,
                int dtype, void* y, hipStream_t stream);

/*
 * moe_dispatch -- send side of the EP token exchange (Moebius review, problem
 * definition: in the EP layout each token reaches the GPU holding its expert
 * by an all-to-all; Sem-MoE notes, motivation: one all-to-all out, one back).
 * This rank's T tokens with their routing (T, kk); rank d < P owns experts
 * [d E_local, (d+1) E_local).  Pair p = t*kk + j is sent to rank
 * topk_ids[p] / E_local when that is < P (ids at or past P*E_local, e.g.
 * shared experts, are not sent): one send row per pair, rank blocks in rank
 * order, ascending pair id inside a block (moe_permute with the rank as key).
 *   x           (T, H) dtype
 *   topk_ids    (T, kk) int32, 16-byte aligned (read as 16-byte vectors)
 *   send_counts (P) int32 [out]      rows for each rank
 *   send_offsets(P + 1) int32 [out]  exclusive prefix sum; [P] = n_sent
 *   send_order  (T*kk) int32 [out]   first n_sent: the pair id of each send row
 *   pair_pos    (T*kk) int32 [out]   send row of each pair, -1 if not sent
 *   send_x      (T*kk, H) dtype [out]  first n_sent rows: x[send_order[i] / kk],
 *                                      exact copies
 *   send_ids    (T*kk) int32 [out]   first n_sent: topk_ids[send_order[i]], the
 *                                    global expert id the receiver needs
 * Rank r's block is rows [send_offsets[r], send_offsets[r+1]).  A receiver
 * concatenates its blocks from ranks 0..P-1, runs moe_permute on the ids with
 * kk = 1, g_begin = r*E_local, n_groups = E_local, then moe_grouped_gemm, and
 * moe_combine(kk = 1, topk_w = NULL) to put its outputs back in arrival
 * order; the sender's moe_combine of the returned rows with this pair_pos and
 * its topk_w is its output.
 * Limits: 1 <= kk <= 64; 1 <= P <= 512; E_local >= 1; P * E_local <= 2^31;
 * H * sizeof(dtype) a multiple of 16.  T == 0 writes zero counts and offsets.
 * Deterministic.
 */
int moe_dispatch(const void* x, const int32_t* topk_ids, int T, int kk, int H, int E_local, int P,
                 int dtype, int32_t* send_counts, int32_t* send_offsets, int32_t* send_order,
                 int32_t* pair_pos, void* send_x, int32_t* send_ids, hipStream_t stream);

/*
 * moe_repack_ep_to_tp -- local-permute phase of the EP->TP expert-weight
 * reshard (Moebius review, §3.1 and Fig. 4): pack this rank's E_local whole
 * experts into one contiguous block per destination peer q < P:
 *   dst13[q] (E_local, 2I/P, H) = rows [q I/P, (q+1) I/P) of the gate half, then
 *                                 the same rows of the up half, of each expert
 *   dst2[q]  (E_local, H, I/P)  = columns [q I/P, (q+1) I/P) of each W2 row
 *   w13_ep (E_local, 2I, H), w2_ep (E_local, H, I) dtype, exact byte copies.
 *   dst13, dst2: HOST arrays of P device pointers (blocks must not overlap the
 *   sources or each other).  A peer-mapped pointer works the same way.
 * Limits: 1 <= P <= 64; I % P == 0; (I/P) * sizeof(dtype) and H * sizeof(dtype)
 * multiples of 16.
 */
int moe_repack_ep_to_tp(const void* w13_ep, const void* w2_ep, int E_local, int H, int I, int P,
                        int dtype, void* const* dst13, void* const* dst2, hipStream_t stream);

/*
 * moe_repack_tp_to_ep -- local-permute phase of the TP->EP expert-weight
 * reshard (Moebius review, §3.1 and Fig. 4, the switch back): after the
 * exchange this rank holds, from each peer q < P, peer q's TP slice of this
 * rank's E_local experts; rebuild the whole experts from those P blocks.  The
 * exact inverse of moe_repack_ep_to_tp:
 *   w13_ep[e] rows [q I/P, (q+1) I/P)     = src13[q][e] rows [0, I/P)
 *   w13_ep[e] rows I + [q I/P, (q+1) I/P) = src13[q][e] rows [I/P, 2I/P)
 *   w2_ep[e][:, q I/P .. (q+1) I/P)       = src2[q][e]
 *   src13, src2: HOST arrays of P device pointers, (E_local, 2I/P, H) and
 *   (E_local, H, I/P) dtype; w13_ep (E_local, 2I, H), w2_ep (E_local, H, I)
 *   dtype [out], exact byte copies (outputs must not overlap the blocks).
 * Limits: those of moe_repack_ep_to_tp.
 */
int moe_repack_tp_to_ep(const void* const* src13, const void* const* src2, int E_local, int H, int I, int P,
                        int dtype, void* w13_ep, void* w2_ep, hipStream_t stream);

/*
 * moe_schedule_requests -- request scheduling under data-parallel attention
 * (Sem-MoE notes, online data scheduling): with every vocabulary id in one
 * cluster (= rank), request r goes to S_r = argmax_j sum_{i in r} R_ij, and
 * every E consecutive requests are spread over all E ranks.
 *   tokens            (n_tokens) int32   the requests' token ids, concatenated
 *   req_offsets       (n_req + 1) int32  request r is tokens[req_offsets[r] ..
 *                                        req_offsets[r+1]) (bounds are clamped
 *                                        into [0, n_tokens])
 *   cluster_of_token  (vocab) int32      cluster (rank) of every id, in [0, E)
 *   scores    (n_req, E) int32 [out]  token positions of r in cluster j (ids
 *                                     outside [0, vocab), clusters outside
 *                                     [0, E) are not counted)
 *   affinity  (n_req) int32 [out]     S_r, ties to the lowest rank
 *   assigned  (n_req) int32 [out]     balanced rank: requests taken in arrival
 *             order in groups of E (the last one may be shorter); each takes
 *             its highest-scoring rank not taken earlier in its group (ties to
 *             the lowest), so a full group covers every rank once
 *   ws        >= moe_schedule_workspace_bytes(n_req, E) bytes, zero-filled
 *             before first use; every completed call leaves it zero.
 * Limits: 1 <= E <= 64; n_tokens < 2^25.  Deterministic.
 */
size_t moe_schedule_workspace_bytes(int n_req, int E);
int moe_schedule_requests(const int32_t* tokens, int n_tokens, const int32_t* req_offsets, int n_req,
                          const int32_t* cluster_of_token, int vocab, int E, int32_t* scores,
                          int32_t* affinity, int32_t* assigned, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * The EP/TP switch policy (Moebius review, §4.5) -- host code, no GPU.
 * A coordinator calls moe_switch_step once per decode iteration, after the
 * step, with the global count of in-flight requests:
 *   - in TP, the mode switches to EP as soon as the count exceeds t_high;
 *   - in EP, it switches back to TP when the mean of the last `window` counts
 *     (counts of either mode; none before `window` of them exist) falls below
 *     t_low; t_low <= t_high is the hysteresis band;
 *   - after a switch, or a switch cancelled because the target mode's KV
 *     capacity (live requests it can hold; <= 0: unlimited) is below the
 *     count, no decision is taken while now_s < that time + cooldown_s.
 * The caller owns the state (no allocation); calls on one state must not
 * overlap.  The pages' evaluation uses t_high = 256, cooldown 5 s, and
 * t_low = 0.8 t_high, window 8 (interactive) or t_low = t_high, window 1
 * (rollout).
 */
#define MOE_SWITCH_WINDOW_MAX 4096

enum moe_mode { MOE_MODE_TP = 0, MOE_MODE_EP = 1 };
enum moe_switch_decision { MOE_SWITCH_STAY = 0, MOE_SWITCH_TO_EP = 1, MOE_SWITCH_TO_TP = 2,
                           MOE_SWITCH_VETOED = 3 };

typedef struct moe_switch_params {
  double t_high;      /* T_h */
  double t_low;       /* T_l, <= t_high */
  int window;         /* W, 1 .. MOE_SWITCH_WINDOW_MAX */
  double cooldown_s;  /* C, >= 0, in the caller's clock */
  double kv_cap_tp;   /* live requests the TP layout's KV cache holds; <= 0: unlimited */
  double kv_cap_ep;   /* same for EP */
} moe_switch_params;

typedef struct moe_switch_state {
  moe_switch_params p;
  int mode;                 /* current mode (moe_mode) */
  int have_last;            /* a switch or cancelled switch has happened */
  double t_last;            /* its time */
  long long n_samples;      /* counts seen */
  int head;                 /* next ring slot (the oldest once the window is full) */
  long long window_sum;     /* exact sum of the counts in the window */
  int ring[MOE_SWITCH_WINDOW_MAX];
} moe_switch_state;

/* Validate p and start in `mode`.  MOE_EINVAL on bad parameters. */
int moe_switch_init(const moe_switch_params* p, int mode, moe_switch_state* s);

/* Record this iteration's count at time now_s and decide; *decision is a
 * moe_switch_decision and the state's mode follows it.  MOE_EINVAL on a
 * negative count, a non-finite time or a null pointer. */
int moe_switch_step(moe_switch_state* s, double now_s, int in_flight, int* decision);

/*
 * Start-up calibration of the threshold (Moebius review, §4.5): the batch at
 * which the EP decode step stops being slower than the TP step.  batches (n,
 * strictly increasing), t_tp and t_ep (n) are host arrays of measured step
 * times.  The first i with t_ep[i] <= t_tp[i] gives batches[0] if i == 0, else
 * the zero of t_ep - t_tp interpolated linearly in the batch between i - 1
 * and i; if there is none, +infinity.
 */
int moe_switch_crossover(const double* batches, const double* t_tp, const double* t_ep, int n,
                         double* b_star);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LAYER_AMD_MOE_H */
