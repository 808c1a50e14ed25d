"""ctypes binding of libmoe_layer_amd.so: argument marshalling only.

Every function takes torch tensors that already live on the GPU (torch is
used for device memory and streams), checks their dtype, shape and
contiguity, and passes raw pointers and sizes to the C entry point of the
same name on the current torch stream.  No computation happens here and
there is no fallback: if the HIP library is missing, loading fails.
"""
import ctypes
import os

import torch  # noqa: F401  (must load first: the library shares torch's HIP runtime)

HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; MOE_LAYER_AMD_LIB names another build of the same
# sources (e.g. the host-sanitized one of build_sanitized.py).
LIB_PATH = os.environ.get("MOE_LAYER_AMD_LIB") or os.path.join(HERE, "libmoe_layer_amd.so")

MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1
MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_GROUPED_GEMM, MOE_OP_COMBINE, MOE_OP_REPACK = range(5)
MOE_OP_EXPERT_UP, MOE_OP_EXPERT_DOWN = 5, 6

EXPORTED = (
    "moe_abi_version", "moe_status_str", "moe_workspace_bytes", "moe_route_workspace_bytes",
    "moe_route", "moe_route_permute", "moe_route_permute_noalloc", "moe_permute", "moe_grouped_gemm", "moe_expert_up",
    "moe_expert_down", "moe_combine", "moe_repack_ep_to_tp", "moe_repack_tp_to_ep", "moe_dispatch",
    "moe_switch_init", "moe_switch_step", "moe_switch_crossover", "moe_schedule_workspace_bytes",
    "moe_schedule_requests",
)


class MoeError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None
_p = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t
_dp = ctypes.POINTER(ctypes.c_double)

MODE_TP, MODE_EP = 0, 1
SWITCH_STAY, SWITCH_TO_EP, SWITCH_TO_TP, SWITCH_VETOED = 0, 1, 2, 3
SWITCH_WINDOW_MAX = 4096


class SwitchParams(ctypes.Structure):
    """moe_switch_params of include/moe.h."""
    _fields_ = [("t_high", ctypes.c_double), ("t_low", ctypes.c_double), ("window", ctypes.c_int),
                ("cooldown_s", ctypes.c_double), ("kv_cap_tp", ctypes.c_double),
                ("kv_cap_ep", ctypes.c_double)]


class SwitchState(ctypes.Structure):
    """moe_switch_state of include/moe.h (caller-owned, fixed size)."""
    _fields_ = [("p", SwitchParams), ("mode", ctypes.c_int), ("have_last", ctypes.c_int),
                ("t_last", ctypes.c_double), ("n_samples", ctypes.c_longlong), ("head", ctypes.c_int),
                ("window_sum", ctypes.c_longlong), ("ring", ctypes.c_int * SWITCH_WINDOW_MAX)]


def lib():
    """Load the HIP library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"HIP library not found at {LIB_PATH}; build it with "
            "`python -m moe_layer_amd.build` (or __graft_entry__.build())")
    L = ctypes.CDLL(LIB_PATH)
    L.moe_abi_version.restype = _i
    L.moe_abi_version.argtypes = []
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_status_str.argtypes = [_i]
    L.moe_workspace_bytes.restype = _sz
    L.moe_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i]
    L.moe_route_workspace_bytes.restype = _sz
    L.moe_route_workspace_bytes.argtypes = [_i, _i, _i, _i]
    L.moe_route.restype = _i
    L.moe_route.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _sz, _p]
    L.moe_route_permute.restype = _i
    L.moe_route_permute.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _i, _i,
                                    _p, _p, _p, _p, _p, _sz, _p]
    L.moe_route_permute_noalloc.restype = _i
    L.moe_route_permute_noalloc.argtypes = [_p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _p, _p, _i, _i,
                                            _p, _p, _p, _p, _p]
    L.moe_permute.restype = _i
    L.moe_permute.argtypes = [_p, _i, _i, _i, _i, _p, _p, _p, _p, _p]
    L.moe_grouped_gemm.restype = _i
    L.moe_grouped_gemm.argtypes = [_p, _p, _p, _i, _i, _i, _p, _p, _i, _i, _i, _p, _p, _sz, _p]
    L.moe_expert_up.restype = _i
    L.moe_expert_up.argtypes = [_p, _p, _p, _i, _i, _i, _p, _i, _i, _i, _p, _p, _sz, _p]
    L.moe_expert_down.restype = _i
    L.moe_expert_down.argtypes = [_p, _p, _i, _i, _i, _p, _i, _i, _i, _p, _p, _sz, _p]
    L.moe_combine.restype = _i
    L.moe_combine.argtypes = [_p, _p, _p, _i, _i, _i, _i, _p, _p]
    L.moe_switch_init.restype = _i
    L.moe_switch_init.argtypes = [ctypes.POINTER(SwitchParams), _i, ctypes.POINTER(SwitchState)]
    L.moe_switch_step.restype = _i
    L.moe_switch_step.argtypes = [ctypes.POINTER(SwitchState), ctypes.c_double, _i, ctypes.POINTER(_i)]
    L.moe_switch_crossover.restype = _i
    L.moe_switch_crossover.argtypes = [_dp, _dp, _dp, _i, _dp]
    L.moe_schedule_workspace_bytes.restype = _sz
    L.moe_schedule_workspace_bytes.argtypes = [_i, _i]
    L.moe_schedule_requests.restype = _i
    L.moe_schedule_requests.argtypes = [_p, _i, _p, _i, _p, _i, _i, _p, _p, _p, _p, _sz, _p]
    L.moe_dispatch.restype = _i
    L.moe_dispatch.argtypes = [_p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p]
    L.moe_repack_ep_to_tp.restype = _i
    L.moe_repack_ep_to_tp.argtypes = [_p, _p, _i, _i, _i, _i, _i, ctypes.POINTER(_p),
                                      ctypes.POINTER(_p), _p]
    L.moe_repack_tp_to_ep.restype = _i
    L.moe_repack_tp_to_ep.argtypes = [ctypes.POINTER(_p), ctypes.POINTER(_p), _i, _i, _i, _i, _i, _p, _p,
                                      _p]
    _lib = L
    return L


def _check(fn, status):
    if status != 0:
        raise MoeError(fn, status, lib().moe_status_str(status).decode())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return MOE_DTYPE_BF16
    if t.dtype == torch.float32:
        return MOE_DTYPE_F32
    raise TypeError(f"unsupported storage dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t, name, dtype=None, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def abi_version():
    return lib().moe_abi_version()


def moe_workspace_bytes(op, T, kk, n_groups, H, I, dtype_code):
    return lib().moe_workspace_bytes(op, T, kk, n_groups, H, I, dtype_code)


def moe_route_workspace_bytes(T, H, E, dtype_code):
    return lib().moe_route_workspace_bytes(T, H, E, dtype_code)


def route_workspace(T, H, E, dtype, device="cuda"):
    """A zero-filled routing workspace (reusable: every call leaves it zeroed)."""
    code = MOE_DTYPE_BF16 if dtype == torch.bfloat16 else MOE_DTYPE_F32
    n = max(moe_route_workspace_bytes(T, H, E, code), 256)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _route_common(x, w_gate, gate_bias, k, n_shared, logits, topk_ids, topk_w):
    T, H = x.shape
    E = w_gate.shape[0]
    kk = k + n_shared
    return (_ptr(x, "x"), _ptr(w_gate, "w_gate", x.dtype, (E, H)),
            _ptr(gate_bias, "gate_bias", torch.float32, (E,)), T, H, E,
            _ptr(logits, "logits", torch.float32, (T, E)),
            _ptr(topk_ids, "topk_ids", torch.int32, (T, kk)),
            _ptr(topk_w, "topk_w", torch.float32, (T, kk)))


def moe_route(x, w_gate, gate_bias, k, renorm, n_shared, logits, topk_ids, topk_w, ws, stream=None):
    px, pw, pb, T, H, E, pl, pi, pww = _route_common(x, w_gate, gate_bias, k, n_shared, logits,
                                                     topk_ids, topk_w)
    st = lib().moe_route(px, pw, pb, T, H, E, k, int(bool(renorm)), n_shared, _dtype_code(x), pl, pi,
                         pww, _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check("moe_route", st)


def moe_route_permute(x, w_gate, gate_bias, k, renorm, n_shared, logits, topk_ids, topk_w,
                      g_begin, n_groups, counts, offsets, sorted_pair, pair_pos, ws, stream=None):
    px, pw, pb, T, H, E, pl, pi, pww = _route_common(x, w_gate, gate_bias, k, n_shared, logits,
                                                     topk_ids, topk_w)
    kk = k + n_shared
    st = lib().moe_route_permute(
        px, pw, pb, T, H, E, k, int(bool(renorm)), n_shared, _dtype_code(x), pl, pi, pww, g_begin,
        n_groups, _ptr(counts, "counts", torch.int32, (n_groups,)),
        _ptr(offsets, "offsets", torch.int32, (n_groups + 1,)),
        _ptr(sorted_pair, "sorted_pair", torch.int32, (T * kk,)),
        _ptr(pair_pos, "pair_pos", torch.int32, (T * kk,)), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream))
    _check("moe_route_permute", st)


def moe_route_permute_noalloc(x, w_gate, gate_bias, k, renorm, n_shared, logits, topk_ids, topk_w,
                              g_begin, n_groups, counts, offsets, sorted_pair, pair_pos, stream=None):
    """moe_route_permute with the library's fixed per-GPU scratch instead of a
    workspace (nothing is allocated; calls on one GPU must not overlap)."""
    px, pw, pb, T, H, E, pl, pi, pww = _route_common(x, w_gate, gate_bias, k, n_shared, logits,
                                                     topk_ids, topk_w)
    kk = k + n_shared
    st = lib().moe_route_permute_noalloc(
        px, pw, pb, T, H, E, k, int(bool(renorm)), n_shared, _dtype_code(x), pl, pi, pww, g_begin,
        n_groups, _ptr(counts, "counts", torch.int32, (n_groups,)),
        _ptr(offsets, "offsets", torch.int32, (n_groups + 1,)),
        _ptr(sorted_pair, "sorted_pair", torch.int32, (T * kk,)),
        _ptr(pair_pos, "pair_pos", torch.int32, (T * kk,)), _stream(stream))
    _check("moe_route_permute_noalloc", st)


def moe_permute(topk_ids, g_begin, n_groups, counts, offsets, sorted_pair, pair_pos, stream=None):
    T, kk = topk_ids.shape
    st = lib().moe_permute(
        _ptr(topk_ids, "topk_ids", torch.int32), T, kk, g_begin, n_groups,
        _ptr(counts, "counts", torch.int32, (n_groups,)),
        _ptr(offsets, "offsets", torch.int32, (n_groups + 1,)),
        _ptr(sorted_pair, "sorted_pair", torch.int32, (T * kk,)),
        _ptr(pair_pos, "pair_pos", torch.int32, (T * kk,)), _stream(stream))
    _check("moe_permute", st)


def moe_grouped_gemm(x, sorted_pair, offsets, kk, w13, w2, y_pair, ws, stream=None):
    T, H = x.shape
    G, two_i, _ = w13.shape
    I = two_i // 2
    dt = _dtype_code(x)
    st = lib().moe_grouped_gemm(
        _ptr(x, "x"), _ptr(sorted_pair, "sorted_pair", torch.int32, (T * kk,)),
        _ptr(offsets, "offsets", torch.int32, (G + 1,)), T, kk, G,
        _ptr(w13, "w13", x.dtype, (G, 2 * I, H)), _ptr(w2, "w2", x.dtype, (G, H, I)), H, I, dt,
        _ptr(y_pair, "y_pair", x.dtype, (T * kk, H)), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream))
    _check("moe_grouped_gemm", st)


def expert_workspace(T, kk, n_groups, H, I, dtype, device="cuda"):
    """A zero-filled workspace that serves both moe_expert_up and
    moe_expert_down for these sizes (each call leaves it zeroed again)."""
    code = MOE_DTYPE_BF16 if dtype == torch.bfloat16 else MOE_DTYPE_F32
    n = max(moe_workspace_bytes(MOE_OP_EXPERT_UP, T, kk, n_groups, H, I, code), 256)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def moe_expert_up(x, sorted_pair, offsets, kk, w13, a, ws, stream=None):
    T, H = x.shape
    G, two_i, _ = w13.shape
    I = two_i // 2
    st = lib().moe_expert_up(
        _ptr(x, "x"), _ptr(sorted_pair, "sorted_pair", torch.int32, (T * kk,)),
        _ptr(offsets, "offsets", torch.int32, (G + 1,)), T, kk, G,
        _ptr(w13, "w13", x.dtype, (G, 2 * I, H)), H, I, _dtype_code(x),
        _ptr(a, "a", x.dtype, (T * kk, I)), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
        _stream(stream))
    _check("moe_expert_up", st)


def moe_expert_down(a, offsets, T, kk, w2, y_pair, ws, stream=None):
    G, H, I = w2.shape
    st = lib().moe_expert_down(
        _ptr(a, "a", w2.dtype, (T * kk, I)), _ptr(offsets, "offsets", torch.int32, (G + 1,)), T, kk, G,
        _ptr(w2, "w2"), H, I, _dtype_code(w2), _ptr(y_pair, "y_pair", w2.dtype, (T * kk, H)),
        _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check("moe_expert_down", st)


def moe_combine(y_pair, pair_pos, topk_w, y, stream=None):
    """topk_w (T, kk) fp32, or None for weight 1 on every slot (then kk is
    pair_pos.numel() // T; kk = 1 is the un-permute y[t] = y_pair[pair_pos[t]])."""
    T, H = y.shape
    kk = topk_w.shape[1] if topk_w is not None else (pair_pos.numel() // T if T else 1)
    st = lib().moe_combine(
        _ptr(y_pair, "y_pair", y.dtype), _ptr(pair_pos, "pair_pos", torch.int32, (T * kk,)),
        _ptr(topk_w, "topk_w", torch.float32, (T, kk)), T, kk, H, _dtype_code(y), _ptr(y, "y"),
        _stream(stream))
    _check("moe_combine", st)


def moe_dispatch(x, topk_ids, E_local, P, send_counts, send_offsets, send_order, pair_pos, send_x,
                 send_ids, stream=None):
    """Send layout of the EP dispatch: pairs by owning rank topk_ids // E_local
    (< P), send_x[i] = x[send_order[i] // kk], send_ids[i] = topk_ids[send_order[i]]."""
    T, H = x.shape
    kk = topk_ids.shape[1]
    st = lib().moe_dispatch(
        _ptr(x, "x"), _ptr(topk_ids, "topk_ids", torch.int32, (T, kk)), T, kk, H, E_local, P,
        _dtype_code(x), _ptr(send_counts, "send_counts", torch.int32, (P,)),
        _ptr(send_offsets, "send_offsets", torch.int32, (P + 1,)),
        _ptr(send_order, "send_order", torch.int32, (T * kk,)),
        _ptr(pair_pos, "pair_pos", torch.int32, (T * kk,)),
        _ptr(send_x, "send_x", x.dtype, (T * kk, H)),
        _ptr(send_ids, "send_ids", torch.int32, (T * kk,)), _stream(stream))
    _check("moe_dispatch", st)


def moe_repack_ep_to_tp(w13_ep, w2_ep, P, dst13, dst2, stream=None):
    E_l, two_i, H = w13_ep.shape
    I = two_i // 2
    if len(dst13) != P or len(dst2) != P:
        raise ValueError("need P destination blocks for each tensor")
    Ip = I // P
    arr13 = (_p * P)(*[_ptr(d, f"dst13[{q}]", w13_ep.dtype, (E_l, 2 * Ip, H)) for q, d in enumerate(dst13)])
    arr2 = (_p * P)(*[_ptr(d, f"dst2[{q}]", w13_ep.dtype, (E_l, H, Ip)) for q, d in enumerate(dst2)])
    st = lib().moe_repack_ep_to_tp(
        _ptr(w13_ep, "w13_ep"), _ptr(w2_ep, "w2_ep", w13_ep.dtype, (E_l, H, I)), E_l, H, I, P,
        _dtype_code(w13_ep), arr13, arr2, _stream(stream))
    _check("moe_repack_ep_to_tp", st)


def moe_repack_tp_to_ep(src13, src2, P, w13_ep, w2_ep, stream=None):
    """Rebuild whole experts w13_ep (E_l, 2I, H), w2_ep (E_l, H, I) from the P
    TP-slice blocks src13[q] (E_l, 2I/P, H), src2[q] (E_l, H, I/P)."""
    E_l, two_i, H = w13_ep.shape
    I = two_i // 2
    if len(src13) != P or len(src2) != P:
        raise ValueError("need P source blocks for each tensor")
    Ip = I // P
    arr13 = (_p * P)(*[_ptr(b, f"src13[{q}]", w13_ep.dtype, (E_l, 2 * Ip, H)) for q, b in enumerate(src13)])
    arr2 = (_p * P)(*[_ptr(b, f"src2[{q}]", w13_ep.dtype, (E_l, H, Ip)) for q, b in enumerate(src2)])
    st = lib().moe_repack_tp_to_ep(
        arr13, arr2, E_l, H, I, P, _dtype_code(w13_ep), _ptr(w13_ep, "w13_ep"),
        _ptr(w2_ep, "w2_ep", w13_ep.dtype, (E_l, H, I)), _stream(stream))
    _check("moe_repack_tp_to_ep", st)


class SwitchPolicy:
    """The EP/TP switch coordinator's decision rule (moe_switch_* of the C ABI):
    one step(now_s, in_flight) per decode iteration."""

    def __init__(self, t_high, t_low, window, cooldown_s, kv_cap_tp=0.0, kv_cap_ep=0.0, mode=MODE_TP):
        self.params = SwitchParams(float(t_high), float(t_low), int(window), float(cooldown_s),
                                   float(kv_cap_tp), float(kv_cap_ep))
        self.state = SwitchState()
        _check("moe_switch_init", lib().moe_switch_init(ctypes.byref(self.params), int(mode),
                                                        ctypes.byref(self.state)))

    @property
    def mode(self):
        return self.state.mode

    def step(self, now_s, in_flight):
        d = ctypes.c_int(-1)
        _check("moe_switch_step", lib().moe_switch_step(ctypes.byref(self.state), float(now_s),
                                                        int(in_flight), ctypes.byref(d)))
        return d.value


def switch_crossover(batches, t_tp, t_ep):
    """Batch where the EP step stops being slower than the TP step (linear
    interpolation between measured batches; inf if never)."""
    n = len(batches)
    arr = lambda v: (ctypes.c_double * n)(*[float(x) for x in v])
    if len(t_tp) != n or len(t_ep) != n:
        raise ValueError("batches, t_tp and t_ep must have the same length")
    out = ctypes.c_double(0.0)
    _check("moe_switch_crossover", lib().moe_switch_crossover(arr(batches), arr(t_tp), arr(t_ep), n,
                                                              ctypes.byref(out)))
    return out.value


def schedule_workspace(n_req, E, device="cuda"):
    """A zero-filled workspace for moe_schedule_requests (left zero by every call)."""
    n = max(lib().moe_schedule_workspace_bytes(n_req, E), 256)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def moe_schedule_requests(tokens, req_offsets, cluster_of_token, E, scores, affinity, assigned, ws,
                          stream=None):
    """Attention-DP request scheduling: per-request cluster counts, the argmax
    rank and the balanced rank (groups of E consecutive requests)."""
    n_req = req_offsets.numel() - 1
    st = lib().moe_schedule_requests(
        _ptr(tokens, "tokens", torch.int32), tokens.numel(),
        _ptr(req_offsets, "req_offsets", torch.int32), n_req,
        _ptr(cluster_of_token, "cluster_of_token", torch.int32), cluster_of_token.numel(), E,
        _ptr(scores, "scores", torch.int32, (n_req, E)), _ptr(affinity, "affinity", torch.int32, (n_req,)),
        _ptr(assigned, "assigned", torch.int32, (n_req,)), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
        _stream(stream))
    _check("moe_schedule_requests", st)
