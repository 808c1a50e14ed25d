"""One MoE-layer forward pass on this GPU's share, as the four C-ABI calls.

``MoeLayerBuffers`` allocates (with torch) every output and workspace the
calls need for a given shape, once, so repeated passes allocate nothing and
can be captured in a HIP graph.  ``moe_layer_forward`` enqueues

    moe_route_permute -> moe_expert_up -> moe_expert_down -> moe_combine

(four launches) on the current stream; ``fused=False`` runs moe_route and
moe_permute as two calls instead.  All arithmetic happens in the HIP library.
"""
from dataclasses import dataclass

import torch

from . import _lib


@dataclass
class MoeLayerBuffers:
    logits: torch.Tensor
    topk_ids: torch.Tensor
    topk_w: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    sorted_pair: torch.Tensor
    pair_pos: torch.Tensor
    a: torch.Tensor
    y_pair: torch.Tensor
    y: torch.Tensor
    route_ws: torch.Tensor
    expert_ws: torch.Tensor

    @classmethod
    def allocate(cls, T, H, E, kk, n_groups, I, dtype, device="cuda"):
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        act = dict(dtype=dtype, device=dev)
        return cls(
            logits=torch.empty((T, E), **f32),
            topk_ids=torch.empty((T, kk), **i32),
            topk_w=torch.empty((T, kk), **f32),
            counts=torch.empty((n_groups,), **i32),
            offsets=torch.empty((n_groups + 1,), **i32),
            sorted_pair=torch.empty((T * kk,), **i32),
            pair_pos=torch.empty((T * kk,), **i32),
            a=torch.empty((T * kk, I), **act),
            y_pair=torch.empty((T * kk, H), **act),
            y=torch.empty((T, H), **act),
            route_ws=_lib.route_workspace(T, H, E, dtype, dev),
            expert_ws=_lib.expert_workspace(T, kk, n_groups, H, I, dtype, dev),
        )


def moe_layer_forward(x, w_gate, gate_bias, w13, w2, k, renorm, n_shared=0, g_begin=0,
                      bufs=None, stream=None, fused=True):
    """Run the layer; returns the buffers (``bufs.y`` is the output).

    x (T, H); w_gate (E, H); gate_bias (E,) fp32 or None; w13 (G, 2I, H);
    w2 (G, H, I), all in one storage dtype (bfloat16 or float32).  The G
    groups held here have global ids g_begin .. g_begin + G - 1.
    """
    T, H = x.shape
    E = w_gate.shape[0]
    G, two_i, _ = w13.shape
    I = two_i // 2
    kk = k + n_shared
    if bufs is None:
        bufs = MoeLayerBuffers.allocate(T, H, E, kk, G, I, x.dtype, x.device)
    if fused:
        _lib.moe_route_permute(x, w_gate, gate_bias, k, renorm, n_shared, bufs.logits,
                               bufs.topk_ids, bufs.topk_w, g_begin, G, bufs.counts, bufs.offsets,
                               bufs.sorted_pair, bufs.pair_pos, bufs.route_ws, stream)
    else:
        _lib.moe_route(x, w_gate, gate_bias, k, renorm, n_shared, bufs.logits, bufs.topk_ids,
                       bufs.topk_w, bufs.route_ws, stream)
        _lib.moe_permute(bufs.topk_ids, g_begin, G, bufs.counts, bufs.offsets, bufs.sorted_pair,
                         bufs.pair_pos, stream)
    _lib.moe_expert_up(x, bufs.sorted_pair, bufs.offsets, kk, w13, bufs.a, bufs.expert_ws, stream)
    _lib.moe_expert_down(bufs.a, bufs.offsets, T, kk, w2, bufs.y_pair, bufs.expert_ws, stream)
    _lib.moe_combine(bufs.y_pair, bufs.pair_pos, bufs.topk_w, bufs.y, stream)
    return bufs
