"""Out-of-bounds writes: every output and workspace buffer of a layer pass is a
window inside a larger allocation whose margins (and, for the row-indexed
outputs, the rows past the kept pairs) are filled with a byte pattern.  After
the four calls (route + permute, up, down, combine) the margins must still
hold the pattern, byte for byte, and the results must still match the oracle.
Cases cover the kernels' edges: ragged batches, fp32, the one-launch sort and
the multi-block permute, the block-cooperative and the wave-streaming
up-projections, the LDS-tiled kernels, wide routing and an EP share."""
import numpy as np
import pytest
import torch

from moe_inputs import LayerConfig, make_layer_inputs

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes on each side (keeps every window 256-byte aligned)
PATTERN = 0xA5


class Guarded:
    """A tensor of `shape`/`dtype` living in the middle of a patterned block."""

    def __init__(self, shape, dtype, fill=None):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.n = n
        self.raw = torch.full((GUARD + n + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.raw[GUARD:GUARD + n].view(dtype).view(shape)
        if fill is not None:
            self.t.fill_(fill)

    def margins_intact(self):
        r = self.raw.cpu().numpy()
        return bool((r[:GUARD] == PATTERN).all() and (r[GUARD + self.n:] == PATTERN).all())


def guarded_buffers(T, H, E, kk, n_groups, I, dtype):
    import moe_layer_amd
    from moe_layer_amd import _lib
    code = 1 if dtype == torch.bfloat16 else 0
    rw = max(_lib.moe_route_workspace_bytes(T, H, E, code), 256)
    ew = max(_lib.moe_workspace_bytes(5, T, kk, n_groups, H, I, code), 256)
    g = dict(
        logits=Guarded((T, E), torch.float32), topk_ids=Guarded((T, kk), torch.int32),
        topk_w=Guarded((T, kk), torch.float32), counts=Guarded((n_groups,), torch.int32),
        offsets=Guarded((n_groups + 1,), torch.int32),
        sorted_pair=Guarded((T * kk,), torch.int32, fill=-12345),
        pair_pos=Guarded((T * kk,), torch.int32), a=Guarded((T * kk, I), dtype, fill=7.0),
        y_pair=Guarded((T * kk, H), dtype, fill=7.0), y=Guarded((T, H), dtype),
        route_ws=Guarded((rw,), torch.uint8, fill=0), expert_ws=Guarded((ew,), torch.uint8, fill=0))
    bufs = moe_layer_amd.MoeLayerBuffers(**{k: v.t for k, v in g.items()})
    return g, bufs


def small(H=256, E=16, k=4, I=128, renorm=True, n_shared=0, dtype="bf16", view="full", P=1, T=37):
    return LayerConfig(name="small", H=H, E=E, k=k, renorm=renorm, I=I, dtype=dtype, T_list=(T,),
                       n_shared=n_shared, view=view, P=P)


@pytest.mark.parametrize("cfg_kw,seed", [
    (dict(T=37), 1),                                           # ragged, one-launch sort
    (dict(T=17, dtype="fp32"), 2),                             # fp32 kernels
    (dict(T=100, H=2048, I=768, E=32, k=4), 3),                # block-cooperative up-projection
    (dict(T=300, H=1568, I=736, E=8, k=2), 4),                 # LDS-tiled kernels, partial stages
    (dict(T=700, H=256, I=64, E=64, k=8), 5),                  # multi-block permute, wave-streaming
    (dict(T=33, H=256, I=64, E=512, k=32), 6),                 # wide routing (32 keys per lane)
    (dict(T=64, H=512, I=128, E=32, k=4, view="ep", P=4), 7),  # EP share: pairs not held here
])
def test_margins_untouched(cfg_kw, seed):
    import gpu_helpers as gh
    import moe_layer_amd
    cfg = small(**cfg_kw)
    T = cfg.T_list[0]
    d = make_layer_inputs(cfg, T, routing="uniform", rank=cfg.P - 1, seed=100 + seed)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    g, bufs = guarded_buffers(T, cfg.H, cfg.E, cfg.kk, cfg.n_groups, cfg.I_local, dt)
    print(f"[case] canary {cfg_kw}", flush=True)
    dev = {key: gh.to_dev(d[key]) for key in ("x", "w_gate", "gate_bias", "w13", "w2")}
    moe_layer_amd.moe_layer_forward(dev["x"], dev["w_gate"], dev["gate_bias"], dev["w13"], dev["w2"],
                                    cfg.k, cfg.renorm, cfg.n_shared, d["g_begin"], bufs=bufs)
    torch.cuda.synchronize()
    bad = [name for name, buf in g.items() if not buf.margins_intact()]
    assert not bad, f"writes past the ends of {bad}"
    # nothing is written past the kept pairs
    n_kept = int(bufs.offsets[-1].item())
    assert (bufs.sorted_pair[n_kept:] == -12345).all()
    ones = torch.full((1,), 7.0, dtype=dt, device="cuda")
    assert (bufs.a[n_kept:] == ones).all() and (bufs.y_pair[n_kept:] == ones).all()
    # and the pass is the real one
    out = {name: gh.from_dev(getattr(bufs, name)) for name in
           ("logits", "topk_ids", "topk_w", "counts", "offsets", "sorted_pair", "pair_pos", "a", "y_pair", "y")}
    gh.check_layer(d, cfg, out)
