"""The allocation-free routing entry point (moe_route_permute_noalloc) against
moe_route_permute with a caller workspace: the same kernel on the same
inputs, so every output must be bit-identical.  Two calls in a row on the
library's one scratch array, the second with a smaller batch (the counters the
first call used must not leak into the second), then the first shape again."""
import numpy as np
import pytest
import torch

from moe_inputs import LayerConfig, get_config, make_layer_inputs

pytestmark = pytest.mark.gpu

OUTS = ("logits", "topk_ids", "topk_w", "counts", "offsets", "sorted_pair", "pair_pos")


def run_both(d, cfg):
    import gpu_helpers as gh
    import moe_layer_amd as M
    T = d["x"].shape[0]
    x, wg, b = gh.to_dev(d["x"]), gh.to_dev(d["w_gate"]), gh.to_dev(d["gate_bias"])
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    res = []
    for noalloc in (False, True):
        bufs = M.MoeLayerBuffers.allocate(T, cfg.H, cfg.E, cfg.kk, cfg.n_groups, cfg.I_local, dt)
        # poison the outputs so stale values cannot pass for results
        for name in OUTS:
            getattr(bufs, name).fill_(-7)
        args = (x, wg, b, cfg.k, cfg.renorm, cfg.n_shared, bufs.logits, bufs.topk_ids, bufs.topk_w,
                d["g_begin"], cfg.n_groups, bufs.counts, bufs.offsets, bufs.sorted_pair, bufs.pair_pos)
        if noalloc:
            M.moe_route_permute_noalloc(*args)
        else:
            M.moe_route_permute(*args, bufs.route_ws)
        torch.cuda.synchronize()
        res.append({n: gh.from_dev(getattr(bufs, n)) for n in OUTS})
    ref, got = res
    n_kept = int(ref["offsets"][-1])
    for n in OUTS:
        a, g = ref[n], got[n]
        if n == "sorted_pair":
            a, g = a[:n_kept], g[:n_kept]
        assert np.array_equal(a.view(np.uint8), g.view(np.uint8)), f"{n} differs (T={T})"
    return n_kept


@pytest.mark.parametrize("name,T1,T2", [
    ("qwen3_235b_ep", 300, 20),     # several token tiles, then one more than a tile
    ("qwen3_235b_tp", 64, 8),       # K slices summed per block, then a single-tile sort
])
def test_noalloc_matches_workspace_call(name, T1, T2):
    cfg = get_config(name)
    d1 = make_layer_inputs(cfg, T1, routing="zipf")
    d2 = dict(d1)
    d2["x"] = d1["x"][:T2]
    print(f"[case] noalloc {name} T={T1} then T={T2} then T={T1}", flush=True)
    k1 = run_both(d1, cfg)
    k2 = run_both(d2, cfg)
    assert 0 < k2 < k1
    assert run_both(d1, cfg) == k1


def test_noalloc_fp32_and_wide():
    cfg = LayerConfig(name="small", H=256, E=512, k=32, renorm=True, I=64, dtype="fp32", T_list=(40,))
    d = make_layer_inputs(cfg, 40, routing="uniform", seed=100)
    print("[case] noalloc fp32 E=512 k=32 T=40 then T=5", flush=True)
    run_both(d, cfg)
    d2 = dict(d)
    d2["x"] = d["x"][:5]
    run_both(d2, cfg)
