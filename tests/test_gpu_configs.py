"""GPU parity on the five workloads at their full sizes, through the C ABI.

Each case runs the whole layer (route, permute, up, down, combine) in the
launch configuration the benchmark times and checks every step against the
float64 oracle (rules in gpu_helpers).  Prints the case before each GPU step.
"""
import sys

import numpy as np
import pytest

from moe_inputs import get_config, make_layer_inputs, make_repack_inputs

pytestmark = pytest.mark.gpu

_models = {}


def model(name, routing):
    """Seeded host inputs at the config's largest batch plus device weights (cached)."""
    import gpu_helpers as gh
    key = (name, routing)
    if key not in _models:
        _models.clear()  # keep one model resident at a time
        cfg = get_config(name)
        d = make_layer_inputs(cfg, cfg.T_max, routing=routing)
        dev = {k: gh.to_dev(d[k]) for k in ("w_gate", "gate_bias", "w13", "w2")}
        _models[key] = (cfg, d, dev)
    return _models[key]


def run_case(name, T, routing):
    import gpu_helpers as gh
    cfg, d, dev = model(name, routing)
    dT = dict(d)
    dT["x"] = np.ascontiguousarray(d["x"][:T])
    print(f"[case] {name} T={T} routing={routing} rank={d.get('rank')}", flush=True)
    sys.stdout.flush()
    g = gh.gpu_layer(dT, cfg, dev=dev)
    stats = gh.check_layer(dT, cfg, g)
    print(f"[ok] {name} T={T} {routing}: " + ", ".join(
        f"{k}={v:.2e}" if isinstance(v, float) else f"{k}={v}" for k, v in stats.items()), flush=True)
    return stats


def test_tiny_fp32():
    run_case("tiny", 16, "uniform")


def test_dsv2_lite_full_layer():
    run_case("dsv2_lite", 256, "uniform")


@pytest.mark.parametrize("routing", ["zipf", "uniform"])
@pytest.mark.parametrize("T", get_config("qwen3_30b").T_list)
def test_qwen3_30b(T, routing):
    run_case("qwen3_30b", T, routing)


@pytest.mark.parametrize("routing", ["uniform", "zipf"])
@pytest.mark.parametrize("B", get_config("qwen3_235b_ep").T_list)
def test_qwen3_235b_ep_share(B, routing):
    run_case("qwen3_235b_ep", B, routing)


@pytest.mark.parametrize("routing", ["uniform", "zipf"])
@pytest.mark.parametrize("B", get_config("qwen3_235b_tp").T_list)
def test_qwen3_235b_tp_share(B, routing):
    run_case("qwen3_235b_tp", B, routing)


def test_qwen3_235b_repack_both_directions_bit_exact():
    import torch

    import gpu_helpers as gh
    import moe_layer_amd
    import oracle
    _models.clear()
    cfg = get_config("qwen3_235b_tp")
    r = make_repack_inputs(cfg, rank=0)
    P = cfg.P
    Ip = cfg.I // P
    E_l = cfg.E // P
    print(f"[case] repack E_local={E_l} H={cfg.H} I={cfg.I} P={P}", flush=True)
    w13, w2 = gh.to_dev(r["w13_ep"]), gh.to_dev(r["w2_ep"])
    d13 = [torch.empty((E_l, 2 * Ip, cfg.H), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    d2 = [torch.empty((E_l, cfg.H, Ip), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    moe_layer_amd.moe_repack_ep_to_tp(w13, w2, P, d13, d2)
    torch.cuda.synchronize()
    b13, b2 = oracle.repack_ep_to_tp(r["w13_ep"], r["w2_ep"], P)
    for q in range(P):
        assert np.array_equal(gh.from_dev(d13[q]), b13[q]), f"W13 block {q}"
        assert np.array_equal(gh.from_dev(d2[q]), b2[q]), f"W2 block {q}"
    # the switch back: the GPU's own blocks gathered into whole experts again
    print(f"[case] repack TP->EP E_local={E_l} H={cfg.H} I={cfg.I} P={P}", flush=True)
    r13, r2 = torch.empty_like(w13), torch.empty_like(w2)
    moe_layer_amd.moe_repack_tp_to_ep(d13, d2, P, r13, r2)
    torch.cuda.synchronize()
    assert np.array_equal(gh.from_dev(r13), r["w13_ep"]), "W13 round trip"
    assert np.array_equal(gh.from_dev(r2), r["w2_ep"]), "W2 round trip"
