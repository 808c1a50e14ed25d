"""The seeded input generators: determinism, layout and the bf16 rounding."""
import numpy as np
import pytest

from moe_inputs import (CONFIGS, bf16_bits_from_f32, ep_rank_for, get_config,
                        make_layer_inputs, make_repack_inputs)
from moe_inputs.gen import gate_bias, make_x


def test_bf16_round_to_nearest_even():
    v = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -8 + 2.0 ** -20,
                  -2.5, 0.0, -0.0], dtype=np.float32)
    assert bf16_bits_from_f32(v).tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x0000, 0x8000]


def test_tiny_inputs_are_deterministic_and_shaped():
    cfg = get_config("tiny")
    a = make_layer_inputs(cfg, 16)
    b = make_layer_inputs(cfg, 16)
    for key in ("x", "w_gate", "w13", "w2", "gate_bias"):
        assert np.array_equal(a[key], b[key])
    assert a["x"].shape == (16, 256) and a["x"].dtype == np.float32
    assert a["w13"].shape == (8, 256, 256) and a["w2"].shape == (8, 256, 128)
    assert np.abs(a["x"]).max() > 1.0
    assert abs(a["w2"].std() - 128 ** -0.5) < 0.01


def test_x_prefixes_are_nested():
    cfg = get_config("qwen3_30b")
    x8 = make_x(cfg, 8)
    x32 = make_x(cfg, 32)
    assert np.array_equal(x8, x32[:8])


def test_zipf_bias_is_log_of_a_permutation():
    cfg = get_config("qwen3_30b")
    b = gate_bias(cfg, "zipf").astype(np.float64)
    rho = np.exp(-b / 1.2)
    assert np.allclose(np.sort(rho), np.arange(1, cfg.E + 1), rtol=1e-5)
    assert (gate_bias(cfg, "uniform") == 0).all()


def test_ep_rank_under_skew_is_the_heaviest_rank():
    cfg = get_config("qwen3_235b_ep")
    assert ep_rank_for(cfg, "uniform") == 0
    r = ep_rank_for(cfg, "zipf")
    prior = np.exp(gate_bias(cfg, "zipf").astype(np.float64)).reshape(8, 16).sum(1)
    assert r == int(prior.argmax())


def test_views_have_the_documented_shapes():
    for name, cfg in CONFIGS.items():
        assert cfg.n_groups * 3 * cfg.H * cfg.I_local > 0
    assert get_config("qwen3_235b_tp").I_local == 192
    assert get_config("qwen3_235b_ep").n_groups == 16
    assert get_config("dsv2_lite").n_groups == 66 and get_config("dsv2_lite").kk == 8


@pytest.mark.parametrize("rank", [0, 3])
def test_expert_weights_are_the_same_in_every_view(rank):
    from moe_inputs import LayerConfig, make_full_model
    cfg = LayerConfig(name="s", H=32, E=8, k=2, renorm=True, I=16, dtype="bf16",
                      T_list=(4,), view="ep", P=4)
    full = make_full_model(cfg, 4)
    ep = make_layer_inputs(cfg, 4, rank=rank)
    assert np.array_equal(ep["w13"], full["w13"][2 * rank:2 * rank + 2])
    rp = make_repack_inputs(cfg, rank=rank)
    assert np.array_equal(rp["w2_ep"], full["w2"][2 * rank:2 * rank + 2])


@pytest.mark.parametrize("routing", ["uniform", "zipf"])
def test_routing_table_is_distinct_seeded_and_skewed(routing):
    from moe_inputs.gen import routing_table
    cfg = get_config("dsv2_lite")
    ids = routing_table(cfg, 500, routing, seed=4)
    assert ids.shape == (500, cfg.k + cfg.n_shared) and ids.dtype == np.int32
    routed = ids[:, :cfg.k]
    assert ((routed >= 0) & (routed < cfg.E)).all()
    assert all(len(set(r)) == cfg.k for r in routed.tolist())
    assert (ids[:, cfg.k:] == cfg.E + np.arange(cfg.n_shared)).all()
    assert np.array_equal(ids, routing_table(cfg, 500, routing, seed=4))
    hist = np.bincount(routed.ravel(), minlength=cfg.E)
    if routing == "zipf":
        assert hist.max() > 4 * np.median(hist)
    else:
        assert hist.max() < 2 * hist.mean()


@pytest.mark.parametrize("kind", ["burst", "rollout", "noise"])
def test_load_traces_are_seeded_and_shaped(kind):
    from moe_inputs.gen import load_trace
    c, dt = load_trace(kind, 2000, seed=1)
    c2, dt2 = load_trace(kind, 2000, seed=1)
    assert np.array_equal(c, c2) and np.array_equal(dt, dt2)
    assert c.shape == dt.shape == (2000,) and (c >= 0).all()
    assert ((dt >= 0.02) & (dt <= 0.06)).all()
    if kind == "burst":
        assert np.median(c) < 100 and c.max() > 400
    if kind == "rollout":
        assert c.max() >= 1000 and (c == 0).any()


def test_requests_are_seeded_and_topical():
    from moe_inputs.gen import make_requests
    tok, off, cl, top = make_requests(200, 8, vocab=5000, seed=2)
    tok2, off2, cl2, top2 = make_requests(200, 8, vocab=5000, seed=2)
    assert np.array_equal(tok, tok2) and np.array_equal(off, off2) and np.array_equal(cl, cl2)
    assert off[0] == 0 and (np.diff(off) >= 1).all() and off[-1] == tok.size
    assert ((tok >= 0) & (tok < 5000)).all()
    assert np.bincount(cl, minlength=8).tolist() == [625] * 8        # balanced clusters
    # most of a request's tokens sit in its topic cluster
    frac = [np.mean(cl[tok[off[r]:off[r + 1]]] == top[r]) for r in range(200)]
    assert np.median(frac) > 0.5
