"""Pins for the CPU oracle: each test checks it against something other than
itself -- a per-token brute force, closed forms, hand-derived values,
invariants of the EP/TP views and special cases that reduce to textbook
operations."""
import math

import numpy as np
import pytest

import oracle
from moe_inputs import LayerConfig, get_config, make_full_model, make_layer_inputs

REL = 1e-12


def rel_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def small_cfg(H=40, E=8, k=3, I=24, renorm=True, n_shared=0, dtype="fp32", T=12):
    return LayerConfig(name="small", H=H, E=E, k=k, renorm=renorm, I=I, dtype=dtype,
                       T_list=(T,), n_shared=n_shared)


def ep_share(model, cfg, r, P):
    E_l = cfg.E // P
    return oracle.moe_layer(model["x"], model["w_gate"], model["gate_bias"],
                            model["w13"][r * E_l:(r + 1) * E_l], model["w2"][r * E_l:(r + 1) * E_l],
                            cfg.k, cfg.renorm, 0, g_begin=r * E_l)


# ---------------------------------------------------------------- P1 brute force

def test_tiny_config_matches_brute_force():
    cfg = get_config("tiny")
    d = make_layer_inputs(cfg, 16)
    r = oracle.moe_layer(d["x"], d["w_gate"], d["gate_bias"], d["w13"], d["w2"], cfg.k, cfg.renorm)
    yb = oracle.brute_force_layer(d["x"], d["w_gate"], d["gate_bias"], d["w13"], d["w2"],
                                  cfg.k, cfg.renorm)
    assert rel_err(r["y"], yb) < REL
    assert np.abs(r["y"]).max() > 0.1


@pytest.mark.parametrize("renorm,n_shared,dtype,routing", [
    (True, 0, "fp32", "uniform"), (False, 2, "fp32", "uniform"),
    (True, 1, "bf16", "zipf"), (False, 0, "bf16", "zipf"),
])
def test_small_shapes_match_brute_force(renorm, n_shared, dtype, routing):
    cfg = small_cfg(renorm=renorm, n_shared=n_shared, dtype=dtype)
    m = make_full_model(cfg, 12, routing=routing, seed=3)
    r = oracle.moe_layer(m["x"], m["w_gate"], m["gate_bias"], m["w13"], m["w2"],
                         cfg.k, cfg.renorm, cfg.n_shared)
    yb = oracle.brute_force_layer(m["x"], m["w_gate"], m["gate_bias"], m["w13"], m["w2"],
                                  cfg.k, cfg.renorm, cfg.n_shared)
    assert rel_err(r["y"], yb) < REL


@pytest.mark.parametrize("P", [2, 4, 8])
def test_ep_and_tp_shares_match_brute_force(P):
    cfg = small_cfg(E=8, I=24, T=10)
    m = make_full_model(cfg, 10, seed=5)
    for r in range(P):
        E_l = cfg.E // P
        sl = slice(r * E_l, (r + 1) * E_l)
        got = ep_share(m, cfg, r, P)["y"]
        want = oracle.brute_force_layer(m["x"], m["w_gate"], m["gate_bias"], m["w13"][sl],
                                        m["w2"][sl], cfg.k, cfg.renorm, g_begin=r * E_l)
        assert rel_err(got, want) < REL or np.abs(want).max() == 0
    for p in range(P):
        w13p, w2p = oracle.tp_slice(m["w13"], m["w2"], p, P)
        got = oracle.moe_layer(m["x"], m["w_gate"], m["gate_bias"], w13p, w2p, cfg.k, cfg.renorm)["y"]
        want = oracle.brute_force_layer(m["x"], m["w_gate"], m["gate_bias"], w13p, w2p,
                                        cfg.k, cfg.renorm)
        assert rel_err(got, want) < REL


# ---------------------------------------------------------------- P2 renormalisation

@pytest.mark.parametrize("name", ["tiny", "qwen3_30b"])
def test_renormalised_weights_sum_to_one(name):
    cfg = get_config(name)
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((64, cfg.E))
    ids, w = oracle.route(logits, cfg.k, True)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    ids2, w2 = oracle.route(logits, cfg.k, False)
    assert (ids == ids2).all()
    assert (w2.sum(axis=1) < 1.0).all()


# ---------------------------------------------------------------- P3/P4 view invariants

@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_sum_of_shares_equals_full_layer(P):
    cfg = small_cfg(E=8, I=32, H=56, k=3, T=20)
    m = make_full_model(cfg, 20, routing="zipf", seed=7)
    full = oracle.moe_layer(m["x"], m["w_gate"], m["gate_bias"], m["w13"], m["w2"], cfg.k, cfg.renorm)
    ep_sum = sum(ep_share(m, cfg, r, P)["y"] for r in range(P))
    tp_sum = 0
    for p in range(P):
        w13p, w2p = oracle.tp_slice(m["w13"], m["w2"], p, P)
        tp_sum = tp_sum + oracle.moe_layer(m["x"], m["w_gate"], m["gate_bias"], w13p, w2p,
                                           cfg.k, cfg.renorm)["y"]
    assert rel_err(ep_sum, full["y"]) < REL
    assert rel_err(tp_sum, full["y"]) < REL


def test_single_rank_views_are_identical():
    cfg = small_cfg()
    m = make_full_model(cfg, 12, seed=2)
    full = oracle.moe_layer(m["x"], m["w_gate"], m["gate_bias"], m["w13"], m["w2"], cfg.k, cfg.renorm)
    ep = ep_share(m, cfg, 0, 1)
    w13p, w2p = oracle.tp_slice(m["w13"], m["w2"], 0, 1)
    tp = oracle.moe_layer(m["x"], m["w_gate"], m["gate_bias"], w13p, w2p, cfg.k, cfg.renorm)
    assert np.array_equal(full["y"], ep["y"])
    assert np.array_equal(full["y"], tp["y"])


def test_ep_rank_keeps_only_its_experts():
    cfg = small_cfg(E=8, k=2, T=16)
    m = make_full_model(cfg, 16, seed=11)
    full = oracle.moe_layer(m["x"], m["w_gate"], m["gate_bias"], m["w13"], m["w2"], cfg.k, cfg.renorm)
    P = 4
    for r in range(P):
        s = ep_share(m, cfg, r, P)
        ids = full["ids"]
        local = (ids >= 2 * r) & (ids < 2 * r + 2)
        assert s["offsets"][-1] == local.sum()
        # tokens with no local pick give an exactly zero partial row
        none = ~local.any(axis=1)
        assert (s["y"][none] == 0).all()


# ---------------------------------------------------------------- P5 k = E closed form

def test_k_equals_E_is_a_dense_softmax_mixture():
    cfg = small_cfg(E=6, k=6, H=24, I=16, T=9)
    m = make_full_model(cfg, 9, seed=4)
    r = oracle.moe_layer(m["x"], m["w_gate"], m["gate_bias"], m["w13"], m["w2"], 6, True)
    x = m["x"].astype(np.float64)
    l = x @ m["w_gate"].astype(np.float64).T
    p = np.exp(l) / np.exp(l).sum(axis=1, keepdims=True)
    w13 = m["w13"].astype(np.float64)
    w2 = m["w2"].astype(np.float64)
    g = np.einsum("eih,th->tei", w13[:, :16], x)
    u = np.einsum("eih,th->tei", w13[:, 16:], x)
    a = g / (1 + np.exp(-g)) * u
    ffn = np.einsum("ehi,tei->teh", w2, a)
    want = np.einsum("te,teh->th", p, ffn)
    assert rel_err(r["y"], want) < 1e-11


# ---------------------------------------------------------------- P6 routing special cases

@pytest.mark.parametrize("renorm", [True, False])
def test_zero_gate_routes_to_lowest_ids(renorm):
    T, E, k = 5, 8, 3
    logits = oracle.gate_logits(np.ones((T, 4)), np.zeros((E, 4)), np.zeros(E))
    ids, w = oracle.route(logits, k, renorm)
    assert (ids == np.arange(k)).all()
    assert np.allclose(w, 1.0 / k if renorm else 1.0 / E, rtol=0, atol=1e-15)
    counts, offsets, _, _ = oracle.permute(ids, 0, E)
    assert counts.tolist() == [T] * k + [0] * (E - k)
    assert offsets.tolist() == [0, T, 2 * T, 3 * T] + [3 * T] * (E - k)


def test_bias_alone_sets_the_routing():
    b = np.array([0.1, 2.0, -1.0, 2.0, 0.5, 3.0])
    logits = oracle.gate_logits(np.ones((3, 2)), np.zeros((6, 2)), b)
    ids, w = oracle.route(logits, 4, False)
    # descending bias, tie between experts 1 and 3 broken to the lower id
    assert (ids == [5, 1, 3, 4]).all()
    z = np.exp(b - 3.0)
    assert np.allclose(w[0], z[[5, 1, 3, 4]] / z.sum(), rtol=1e-14)


def test_signed_zero_logits_tie_to_lower_index():
    l = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0]])
    ids = oracle.topk_desc(l, 2)
    assert ids.tolist() == [[0, 1], [0, 1]]


def test_shared_experts_are_appended_with_unit_weight():
    l = np.array([[0.0, 1.0, 2.0, 3.0]])
    ids, w = oracle.route(l, 2, False, n_shared=2)
    assert ids.tolist() == [[3, 2, 4, 5]]
    assert w[0, 2:].tolist() == [1.0, 1.0]


# ---------------------------------------------------------------- P7 hand-derived values

def test_single_expert_swiglu_by_hand():
    # H=2, I=1, one expert, k=1: gate = 1*1 + 0.5*2 = 2, up = -1*1 + 1*2 = 1,
    # a = silu(2) * 1 = 2 / (1 + e^-2), y = W2 a = (3a, -a).
    x = np.array([[1.0, 2.0]])
    w13 = np.array([[[1.0, 0.5], [-1.0, 1.0]]])
    w2 = np.array([[[3.0], [-1.0]]])
    r = oracle.moe_layer(x, np.zeros((1, 2)), np.zeros(1), w13, w2, 1, True)
    a = 2.0 / (1.0 + math.exp(-2.0))
    assert np.allclose(r["y"], [[3 * a, -a]], rtol=1e-15, atol=0)
    assert np.allclose(r["A"], [[a]], rtol=1e-15, atol=0)


def test_two_experts_top1_by_hand():
    # logits = (ln 3, 0): softmax = (3/4, 1/4); top-1 picks expert 0 with
    # weight 3/4 (no renorm).  Expert 0: gate = 2, up = 1, W2 = (1, 0)^T.
    x = np.array([[1.0, 0.0]])
    wg = np.array([[math.log(3.0), 0.0], [0.0, 0.0]])
    w13 = np.array([[[2.0, 0.0], [1.0, 0.0]], [[5.0, 5.0], [5.0, 5.0]]])
    w2 = np.array([[[1.0], [0.0]], [[7.0], [7.0]]])
    r = oracle.moe_layer(x, wg, np.zeros(2), w13, w2, 1, False)
    a = 2.0 / (1.0 + math.exp(-2.0))
    assert r["ids"].tolist() == [[0]]
    assert np.allclose(r["w"], [[0.75]], rtol=1e-15)
    assert np.allclose(r["y"], [[0.75 * a, 0.0]], rtol=1e-15, atol=0)
    # renormalised over one pick the weight becomes 1
    r1 = oracle.moe_layer(x, wg, np.zeros(2), w13, w2, 1, True)
    assert np.allclose(r1["y"], [[a, 0.0]], rtol=1e-15, atol=0)


def test_combine_uses_slot_weights_in_order():
    # two tokens, kk=2; token 1's second slot is not held (pos -1)
    y_pair = np.array([[1.0, 0.0], [0.0, 1.0], [2.0, 2.0]])
    pos = np.array([0, 2, 1, -1])
    w = np.array([[0.5, 0.25], [0.125, 9.0]])
    y = oracle.combine(y_pair, pos, w, 2, 2)
    assert y.tolist() == [[1.0, 0.5], [0.0, 0.125]]


# ---------------------------------------------------------------- P8 permutation

@pytest.mark.parametrize("g_begin,n_groups", [(0, 10), (3, 4), (8, 2)])
def test_permute_is_the_stable_argsort(g_begin, n_groups):
    rng = np.random.default_rng(9)
    T, kk = 37, 3
    ids = rng.integers(0, 10, size=(T, kk)).astype(np.int32)
    counts, offsets, sp, pos = oracle.permute(ids, g_begin, n_groups)
    flat = ids.ravel().astype(np.int64) - g_begin
    keep = (flat >= 0) & (flat < n_groups)
    idx = np.nonzero(keep)[0]
    want = idx[np.argsort(flat[idx], kind="stable")]
    assert sp.tolist() == want.tolist()
    assert counts.sum() == keep.sum() == offsets[-1]
    assert (np.diff(offsets) == counts).all() and offsets[0] == 0
    assert (pos[sp] == np.arange(sp.size)).all()
    assert (pos[~keep] == -1).all()
    keys = flat[sp]
    assert (np.diff(keys) >= 0).all()
    for g in range(n_groups):
        seg = sp[offsets[g]:offsets[g + 1]]
        assert (np.diff(seg) > 0).all()


def test_permute_hand_example():
    # T=3, kk=2; ids (0,2), (2,1), (0,1) with window [0,3)
    counts, offsets, sp, pos = oracle.permute(np.array([[0, 2], [2, 1], [0, 1]]), 0, 3)
    assert counts.tolist() == [2, 2, 2]
    assert offsets.tolist() == [0, 2, 4, 6]
    assert sp.tolist() == [0, 4, 3, 5, 1, 2]
    assert pos.tolist() == [0, 4, 5, 2, 1, 3]


# ---------------------------------------------------------------- P9 repack

@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_repack_round_trip_and_layout(P):
    E_l, I, H = 3, 16, 6
    # each element encodes (expert, row, column), so a wrong index shows up exactly
    e, r, c = np.meshgrid(np.arange(E_l), np.arange(2 * I), np.arange(H), indexing="ij")
    w13 = (e * 10000 + r * 100 + c).astype(np.uint16)
    e2, h2, i2 = np.meshgrid(np.arange(E_l), np.arange(H), np.arange(I), indexing="ij")
    w2 = (e2 * 10000 + h2 * 100 + i2).astype(np.uint16)
    b13, b2 = oracle.repack_ep_to_tp(w13, w2, P)
    Ip = I // P
    for q in range(P):
        assert b13[q].shape == (E_l, 2 * Ip, H) and b2[q].shape == (E_l, H, Ip)
        for i in range(2 * Ip):
            src_row = q * Ip + i if i < Ip else I + q * Ip + (i - Ip)
            assert (b13[q][:, i, :] == w13[:, src_row, :]).all()
        assert (b2[q] == w2[:, :, q * Ip:(q + 1) * Ip]).all()
    r13, r2 = oracle.repack_tp_to_ep(b13, b2)
    assert np.array_equal(r13, w13) and np.array_equal(r2, w2)


def test_repack_block_equals_tp_view_of_local_experts():
    cfg = small_cfg(E=8, I=32)
    m = make_full_model(cfg, 4)
    P, r = 4, 1
    E_l = cfg.E // P
    b13, b2 = oracle.repack_ep_to_tp(m["w13"][r * E_l:(r + 1) * E_l],
                                     m["w2"][r * E_l:(r + 1) * E_l], P)
    for q in range(P):
        t13, t2 = oracle.tp_slice(m["w13"], m["w2"], q, P)
        assert np.array_equal(b13[q], t13[r * E_l:(r + 1) * E_l])
        assert np.array_equal(b2[q], t2[r * E_l:(r + 1) * E_l])


# ---------------------------------------------------------------- P11 EP dispatch

@pytest.mark.parametrize("E_l,P", [(2, 4), (3, 3), (1, 8), (8, 1)])
def test_dispatch_is_the_stable_argsort_by_rank(E_l, P):
    rng = np.random.default_rng(21)
    T, kk, H = 29, 3, 5
    E = E_l * P
    ids = rng.integers(0, E + 2, size=(T, kk)).astype(np.int32)   # ids >= E: shared, stay local
    x = rng.integers(0, 60000, size=(T, H)).astype(np.uint16)
    d = oracle.dispatch(x, ids, E_l, P)
    flat = ids.ravel().astype(np.int64)
    dest = flat // E_l
    sent = flat < E
    idx = np.nonzero(sent)[0]
    want = idx[np.argsort(dest[idx], kind="stable")]
    assert d["send_order"].tolist() == want.tolist()
    assert d["counts"].tolist() == np.bincount(dest[idx], minlength=P).tolist()
    assert d["offsets"].tolist() == [0] + np.cumsum(d["counts"]).tolist()
    assert (d["pair_pos"][want] == np.arange(want.size)).all()
    assert (d["pair_pos"][~sent] == -1).all()
    assert np.array_equal(d["send_x"], x[want // kk])
    assert d["send_x"].dtype == x.dtype
    assert d["send_ids"].tolist() == flat[want].tolist()
    for r in range(P):
        blk = d["send_ids"][d["offsets"][r]:d["offsets"][r + 1]]
        assert ((blk >= r * E_l) & (blk < (r + 1) * E_l)).all()


def test_dispatch_hand_example():
    # T=3, kk=2, two ranks of two experts: ids (3,0), (1,2), (2,3)
    # -> ranks (1,0), (0,1), (1,1): rank 0 gets pairs 1, 2; rank 1 gets 0, 3, 4, 5
    x = np.array([[10.0], [20.0], [30.0]])
    d = oracle.dispatch(x, np.array([[3, 0], [1, 2], [2, 3]]), 2, 2)
    assert d["counts"].tolist() == [2, 4]
    assert d["offsets"].tolist() == [0, 2, 6]
    assert d["send_order"].tolist() == [1, 2, 0, 3, 4, 5]
    assert d["pair_pos"].tolist() == [2, 0, 1, 3, 4, 5]
    assert d["send_x"][:, 0].tolist() == [10.0, 20.0, 10.0, 20.0, 30.0, 30.0]
    assert d["send_ids"].tolist() == [0, 1, 3, 2, 2, 3]


@pytest.mark.parametrize("P,routing", [(2, "uniform"), (4, "zipf"), (8, "uniform")])
def test_ep_exchange_equals_full_layer(P, routing):
    # P ranks each own T/P tokens; after dispatch, expert work and return the
    # concatenated outputs are the full layer on the whole batch.
    cfg = small_cfg(E=8, I=24, H=32, k=3, T=24)
    m = make_full_model(cfg, 24, routing=routing, seed=13)
    shares = np.split(m["x"], P)
    ex = oracle.ep_exchange_layer(shares, m["w_gate"], m["gate_bias"], m["w13"], m["w2"],
                                  cfg.k, cfg.renorm)
    full = oracle.moe_layer(m["x"], m["w_gate"], m["gate_bias"], m["w13"], m["w2"], cfg.k, cfg.renorm)
    assert rel_err(np.concatenate(ex["y"]), full["y"]) < REL
    yb = oracle.brute_force_layer(m["x"], m["w_gate"], m["gate_bias"], m["w13"], m["w2"],
                                  cfg.k, cfg.renorm)
    assert rel_err(np.concatenate(ex["y"]), yb) < REL
    # every pair is sent exactly once, to the rank owning its expert
    n_pairs = sum(s["offsets"][-1] for s in ex["dispatch"])
    assert n_pairs == m["x"].shape[0] * cfg.k


# ---------------------------------------------------------------- P10 silu

def test_silu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 40.0, -40.0, 100.0, -100.0, -1000.0])
    s = oracle.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(s[2] + math.exp(-1.0) / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(s[3] - 40.0) < 1e-12 and s[5] == 100.0
    assert -1e-15 < s[4] < 0 and -1e-40 < s[6] <= 0 and s[7] == 0
    assert np.isfinite(s).all()


def test_widen_is_exact_for_bf16():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x3F81], dtype=np.uint16)
    v = oracle.widen(bits)
    assert v.tolist()[:3] == [1.0, -1.0, 3.140625]
    assert v[3] == 0.0 and math.copysign(1.0, v[4]) == -1.0
    assert v[5] == 1.0 + 2.0 ** -7


# ---------------------------------------------------------------- P12 switch policy and calibration

HAND_TRACE = [5, 8, 11, 12, 9, 7, 5, 4, 3, 12]


def run_policy(trace, **kw):
    from oracle import switch_policy as sp
    p = sp.SwitchPolicy(**kw)
    out = [p.step(float(i + 1), c) for i, c in enumerate(trace)]
    return out, p


def test_policy_hand_trace():
    # T_h = 10, T_l = 6, W = 3, no cooldown; times 1, 2, ..., 10.
    # t3: 11 > 10 in TP -> EP.  t4..t7: window means 10.33, 10.67, 9.33, 7 >= 6.
    # t8: mean(7, 5, 4) = 5.33 < 6 -> TP.  t10: 12 > 10 -> EP.
    out, p = run_policy(HAND_TRACE, t_high=10, t_low=6, window=3, cooldown_s=0)
    assert out == [0, 0, 1, 0, 0, 0, 0, 2, 0, 1]
    assert p.mode == 1


def test_policy_cooldown_blocks_decisions():
    # C = 6: after the switch at t3 nothing is decided before t9; at t9 the
    # window (5, 4, 3) has mean 4 < 6 -> TP; t10 is inside the new cooldown.
    out, _ = run_policy(HAND_TRACE, t_high=10, t_low=6, window=3, cooldown_s=6)
    assert out == [0, 0, 1, 0, 0, 0, 0, 0, 2, 0]


def test_policy_kv_capacity_veto():
    # EP holds at most 10 live requests: the switches at t3 (11) and t10 (12)
    # are cancelled, the first one starting a cooldown of 2 s.
    out, p = run_policy(HAND_TRACE, t_high=10, t_low=6, window=3, cooldown_s=2, kv_cap_ep=10)
    assert out == [0, 0, 3, 0, 0, 0, 0, 0, 0, 3]
    assert p.mode == 0
    # a capacity that holds the count does not veto
    out, _ = run_policy(HAND_TRACE, t_high=10, t_low=6, window=3, cooldown_s=0, kv_cap_ep=11)
    assert out[2] == 1


def test_policy_thresholds_are_strict_and_window_must_fill():
    # rollout setting: T_l = T_h, W = 1
    out, _ = run_policy([256, 257, 256, 255], t_high=256, t_low=256, window=1, cooldown_s=0)
    assert out == [0, 1, 0, 2]
    # EP from the start: no decision until W samples exist
    out, _ = run_policy([0, 0, 0, 0], t_high=10, t_low=6, window=3, cooldown_s=0, mode=1)
    assert out == [0, 0, 2, 0]


def test_crossover_of_two_lines_is_exact():
    from oracle import switch_policy as sp
    B = [8, 16, 32, 64, 128, 256, 512]
    t_tp = [10 + 0.5 * b for b in B]
    t_ep = [30 + 0.3 * b for b in B]
    assert abs(sp.crossover(B, t_tp, t_ep) - 100.0) < 1e-12       # 10 + 0.5B = 30 + 0.3B
    assert sp.crossover(B, t_ep, t_tp) == 8.0                       # EP faster from the start
    assert sp.crossover(B, [1.0] * 7, [2.0] * 7) == math.inf        # EP never catches up
    assert sp.crossover([8, 16], [2.0, 3.0], [3.0, 3.0]) == 16.0    # equal at a grid point


def test_simulation_time_and_modes():
    from oracle import switch_policy as sp
    p = sp.SwitchPolicy(t_high=10, t_low=6, window=1, cooldown_s=0)
    step = lambda mode, c: (1.0 if mode == sp.TP else 2.0)
    r = sp.simulate([5, 20, 20, 1, 1], step, p, switch_time_s=0.5)
    # TP, TP(->EP after), EP, EP(->TP after), TP
    assert r["modes"] == [0, 0, 1, 1, 0]
    assert r["decisions"] == [0, 1, 0, 2, 0]
    assert r["time"] == 1 + 1 + 0.5 + 2 + 2 + 0.5 + 1


# ---------------------------------------------------------------- P13 request scheduling (Attention-DP)

def test_request_scores_hand_example():
    from oracle import request_schedule as rs
    # vocabulary of 6 ids in 3 clusters; three requests (the second one empty)
    cl = [0, 2, 1, 1, 0, 2]
    tokens = [1, 1, 3, 0, 5, 4, 4, 2]
    offsets = [0, 5, 5, 8]
    s = rs.cluster_scores(tokens, offsets, cl, 3)
    # request 0: ids 1,1,3,0,5 -> clusters 2,2,1,0,2; request 2: ids 4,4,2 -> 0,0,1
    assert s.tolist() == [[1, 1, 3], [0, 0, 0], [2, 1, 0]]
    assert rs.affinity_rank(s).tolist() == [2, 0, 0]          # the empty request ties -> 0
    # group of E = 3: request 0 takes 2, request 1 takes its best free rank 0
    # (tie among 0 and 1 -> 0), request 2 is left with rank 1
    assert rs.balanced_ranks(s).tolist() == [2, 0, 1]


def test_request_scores_are_bincounts():
    from oracle import request_schedule as rs
    rng = np.random.default_rng(5)
    V, E = 50, 7
    cl = rng.integers(0, E, size=V)
    lens = rng.integers(0, 40, size=30)
    offsets = np.concatenate([[0], np.cumsum(lens)])
    tokens = rng.integers(0, V, size=offsets[-1])
    s = rs.cluster_scores(tokens, offsets, cl, E)
    for r in range(30):
        seg = tokens[offsets[r]:offsets[r + 1]]
        assert s[r].tolist() == np.bincount(cl[seg], minlength=E).tolist()
    assert rs.affinity_rank(s).tolist() == np.argmax(s, axis=1).tolist()   # numpy: first maximum


@pytest.mark.parametrize("n,E", [(24, 8), (29, 8), (5, 8), (12, 1)])
def test_balanced_groups_cover_every_rank(n, E):
    from oracle import request_schedule as rs
    rng = np.random.default_rng(n * 10 + E)
    s = rng.integers(0, 6, size=(n, E))
    b = rs.balanced_ranks(s)
    for g0 in range(0, n, E):
        grp = b[g0:g0 + E].tolist()
        assert len(set(grp)) == len(grp)                          # distinct inside a group
        if len(grp) == E:
            assert sorted(grp) == list(range(E))                  # a full group covers all ranks
    # the first request of a group always gets its own argmax
    a = rs.affinity_rank(s)
    assert (b[::E] == a[::E]).all()
    # distinct preferences inside every group: balancing changes nothing
    s2 = np.zeros((n, E), dtype=np.int64)
    for r in range(n):
        s2[r, r % E] = 5
    assert (rs.balanced_ranks(s2) == rs.affinity_rank(s2)).all()
