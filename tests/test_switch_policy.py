"""The EP/TP switch policy and the crossover calibration of the C ABI (host
code: these run without a GPU) against the oracle, decision by decision, on
seeded synthetic load traces, plus the argument checks."""
import math

import numpy as np
import pytest

import oracle
from moe_inputs.gen import load_trace

sp = oracle.switch_policy


def lib_policy(**kw):
    import moe_layer_amd
    return moe_layer_amd.SwitchPolicy(**kw)


def test_state_layout_round_trips():
    p = lib_policy(t_high=256, t_low=204.8, window=8, cooldown_s=5, kv_cap_tp=900, kv_cap_ep=3000)
    st = p.state
    assert (st.p.t_high, st.p.t_low, st.p.window, st.p.cooldown_s) == (256, 204.8, 8, 5)
    assert (st.p.kv_cap_tp, st.p.kv_cap_ep, st.mode, st.n_samples) == (900, 3000, 0, 0)
    for i, c in enumerate([3, 1, 4, 1, 5, 9, 2, 6, 5, 3]):
        p.step(float(i), c)
    assert st.n_samples == 10 and st.window_sum == 4 + 1 + 5 + 9 + 2 + 6 + 5 + 3   # the last 8


@pytest.mark.parametrize("t_high,t_low,window,cooldown,cap_tp,cap_ep,kind", [
    (256, 204.8, 8, 5.0, 0, 0, "burst"),        # interactive setting of the pages
    (256, 256, 1, 5.0, 0, 0, "rollout"),        # rollout setting
    (256, 204.8, 8, 0.0, 0, 0, "burst"),        # no cooldown: every crossing decides
    (128, 64, 3, 0.05, 0, 1200, "rollout"),     # EP capacity below a round's start: vetoes
    (300, 100, 16, 0.02, 90, 0, "burst"),       # TP capacity: vetoes on the way back
    (64, 64, 4, 0.0, 0, 0, "noise"),
])
def test_policy_matches_oracle_on_traces(t_high, t_low, window, cooldown, cap_tp, cap_ep, kind):
    trace, dt = load_trace(kind, 3000, seed=window + int(t_high))
    kw = dict(t_high=t_high, t_low=t_low, window=window, cooldown_s=cooldown, kv_cap_tp=cap_tp,
              kv_cap_ep=cap_ep)
    ref = sp.SwitchPolicy(**kw)
    got = lib_policy(**kw)
    now = 0.0
    decisions = []
    for c, d in zip(trace, dt):
        now += d
        want = ref.step(now, int(c))
        assert got.step(now, int(c)) == want
        assert got.mode == ref.mode
        decisions.append(want)
    # the traces exercise every branch they are meant to
    assert decisions.count(sp.TO_EP) >= 1 and decisions.count(sp.TO_TP) >= 1
    if cap_ep or cap_tp:
        assert decisions.count(sp.VETOED) >= 1


def test_crossover_matches_oracle():
    import moe_layer_amd
    rng = np.random.default_rng(4)
    B = [8, 16, 32, 64, 128, 256, 512, 1024, 2048]
    for _ in range(200):
        t_tp = rng.uniform(50, 500, size=len(B)).tolist()
        t_ep = rng.uniform(50, 500, size=len(B)).tolist()
        assert moe_layer_amd.switch_crossover(B, t_tp, t_ep) == sp.crossover(B, t_tp, t_ep)
    assert moe_layer_amd.switch_crossover(B, [1.0] * 9, [2.0] * 9) == math.inf
    assert moe_layer_amd.switch_crossover([8], [2.0], [1.0]) == 8.0


def test_argument_checks():
    import moe_layer_amd
    from moe_layer_amd import MoeError
    with pytest.raises(MoeError):
        lib_policy(t_high=10, t_low=11, window=2, cooldown_s=0)     # t_low > t_high
    with pytest.raises(MoeError):
        lib_policy(t_high=10, t_low=5, window=0, cooldown_s=0)
    with pytest.raises(MoeError):
        lib_policy(t_high=10, t_low=5, window=4097, cooldown_s=0)
    with pytest.raises(MoeError):
        lib_policy(t_high=10, t_low=5, window=2, cooldown_s=-1)
    with pytest.raises(MoeError):
        lib_policy(t_high=math.nan, t_low=5, window=2, cooldown_s=0)
    p = lib_policy(t_high=10, t_low=5, window=2, cooldown_s=0)
    with pytest.raises(MoeError):
        p.step(1.0, -1)
    with pytest.raises(MoeError):
        p.step(math.inf, 3)
    with pytest.raises(MoeError):
        moe_layer_amd.switch_crossover([8, 8], [1, 1], [1, 1])      # not increasing
    with pytest.raises(MoeError):
        moe_layer_amd.switch_crossover([], [], [])
    with pytest.raises(MoeError):
        moe_layer_amd.switch_crossover([8, 16], [1, math.nan], [1, 1])
