"""CPU oracle of the EP/TP switch policy and its start-up calibration.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``: only the
tests, the package's smoke check and the benchmark's CPU-baseline leg use it).

What it follows -- Moebius review, §4.5 (switch policy) and §6.1 (the values
used in the evaluation):

* The control signal is the global count of in-flight requests, sampled once
  per decode iteration, after the step and before the next one.
* In TP the coordinator switches to EP as soon as the latest count exceeds the
  high threshold T_h.
* In EP it switches back to TP only when the mean of the most recent W counts
  falls below the low threshold T_l (T_l <= T_h: the hysteresis band).
* After a switch, a cooldown C bounds the switch rate.
* Before committing, the target mode's KV capacity must hold the live
  requests; otherwise the switch is cancelled and retried after the cooldown.
* The thresholds start from a start-up calibration that times the EP and TP
  decode step and takes their crossover.
* Evaluation values: T_h = 256, C = 5 s; interactive T_l = 0.8 T_h, W = 8;
  rollout T_l = T_h, W = 1.

Readings where the pages are silent (each one is a pin in tests/test_oracle.py):

* "Exceeds" and "falls below" are strict: count > T_h, mean < T_l.
* The window is the last W samples of the count, whatever mode they were taken
  in; until W samples exist there is no EP->TP decision.
* The cooldown runs from the time of the last switch or cancelled switch: no
  decision is taken while now < t_last + C.  Time is the caller's clock.
* A capacity <= 0 means "unlimited".
* The crossover is the batch where the EP step time stops being larger than
  the TP step time: on a grid of measured batches B_0 < B_1 < ..., the first
  i with t_ep(B_i) <= t_tp(B_i); if i > 0 the difference d = t_ep - t_tp is
  interpolated linearly in B between B_{i-1} and B_i (d(B_{i-1}) > 0 >= d(B_i))
  and its zero is returned; if i == 0, B_0; if EP never catches up, +inf.
"""
import math

TP, EP = 0, 1
STAY, TO_EP, TO_TP, VETOED = 0, 1, 2, 3


class SwitchPolicy:
    """The coordinator's decision rule, one call per decode iteration."""

    def __init__(self, t_high, t_low, window, cooldown_s, kv_cap_tp=0.0, kv_cap_ep=0.0, mode=TP):
        assert t_low <= t_high and window >= 1 and cooldown_s >= 0
        self.t_high, self.t_low, self.window, self.cooldown = t_high, t_low, window, cooldown_s
        self.cap = {TP: kv_cap_tp, EP: kv_cap_ep}
        self.mode = mode
        self.samples = []          # every count seen, oldest first
        self.t_last = None         # time of the last switch or cancelled switch

    def step(self, now_s, count):
        """Record this iteration's count at time now_s; return the decision
        (STAY, TO_EP, TO_TP or VETOED) and apply it to the mode."""
        self.samples.append(count)
        if self.t_last is not None and now_s < self.t_last + self.cooldown:
            return STAY
        if self.mode == TP:
            want = count > self.t_high
            target = EP
        else:
            recent = self.samples[-self.window:]
            want = len(recent) == self.window and sum(recent) / self.window < self.t_low
            target = TP
        if not want:
            return STAY
        self.t_last = now_s
        cap = self.cap[target]
        if cap > 0 and count > cap:
            return VETOED
        self.mode = target
        return TO_EP if target == EP else TO_TP


def crossover(batches, t_tp, t_ep):
    """Batch at which the EP step time stops exceeding the TP step time (see
    the module notes); +inf if it never does."""
    assert len(batches) == len(t_tp) == len(t_ep) >= 1
    assert all(b0 < b1 for b0, b1 in zip(batches, batches[1:]))
    for i, (b, tt, te) in enumerate(zip(batches, t_tp, t_ep)):
        if te <= tt:
            if i == 0:
                return float(b)
            d0 = t_ep[i - 1] - t_tp[i - 1]
            d1 = te - tt
            b0 = batches[i - 1]
            return b0 + (b - b0) * d0 / (d0 - d1)
    return math.inf


def simulate(trace, step_time, policy, switch_time_s=0.0):
    """Drive ``policy`` over a trace of in-flight counts, one decode iteration
    per entry.  step_time(mode, count) is the iteration's duration in seconds;
    a switch adds switch_time_s.  Returns the total time, the mode of every
    iteration and the decision after it."""
    now = 0.0
    modes, decisions = [], []
    for count in trace:
        modes.append(policy.mode)
        now += step_time(policy.mode, count)
        d = policy.step(now, count)
        decisions.append(d)
        if d in (TO_EP, TO_TP):
            now += switch_time_s
    return {"time": now, "modes": modes, "decisions": decisions}
