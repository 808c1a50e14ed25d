// The EP/TP switch policy and its start-up crossover calibration (Moebius
// review, §4.5): host code, no GPU.  Declared in include/moe.h.
//
// One call per decode iteration, after the step: the count of in-flight
// requests enters a window of the last W counts; in TP the mode switches to EP
// as soon as the count exceeds T_h, in EP it switches back when the window's
// mean falls below T_l (T_l <= T_h: hysteresis).  After a switch, or a switch
// cancelled because the target mode's KV capacity cannot hold the live
// requests, no decision is taken for the cooldown C.  The window keeps an
// exact integer sum, so the mean is one correctly rounded division.
#include <cmath>

#include "moe.h"

namespace {

bool is_fin(double v) { return std::isfinite(v); }

bool params_ok(const moe_switch_params* p) {
  return p && is_fin(p->t_high) && is_fin(p->t_low) && p->t_low <= p->t_high && p->window >= 1 &&
         p->window <= MOE_SWITCH_WINDOW_MAX && is_fin(p->cooldown_s) && p->cooldown_s >= 0 &&
         is_fin(p->kv_cap_tp) && is_fin(p->kv_cap_ep);
}

}  // namespace

extern "C" {

int moe_switch_init(const moe_switch_params* p, int mode, moe_switch_state* s) {
  if (!params_ok(p) || !s || (mode != MOE_MODE_TP && mode != MOE_MODE_EP)) return MOE_EINVAL;
  s->p = *p;
  s->mode = mode;
  s->have_last = 0;
  s->t_last = 0.0;
  s->n_samples = 0;
  s->head = 0;
  s->window_sum = 0;
  for (int i = 0; i < MOE_SWITCH_WINDOW_MAX; ++i) s->ring[i] = 0;
  return MOE_OK;
}

int moe_switch_step(moe_switch_state* s, double now_s, int in_flight, int* decision) {
  if (!s || !decision || !is_fin(now_s) || in_flight < 0 || !params_ok(&s->p)) return MOE_EINVAL;
  const moe_switch_params& p = s->p;
  // window of the last W counts: ring slot `head` holds the oldest once full
  if (s->n_samples >= p.window) s->window_sum -= s->ring[s->head];
  s->ring[s->head] = in_flight;
  s->window_sum += in_flight;
  s->head = (s->head + 1) % p.window;
  s->n_samples += 1;

  *decision = MOE_SWITCH_STAY;
  if (s->have_last && now_s < s->t_last + p.cooldown_s) return MOE_OK;
  bool want;
  int target;
  if (s->mode == MOE_MODE_TP) {
    want = static_cast<double>(in_flight) > p.t_high;
    target = MOE_MODE_EP;
  } else {
    want = s->n_samples >= p.window &&
           static_cast<double>(s->window_sum) / static_cast<double>(p.window) < p.t_low;
    target = MOE_MODE_TP;
  }
  if (!want) return MOE_OK;
  s->have_last = 1;
  s->t_last = now_s;
  const double cap = target == MOE_MODE_EP ? p.kv_cap_ep : p.kv_cap_tp;
  if (cap > 0 && static_cast<double>(in_flight) > cap) {
    *decision = MOE_SWITCH_VETOED;
    return MOE_OK;
  }
  s->mode = target;
  *decision = target == MOE_MODE_EP ? MOE_SWITCH_TO_EP : MOE_SWITCH_TO_TP;
  return MOE_OK;
}

int moe_switch_crossover(const double* batches, const double* t_tp, const double* t_ep, int n,
                         double* b_star) {
  if (!batches || !t_tp || !t_ep || !b_star || n < 1) return MOE_EINVAL;
  for (int i = 0; i < n; ++i) {
    if (!is_fin(batches[i]) || !is_fin(t_tp[i]) || !is_fin(t_ep[i])) return MOE_EINVAL;
    if (i > 0 && !(batches[i - 1] < batches[i])) return MOE_EINVAL;
  }
  for (int i = 0; i < n; ++i) {
    if (t_ep[i] <= t_tp[i]) {
      if (i == 0) {
        *b_star = batches[0];
      } else {
        // d = t_ep - t_tp is > 0 at i - 1 and <= 0 at i: its linear zero
        const double d0 = t_ep[i - 1] - t_tp[i - 1];
        const double d1 = t_ep[i] - t_tp[i];
        const double b0 = batches[i - 1];
        *b_star = b0 + (batches[i] - b0) * d0 / (d0 - d1);
      }
      return MOE_OK;
    }
  }
  *b_star = INFINITY;
  return MOE_OK;
}

}  // extern "C"
