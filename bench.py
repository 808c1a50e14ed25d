"""Benchmark: MoE-layer forward tokens/s against the global batch B on one
MI355X, with the HBM roofline fraction of every point and the CPU oracle
timed beside the headline point.

    python bench.py [--steps K] [--warmup W]          # the batch sweep (one JSON line)
    python bench.py --workload NAME --tokens T --routing R   # one point only
    python bench.py --workload repack               # EP<->TP expert-weight repack
    python bench.py --workload dispatch [--tokens T] # EP dispatch send layout + return combine
    python bench.py --workload calibrate --steps 20  # EP/TP crossover across B + switch policy
    python bench.py --workload schedule              # Attention-DP request scheduling
    python bench.py --ingest-counters FETCH.csv WRITE.csv --workload NAME --tokens T --routing R

A step is one pass of the whole hot path (gate GEMM + softmax/top-k + permute
in one launch, expert up-projection with SiLU*up, down-projection, combine:
four launches) over one batch of seeded synthetic input already resident in
HBM.  Weights are rotated over enough bit-identical copies (>= 1 GB in total)
that the 256 MB Infinity Cache cannot serve them.

The default run times the Qwen3-235B-A22B EP rank share (16 whole experts of
128) and TP rank share (every expert's 1/8 slice), P = 8, for B = 8 .. 2048
under uniform and Zipf routing (the decode-step sweep of the Moebius review,
section 2.1 and Fig. 2), then the Qwen3-30B-A3B batch sweep and the
DeepSeek-V2-Lite layer at T = 256.  `value` is the EP share at B = 64,
uniform routing; every point of the sweep is in `by_batch`.  Prints ONE JSON
line (the benchmark runs on one GPU only: the path is one GPU's share of a
sharded layer); progress goes to stderr.
"""
import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s vs batch B at 1 GPU; achieved HBM TB/s (% of peak)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 1.0e9
HEADLINE = ("qwen3_235b_ep", 64, "uniform")
SWEEP = ("qwen3_235b_ep", "qwen3_235b_tp")
EXTRA_SWEEP = "qwen3_30b"
C2 = ("dsv2_lite", 256, "uniform")
DECODE_TARGET = 0.70          # fraction of HBM peak on the EP/TP decode points
DECODE_BATCHES = (16, 32, 64, 128, 256)
MEDIAN_BLOCKS = 5             # blocks of K steps behind ms_per_step_median
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "expert_up_counters.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def bench_repack(steps, warmup):
    """EP->TP local permute of one Qwen3-235B-shaped EP rank (16 experts, P=8):
    a pure copy of 604 MB read + 604 MB written; the TP->EP inverse (the
    switch back) is timed beside it."""
    import torch

    import moe_layer_amd
    from moe_inputs import get_config, make_repack_inputs
    cfg = get_config("qwen3_235b_tp")
    r = make_repack_inputs(cfg, rank=0)
    import numpy as np
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    w13, w2 = dev(r["w13_ep"]), dev(r["w2_ep"])
    P, E_l, Ip = cfg.P, cfg.E // cfg.P, cfg.I // cfg.P
    d13 = [torch.empty((E_l, 2 * Ip, cfg.H), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    d2 = [torch.empty((E_l, cfg.H, Ip), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    r13, r2 = torch.empty_like(w13), torch.empty_like(w2)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps * 1e-3

    t = timed(lambda: moe_layer_amd.moe_repack_ep_to_tp(w13, w2, P, d13, d2))
    t_back = timed(lambda: moe_layer_amd.moe_repack_tp_to_ep(d13, d2, P, r13, r2))
    moved = 2 * (w13.numel() + w2.numel()) * 2
    gbs = moved / t / 1e9
    gbs_back = moved / t_back / 1e9
    return {
        "metric": "EP->TP expert-weight repack throughput (read + write)",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": t * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "repack 16 EP experts of Qwen3-235B-A22B shape into 8 TP blocks",
                   "bytes_read": moved // 2, "bytes_written": moved // 2},
        "roofline": {"bound": "hbm", "kernel": "repack", "achieved": gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": None},
        "tp_to_ep": {"ms_per_step": t_back * 1e3, "achieved_GBs": gbs_back,
                     "frac": gbs_back / HBM_PEAK_GBS},
    }


def bench_dispatch(steps, warmup, T_main, routing, cpu=True):
    """EP dispatch send side on one Qwen3-235B-shaped EP rank (P = 8, 16
    experts per rank, H = 4096, top-8): pairs sorted by owning rank and their
    token rows copied into the send buffer (moe_dispatch: two launches), and
    the return leg beside it (moe_combine of the returned rows with the
    dispatch's pair positions and the routing weights).  T is this rank's own
    (data-parallel) tokens; the routing table is a seeded draw.  Each call is
    timed inside a replayed HIP graph of 20 calls."""
    import numpy as np
    import torch

    import moe_layer_amd as M
    from moe_inputs import get_config
    from moe_inputs.gen import make_x, routing_table
    cfg = get_config("qwen3_235b_ep")
    P, E_l, H, k = cfg.P, cfg.E // cfg.P, cfg.H, cfg.k

    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    def one(T):
        xh, idh = make_x(cfg, T, T_draw=T), routing_table(cfg, T, routing)
        x, ids = dev(xh), dev(idh)
        w = torch.rand((T, k), dtype=torch.float32, device="cuda")
        n = T * k
        i32 = lambda m: torch.empty(m, dtype=torch.int32, device="cuda")
        counts, offsets, order, pos, sids = i32(P), i32(P + 1), i32(n), i32(n), i32(n)
        send_x = torch.empty((n, H), dtype=torch.bfloat16, device="cuda")
        y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        go = lambda: M.moe_dispatch(x, ids, E_l, P, counts, offsets, order, pos, send_x, sids)
        back = lambda: M.moe_combine(send_x, pos, w, y)   # returned rows stand in for expert outputs

        def timed(fn, reps=20):
            """Mean time per call: `reps` calls captured in one HIP graph,
            replayed `steps` times between two events on the replay stream
            (the calls are a few microseconds each; replay keeps the host's
            launch cost out of the figure)."""
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                fn()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(reps):
                    fn()
            for _ in range(max(1, warmup)):
                g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e-3 / (steps * reps)

        t_d, t_c = timed(go), timed(back)
        n_sent = int(offsets[-1].item())
        bytes_d = 2 * H * (T + n_sent) + 4 * (2 * T * k + 2 * n_sent)
        bytes_c = 2 * H * (n_sent + T) + 8 * T * k
        return {"T": T, "n_sent": n_sent, "dispatch_us": t_d * 1e6, "dispatch_GBs": bytes_d / t_d / 1e9,
                "dispatch_bytes": bytes_d, "return_combine_us": t_c * 1e6,
                "return_combine_GBs": bytes_c / t_c / 1e9, "host": (xh, idh)}

    rows = [one(T) for T in sorted({32, 256, 1024, 2048, T_main})]
    main = next(r for r in rows if r["T"] == T_main)
    frac = main["dispatch_GBs"] / HBM_PEAK_GBS
    cpu_line = None
    if cpu:
        import oracle
        xh, idh = main["host"]
        runs, tot = 0, 0.0
        while runs == 0 or (tot < 10.0 and runs < 200):
            t0 = time.perf_counter()
            oracle.dispatch(xh, idh, E_l, P)
            tot += time.perf_counter() - t0
            runs += 1
        cpu_line = {"value": main["dispatch_bytes"] / (tot / runs) / 1e9, "unit": "GB/s", "cores": 1,
                    "kind": "oracle", "sample": f"oracle.dispatch on the same T={T_main} rank share, "
                                                f"{runs} run(s), mean {tot / runs * 1e3:.2f} ms (numpy, one thread)"}
    for r in rows:
        r.pop("host")
    return {
        "metric": "EP dispatch send-layout throughput (algorithmic HBM bytes / time)",
        "value": main["dispatch_GBs"], "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": main["dispatch_us"] * 1e-3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded x, seeded routing table)",
        "config": {"workload": f"EP dispatch of one Qwen3-235B-A22B-shaped rank share: T={T_main} own "
                               f"tokens, top-{k} of 128 experts, P={P} ranks of {E_l}, H={H}, {routing}",
                   "rows_sent": main["n_sent"]},
        "roofline": {"bound": "hbm", "kernel": "dispatch_kernel (rank counts, ranking and row copy in one launch)",
                     "achieved": main["dispatch_GBs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": frac, "traffic": None,
                     "algorithmic_bytes_per_launch": main["dispatch_bytes"]},
        "by_tokens": [{k2: (round(v, 3) if isinstance(v, float) else v) for k2, v in r.items()}
                      for r in rows],
        "cpu_baseline": cpu_line,
    }


def bench_calibrate(steps, warmup):
    """The start-up calibration of the EP/TP switch on this GPU: the layer
    step of one Qwen3-235B-A22B EP rank share and one TP rank share (P = 8,
    uniform routing) across the global batch B, their crossover
    (moe_switch_crossover), and the switch policy driven over seeded
    synthetic load traces with those step times (one layer per iteration;
    a switch costs one measured EP->TP repack of the layer).  One GPU shows
    the expert side only: the exchange (all-reduce or all-to-all) and
    attention, which move the pages' crossover, are not in these times."""
    import numpy as np
    import torch

    import moe_layer_amd as M
    from moe_inputs import get_config
    from moe_inputs.gen import load_trace
    batches = list(get_config("qwen3_235b_ep").T_list)
    t = {"tp": [], "ep": []}
    for view in ("tp", "ep"):
        ws = WeightSet(f"qwen3_235b_{view}", "uniform")
        for B in batches:
            wl = Workload(ws, B)
            tm = time_workload(wl, steps, warmup)
            t[view].append(tm["t_step_s"])
            del wl
        del ws
        torch.cuda.empty_cache()
    b_star = M.switch_crossover(batches, t["tp"], t["ep"])
    rep = bench_repack(max(3, steps // 4), 1)
    switch_s = rep["ms_per_step"] * 1e-3
    logb = np.log2(np.asarray(batches, dtype=np.float64))

    def step_time(mode, count):
        x = np.log2(min(max(count, batches[0]), batches[-1]))
        return float(np.interp(x, logb, t["ep"] if mode == M.MODE_EP else t["tp"]))

    sims = {}
    for kind, (t_low_f, window) in (("burst", (0.8, 8)), ("rollout", (1.0, 1))):
        counts, _ = load_trace(kind, 3000, seed=0)
        out = {}
        for name, th in (("pages_T_h_256", 256.0), ("calibrated", b_star)):
            if not math.isfinite(th):
                continue
            pol = M.SwitchPolicy(th, t_low_f * th, window, 5e-3)   # cooldown scaled to one-layer steps
            now, switches = 0.0, 0
            for c in counts:
                now += step_time(pol.mode, int(c))
                d = pol.step(now, int(c))
                if d in (M.SWITCH_TO_EP, M.SWITCH_TO_TP):
                    now += switch_s
                    switches += 1
            out[name] = {"T_h": th, "time_s": now, "switches": switches}
        out["always_tp_s"] = sum(step_time(M.MODE_TP, int(c)) for c in counts)
        out["always_ep_s"] = sum(step_time(M.MODE_EP, int(c)) for c in counts)
        sims[kind] = out
    return {
        "metric": "EP/TP layer-step crossover batch on one GPU (start-up switch calibration)",
        "value": b_star, "unit": "global batch B", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": None, "higher_is_better": None, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Qwen3-235B-A22B EP and TP rank shares (P = 8), uniform routing, "
                               "B = 8..2048; policy over seeded burst / rollout load traces"},
        "layer_step_us": {"B": batches, "tp": [round(v * 1e6, 2) for v in t["tp"]],
                          "ep": [round(v * 1e6, 2) for v in t["ep"]]},
        "switch_cost_us": round(switch_s * 1e6, 1),
        "policy_simulation": sims,
    }


def bench_schedule(steps, warmup, n_req=2048, E=8, cpu=True):
    """Attention-DP request scheduling (Sem-MoE notes): 2048 synthetic requests
    (log-normal lengths, median 300 tokens, 60 % of tokens from a topic
    cluster) over E = 8 ranks, Qwen3 vocabulary (151 936 ids); one call =
    per-request cluster counts, argmax ranks and balanced ranks, timed inside
    a replayed HIP graph of 20 calls."""
    import numpy as np
    import torch

    import moe_layer_amd as M
    from moe_inputs.gen import make_requests
    tok, off, cl, _ = make_requests(n_req, E, seed=0)
    t = torch.from_numpy(tok).cuda()
    o = torch.from_numpy(off).cuda()
    c = torch.from_numpy(cl).cuda()
    scores = torch.empty((n_req, E), dtype=torch.int32, device="cuda")
    aff = torch.empty(n_req, dtype=torch.int32, device="cuda")
    asg = torch.empty(n_req, dtype=torch.int32, device="cuda")
    ws = M.schedule_workspace(n_req, E)
    go = lambda: M.moe_schedule_requests(t, o, c, E, scores, aff, asg, ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        go()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    reps = 20
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            go()
    for _ in range(max(1, warmup)):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    t_call = e0.elapsed_time(e1) * 1e-3 / (steps * reps)
    n_tok = int(tok.size)
    nbytes = 4 * n_tok + 4 * cl.size + 4 * (n_req + 1) + 4 * n_req * (E + 2)
    gbs = nbytes / t_call / 1e9
    cpu_line = None
    if cpu:
        import oracle
        rs = oracle.request_schedule
        k = 64
        t0 = time.perf_counter()
        sc = rs.cluster_scores(tok[:off[k]], off[:k + 1], cl, E)
        rs.balanced_ranks(sc)
        dt = time.perf_counter() - t0
        cpu_line = {"value": k / dt, "unit": "requests/s", "cores": 1, "kind": "oracle",
                    "sample": f"oracle cluster_scores + balanced_ranks on the first {k} requests "
                              f"({int(off[k])} tokens), {dt:.2f} s (pure Python, one thread)"}
    return {
        "metric": "Attention-DP request scheduling throughput",
        "value": n_req / t_call, "unit": "requests/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": t_call * 1e3, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "int32", "data": "synthetic (seeded requests and token clusters)",
        "config": {"workload": f"{n_req} requests, {n_tok} tokens, E = {E} ranks, vocabulary {cl.size}"},
        "roofline": {"bound": "hbm", "kernel": "schedule_kernel", "achieved": gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": nbytes},
        "tokens_per_s": n_tok / t_call,
        "cpu_baseline": cpu_line,
    }


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=None)
    p.add_argument("--tokens", type=int, default=None)
    p.add_argument("--routing", default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="default run: leave out the Qwen3-30B sweep and the DeepSeek-V2-Lite point")
    p.add_argument("--graph", action="store_true", help="single point: also time HIP-graph replay")
    p.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"), default=None,
                   help="record rocprofv3 FETCH_SIZE / WRITE_SIZE counter files of the up-projection "
                        "for --workload/--tokens/--routing in the profiles' counter table")
    p.add_argument("--command", default="", help="with --ingest-counters: the commands that made the files")
    return p.parse_args()


def kernel_source_sha():
    h = hashlib.sha256()
    for f in ("expert_gemm.hip", "expert_coop.hip", "expert_tile.hip", "stream_ops.hpp", "common.hpp",
              "moe_internal.h"):
        with open(os.path.join(ROOT, "moe_layer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _to_dev(a):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


class WeightSet:
    """One view's seeded inputs on the GPU, drawn once at the largest batch:
    x (T_max, H) -- a batch of T tokens is its first T rows --, the gate, the
    bias of the routing variant and the expert weights, replicated for cache
    rotation."""

    def __init__(self, name, routing):
        from moe_inputs import get_config, make_layer_inputs
        self.cfg = cfg = get_config(name)
        self.routing = routing
        self.host = make_layer_inputs(cfg, cfg.T_max, routing=routing)
        self.x = _to_dev(self.host["x"])
        self.w_gate = _to_dev(self.host["w_gate"])
        self.bias = _to_dev(self.host["gate_bias"])
        w13, w2 = _to_dev(self.host["w13"]), _to_dev(self.host["w2"])
        wbytes = (w13.numel() + w2.numel()) * w13.element_size()
        self.copies = max(1, math.ceil(ROTATE_BYTES / wbytes))
        self.w13 = [w13] + [w13.clone() for _ in range(self.copies - 1)]
        self.w2 = [w2] + [w2.clone() for _ in range(self.copies - 1)]
        self.g_begin = self.host["g_begin"]
        self.rank = self.host["rank"]


class Workload:
    """A batch of T tokens on a WeightSet, with its output buffers."""

    def __init__(self, ws, T):
        import torch

        import moe_layer_amd
        self.ws, self.cfg, self.T, self.routing = ws, ws.cfg, T, ws.routing
        self.x = ws.x[:T]
        self.w_gate, self.bias, self.g_begin = ws.w_gate, ws.bias, ws.g_begin
        self.w13, self.w2, self.copies = ws.w13, ws.w2, ws.copies
        self.dtype = torch.bfloat16 if self.cfg.dtype == "bf16" else torch.float32
        self.elem = 2 if self.cfg.dtype == "bf16" else 4
        c = self.cfg
        self.bufs = moe_layer_amd.MoeLayerBuffers.allocate(T, c.H, c.E, c.kk, c.n_groups, c.I_local,
                                                           self.dtype)

    def host_inputs(self):
        d = dict(self.ws.host)
        d["x"] = d["x"][:self.T]
        return d

    def describe(self):
        c = self.cfg
        return {
            "workload": f"{c.name} B={self.T} {self.routing} ({c.view} view"
                        + (f", rank {self.ws.rank} of {c.P}" if c.view != "full" else "") + ")",
            "tokens": self.T, "hidden": c.H, "experts": c.E, "top_k": c.k,
            "renormalised": c.renorm, "shared_experts": c.n_shared, "intermediate_local": c.I_local,
            "groups_held": c.n_groups, "view": c.view, "ranks_P": c.P, "rank": self.ws.rank,
            "routing": self.routing, "weight_copies_rotated": self.copies,
        }


def run_step(wl, i, events=None, up_events=None):
    """One pass of the hot path; optional events bracket each call (events)
    or the up-projection only (up_events)."""
    import moe_layer_amd as m
    c, b = wl.cfg, wl.bufs
    w13, w2 = wl.w13[i % wl.copies], wl.w2[i % wl.copies]
    ev = events
    if ev: ev[0].record()
    m.moe_route_permute(wl.x, wl.w_gate, wl.bias, c.k, c.renorm, c.n_shared, b.logits, b.topk_ids,
                        b.topk_w, wl.g_begin, c.n_groups, b.counts, b.offsets, b.sorted_pair,
                        b.pair_pos, b.route_ws)
    if ev: ev[1].record()
    if up_events: up_events[0].record()
    m.moe_expert_up(wl.x, b.sorted_pair, b.offsets, c.kk, w13, b.a, b.expert_ws)
    if up_events: up_events[1].record()
    if ev: ev[2].record()
    m.moe_expert_down(b.a, b.offsets, wl.T, c.kk, w2, b.y_pair, b.expert_ws)
    if ev: ev[3].record()
    m.moe_combine(b.y_pair, b.pair_pos, b.topk_w, b.y)
    if ev: ev[4].record()


def algorithmic(wl):
    """Bytes and flops the method must move / do (intermediates excluded):
    the gate matrix, x, y and the W13 + W2 of every touched group (touched =
    a non-zero count on the GPU's own routing)."""
    c, s, T = wl.cfg, wl.elem, wl.T
    counts = wl.bufs.counts.cpu().numpy()
    touched = int((counts > 0).sum())
    kept = int(counts.sum())
    w13_bytes = touched * 2 * c.I_local * c.H * s
    w2_bytes = touched * c.H * c.I_local * s
    layer_bytes = s * c.E * c.H + 2 * s * T * c.H + w13_bytes + w2_bytes
    layer_flops = 2 * T * c.H * c.E + kept * 6 * c.H * c.I_local
    up_bytes = w13_bytes + s * T * c.H
    up_flops = kept * 4 * c.H * c.I_local
    return dict(touched=touched, kept=kept, layer_bytes=layer_bytes, layer_flops=layer_flops,
                up_bytes=up_bytes, up_flops=up_flops)


def time_workload(wl, steps, warmup, graph=False):
    """K timed steps between two synchronisations, with nothing but the four
    calls in the loop: an event record is a queue packet of its own and costs
    the GPU ~5 us of idle time, so events would inflate the step.  Then
    MEDIAN_BLOCKS - 1 more blocks of K steps (the median of the block means
    is ms_per_step_median).  Then K up-projection launches back to back on
    the last step's routing between two HIP events on the launch stream: the
    dominant kernel's duration.  A last pass with events around every call
    gives the other kernels' durations (those include the event packets).
    With graph=True the step is also captured in HIP graphs (one per weight
    copy) and K replays are timed the same way."""
    import torch
    for i in range(warmup):
        run_step(wl, i)
    torch.cuda.synchronize()
    blocks = []
    for blk in range(MEDIAN_BLOCKS):
        t0 = time.perf_counter()
        for i in range(steps):
            run_step(wl, i)
        torch.cuda.synchronize()
        blocks.append((time.perf_counter() - t0) / steps)
    t_step = blocks[0]          # the K timed steps
    # The up-projection's own duration: K launches back to back (on the last
    # step's routing, weight copies rotated) between two events on the launch
    # stream, so no event packet sits between launches.
    import moe_layer_amd as m
    c, b = wl.cfg, wl.bufs
    e_up0, e_up1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e_up0.record()
    for i in range(steps):
        m.moe_expert_up(wl.x, b.sorted_pair, b.offsets, c.kk, wl.w13[i % wl.copies], b.a, b.expert_ws)
    e_up1.record()
    torch.cuda.synchronize()
    t_up_us = e_up0.elapsed_time(e_up1) / steps * 1e3
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        run_step(wl, i, evs[i])
    torch.cuda.synchronize()
    names = ("route_permute", "expert_up", "expert_down", "combine")
    per = {n: sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)) / steps * 1e3
           for j, n in enumerate(names)}
    out = {"t_step_s": t_step, "t_step_median_s": statistics.median(blocks), "t_up_us": t_up_us,
           "kernels_us": per, "steps": steps, "warmup": warmup}
    if graph:
        out["t_step_graph_s"] = time_graph(wl, steps)
    return out


def time_graph(wl, steps):
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run_step(wl, 0)
    torch.cuda.current_stream().wait_stream(s)
    graphs = []
    for c in range(wl.copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run_step(wl, c)
        graphs.append(g)
    for i in range(3):
        graphs[i % wl.copies].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % wl.copies].replay()
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / steps
    del graphs
    return t


def _load_counters():
    try:
        with open(PROFILE_COUNTERS) as f:
            return json.load(f)
    except (OSError, ValueError):
        return None


def measured_traffic(name, T, routing):
    """HBM bytes per up-projection launch of exactly this workload, batch and
    routing, from committed rocprofv3 counters (FETCH_SIZE and WRITE_SIZE in
    KiB per dispatch, each scaled by what the same counter reads for a copy of
    known size), or None when no entry matches or the entry was taken on a
    different kernel source."""
    c = _load_counters()
    if not c:
        return None
    sha = kernel_source_sha()
    for e in c.get("entries", []):
        if (e.get("workload"), e.get("T"), e.get("routing"), e.get("source_sha")) == (name, T, routing, sha):
            return (e["fetch_kib"] * c["fetch_scale"] + e["write_kib"] * c["write_scale"]) * 1024.0
    return None


def ingest_counters(fetch_csv, write_csv, name, T, routing, command):
    """Record the up-projection's mean FETCH_SIZE and WRITE_SIZE per dispatch
    (rocprofv3 --pmc counter_collection.csv files, one counter per run) for
    this workload in the counter table bench.py reads."""
    import csv

    def mean_kib(path, counter):
        vals = {}
        with open(path) as f:
            for row in csv.DictReader(f):
                kname = row.get("Kernel_Name", "")
                if not ("expert_wave_kernel" in kname or "expert_coop_kernel" in kname) or ", 0, " not in kname:
                    continue   # the up-projection: expert_{wave,coop}_kernel<T, 0, ...>
                if row.get("Counter_Name") != counter:
                    continue
                vals.setdefault(row.get("Dispatch_Id"), 0.0)
                vals[row.get("Dispatch_Id")] += float(row["Counter_Value"])
        if not vals:
            raise SystemExit(f"no {counter} rows of the up-projection in {path}")
        return sum(vals.values()) / len(vals), len(vals)

    fk, nf = mean_kib(fetch_csv, "FETCH_SIZE")
    wk, nw = mean_kib(write_csv, "WRITE_SIZE")
    c = _load_counters() or {}
    c.setdefault("fetch_scale", 1.9994)
    c.setdefault("write_scale", 0.9997)
    entries = [e for e in c.get("entries", []) if (e.get("workload"), e.get("T"), e.get("routing")) != (name, T, routing)]
    new = {"workload": name, "T": T, "routing": routing, "kernel": "moe_expert_up (expert_{wave,coop}_kernel<bf16, UP, ...>)",
           "source_sha": kernel_source_sha(), "fetch_kib": round(fk, 1), "write_kib": round(wk, 1),
           "dispatches": min(nf, nw), "commands": command}
    c["entries"] = sorted(entries + [new], key=lambda e: (e["workload"], e["routing"], e["T"]))
    with open(PROFILE_COUNTERS, "w") as f:
        json.dump(c, f, indent=1)
        f.write("\n")
    print(json.dumps(new))


def cpu_baseline(wl, budget_s=10.0):
    """The oracle (numpy float64) on the same inputs, on this host's cores."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - reporting only
        cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    c, d = wl.cfg, wl.host_inputs()
    runs, t_total = 0, 0.0
    while runs == 0 or (t_total < budget_s and runs < 30):
        t0 = time.perf_counter()
        oracle.moe_layer(d["x"], d["w_gate"], d["gate_bias"], d["w13"], d["w2"], c.k, c.renorm,
                         c.n_shared, d["g_begin"])
        t_total += time.perf_counter() - t0
        runs += 1
    t = t_total / runs
    return {"value": wl.T / t, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"whole layer of {wl.describe()['workload']}, {runs} run(s), mean {t:.2f} s per pass "
                      f"(numpy float64, BLAS threads={cores}, CPUs visible={len(os.sched_getaffinity(0))})"}


def copy_ceiling(nbytes=1 << 30, reps=20):
    """A plain device copy (torch's copy kernel) of nbytes: read + write rate,
    the measured ceiling beside the 8 TB/s peak."""
    import torch
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    gbs = 2 * nbytes / t / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"kernel": "torch copy_ of a 1 GiB bf16 tensor (read + write)", "GBs": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "us": round(t * 1e6, 1)}


def point(wl, tm):
    """One sweep point: tokens/s, step times, the up-projection's and the
    layer's HBM fractions (algorithmic bytes / time)."""
    a = algorithmic(wl)
    t, tg = tm["t_step_s"], tm.get("t_step_graph_s")
    up_gbs = a["up_bytes"] / (tm["t_up_us"] * 1e-6) / 1e9
    row = {
        "view": wl.cfg.view, "routing": wl.routing, "B": wl.T,
        "tokens_per_s": round(wl.T / t, 1),
        "ms_per_step": round(t * 1e3, 5),
        "ms_per_step_median": round(tm["t_step_median_s"] * 1e3, 5),
        "graph_ms_per_step": round(tg * 1e3, 5) if tg else None,
        "layer_hbm_frac": round(a["layer_bytes"] / t / 1e9 / HBM_PEAK_GBS, 4),
        "layer_hbm_frac_median": round(a["layer_bytes"] / tm["t_step_median_s"] / 1e9 / HBM_PEAK_GBS, 4),
        "layer_mfma_frac": round(a["layer_flops"] / t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "up_frac": round(up_gbs / HBM_PEAK_GBS, 4),
        "up_us": round(tm["t_up_us"], 2),
        "layer_bytes": a["layer_bytes"], "up_bytes": a["up_bytes"],
        "touched_groups": a["touched"], "kept_pairs": a["kept"],
        "kernels_us": {k: round(v, 2) for k, v in tm["kernels_us"].items()},
        "up_traffic": measured_traffic(wl.cfg.name, wl.T, wl.routing),
    }
    if wl.cfg.view == "ep":
        row["rank"] = wl.ws.rank
    return row


def report(wl, tm, cpu=None):
    """The full line of one point (the headline, or a single-point run)."""
    a = algorithmic(wl)
    t = tm["t_step_s"]
    t_up = tm["t_up_us"] * 1e-6
    achieved = a["up_bytes"] / t_up / 1e9
    line = {
        "metric": METRIC,
        "value": wl.T / t,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": tm["steps"],
        "warmup": tm["warmup"],
        "ms_per_step": t * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,1/fan_in) weights; no trained weights)",
        "config": wl.describe(),
        "roofline": {
            "bound": "hbm",
            "kernel": "expert_up (W13 grouped GEMM + SiLU*up)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(wl.cfg.name, wl.T, wl.routing),
            "algorithmic_bytes_per_launch": a["up_bytes"],
        },
        "layer": {
            "hbm_achieved_GBs": a["layer_bytes"] / t / 1e9,
            "hbm_frac": a["layer_bytes"] / t / 1e9 / HBM_PEAK_GBS,
            "tflops": a["layer_flops"] / t / 1e12,
            "mfma_frac": a["layer_flops"] / t / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "algorithmic_bytes": a["layer_bytes"],
            "touched_groups": a["touched"],
            "kept_pairs": a["kept"],
            "kernels_us": {k: round(v, 2) for k, v in tm["kernels_us"].items()},
            "expert_up_us_timed_region": round(tm["t_up_us"], 2),
            "ms_per_step_median": tm["t_step_median_s"] * 1e3,
        },
        "cpu_baseline": cpu,
    }
    if "t_step_graph_s" in tm:
        tg = tm["t_step_graph_s"]
        line["layer"]["graph_replay"] = {"ms_per_step": tg * 1e3, "tokens_per_s": wl.T / tg,
                                         "hbm_frac": a["layer_bytes"] / tg / 1e9 / HBM_PEAK_GBS}
    return line


def bench_default(steps, warmup, cpu=True, extra=True):
    """The batch sweep on the Qwen3-235B-A22B EP and TP rank shares (and,
    with extra, the Qwen3-30B-A3B sweep and the DeepSeek-V2-Lite layer)."""
    import torch
    from moe_inputs import get_config
    rows, extra_rows, head, c2 = [], [], None, None
    plan = [(name, r) for name in SWEEP for r in get_config(name).routing]
    if extra:
        plan += [(EXTRA_SWEEP, r) for r in get_config(EXTRA_SWEEP).routing]
    for name, routing in plan:
        ws = WeightSet(name, routing)
        for T in ws.cfg.T_list:
            wl = Workload(ws, T)
            tm = time_workload(wl, steps, warmup, graph=True)
            row = point(wl, tm)
            (rows if name in SWEEP else extra_rows).append(row)
            log(f"{name} {routing} B={T}: {row['ms_per_step'] * 1e3:.1f} us/step, layer "
                f"{row['layer_hbm_frac']:.3f}, up {row['up_frac']:.3f} of HBM peak")
            if (name, T, routing) == HEADLINE:
                head = report(wl, tm, cpu_baseline(wl) if cpu else None)
                log(f"headline cpu baseline: {head['cpu_baseline']}")
            del wl
        del ws
        torch.cuda.empty_cache()
    if extra:
        ws = WeightSet(C2[0], C2[2])
        wl = Workload(ws, C2[1])
        tm = time_workload(wl, steps, warmup, graph=True)
        c2 = point(wl, tm)
        c2["workload"] = wl.describe()["workload"]
        c2["up_traffic"] = measured_traffic(*C2)
        log(f"{C2}: {c2['ms_per_step'] * 1e3:.1f} us/step, layer {c2['layer_hbm_frac']:.3f}")
        del wl, ws
        torch.cuda.empty_cache()
    line = head
    line["config"] = {
        "workload": "Qwen3-235B-A22B-shaped EP rank share (16 of 128 experts, W13 (16,3072,4096)) and TP "
                    "rank share (128 experts sharded I/8, W13 (128,384,4096)), P=8, layer step across "
                    "global batch B=8..2048, uniform and Zipf(1.2) routing; value = EP share, B=64, uniform",
        "headline": head["config"],
        "batches": list(get_config(SWEEP[0]).T_list),
        "views": ["ep", "tp"],
        "routings": ["uniform", "zipf"],
    }
    line["by_batch"] = rows
    dec = [r for r in rows if r["routing"] == "uniform" and r["B"] in DECODE_BATCHES]
    line["decode_target"] = {
        "points": "EP and TP shares, uniform routing, B=" + ",".join(map(str, DECODE_BATCHES)),
        "target_layer_hbm_frac": DECODE_TARGET,
        "min_layer_hbm_frac": min(r["layer_hbm_frac"] for r in dec),
        "min_layer_hbm_frac_median": min(r["layer_hbm_frac_median"] for r in dec),
        "met": all(r["layer_hbm_frac"] >= DECODE_TARGET for r in dec),
    }
    if extra:
        line["qwen3_30b_by_batch"] = extra_rows
        line["dsv2_lite"] = c2
    line["copy_ceiling"] = copy_ceiling()
    return line


def main():
    args = parse()
    if args.ingest_counters:
        if not (args.workload and args.tokens and args.routing):
            raise SystemExit("--ingest-counters needs --workload, --tokens and --routing")
        ingest_counters(*args.ingest_counters, args.workload, args.tokens, args.routing, args.command)
        return
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only (asked for --gpus {args.gpus}); "
              "it times one GPU's share (the EP and TP rank views), and no collectives are run.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    import moe_layer_amd
    moe_layer_amd.lib()

    if args.workload is None:
        print(json.dumps(bench_default(args.steps, args.warmup, cpu=not args.no_cpu_baseline,
                                       extra=not args.no_extra)), flush=True)
        return
    if args.workload == "repack":
        print(json.dumps(bench_repack(args.steps, args.warmup)), flush=True)
        return
    if args.workload == "schedule":
        print(json.dumps(bench_schedule(args.steps, args.warmup, cpu=not args.no_cpu_baseline)), flush=True)
        return
    if args.workload == "calibrate":
        print(json.dumps(bench_calibrate(args.steps, args.warmup)), flush=True)
        return
    if args.workload == "dispatch":
        print(json.dumps(bench_dispatch(args.steps, args.warmup, args.tokens or 256,
                                        args.routing or "uniform", not args.no_cpu_baseline)),
              flush=True)
        return

    from moe_inputs import get_config
    cfg = get_config(args.workload)
    T = args.tokens or cfg.T_list[-1]
    routing = args.routing or cfg.routing[0]
    wl = Workload(WeightSet(args.workload, routing), T)
    tm = time_workload(wl, args.steps, args.warmup, graph=args.graph)
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl)
    print(json.dumps(report(wl, tm, cpu)), flush=True)


if __name__ == "__main__":
    main()
