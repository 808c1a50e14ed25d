"""GPU parity of the EP dispatch: the send layout bit-exact against the
oracle (counts, offsets, send order, pair positions, expert ids and the
copied rows), and the whole exchange -- every rank's dispatch, the receivers'
expert pass and un-permute, the senders' combine -- against the oracle's
P-rank layer.  The all-to-all itself is plain tensor slicing here: this GPU
plays every rank in turn."""
import numpy as np
import pytest

import oracle
from moe_inputs import LayerConfig, get_config, make_full_model
from moe_inputs.gen import make_x, routing_table

pytestmark = pytest.mark.gpu


def run_dispatch(x_host, ids_host, E_l, P):
    import torch
    import gpu_helpers as gh
    import moe_layer_amd
    x = gh.to_dev(x_host)
    ids = gh.to_dev(np.ascontiguousarray(ids_host, dtype=np.int32))
    T, kk = ids_host.shape
    H = x_host.shape[1]
    out = {
        "counts": torch.full((P,), -7, dtype=torch.int32, device="cuda"),
        "offsets": torch.full((P + 1,), -7, dtype=torch.int32, device="cuda"),
        "send_order": torch.full((T * kk,), -7, dtype=torch.int32, device="cuda"),
        "pair_pos": torch.full((T * kk,), -7, dtype=torch.int32, device="cuda"),
        "send_x": torch.zeros((T * kk, H), dtype=x.dtype, device="cuda"),
        "send_ids": torch.full((T * kk,), -7, dtype=torch.int32, device="cuda"),
    }
    moe_layer_amd.moe_dispatch(x, ids, E_l, P, out["counts"], out["offsets"], out["send_order"],
                               out["pair_pos"], out["send_x"], out["send_ids"])
    torch.cuda.synchronize()
    return {k: gh.from_dev(v) for k, v in out.items()}


def check_dispatch(x_host, ids_host, E_l, P):
    g = run_dispatch(x_host, ids_host, E_l, P)
    ref = oracle.dispatch(x_host, ids_host, E_l, P)
    n = int(ref["offsets"][-1])
    assert np.array_equal(g["counts"], ref["counts"])
    assert np.array_equal(g["offsets"], ref["offsets"])
    assert np.array_equal(g["send_order"][:n], ref["send_order"])
    assert np.array_equal(g["pair_pos"], ref["pair_pos"])
    assert np.array_equal(g["send_ids"][:n], ref["send_ids"])
    assert np.array_equal(g["send_x"][:n], ref["send_x"])       # exact bytes
    return ref


def cfg_of(H, E, k, dtype="bf16", n_shared=0):
    return LayerConfig(name="d", H=H, E=E, k=k, renorm=True, I=64, dtype=dtype, T_list=(1,),
                       n_shared=n_shared)


# Per-rank token counts of the Qwen3-235B EP shape (P = 8, 16 experts per
# rank, H = 4096), a DSv2-Lite shape whose two shared slots stay local, row
# lengths that end inside a 64-lane column block (bf16 H = 1000: 125
# vectors; H = 4104: 513 vectors), fp32 rows, one rank, 64 ranks of one
# expert each, ranks of 12 experts (a division, not a shift), and routing
# tables of 8192 ids or more (counted in packed per-lane fields), one of
# them with T*kk not a multiple of 4.
@pytest.mark.parametrize("H,E,k,n_shared,P,T,dtype,routing", [
    (4096, 128, 8, 0, 8, 1, "bf16", "uniform"),
    (4096, 128, 8, 0, 8, 37, "bf16", "zipf"),
    (4096, 128, 8, 0, 8, 256, "bf16", "uniform"),
    (2048, 64, 6, 2, 8, 61, "bf16", "uniform"),
    (1000, 32, 4, 0, 4, 45, "bf16", "zipf"),
    (4104, 16, 2, 0, 2, 33, "bf16", "uniform"),
    (256, 8, 2, 0, 4, 17, "fp32", "uniform"),
    (512, 8, 3, 0, 1, 29, "bf16", "uniform"),
    (128, 64, 8, 0, 64, 50, "bf16", "uniform"),
    (256, 48, 4, 0, 4, 70, "bf16", "zipf"),        # 12 experts per rank (no shift)
    (512, 96, 6, 0, 8, 2049, "bf16", "zipf"),      # large table, 12 per rank, T*kk % 4 = 2
    (256, 64, 8, 0, 4, 1100, "bf16", "uniform"),   # large table, 4 ranks
])
def test_dispatch_matches_oracle(H, E, k, n_shared, P, T, dtype, routing):
    cfg = cfg_of(H, E, k, dtype, n_shared)
    x = make_x(cfg, T, seed=T)
    ids = routing_table(cfg, T, routing, seed=T)
    print(f"[case] dispatch H={H} E={E} k={k} shared={n_shared} P={P} T={T} {dtype} {routing}", flush=True)
    ref = check_dispatch(x, ids, E // P, P)
    assert ref["offsets"][-1] == T * k           # every routed pair, no shared pair, is sent


def test_dispatch_edge_cases():
    cfg = cfg_of(1024, 16, 4)
    x = make_x(cfg, 40, seed=2)
    print("[case] dispatch: every pair to one rank", flush=True)
    ids = np.tile(np.array([[12, 13, 14, 15]], dtype=np.int32), (40, 1))
    ref = check_dispatch(x, ids, 4, 4)
    assert ref["counts"].tolist() == [0, 0, 0, 160]
    print("[case] dispatch: repeated ids and ids past the last rank", flush=True)
    rng = np.random.default_rng(3)
    ids = rng.integers(0, 24, size=(40, 4)).astype(np.int32)   # 16..23 are not sent
    ids[::3, 1] = ids[::3, 0]
    check_dispatch(x, ids, 4, 4)
    print("[case] dispatch: nothing sent", flush=True)
    ref = check_dispatch(x, np.full((40, 4), 99, dtype=np.int32), 4, 4)
    assert ref["offsets"][-1] == 0


def test_dispatch_empty_batch_writes_zero_counts():
    import torch
    import moe_layer_amd
    print("[case] dispatch T=0", flush=True)
    counts = torch.full((8,), 5, dtype=torch.int32, device="cuda")
    offsets = torch.full((9,), 5, dtype=torch.int32, device="cuda")
    e32 = torch.empty(0, dtype=torch.int32, device="cuda")
    x = torch.empty((0, 4096), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((0, 8), dtype=torch.int32, device="cuda")
    moe_layer_amd.moe_dispatch(x, ids, 16, 8, counts, offsets, e32, e32,
                               torch.empty((0, 4096), dtype=torch.bfloat16, device="cuda"), e32)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0] * 8 and offsets.cpu().tolist() == [0] * 9


def test_dispatch_full_size_qwen3_235b_T2048():
    # the largest per-rank batch of the sweep: 16384 send rows of 8 KiB
    cfg = get_config("qwen3_235b_ep")
    T = 2048
    print("[case] dispatch Qwen3-235B EP T=2048 zipf", flush=True)
    check_dispatch(make_x(cfg, T, seed=0), routing_table(cfg, T, "zipf", seed=0), 16, 8)


def run_exchange(m, cfg, P):
    """Every rank: route its share, dispatch; every receiver: permute its rows
    by local expert, expert pass, un-permute; every sender: combine."""
    import torch
    import gpu_helpers as gh
    import moe_layer_amd as M
    E_l = cfg.E // P
    H = cfg.H
    shares = np.split(m["x"], P)
    wg, gb = gh.to_dev(m["w_gate"]), gh.to_dev(m["gate_bias"])
    w13, w2 = gh.to_dev(m["w13"]), gh.to_dev(m["w2"])
    I = cfg.I
    sent = []
    for q in range(P):
        x = gh.to_dev(shares[q])
        T = x.shape[0]
        kk = cfg.k
        logits = torch.empty((T, cfg.E), dtype=torch.float32, device="cuda")
        ids = torch.empty((T, kk), dtype=torch.int32, device="cuda")
        w = torch.empty((T, kk), dtype=torch.float32, device="cuda")
        ws = M.route_workspace(T, H, cfg.E, x.dtype)
        M.moe_route(x, wg, gb, cfg.k, cfg.renorm, 0, logits, ids, w, ws)
        d = {n: torch.empty(T * kk, dtype=torch.int32, device="cuda")
             for n in ("send_order", "pair_pos", "send_ids")}
        d["counts"] = torch.empty(P, dtype=torch.int32, device="cuda")
        d["offsets"] = torch.empty(P + 1, dtype=torch.int32, device="cuda")
        d["send_x"] = torch.empty((T * kk, H), dtype=x.dtype, device="cuda")
        M.moe_dispatch(x, ids, E_l, P, d["counts"], d["offsets"], d["send_order"], d["pair_pos"],
                       d["send_x"], d["send_ids"])
        d.update(logits=logits, ids=ids, w=w, T=T)
        sent.append(d)
    torch.cuda.synchronize()
    off = [d["offsets"].cpu().numpy() for d in sent]
    back = [[None] * P for _ in range(P)]
    unperm_exact = True
    for r in range(P):
        rx = torch.cat([sent[q]["send_x"][off[q][r]:off[q][r + 1]] for q in range(P)]).contiguous()
        rid = torch.cat([sent[q]["send_ids"][off[q][r]:off[q][r + 1]] for q in range(P)]).contiguous()
        R = rx.shape[0]
        counts = torch.empty(E_l, dtype=torch.int32, device="cuda")
        offsets = torch.empty(E_l + 1, dtype=torch.int32, device="cuda")
        sp = torch.empty(R, dtype=torch.int32, device="cuda")
        pos = torch.empty(R, dtype=torch.int32, device="cuda")
        M.moe_permute(rid.view(R, 1), r * E_l, E_l, counts, offsets, sp, pos)
        y_pair = torch.empty((R, H), dtype=rx.dtype, device="cuda")
        ws = torch.zeros(max(M.moe_workspace_bytes(M.MOE_OP_GROUPED_GEMM, R, 1, E_l, H, I,
                                                   M.MOE_DTYPE_BF16), 256),
                         dtype=torch.uint8, device="cuda")
        M.moe_grouped_gemm(rx, sp, offsets, 1, w13[r * E_l:(r + 1) * E_l], w2[r * E_l:(r + 1) * E_l],
                           y_pair, ws)
        y_ret = torch.empty((R, H), dtype=rx.dtype, device="cuda")
        M.moe_combine(y_pair, pos, None, y_ret)                  # back to arrival order
        if R:
            unperm_exact &= bool(torch.equal(y_ret, y_pair[pos.long()]))
        start = 0
        for q in range(P):
            n = int(off[q][r + 1] - off[q][r])
            back[q][r] = y_ret[start:start + n]
            start += n
    ys = []
    for q in range(P):
        d = sent[q]
        recv = torch.cat(back[q]).contiguous()
        y = torch.empty((d["T"], H), dtype=recv.dtype, device="cuda")
        M.moe_combine(recv, d["pair_pos"], d["w"], y)
        ys.append(y)
    torch.cuda.synchronize()
    return {"y": np.concatenate([gh.from_dev(y) for y in ys]),
            "ids": [gh.from_dev(d["ids"]) for d in sent],
            "logits": [gh.from_dev(d["logits"]) for d in sent],
            "unperm_exact": unperm_exact}


# Qwen3-style routing (top-k renormalised) at a reduced width, ragged
# per-rank shares, both routing variants; the seeds give every token a clear
# top-k margin, so the fp64 oracle routes exactly as the GPU does.
@pytest.mark.parametrize("P,T,routing,seed", [(4, 148, "uniform", 5), (8, 200, "zipf", 6),
                                              (2, 2, "uniform", 7)])
def test_ep_exchange_matches_oracle(P, T, routing, seed):
    import gpu_helpers as gh
    cfg = LayerConfig(name="x", H=1024, E=32, k=4, renorm=True, I=256, dtype="bf16", T_list=(T,))
    m = make_full_model(cfg, T, routing=routing, seed=seed)
    print(f"[case] EP exchange P={P} T={T} {routing} seed={seed}", flush=True)
    g = run_exchange(m, cfg, P)
    ref = oracle.ep_exchange_layer(np.split(m["x"], P), m["w_gate"], m["gate_bias"], m["w13"],
                                   m["w2"], cfg.k, cfg.renorm)
    for q in range(P):
        assert np.array_equal(g["ids"][q], ref["routed"][q][0]), f"routing of rank {q}"
    assert g["unperm_exact"]
    gh.assert_close(g["y"], np.concatenate(ref["y"]), "bf16", "EP exchange output")
