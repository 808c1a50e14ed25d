"""GPU parity on edge cases and properties: ragged and tiny batches, empty
EP shares, ties, arbitrary permutation inputs, the repack at small shapes,
the sum over ranks of the EP and TP shares, determinism and graph replay."""
import numpy as np
import pytest

import oracle
from moe_inputs import LayerConfig, make_full_model, make_layer_inputs

pytestmark = pytest.mark.gpu


def small(H=256, E=16, k=4, I=128, renorm=True, n_shared=0, dtype="bf16", view="full", P=1, T=37):
    return LayerConfig(name="small", H=H, E=E, k=k, renorm=renorm, I=I, dtype=dtype, T_list=(T,),
                       n_shared=n_shared, view=view, P=P)


@pytest.mark.parametrize("T", [1, 2, 15, 17, 37, 100])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_ragged_batches(T, dtype):
    import gpu_helpers as gh
    cfg = small(dtype=dtype, T=T)
    d = make_layer_inputs(cfg, T, routing="uniform", seed=T)
    print(f"[case] ragged T={T} {dtype}", flush=True)
    gh.check_layer(d, cfg, gh.gpu_layer(d, cfg))


# For T > 256 (bf16), groups with more than 32 rows go to the LDS-tiled
# kernels (128 token rows x 128 weight rows per tile, K split over blocks
# stream-K style) when they make at least a third of a tile per compute
# unit; otherwise the wave-streaming kernel keeps them.  These shapes put
# ragged groups on both sides of the 32-row line, leave every kind of
# partial tile (I' and H not multiples of 64 / 128, K ending half-way
# through a 64-element stage: H = 1568, I' = 736), several token tiles per
# group, shared groups, both views, and one case with too few tiles.
@pytest.mark.parametrize("H,E,k,I,T,n_shared,view,P", [
    (1568, 8, 2, 736, 300, 0, "full", 1),    # ragged, partial tiles and stages
    (1536, 4, 2, 768, 600, 0, "full", 1),    # ~300 rows per group: 3 token tiles
    (1536, 16, 4, 768, 300, 2, "full", 1),   # shared groups of 300 rows with the routed ones
    (2048, 16, 4, 1536, 300, 0, "tp", 2),    # TP slice: I' = 768
    (1536, 16, 4, 768, 600, 0, "ep", 2),     # EP share of 8 experts
    (1536, 4, 1, 768, 300, 0, "full", 1),    # too few tiles: all groups streamed
])
def test_tiled_groups(H, E, k, I, T, n_shared, view, P):
    import gpu_helpers as gh
    cfg = small(H=H, E=E, k=k, I=I, T=T, n_shared=n_shared, view=view, P=P, renorm=n_shared == 0)
    d = make_layer_inputs(cfg, T, routing="uniform", rank=P - 1, seed=H + T + 1)  # no near-ties
    print(f"[case] tiled H={H} E={E} k={k} I={I} T={T} shared={n_shared} {view} P={P}", flush=True)
    g = gh.gpu_layer(d, cfg)
    counts = g["counts"]
    assert counts.max() > 32, counts  # groups on the tiled side of the line
    gh.check_layer(d, cfg, g)


# From 1024 tokens on the LDS-tiled kernels take every group and no
# wave-streaming launch follows, whatever the group sizes: 1030 tokens over
# 128 experts with k = 2 make groups of 7-27 rows (none would qualify under
# the hot-group rule), each in one 128-row token tile, and a ragged last
# token tile of the batch.
def test_small_groups_from_1024_tokens_in_tiles():
    import gpu_helpers as gh
    cfg = small(H=512, E=128, k=2, I=256, T=1030)
    d = make_layer_inputs(cfg, 1030, routing="uniform", seed=43)  # no near-ties
    print("[case] small groups in tiles T=1030 E=128 k=2 H=512 I=256", flush=True)
    g = gh.gpu_layer(d, cfg)
    assert g["counts"].max() <= 32, g["counts"]
    gh.check_layer(d, cfg, g)


# A single hot expert holding every token: one group far above the 32-row
# line, too few tiles for the tiled kernels, so the wave-streaming kernel
# takes it in passes of 32 rows.
@pytest.mark.parametrize("T", [33, 64, 300])
def test_hot_expert_split_tiles(T):
    import gpu_helpers as gh
    cfg = small(H=2048, E=8, k=2, I=1024, T=T)
    d = make_layer_inputs(cfg, T, routing="uniform", seed=T)
    b = np.zeros(8, dtype=np.float32)
    b[5] = 40.0            # every token picks expert 5 first
    d["gate_bias"] = b
    print(f"[case] hot expert T={T}", flush=True)
    g = gh.gpu_layer(d, cfg)
    assert g["counts"][5] == T
    gh.check_layer(d, cfg, g)


# Batches of 384..767 tokens with more than 24 rows per group on average take
# the wave-streaming kernel with four token tiles (passes of 64 rows); the
# LDS-tiled kernels then keep only groups above 64 rows.  Ragged groups of
# 16 to 54 rows (one to four token tiles in use), K ending part-way through a
# 512-byte chunk (H = 1568) and a hot expert of 500 rows taking eight passes.
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("T,E,k,hot", [(400, 32, 2, False), (700, 32, 2, False), (500, 16, 2, True)])
def test_four_token_tiles(T, E, k, hot, dtype):
    import gpu_helpers as gh
    cfg = small(H=1568, E=E, k=k, I=736, T=T, dtype=dtype)
    d = make_layer_inputs(cfg, T, routing="uniform", seed=T + E)
    if hot:
        b = np.zeros(E, dtype=np.float32)
        b[3] = 40.0        # every token picks expert 3 first
        d["gate_bias"] = b
    print(f"[case] four token tiles T={T} E={E} k={k} hot={hot} {dtype}", flush=True)
    g = gh.gpu_layer(d, cfg)
    counts = g["counts"]
    assert counts.max() > 32, counts  # groups past two token tiles
    gh.check_layer(d, cfg, g)


# A launch whose wave-streaming kernel holds four token tiles hands its
# groups to the LDS-tiled kernels only when those above 64 rows hold a
# quarter of the rows and all make a tile per compute unit: 600 tokens over
# 8 experts (137-166 rows each, two token tiles) with I = 1024 and H = 2048
# make 256 up and 256 down tiles (one per MI355X compute unit), so the tiled
# kernels take every group, and the wave-streaming launch, deciding by the
# same device-side rule, finds nothing left.
def test_four_token_tiles_with_tiled_groups():
    import gpu_helpers as gh
    cfg = small(H=2048, E=8, k=2, I=1024, T=600)
    d = make_layer_inputs(cfg, 600, routing="uniform", seed=77)
    print("[case] four token tiles with tiled groups T=600 E=8 k=2 H=2048 I=1024", flush=True)
    g = gh.gpu_layer(d, cfg)
    counts = g["counts"]
    assert (counts > 128).sum() >= 4, counts   # several groups past one 128-row tile
    gh.check_layer(d, cfg, g)


# Down-projections whose W2 rows are at most 512 bytes (bf16, I' <= 256) take
# whole 16-row tiles per step with the pass's token fragments held in
# registers: every row length (1..8 fragments of 64 bytes), passes of 16 and
# 32 rows, a hot expert with several passes, empty experts, and ranges of
# steps that cross from one pass or group to the next (H = 4096: 256 tiles per
# pass, a few thousand steps over the chip's waves).
@pytest.mark.parametrize("T,E,k,H,I,hot", [
    (64, 16, 8, 4096, 192, False),    # the TP share's row length; ~32 rows per expert, one or two passes
    (40, 16, 4, 1024, 32, True),      # one fragment per row; a hot expert of 40 rows (passes of 32)
    (12, 32, 2, 2048, 96, False),     # three fragments; passes of 16 rows, empty experts
    (200, 8, 3, 512, 256, True),      # eight fragments, 32 tiles per pass; a 200-row expert
    (300, 8, 2, 1024, 160, False),    # five fragments; T above 256 (the tiled kernels' rule is evaluated)
])
def test_short_row_down(T, E, k, H, I, hot):
    import gpu_helpers as gh
    cfg = small(H=H, E=E, k=k, I=I, T=T)
    d = make_layer_inputs(cfg, T, routing="uniform", seed=T + I)
    if hot:
        b = np.zeros(E, dtype=np.float32)
        b[1] = 40.0        # every token picks expert 1 first
        d["gate_bias"] = b
    print(f"[case] short-row down T={T} E={E} k={k} H={H} I={I} hot={hot}", flush=True)
    g = gh.gpu_layer(d, cfg)
    gh.check_layer(d, cfg, g)


@pytest.mark.parametrize("n_shared,renorm", [(2, False), (1, True)])
def test_shared_experts(n_shared, renorm):
    import gpu_helpers as gh
    cfg = small(n_shared=n_shared, renorm=renorm, T=40)
    d = make_layer_inputs(cfg, 40, seed=1)
    print(f"[case] shared n_shared={n_shared}", flush=True)
    gh.check_layer(d, cfg, gh.gpu_layer(d, cfg))


# The routing limits the ABI advertises: E up to 512 experts (lanes holding
# 8, 16 or 32 candidate keys each) and k up to 32 picks (rounds 16..31 go to
# a lane's second pick register), with and without shared slots, an expert
# count that is not a multiple of 16, fp32 storage, one and several token
# tiles, and both the one-launch and the two-call routing.  Seeds chosen so
# that no token's k-th and (k+1)-th logits lie within 1e-4 of each other.
@pytest.mark.parametrize("E,k,n_shared,dtype,T,fused", [
    (192, 17, 0, "bf16", 40, True),
    (512, 32, 0, "bf16", 33, True),
    (510, 32, 2, "bf16", 16, True),     # one token tile: keys sorted from LDS; 512 groups
    (512, 32, 0, "bf16", 33, False),    # moe_route + moe_permute
    (200, 20, 0, "fp32", 24, True),     # 13 expert tiles, the last half full
    (256, 32, 0, "bf16", 8, True),
    (384, 24, 1, "bf16", 70, False),
])
def test_wide_routing(E, k, n_shared, dtype, T, fused):
    import gpu_helpers as gh
    cfg = small(H=256, E=E, k=k, I=64, renorm=n_shared == 0, n_shared=n_shared, dtype=dtype, T=T)
    d = make_layer_inputs(cfg, T, routing="uniform", seed=100)
    print(f"[case] wide routing E={E} k={k} shared={n_shared} {dtype} T={T} fused={fused}", flush=True)
    g = gh.gpu_layer(d, cfg, fused=fused)
    assert g["topk_ids"].shape == (T, k + n_shared)
    gh.check_layer(d, cfg, g)


def test_k_equals_E():
    import gpu_helpers as gh
    cfg = small(E=8, k=8, T=20)
    d = make_layer_inputs(cfg, 20, seed=2)
    print("[case] k=E", flush=True)
    gh.check_layer(d, cfg, gh.gpu_layer(d, cfg))


@pytest.mark.parametrize("renorm", [True, False])
def test_all_logits_tied(renorm):
    import gpu_helpers as gh
    cfg = small(renorm=renorm, T=24)
    d = make_layer_inputs(cfg, 24, seed=3)
    d["w_gate"] = np.zeros_like(d["w_gate"])
    print("[case] tied logits", flush=True)
    g = gh.gpu_layer(d, cfg)
    assert (g["topk_ids"] == np.arange(cfg.k)).all()
    assert np.allclose(g["topk_w"], 1 / cfg.k if renorm else 1 / cfg.E, atol=1e-7)
    assert g["counts"].tolist() == [24] * cfg.k + [0] * (cfg.E - cfg.k)
    gh.check_layer(d, cfg, g, expect_near_ties=24)


def test_bias_ties_and_signed_zero():
    import gpu_helpers as gh
    cfg = small(E=16, k=4, T=8)
    d = make_layer_inputs(cfg, 8, seed=4)
    d["w_gate"] = np.zeros_like(d["w_gate"])
    b = np.zeros(16, dtype=np.float32)
    b[[3, 9]] = 2.0        # tie at the top: 3 before 9
    b[[5, 6, 12]] = 1.0    # three-way tie for two places: 5 and 6
    b[7] = -0.0
    d["gate_bias"] = b
    print("[case] bias ties", flush=True)
    g = gh.gpu_layer(d, cfg)
    assert (g["topk_ids"] == [3, 9, 5, 6]).all()


def test_ep_rank_with_no_local_pairs():
    import gpu_helpers as gh
    cfg = small(E=16, k=2, view="ep", P=4, T=12)
    d = make_layer_inputs(cfg, 12, rank=3, seed=5)
    b = np.zeros(16, dtype=np.float32)
    b[:4] = 50.0           # everything goes to rank 0's experts
    d["gate_bias"] = b
    print("[case] empty EP share", flush=True)
    g = gh.gpu_layer(d, cfg)
    assert g["counts"].sum() == 0 and (g["pair_pos"] == -1).all()
    assert (oracle.widen(g["y"]) == 0).all()
    gh.check_layer(d, cfg, g)


def test_permute_arbitrary_ids():
    import torch

    import gpu_helpers as gh
    import moe_layer_amd
    rng = np.random.default_rng(11)
    # One block sorts up to 4096 pairs; above that one block per 1024-pair
    # segment (the first cases): ragged last segments, 512 groups, a window
    # holding none of the ids, and the 4096 / 4097 boundary.
    for T, kk, g_begin, n_groups in [(1000, 7, 5, 40), (3, 1, 0, 1), (2048, 8, 0, 130), (64, 64, 100, 7),
                                     (4097, 1, 0, 512), (4096, 1, 0, 512), (700, 8, 3, 509),
                                     (20000, 3, 0, 16), (3000, 2, 900, 5)]:
        ids = rng.integers(-3, g_begin + n_groups + 5, size=(T, kk)).astype(np.int32)
        if g_begin == 900:
            ids = rng.integers(0, 800, size=(T, kk)).astype(np.int32)   # nothing in the window
        print(f"[case] permute T={T} kk={kk} window=({g_begin},{n_groups})", flush=True)
        dev = gh.to_dev(ids)
        out = [torch.empty(s, dtype=torch.int32, device="cuda") for s in
               (n_groups, n_groups + 1, T * kk, T * kk)]
        moe_layer_amd.moe_permute(dev, g_begin, n_groups, *out)
        torch.cuda.synchronize()
        c, o, sp, pos = oracle.permute(ids, g_begin, n_groups)
        got = [gh.from_dev(t) for t in out]
        assert np.array_equal(got[0], c) and np.array_equal(got[1], o)
        assert np.array_equal(got[2][:o[-1]], sp) and np.array_equal(got[3], pos)


def stable_sort_properties(ids, g_begin, n_groups, counts, offsets, sorted_pair, pair_pos):
    """What fixes a stable counting sort at any size, checked with vector ops:
    the counts are the histogram, the offsets its exclusive sum, sorted_pair
    lists every held pair once, in group order and ascending inside a group,
    and pair_pos is its inverse (-1 for pairs not held)."""
    key = ids.ravel().astype(np.int64) - g_begin
    held = (key >= 0) & (key < n_groups)
    hist = np.bincount(key[held], minlength=n_groups)
    assert np.array_equal(counts, hist)
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets.astype(np.int64)), hist)
    n_kept = int(offsets[-1])
    sp = sorted_pair[:n_kept].astype(np.int64)
    assert np.array_equal(np.sort(sp), np.flatnonzero(held))
    g_of_row = key[sp]
    assert (np.diff(g_of_row) >= 0).all()
    same = np.diff(g_of_row) == 0
    assert (np.diff(sp)[same] > 0).all()
    expect_pos = np.full(key.size, -1, dtype=np.int64)
    expect_pos[sp] = np.arange(n_kept)
    assert np.array_equal(pair_pos, expect_pos)


def test_permute_large_tables():
    import torch

    import gpu_helpers as gh
    import moe_layer_amd
    rng = np.random.default_rng(12)
    # Above 65536 pairs the sort runs as count / column-scan / scatter launches
    # with per-segment counts parked in pair_pos: both sides of the line, a
    # ragged last segment, every pair in one group, an empty window, 2048
    # segments of 1024 pairs and 2048 segments of 4096 pairs.
    cases = [(65536, 1, 0, 512, True), (65537, 1, 0, 512, True), (40000, 8, 0, 128, True),
             (70000, 2, 0, 3, True), (80000, 1, 900, 5, True), (262144, 8, 64, 16, False),
             (1 << 20, 8, 0, 512, False)]
    for T, kk, g_begin, n_groups, use_oracle in cases:
        if g_begin == 900:
            ids = rng.integers(0, 800, size=(T, kk)).astype(np.int32)
        elif n_groups == 3:
            ids = np.where(rng.random((T, kk)) < 0.97, 1, rng.integers(-1, 4, size=(T, kk))).astype(np.int32)
        else:
            ids = rng.integers(-3, g_begin + n_groups + 5, size=(T, kk)).astype(np.int32)
        print(f"[case] permute large T={T} kk={kk} window=({g_begin},{n_groups})", flush=True)
        dev = gh.to_dev(ids)
        out = [torch.full((s,), -7, dtype=torch.int32, device="cuda") for s in
               (n_groups, n_groups + 1, T * kk, T * kk)]
        moe_layer_amd.moe_permute(dev, g_begin, n_groups, *out)
        torch.cuda.synchronize()
        got = [gh.from_dev(t) for t in out]
        if use_oracle:
            c, o, sp, pos = oracle.permute(ids, g_begin, n_groups)
            assert np.array_equal(got[0], c) and np.array_equal(got[1], o)
            assert np.array_equal(got[2][:o[-1]], sp) and np.array_equal(got[3], pos)
        else:
            stable_sort_properties(ids, g_begin, n_groups, *got)
        del dev, out


def test_permute_empty_batch_writes_zero_counts():
    import torch

    import moe_layer_amd
    counts = torch.full((9,), 7, dtype=torch.int32, device="cuda")
    offsets = torch.full((10,), 7, dtype=torch.int32, device="cuda")
    ids = torch.empty((0, 4), dtype=torch.int32, device="cuda")
    e = torch.empty((0,), dtype=torch.int32, device="cuda")
    moe_layer_amd.moe_permute(ids, 0, 9, counts, offsets, e, e)
    torch.cuda.synchronize()
    assert counts.cpu().tolist() == [0] * 9 and offsets.cpu().tolist() == [0] * 10


# W2 rows of 1..4 chunks per lane (several rows per wave step, row counts
# that do not divide evenly) and of more (one row at a time).
@pytest.mark.parametrize("dtype,P,E_l,H,I", [
    ("bf16", 1, 2, 256, 64), ("bf16", 2, 3, 128, 64), ("bf16", 8, 2, 512, 128),
    ("fp32", 4, 3, 64, 32), ("bf16", 16, 1, 64, 128),
    ("bf16", 8, 1, 64, 1536), ("bf16", 4, 2, 40, 1024), ("fp32", 2, 1, 56, 1024), ("bf16", 2, 2, 48, 2560),
])
def test_repack_small(dtype, P, E_l, H, I):
    import torch

    import gpu_helpers as gh
    import moe_layer_amd
    rng = np.random.default_rng(P)
    if dtype == "bf16":
        w13 = rng.integers(0, 65535, size=(E_l, 2 * I, H), dtype=np.uint16)
        w2 = rng.integers(0, 65535, size=(E_l, H, I), dtype=np.uint16)
        # keep the bit patterns finite-valued (no NaN/Inf exponent)
        w13 &= 0xBFFF
        w2 &= 0xBFFF
        tdt = torch.bfloat16
    else:
        w13 = rng.standard_normal((E_l, 2 * I, H)).astype(np.float32)
        w2 = rng.standard_normal((E_l, H, I)).astype(np.float32)
        tdt = torch.float32
    Ip = I // P
    print(f"[case] repack {dtype} P={P}", flush=True)
    d13 = [torch.empty((E_l, 2 * Ip, H), dtype=tdt, device="cuda") for _ in range(P)]
    d2 = [torch.empty((E_l, H, Ip), dtype=tdt, device="cuda") for _ in range(P)]
    moe_layer_amd.moe_repack_ep_to_tp(gh.to_dev(w13), gh.to_dev(w2), P, d13, d2)
    torch.cuda.synchronize()
    b13, b2 = oracle.repack_ep_to_tp(w13, w2, P)
    for q in range(P):
        assert np.array_equal(gh.from_dev(d13[q]), b13[q])
        assert np.array_equal(gh.from_dev(d2[q]), b2[q])
    # the inverse from the oracle's blocks rebuilds the experts the oracle
    # rebuilds (the originals), byte for byte
    r13 = torch.empty((E_l, 2 * I, H), dtype=tdt, device="cuda")
    r2 = torch.empty((E_l, H, I), dtype=tdt, device="cuda")
    moe_layer_amd.moe_repack_tp_to_ep([gh.to_dev(b) for b in b13], [gh.to_dev(b) for b in b2], P, r13, r2)
    torch.cuda.synchronize()
    o13, o2 = oracle.repack_tp_to_ep(b13, b2)
    assert np.array_equal(gh.from_dev(r13), o13) and np.array_equal(gh.from_dev(r2), o2)
    assert np.array_equal(o13, w13) and np.array_equal(o2, w2)


@pytest.mark.parametrize("routing", ["uniform", "zipf"])
def test_sum_of_rank_shares_is_the_full_layer(routing):
    """All P EP shares and all P TP shares of one model on this GPU; the TP
    weights are built by the GPU repack of each EP rank's experts."""
    import torch

    import gpu_helpers as gh
    import moe_layer_amd
    P, T = 8, 96
    cfg = LayerConfig(name="ranks", H=512, E=32, k=4, renorm=True, I=256, dtype="bf16", T_list=(T,))
    m = make_full_model(cfg, T, routing=routing, seed=21)
    full = oracle.moe_layer(m["x"], m["w_gate"], m["gate_bias"], m["w13"], m["w2"], cfg.k, cfg.renorm)
    E_l, Ip = cfg.E // P, cfg.I // P
    x, wg, b = gh.to_dev(m["x"]), gh.to_dev(m["w_gate"]), gh.to_dev(m["gate_bias"])
    w13_all, w2_all = gh.to_dev(m["w13"]), gh.to_dev(m["w2"])
    print(f"[case] rank shares {routing}", flush=True)
    ep_sum = np.zeros((T, cfg.H))
    tp13 = [torch.empty((cfg.E, 2 * Ip, cfg.H), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    tp2 = [torch.empty((cfg.E, cfg.H, Ip), dtype=torch.bfloat16, device="cuda") for _ in range(P)]
    for r in range(P):
        sl = slice(r * E_l, (r + 1) * E_l)
        w13_r, w2_r = w13_all[sl].contiguous(), w2_all[sl].contiguous()
        bufs = moe_layer_amd.moe_layer_forward(x, wg, b, w13_r, w2_r, cfg.k, cfg.renorm, 0, r * E_l)
        ep_sum += oracle.widen(gh.from_dev(bufs.y))
        # rank r's repack writes rows G_r of every peer's TP tensors
        moe_layer_amd.moe_repack_ep_to_tp(w13_r, w2_r, P, [t[sl] for t in tp13], [t[sl] for t in tp2])
    tp_sum = np.zeros((T, cfg.H))
    for p in range(P):
        bufs = moe_layer_amd.moe_layer_forward(x, wg, b, tp13[p], tp2[p], cfg.k, cfg.renorm)
        tp_sum += oracle.widen(gh.from_dev(bufs.y))
        want13, want2 = oracle.tp_slice(m["w13"], m["w2"], p, P)
        assert np.array_equal(gh.from_dev(tp13[p]), want13)
        assert np.array_equal(gh.from_dev(tp2[p]), want2)
    torch.cuda.synchronize()
    gh.assert_close(ep_sum, full["y"], "bf16", "sum of EP shares")
    gh.assert_close(tp_sum, full["y"], "bf16", "sum of TP shares")


def test_repeated_runs_are_bit_identical():
    import gpu_helpers as gh
    cfg = small(E=64, k=6, T=200, n_shared=2, renorm=False)
    d = make_layer_inputs(cfg, 200, seed=6)
    print("[case] determinism", flush=True)
    a = gh.gpu_layer(d, cfg)
    b = gh.gpu_layer(d, cfg)
    for key in a:
        n = int(a["offsets"][-1])
        va, vb = (a[key][:n], b[key][:n]) if key in ("sorted_pair", "a", "y_pair") else (a[key], b[key])
        assert np.array_equal(va, vb), key


# The LDS-tiled kernels hand the few tiles left after one tile per block to
# whichever blocks finish first, cut along K into pieces, through a claim
# counter in the workspace that the last block clears; the last piece of a
# tile to finish sums the pieces.  1950 tokens over 16 experts (195-278 rows
# each) make 576 up tiles, 8 more per XCD than its 64 blocks on MI355X,
# so the up launch claims: with H = 1024 (16 K stages) whole leftover tiles,
# with H = 4096 (64 stages) halves of them.  Two passes on one set of
# buffers (the workspace included) must both match the oracle: counters left
# set would drop tiles in the second.
@pytest.mark.parametrize("H", [1024, 4096])
def test_tile_claims_leave_workspace_reusable(H):
    import torch

    import gpu_helpers as gh
    import moe_layer_amd
    cfg = small(H=H, E=16, k=2, I=1024, T=1950)
    d = make_layer_inputs(cfg, 1950, routing="uniform", seed=31 if H == 1024 else 32)  # no near-ties
    x, wg, b = gh.to_dev(d["x"]), gh.to_dev(d["w_gate"]), gh.to_dev(d["gate_bias"])
    w13, w2 = gh.to_dev(d["w13"]), gh.to_dev(d["w2"])
    print(f"[case] tile claims, two passes on one workspace, H={H}", flush=True)
    bufs = None
    for _ in range(2):
        bufs = moe_layer_amd.moe_layer_forward(x, wg, b, w13, w2, cfg.k, cfg.renorm, bufs=bufs)
        torch.cuda.synchronize()
        g = {name: gh.from_dev(getattr(bufs, name)) for name in
             ("logits", "topk_ids", "topk_w", "counts", "offsets", "sorted_pair", "pair_pos", "a", "y_pair", "y")}
        assert g["counts"].min() > 128, g["counts"]   # every group past one 128-row token tile
        gh.check_layer(d, cfg, g)


# T = 600 under Zipf routing (groups of 10-556 rows) runs both expert kernels
# of each projection in the graph: the LDS-tiled one (claims, split tiles)
# and the wave-streaming one, each checked against the oracle first.
@pytest.mark.parametrize("T,E,k,H,I,routing", [(64, 32, 4, 256, 128, "uniform"), (600, 16, 4, 512, 512, "zipf")])
def test_graph_replay_matches_eager(T, E, k, H, I, routing):
    import torch

    import gpu_helpers as gh
    import moe_layer_amd
    cfg = small(E=E, k=k, T=T, H=H, I=I)
    d = make_layer_inputs(cfg, T, routing=routing, seed=8 if T == 64 else 9)
    x, wg, b = gh.to_dev(d["x"]), gh.to_dev(d["w_gate"]), gh.to_dev(d["gate_bias"])
    w13, w2 = gh.to_dev(d["w13"]), gh.to_dev(d["w2"])
    print(f"[case] graph replay T={T} {routing}", flush=True)
    eager = moe_layer_amd.moe_layer_forward(x, wg, b, w13, w2, cfg.k, cfg.renorm)
    torch.cuda.synchronize()
    want = gh.from_dev(eager.y).copy()
    if T > 256:
        g = {name: gh.from_dev(getattr(eager, name)) for name in
             ("logits", "topk_ids", "topk_w", "counts", "offsets", "sorted_pair", "pair_pos", "a", "y_pair", "y")}
        assert g["counts"].min() <= 32 < g["counts"].max() // 4   # both kernels of a projection have groups
        gh.check_layer(d, cfg, g)
    bufs = moe_layer_amd.MoeLayerBuffers.allocate(T, cfg.H, cfg.E, cfg.k, cfg.E, cfg.I, torch.bfloat16)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        moe_layer_amd.moe_layer_forward(x, wg, b, w13, w2, cfg.k, cfg.renorm, bufs=bufs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe_layer_amd.moe_layer_forward(x, wg, b, w13, w2, cfg.k, cfg.renorm, bufs=bufs)
    for _ in range(4):
        bufs.y.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(gh.from_dev(bufs.y), want)
        eager = moe_layer_amd.moe_layer_forward(x, wg, b, w13, w2, cfg.k, cfg.renorm)
        torch.cuda.synchronize()


@pytest.mark.parametrize("T,E,k,n_shared,H", [(3000, 64, 8, 0, 256), (8, 128, 8, 0, 4096),
                                               (40, 64, 6, 2, 2048), (1, 128, 8, 0, 4096),
                                               (13, 128, 8, 2, 4096), (16, 64, 6, 2, 2048),
                                               (17, 128, 8, 0, 4096), (9000, 64, 8, 0, 256),
                                               (1100, 128, 8, 0, 1024), (1030, 128, 2, 1, 1024),
                                               (1040, 256, 4, 0, 2048)])
def test_fused_route_matches_two_calls_and_leaves_workspace_zero(T, E, k, n_shared, H):
    """One launch (routing + sort) against moe_route then moe_permute; the
    3000-token case has more pairs than the sort stages in LDS, and 9000
    tokens (72 000 pairs) route and then sort in the three-launch permute.  At H = 2048
    and 4096 the gate GEMM runs 8 or 16 K slices summed per block; T <= 16
    (one token tile, T = 1 and 13 ragged) sorts in the top-k block from LDS,
    and T = 17 hands a one-token second tile to the sorting block.  T = 1100
    and 1030 end in a ragged token tile (1030 x 3 pairs sort in the routing
    launch, with a shared slot); E = 256 takes two blocks per K slice of a
    token tile.  The logits are checked against the fp64 oracle too."""
    import torch

    import gpu_helpers as gh
    import moe_layer_amd
    cfg = small(H=H, E=E, k=k, n_shared=n_shared, renorm=False, T=T)
    d = make_layer_inputs(cfg, T, routing="zipf", seed=12)
    x, wg, b = gh.to_dev(d["x"]), gh.to_dev(d["w_gate"]), gh.to_dev(d["gate_bias"])
    kk, G = k + n_shared, E + n_shared
    print(f"[case] fused route T={T} E={E}", flush=True)
    outs = []
    for fused in (True, False, True):
        bufs = moe_layer_amd.MoeLayerBuffers.allocate(T, H, E, kk, G, cfg.I, torch.bfloat16)
        if fused:
            moe_layer_amd.moe_route_permute(x, wg, b, k, False, n_shared, bufs.logits, bufs.topk_ids,
                                            bufs.topk_w, 0, G, bufs.counts, bufs.offsets,
                                            bufs.sorted_pair, bufs.pair_pos, bufs.route_ws)
        else:
            moe_layer_amd.moe_route(x, wg, b, k, False, n_shared, bufs.logits, bufs.topk_ids,
                                    bufs.topk_w, bufs.route_ws)
            moe_layer_amd.moe_permute(bufs.topk_ids, 0, G, bufs.counts, bufs.offsets,
                                      bufs.sorted_pair, bufs.pair_pos)
        torch.cuda.synchronize()
        n = moe_layer_amd.moe_route_workspace_bytes(T, H, E, 1)
        head = (T + 15) // 16 + 1
        assert int(bufs.route_ws[: 4 * head].count_nonzero()) == 0, "counters not reset"
        assert n >= 4 * head
        outs.append({k_: gh.from_dev(getattr(bufs, k_)) for k_ in
                     ("logits", "topk_ids", "topk_w", "counts", "offsets", "pair_pos")})
    for key in outs[0]:
        assert np.array_equal(outs[0][key], outs[1][key]), key
        assert np.array_equal(outs[0][key], outs[2][key]), key
    lg_ref = oracle.gate_logits(d["x"], d["w_gate"], d["gate_bias"])
    lerr = np.abs(outs[0]["logits"].astype(np.float64) - lg_ref).max()
    assert lerr <= gh.LOGIT_REL * np.abs(lg_ref).max(), f"logits max err {lerr:.3e}"
    ids_ref, w_ref = oracle.route(outs[0]["logits"].astype(np.float64), k, False, n_shared)
    assert np.array_equal(outs[0]["topk_ids"], ids_ref)
    assert np.abs(outs[0]["topk_w"] - w_ref).max() <= 1e-5
    c, o, _, pos = oracle.permute(outs[0]["topk_ids"], 0, G)
    assert np.array_equal(outs[0]["counts"], c) and np.array_equal(outs[0]["pair_pos"], pos)


def test_route_workspace_reused_across_shapes():
    """One zeroed workspace serves calls of different batch sizes in turn."""
    import torch

    import gpu_helpers as gh
    import moe_layer_amd
    cfg = small(E=32, k=4, T=300)
    d = make_layer_inputs(cfg, 300, seed=13)
    wg, b = gh.to_dev(d["w_gate"]), gh.to_dev(d["gate_bias"])
    ws = moe_layer_amd.route_workspace(300, cfg.H, cfg.E, torch.bfloat16)
    print("[case] workspace reuse", flush=True)
    for T in (300, 5, 77, 300):
        x = gh.to_dev(d["x"][:T])
        bufs = moe_layer_amd.MoeLayerBuffers.allocate(T, cfg.H, cfg.E, cfg.k, cfg.E, cfg.I, torch.bfloat16)
        moe_layer_amd.moe_route_permute(x, wg, b, cfg.k, True, 0, bufs.logits, bufs.topk_ids, bufs.topk_w,
                                        0, cfg.E, bufs.counts, bufs.offsets, bufs.sorted_pair,
                                        bufs.pair_pos, ws)
        torch.cuda.synchronize()
        ids_ref, _ = oracle.route(gh.from_dev(bufs.logits).astype(np.float64), cfg.k, True)
        assert np.array_equal(gh.from_dev(bufs.topk_ids), ids_ref)
        c, o, sp, pos = oracle.permute(ids_ref, 0, cfg.E)
        assert np.array_equal(gh.from_dev(bufs.offsets), o)
        assert np.array_equal(gh.from_dev(bufs.sorted_pair)[: o[-1]], sp)


@pytest.mark.gpu
def test_expert_workspace_reused_across_shapes():
    """The expert GEMMs split items along K over waves; the split-item
    counters come back to zero after every call, so one workspace serves
    calls of different batch sizes in turn with bit-identical results."""
    import torch

    import gpu_helpers as gh
    import moe_layer_amd
    cfg = small(H=2048, E=16, k=4, I=256, T=200)
    d = make_layer_inputs(cfg, 200, seed=21)
    wg, b = gh.to_dev(d["w_gate"]), gh.to_dev(d["gate_bias"])
    w13, w2 = gh.to_dev(d["w13"]), gh.to_dev(d["w2"])
    shared = moe_layer_amd.expert_workspace(200, cfg.k, cfg.E, cfg.H, cfg.I, torch.bfloat16)
    print("[case] expert workspace reuse", flush=True)
    for T in (200, 3, 64, 200):
        x = gh.to_dev(d["x"][:T])
        outs = []
        for ws in (shared, moe_layer_amd.expert_workspace(T, cfg.k, cfg.E, cfg.H, cfg.I, torch.bfloat16)):
            bufs = moe_layer_amd.MoeLayerBuffers.allocate(T, cfg.H, cfg.E, cfg.k, cfg.E, cfg.I, torch.bfloat16)
            moe_layer_amd.moe_route_permute(x, wg, b, cfg.k, True, 0, bufs.logits, bufs.topk_ids,
                                            bufs.topk_w, 0, cfg.E, bufs.counts, bufs.offsets,
                                            bufs.sorted_pair, bufs.pair_pos, bufs.route_ws)
            moe_layer_amd.moe_expert_up(x, bufs.sorted_pair, bufs.offsets, cfg.k, w13, bufs.a, ws)
            moe_layer_amd.moe_expert_down(bufs.a, bufs.offsets, T, cfg.k, w2, bufs.y_pair, ws)
            torch.cuda.synchronize()
            n = int(gh.from_dev(bufs.offsets)[-1])
            outs.append((gh.from_dev(bufs.a)[:n].copy(), gh.from_dev(bufs.y_pair)[:n].copy()))
        assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1]), T
