"""Host-side plumbing for the GPU parity tests: moving seeded host arrays to
the device and back, running the library's calls, and the comparison rules.

Comparison rules (written out once here, used by every parity test):
* integer outputs (routing ids, counts, offsets, permutation, repacked bytes):
  bit-exact.
* routing ids are compared with the oracle's top-k run on the GPU's own fp32
  logits (the same decision in the same precision); the GPU logits match the
  oracle's fp64 logits to 1e-4 of their largest magnitude.
* bf16 float outputs: relative L2 error <= 5e-3 and max abs error
  <= 2e-2 * max|ref| against the fp64 oracle; fp32 storage: relative L2 <= 1e-5.
"""
import numpy as np
import torch

import oracle

BF16_REL_L2 = 5e-3
BF16_MAX_ABS = 2e-2
F32_REL_L2 = 1e-5
LOGIT_REL = 1e-4
WEIGHT_ABS = 1e-5


def to_dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def from_dev(t):
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def rel_l2(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def assert_close(got_bits_or_vals, ref, dtype, what):
    got = oracle.widen(got_bits_or_vals)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    if ref.size == 0:
        return
    if np.abs(ref).max() == 0:
        assert np.abs(got).max() == 0, what
        return
    e = rel_l2(got, ref)
    if dtype == "fp32":
        assert e <= F32_REL_L2, f"{what}: rel L2 {e:.3e} > {F32_REL_L2}"
    else:
        m = float(np.abs(got - ref).max() / np.abs(ref).max())
        assert e <= BF16_REL_L2, f"{what}: rel L2 {e:.3e} > {BF16_REL_L2}"
        assert m <= BF16_MAX_ABS, f"{what}: max abs {m:.3e} x max|ref| > {BF16_MAX_ABS}"
    return e


def ulp(v, dtype):
    """Spacing of the storage format at |v| (bf16: 8 significant bits; fp32:
    24), floored at the smallest normal."""
    a = np.maximum(np.abs(np.asarray(v, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - (7 if dtype == "bf16" else 23))


def check_combine(y, y_pair, pair_pos, topk_w, T, kk, dtype):
    """The combine, element by element, against the oracle's fp64 combine of
    the same pair outputs and weights.  The GPU sums the slots in fp32 in slot
    order and rounds once to the storage type, so each element may differ by
    one unit in the last place of the storage type plus the fp32 summation
    error, at most kk * 2^-23 times the sum of the terms' magnitudes."""
    yp = oracle.widen(y_pair) if len(y_pair) else np.zeros((0, np.asarray(y).shape[1]))
    y_c = oracle.combine(yp, pair_pos, topk_w, T, kk)
    mag = oracle.combine(np.abs(yp), pair_pos, np.abs(np.asarray(topk_w, dtype=np.float64)), T, kk)
    err = np.abs(oracle.widen(y) - y_c)
    bound = ulp(y_c, dtype) + kk * 2.0 ** -23 * mag
    bad = err > bound
    assert not bad.any(), (f"combine: {int(bad.sum())} elements off by more than one ulp; worst "
                           f"{float((err / bound).max()):.2f} x bound")


def gpu_layer(d, cfg, k=None, renorm=None, n_shared=None, g_begin=None, dev=None, fused=True):
    """Run the layer through the C ABI on host inputs ``d``; return numpy results.

    ``dev`` may hold already-uploaded "w_gate", "gate_bias", "w13", "w2";
    ``fused=False`` routes with moe_route + moe_permute instead of
    moe_route_permute.
    """
    import moe_layer_amd
    k = cfg.k if k is None else k
    renorm = cfg.renorm if renorm is None else renorm
    n_shared = cfg.n_shared if n_shared is None else n_shared
    g_begin = d.get("g_begin", 0) if g_begin is None else g_begin
    dev = dict(dev or {})
    for key in ("w_gate", "gate_bias", "w13", "w2"):
        if key not in dev:
            dev[key] = to_dev(d[key])
    x = to_dev(d["x"])
    bufs = moe_layer_amd.moe_layer_forward(x, dev["w_gate"], dev["gate_bias"], dev["w13"], dev["w2"],
                                           k, renorm, n_shared, g_begin, fused=fused)
    torch.cuda.synchronize()
    out = {name: from_dev(getattr(bufs, name)) for name in
           ("logits", "topk_ids", "topk_w", "counts", "offsets", "sorted_pair", "pair_pos", "a",
            "y_pair", "y")}
    return out


def check_layer(d, cfg, g, k=None, renorm=None, n_shared=None, g_begin=None, expect_near_ties=0):
    """Compare a GPU pass with the oracle, step by step and end to end.

    Returns a dict of measured errors.
    """
    k = cfg.k if k is None else k
    renorm = cfg.renorm if renorm is None else renorm
    n_shared = cfg.n_shared if n_shared is None else n_shared
    g_begin = d.get("g_begin", 0) if g_begin is None else g_begin
    T = d["x"].shape[0]
    kk = k + n_shared
    n_groups = d["w13"].shape[0]
    ref = oracle.moe_layer(d["x"], d["w_gate"], d["gate_bias"], d["w13"], d["w2"], k, renorm,
                           n_shared, g_begin)
    stats = {}

    # gate logits: fp32 GPU vs fp64 oracle
    lmax = np.abs(ref["logits"]).max()
    lerr = float(np.abs(g["logits"].astype(np.float64) - ref["logits"]).max())
    assert lerr <= LOGIT_REL * lmax, f"logits max err {lerr:.3e} > {LOGIT_REL} * {lmax:.3e}"
    stats["logit_err"] = lerr

    # routing decision on the GPU's own logits: bit-exact ids, weights to 1e-5
    ids_g, w_g = oracle.route(g["logits"].astype(np.float64), k, renorm, n_shared)
    assert np.array_equal(g["topk_ids"], ids_g), "topk ids differ from oracle top-k on GPU logits"
    werr = float(np.abs(g["topk_w"] - w_g).max())
    assert werr <= WEIGHT_ABS, f"topk weights max err {werr:.3e}"

    # permutation of the GPU's ids: bit-exact
    counts, offsets, sp, pos = oracle.permute(g["topk_ids"], g_begin, n_groups)
    n_kept = int(offsets[-1])
    assert np.array_equal(g["counts"], counts)
    assert np.array_equal(g["offsets"], offsets)
    assert np.array_equal(g["sorted_pair"][:n_kept], sp)
    assert np.array_equal(g["pair_pos"], pos)

    # end-to-end routing vs the fp64 oracle: equal except near-ties
    lr = np.sort(ref["logits"], axis=1)[:, ::-1]
    E = lr.shape[1]
    margin = lr[:, k - 1] - lr[:, k] if k < E else np.full(T, np.inf)
    near = margin <= 4 * max(lerr, 1e-30)
    # (the order inside the top-k was already checked on the GPU's own logits)
    same = (np.sort(g["topk_ids"][:, :k], axis=1) == np.sort(ref["ids"][:, :k], axis=1)).all(axis=1)
    assert same[~near].all(), "routing differs from the fp64 oracle on a token with a clear margin"
    stats["near_ties"] = int(near.sum())
    assert stats["near_ties"] <= expect_near_ties, f"{stats['near_ties']} near-tie tokens"

    # expert GEMMs on the same permutation
    A_ref, Y_ref = oracle.grouped_ffn(d["x"], sp, offsets, kk, d["w13"], d["w2"])
    stats["a_err"] = assert_close(g["a"][:n_kept], A_ref, cfg.dtype, "A (silu(gate)*up)")
    stats["ypair_err"] = assert_close(g["y_pair"][:n_kept], Y_ref, cfg.dtype, "y_pair")

    # combine on the GPU's own pair outputs, element by element
    check_combine(g["y"], g["y_pair"][:n_kept], g["pair_pos"], g["topk_w"], T, kk, cfg.dtype)

    # end to end (tokens at a near-tie excluded)
    keep = ~near
    stats["y_err"] = assert_close(g["y"][keep], ref["y"][keep], cfg.dtype, "y (layer output)")
    return stats
