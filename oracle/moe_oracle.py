"""CPU oracle for one MoE layer's forward pass (numpy, float64).

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module.  The GPU library never
calls it and shares no code with it; both sides only read the same seeded
inputs from ``moe_inputs``.

What it computes (plain definitions, evaluated in float64 on the exact input
values; bf16 inputs are widened exactly, nothing is rounded in between):

* gate: ``logits = x W_g^T + b`` and ``top-k(softmax(logits))`` -- Sem-MoE notes,
  Key design 1 (the gate formula G_L(h) = top-k(softmax(W_{L,g} h + b_{L,g}))).
* the experts each rank holds in the EP and TP views, and the weight shapes
  W13 (., 2I, H) / W2 (., H, I) -- Moebius review, §3.1 (weight resharding).
* the local permute that packs each expert's slice for peer q into one block
  per destination -- Moebius review, §3.1 and Fig. 4.
* the argsort of tokens by expert -- Sem-MoE notes, Key design 4 (the argsort
  kernel used to reorder tokens).
* the EP token exchange: each token goes to the GPU that owns its expert and
  its result comes back -- Moebius review, problem definition (EP layout), and
  Sem-MoE notes, motivation (two all-to-alls per MoE layer).

Readings where the pages are silent (each one is also a test pin):

* W13 rows [0, I) are the gate projection W1 and rows [I, 2I) the up
  projection W3; the expert output is W2 (silu(W1 x) * W3 x) with
  silu(z) = z / (1 + exp(-z)).
* TP slice p of an expert is rows S_p and I + S_p of W13 (gate half first) and
  columns S_p of W2, with S_p = [p I/P, (p+1) I/P).
* EP rank r owns experts [r E/P, (r+1) E/P).
* Top-k selects on the logits (the same set as on the softmax), in
  descending order, ties to the lower expert index.
* Weights are the softmax over all E routed experts at the picked ids,
  optionally renormalised to sum to 1 over the k picks.  Shared experts are
  groups E, E+1, ... with weight 1, placed after the routed slots.
* No capacity limit: every picked (token, expert) pair is computed.
* The EP and TP outputs are partial sums: the EP rank adds only its local
  experts' terms; the TP rank adds every term restricted to its I-slice.
* EP dispatch: one send row per routed (token, slot) pair, grouped by the
  rank d = id // E_local that owns the expert, ascending pair index inside a
  group (a token picking two experts of one rank is sent twice; shared
  experts, ids >= E, stay local and are not sent).  The receiver answers with
  one unweighted expert-output row per received row, in arrival order (sender
  0's rows first); the sender applies its own routing weights when it sums.
"""
import numpy as np

__all__ = [
    "widen", "gate_logits", "softmax_rows", "topk_desc", "route", "local_ids",
    "permute", "silu", "expert_ffn", "grouped_ffn", "combine", "moe_layer",
    "tp_slice", "repack_ep_to_tp", "repack_tp_to_ep", "brute_force_layer",
    "dispatch", "ep_exchange_layer",
]


def widen(a: np.ndarray) -> np.ndarray:
    """Exact float64 value of an input array (uint16 = bf16 bit pattern)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def gate_logits(x, w_gate, bias) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] W_g[e, h] + b[e]   (Sem-MoE notes, Key design 1)."""
    return widen(x) @ widen(w_gate).T + np.asarray(bias, dtype=np.float64)[None, :]


def softmax_rows(logits: np.ndarray) -> np.ndarray:
    """Row-wise softmax over the routed experts, with the row maximum subtracted."""
    l = np.asarray(logits, dtype=np.float64)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def topk_desc(logits: np.ndarray, k: int) -> np.ndarray:
    """k rounds of argmax over the experts not yet chosen.

    Order is descending; ``np.argmax`` returns the first maximum, so equal
    logits (including -0.0 and +0.0) go to the lower expert index.
    """
    work = np.array(logits, dtype=np.float64, copy=True)
    T = work.shape[0]
    ids = np.empty((T, k), dtype=np.int32)
    rows = np.arange(T)
    for j in range(k):
        a = np.argmax(work, axis=1)
        ids[:, j] = a
        work[rows, a] = -np.inf
    return ids


def route(logits, k: int, renorm: bool, n_shared: int = 0):
    """Top-k routing table from gate logits.

    Returns ids (T, k + n_shared) int32 and weights (T, k + n_shared) float64.
    Routed slots come first in descending-logit order; shared expert s is
    id E + s with weight 1.
    """
    logits = np.asarray(logits, dtype=np.float64)
    T, E = logits.shape
    p = softmax_rows(logits)
    ids = topk_desc(logits, k)
    w = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    if n_shared:
        sid = np.broadcast_to(E + np.arange(n_shared, dtype=np.int32), (T, n_shared))
        ids = np.concatenate([ids, sid], axis=1)
        w = np.concatenate([w, np.ones((T, n_shared))], axis=1)
    return ids, w


def local_ids(ids, g_begin: int, n_groups: int) -> np.ndarray:
    """Group index of each pair inside the window [g_begin, g_begin + n_groups),
    or -1 for a pair whose expert this GPU does not hold (EP view)."""
    lg = np.asarray(ids, dtype=np.int64) - g_begin
    lg[(lg < 0) | (lg >= n_groups)] = -1
    return lg


def permute(ids, g_begin: int, n_groups: int):
    """Stable counting sort of the (token, slot) pairs by local expert group.

    Pair p = t * kk + j.  Returns counts (n_groups), offsets (n_groups + 1,
    exclusive prefix sum), sorted_pair (n_kept: the pairs in group order,
    ascending pair index inside a group) and pair_pos (T * kk: each pair's row
    in sorted order, -1 if dropped), all int32.
    """
    flat = local_ids(ids, g_begin, n_groups).ravel()
    counts = np.zeros(n_groups, dtype=np.int64)
    for g in flat:
        if g >= 0:
            counts[g] += 1
    offsets = np.zeros(n_groups + 1, dtype=np.int64)
    for g in range(n_groups):
        offsets[g + 1] = offsets[g] + counts[g]
    cursor = offsets[:-1].copy()
    sorted_pair = np.empty(int(offsets[-1]), dtype=np.int64)
    pair_pos = np.full(flat.size, -1, dtype=np.int64)
    for p, g in enumerate(flat):          # ascending pair index: stable
        if g >= 0:
            sorted_pair[cursor[g]] = p
            pair_pos[p] = cursor[g]
            cursor[g] += 1
    return (counts.astype(np.int32), offsets.astype(np.int32),
            sorted_pair.astype(np.int32), pair_pos.astype(np.int32))


def silu(z):
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z)), evaluated without overflow."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def expert_ffn(xs, w13_g, w2_g):
    """One expert on a batch of rows: a = silu(W1 x) * (W3 x); y = W2 a.

    w13_g is (2I', H) with the gate rows first; w2_g is (H, I').
    Returns (a, y) in float64.
    """
    xs = widen(xs)
    w13_g = widen(w13_g)
    w2_g = widen(w2_g)
    I = w2_g.shape[1]
    gate = xs @ w13_g[:I].T
    up = xs @ w13_g[I:].T
    a = silu(gate) * up
    return a, a @ w2_g.T


def grouped_ffn(x, sorted_pair, offsets, kk: int, w13, w2):
    """Evaluate every kept pair's expert output, one expert group at a time.

    Row r of the results belongs to pair sorted_pair[r], token sorted_pair[r] // kk.
    Returns A (n_kept, I') and y_pair (n_kept, H) in float64.
    """
    n_groups = w13.shape[0]
    H, I = w2.shape[1], w2.shape[2]
    n_kept = int(offsets[-1])
    A = np.zeros((n_kept, I))
    Y = np.zeros((n_kept, H))
    xw = widen(x)
    for g in range(n_groups):
        s, e = int(offsets[g]), int(offsets[g + 1])
        if e > s:
            tok = np.asarray(sorted_pair[s:e], dtype=np.int64) // kk
            A[s:e], Y[s:e] = expert_ffn(xw[tok], w13[g], w2[g])
    return A, Y


def combine(y_pair, pair_pos, w, T: int, kk: int) -> np.ndarray:
    """y[t] = sum over slots j = 0..kk-1 (in order) of w[t, j] * y_pair[pos[t, j]];
    slots whose pair is not held here add nothing."""
    y_pair = np.asarray(y_pair, dtype=np.float64)
    H = y_pair.shape[1]
    pos = np.asarray(pair_pos, dtype=np.int64).reshape(T, kk)
    w = np.asarray(w, dtype=np.float64).reshape(T, kk)
    y = np.zeros((T, H))
    for j in range(kk):
        m = pos[:, j] >= 0
        y[m] += w[m, j, None] * y_pair[pos[m, j]]
    return y


def moe_layer(x, w_gate, gate_bias, w13, w2, k: int, renorm: bool, n_shared: int = 0,
              g_begin: int = 0) -> dict:
    """The whole layer on one GPU's share.

    ``w13`` / ``w2`` hold ``n_groups = w13.shape[0]`` expert groups with global
    ids ``g_begin ..``: all E (+ shared) groups for the full and TP views (TP
    weights are slices along I), E/P whole experts for an EP rank.
    """
    x = np.asarray(x)
    T = x.shape[0]
    E = np.asarray(w_gate).shape[0]
    kk = k + n_shared
    n_groups = w13.shape[0]
    logits = gate_logits(x, w_gate, gate_bias)
    ids, w = route(logits, k, renorm, n_shared)
    counts, offsets, sorted_pair, pair_pos = permute(ids, g_begin, n_groups)
    A, y_pair = grouped_ffn(x, sorted_pair, offsets, kk, w13, w2)
    y = combine(y_pair, pair_pos, w, T, kk)
    return {
        "logits": logits, "ids": ids, "w": w, "counts": counts, "offsets": offsets,
        "sorted_pair": sorted_pair, "pair_pos": pair_pos, "A": A, "y_pair": y_pair,
        "y": y, "E": E,
    }


def tp_slice(w13, w2, p: int, P: int):
    """TP rank p's slice of whole experts: W13 rows S_p then I + S_p; W2 columns S_p
    (Moebius review, §3.1: TP shapes (E, 2I/P, H) and (E, H, I/P))."""
    I = w2.shape[2]
    Ip = I // P
    lo, hi = p * Ip, (p + 1) * Ip
    return (np.concatenate([w13[:, lo:hi, :], w13[:, I + lo:I + hi, :]], axis=1),
            np.ascontiguousarray(w2[:, :, lo:hi]))


def repack_ep_to_tp(w13_ep, w2_ep, P: int):
    """Local permute of the EP->TP reshard (Moebius review, §3.1 and Fig. 4).

    Packs each local expert's slice for peer q into one contiguous block per
    peer: block q of W13 is (E_local, 2I/P, H), block q of W2 is (E_local, H, I/P).
    Exact copies.  Returns two lists of P arrays.
    """
    b13, b2 = [], []
    for q in range(P):
        a, b = tp_slice(w13_ep, w2_ep, q, P)
        b13.append(a)
        b2.append(b)
    return b13, b2


def repack_tp_to_ep(blocks13, blocks2):
    """Inverse of ``repack_ep_to_tp``: rebuild whole experts from the P blocks."""
    Ip = blocks2[0].shape[2]
    gate = np.concatenate([b[:, :Ip, :] for b in blocks13], axis=1)
    up = np.concatenate([b[:, Ip:, :] for b in blocks13], axis=1)
    return np.concatenate([gate, up], axis=1), np.concatenate(list(blocks2), axis=2)


def dispatch(x, ids, E_local: int, P: int) -> dict:
    """Send side of the EP dispatch on one rank (Moebius review, problem
    definition: tokens reach the GPU that owns their expert by an all-to-all).

    Pair p = t * kk + j goes to rank ids[p] // E_local when that is < P.  The
    send layout is the stable argsort of the pairs by destination rank (the
    expert argsort above with the rank as the key): block r of the send buffer
    holds rank r's rows, ascending pair index.  Returns counts (P), offsets
    (P + 1), send_order (n_sent pair ids), pair_pos (T * kk, -1 if not sent),
    send_x (n_sent, H) exact copies of x[send_order // kk] and send_ids
    (n_sent) the global expert id of each row.
    """
    ids = np.asarray(ids, dtype=np.int64)
    kk = ids.shape[1]
    counts, offsets, send_order, pair_pos = permute(ids // E_local, 0, P)
    send_x = np.asarray(x)[send_order.astype(np.int64) // kk]
    send_ids = ids.ravel()[send_order].astype(np.int32)
    return {"counts": counts, "offsets": offsets, "send_order": send_order,
            "pair_pos": pair_pos, "send_x": send_x, "send_ids": send_ids}


def ep_exchange_layer(x_shares, w_gate, gate_bias, w13, w2, k: int, renorm: bool) -> dict:
    """The EP layer across P ranks with both exchanges written out.

    x_shares[q] is rank q's own tokens; P = len(x_shares) ranks, rank r owns
    whole experts [r E/P, (r+1) E/P) of w13 (E, 2I, H) / w2 (E, H, I).  Every
    rank routes its tokens and dispatches them; rank r takes block r of every
    sender in sender order, evaluates each received row with the expert its id
    names, and sends the unweighted outputs back in arrival order; sender q
    sums them per token with its routing weights in slot order.  Returns the
    per-rank outputs y (list) and the per-rank dispatch results.
    """
    P = len(x_shares)
    E = np.asarray(w_gate).shape[0]
    E_l = E // P
    H = np.asarray(x_shares[0]).shape[1]
    routed, sends = [], []
    for q in range(P):
        ids, w = route(gate_logits(x_shares[q], w_gate, gate_bias), k, renorm)
        routed.append((ids, w))
        sends.append(dispatch(x_shares[q], ids, E_l, P))
    back = [[None] * P for _ in range(P)]          # back[q][r]: rows rank r returns to q
    for r in range(P):
        parts = [(s["offsets"][r], s["offsets"][r + 1]) for s in sends]
        rx = np.concatenate([widen(s["send_x"][a:b]) for s, (a, b) in zip(sends, parts)])
        rid = np.concatenate([s["send_ids"][a:b] for s, (a, b) in zip(sends, parts)])
        ry = np.zeros((rx.shape[0], H))
        for e in np.unique(rid):
            rows = np.nonzero(rid == e)[0]
            _, ry[rows] = expert_ffn(rx[rows], w13[e], w2[e])
        start = 0
        for q, (a, b) in enumerate(parts):
            back[q][r] = ry[start:start + (b - a)]
            start += b - a
    ys = []
    for q in range(P):
        ids, w = routed[q]
        recv = np.concatenate(back[q], axis=0)     # rank order = send order
        ys.append(combine(recv, sends[q]["pair_pos"], w, ids.shape[0], ids.shape[1]))
    return {"y": ys, "dispatch": sends, "routed": routed}


def brute_force_layer(x, w_gate, gate_bias, w13, w2, k: int, renorm: bool,
                      n_shared: int = 0, g_begin: int = 0) -> np.ndarray:
    """Per-token dense loop, for tiny inputs only.

    For every token: logits by one dot product per expert, softmax, top-k by a
    full sort on (-logit, id); then for every expert group held here, evaluate
    its FFN densely on that token and add weight * FFN if the token picked it.
    Written independently of the grouped evaluation above (no permutation,
    no shared helpers).
    """
    from scipy.special import expit

    xs, wg, b = widen(x), widen(w_gate), np.asarray(gate_bias, dtype=np.float64)
    w13f, w2f = widen(w13), widen(w2)
    T, H = xs.shape
    E = wg.shape[0]
    G = w13f.shape[0]
    I = w2f.shape[2]
    y = np.zeros((T, H))
    for t in range(T):
        l = [float(np.dot(wg[e], xs[t])) + b[e] for e in range(E)]
        mx = max(l)
        ex = [np.exp(v - mx) for v in l]
        tot = sum(ex)
        order = sorted(range(E), key=lambda e: (-l[e], e))[:k]
        weight = {e: ex[e] / tot for e in order}
        if renorm:
            s = sum(weight.values())
            weight = {e: v / s for e, v in weight.items()}
        for s_ in range(n_shared):
            weight[E + s_] = 1.0
        for g in range(G):
            gid = g_begin + g
            if gid not in weight:
                continue
            gate = np.array([np.dot(w13f[g, i], xs[t]) for i in range(I)])
            up = np.array([np.dot(w13f[g, I + i], xs[t]) for i in range(I)])
            a = gate * expit(gate) * up
            ffn = np.array([np.dot(w2f[g, h], a) for h in range(H)])
            y[t] += weight[gid] * ffn
    return y
