"""GPU parity of the Attention-DP request scheduling: per-request cluster
counts, argmax ranks and balanced ranks bit-exact against the oracle, over
ragged request batches, partial last groups, empty requests, out-of-range ids
and a reused workspace."""
import numpy as np
import pytest

import oracle
from moe_inputs.gen import make_requests

pytestmark = pytest.mark.gpu
rs = oracle.request_schedule


def run(tokens, offsets, cluster, E, ws=None):
    import torch
    import moe_layer_amd as M
    n = len(offsets) - 1
    t = torch.from_numpy(np.ascontiguousarray(tokens, dtype=np.int32)).cuda()
    o = torch.from_numpy(np.ascontiguousarray(offsets, dtype=np.int32)).cuda()
    c = torch.from_numpy(np.ascontiguousarray(cluster, dtype=np.int32)).cuda()
    scores = torch.full((n, E), -3, dtype=torch.int32, device="cuda")
    aff = torch.full((n,), -3, dtype=torch.int32, device="cuda")
    asg = torch.full((n,), -3, dtype=torch.int32, device="cuda")
    ws = M.schedule_workspace(n, E) if ws is None else ws
    M.moe_schedule_requests(t, o, c, E, scores, aff, asg, ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero()) == 0          # every call leaves the counters zero
    return scores.cpu().numpy(), aff.cpu().numpy(), asg.cpu().numpy()


def check(tokens, offsets, cluster, E, ws=None):
    s, a, b = run(tokens, offsets, cluster, E, ws)
    ref = rs.cluster_scores(tokens, offsets, cluster, E)
    assert np.array_equal(s, ref)
    assert np.array_equal(a, rs.affinity_rank(ref))
    assert np.array_equal(b, rs.balanced_ranks(ref))
    return ref


# request batches with full and partial last groups, one rank, 64 ranks, and
# a few long requests (up to 8192 tokens)
@pytest.mark.parametrize("n_req,E,median", [(1, 8, 300), (7, 8, 300), (8, 8, 300), (9, 8, 300),
                                            (100, 4, 50), (2048, 8, 300), (130, 64, 100), (33, 1, 20),
                                            (40, 8, 3000)])
def test_schedule_matches_oracle(n_req, E, median):
    tok, off, cl, _ = make_requests(n_req, E, vocab=151936, seed=n_req + E, median_len=median)
    print(f"[case] schedule n_req={n_req} E={E} tokens={tok.size}", flush=True)
    check(tok, off, cl, E)


def test_schedule_edge_cases():
    import moe_layer_amd as M
    rng = np.random.default_rng(0)
    V, E = 1000, 8
    cl = rng.integers(0, E, size=V).astype(np.int32)
    print("[case] schedule: empty requests", flush=True)
    off = np.array([0, 0, 5, 5, 5, 12, 12], dtype=np.int32)
    tok = rng.integers(0, V, size=12).astype(np.int32)
    check(tok, off, cl, E)
    print("[case] schedule: ids and clusters out of range are not counted", flush=True)
    bad = tok.copy()
    bad[[1, 6, 9]] = [-5, V, V + 100]
    cl_bad = cl.copy()
    cl_bad[tok[3]] = E + 3                       # a cluster past the last rank
    s, a, b = run(bad, off, cl_bad, E)
    keep = (bad >= 0) & (bad < V)
    kept_tok = np.where(keep, bad, 0)
    ref = np.zeros((len(off) - 1, E), dtype=np.int64)
    for r in range(len(off) - 1):
        for p in range(off[r], off[r + 1]):
            if keep[p] and 0 <= cl_bad[kept_tok[p]] < E:
                ref[r, cl_bad[kept_tok[p]]] += 1
    assert np.array_equal(s, ref)
    assert np.array_equal(b, rs.balanced_ranks(ref))
    print("[case] schedule: one workspace, two calls of different sizes", flush=True)
    tok1, off1, cl1, _ = make_requests(300, E, vocab=V, seed=1, median_len=40)
    ws = M.schedule_workspace(300, E)
    check(tok1, off1, cl1, E, ws)
    tok2, off2, cl2, _ = make_requests(37, E, vocab=V, seed=2, median_len=40)
    check(tok2, off2, cl2, E, ws)
