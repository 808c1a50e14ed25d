"""CPU oracle of Sem-MoE's request scheduling under data-parallel attention.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``).

What it follows -- Sem-MoE notes, online data scheduling (the Attention-DP
branch): once the co-clustering has fixed which cluster (= DP/EP rank) every
token belongs to (the 0-1 matrix R, one cluster per token), a whole request r
goes to the rank its tokens are most affine to,

    S_r = argmax_j  sum_{i in r} R_ij ,

and a workload-aware balancing rule makes every E consecutive requests cover
all E ranks, so decoding load does not skew.

Readings where the notes are silent (each one is a pin in tests/test_oracle.py):

* R is given as cluster_of_token[v] for every vocabulary id v (each token in
  exactly one cluster); i ranges over the request's token positions, so a
  repeated token counts once per occurrence.
* argmax ties go to the lowest rank.
* Balancing: requests are taken in arrival order in consecutive groups of E
  (the last group may be shorter); inside a group each request takes, among
  the ranks no earlier request of its group has taken, the one with the
  largest score (ties to the lowest rank).
"""
import numpy as np


def cluster_scores(tokens, offsets, cluster_of_token, E):
    """scores[r, j] = number of token positions of request r whose token is in
    cluster j.  Request r is tokens[offsets[r]:offsets[r+1]]."""
    tokens = np.asarray(tokens, dtype=np.int64)
    offsets = np.asarray(offsets, dtype=np.int64)
    cl = np.asarray(cluster_of_token, dtype=np.int64)
    n = len(offsets) - 1
    scores = np.zeros((n, E), dtype=np.int64)
    for r in range(n):
        for pos in range(offsets[r], offsets[r + 1]):
            scores[r, cl[tokens[pos]]] += 1
    return scores


def affinity_rank(scores):
    """S_r: the rank with the largest score, ties to the lowest."""
    scores = np.asarray(scores)
    out = np.empty(scores.shape[0], dtype=np.int64)
    for r, row in enumerate(scores):
        best = 0
        for j in range(1, len(row)):
            if row[j] > row[best]:
                best = j
        out[r] = best
    return out


def balanced_ranks(scores):
    """Every group of E consecutive requests takes E distinct ranks: in
    arrival order, each request takes its best rank not yet taken in its
    group (ties to the lowest)."""
    scores = np.asarray(scores)
    n, E = scores.shape
    out = np.empty(n, dtype=np.int64)
    for g0 in range(0, n, E):
        taken = set()
        for r in range(g0, min(g0 + E, n)):
            best = None
            for j in range(E):
                if j in taken:
                    continue
                if best is None or scores[r, j] > scores[r, best]:
                    best = j
            out[r] = best
            taken.add(best)
    return out
