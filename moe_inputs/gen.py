"""Seeded generators for the synthetic MoE-layer workloads.

Recipe (every draw is reproducible from ``seed`` alone):

* Each tensor (and, for expert weights, each expert) draws from its own numpy
  ``Generator`` seeded by ``SeedSequence(seed, spawn_key=(tensor_id, index))``,
  so a tensor's values do not depend on which other tensors or how many tokens
  are drawn, and expert ``e`` has the same weights in every view that holds it.
* Normals are drawn in float32 and scaled by the standard deviation: x ~ N(0,1);
  gate weights and W13 ~ N(0, 1/H); W2 ~ N(0, 1/I) with the *full* I, also for
  the tensor-parallel slices.  bf16 inputs are then rounded to nearest even
  on the float32 bit pattern and kept as uint16 bit patterns.
* x is drawn once at (T_max, H); a batch of T tokens is its first T rows, so
  the routing of the sweep's batches is nested.
* The skewed workloads add a fixed gate bias b_e = -1.2 ln(rho_e), where rho is
  1 + a seeded permutation of 0..E-1: the routing prior is then proportional
  to rho^-1.2 (a Zipf law with s = 1.2), standing in for the concentrated
  token-expert affinity that the Sem-MoE notes report (profiled activation
  statistics, Key design 1).  The uniform workloads use b = 0.

Nothing here computes any part of the layer.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import LayerConfig

# tensor ids used as the first spawn-key element
(_X, _W_GATE, _RHO, _W13, _W2, _W13_SHARED, _W2_SHARED, _W13_TP, _W2_TP, _IDS, _TRACE,
 _REQ) = range(12)

ZIPF_S = 1.2


def _rng(seed: int, tensor_id: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tensor_id, index)))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs must be finite.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def _normal_block(seed, tensor_id, index, shape, std, dtype):
    z = _rng(seed, tensor_id, index).standard_normal(shape, dtype=np.float32)
    z *= np.float32(std)
    return bf16_bits_from_f32(z) if dtype == "bf16" else z


def _stack(seed, tensor_id, indices, shape, std, dtype):
    """Draw one block per index (in parallel threads) and stack them."""
    out_dtype = np.uint16 if dtype == "bf16" else np.float32
    out = np.empty((len(indices),) + tuple(shape), dtype=out_dtype)

    def fill(j):
        out[j] = _normal_block(seed, tensor_id, indices[j], shape, std, dtype)

    workers = max(1, min(16, os.cpu_count() or 1, len(indices)))
    if workers == 1:
        for j in range(len(indices)):
            fill(j)
    else:
        with ThreadPoolExecutor(workers) as pool:
            list(pool.map(fill, range(len(indices))))
    return out


def gate_bias(cfg: LayerConfig, routing: str, seed: int = 0) -> np.ndarray:
    if routing == "uniform":
        return np.zeros(cfg.E, dtype=np.float32)
    if routing != "zipf":
        raise ValueError(f"unknown routing variant {routing!r}")
    rho = 1.0 + _rng(seed, _RHO).permutation(cfg.E).astype(np.float64)
    return (-ZIPF_S * np.log(rho)).astype(np.float32)


def ep_rank_for(cfg: LayerConfig, routing: str, seed: int = 0) -> int:
    """Which EP rank's share to emulate: rank 0 under uniform routing; under
    skewed routing the rank whose contiguous experts carry the largest prior
    mass (the straggler that sets an EP step's time)."""
    if routing == "uniform" or cfg.view != "ep":
        return 0
    prior = np.exp(gate_bias(cfg, routing, seed).astype(np.float64))
    per_rank = prior.reshape(cfg.P, cfg.E // cfg.P).sum(axis=1)
    return int(np.argmax(per_rank))


def make_x(cfg: LayerConfig, T: int, seed: int = 0, T_draw: int = None) -> np.ndarray:
    T_draw = max(T, T_draw or cfg.T_max)
    x = _normal_block(seed, _X, 0, (T_draw, cfg.H), 1.0, cfg.dtype)
    return np.ascontiguousarray(x[:T])


def make_gate(cfg: LayerConfig, seed: int = 0) -> np.ndarray:
    return _normal_block(seed, _W_GATE, 0, (cfg.E, cfg.H), cfg.H ** -0.5, cfg.dtype)


def expert_weights(cfg: LayerConfig, experts, seed: int = 0):
    """Whole routed experts (ids into 0..E-1): W13 (n, 2I, H), W2 (n, H, I)."""
    experts = list(experts)
    w13 = _stack(seed, _W13, experts, (2 * cfg.I, cfg.H), cfg.H ** -0.5, cfg.dtype)
    w2 = _stack(seed, _W2, experts, (cfg.H, cfg.I), cfg.I ** -0.5, cfg.dtype)
    return w13, w2


def shared_weights(cfg: LayerConfig, seed: int = 0):
    idx = list(range(cfg.n_shared))
    w13 = _stack(seed, _W13_SHARED, idx, (2 * cfg.I, cfg.H), cfg.H ** -0.5, cfg.dtype)
    w2 = _stack(seed, _W2_SHARED, idx, (cfg.H, cfg.I), cfg.I ** -0.5, cfg.dtype)
    return w13, w2


def routing_table(cfg: LayerConfig, T: int, routing: str = "uniform", seed: int = 0) -> np.ndarray:
    """A synthetic routing table (T, k + n_shared) int32 for the steps after
    the gate: per token, k distinct routed ids drawn without replacement with
    probabilities proportional to exp(gate bias) (uniform, or the Zipf prior
    above), then the shared ids E, E+1, ...  Draws only; no gate involved."""
    prior = np.exp(gate_bias(cfg, routing, seed).astype(np.float64))
    prior /= prior.sum()
    rng = _rng(seed, _IDS, T)
    ids = np.empty((T, cfg.kk), dtype=np.int32)
    for t in range(T):
        ids[t, :cfg.k] = rng.choice(cfg.E, size=cfg.k, replace=False, p=prior)
    ids[:, cfg.k:] = cfg.E + np.arange(cfg.n_shared, dtype=np.int32)
    return ids


def make_layer_inputs(cfg: LayerConfig, T: int, routing: str = "uniform", seed: int = 0,
                      rank: int = None) -> dict:
    """Host arrays for one forward pass of ``cfg`` on T tokens.

    Returns x (T,H), w_gate (E,H), gate_bias (E,) float32, w13 (n_groups,2I',H),
    w2 (n_groups,H,I') and the view parameters (g_begin, rank).  bf16 arrays are
    uint16 bit patterns; fp32 arrays are float32.
    """
    d = {
        "x": make_x(cfg, T, seed),
        "w_gate": make_gate(cfg, seed),
        "gate_bias": gate_bias(cfg, routing, seed),
        "routing": routing,
        "T": T,
    }
    if cfg.view == "ep":
        r = ep_rank_for(cfg, routing, seed) if rank is None else rank
        E_l = cfg.E // cfg.P
        d["w13"], d["w2"] = expert_weights(cfg, range(r * E_l, (r + 1) * E_l), seed)
        d["rank"], d["g_begin"] = r, r * E_l
    elif cfg.view == "tp":
        # This GPU's slice of every expert, drawn directly at the slice's shape.
        Il = cfg.I_local
        idx = list(range(cfg.E))
        d["w13"] = _stack(seed, _W13_TP, idx, (2 * Il, cfg.H), cfg.H ** -0.5, cfg.dtype)
        d["w2"] = _stack(seed, _W2_TP, idx, (cfg.H, Il), cfg.I ** -0.5, cfg.dtype)
        d["rank"] = 0 if rank is None else rank
        d["g_begin"] = 0
    else:
        w13, w2 = expert_weights(cfg, range(cfg.E), seed)
        if cfg.n_shared:
            s13, s2 = shared_weights(cfg, seed)
            w13 = np.concatenate([w13, s13])
            w2 = np.concatenate([w2, s2])
        d["w13"], d["w2"] = w13, w2
        d["rank"], d["g_begin"] = 0, 0
    return d


def make_full_model(cfg: LayerConfig, T: int, routing: str = "uniform", seed: int = 0) -> dict:
    """Whole-model weights (every routed expert at full I, plus shared experts).

    Used to build every rank's share of a small model, so that the sum over
    ranks can be checked against the whole layer.
    """
    w13, w2 = expert_weights(cfg, range(cfg.E), seed)
    if cfg.n_shared:
        s13, s2 = shared_weights(cfg, seed)
        w13 = np.concatenate([w13, s13])
        w2 = np.concatenate([w2, s2])
    return {
        "x": make_x(cfg, T, seed),
        "w_gate": make_gate(cfg, seed),
        "gate_bias": gate_bias(cfg, routing, seed),
        "w13": w13,
        "w2": w2,
        "routing": routing,
        "T": T,
    }


def make_repack_inputs(cfg: LayerConfig, seed: int = 0, rank: int = 0) -> dict:
    """EP-layout expert weights of one rank (its E/P whole experts)."""
    E_l = cfg.E // cfg.P
    w13, w2 = expert_weights(cfg, range(rank * E_l, (rank + 1) * E_l), seed)
    return {"w13_ep": w13, "w2_ep": w2, "rank": rank}


def load_trace(kind: str, n: int, seed: int = 0):
    """A synthetic serving load: the count of in-flight requests at each of n
    decode iterations, and each iteration's duration in seconds.

    * "burst": online serving with bursts (the bursty serving workload of the
      Moebius review): a base load of about 60 requests with Poisson noise,
      and bursts that ramp up to 400-1600 requests over some tens of
      iterations and drain over a few hundred;
    * "rollout": RL rollout rounds: each round starts with 1000-2048 requests
      that finish one by one (geometric lifetimes), a long tail of stragglers
      at the end of every round;
    * "noise": a random walk between 0 and 200 requests.
    Iterations take 20-60 ms.  Draws only; no policy involved.
    """
    rng = _rng(seed, _TRACE, {"burst": 0, "rollout": 1, "noise": 2}[kind])
    if kind == "burst":
        base = rng.poisson(60, size=n).astype(np.float64)
        load = base.copy()
        t = int(rng.integers(100, 300))
        while t < n:
            peak = rng.uniform(400, 1600)
            up, down = int(rng.integers(10, 60)), int(rng.integers(150, 500))
            shape = np.concatenate([np.linspace(0, 1, up, endpoint=False), np.linspace(1, 0, down)])
            seg = min(len(shape), n - t)
            load[t:t + seg] += peak * shape[:seg]
            t += seg + int(rng.integers(200, 700))
        counts = np.maximum(load, 0).round().astype(np.int64)
    elif kind == "rollout":
        counts = np.zeros(n, dtype=np.int64)
        t = 0
        while t < n:
            start = int(rng.integers(1000, 2049))
            life = rng.geometric(1.0 / rng.uniform(150, 400), size=start)
            length = min(int(life.max()) + 1, n - t)
            steps = np.arange(length)
            counts[t:t + length] = (life[None, :] > steps[:, None]).sum(axis=1)
            t += length + int(rng.integers(5, 30))
    elif kind == "noise":
        counts = np.clip(np.cumsum(rng.integers(-8, 9, size=n)) + 100, 0, 200).astype(np.int64)
    else:
        raise ValueError(f"unknown trace kind {kind!r}")
    dt = rng.uniform(0.02, 0.06, size=n)
    return counts, dt


def make_requests(n_req: int, E: int, vocab: int = 151936, seed: int = 0, topical: float = 0.6,
                  median_len: float = 300.0):
    """Synthetic requests and a token->cluster map for request scheduling.

    * cluster_of_token: the vocabulary split into E equal clusters by a seeded
      permutation (the co-clustering's output stands in as a random balanced
      partition);
    * each request has a topic cluster (uniform) and a length drawn from a
      log-normal law (median ``median_len``, sigma 1, clipped to 1..8192), a
      conversational prompt-length mix; each token is, with probability
      ``topical``, a uniform id of the topic cluster, else a uniform id of
      the whole vocabulary.
    Returns tokens (int32, concatenated), offsets (n_req + 1, int32),
    cluster_of_token (vocab, int32) and the topics (int32).
    """
    rng = _rng(seed, _REQ, E)
    perm = rng.permutation(vocab)
    cluster = np.empty(vocab, dtype=np.int32)
    cluster[perm] = (np.arange(vocab) * E // vocab).astype(np.int32)
    members = [perm[(np.arange(vocab) * E // vocab) == c] for c in range(E)]
    lens = np.clip(np.round(rng.lognormal(np.log(median_len), 1.0, size=n_req)), 1, 8192).astype(np.int64)
    topics = rng.integers(0, E, size=n_req).astype(np.int32)
    offsets = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    tokens = np.empty(int(offsets[-1]), dtype=np.int32)
    for r in range(n_req):
        n = int(lens[r])
        own = rng.random(n) < topical
        mem = members[topics[r]]
        ids = rng.integers(0, vocab, size=n)
        ids[own] = mem[rng.integers(0, len(mem), size=int(own.sum()))]
        tokens[offsets[r]:offsets[r + 1]] = ids
    return tokens, offsets, cluster, topics
