"""Seeded synthetic inputs for the DDTree verify step.

This module only draws random inputs with the shapes and value distributions of
the benchmark workloads; it holds none of the method's arithmetic (no tree
construction, attention or acceptance).  Both the HIP library's tests/benchmark
and the CPU oracle consume what it produces.

Workloads (drafter top-K log-probs = log-softmax over the K drafted logits, which
are N(0, sigma=2), sorted best first; token ids distinct per depth; KV and
queries N(0, 1), cast to bf16 with round-to-nearest-even except the fp32 tiny
case; one pool slot per token, prefix then tree entries per request):

  tiny_fp32    B=1  H=4  64+16 fp32  L=32      D=4  K=4   budget 8   p=0.7
  b1_l2k_q9    B=1  H=64 512+64 bf16 L=2048    D=8  K=8   budget 8   p=0.7
  b4_l4k_q17   B=4  H=64 512+64 bf16 L~4096+-25% D=15 K=8 budget 16  p=0.8
  b4_l4k_q33   as above, budget 32
  b64_l2k_q9   B=64 H=64 512+64 bf16 L=2048    D=8  K=8   budget 8   p=0.7,
               every 4th request has top-1 prob 0.995 (tree degenerates to a chain)
  b8_l32k_q65  B=8  H=64 512+64 bf16 L=32768   D=15 K=16  budget 64, top-1 prob 0.9,
               accept length drawn uniformly from 1..16 through the target tokens
  b64_l2k_q9_h8, b8_l32k_q65_h8   the two above with H=8 (a tensor-parallel
               rank's head share)
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

VOCAB_TINY = 512
VOCAB_K2 = 160000

CONFIGS = {
    "tiny_fp32": dict(B=1, H=4, d_lat=64, d_rope=16, dtype="f32", L=32, L_jitter=0.0,
                      D=4, K=4, budget=8, vocab=VOCAB_TINY, p_match=0.7, seed=0,
                      sm_scale=1.0 / math.sqrt(64 + 16)),
    "b1_l2k_q9": dict(B=1, H=64, d_lat=512, d_rope=64, dtype="bf16", L=2048, L_jitter=0.0,
                      D=8, K=8, budget=8, vocab=VOCAB_K2, p_match=0.7, seed=1),
    "b4_l4k_q17": dict(B=4, H=64, d_lat=512, d_rope=64, dtype="bf16", L=4096, L_jitter=0.25,
                       D=15, K=8, budget=16, vocab=VOCAB_K2, p_match=0.8, seed=2),
    "b4_l4k_q33": dict(B=4, H=64, d_lat=512, d_rope=64, dtype="bf16", L=4096, L_jitter=0.25,
                       D=15, K=8, budget=32, vocab=VOCAB_K2, p_match=0.8, seed=2),
    "b64_l2k_q9": dict(B=64, H=64, d_lat=512, d_rope=64, dtype="bf16", L=2048, L_jitter=0.0,
                       D=8, K=8, budget=8, vocab=VOCAB_K2, p_match=0.7, seed=3,
                       chain_every=4, chain_p1=0.995),
    "b8_l32k_q65": dict(B=8, H=64, d_lat=512, d_rope=64, dtype="bf16", L=32768, L_jitter=0.0,
                        D=15, K=16, budget=64, vocab=VOCAB_K2, p_match=None, seed=4,
                        all_p1=0.9, accept_lengths=(1, 16)),
}
# One GPU's share of the heads under 8-way tensor parallelism (64 / 8 = 8 heads):
# the same requests with H = 8.
CONFIGS["b64_l2k_q9_h8"] = dict(CONFIGS["b64_l2k_q9"], H=8)
CONFIGS["b8_l32k_q65_h8"] = dict(CONFIGS["b8_l32k_q65"], H=8)
DEFAULT_SM_SCALE = 1.0 / math.sqrt(128 + 64)


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    H: int
    d_lat: int
    d_rope: int
    dtype: str            # "f32" or "bf16"
    D: int
    K: int
    budget: int
    vocab: int
    sm_scale: float
    seed: int
    spec: dict
    # drafter side
    topk_logp: np.ndarray   # [B,D,K] f32
    topk_ids: np.ndarray    # [B,D,K] i32
    root_token: np.ndarray  # [B] i32
    prefix_len: np.ndarray  # [B] i32
    # KV side (torch CPU tensors in the workload dtype), may be None
    q_lat: torch.Tensor | None = None   # [B,Q,H,d_lat]
    q_pe: torch.Tensor | None = None    # [B,Q,H,d_rope]
    c_kv: torch.Tensor | None = None    # [S,d_lat]
    k_pe: torch.Tensor | None = None    # [S,d_rope]
    req_to_slot: np.ndarray | None = None  # [B,max_kv] i32

    @property
    def Q(self) -> int:
        return self.budget + 1

    @property
    def max_kv(self) -> int:
        return int(self.prefix_len.max()) + self.Q

    @property
    def num_slots(self) -> int:
        return 0 if self.c_kv is None else int(self.c_kv.shape[0])

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


def _log_softmax(x: np.ndarray) -> np.ndarray:
    m = x.max(axis=-1, keepdims=True)
    z = np.log(np.exp(x - m).sum(axis=-1, keepdims=True))
    return x - m - z


def _drafter_logp(rng, B, D, K, spec) -> np.ndarray:
    """Per-depth top-K log-probs, sorted best first ([B,D,K] f32)."""
    logits = rng.normal(0.0, 2.0, size=(B, D, K))
    logp = _log_softmax(logits)
    p1_rows = np.zeros((B,), dtype=bool)
    p1 = None
    if "all_p1" in spec:
        p1_rows[:] = True
        p1 = spec["all_p1"]
    elif "chain_every" in spec:
        p1_rows[spec["chain_every"] - 1::spec["chain_every"]] = True
        p1 = spec["chain_p1"]
    if p1 is not None and K >= 2:
        # Top-1 probability forced to p1; the other K-1 share 1-p1 in proportion
        # to their own softmax.
        rest = _log_softmax(logits[..., 1:]) + math.log1p(-p1)
        forced = np.concatenate([np.full((B, D, 1), math.log(p1)), rest], axis=-1)
        logp = np.where(p1_rows[:, None, None], forced, logp)
    logp = -np.sort(-logp, axis=-1)
    return logp.astype(np.float32)


def make_workload(name: str, seed: int | None = None, with_kv: bool = True,
                  shuffle_slots: bool = False, **overrides) -> Workload:
    """Draw the named workload.  `overrides` replace entries of its spec
    (e.g. B=2, L=100) to derive smaller parity cases of the same shape family."""
    spec = dict(CONFIGS[name])
    spec.update(overrides)
    seed = spec["seed"] if seed is None else seed
    rng = np.random.default_rng(seed)
    B, D, K, V = spec["B"], spec["D"], spec["K"], spec["vocab"]
    Q = spec["budget"] + 1

    if spec["L_jitter"] > 0:
        lens = np.rint(spec["L"] * rng.uniform(1 - spec["L_jitter"], 1 + spec["L_jitter"], B))
    else:
        lens = np.full((B,), spec["L"])
    prefix_len = lens.astype(np.int32)

    # Token ids: K distinct ids per (request, depth).
    ids = np.empty((B, D, K), dtype=np.int32)
    for b in range(B):
        for d in range(D):
            ids[b, d] = rng.choice(V, size=K, replace=False)
    root = rng.integers(0, V, size=B).astype(np.int32)
    logp = _drafter_logp(rng, B, D, K, spec)

    wl = Workload(name=name, B=B, H=spec["H"], d_lat=spec["d_lat"], d_rope=spec["d_rope"],
                  dtype=spec["dtype"], D=D, K=K, budget=spec["budget"], vocab=V,
                  sm_scale=float(np.float32(spec.get("sm_scale", DEFAULT_SM_SCALE))),
                  seed=seed, spec=spec, topk_logp=logp, topk_ids=ids, root_token=root,
                  prefix_len=prefix_len)
    if not with_kv:
        return wl

    # Pool: request b owns L_b prefix slots then Q tree slots, contiguous.
    per_req = prefix_len.astype(np.int64) + Q
    base = np.concatenate([[0], np.cumsum(per_req)[:-1]])
    S = int(per_req.sum())
    max_kv = int(prefix_len.max()) + Q
    r2s = np.full((B, max_kv), -1, dtype=np.int64)
    for b in range(B):
        r2s[b, :per_req[b]] = base[b] + np.arange(per_req[b])

    tdt = torch.float32 if spec["dtype"] == "f32" else torch.bfloat16
    c_kv = rng.standard_normal((S, spec["d_lat"]), dtype=np.float32)
    k_pe = rng.standard_normal((S, spec["d_rope"]), dtype=np.float32)
    q_lat = rng.standard_normal((B, Q, spec["H"], spec["d_lat"]), dtype=np.float32)
    q_pe = rng.standard_normal((B, Q, spec["H"], spec["d_rope"]), dtype=np.float32)
    if shuffle_slots:
        perm = rng.permutation(S)
        r2s = np.where(r2s >= 0, perm[np.maximum(r2s, 0)], -1)
    wl.c_kv = torch.from_numpy(c_kv).to(tdt)
    wl.k_pe = torch.from_numpy(k_pe).to(tdt)
    wl.q_lat = torch.from_numpy(q_lat).to(tdt)
    wl.q_pe = torch.from_numpy(q_pe).to(tdt)
    wl.req_to_slot = r2s.astype(np.int32)
    return wl


def synth_target_argmax(wl: Workload, node_token: np.ndarray, parent: np.ndarray,
                        depth: np.ndarray, n_nodes: np.ndarray,
                        seed: int | None = None) -> np.ndarray:
    """Synthetic target-model greedy tokens [B,Q] for a drafted tree.

    Default: at a node of depth d < D the target agrees with the drafter's top-1
    token for depth d+1 with probability p_match, otherwise it draws a different
    token uniformly; deeper nodes get uniform tokens.  Workloads with
    `accept_lengths` instead draw A uniformly, pick a random node at depth A-1 and
    make the target follow the root path to it, then disagree with all of that
    node's children, so exactly A tree nodes are accepted."""
    spec = wl.spec
    rng = np.random.default_rng((wl.seed if seed is None else seed, 7))
    B, Q = node_token.shape
    V = wl.vocab
    tgt = rng.integers(0, V, size=(B, Q)).astype(np.int64)
    if spec.get("accept_lengths") is None:
        u = rng.random((B, Q))
        other = rng.integers(0, V - 1, size=(B, Q))
        for b in range(B):
            for n in range(int(n_nodes[b])):
                d = int(depth[b, n])
                if d < wl.D:
                    top1 = int(wl.topk_ids[b, d, 0])
                    tgt[b, n] = top1 if u[b, n] < spec["p_match"] else (
                        other[b, n] + (other[b, n] >= top1))
        return tgt.astype(np.int32)

    lo, hi = spec["accept_lengths"]
    for b in range(B):
        nb = int(n_nodes[b])
        dep = depth[b, :nb]
        A = int(rng.integers(lo, hi + 1))
        A = min(A, int(dep.max()) + 1)
        cands = np.flatnonzero(dep == A - 1)
        node = int(cands[rng.integers(0, len(cands))])
        path = [node]
        while path[-1] != 0:
            path.append(int(parent[b, path[-1]]))
        path.reverse()
        for k in range(len(path) - 1):
            tgt[b, path[k]] = node_token[b, path[k + 1]]
        child_tokens = {int(node_token[b, c]) for c in range(nb) if parent[b, c] == node}
        t = int(rng.integers(0, V))
        while t in child_tokens:
            t = int(rng.integers(0, V))
        tgt[b, node] = t
    return tgt.astype(np.int32)


SAMPLING_TEMPERATURES = (0.0, 0.7, 1.0, 1.5)


def sampling_inputs(node_token: np.ndarray, parent: np.ndarray, n_nodes: np.ndarray, V: int,
                    seed: int = 0, temperatures=SAMPLING_TEMPERATURES, sigma: float = 2.0,
                    p_hit: float = 0.7, dtype=torch.bfloat16):
    """Target-side inputs of sampling acceptance for a drafted tree.

    logits [B,Q,V]: N(0, sigma) per node; at a node with children, with
    probability p_hit one child's token (uniform among the children) gets the
    row's log-sum-exp plus delta ~ U(-1, 3), so the target gives it roughly
    27%..95% of its mass at temperature 1 and drafts are accepted at a useful
    rate.  Returned as a torch tensor of `dtype` (the boosted entry is set
    after rounding the row).  temperature [B] cycles through `temperatures`;
    coins [B,Q] and coin_final [B] are U[0, 1) float32."""
    rng = np.random.default_rng((seed, 11))
    B, Q = node_token.shape
    x = torch.from_numpy(rng.standard_normal((B, Q, V), dtype=np.float32) * np.float32(sigma))
    x = x.to(dtype)
    for b in range(B):
        nb = int(n_nodes[b])
        for n in range(nb):
            kids = [c for c in range(n + 1, nb) if parent[b, c] == n]
            if not kids or rng.random() >= p_hit:
                continue
            c = kids[int(rng.integers(0, len(kids)))]
            t = int(node_token[b, c])
            if not 0 <= t < V:
                continue
            row = x[b, n].double()
            lse = float(torch.logsumexp(row, 0))
            x[b, n, t] = lse + float(rng.uniform(-1.0, 3.0))
    temperature = np.array([temperatures[b % len(temperatures)] for b in range(B)], np.float32)
    coins = rng.random((B, Q), dtype=np.float32)
    coin_final = rng.random((B,), dtype=np.float32)
    return x, temperature, coins, coin_final
