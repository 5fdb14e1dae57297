"""A multi-step DDTree decode loop driven by a synthetic deterministic target.

The check the pages hold every engine to ("The Milestone Message ...": greedy
DDTree output equals autoregressive greedy output): with a target model that is
a pure function of the token sequence, every step (draft -> build -> verify ->
accept -> commit) must extend each request's sequence exactly as autoregressive
greedy decoding with the same target would.  No model is involved:

* target(seq) -- the "greedy next token" -- is an FNV-1a hash of the last three
  tokens and the length, modulo the vocabulary;
* the drafter's per-depth top-K holds the true continuation at rank 0 with
  probability p_hit, at a lower rank or not at all otherwise, among distinct
  random tokens, with log-probs from sorted N(0, 2) logits.

The loop keeps a paged KV slot table the way a caller of the library would:
tree nodes get fresh pool slots before verification, the commit returns the
rejected ones, and the committed prefix always covers every token but the
current root.  The backend is either the CPU oracle or the HIP library.
"""
from __future__ import annotations

import numpy as np

FNV_OFFSET, FNV_PRIME = 0x811C9DC5, 0x01000193


def target(seq, vocab: int) -> int:
    h = FNV_OFFSET
    for t in list(seq[-3:]) + [len(seq)]:
        for k in range(4):
            h ^= (int(t) >> (8 * k)) & 0xFF
            h = (h * FNV_PRIME) & 0xFFFFFFFF
    return h % vocab


def ar_continue(seq, n: int, vocab: int):
    s = list(seq)
    for _ in range(n):
        s.append(target(s, vocab))
    return s


def draft_topk(rng, seqs, D: int, K: int, vocab: int, p_hit: float):
    """Per-depth top-K (log-probs, ids) for each request's current root."""
    B = len(seqs)
    logp = np.empty((B, D, K), np.float32)
    ids = np.empty((B, D, K), np.int32)
    for b, seq in enumerate(seqs):
        truth = ar_continue(seq, D, vocab)[len(seq):]
        for d in range(D):
            x = np.sort(rng.normal(0.0, 2.0, size=K))[::-1]
            lp = x - (x.max() + np.log(np.exp(x - x.max()).sum()))
            logp[b, d] = lp.astype(np.float32)
            row = rng.choice(vocab, size=K + 1, replace=False)
            row = row[row != truth[d]][:K]
            u = rng.random()
            if u < p_hit:
                rank = 0
            elif u < p_hit + (1 - p_hit) / 2 and K > 1:
                rank = int(rng.integers(1, K))
            else:
                rank = -1  # the true token is not drafted
            row = list(row[:K])
            if rank >= 0:
                row.insert(rank, truth[d])
            ids[b, d] = np.array(row[:K], np.int32)
    return logp, ids


def targets_for_tree(seqs, node_token, parent, n_nodes, vocab: int):
    """target_argmax[b][i] = target(seq_b + tokens on the path root -> i, root excluded)."""
    B, Q = node_token.shape
    out = np.zeros((B, Q), np.int32)
    for b in range(B):
        for i in range(int(n_nodes[b])):
            path = []
            k = i
            while k > 0:
                path.append(int(node_token[b, k]))
                k = int(parent[b, k])
            out[b, i] = target(list(seqs[b]) + path[::-1], vocab)
    return out


class Pool:
    """Free list of pool slots (the caller's allocator)."""

    def __init__(self, rng, n: int):
        self.free = list(rng.permutation(n).astype(np.int64))

    def take(self, k: int):
        assert len(self.free) >= k, "pool exhausted"
        out, self.free = self.free[:k], self.free[k:]
        return out

    def give(self, slots):
        self.free.extend(int(s) for s in slots)


def run_loop(backend, steps: int, B: int = 3, D: int = 6, K: int = 4, budget: int = 12,
             vocab: int = 509, p_hit: float = 0.75, prompt_len: int = 20, seed: int = 0):
    """Run `steps` DDTree steps; returns (sequences, per-step records).

    `backend` provides build(logp, ids, root, plen, budget) -> tree dict,
    verify(r2s, plen, tree) (may do nothing), accept(tree, tgt) -> dict and
    commit(r2s, plen, n_nodes, accept_len, accept_nodes) -> (r2s, plen, freed,
    n_freed), all on numpy arrays."""
    rng = np.random.default_rng(seed)
    Q = budget + 1
    seqs = [list(rng.integers(0, vocab, size=prompt_len)) for _ in range(B)]
    max_kv = prompt_len + steps * (D + 2) + Q + 4
    pool = Pool(rng, B * max_kv + 64)
    r2s = np.full((B, max_kv), -1, np.int32)
    plen = np.full((B,), prompt_len - 1, np.int32)  # every token but the root is committed
    for b in range(B):
        r2s[b, :prompt_len - 1] = pool.take(prompt_len - 1)
    records = []
    for _ in range(steps):
        logp, ids = draft_topk(rng, seqs, D, K, vocab, p_hit)
        root = np.array([s[-1] for s in seqs], np.int32)
        tree = backend.build(logp, ids, root, plen, budget)
        n = tree["n_nodes"]
        for b in range(B):
            L = int(plen[b])
            r2s[b, L:L + int(n[b])] = pool.take(int(n[b]))
        backend.verify(r2s, plen, tree)
        tgt = targets_for_tree(seqs, tree["node_token"], tree["parent"], n, vocab)
        acc = backend.accept(tree, tgt)
        r2s, plen, freed, n_freed = backend.commit(r2s, plen, n, acc["accept_len"],
                                                   acc["accept_nodes"])
        for b in range(B):
            pool.give(freed[b][:int(n_freed[b])])
            k = int(acc["accept_len"][b])
            seqs[b].extend(int(t) for t in acc["out_tokens"][b][:k])
            assert int(plen[b]) == len(seqs[b]) - 1
            live = r2s[b][:int(plen[b])]
            assert len(set(live.tolist())) == len(live), "a committed slot appears twice"
            assert not (set(live.tolist()) & set(pool.free)), "a committed slot is free"
        records.append({"accept_len": acc["accept_len"].copy(), "plen": plen.copy(),
                        "r2s": r2s.copy()})
    return seqs, records
