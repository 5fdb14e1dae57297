"""Multi-step DDTree loop on the CPU oracle: greedy DDTree output equals
autoregressive greedy output with the same target ("The Milestone Message ...",
the validation it leads with), over many steps, with the KV slot table kept by
the commit step (see loop_harness)."""
import numpy as np
import pytest

import oracle
from loop_harness import ar_continue, run_loop


class OracleBackend:
    def build(self, logp, ids, root, plen, budget):
        return oracle.tree_build(logp, ids, root, plen, budget)

    def verify(self, r2s, plen, tree):
        pass  # the synthetic target does not read the attention output

    def accept(self, tree, tgt):
        return oracle.tree_accept(tree["node_token"], tree["parent"], tree["n_nodes"], tgt)

    def commit(self, r2s, plen, n, alen, anodes):
        c = oracle.kv_commit(r2s, plen, n, alen, anodes)
        return c["req_to_slot"], c["prefix_len"], c["freed_slots"], c["n_freed"]


@pytest.mark.parametrize("seed,p_hit,K,D,budget", [(0, 0.75, 4, 6, 12), (1, 0.95, 3, 8, 8),
                                                   (2, 0.3, 5, 4, 16), (3, 1.0, 1, 5, 5)])
def test_ddtree_greedy_equals_ar_greedy(seed, p_hit, K, D, budget):
    vocab = 509
    seqs, rec = run_loop(OracleBackend(), steps=25, K=K, D=D, budget=budget, vocab=vocab,
                         p_hit=p_hit, seed=seed)
    for s in seqs:
        prompt = s[:20]
        assert s == ar_continue(prompt, len(s) - 20, vocab)
    total = sum(int(r["accept_len"].sum()) for r in rec)
    # Every step commits at least the root; with a good drafter, more.
    assert total >= 25 * len(seqs)
    if p_hit == 1.0 and K == 1:
        # A chain drafter that is always right accepts every draft (depth D).
        assert all((r["accept_len"] == min(D, budget) + 1).all() for r in rec)
