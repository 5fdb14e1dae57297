"""Pins for the oracle's greedy follow-the-verified-tree acceptance.

What it computes ("The Architecture of Closure ...", "The Table as a Decision
Artifact": greedy follow of the verified tree on a synthesized target
prediction): from the root, keep moving to the child whose token equals the
target model's greedy token at the current node; commit the accepted draft
tokens plus the target's token at the last accepted node.

Checked against:
* brute force: with distinct sibling tokens the accepted path is the unique
  longest root path whose every token equals the target's token at its parent
  -- found by enumerating every node's root path;
* closed forms: a target that never agrees accepts only the root; a chain whose
  target always agrees accepts every node;
* a hand-made tie (two siblings with the same token): the lower index wins.
"""
import numpy as np
import pytest

import oracle
from tree_verify_mla_ddt_amd import workloads


def accept1(tok, par, n, tgt):
    r = oracle.tree_accept(np.array([tok], np.int32), np.array([par], np.int32),
                           np.array([n], np.int32), np.array([tgt], np.int32))
    return {k: v[0] for k, v in r.items()}


def brute_force(tok, par, n, tgt):
    best = [0]
    for node in range(n):
        path = [node]
        while path[-1] != 0:
            path.append(par[path[-1]])
        path.reverse()
        if all(tok[path[k]] == tgt[path[k - 1]] for k in range(1, len(path))):
            if len(path) > len(best):
                best = path
    Q = len(tok)
    nodes = np.full(Q, -1, np.int32)
    out = np.full(Q, -1, np.int32)
    nodes[: len(best)] = best
    out[: len(best) - 1] = [tok[p] for p in best[1:]]
    out[len(best) - 1] = tgt[best[-1]]
    return len(best), nodes, out, tgt[best[-1]]


@pytest.mark.parametrize("name", ["tiny_fp32", "b1_l2k_q9", "b4_l4k_q17", "b4_l4k_q33",
                                  "b64_l2k_q9", "b8_l32k_q65"])
def test_brute_force_on_workload_trees(name):
    wl = workloads.make_workload(name, with_kv=False)
    t = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
    for seed in range(4):
        tgt = workloads.synth_target_argmax(wl, t["node_token"], t["parent"], t["depth"],
                                            t["n_nodes"], seed=seed)
        a = oracle.tree_accept(t["node_token"], t["parent"], t["n_nodes"], tgt)
        for b in range(wl.B):
            n = int(t["n_nodes"][b])
            L, nodes, out, bonus = brute_force(t["node_token"][b], t["parent"][b], n, tgt[b])
            assert a["accept_len"][b] == L
            np.testing.assert_array_equal(a["accept_nodes"][b], nodes)
            np.testing.assert_array_equal(a["out_tokens"][b], out)
            assert a["next_root"][b] == bonus


def test_accept_lengths_follow_the_drawn_lengths():
    # the 32K workload draws accept lengths 1..16 through its target tokens
    wl = workloads.make_workload("b8_l32k_q65", with_kv=False)
    t = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
    seen = set()
    for seed in range(40):
        tgt = workloads.synth_target_argmax(wl, t["node_token"], t["parent"], t["depth"],
                                            t["n_nodes"], seed=seed)
        seen |= set(oracle.tree_accept(t["node_token"], t["parent"], t["n_nodes"],
                                       tgt)["accept_len"].tolist())
    assert seen == set(range(1, 17))


def test_random_trees_brute_force():
    rng = np.random.default_rng(0)
    for _ in range(300):
        Q = int(rng.integers(1, 40))
        n = int(rng.integers(1, Q + 1))
        par = [-1] + [int(rng.integers(0, i)) for i in range(1, Q)]
        # distinct tokens among siblings: token = 10 * parent + child ordinal
        tok, count = [0] * Q, {}
        for i in range(1, Q):
            count[par[i]] = count.get(par[i], 0) + 1
            tok[i] = 10 * par[i] + count[par[i]]
        tgt = [int(rng.integers(0, 10 * Q)) for _ in range(Q)]
        for i in range(1, n):           # make ~half the edges agree
            if rng.random() < 0.5:
                tgt[par[i]] = tok[i]
        a = accept1(tok, par, n, tgt)
        L, nodes, out, bonus = brute_force(tok, par, n, tgt)
        assert a["accept_len"] == L
        np.testing.assert_array_equal(a["accept_nodes"], nodes)
        np.testing.assert_array_equal(a["out_tokens"], out)
        assert a["next_root"] == bonus


def test_no_agreement_accepts_root_only():
    tok = [5, 6, 7, 8]
    par = [-1, 0, 0, 1]
    a = accept1(tok, par, 4, [99, 99, 99, 99])
    assert a["accept_len"] == 1
    assert a["accept_nodes"].tolist() == [0, -1, -1, -1]
    assert a["out_tokens"].tolist() == [99, -1, -1, -1]
    assert a["next_root"] == 99


def test_full_chain_agreement_accepts_everything():
    Q = 9
    tok = list(range(100, 100 + Q))
    par = list(range(-1, Q - 1))
    tgt = tok[1:] + [777]
    a = accept1(tok, par, Q, tgt)
    assert a["accept_len"] == Q
    assert a["accept_nodes"].tolist() == list(range(Q))
    assert a["out_tokens"].tolist() == tok[1:] + [777]
    assert a["next_root"] == 777


def test_duplicate_sibling_tokens_take_lowest_index():
    # root -> {1: tok 5, 2: tok 5}; node 2 has a child that would extend the path
    tok = [0, 5, 5, 9]
    par = [-1, 0, 0, 2]
    a = accept1(tok, par, 4, [5, 1, 9, 3])
    assert a["accept_nodes"].tolist()[:2] == [0, 1] and a["accept_len"] == 2
    assert a["out_tokens"].tolist() == [5, 1, -1, -1]


def test_nodes_beyond_n_nodes_are_ignored_and_clamped():
    tok = [0, 5, 6]
    par = [-1, 0, 1]
    tgt = [5, 6, 0]
    assert accept1(tok, par, 2, tgt)["accept_len"] == 2      # node 2 is padding
    assert accept1(tok, par, 3, tgt)["accept_len"] == 3
    assert accept1(tok, par, 99, tgt)["accept_len"] == 3     # n clamps to Q
    assert accept1(tok, par, 0, tgt)["accept_len"] == 1      # n clamps to 1
    # a link that does not point forward is ignored
    assert accept1([0, 5, 6], [-1, 2, 0], 3, [6, 0, 5])["accept_nodes"].tolist() == [0, 2, -1]
