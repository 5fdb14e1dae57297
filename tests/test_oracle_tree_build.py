"""Pins for the oracle's best-first tree builder.

What the builder computes is fixed by the best-first top-k expansion of "The
Architecture of a Thousand-Parameter Decision: Designing a Native DDTree
Inference Engine for Kimi K2.6" ("What to Build New", item 3) with the readings
R1 (cumulative fp32 log-prob, ties by parent index then rank) and R2 (-inf never
offered).  These tests check the heap-based oracle against things other than
itself:

* a hand-worked example;
* brute force: when every depth's log-probs are <= 0 and sorted, fp32 addition
  is monotone along child and next-sibling edges, so best-first pops exactly
  the first budget paths of one total order over all finite rank paths (score
  descending, then the parent's place in that same order, then rank).  The test
  enumerates every path and sorts by that nested key -- a global sort instead of
  a heap;
* closed forms: K=1 chains, equal log-probs give level order, a budget that
  covers every path gives the complete tree, a dominant top-1 gives a chain;
* structural invariants.
"""
import itertools
import math

import numpy as np
import pytest

import oracle

F32 = np.float32


def build1(logp, ids, budget, root=7, L=100):
    """Oracle on a single request; returns per-request arrays."""
    t = oracle.tree_build(logp[None], ids[None], np.array([root], np.int32),
                          np.array([L], np.int32), budget)
    return {k: v[0] for k, v in t.items()}


def brute_force(logp, ids, budget, root=7, L=100):
    """Independent construction: enumerate all finite rank paths, sort by the
    nested key, keep the first `budget`."""
    D, K = logp.shape
    score = {(): F32(0.0)}
    level = [()]
    for d in range(1, D + 1):
        nxt = []
        for p in level:
            for r in range(K):
                s = F32(score[p] + logp[d - 1, r])
                if not s > -np.inf:
                    continue
                score[p + (r,)] = s
                nxt.append(p + (r,))
        level = nxt
    key = {(): (-math.inf,)}

    def k(path):
        if path not in key:
            key[path] = (-float(score[path]), k(path[:-1]), path[-1])
        return key[path]

    order = [()] + sorted((p for p in score if p), key=k)[:budget]
    index = {p: i for i, p in enumerate(order)}
    Q = budget + 1
    W = (Q + 63) // 64
    n = len(order)
    exp = {name: np.full(Q, -1, np.int32) for name in
           ("node_token", "parent", "depth", "position", "first_child", "next_sibling")}
    exp["score"] = np.full(Q, -np.inf, np.float32)
    exp["vis"] = np.zeros((Q, W), np.uint64)
    exp["n_nodes"] = np.int32(n)
    for i, p in enumerate(order):
        exp["node_token"][i] = root if not p else ids[len(p) - 1, p[-1]]
        exp["parent"][i] = -1 if not p else index[p[:-1]]
        exp["depth"][i] = len(p)
        exp["position"][i] = L + len(p)
        exp["score"][i] = score[p]
        kids = [index[c] for c in order if len(c) == len(p) + 1 and c[:-1] == p]
        exp["first_child"][i] = min(kids) if kids else -1
        if p:
            sibs = [index[c] for c in order
                    if len(c) == len(p) and c[:-1] == p[:-1] and index[c] > i]
            exp["next_sibling"][i] = min(sibs) if sibs else -1
        for a in range(len(p) + 1):  # every prefix of the path, itself included
            j = index[p[:a]]
            exp["vis"][i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return exp


def assert_tree_equal(got, exp):
    for name, e in exp.items():
        g = got[name]
        if name == "score":
            np.testing.assert_array_equal(g.view(np.uint32), np.asarray(e, np.float32).view(np.uint32),
                                          err_msg=name)
        else:
            np.testing.assert_array_equal(g, e, err_msg=name)


def test_hand_worked_example():
    # D=2, K=2.  Depth-1 log-probs (-0.1, -2.5), depth-2 (-0.5, -1.0).
    # Pops: a(-0.1) -> a's child aa(-0.6) -> aa's sibling ab(-1.1) -> b(-2.5)
    # -> ba(-3.0) -> bb(-3.5).  Tokens: depth1 (10, 11), depth2 (20, 21).
    logp = np.array([[-0.1, -2.5], [-0.5, -1.0]], np.float32)
    ids = np.array([[10, 11], [20, 21]], np.int32)
    t = build1(logp, ids, budget=6, root=7, L=100)
    assert t["n_nodes"] == 7
    assert t["node_token"].tolist() == [7, 10, 20, 21, 11, 20, 21]
    assert t["parent"].tolist() == [-1, 0, 1, 1, 0, 4, 4]
    assert t["depth"].tolist() == [0, 1, 2, 2, 1, 2, 2]
    assert t["position"].tolist() == [100, 101, 102, 102, 101, 102, 102]
    assert t["first_child"].tolist() == [1, 2, -1, -1, 5, -1, -1]
    assert t["next_sibling"].tolist() == [-1, 4, 3, -1, -1, 6, -1]
    f = np.float32
    assert t["score"].tolist() == [0.0, f(-0.1), f(f(-0.1) + f(-0.5)), f(f(-0.1) + f(-1.0)),
                                   f(-2.5), f(f(-2.5) + f(-0.5)), f(f(-2.5) + f(-1.0))]
    # ancestors + self: 0:{0} 1:{0,1} 2:{0,1,2} 3:{0,1,3} 4:{0,4} 5:{0,4,5} 6:{0,4,6}
    assert t["vis"][:, 0].tolist() == [1, 3, 7, 11, 17, 49, 81]
    # budget 3 keeps the first three pops only
    t3 = build1(logp, ids, budget=3)
    assert t3["node_token"].tolist() == [7, 10, 20, 21]
    assert t3["n_nodes"] == 4


@pytest.mark.parametrize("seed", range(60))
def test_brute_force_matches_heap(seed):
    rng = np.random.default_rng(1000 + seed)
    D = int(rng.integers(1, 5))
    K = int(rng.integers(1, 5))
    if seed % 3 == 0:   # a small value set -> many exact ties
        vals = np.array([0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -np.inf], np.float32)
        logp = rng.choice(vals, size=(D, K), p=[.15, .2, .2, .15, .1, .1, .1])
    elif seed % 3 == 1:
        logp = np.log(rng.dirichlet(np.ones(K), size=D)).astype(np.float32)
    else:               # random log-softmax of N(0,2) logits
        x = rng.normal(0, 2, size=(D, K))
        logp = (x - x.max(1, keepdims=True)
                - np.log(np.exp(x - x.max(1, keepdims=True)).sum(1, keepdims=True))).astype(np.float32)
    logp = -np.sort(-logp, axis=1)
    ids = rng.integers(0, 1000, size=(D, K)).astype(np.int32)
    total = sum(K ** d for d in range(1, D + 1))
    budget = int(rng.integers(0, min(total + 3, 127) + 1))
    assert_tree_equal(build1(logp, ids, budget), brute_force(logp, ids, budget))


def test_brute_force_two_visibility_words():
    # Q > 64 exercises the second 64-bit word of every visibility row.
    rng = np.random.default_rng(5)
    D, K = 4, 4
    logp = -np.sort(-np.log(rng.dirichlet(np.ones(K), size=D)), axis=1).astype(np.float32)
    ids = rng.integers(0, 1000, size=(D, K)).astype(np.int32)
    for budget in (63, 64, 100, 127):
        assert_tree_equal(build1(logp, ids, budget), brute_force(logp, ids, budget))


@pytest.mark.parametrize("D,budget", [(1, 0), (1, 5), (5, 3), (8, 8), (15, 64)])
def test_k1_is_a_chain(D, budget):
    logp = np.full((D, 1), -0.25, np.float32)
    ids = np.arange(D, dtype=np.int32)[:, None] + 40
    t = build1(logp, ids, budget)
    n = 1 + min(D, budget)
    assert t["n_nodes"] == n
    assert t["parent"][:n].tolist() == list(range(-1, n - 1))
    assert t["depth"][:n].tolist() == list(range(n))
    assert t["node_token"][1:n].tolist() == list(range(40, 40 + n - 1))
    assert (t["node_token"][n:] == -1).all() and (t["vis"][n:] == 0).all()


def test_equal_logprobs_give_level_order():
    # Every log-prob is -1 (exact in fp32): scores tie within a level, and the
    # key falls back to parent index then rank -> breadth-first order.
    D, K = 3, 3
    logp = np.full((D, K), -1.0, np.float32)
    ids = np.arange(D * K, dtype=np.int32).reshape(D, K)
    t = build1(logp, ids, budget=3 + 9 + 5)
    exp_parent = [-1] + [0] * 3 + [1] * 3 + [2] * 3 + [3] * 3 + [4] * 3 + [5, 5]
    exp_rank = [None] + [0, 1, 2] * 5 + [0, 1]
    assert t["parent"].tolist() == exp_parent
    assert t["depth"].tolist() == [0] + [1] * 3 + [2] * 9 + [3] * 5
    for i in range(1, len(exp_parent)):
        assert t["node_token"][i] == ids[t["depth"][i] - 1, exp_rank[i]]
    # all-zero log-probs (score 0 everywhere) give the same shape
    t0 = build1(np.zeros((D, K), np.float32), ids, budget=3 + 9 + 5)
    assert t0["parent"].tolist() == exp_parent


@pytest.mark.parametrize("D,K", [(1, 4), (2, 3), (3, 2), (4, 2)])
def test_budget_covering_all_paths_gives_complete_tree(D, K):
    rng = np.random.default_rng(D * 10 + K)
    logp = -np.sort(-np.log(rng.dirichlet(np.ones(K), size=D)), axis=1).astype(np.float32)
    ids = rng.integers(0, 99, size=(D, K)).astype(np.int32)
    total = sum(K ** d for d in range(1, D + 1))
    t = build1(logp, ids, budget=total + 10)
    assert t["n_nodes"] == 1 + total
    for d in range(D + 1):
        assert (t["depth"][: 1 + total] == d).sum() == K ** d


def test_dominant_top1_gives_chain():
    # top-1 prob 0.995 at every depth and D >= budget: the whole budget goes to
    # the top-1 spine (log 0.995 * budget > log of any runner-up).
    K, D, budget = 8, 8, 8
    rest = np.full(K - 1, 0.005 / (K - 1))
    logp = np.tile(np.log(np.concatenate([[0.995], rest])), (D, 1)).astype(np.float32)
    ids = np.arange(D * K, dtype=np.int32).reshape(D, K)
    t = build1(logp, ids, budget)
    assert t["n_nodes"] == budget + 1
    assert t["parent"].tolist() == list(range(-1, budget))
    assert t["node_token"][1:].tolist() == [ids[d, 0] for d in range(budget)]


def test_minus_inf_makes_underfull_trees():
    D, K = 4, 3
    logp = np.full((D, K), -np.inf, np.float32)
    logp[:, 0] = -0.5
    t = build1(logp, np.zeros((D, K), np.int32), budget=10)
    assert t["n_nodes"] == 1 + D          # only the rank-0 chain is finite
    assert np.isneginf(t["score"][1 + D:]).all()
    t = build1(np.full((D, K), -np.inf, np.float32), np.zeros((D, K), np.int32), budget=10)
    assert t["n_nodes"] == 1 and t["parent"][0] == -1 and t["vis"][0, 0] == 1
    # NaN behaves like -inf (never offered)
    logp = np.full((D, K), np.nan, np.float32)
    logp[0, 0] = -1.0
    assert build1(logp, np.zeros((D, K), np.int32), budget=10)["n_nodes"] == 2


def test_degenerate_shapes():
    for D, K in ((0, 4), (4, 0), (0, 0)):
        t = build1(np.zeros((D, K), np.float32), np.zeros((D, K), np.int32), budget=5)
        assert t["n_nodes"] == 1 and t["node_token"][0] == 7 and (t["parent"][1:] == -1).all()


@pytest.mark.parametrize("name", ["tiny_fp32", "b1_l2k_q9", "b4_l4k_q33", "b64_l2k_q9",
                                  "b8_l32k_q65"])
def test_structural_invariants_on_workloads(name):
    from tree_verify_mla_ddt_amd import workloads
    wl = workloads.make_workload(name, with_kv=False)
    t = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
    for b in range(wl.B):
        n = int(t["n_nodes"][b])
        par, sc, dep = t["parent"][b], t["score"][b], t["depth"][b]
        assert np.all(np.diff(sc[:n]) <= 0)                       # best-first order
        assert all(par[i] < i for i in range(1, n))               # parents come first
        assert all(dep[i] == dep[par[i]] + 1 for i in range(1, n))
        assert (t["position"][b, :n] == wl.prefix_len[b] + dep[:n]).all()
        # closed under parent and under elder sibling: the rank-r child of p is
        # present only if the rank-(r-1) child is, with a lower index
        for i in range(1, n):
            d = dep[i]
            r = int(np.flatnonzero(wl.topk_ids[b, d - 1] == t["node_token"][b, i])[0])
            if r > 0:
                elder = [j for j in range(1, n) if par[j] == par[i]
                         and t["node_token"][b, j] == wl.topk_ids[b, d - 1, r - 1]]
                assert len(elder) == 1 and elder[0] < i
    # every b%4==3 request of the chain-heavy workload is a chain
    if name == "b64_l2k_q9":
        for b in range(3, wl.B, 4):
            assert t["parent"][b].tolist() == list(range(-1, wl.budget))


def test_exhaustive_tiny_space():
    # every sorted assignment from {0,-1,-2} for D=2, K=2, every budget
    vals = [0.0, -1.0, -2.0]
    ids = np.array([[1, 2], [3, 4]], np.int32)
    for a in itertools.product(vals, repeat=4):
        logp = -np.sort(-np.array(a, np.float32).reshape(2, 2), axis=1)
        for budget in range(0, 8):
            assert_tree_equal(build1(logp, ids, budget), brute_force(logp, ids, budget))
