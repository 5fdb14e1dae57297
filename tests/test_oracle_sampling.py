"""Pins for the oracle's sampling acceptance.

What it computes ("The Architecture of a Thousand-Parameter Decision ...",
"What to Build New", item 2: the sampling-probability path of tree verification;
"What to Reuse", item 3: target-only tree speculative sampling from the verified
distribution), with readings R16 (children tried in index order, accepted with
probability p(t) over the mass not yet rejected, the bonus token drawn by
inverse CDF from the residual) and R17 (temperature <= 0 or non-finite, and
nodes whose largest logit is not finite, are greedy).

Checked against things other than the oracle's own code:

* the defining property of speculative sampling: the tokens it emits are
  distributed exactly as sampling the target autoregressively.  A Monte Carlo
  over 200000 coin draws on a small tree (with a duplicate sibling token and an
  out-of-range token) must match softmax(logits / T) of the node reached, by a
  chi-square test, for the first, second and third token;
* greedy acceptance (itself pinned by brute force) against the argmax tokens,
  for every non-positive or non-finite temperature and for a tiny positive one;
* closed forms with equal logits, where every acceptance test and the bonus
  draw can be worked by hand (1/V, then 1/(V-1) after a rejection; the
  inverse CDF over the tokens left);
* invariance under scaling logits and temperature together (exact in binary
  floating point), masked entries never drawn, point-mass rows.
"""
import numpy as np
import pytest
import scipy.special
import scipy.stats

import oracle
from tree_verify_mla_ddt_amd import workloads


def run(logits, T, tok, par, n, coins, cfin, eps=0.0):
    return oracle.tree_accept_sampling(np.asarray(logits, np.float32), np.asarray(T, np.float32),
                                       np.asarray(tok, np.int32), np.asarray(par, np.int32),
                                       np.asarray(n, np.int32), np.asarray(coins, np.float32),
                                       np.asarray(cfin, np.float32), eps)


# A small tree over V = 6 tokens (the root's own token is not used):
#   0 -> 1 (tok 2), 2 (tok 0), 3 (tok 2, a duplicate sibling), 4 (tok 5)
#   1 -> 5 (tok 1), 6 (tok 3);  2 -> 7 (tok 99, outside the vocabulary)
V_SMALL = 6
TOK = np.array([4, 2, 0, 2, 5, 1, 3, 99], np.int32)
PAR = np.array([-1, 0, 0, 0, 0, 1, 1, 2], np.int32)
NODE_OF_ROOT_CHILD = {2: 1, 0: 2, 5: 4}  # first drafted child per token


def test_emitted_tokens_follow_the_target_distribution():
    rng = np.random.default_rng(123)
    N, Q, T = 200000, len(TOK), 0.8
    x = rng.normal(0, 1.5, size=(Q, V_SMALL)).astype(np.float32)
    p = scipy.special.softmax(x.astype(np.float64) / T, axis=-1)
    logits = np.broadcast_to(x, (N, Q, V_SMALL))
    o = run(logits, np.full(N, T), np.tile(TOK, (N, 1)), np.tile(PAR, (N, 1)), np.full(N, Q),
            rng.random((N, Q), dtype=np.float32), rng.random(N, dtype=np.float32))
    t1 = o["out_tokens"][:, 0]

    def chi2_ok(samples, probs):
        counts = np.bincount(samples, minlength=V_SMALL)
        return scipy.stats.chisquare(counts, probs * len(samples)).pvalue > 1e-4

    assert chi2_ok(t1, p[0])
    # A drafted first token moves the walk to that child: the next token is
    # distributed as the target at that node; any other first token is the
    # bonus and ends the step.
    drafted = np.isin(t1, list(NODE_OF_ROOT_CHILD))
    np.testing.assert_array_equal(o["accept_len"] == 1, ~drafted)
    for t, node in NODE_OF_ROOT_CHILD.items():
        sel = t1 == t
        assert (o["accept_nodes"][sel, 1] == node).all()
        assert chi2_ok(o["out_tokens"][sel, 1], p[node])
    # Third token after 0 -> 1 -> 5 (token 2 then token 1): the target at node 5.
    sel = (t1 == 2) & (o["out_tokens"][:, 1] == 1)
    assert (o["accept_nodes"][sel, 2] == 5).all()
    assert chi2_ok(o["out_tokens"][sel, 2], p[5])
    # The duplicate sibling (node 3) and the out-of-range token (node 7) are never taken.
    assert not np.isin(o["accept_nodes"], [3, 7]).any()


def greedy_reference(logits, tok, par, n):
    x = np.where(np.isnan(logits), -np.inf, logits)
    return oracle.tree_accept(tok, par, n, np.argmax(x, axis=-1).astype(np.int32))


def workload_tree(name, vocab, seed=0):
    wl = workloads.make_workload(name, with_kv=False, seed=seed)
    ids = (wl.topk_ids % vocab).astype(np.int32)
    # Distinct ids per depth after the reduction, so siblings stay distinct.
    for b in range(wl.B):
        for d in range(wl.D):
            ids[b, d] = np.random.default_rng((seed, b, d)).choice(vocab, wl.K, replace=False)
    t = oracle.tree_build(wl.topk_logp, ids, wl.root_token, wl.prefix_len, wl.budget)
    return t


@pytest.mark.parametrize("name", ["b4_l4k_q17", "b64_l2k_q9", "b8_l32k_q65"])
def test_greedy_temperatures_equal_greedy_accept(name):
    V = 300
    t = workload_tree(name, V)
    B = t["node_token"].shape[0]
    x, _, coins, cfin = workloads.sampling_inputs(t["node_token"], t["parent"], t["n_nodes"], V,
                                                  seed=3, dtype=__import__("torch").float32)
    x = x.numpy()
    for T in (0.0, -1.0, np.inf, np.nan):
        o = run(x, np.full(B, T), t["node_token"], t["parent"], t["n_nodes"], coins, cfin)
        g = greedy_reference(x, t["node_token"], t["parent"], t["n_nodes"])
        for k in g:
            np.testing.assert_array_equal(o[k], g[k], err_msg=f"{k} T={T}")


def test_tiny_temperature_equals_greedy():
    V = 300
    t = workload_tree("b4_l4k_q33", V, seed=1)
    B = t["node_token"].shape[0]
    x, _, _, _ = workloads.sampling_inputs(t["node_token"], t["parent"], t["n_nodes"], V, seed=4,
                                           dtype=__import__("torch").float32)
    x = x.numpy()
    srt = np.sort(x, axis=-1)
    gap = float((srt[..., -1] - srt[..., -2]).min())
    assert gap > 0
    rng = np.random.default_rng(5)
    coins = rng.uniform(0.01, 0.99, size=(B, x.shape[1])).astype(np.float32)
    cfin = rng.uniform(0.01, 0.99, size=B).astype(np.float32)
    # exp(-gap / T) = exp(-200): every non-argmax probability is negligible.
    o = run(x, np.full(B, gap / 200), t["node_token"], t["parent"], t["n_nodes"], coins, cfin)
    g = greedy_reference(x, t["node_token"], t["parent"], t["n_nodes"])
    for k in g:
        np.testing.assert_array_equal(o[k], g[k], err_msg=k)


def test_equal_logits_worked_by_hand():
    """V = 10 equal logits, root children with tokens 3, 4, 5 (nodes 1, 2, 3).
    Node 1 is accepted with probability 1/10, node 2 after rejecting token 3 with
    1/9, node 3 after two rejections with 1/8; the bonus is uniform over the
    7 tokens left."""
    V, Q = 10, 4
    tok = np.array([0, 3, 4, 5], np.int32)
    par = np.array([-1, 0, 0, 0], np.int32)
    x = np.zeros((1, Q, V), np.float32)

    def go(c1, c2, c3, cf, T=1.0):
        o = run(x, [T], tok[None], par[None], [Q], [[0.5, c1, c2, c3]], [cf])
        return int(o["accept_len"][0]), int(o["out_tokens"][0, 0]), int(o["next_root"][0])

    assert go(0.099, 0.9, 0.9, 0.5)[:2] == (2, 3)      # 0.099 < 1/10
    assert go(0.101, 0.110, 0.9, 0.5)[:2] == (2, 4)    # rejected, then 0.110 < 1/9
    assert go(0.101, 0.112, 0.124, 0.5)[:2] == (2, 5)  # 0.124 < 1/8
    assert go(0.101, 0.112, 0.126, 0.5)[0] == 1        # all three rejected
    # Bonus over tokens {0, 1, 2, 6, 7, 8, 9}, each 1/7, first CDF value above u.
    for u, want in [(0.0, 0), (0.14, 0), (0.15, 1), (0.43, 6), (0.71, 7), (0.999, 9)]:
        assert go(0.5, 0.5, 0.5, u) == (1, want, want), u
    # A draw at or above 1 takes the last token left (R16).
    assert go(0.5, 0.5, 0.5, 1.0)[1] == 9
    # Any temperature gives the same answers on equal logits.
    assert go(0.101, 0.110, 0.9, 0.5, T=3.0)[:2] == (2, 4)


def test_scaling_logits_and_temperature_together():
    rng = np.random.default_rng(8)
    B, Q, V = 64, len(TOK), V_SMALL
    x = rng.normal(0, 2, size=(B, Q, V)).astype(np.float32)
    T = rng.uniform(0.3, 2.0, size=B).astype(np.float32)
    coins, cfin = rng.random((B, Q), dtype=np.float32), rng.random(B, dtype=np.float32)
    args = (np.tile(TOK, (B, 1)), np.tile(PAR, (B, 1)), np.full(B, Q), coins, cfin)
    a = run(x, T, *args, eps=1e-6)
    b = run(x * np.float32(2), T * np.float32(2), *args, eps=1e-6)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_masked_entries_point_masses_and_nonfinite_rows():
    V, Q = 8, 3
    tok = np.array([[0, 5, 6]], np.int32)
    par = np.array([[-1, 0, 0]], np.int32)
    x = np.full((1, Q, V), -np.inf, np.float32)
    # Root: only tokens 1 and 6 are finite; token 5 (node 1) is masked and
    # never accepted, token 6 (node 2) competes with token 1.
    x[0, 0, 1], x[0, 0, 6] = 0.0, 0.0
    x[0, 0, 4] = np.nan
    for c2 in (0.49, 0.51):
        o = run(x, [1.0], tok, par, [Q], [[0.5, 0.0, c2]], [0.3])
        if c2 < 0.5:
            assert o["accept_nodes"][0, 1] == 2
        else:  # bonus from the residual: token 1 alone
            assert o["accept_len"][0] == 1 and o["next_root"][0] == 1
    # A point mass: the child holding it is accepted whatever its coin (< 1).
    y = np.full((1, Q, V), -np.inf, np.float32)
    y[0, :, 6] = 2.0
    o = run(y, [0.9], tok, par, [Q], [[0.0, 0.0, 0.9999]], [0.5])
    assert list(o["accept_nodes"][0, :2]) == [0, 2]
    # An all -inf node and a node with a +inf entry are taken greedily: the
    # lowest index among the largest logits.
    z = np.random.default_rng(2).normal(size=(1, Q, V)).astype(np.float32)
    z[0, 0] = -np.inf
    o = run(z, [1.0], tok, par, [Q], [[0.5, 0.0, 0.0]], [0.5])
    assert o["accept_len"][0] == 1 and o["next_root"][0] == 0
    z[0, 0] = 0.0
    z[0, 0, 3] = np.inf
    z[0, 0, 7] = np.inf
    o = run(z, [1.0], tok, par, [Q], [[0.5, 0.0, 0.0]], [0.99])
    assert o["accept_len"][0] == 1 and o["next_root"][0] == 3


def test_band_and_margin_diagnostics():
    V = 300
    t = workload_tree("b4_l4k_q17", V, seed=2)
    B = t["node_token"].shape[0]
    x, T, coins, cfin = workloads.sampling_inputs(t["node_token"], t["parent"], t["n_nodes"], V,
                                                  seed=6, dtype=__import__("torch").float32)
    o = run(x.numpy(), T, t["node_token"], t["parent"], t["n_nodes"], coins, cfin, eps=1e-3)
    assert ((o["bonus_lo"] <= o["next_root"]) & (o["next_root"] <= o["bonus_hi"])).all()
    assert (o["margin"] > 0).all()
    o0 = run(x.numpy(), T, t["node_token"], t["parent"], t["n_nodes"], coins, cfin, eps=0.0)
    np.testing.assert_array_equal(o0["bonus_lo"], o0["next_root"])
    np.testing.assert_array_equal(o0["bonus_hi"], o0["next_root"])


def _numpy_band(x, T, rejected, coin_final, eps):
    """The bonus band written out with NumPy: the residual distribution
    (softmax(x / T) in float64 without the rejected tokens), its CDF by
    cumulative sum, and every entry with mass whose CDF interval
    [cdf - p, cdf] comes within eps * Zr of the draw coin_final * Zr."""
    p = scipy.special.softmax(x.astype(np.float64) / T)
    keep = np.ones_like(p, dtype=bool)
    keep[list(rejected)] = False
    keep &= p > 0
    r = np.where(keep, p, 0.0)
    Zr = r.sum()
    target = float(coin_final) * Zr
    hi = np.cumsum(r)
    lo = hi - r
    inband = keep & (hi >= target - eps * Zr) & (lo <= target + eps * Zr)
    drawn = int(np.flatnonzero(keep & (hi > target))[0])
    idx = np.flatnonzero(inband)
    return drawn, int(idx.min()), int(idx.max())


@pytest.mark.parametrize("eps", [1e-5, 1e-3, 3e-2])
def test_bonus_band_width_against_numpy_cdf(eps):
    """The band the oracle reports at eps > 0 (the set of bonus tokens a
    sampler within eps of the draw may return) equals the band computed
    independently from a NumPy cumulative sum, on a root-only tree (residual =
    target) and on a root whose two children are both rejected (residual
    without their tokens)."""
    rng = np.random.default_rng(17)
    V = 4000
    for case in range(40):
        T = float(rng.choice([0.5, 1.0, 1.7]))
        x = (rng.normal(0, 2, size=V)).astype(np.float32)
        cf = np.float32(rng.random())
        if case % 2 == 0:
            tok = np.array([[0, -1, -1]], np.int32)
            par = np.array([[-1, -1, -1]], np.int32)
            nn, rejected = 1, set()
            coins = np.zeros((1, 3), np.float32)
        else:
            t1, t2 = (int(v) for v in rng.choice(V, size=2, replace=False))
            tok = np.array([[0, t1, t2]], np.int32)
            par = np.array([[-1, 0, 0]], np.int32)
            nn, rejected = 3, {t1, t2}
            coins = np.array([[0.0, 0.999999, 0.999999]], np.float32)
            x[t1] = x[t2] = -3.0  # small enough that both are rejected
        z = np.zeros((1, 3, V), np.float32)
        z[0, 0] = x
        o = run(z, [T], tok, par, [nn], coins, [cf], eps=eps)
        assert o["accept_len"][0] == 1
        drawn, lo, hi = _numpy_band(x, T, rejected, cf, eps)
        assert o["next_root"][0] == drawn
        assert (o["bonus_lo"][0], o["bonus_hi"][0]) == (lo, hi), (case, eps)
