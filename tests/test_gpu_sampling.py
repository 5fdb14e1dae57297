"""GPU parity of ddt_tree_accept_sampling (through its C ABI) against the CPU oracle.

The oracle decides in float64 and the kernel in fp32, so a decision whose coin
lies within rounding distance of its threshold may legitimately differ.  The
bar, per request:
* greedy requests (temperature 0, negative, inf, NaN) and greedy nodes: every
  output bit-exact;
* sampled requests whose smallest acceptance margin |coin - p_res| in the
  oracle exceeds ACC_EPS: accept_len, accept_nodes and the accepted draft
  tokens bit-exact, and the bonus token inside the oracle's band of entries
  whose residual-CDF interval comes within BAND_EPS (relative to the residual
  mass) of the draw -- fp32 sums over up to 160000 entries stay well inside
  it.  A request within ACC_EPS of a threshold (a handful at most) must equal
  the oracle run with that request's coins moved down or up by NUDGE.
Outputs are pre-filled with sentinels, so every element must be written.
Also: the emitted tokens' distribution on the GPU against softmax(logits / T)
(chi-square over 32768 draws), and replays of a captured HIP graph.
"""
import sys

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import oracle
import tree_verify_mla_ddt_amd as ddt
from tree_verify_mla_ddt_amd import workloads

pytestmark = pytest.mark.gpu
ACC_EPS = 2e-5
NUDGE = 3e-5  # > ACC_EPS: moves a near-threshold coin clear of its threshold
BAND_EPS = 1e-5
KEYS = ("accept_len", "accept_nodes", "out_tokens", "next_root")


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ddt.load_library()
    yield


def dev(a, dtype=None):
    t = torch.as_tensor(np.ascontiguousarray(a)) if not isinstance(a, torch.Tensor) else a
    if dtype is not None:
        t = t.to(dtype)
    return t.contiguous().cuda()


def gpu_sampling(logits, T, tok, par, nn, coins, cfin):
    B, Q, _ = logits.shape
    out = {"accept_len": torch.full((B,), -77, dtype=torch.int32, device="cuda"),
           "accept_nodes": torch.full((B, Q), -77, dtype=torch.int32, device="cuda"),
           "out_tokens": torch.full((B, Q), -77, dtype=torch.int32, device="cuda"),
           "next_root": torch.full((B,), -77, dtype=torch.int32, device="cuda")}
    ddt.tree_accept_sampling(dev(logits), dev(T, torch.float32), dev(tok, torch.int32),
                             dev(par, torch.int32), dev(nn, torch.int32),
                             dev(coins, torch.float32), dev(cfin, torch.float32), out=out)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def matches(g, o, b, ob=None):
    """The GPU result of request b is the oracle's decision path (request ob of
    o) with a bonus token inside the oracle's band."""
    ob = b if ob is None else ob
    n = int(o["accept_len"][ob])
    if g["accept_len"][b] != n or not np.array_equal(g["accept_nodes"][b], o["accept_nodes"][ob]):
        return False
    if not np.array_equal(g["out_tokens"][b, :n - 1], o["out_tokens"][ob, :n - 1]):
        return False
    bonus = int(g["next_root"][b])
    return bool((g["out_tokens"][b, n:] == -1).all() and g["out_tokens"][b, n - 1] == bonus and
                o["bonus_lo"][ob] <= bonus <= o["bonus_hi"][ob])


def compare(g, o, T, max_skipped, inputs=None):
    """inputs = (logits, T, tok, par, nn, coins, cfin): a request whose smallest
    margin is within ACC_EPS must equal the oracle run with that request's
    coins moved down or up by NUDGE, i.e. one of the two outcomes a sampler
    within rounding distance of the threshold may produce."""
    B = len(o["accept_len"])
    greedy = ~((T > 0) & np.isfinite(T))
    near = 0
    for b in range(B):
        if greedy[b]:
            for k in KEYS:
                np.testing.assert_array_equal(g[k][b], o[k][b], err_msg=f"{k} greedy b={b}")
            continue
        if not o["margin"][b] > ACC_EPS:
            near += 1
            assert inputs is not None, f"b={b}: within {ACC_EPS} of a threshold"
            x, Tn, tok, par, nn, coins, cfin = inputs
            sl = slice(b, b + 1)
            xb = x[sl].float().numpy() if isinstance(x, torch.Tensor) else x[sl]
            ok = False
            for d in (-NUDGE, NUDGE):
                cb = np.clip(coins[sl].astype(np.float64) + d, 0.0, 0.99999994).astype(np.float32)
                ob = oracle.tree_accept_sampling(xb, Tn[sl], tok[sl], par[sl], nn[sl], cb,
                                                 cfin[sl], BAND_EPS)
                ok = ok or matches(g, ob, b, 0)
            assert ok, f"b={b}: matches neither nudged outcome"
            continue
        assert matches(g, o, b), (b, g["accept_len"][b], o["accept_len"][b], g["next_root"][b],
                                  o["bonus_lo"][b], o["bonus_hi"][b])
    assert near <= max_skipped, f"{near} requests within {ACC_EPS} of a threshold"
    return near


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_workload_trees(name):
    """The workloads' drafted trees (oracle builder) with target logits over the
    full vocabulary (bf16; f32 for the tiny case), temperatures 0/0.7/1/1.5."""
    note(f"tree_accept_sampling {name}")
    wl = workloads.make_workload(name, with_kv=False)
    t = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
    dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    x, T, coins, cfin = workloads.sampling_inputs(t["node_token"], t["parent"], t["n_nodes"],
                                                  wl.vocab, seed=1, dtype=dt)
    g = gpu_sampling(x, T, t["node_token"], t["parent"], t["n_nodes"], coins, cfin)
    o = oracle.tree_accept_sampling(x, T, t["node_token"], t["parent"], t["n_nodes"], coins, cfin,
                                    BAND_EPS)
    compare(g, o, T, max_skipped=wl.B // 16 + 1,
            inputs=(x, T, t["node_token"], t["parent"], t["n_nodes"], coins, cfin))


@pytest.mark.parametrize("V,dtype,B", [(37, torch.float32, 24), (1000, torch.bfloat16, 24),
                                       (70001, torch.float32, 24),
                                       (300000, torch.bfloat16, 20)])
def test_adversarial_values(V, dtype, B):
    """Random trees with duplicate and out-of-range tokens, bad parents, clamped
    n_nodes, -inf/NaN/+inf logits, edge temperatures and coins.  With V = 300000 a
    row spans more than 16 chunks and a request's nodes more than one staging
    batch of chunk records (the per-wavefront combine); the other shapes take the
    per-thread combine."""
    note(f"tree_accept_sampling adversarial V={V} {dtype} B={B}")
    rng = np.random.default_rng(V)
    Q = 33
    tok = rng.integers(-2, V + 2, size=(B, Q)).astype(np.int32)
    par = np.zeros((B, Q), np.int32)
    for b in range(B):
        for c in range(1, Q):
            par[b, c] = rng.integers(0, c) if rng.random() < 0.9 else rng.integers(-2, Q + 2)
        kids = [c for c in range(1, Q) if par[b, c] == 0]
        if len(kids) >= 2:
            tok[b, kids[1]] = tok[b, kids[0]]  # a duplicate sibling token
    nn = rng.integers(-1, Q + 3, size=B).astype(np.int32)
    x = torch.tensor(rng.normal(0, 2, size=(B, Q, V)), dtype=torch.float32)
    for b in range(B):  # push mass onto some children so walks go deep
        for c in range(1, Q):
            p, tk = int(par[b, c]), int(tok[b, c])
            if 0 <= p < c and 0 <= tk < V and rng.random() < 0.5:
                x[b, p, tk] = 12.0
    x[0, 0, : V // 2] = float("-inf")
    x[1, 0] = float("-inf")                    # an all -inf row: greedy, argmax 0
    x[2, 0, 5] = float("inf")                  # a +inf entry: greedy
    x[3, 0, ::3] = float("nan")
    x[4, :, :] = 1.5                           # equal logits
    x = x.to(dtype)
    T = np.array(([0.0, 1.0, 1.0, 1.0, 1.0, -1.0, np.inf, np.nan, 1e-30, 1e30, 0.5, 2.0] * 2)[:B],
                 np.float32)
    coins = rng.random((B, Q), dtype=np.float32)
    coins[12] = 0.0
    coins[13] = np.float32(0.99999994)
    coins[14, 1::2] = np.nan
    cfin = rng.random(B, dtype=np.float32)
    cfin[15], cfin[16], cfin[17], cfin[18] = 0.0, 1.0, np.nan, np.float32(0.99999994)
    g = gpu_sampling(x, T, tok, par, nn, coins, cfin)
    o = oracle.tree_accept_sampling(x, T, tok, par, nn, coins, cfin, BAND_EPS)
    compare(g, o, T, max_skipped=2, inputs=(x, T, tok, par, nn, coins, cfin))


def test_gpu_draws_follow_the_target_distribution():
    """32768 requests on one small tree: the first emitted token is distributed
    as softmax(logits[root] / T), the second (after the drafted token 2) as
    the target at node 1."""
    rng = np.random.default_rng(321)
    V, T = 6, 0.8
    tok = np.array([4, 2, 0, 2, 5, 1, 3, 99], np.int32)
    par = np.array([-1, 0, 0, 0, 0, 1, 1, 2], np.int32)
    N, Q = 32768, len(tok)
    x = rng.normal(0, 1.5, size=(Q, V)).astype(np.float32)
    p = scipy.special.softmax(x.astype(np.float64) / T, axis=-1)
    logits = torch.from_numpy(np.ascontiguousarray(np.broadcast_to(x, (N, Q, V))))
    g = gpu_sampling(logits, np.full(N, T, np.float32), np.tile(tok, (N, 1)), np.tile(par, (N, 1)),
                     np.full(N, Q, np.int32), rng.random((N, Q), dtype=np.float32),
                     rng.random(N, dtype=np.float32))
    t1 = g["out_tokens"][:, 0]
    cnt = np.bincount(t1, minlength=V)
    assert scipy.stats.chisquare(cnt, p[0] * N).pvalue > 1e-4
    sel = t1 == 2
    assert (g["accept_nodes"][sel, 1] == 1).all()
    cnt2 = np.bincount(g["out_tokens"][sel, 1], minlength=V)
    assert scipy.stats.chisquare(cnt2, p[1] * sel.sum()).pvalue > 1e-4
    assert not np.isin(g["accept_nodes"], [3, 7]).any()


def test_graph_replays_match_eager():
    wl = workloads.make_workload("b4_l4k_q33", with_kv=False)
    t = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
    x, T, coins, cfin = workloads.sampling_inputs(t["node_token"], t["parent"], t["n_nodes"],
                                                  wl.vocab, seed=2)
    args = [dev(x), dev(T, torch.float32), dev(t["node_token"], torch.int32),
            dev(t["parent"], torch.int32), dev(t["n_nodes"], torch.int32),
            dev(coins, torch.float32), dev(cfin, torch.float32)]
    eager = ddt.tree_accept_sampling(*args)
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in eager.items()}
    B, Q = t["node_token"].shape
    out = {k: torch.full_like(v, -77) for k, v in eager.items()}
    ws = torch.empty((int(ddt.load_library().ddt_tree_accept_sampling_workspace_size(
        B, Q, wl.vocab)),), dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ddt.tree_accept_sampling(*args, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ddt.tree_accept_sampling(*args, out=out, workspace=ws)
    for _ in range(3):
        for v in out.values():
            v.fill_(-77)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in eager:
            torch.testing.assert_close(out[k], eager[k], rtol=0, atol=0)
