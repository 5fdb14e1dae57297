"""GPU parity: the HIP library (called through its C ABI) against the CPU oracle.

* tree build and accept: bit-exact on every output array, padding included
  (scores compared as bit patterns);
* verify attention: max |GPU - oracle| <= 2e-3 for bf16 inputs and <= 1e-5 for
  fp32 inputs (the tolerances of the build's brief), lse within the same bound;
  every output element is written (outputs are pre-filled with NaN);
* composition: build -> attention -> accept chained on one stream without a
  host round-trip equals the oracle chain.

Workloads are the seeded generators of tree_verify_mla_ddt_amd.workloads, at the
benchmark's full sizes (every row; at the max shape every row of the request
whose row tiles take the most merged ranges, sampled rows elsewhere) and at
reduced sizes that still span several row tiles, key tiles and a ragged tail.
"""
import math
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
import tree_verify_mla_ddt_amd as ddt
from tree_verify_mla_ddt_amd import workloads

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-3, "f32": 1e-5}


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
    t = torch.as_tensor(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.contiguous().cuda()


def sentinel_tree_out(B, Q):
    W = (Q + 63) // 64
    out = {k: torch.full((B, Q), 12345, dtype=torch.int32, device="cuda") for k in
           ("node_token", "parent", "depth", "position", "first_child", "next_sibling")}
    out["score"] = torch.full((B, Q), float("nan"), dtype=torch.float32, device="cuda")
    out["vis"] = torch.full((B, Q, W), -7, dtype=torch.int64, device="cuda")
    out["n_nodes"] = torch.full((B,), -9, dtype=torch.int32, device="cuda")
    return out


def gpu_build(logp, ids, root, plen, budget):
    B = logp.shape[0]
    out = sentinel_tree_out(B, budget + 1)
    ddt.tree_build(dev(logp), dev(ids), dev(root), dev(plen), budget, out=out)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def assert_tree_bits(g, o):
    for k in o:
        gv = g[k]
        ov = o[k]
        if k == "score":
            np.testing.assert_array_equal(gv.view(np.uint32), ov.view(np.uint32), err_msg=k)
        elif k == "vis":
            np.testing.assert_array_equal(gv.view(np.uint64), ov, err_msg=k)
        else:
            np.testing.assert_array_equal(gv, ov, err_msg=k)


# ----------------------------------------------------------------------------- tree build

@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_tree_build_workloads_bit_exact(name):
    note(f"tree_build {name}")
    wl = workloads.make_workload(name, with_kv=False)
    o = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
    g = gpu_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
    assert_tree_bits(g, o)


def random_drafts(rng, B, D, K, kind):
    if kind == "ties":
        vals = np.array([0.0, -0.5, -1.0, -1.5, -2.0, -np.inf], np.float32)
        logp = rng.choice(vals, size=(B, D, K))
    elif kind == "unsorted":      # precondition violated: still the same algorithm
        logp = -rng.exponential(1.0, size=(B, D, K)).astype(np.float32)
    elif kind == "denormal":
        logp = -np.abs(rng.normal(0, 1, size=(B, D, K))).astype(np.float32) * np.float32(1e-39)
    elif kind == "nan":
        logp = -np.abs(rng.normal(0, 2, size=(B, D, K))).astype(np.float32)
        logp[rng.random((B, D, K)) < 0.2] = np.nan
    else:
        x = rng.normal(0, 2, size=(B, D, K))
        logp = (x - np.log(np.exp(x).sum(-1, keepdims=True))).astype(np.float32)
    if kind not in ("unsorted", "nan"):
        logp = -np.sort(-logp, axis=-1)
    ids = rng.integers(0, 160000, size=(B, D, K)).astype(np.int32)
    root = rng.integers(0, 160000, size=B).astype(np.int32)
    plen = rng.integers(0, 40000, size=B).astype(np.int32)
    return logp.astype(np.float32), ids, root, plen


@pytest.mark.parametrize("kind", ["ties", "unsorted", "denormal", "nan", "plain"])
@pytest.mark.parametrize("D,K,budget,B", [(1, 1, 0, 3), (4, 4, 8, 5), (15, 8, 32, 7),
                                          (15, 16, 64, 8), (8, 8, 127, 4), (64, 64, 127, 2),
                                          (3, 2, 100, 3), (0, 5, 10, 2), (5, 0, 10, 2)])
def test_tree_build_adversarial_bit_exact(kind, D, K, budget, B):
    rng = np.random.default_rng(zlib.crc32(repr((kind, D, K, budget)).encode()))
    logp, ids, root, plen = random_drafts(rng, B, D, K, kind)
    o = oracle.tree_build(logp, ids, root, plen, budget)
    g = gpu_build(logp, ids, root, plen, budget)
    assert_tree_bits(g, o)


def test_tree_build_large_batch_and_determinism():
    rng = np.random.default_rng(11)
    logp, ids, root, plen = random_drafts(rng, 1000, 15, 16, "plain")
    o = oracle.tree_build(logp, ids, root, plen, 64)
    g1 = gpu_build(logp, ids, root, plen, 64)
    g2 = gpu_build(logp, ids, root, plen, 64)
    assert_tree_bits(g1, o)
    assert_tree_bits(g2, o)


# ----------------------------------------------------------------------------- accept

def sentinel_accept_out(B, Q):
    return {"accept_len": torch.full((B,), -5, dtype=torch.int32, device="cuda"),
            "accept_nodes": torch.full((B, Q), 777, dtype=torch.int32, device="cuda"),
            "out_tokens": torch.full((B, Q), 777, dtype=torch.int32, device="cuda"),
            "next_root": torch.full((B,), -5, dtype=torch.int32, device="cuda")}


def gpu_accept(tok, par, nn, tgt):
    B, Q = tok.shape
    out = sentinel_accept_out(B, Q)
    ddt.tree_accept(dev(tok), dev(par), dev(nn), dev(tgt), out=out)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_tree_accept_workloads_bit_exact(name):
    note(f"tree_accept {name}")
    wl = workloads.make_workload(name, with_kv=False)
    t = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
    lens = set()
    for seed in range(6):
        tgt = workloads.synth_target_argmax(wl, t["node_token"], t["parent"], t["depth"],
                                            t["n_nodes"], seed=seed)
        o = oracle.tree_accept(t["node_token"], t["parent"], t["n_nodes"], tgt)
        g = gpu_accept(t["node_token"], t["parent"], t["n_nodes"], tgt)
        for k in o:
            np.testing.assert_array_equal(g[k], o[k], err_msg=k)
        lens |= set(o["accept_len"].tolist())
    note(f"  accept lengths seen: {sorted(lens)}")


def test_tree_accept_adversarial_bit_exact():
    rng = np.random.default_rng(3)
    for Q in (1, 2, 9, 64, 65, 127, 128):
        B = 40
        par = np.full((B, Q), -1, np.int32)
        for b in range(B):
            for i in range(1, Q):
                par[b, i] = rng.integers(0, i) if rng.random() > 0.05 else rng.integers(-3, Q + 3)
        tok = rng.integers(0, 6, size=(B, Q)).astype(np.int32)   # many duplicate tokens
        tgt = rng.integers(0, 6, size=(B, Q)).astype(np.int32)
        nn = rng.integers(-2, Q + 3, size=B).astype(np.int32)
        o = oracle.tree_accept(tok, par, nn, tgt)
        g = gpu_accept(tok, par, nn, tgt)
        for k in o:
            np.testing.assert_array_equal(g[k], o[k], err_msg=f"{k} Q={Q}")


# ----------------------------------------------------------------------------- attention

def gpu_attn(wl, r2s, plen, nn, vis_u64, q_lat=None, q_pe=None, c_kv=None, k_pe=None):
    B, Q, H = wl.B, wl.Q, wl.H
    out = torch.full((B, Q, H, wl.d_lat), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Q, H), float("nan"), dtype=torch.float32, device="cuda")
    ddt.verify_attn(dev(wl.q_lat if q_lat is None else q_lat), dev(wl.q_pe if q_pe is None else q_pe),
                    dev(wl.c_kv if c_kv is None else c_kv), dev(wl.k_pe if k_pe is None else k_pe),
                    dev(r2s), dev(plen), dev(nn), dev(vis_u64.view(np.int64)), wl.sm_scale,
                    out=out, lse=lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def oracle_attn(wl, r2s, plen, nn, vis, rows=None, q_lat=None, q_pe=None, c_kv=None, k_pe=None):
    f = lambda t: t.float().numpy()
    return oracle.verify_attn(f(wl.q_lat if q_lat is None else q_lat),
                              f(wl.q_pe if q_pe is None else q_pe),
                              f(wl.c_kv if c_kv is None else c_kv),
                              f(wl.k_pe if k_pe is None else k_pe),
                              r2s, plen, nn, vis, wl.sm_scale, rows=rows)


def check_attn(g_out, g_lse, o_out, o_lse, tol, label):
    assert np.isfinite(g_out).all(), f"{label}: non-finite output (unwritten element?)"
    err = np.abs(g_out.astype(np.float64) - o_out).max() if o_out.size else 0.0
    fin = np.isfinite(o_lse)
    assert (np.isneginf(g_lse) == ~fin).all(), f"{label}: lse -inf pattern differs"
    lerr = np.abs(g_lse[fin].astype(np.float64) - o_lse[fin]).max() if fin.any() else 0.0
    note(f"  {label}: max_abs out {err:.3e}, lse {lerr:.3e} (tol {tol})")
    assert err <= tol and lerr <= tol, f"{label}: max_abs {err:.3e} / lse {lerr:.3e} > {tol}"


def tree_for(wl):
    t = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
    return t


@pytest.mark.parametrize("name,overrides,shuffle", [
    ("tiny_fp32", {}, False),
    ("tiny_fp32", {}, True),
    ("b1_l2k_q9", {}, False),
    ("b1_l2k_q9", {"L": 999}, True),
    ("b4_l4k_q17", {"L": 700}, True),
    ("b4_l4k_q33", {"L": 600, "B": 3}, False),
    ("b64_l2k_q9", {"B": 6, "L": 300}, True),
    # Uniform batches of at least one row tile per workgroup take the aligned
    # split: whole row tiles, then leftover ranges of 0-1 key tiles (L 40) or
    # ranges crossing row tiles (L 520); ragged prefixes on the doubled grid fall
    # back to the linear split.
    ("b64_l2k_q9", {"L": 40}, True),
    ("b64_l2k_q9", {"L": 520}, False),
    ("b64_l2k_q9", {"L": 300, "L_jitter": 0.25}, True),
    # 100 uniform requests: 500 row tiles on a 256-range grid, so the aligned
    # split leaves 244 row tiles that do not divide the grid and charges their
    # start cost: leftover ranges cross row tiles and some end inside a start
    # cost (nothing to run).
    ("b64_l2k_q9", {"B": 100, "L": 100}, True),
    ("b8_l32k_q65", {"B": 2, "L": 600}, True),
    # Q=65 with eight uniform requests: 264 row tiles, at least one per
    # workgroup, so the aligned split runs (eight leftover row tiles, each
    # merged from about 32 contributors).
    ("b8_l32k_q65", {"L": 600}, True),
    # The bf16 64+16 instantiation: one row tile, and several with ragged
    # prefixes and two-word bitsets.
    ("tiny_fp32", {"dtype": "bf16"}, True),
    ("tiny_fp32", {"dtype": "bf16", "B": 3, "H": 16, "L": 300, "L_jitter": 0.3,
                   "budget": 70, "D": 9, "K": 4}, True),
])
def test_verify_attn_full_oracle(name, overrides, shuffle):
    """Every row against the oracle at sizes it evaluates in seconds."""
    note(f"verify_attn full-oracle {name} {overrides} shuffle={shuffle}")
    wl = workloads.make_workload(name, shuffle_slots=shuffle, **overrides)
    t = tree_for(wl)
    g_out, g_lse = gpu_attn(wl, wl.req_to_slot, wl.prefix_len, t["n_nodes"], t["vis"])
    o_out, o_lse = oracle_attn(wl, wl.req_to_slot, wl.prefix_len, t["n_nodes"], t["vis"])
    check_attn(g_out, g_lse, o_out, o_lse, TOL[wl.dtype], name)


@pytest.mark.parametrize("name", ["b1_l2k_q9", "b4_l4k_q17", "b4_l4k_q33", "b64_l2k_q9",
                                  "b64_l2k_q9_h8", "b8_l32k_q65_h8"])
def test_verify_attn_full_size_every_row(name):
    """The benchmark's full workloads, in the benchmark's launch configuration,
    every row against the oracle."""
    note(f"verify_attn full-size every row {name}")
    wl = workloads.make_workload(name)
    t = tree_for(wl)
    g_out, g_lse = gpu_attn(wl, wl.req_to_slot, wl.prefix_len, t["n_nodes"], t["vis"])
    o_out, o_lse = oracle_attn(wl, wl.req_to_slot, wl.prefix_len, t["n_nodes"], t["vis"])
    check_attn(g_out, g_lse, o_out, o_lse, TOL[wl.dtype], name)


def test_verify_attn_max_shape():
    """The max shape (batch 8, prefix 32768, q_len 65) in the benchmark's launch
    configuration: every row of the last request (its row tiles hold the
    aligned split's leftover ranges, merged from about 32 contributors each)
    and 12 sampled rows of every other request against the oracle, and every
    output finite."""
    note("verify_attn max shape")
    wl = workloads.make_workload("b8_l32k_q65")
    t = tree_for(wl)
    g_out, g_lse = gpu_attn(wl, wl.req_to_slot, wl.prefix_len, t["n_nodes"], t["vis"])
    assert np.isfinite(g_out).all()
    rng = np.random.default_rng(5)
    last = wl.B - 1
    rows = [(last, i, h) for i in range(wl.Q) for h in range(wl.H)]
    for b in range(last):
        nodes = rng.integers(0, int(t["n_nodes"][b]), size=12)
        nodes[:2] = [0, int(t["n_nodes"][b]) - 1]
        rows += [(b, int(i), int(h)) for i, h in zip(nodes, rng.integers(0, wl.H, size=12))]
    rows = np.array(rows, np.int32)
    o_out, o_lse = oracle_attn(wl, wl.req_to_slot, wl.prefix_len, t["n_nodes"], t["vis"], rows=rows)
    check_attn(g_out[rows[:, 0], rows[:, 1], rows[:, 2]], g_lse[rows[:, 0], rows[:, 1], rows[:, 2]],
               o_out, o_lse, TOL[wl.dtype], "b8_l32k_q65")


@pytest.mark.parametrize("name,overrides", [
    ("b1_l2k_q9", {}),                                   # narrow form, linear split
    ("b4_l4k_q33", {"L": 900}),                          # wide form, linear split
    ("b8_l32k_q65", {"L": 600}),                         # wide form, aligned split
    ("b64_l2k_q9", {"H": 8, "L": 700}),                  # narrow form, aligned split
    ("tiny_fp32", {"dtype": "bf16", "B": 3, "H": 16, "L": 300, "budget": 70, "D": 9,
                   "K": 4}),                             # 64+16 kernel
])
def test_verify_attn_far_larger_later_scores(name, overrides):
    """Keys whose rotary part is scaled by 128 (exactly, in bf16) score far
    above everything else, so a key range that meets one after its first tile
    sees scores more than 2^64 above the reference the 512-wide kernels fix at
    their first tile, and runs again with the range's largest score (and the
    64-wide kernel rescales).  Every row against the oracle."""
    note(f"verify_attn far larger later scores {name} {overrides}")
    wl = workloads.make_workload(name, **overrides)
    t = tree_for(wl)
    k_pe = wl.k_pe.clone()
    for b in range(wl.B):
        for j in (40, 100, 333, 700, 1500, 2000):
            if j < int(wl.prefix_len[b]):
                k_pe[int(wl.req_to_slot[b, j])] *= 128
    g_out, g_lse = gpu_attn(wl, wl.req_to_slot, wl.prefix_len, t["n_nodes"], t["vis"], k_pe=k_pe)
    o_out, o_lse = oracle_attn(wl, wl.req_to_slot, wl.prefix_len, t["n_nodes"], t["vis"], k_pe=k_pe)
    check_attn(g_out, g_lse, o_out, o_lse, TOL[wl.dtype], name)


def test_verify_attn_edge_cases():
    """Underfull trees, empty prefixes, single-node trees, out-of-range slot
    ids and clamped lengths, all against the oracle."""
    rng = np.random.default_rng(9)
    wl = workloads.make_workload("b4_l4k_q33", B=4, L=200)
    t = tree_for(wl)
    plen = wl.prefix_len.copy()
    nn = t["n_nodes"].copy()
    r2s = wl.req_to_slot.copy()
    plen[0] = 0                    # no prefix: the tree only
    nn[1] = 1                      # root only
    nn[2] = 7                      # underfull
    r2s[3, 5] = wl.num_slots + 10  # invalid slot ids are invisible
    r2s[3, 17] = -4
    for label, p, n in (("edges", plen, nn),
                        ("clamps", np.array([10 ** 6, -5, 3, 9], np.int32),
                         np.array([99, 0, -1, 2], np.int32))):
        g_out, g_lse = gpu_attn(wl, r2s, p, n, t["vis"])
        o_out, o_lse = oracle_attn(wl, r2s, p, n, t["vis"])
        check_attn(g_out, g_lse, o_out, o_lse, TOL[wl.dtype], label)


@pytest.mark.parametrize("Q,H,L,B,jitter", [
    (1, 64, 2048, 2, 0.0), (128, 8, 333, 2, 0.0), (65, 64, 70, 1, 0.0), (2, 1, 31, 3, 0.0),
    (9, 3, 1, 2, 0.0),
    # The limits: 512 requests (two per thread in the work prefix), uniform
    # (aligned split of 512 row tiles) and ragged (one stream); the widest tree
    # at 64 heads (64 row tiles of one request); 128 heads (a node per row tile).
    (2, 8, 20, 512, 0.0), (3, 8, 40, 512, 0.9), (128, 64, 50, 1, 0.0), (9, 128, 100, 2, 0.0),
])
def test_verify_attn_shapes(Q, H, L, B, jitter):
    """Decode (Q=1), the widest tree (Q=128, two bitset words), odd head counts,
    tiny prefixes and the batch limit, with random trees."""
    note(f"verify_attn shape Q={Q} H={H} L={L} B={B} jitter={jitter}")
    rng = np.random.default_rng(Q * 1000 + H + B)
    wl = workloads.make_workload("b1_l2k_q9", B=B, L=L, budget=Q - 1, H=H, D=8, K=16,
                                 L_jitter=jitter)
    par = np.full((B, Q), -1, np.int32)
    for b in range(B):
        for i in range(1, Q):
            par[b, i] = rng.integers(0, i)
    W = (Q + 63) // 64
    vis = np.zeros((B, Q, W), np.uint64)
    for b in range(B):
        for i in range(Q):
            a = i
            while a >= 0:
                vis[b, i, a // 64] |= np.uint64(1) << np.uint64(a % 64)
                a = par[b, a]
    nn = np.full((B,), Q, np.int32)
    g_out, g_lse = gpu_attn(wl, wl.req_to_slot, wl.prefix_len, nn, vis)
    o_out, o_lse = oracle_attn(wl, wl.req_to_slot, wl.prefix_len, nn, vis)
    check_attn(g_out, g_lse, o_out, o_lse, TOL["bf16"], f"Q{Q}H{H}L{L}")


def test_verify_attn_determinism():
    wl = workloads.make_workload("b4_l4k_q17", L=900)
    t = tree_for(wl)
    a1, l1 = gpu_attn(wl, wl.req_to_slot, wl.prefix_len, t["n_nodes"], t["vis"])
    a2, l2 = gpu_attn(wl, wl.req_to_slot, wl.prefix_len, t["n_nodes"], t["vis"])
    np.testing.assert_array_equal(a1.view(np.uint32), a2.view(np.uint32))
    np.testing.assert_array_equal(l1.view(np.uint32), l2.view(np.uint32))


@pytest.mark.parametrize("name,overrides", [("b1_l2k_q9", {"L": 600}),
                                            ("b4_l4k_q17", {"L": 900}),
                                            ("b64_l2k_q9", {"L": 300}),
                                            ("tiny_fp32", {})])
def test_verify_attn_kernel_times_matches_call(name, overrides):
    """The kernel-time measurement leaves the call's exact result in out / lse
    and reports positive per-launch times."""
    note(f"verify_attn kernel times {name} {overrides}")
    wl = workloads.make_workload(name, **overrides)
    t = tree_for(wl)
    a1, l1 = gpu_attn(wl, wl.req_to_slot, wl.prefix_len, t["n_nodes"], t["vis"])
    args = (dev(wl.q_lat), dev(wl.q_pe), dev(wl.c_kv), dev(wl.k_pe), dev(wl.req_to_slot),
            dev(wl.prefix_len), dev(t["n_nodes"]), dev(t["vis"].view(np.int64)), wl.sm_scale)
    ms_a, ms_m, out, lse = ddt.verify_attn_kernel_times(*args, reps=5)
    torch.cuda.synchronize()
    assert ms_a > 0.0 and ms_m > 0.0
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), a1.view(np.uint32))
    np.testing.assert_array_equal(lse.cpu().numpy().view(np.uint32), l1.view(np.uint32))


# ----------------------------------------------------------------------------- composition

@pytest.mark.parametrize("name", ["tiny_fp32", "b64_l2k_q9", "b4_l4k_q33"])
def test_composition_on_device(name):
    """build -> attention -> accept on one stream, no host round-trip, against
    the oracle chain.  The target tokens are synthesized from the oracle's tree
    (the GPU tree is bit-identical to it) and uploaded before the chain runs."""
    note(f"composition {name}")
    wl = workloads.make_workload(name, L=min(wl_L(name), 600))
    ot = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
    tgt = workloads.synth_target_argmax(wl, ot["node_token"], ot["parent"], ot["depth"],
                                        ot["n_nodes"])
    oa = oracle.tree_accept(ot["node_token"], ot["parent"], ot["n_nodes"], tgt)
    o_out, _ = oracle_attn(wl, wl.req_to_slot, wl.prefix_len, ot["n_nodes"], ot["vis"])

    ins = [dev(wl.topk_logp), dev(wl.topk_ids), dev(wl.root_token), dev(wl.prefix_len)]
    q_lat, q_pe, c_kv, k_pe = dev(wl.q_lat), dev(wl.q_pe), dev(wl.c_kv), dev(wl.k_pe)
    r2s, d_tgt = dev(wl.req_to_slot), dev(tgt)
    torch.cuda.synchronize()
    tree = ddt.tree_build(*ins, wl.budget)
    out, lse = ddt.verify_attn(q_lat, q_pe, c_kv, k_pe, r2s, ins[3], tree["n_nodes"],
                               tree["vis"], wl.sm_scale)
    acc = ddt.tree_accept(tree["node_token"], tree["parent"], tree["n_nodes"], d_tgt)
    torch.cuda.synchronize()
    for k in oa:
        np.testing.assert_array_equal(acc[k].cpu().numpy(), oa[k], err_msg=k)
    err = np.abs(out.cpu().numpy().astype(np.float64) - o_out).max()
    assert err <= TOL[wl.dtype]


def wl_L(name):
    return workloads.CONFIGS[name]["L"]


def test_graph_capture_replays():
    """The three stages captured into one HIP graph and replayed several times,
    with eager work in between, give the eager result every time."""
    wl = workloads.make_workload("b64_l2k_q9", B=8, L=400)
    ot = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
    tgt = dev(workloads.synth_target_argmax(wl, ot["node_token"], ot["parent"], ot["depth"],
                                            ot["n_nodes"]))
    ins = [dev(wl.topk_logp), dev(wl.topk_ids), dev(wl.root_token), dev(wl.prefix_len)]
    q_lat, q_pe, c_kv, k_pe, r2s = (dev(wl.q_lat), dev(wl.q_pe), dev(wl.c_kv), dev(wl.k_pe),
                                    dev(wl.req_to_slot))
    B, Q, H = wl.B, wl.Q, wl.H
    tree = sentinel_tree_out(B, Q)
    out = torch.empty((B, Q, H, wl.d_lat), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Q, H), dtype=torch.float32, device="cuda")
    ws = torch.empty((ddt.workspace_size(B, Q, H, r2s.shape[1], wl.d_lat),), dtype=torch.uint8,
                     device="cuda")
    acc = sentinel_accept_out(B, Q)

    def step():
        ddt.tree_build(*ins, wl.budget, out=tree)
        ddt.verify_attn(q_lat, q_pe, c_kv, k_pe, r2s, ins[3], tree["n_nodes"], tree["vis"],
                        wl.sm_scale, out=out, lse=lse, workspace=ws)
        ddt.tree_accept(tree["node_token"], tree["parent"], tree["n_nodes"], tgt, out=acc)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref_out = out.clone()
    ref_acc = {k: v.clone() for k, v in acc.items()}
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        out.fill_(float("nan"))
        for v in acc.values():
            v.fill_(-3)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {rep}"
        for k in acc:
            assert torch.equal(acc[k], ref_acc[k]), f"replay {rep} {k}"
        _ = (q_lat.float() * 2).sum().item()   # unrelated eager work between replays
