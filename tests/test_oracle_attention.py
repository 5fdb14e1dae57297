"""Pins for the oracle's tree-verify attention.

The operation is absorbed MLA attention of every tree node over the shared
latent prefix plus its own ancestors ("The Architecture of a Thousand-Parameter
Decision ...", "What to Build New" item 2; "The Milestone Message ...", "MLA"
and "Architectural Abstraction").  The oracle is checked against:

* special cases that reduce to torch's scaled_dot_product_attention (float64 on
  the CPU): a one-node tree is plain decode attention; a chain tree is causal
  attention over [prefix | chain]; a random tree is SDPA with a boolean mask
  built from the parent array (not from the visibility bitsets the oracle reads);
* the MLA absorb identity: non-absorbed multi-head attention with explicit
  W_UK / W_UV projections equals W_UV applied to the latent output;
* closed forms: zero queries give the mean of the visible values and
  lse = ln(count); a constant value vector comes back unchanged; a single
  visible key has lse equal to its score;
* invariants: prefix order does not matter, an out-of-range slot is the same as
  a missing key, padding rows are zero with lse = -inf.
"""
import math

import numpy as np
import pytest
import torch

import oracle



@pytest.fixture(autouse=True)
def _float64_default():
    """Float64 as torch's default dtype inside this module's tests only (set at
    import time it would leak into every module collected after this one)."""
    prev = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(prev)


def f32(x):
    """sm_scale crosses the ABI as fp32; references use the same rounded value."""
    return float(np.float32(x))


def make_case(rng, B, Q, H, d_lat, d_rope, L, n_nodes, parents=None):
    """Random absorbed-MLA inputs with contiguous slots per request."""
    max_kv = max(L) + Q
    S = sum(L) + B * Q
    c_kv = rng.standard_normal((S, d_lat)).astype(np.float32)
    k_pe = rng.standard_normal((S, d_rope)).astype(np.float32)
    q_lat = rng.standard_normal((B, Q, H, d_lat)).astype(np.float32)
    q_pe = rng.standard_normal((B, Q, H, d_rope)).astype(np.float32)
    r2s = np.full((B, max_kv), -1, np.int32)
    base = 0
    for b in range(B):
        r2s[b, : L[b] + Q] = base + np.arange(L[b] + Q)
        base += L[b] + Q
    if parents is None:
        parents = []
        for b in range(B):
            p = [-1] + [int(rng.integers(0, i)) for i in range(1, Q)]
            parents.append(p)
    parents = np.array(parents, np.int32)
    return dict(q_lat=q_lat, q_pe=q_pe, c_kv=c_kv, k_pe=k_pe, req_to_slot=r2s,
                prefix_len=np.array(L, np.int32), n_nodes=np.array(n_nodes, np.int32),
                parents=parents)


def vis_from_parents(parents, Q):
    """Ancestor-or-self bitsets, packed by the test itself."""
    B = parents.shape[0]
    W = (Q + 63) // 64
    vis = np.zeros((B, Q, W), np.uint64)
    for b in range(B):
        for i in range(Q):
            a = i
            while a >= 0:
                vis[b, i, a // 64] |= np.uint64(1) << np.uint64(a % 64)
                a = parents[b, a]
    return vis


def dense_mask_from_parents(parents_b, L, n):
    """Bool [n, L+n]: the whole prefix, then node i sees k iff k is on i's root path."""
    m = torch.zeros((n, L + n), dtype=torch.bool)
    m[:, :L] = True
    for i in range(n):
        a = i
        while a >= 0:
            m[i, L + a] = True
            a = int(parents_b[a])
    return m


def run_oracle(c, vis, scale):
    return oracle.verify_attn(c["q_lat"], c["q_pe"], c["c_kv"], c["k_pe"], c["req_to_slot"],
                              c["prefix_len"], c["n_nodes"], vis, scale)


def sdpa_reference(c, b, mask, scale):
    """torch SDPA over keys [c_kv | k_pe], values c_kv, for all heads of request b."""
    L, n = int(c["prefix_len"][b]), int(c["n_nodes"][b])
    slots = torch.from_numpy(c["req_to_slot"][b, : L + n].astype(np.int64))
    k = torch.cat([torch.from_numpy(c["c_kv"]).double()[slots],
                   torch.from_numpy(c["k_pe"]).double()[slots]], dim=-1)       # [L+n, 576]
    v = torch.from_numpy(c["c_kv"]).double()[slots]                            # [L+n, 512]
    q = torch.cat([torch.from_numpy(c["q_lat"][b, :n]).double(),
                   torch.from_numpy(c["q_pe"][b, :n]).double()], dim=-1)      # [n, H, 576]
    q = q.transpose(0, 1)                                                      # [H, n, 576]
    out = torch.nn.functional.scaled_dot_product_attention(
        q, k[None].expand(q.shape[0], -1, -1), v[None].expand(q.shape[0], -1, -1),
        attn_mask=mask, scale=scale)
    return out.transpose(0, 1).numpy()                                         # [n, H, 512]


@pytest.mark.parametrize("d_lat,d_rope", [(64, 16), (512, 64)])
def test_one_node_tree_is_decode_attention(d_lat, d_rope):
    rng = np.random.default_rng(1)
    c = make_case(rng, B=2, Q=1, H=3, d_lat=d_lat, d_rope=d_rope, L=[37, 5], n_nodes=[1, 1])
    scale = f32(1.0 / math.sqrt(192))
    out, lse = run_oracle(c, vis_from_parents(c["parents"], 1), scale)
    for b in range(2):
        ref = sdpa_reference(c, b, None, scale)
        np.testing.assert_allclose(out[b, :1], ref, rtol=0, atol=1e-12)
        # lse of decode = logsumexp of the scaled scores over prefix + self
        L = int(c["prefix_len"][b])
        slots = c["req_to_slot"][b, : L + 1]
        k = np.concatenate([c["c_kv"][slots], c["k_pe"][slots]], 1).astype(np.float64)
        q = np.concatenate([c["q_lat"][b, 0], c["q_pe"][b, 0]], 1).astype(np.float64)
        ref_lse = torch.logsumexp(torch.from_numpy(scale * q @ k.T), dim=-1).numpy()
        np.testing.assert_allclose(lse[b, 0], ref_lse, rtol=0, atol=1e-12)


def test_chain_tree_is_causal_attention():
    rng = np.random.default_rng(2)
    Q, L = 9, 50
    c = make_case(rng, B=1, Q=Q, H=4, d_lat=64, d_rope=16, L=[L], n_nodes=[Q],
                  parents=[[-1] + list(range(Q - 1))])
    scale = f32(0.11)
    out, _ = run_oracle(c, vis_from_parents(c["parents"], Q), scale)
    causal = torch.ones((Q, L + Q), dtype=torch.bool).tril(diagonal=L)  # bottom-right aligned
    ref = sdpa_reference(c, 0, causal, scale)
    np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("Q", [17, 65, 100])
def test_random_tree_matches_masked_sdpa(Q):
    rng = np.random.default_rng(Q)
    B = 2
    L = [int(rng.integers(0, 40)), int(rng.integers(1, 40))]
    n_nodes = [Q, max(1, Q - 5)]
    c = make_case(rng, B=B, Q=Q, H=2, d_lat=64, d_rope=16, L=L, n_nodes=n_nodes)
    scale = f32(1.0 / math.sqrt(80))
    out, lse = run_oracle(c, vis_from_parents(c["parents"], Q), scale)
    for b in range(B):
        n = n_nodes[b]
        mask = dense_mask_from_parents(c["parents"][b], L[b], n)
        ref = sdpa_reference(c, b, mask, scale)
        np.testing.assert_allclose(out[b, :n], ref, rtol=0, atol=1e-12)
        assert (out[b, n:] == 0).all() and np.isneginf(lse[b, n:]).all()


def test_mla_absorb_identity():
    # Non-absorbed MHA: k_h = W_UK[h] c, v_h = W_UV[h] c, q = [q_nope | q_pe].
    # Absorbed: q_lat = W_UK[h]^T q_nope; output o_h = W_UV[h] out_lat.
    rng = np.random.default_rng(3)
    H, d_nope, d_lat, d_rope, d_v, Q, L = 4, 128, 512, 64, 128, 9, 30
    c = make_case(rng, B=1, Q=Q, H=H, d_lat=d_lat, d_rope=d_rope, L=[L], n_nodes=[Q])
    # Dyadic W_UK and q_nope keep q_lat = W_UK^T q_nope exact in fp32, so the
    # absorbed and non-absorbed forms see the same query.
    w_uk = rng.integers(-1, 2, size=(H, d_nope, d_lat)) / 8.0
    q_nope = rng.integers(-16, 17, size=(Q, H, d_nope)) / 8.0
    w_uv = rng.standard_normal((H, d_v, d_lat)) / math.sqrt(d_lat)
    q_lat = np.einsum("hnc,ihn->ihc", w_uk, q_nope)
    assert (q_lat.astype(np.float32) == q_lat).all()
    c["q_lat"] = q_lat[None].astype(np.float32)
    q_nope_used = q_nope
    scale = f32(1.0 / math.sqrt(d_nope + d_rope))
    out, _ = run_oracle(c, vis_from_parents(c["parents"], Q), scale)

    slots = c["req_to_slot"][0, : L + Q]
    lat = torch.from_numpy(c["c_kv"][slots].astype(np.float64))               # [N, 512]
    pe = torch.from_numpy(c["k_pe"][slots].astype(np.float64))
    k = torch.cat([torch.einsum("hnc,jc->hjn", torch.from_numpy(w_uk), lat),
                   pe[None].expand(H, -1, -1)], dim=-1)                         # [H, N, 192]
    v = torch.einsum("hvc,jc->hjv", torch.from_numpy(w_uv), lat)               # [H, N, 128]
    q = torch.cat([torch.from_numpy(q_nope_used),
                   torch.from_numpy(c["q_pe"][0].astype(np.float64))], dim=-1).transpose(0, 1)
    mask = dense_mask_from_parents(c["parents"][0], L, Q)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
    expect = o.transpose(0, 1).numpy()                                          # [Q, H, 128]
    got = np.einsum("hvc,ihc->ihv", w_uv, out[0])
    np.testing.assert_allclose(got, expect, rtol=0, atol=1e-9)


def test_zero_query_gives_mean_and_log_count():
    rng = np.random.default_rng(4)
    Q, L = 12, 21
    c = make_case(rng, B=1, Q=Q, H=2, d_lat=64, d_rope=16, L=[L], n_nodes=[Q])
    c["q_lat"][:] = 0
    c["q_pe"][:] = 0
    vis = vis_from_parents(c["parents"], Q)
    out, lse = run_oracle(c, vis, 0.3)
    for i in range(Q):
        anc = []
        a = i
        while a >= 0:
            anc.append(a)
            a = c["parents"][0, a]
        rows = list(range(L)) + [L + a for a in anc]
        mean = c["c_kv"][c["req_to_slot"][0, rows]].astype(np.float64).mean(0)
        for h in range(2):
            np.testing.assert_allclose(out[0, i, h], mean, rtol=0, atol=1e-13)
            assert abs(lse[0, i, h] - math.log(len(rows))) < 1e-13


def test_constant_values_and_single_key():
    rng = np.random.default_rng(5)
    c = make_case(rng, B=1, Q=4, H=2, d_lat=64, d_rope=16, L=[0], n_nodes=[4],
                  parents=[[-1, 0, 0, 1]])
    # single visible key for the root: lse equals the root's own score
    out, lse = run_oracle(c, vis_from_parents(c["parents"], 4), 0.25)
    s = c["req_to_slot"][0, 0]
    for h in range(2):
        score = 0.25 * (np.dot(c["q_lat"][0, 0, h].astype(np.float64), c["c_kv"][s].astype(np.float64))
                        + np.dot(c["q_pe"][0, 0, h].astype(np.float64), c["k_pe"][s].astype(np.float64)))
        assert abs(lse[0, 0, h] - score) < 1e-12
        np.testing.assert_allclose(out[0, 0, h], c["c_kv"][s], rtol=0, atol=1e-14)
    # constant value rows come back unchanged whatever the weights
    c["c_kv"][:] = 1.0
    out, _ = run_oracle(c, vis_from_parents(c["parents"], 4), 0.25)
    np.testing.assert_allclose(out[0], 1.0, rtol=0, atol=1e-14)


def test_prefix_permutation_invariance_and_bad_slots():
    rng = np.random.default_rng(6)
    Q, L = 5, 40
    c = make_case(rng, B=1, Q=Q, H=3, d_lat=64, d_rope=16, L=[L], n_nodes=[Q])
    vis = vis_from_parents(c["parents"], Q)
    out, lse = run_oracle(c, vis, 0.2)
    c2 = dict(c)
    r2s = c["req_to_slot"].copy()
    r2s[0, :L] = rng.permutation(r2s[0, :L])
    c2["req_to_slot"] = r2s
    out2, lse2 = run_oracle(c2, vis, 0.2)
    np.testing.assert_allclose(out2, out, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-13)
    # a slot id outside the pool is the same as dropping that prefix entry
    r3 = c["req_to_slot"].copy()
    r3[0, 7] = 10 ** 6
    out3, _ = run_oracle(dict(c, req_to_slot=r3), vis, 0.2)
    r4 = np.concatenate([c["req_to_slot"][:, :7], c["req_to_slot"][:, 8:],
                         np.full((1, 1), -1, np.int32)], axis=1)
    out4, _ = run_oracle(dict(c, req_to_slot=r4, prefix_len=np.array([L - 1], np.int32)), vis, 0.2)
    np.testing.assert_allclose(out3, out4, rtol=0, atol=1e-13)


def test_range_clamps_and_padding():
    rng = np.random.default_rng(7)
    Q, L = 6, 10
    c = make_case(rng, B=1, Q=Q, H=2, d_lat=64, d_rope=16, L=[L], n_nodes=[3])
    vis = vis_from_parents(c["parents"], Q)
    out, lse = run_oracle(c, vis, 0.2)
    assert (out[0, 3:] == 0).all() and np.isneginf(lse[0, 3:]).all()
    # n_nodes above Q behaves as Q; negative n_nodes as 0 (all rows padding)
    o_hi, _ = run_oracle(dict(c, n_nodes=np.array([99], np.int32)), vis, 0.2)
    o_q, _ = run_oracle(dict(c, n_nodes=np.array([Q], np.int32)), vis, 0.2)
    np.testing.assert_array_equal(o_hi, o_q)
    o_neg, l_neg = run_oracle(dict(c, n_nodes=np.array([-3], np.int32)), vis, 0.2)
    assert (o_neg == 0).all() and np.isneginf(l_neg).all()
