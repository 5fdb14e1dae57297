"""GPU parity of ddt_kv_commit (through its C ABI) against the CPU oracle.

Bit-exact on every output: the rewritten slot table, the new prefix lengths,
the released slots (pre-filled with a sentinel, so every element must be
written) and their counts.  Cases: the build -> accept -> commit chain on every
workload, and adversarial tables (clamped prefix lengths and tree sizes,
accept lengths past the tree, malformed paths).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_verify_mla_ddt_amd as ddt
from tree_verify_mla_ddt_amd import workloads

pytestmark = pytest.mark.gpu


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ddt.load_library()
    yield


def dev(a):
    return torch.as_tensor(np.ascontiguousarray(a)).contiguous().cuda()


def gpu_commit(r2s, plen, nn, alen, anodes):
    B, Q = anodes.shape
    d_r2s, d_plen = dev(r2s.astype(np.int32)), dev(plen.astype(np.int32))
    out = {"freed_slots": torch.full((B, Q), 777, dtype=torch.int32, device="cuda"),
           "n_freed": torch.full((B,), -555, dtype=torch.int32, device="cuda")}
    ddt.kv_commit(d_r2s, d_plen, dev(nn.astype(np.int32)), dev(alen.astype(np.int32)),
                  dev(anodes.astype(np.int32)), out=out)
    torch.cuda.synchronize()
    return {"req_to_slot": d_r2s.cpu().numpy(), "prefix_len": d_plen.cpu().numpy(),
            "freed_slots": out["freed_slots"].cpu().numpy(), "n_freed": out["n_freed"].cpu().numpy()}


def assert_same(g, o):
    for k in ("req_to_slot", "prefix_len", "freed_slots", "n_freed"):
        np.testing.assert_array_equal(g[k], o[k], err_msg=k)


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_commit_chain_workloads(name):
    """build -> accept -> commit on the GPU, chained on one stream, against the
    oracle chain on the same seeded inputs."""
    note(f"kv_commit chain {name}")
    wl = workloads.make_workload(name, L=min(workloads.CONFIGS[name]["L"], 3000))
    ot = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
    tgt = workloads.synth_target_argmax(wl, ot["node_token"], ot["parent"], ot["depth"],
                                        ot["n_nodes"])
    oa = oracle.tree_accept(ot["node_token"], ot["parent"], ot["n_nodes"], tgt)
    oc = oracle.kv_commit(wl.req_to_slot, wl.prefix_len, ot["n_nodes"], oa["accept_len"],
                          oa["accept_nodes"])

    ins = [dev(wl.topk_logp), dev(wl.topk_ids), dev(wl.root_token), dev(wl.prefix_len)]
    r2s, plen = dev(wl.req_to_slot), dev(wl.prefix_len)
    torch.cuda.synchronize()
    tree = ddt.tree_build(*ins, wl.budget)
    acc = ddt.tree_accept(tree["node_token"], tree["parent"], tree["n_nodes"], dev(tgt))
    com = ddt.kv_commit(r2s, plen, tree["n_nodes"], acc["accept_len"], acc["accept_nodes"])
    torch.cuda.synchronize()
    g = {"req_to_slot": r2s.cpu().numpy(), "prefix_len": plen.cpu().numpy(),
         "freed_slots": com["freed_slots"].cpu().numpy(), "n_freed": com["n_freed"].cpu().numpy()}
    assert_same(g, oc)


def random_case(rng, B, Q, max_kv):
    r2s = rng.integers(-5, 1 << 20, size=(B, max_kv)).astype(np.int32)
    plen = rng.integers(-3, max_kv + 4, size=B).astype(np.int32)
    nn = rng.integers(-2, Q + 5, size=B).astype(np.int32)
    alen = rng.integers(-1, Q + 3, size=B).astype(np.int32)
    an = np.full((B, Q), -1, np.int32)
    for b in range(B):
        kind = rng.integers(0, 4)
        if kind == 0:  # a valid increasing path from the root
            k = int(rng.integers(1, Q + 1))
            rest = (np.sort(rng.choice(np.arange(1, Q), size=min(k - 1, Q - 1), replace=False))
                    if Q > 1 else np.array([], np.int64))
            p = np.concatenate([[0], rest]).astype(np.int32)
            an[b, :len(p)] = p
        elif kind == 1:  # garbage
            an[b] = rng.integers(-3, Q + 3, size=Q)
        elif kind == 2:  # increasing then a repeat
            k = rng.integers(2, Q + 1) if Q >= 2 else 1
            p = np.arange(k)
            if k >= 2:
                p[k // 2] = p[k // 2 - 1]
            an[b, :k] = p
        else:  # chain
            an[b] = np.arange(Q)
    return r2s, plen, nn, alen, an


@pytest.mark.parametrize("B,Q,max_kv,seed", [(1, 1, 1, 0), (3, 9, 20, 1), (17, 65, 70, 2),
                                             (8, 128, 300, 3), (64, 33, 33, 4), (5, 128, 128, 5)])
def test_commit_adversarial(B, Q, max_kv, seed):
    note(f"kv_commit adversarial B={B} Q={Q} max_kv={max_kv}")
    rng = np.random.default_rng(seed)
    case = random_case(rng, B, Q, max_kv)
    assert_same(gpu_commit(*case), oracle.kv_commit(*case))


def test_commit_twice_in_a_row():
    """A second commit on the committed table (next step, same tree sizes) matches
    the oracle applied twice."""
    rng = np.random.default_rng(9)
    B, Q, max_kv = 6, 17, 80
    r2s = rng.permutation(10000)[:B * max_kv].reshape(B, max_kv).astype(np.int32)
    plen = rng.integers(0, 40, size=B).astype(np.int32)
    nn = np.full(B, Q, np.int32)
    alen = rng.integers(1, 6, size=B).astype(np.int32)
    an = np.tile(np.arange(Q, dtype=np.int32), (B, 1))
    o1 = oracle.kv_commit(r2s, plen, nn, alen, an)
    o2 = oracle.kv_commit(o1["req_to_slot"], o1["prefix_len"], nn, alen, an)
    d_r2s, d_plen = dev(r2s), dev(plen)
    args = (dev(nn), dev(alen), dev(an))
    ddt.kv_commit(d_r2s, d_plen, *args)
    g2 = ddt.kv_commit(d_r2s, d_plen, *args)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d_r2s.cpu().numpy(), o2["req_to_slot"])
    np.testing.assert_array_equal(d_plen.cpu().numpy(), o2["prefix_len"])
    np.testing.assert_array_equal(g2["freed_slots"].cpu().numpy(), o2["freed_slots"])
    np.testing.assert_array_equal(g2["n_freed"].cpu().numpy(), o2["n_freed"])


@pytest.mark.parametrize("slack", [-3, 0, 1, 5])
def test_step_at_slot_table_capacity(slack):
    """A verify step whose longest tree ends exactly at the slot table's capacity
    (slack 0: L_b + n_b = max_kv), short of it, or past it (slack -3, against the
    stated precondition): attention against the oracle, accept bit-exact, and the
    commit bit-exact.  Attention and commit clamp an overrunning tree to
    max_kv - L_b alike; accept does not see max_kv, and the commit cuts the path
    at the clamp.  Requests that fit commit their whole accepted path."""
    note(f"capacity edge slack={slack}")
    wl = workloads.make_workload("b4_l4k_q33", L=700)
    t = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
    need = wl.prefix_len.astype(np.int64) + t["n_nodes"]
    max_kv = int(need.max()) + slack
    r2s = np.ascontiguousarray(wl.req_to_slot[:, :max_kv])
    tgt = workloads.synth_target_argmax(wl, t["node_token"], t["parent"], t["depth"],
                                        t["n_nodes"])
    # attention on the clamped table
    f = lambda x: x.float().numpy()
    o_out, o_lse = oracle.verify_attn(f(wl.q_lat), f(wl.q_pe), f(wl.c_kv), f(wl.k_pe), r2s,
                                      wl.prefix_len, t["n_nodes"], t["vis"], wl.sm_scale)
    tdev = lambda x: x.contiguous().cuda()
    g_out, g_lse = ddt.verify_attn(tdev(wl.q_lat), tdev(wl.q_pe), tdev(wl.c_kv), tdev(wl.k_pe),
                                   dev(r2s), dev(wl.prefix_len), dev(t["n_nodes"]),
                                   dev(t["vis"].view(np.int64)), wl.sm_scale)
    torch.cuda.synchronize()
    err = float(np.abs(g_out.cpu().numpy().astype(np.float64) - o_out).max())
    assert err <= 2e-3, err
    # accept, then commit into the table
    oa = oracle.tree_accept(t["node_token"], t["parent"], t["n_nodes"], tgt)
    acc = ddt.tree_accept(dev(t["node_token"]), dev(t["parent"]), dev(t["n_nodes"]), dev(tgt))
    torch.cuda.synchronize()
    for k in oa:
        np.testing.assert_array_equal(acc[k].cpu().numpy(), oa[k], err_msg=k)
    oc = oracle.kv_commit(r2s, wl.prefix_len, t["n_nodes"], oa["accept_len"], oa["accept_nodes"])
    gc = gpu_commit(r2s, wl.prefix_len, t["n_nodes"], oa["accept_len"], oa["accept_nodes"])
    assert_same(gc, oc)
    assert (oc["prefix_len"] <= max_kv).all()
    fits = need <= max_kv
    assert fits.any() and (slack < 0) == (not fits.all())
    np.testing.assert_array_equal(oc["prefix_len"][fits], (wl.prefix_len + oa["accept_len"])[fits])
