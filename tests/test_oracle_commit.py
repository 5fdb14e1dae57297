"""Pins for the oracle's KV commit after acceptance.

What it computes ("The Architecture of a Thousand-Parameter Decision ...",
"What to Build New", item 5: the paged latent KV cache and the append step of
each DDTree step; "The Milestone Message ...", "Architectural Abstraction":
tree entries sit at positions L + depth): with one token per page the accepted
root path is committed by rewriting the request's slot table -- path node j
becomes prefix entry L + j, the other tree nodes' slots are released.

Checked against:
* closed forms: a chain accepted in full leaves the table as it was and grows
  the prefix by n; a root-only accept keeps entry L and releases every other
  tree slot in node order; an empty path commits nothing;
* the positions the pages fix: on every workload, for trees and targets from
  the oracle's own builder and acceptance, path node j has depth j, so its KV
  (written at L + depth) already sits at the prefix entry it is committed to;
* conservation: committed slots and released slots together are exactly the
  tree's slots, each once; entries outside the tree are untouched;
* malformed paths (an index outside the tree, a repeated or decreasing index)
  are cut before the first bad entry.
"""
import numpy as np
import pytest

import oracle
from tree_verify_mla_ddt_amd import workloads


def commit1(row, L, n, path, Q):
    """One request: row = slot table, path = accepted node list (len = accept_len)."""
    an = np.full((1, Q), -1, np.int32)
    an[0, :len(path)] = path
    return oracle.kv_commit(np.array([row], np.int32), np.array([L], np.int32),
                            np.array([n], np.int32), np.array([len(path)], np.int32), an)


def test_chain_full_accept_is_identity():
    Q, L, n, max_kv = 9, 5, 9, 20
    row = np.arange(100, 100 + max_kv, dtype=np.int32)
    r = commit1(row, L, n, list(range(n)), Q)
    np.testing.assert_array_equal(r["req_to_slot"][0], row)
    assert r["prefix_len"][0] == L + n
    assert r["n_freed"][0] == 0
    assert (r["freed_slots"][0] == -1).all()


def test_root_only_releases_rest_in_order():
    Q, L, n, max_kv = 9, 3, 7, 16
    rng = np.random.default_rng(1)
    row = rng.permutation(1000)[:max_kv].astype(np.int32)
    r = commit1(row, L, n, [0], Q)
    out = r["req_to_slot"][0]
    assert out[L] == row[L]
    assert (out[L + 1:L + n] == -1).all()
    np.testing.assert_array_equal(out[:L], row[:L])
    np.testing.assert_array_equal(out[L + n:], row[L + n:])
    assert r["prefix_len"][0] == L + 1
    assert r["n_freed"][0] == n - 1
    np.testing.assert_array_equal(r["freed_slots"][0][:n - 1], row[L + 1:L + n])
    assert (r["freed_slots"][0][n - 1:] == -1).all()


def test_empty_path_commits_nothing():
    Q, L, n, max_kv = 5, 2, 4, 8
    row = np.arange(max_kv, dtype=np.int32) + 7
    r = commit1(row, L, n, [], Q)
    assert r["prefix_len"][0] == L
    assert (r["req_to_slot"][0][L:L + n] == -1).all()
    np.testing.assert_array_equal(r["freed_slots"][0][:n], row[L:L + n])


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_workload_paths_land_at_their_positions(name):
    wl = workloads.make_workload(name, L=min(workloads.CONFIGS[name]["L"], 3000))
    t = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
    tgt = workloads.synth_target_argmax(wl, t["node_token"], t["parent"], t["depth"],
                                        t["n_nodes"])
    a = oracle.tree_accept(t["node_token"], t["parent"], t["n_nodes"], tgt)
    r = oracle.kv_commit(wl.req_to_slot, wl.prefix_len, t["n_nodes"], a["accept_len"],
                         a["accept_nodes"])
    for b in range(wl.B):
        L, n, k = int(wl.prefix_len[b]), int(t["n_nodes"][b]), int(a["accept_len"][b])
        path = a["accept_nodes"][b][:k]
        # The position the verify step wrote each path node's KV at is the
        # prefix entry it is committed to.
        np.testing.assert_array_equal(t["depth"][b][path], np.arange(k))
        np.testing.assert_array_equal(t["position"][b][path], L + np.arange(k))
        old = wl.req_to_slot[b]
        new = r["req_to_slot"][b]
        np.testing.assert_array_equal(new[L:L + k], old[L + path])
        assert (new[L + k:L + n] == -1).all()
        np.testing.assert_array_equal(new[:L], old[:L])
        np.testing.assert_array_equal(new[L + n:], old[L + n:])
        assert r["prefix_len"][b] == L + k
        # Conservation: committed + released = the tree's slots, each once.
        freed = r["freed_slots"][b][:r["n_freed"][b]]
        assert r["n_freed"][b] == n - k
        assert sorted(np.concatenate([new[L:L + k], freed]).tolist()) == \
            sorted(old[L:L + n].tolist())
        # Released in node order: their tree indices increase.
        pos = {int(s): i for i, s in enumerate(old[L:L + n])}
        idx = [pos[int(s)] for s in freed]
        assert idx == sorted(idx)


@pytest.mark.parametrize("path,cut", [([0, 2, 9, 3], 2),    # 9 is outside the tree (n = 6)
                                      ([0, 2, 2, 4], 2),    # repeated index
                                      ([0, 3, 1], 2),       # decreasing index
                                      ([-1, 1], 0),         # negative first entry
                                      ([0, 1, 4, 5], 4)])   # valid
def test_malformed_paths_are_cut(path, cut):
    Q, L, n, max_kv = 8, 4, 6, 12
    row = np.arange(max_kv, dtype=np.int32) * 3 + 1
    r = commit1(row, L, n, path, Q)
    assert r["prefix_len"][0] == L + cut
    np.testing.assert_array_equal(r["req_to_slot"][0][L:L + cut], row[L + np.array(path[:cut],
                                                                                   dtype=int)])
    assert r["n_freed"][0] == n - cut


def test_clamps():
    # prefix_len past max_kv and n_nodes past the room left: nothing to commit.
    Q, max_kv = 4, 6
    row = np.arange(max_kv, dtype=np.int32)
    an = np.array([[0, 1, 2, 3]], np.int32)
    r = oracle.kv_commit(np.array([row]), np.array([9], np.int32), np.array([4], np.int32),
                         np.array([4], np.int32), an)
    assert r["prefix_len"][0] == max_kv
    np.testing.assert_array_equal(r["req_to_slot"][0], row)
    assert r["n_freed"][0] == 0
    # n_nodes larger than the room: clamped to max_kv - L = 2.
    r = oracle.kv_commit(np.array([row]), np.array([4], np.int32), np.array([4], np.int32),
                         np.array([4], np.int32), an)
    assert r["prefix_len"][0] == 6
    np.testing.assert_array_equal(r["req_to_slot"][0], row)
