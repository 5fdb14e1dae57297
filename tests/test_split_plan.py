"""The verify-attention work split, checked on the CPU.

libddt_split_check.so runs the split arithmetic the attention and merge kernels
call (attn_split.h) for every workgroup of a launch and checks that every tile
with work is taken exactly once, that partial results land in distinct
workspace slots inside the workspace, and that the merge's contributor rule
names exactly the slots written for each cut row tile (see
csrc/split_check.hip).  Swept over batch sizes, tree sizes, head counts,
ragged and clamped prefix lengths and compute-unit counts, including every
benchmark shape and the launches that take the aligned split."""
import ctypes
import os

import numpy as np
import pytest

from tree_verify_mla_ddt_amd import build as libbuild
from tree_verify_mla_ddt_amd import workloads


@pytest.fixture(scope="module")
def checker():
    if not os.path.exists(libbuild.CHECK_PATH):
        libbuild.build_split_check()
    lib = ctypes.CDLL(libbuild.CHECK_PATH)
    lib.ddt_split_check.argtypes = [ctypes.c_int] * 4 + [ctypes.c_void_p] * 2 + \
        [ctypes.c_int] * 3 + [ctypes.c_char_p, ctypes.c_int, ctypes.c_void_p]
    lib.ddt_split_check.restype = ctypes.c_int
    return lib


def run(lib, plen, nn, Q, H, max_kv, num_cu=256, d_lat=512, plant=0, stats=None):
    plen = np.ascontiguousarray(plen, np.int32)
    nn = np.ascontiguousarray(nn, np.int32)
    msg = ctypes.create_string_buffer(256)
    st = np.zeros(5, np.int64)
    rc = lib.ddt_split_check(len(plen), Q, H, max_kv, plen.ctypes.data, nn.ctypes.data, num_cu,
                             d_lat, plant, msg, 256, st.ctypes.data)
    if stats is not None:
        stats[:] = st
    return rc, msg.value.decode()


def check(lib, plen, nn, Q, H, max_kv, num_cu=256, d_lat=512):
    st = np.zeros(5, np.int64)
    rc, msg = run(lib, plen, nn, Q, H, max_kv, num_cu, d_lat, stats=st)
    assert rc == 0, (msg, len(plen), Q, H, max_kv, num_cu)
    return st


@pytest.mark.parametrize("name", list(workloads.CONFIGS))
def test_benchmark_shapes(checker, name):
    import oracle
    wl = workloads.make_workload(name, with_kv=False)
    t = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
    for cu in (256, 304, 80):
        check(checker, wl.prefix_len, t["n_nodes"], wl.Q, wl.H, int(wl.prefix_len.max()) + wl.Q,
              cu, wl.d_lat)


def test_random_shapes(checker):
    rng = np.random.default_rng(123)
    seen = np.zeros(3, np.int64)  # start cost charged, ranges ending inside one, ranges over 2+ tiles
    for case in range(1500):
        B = int(rng.choice([1, 2, 3, 4, 7, 8, 16, 33, 64, 100, 512]))
        Q = int(rng.choice([1, 2, 9, 17, 33, 65, 100, 128]))
        H = int(rng.choice([1, 3, 4, 8, 16, 64, 128]))
        Lmax = int(rng.choice([0, 1, 31, 32, 33, 300, 2048, 5000, 40000]))
        kind = case % 4
        if kind == 0:      # uniform requests, full trees (aligned split when it fits)
            plen = np.full(B, Lmax)
            nn = np.full(B, Q)
        elif kind == 1:    # ragged prefixes
            plen = rng.integers(0, Lmax + 1, size=B)
            nn = np.full(B, Q)
        elif kind == 2:    # ragged trees, some empty or clamped
            plen = np.full(B, Lmax)
            nn = rng.integers(-2, Q + 3, size=B)
        else:              # lengths past max_kv and negative (clamped)
            plen = rng.integers(-5, Lmax + 50, size=B)
            nn = rng.integers(0, Q + 1, size=B)
        max_kv = max(1, Lmax + Q - int(rng.integers(0, 3)))
        cu = int(rng.choice([256, 256, 304, 120, 64, 1024]))
        st = check(checker, plen, nn, Q, H, max_kv, cu, int(rng.choice([64, 512])))
        seen += [st[0] > 0, st[1], st[2]]
    assert (seen > 0).all(), seen


def test_start_cost_balances_ranges(checker):
    """Ragged batch-4 requests (4096 +-25% keys, 17 tree nodes, 64 heads): the
    ranges cross row tiles, so starting one is charged; no range then carries
    more than its share of the stream plus one start cost, counting a start
    cost for every row tile it begins; with requests of equal length cut into
    whole multiples of the row-tile count nothing is charged."""
    rng = np.random.default_rng(7)
    for _ in range(20):
        plen = rng.integers(3072, 5121, size=4)
        st = check(checker, plen, [17] * 4, 17, 64, int(plen.max()) + 17)
        assert st[0] == 6 and st[2] > 0
        assert st[3] <= st[4] + st[0], st
    st = check(checker, [2048], [9], 9, 64, 2057)
    assert st[0] == 0 and st[2] == 0


@pytest.mark.parametrize("plant", [1, 2])
def test_planted_mistake_is_caught(checker, plant):
    """The same check with a mistake planted in the merge's contributor rule
    (head and tail slots swapped; the last contributor dropped) fails on
    shapes with cut row tiles: batch 1 (linear split) and the max shape
    (aligned split's leftover tiles)."""
    for plen, nn, Q, H in (([2048], [9], 9, 64), ([32768] * 8, [65] * 8, 65, 64)):
        rc, msg = run(checker, plen, nn, Q, H, max(plen) + Q, plant=plant)
        assert rc != 0 and "contributors" in msg, (plant, msg)


def plan(lib, B, Q, H, max_kv, d_lat=512, num_cu=256):
    lib.ddt_split_plan.argtypes = [ctypes.c_int] * 6 + [ctypes.c_void_p] * 4
    g, nar, rt = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    ws = ctypes.c_ulonglong()
    lib.ddt_split_plan(B, Q, H, max_kv, d_lat, num_cu, ctypes.byref(g), ctypes.byref(nar),
                       ctypes.byref(rt), ctypes.byref(ws))
    return g.value, bool(nar.value), rt.value, ws.value


@pytest.mark.parametrize("B,Q,H,L,narrow", [
    (1, 9, 64, 2048, True),      # 5 row tiles: quarter workgroups
    (3, 9, 64, 2048, True),      # 15 row tiles
    (4, 17, 64, 5120, False),    # 36 row tiles: the 128-row form
    (4, 33, 64, 5120, False),
    (64, 9, 64, 2048, False),
    (8, 65, 64, 32768, False),
    (64, 9, 8, 2048, False),     # the 8-head share: one row tile per request
    (16, 9, 8, 2048, True),
])
def test_narrow_form_choice(checker, B, Q, H, L, narrow):
    g, nar, rt, ws = plan(checker, B, Q, H, L + Q)
    assert nar == narrow
    assert 1 <= g <= (64 if nar else 256)
    assert (not nar) or B * rt * 16 <= 256
    assert ws == 2 * g * 128 * 513 * 4 + (B + 3) * 8
    # the 64-wide latent form never takes it
    assert not plan(checker, B, Q, H, L + Q, d_lat=64)[1]
