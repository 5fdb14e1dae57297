"""A pair wait that gives up is visible in the result.

The pair kernel (the 64+16 variants) synchronises the two waves of a pair with a
bounded wait.  Run with DDT_PAIR_SPIN_LIMIT=0 every wait gives up at once (and
still ends); the live rows must then come out as NaN and the call must return
normally.  Runs in a child process so that the limit applies from the library's
first call."""
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, numpy as np, torch
sys.path.insert(0, sys.argv[1])
import oracle
import tree_verify_mla_ddt_amd as ddt
from tree_verify_mla_ddt_amd import workloads
wl = workloads.make_workload("tiny_fp32")
t = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
dev = lambda a: torch.as_tensor(a).contiguous().cuda()
out, lse = ddt.verify_attn(dev(wl.q_lat), dev(wl.q_pe), dev(wl.c_kv), dev(wl.k_pe),
                           dev(wl.req_to_slot), dev(wl.prefix_len), dev(t["n_nodes"]),
                           dev(t["vis"].view(np.int64)), wl.sm_scale)
torch.cuda.synchronize()
o = out.cpu().numpy()
n = int(t["n_nodes"][0])
live = o[0, :n]
print("nan rows", int(np.isnan(live).any(axis=-1).sum()), "of", live.shape[0] * live.shape[1])
assert np.isnan(live).any(axis=-1).all(), "a give-up passed as a result"
print("ok")
"""


def test_pair_wait_give_up_poisons_rows():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    env = dict(os.environ, DDT_PAIR_SPIN_LIMIT="0")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], env=env, capture_output=True,
                       text=True, timeout=120)
    print(r.stdout, r.stderr[-2000:])
    assert r.returncode == 0 and "ok" in r.stdout
