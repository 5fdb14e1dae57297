"""The first attention calls of a process made under HIP graph capture.

Two things in the launch path are set up on first use: the wide merge's grid
bound (the runtime's occupancy figure for the compiled kernel) and, for
ddt_verify_attn_noalloc, the device address of the static scratch array.  A
caller that captures before ever calling eagerly runs that set-up inside the
capture.  A child process (so that nothing is set up yet) captures one
ddt_verify_attn call with a batch that takes the wide merge and one
ddt_verify_attn_noalloc call, replays each graph three times with other work
in between, and compares every replay bit for bit with an eager call made
afterwards."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys
import numpy as np
import torch
sys.path.insert(0, ROOT)
import tree_verify_mla_ddt_amd as ddt
from tree_verify_mla_ddt_amd import workloads
import oracle

def dev(a):
    return torch.as_tensor(a).contiguous().cuda()

wl = workloads.make_workload("b4_l4k_q17")
t = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
args = (dev(wl.q_lat), dev(wl.q_pe), dev(wl.c_kv), dev(wl.k_pe), dev(wl.req_to_slot),
        dev(wl.prefix_len), dev(t["n_nodes"]), dev(t["vis"].view(np.int64)), wl.sm_scale)
B, Q, H = wl.B, wl.Q, wl.H
ws = torch.empty((ddt.workspace_size(B, Q, H, wl.req_to_slot.shape[1], wl.d_lat),),
                 dtype=torch.uint8, device="cuda")
torch.cuda.synchronize()
results = {}
for name, fn, kw in (("verify_attn", ddt.verify_attn, {"workspace": ws}),
                     ("verify_attn_noalloc", ddt.verify_attn_noalloc, {})):
    out = torch.full((B, Q, H, wl.d_lat), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, Q, H), float("nan"), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn(*args, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    reps = []
    for _ in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        reps.append((out.cpu().numpy().copy(), lse.cpu().numpy().copy()))
    results[name] = reps
o_e, l_e = ddt.verify_attn(*args)
torch.cuda.synchronize()
o_e, l_e = o_e.cpu().numpy(), l_e.cpu().numpy()
for name, reps in results.items():
    for k, (o, l) in enumerate(reps):
        assert np.array_equal(o, o_e, equal_nan=False), (name, k, "out")
        assert np.array_equal(l, l_e, equal_nan=False), (name, k, "lse")
print("CAPTURE-FIRST OK", flush=True)
'''


def test_first_calls_under_capture():
    code = "ROOT = %r\n" % ROOT + CHILD
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=300)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0 and "CAPTURE-FIRST OK" in r.stdout, tail
