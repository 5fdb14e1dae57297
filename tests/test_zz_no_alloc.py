"""ddt_verify_attn_noalloc (static scratch array) against ddt_verify_attn
(caller workspace): the same kernels, so the outputs must agree bit for bit, on
two calls in a row, the second with a smaller input."""
import numpy as np
import pytest
import torch

import tree_verify_mla_ddt_amd as ddt
from tree_verify_mla_ddt_amd import workloads

import oracle

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.as_tensor(a).contiguous().cuda()


def inputs(name, **overrides):
    wl = workloads.make_workload(name, **overrides)
    t = oracle.tree_build(wl.topk_logp, wl.topk_ids, wl.root_token, wl.prefix_len, wl.budget)
    return wl, (dev(wl.q_lat), dev(wl.q_pe), dev(wl.c_kv), dev(wl.k_pe), dev(wl.req_to_slot),
                dev(wl.prefix_len), dev(t["n_nodes"]), dev(t["vis"].view(np.int64)),
                wl.sm_scale)


def run_both(wl, args):
    B, Q, H = wl.B, wl.Q, wl.H
    outs = []
    for fn in (ddt.verify_attn, ddt.verify_attn_noalloc):
        out = torch.full((B, Q, H, wl.d_lat), float("nan"), dtype=torch.float32, device="cuda")
        lse = torch.full((B, Q, H), float("nan"), dtype=torch.float32, device="cuda")
        fn(*args, out=out, lse=lse)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), lse.cpu().numpy()))
    return outs


def check_equal(a, b, label):
    (o1, l1), (o2, l2) = a, b
    assert np.isfinite(o1).all(), label
    np.testing.assert_array_equal(o2.view(np.uint32), o1.view(np.uint32), err_msg=label)
    np.testing.assert_array_equal(l2.view(np.uint32), l1.view(np.uint32), err_msg=label)


@pytest.mark.parametrize("first,second", [
    # aligned split over the whole grid (largest scratch use), then a smaller
    # linear-split call that reads fewer slots of the same array
    (("b64_l2k_q9", {}), ("b4_l4k_q17", {"L": 900})),
    # the bf16 64+16 and fp32 64+16 kernels
    (("tiny_fp32", {"dtype": "bf16", "B": 3, "H": 16, "L": 300, "budget": 70, "D": 9, "K": 4}),
     ("tiny_fp32", {})),
])
def test_noalloc_matches_workspace_call(first, second):
    for name, ov in (first, second):
        print(f"[noalloc] {name} {ov}", flush=True)
        wl, args = inputs(name, **ov)
        a, b = run_both(wl, args)
        check_equal(a, b, f"{name} {ov}")


def test_noalloc_max_bytes_covers_every_plan():
    lib = ddt.load_library()
    cap = int(lib.ddt_verify_attn_noalloc_max_bytes())
    assert cap >= int(lib.ddt_verify_attn_workspace_size(512, 128, 128, 1 << 20, 512))
