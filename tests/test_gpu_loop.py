"""Multi-step DDTree loop on the HIP library: every step runs build -> verify
attention -> accept -> KV commit on the device (the synthetic target is
computed on the host between accept's inputs and the tree, as a model would
be); the sequences equal autoregressive greedy decoding with the same target,
and every step's slot table, prefix lengths and accept lengths equal the CPU
oracle's loop on the same seeds (see loop_harness)."""
import sys

import numpy as np
import pytest
import torch

import tree_verify_mla_ddt_amd as ddt
from loop_harness import ar_continue, run_loop
from test_oracle_loop import OracleBackend

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ddt.load_library()
    yield


def dev(a):
    return torch.as_tensor(np.ascontiguousarray(a)).contiguous().cuda()


class GpuBackend:
    """The library's entry points on device buffers; numpy in and out."""

    def __init__(self, B, H=4, d_lat=64, d_rope=16, pool=4096, seed=7):
        g = torch.Generator().manual_seed(seed)
        f32 = torch.float32  # explicit: another test module changes torch's default dtype
        self.c_kv = torch.randn(pool, d_lat, generator=g, dtype=f32).cuda()
        self.k_pe = torch.randn(pool, d_rope, generator=g, dtype=f32).cuda()
        self.H, self.d_lat, self.d_rope = H, d_lat, d_rope

    def build(self, logp, ids, root, plen, budget):
        t = ddt.tree_build(dev(logp), dev(ids), dev(root), dev(plen), budget)
        self.tree_dev = t
        torch.cuda.synchronize()
        out = {k: v.cpu().numpy() for k, v in t.items()}
        out["vis"] = out["vis"].view(np.uint64)
        return out

    def verify(self, r2s, plen, tree):
        B, Q = tree["node_token"].shape
        q_lat = torch.randn(B, Q, self.H, self.d_lat, device="cuda", dtype=torch.float32)
        q_pe = torch.randn(B, Q, self.H, self.d_rope, device="cuda", dtype=torch.float32)
        out, lse = ddt.verify_attn(q_lat, q_pe, self.c_kv, self.k_pe, dev(r2s), dev(plen),
                                   self.tree_dev["n_nodes"], self.tree_dev["vis"],
                                   1.0 / np.sqrt(self.d_lat + self.d_rope))
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()

    def accept(self, tree, tgt):
        t = self.tree_dev
        a = ddt.tree_accept(t["node_token"], t["parent"], t["n_nodes"], dev(tgt))
        self.acc_dev = a
        torch.cuda.synchronize()
        return {k: v.cpu().numpy() for k, v in a.items()}

    def commit(self, r2s, plen, n, alen, anodes):
        d_r2s, d_plen = dev(r2s), dev(plen)
        c = ddt.kv_commit(d_r2s, d_plen, self.tree_dev["n_nodes"], self.acc_dev["accept_len"],
                          self.acc_dev["accept_nodes"])
        torch.cuda.synchronize()
        return (d_r2s.cpu().numpy(), d_plen.cpu().numpy(), c["freed_slots"].cpu().numpy(),
                c["n_freed"].cpu().numpy())


@pytest.mark.parametrize("seed,p_hit,K,D,budget,B", [(0, 0.75, 4, 6, 12, 3), (1, 0.95, 3, 8, 8, 5),
                                                     (2, 0.3, 5, 4, 16, 2), (4, 0.8, 8, 15, 64, 2)])
def test_gpu_loop_matches_ar_and_oracle(seed, p_hit, K, D, budget, B):
    print(f"gpu loop seed={seed} K={K} D={D} budget={budget} B={B}", flush=True)
    sys.stdout.flush()
    kw = dict(steps=20, B=B, K=K, D=D, budget=budget, vocab=509, p_hit=p_hit, seed=seed)
    seqs_g, rec_g = run_loop(GpuBackend(B), **kw)
    seqs_o, rec_o = run_loop(OracleBackend(), **kw)
    assert seqs_g == seqs_o
    for s in seqs_g:
        assert s == ar_continue(s[:20], len(s) - 20, 509)
    for rg, ro in zip(rec_g, rec_o):
        for k in ("accept_len", "plen", "r2s"):
            np.testing.assert_array_equal(rg[k], ro[k], err_msg=k)
