"""GPU parity of ddt_draft_topk (through its C ABI) against the CPU oracle.

ids bit-exact; log-probs within 1e-5 (fp32 accumulation of up to 2^20 exp
terms and the fp32 log stay about 1e-6 from the exact value: the bound the
entry point documents, with margin); -inf exactly where the oracle has it.
Outputs are pre-filled with sentinels, so every element must be written.
Cases: the drafter shapes of the workloads at full vocabulary (160000, bf16),
fp32 and bf16 rows with ties, -inf and NaN entries, an unaligned vocabulary,
K = 1 and K = 64, all -inf rows, and chunks shorter than K.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import tree_verify_mla_ddt_amd as ddt

pytestmark = pytest.mark.gpu
TOL = 1e-5


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ddt.load_library()
    yield


def check(x, K):
    """x: CPU tensor [B,D,V] (f32 or bf16)."""
    B, D, V = x.shape
    out = {"topk_logp": torch.full((B, D, K), float("nan"), device="cuda", dtype=torch.float32),
           "topk_ids": torch.full((B, D, K), -77, device="cuda", dtype=torch.int32)}
    ddt.draft_topk(x.contiguous().cuda(), K, out=out)
    torch.cuda.synchronize()
    o = oracle.draft_topk(x, K)
    np.testing.assert_array_equal(out["topk_ids"].cpu().numpy(), o["topk_ids"])
    g = out["topk_logp"].cpu().numpy().astype(np.float64)
    fin = np.isfinite(o["topk_logp"])
    np.testing.assert_array_equal(np.isfinite(g), fin)
    assert (g[~fin] == -np.inf).all()
    err = np.abs(g[fin] - o["topk_logp"][fin]).max() if fin.any() else 0.0
    assert err <= TOL, err
    return err


@pytest.mark.parametrize("B,D,K", [(1, 8, 8), (4, 15, 8), (64, 8, 8), (8, 15, 16)])
def test_workload_drafter_shapes(B, D, K):
    """The drafter side of the workloads: D depths x V = 160000 bf16 logits."""
    note(f"draft_topk B={B} D={D} K={K} V=160000 bf16")
    g = torch.Generator().manual_seed(B * 100 + D)
    x = (torch.randn(B, D, 160000, generator=g, dtype=torch.float32) * 2).to(torch.bfloat16)
    check(x, K)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V,K", [(512, 4), (4099, 8), (70, 64), (8, 8), (9, 1), (20000, 33),
                                 (1048576, 64)])
def test_shapes_ties_and_masks(dtype, V, K):
    note(f"draft_topk V={V} K={K} {dtype}")
    rng = np.random.default_rng(V + K)
    B, D = 2, 3
    x = torch.tensor(rng.normal(0, 2, size=(B, D, V)), dtype=torch.float32).to(dtype)
    x[0, 0, :min(V, 37)] = float("-inf")          # masked entries
    if V > 50:
        x[0, 1, 40] = float("nan")
        x[1, 0, : V // 2] = 1.25                      # a wide tie
    x[1, 2] = float("-inf")                           # an all -inf row
    check(x, K)


def test_equal_logits_and_signed_zero():
    x = torch.zeros(1, 2, 3000, dtype=torch.float32)
    x[0, 1, ::2] = -0.0
    check(x, 16)
