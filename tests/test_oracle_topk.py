"""Pins for the oracle's per-depth top-K extraction.

What it computes ("The Architecture of a Thousand-Parameter Decision ...",
"What to Build New", item 4: per-depth top-k logit extraction, the input of the
tree builder): per (request, depth) row of drafter logits, the log-softmax over
the vocabulary and the K largest logits (largest first, lower index first among
equal logits).

Checked against:
* library routines it does not use itself: numpy's stable argsort on (-logit,
  index) for the ids and scipy's logsumexp for the normaliser;
* closed forms: equal logits give log(1/V) and ids 0..K-1; K = V covers the row
  and its probabilities sum to 1;
* shift invariance of the log-probs and ids; -inf entries never chosen while
  enough finite ones remain; a row of -inf gives -inf log-probs.
"""
import numpy as np
import pytest
import scipy.special
import torch

import oracle


def reference(x, K):
    x = np.where(np.isnan(x), -np.inf, x.astype(np.float64))
    lse = scipy.special.logsumexp(x, axis=-1, keepdims=True)
    order = np.argsort(-x, axis=-1, kind="stable")[..., :K]
    return np.take_along_axis(x, order, -1) - lse, order


@pytest.mark.parametrize("B,D,V,K,seed", [(1, 4, 512, 4, 0), (2, 8, 4099, 8, 1),
                                          (3, 3, 160000, 16, 2), (1, 2, 70, 64, 3)])
def test_matches_sort_and_logsumexp(B, D, V, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 2, size=(B, D, V)).astype(np.float32)
    o = oracle.draft_topk(x, K)
    lp, ids = reference(x, K)
    np.testing.assert_array_equal(o["topk_ids"], ids)
    np.testing.assert_allclose(o["topk_logp"], lp, rtol=0, atol=1e-12)


def test_bf16_ties_break_by_index():
    rng = np.random.default_rng(5)
    x = torch.tensor(rng.normal(0, 1, size=(2, 3, 3000)), dtype=torch.bfloat16)  # many ties
    o = oracle.draft_topk(x, 32)
    lp, ids = reference(x.float().numpy(), 32)
    np.testing.assert_array_equal(o["topk_ids"], ids)
    np.testing.assert_allclose(o["topk_logp"], lp, rtol=0, atol=1e-12)


def test_equal_logits():
    V, K = 1000, 7
    o = oracle.draft_topk(np.full((1, 1, V), 3.5, np.float32), K)
    np.testing.assert_array_equal(o["topk_ids"][0, 0], np.arange(K))
    np.testing.assert_allclose(o["topk_logp"][0, 0], -np.log(V), rtol=0, atol=1e-14)


def test_full_row_sums_to_one_and_shift_invariance():
    rng = np.random.default_rng(7)
    x = rng.normal(0, 3, size=(1, 2, 64)).astype(np.float32)
    o = oracle.draft_topk(x, 64)
    np.testing.assert_allclose(np.exp(o["topk_logp"]).sum(-1), 1.0, rtol=1e-13)
    assert (np.diff(o["topk_logp"], axis=-1) <= 0).all()
    o2 = oracle.draft_topk(x + np.float32(8.0), 64)  # exact in fp32 at this range
    np.testing.assert_array_equal(o2["topk_ids"], o["topk_ids"])
    np.testing.assert_allclose(o2["topk_logp"], o["topk_logp"], rtol=0, atol=1e-5)


def test_minus_inf_and_nan():
    V, K = 50, 4
    x = np.full((1, 2, V), -np.inf, np.float32)
    x[0, 0, [3, 17, 40]] = [1.0, 2.0, 1.0]
    x[0, 0, 5] = np.nan
    o = oracle.draft_topk(x, K)
    # Three finite entries, then the lowest-index -inf one (the NaN counts as -inf).
    np.testing.assert_array_equal(o["topk_ids"][0, 0], [17, 3, 40, 0])
    assert o["topk_logp"][0, 0, 3] == -np.inf
    np.testing.assert_array_equal(o["topk_ids"][0, 1], np.arange(K))
    assert (o["topk_logp"][0, 1] == -np.inf).all()
