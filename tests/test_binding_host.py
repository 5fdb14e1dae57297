"""The binding refuses host tensors before it reaches the C ABI (which takes
device pointers): every entry point raises on CPU tensors, without a GPU."""
import pytest
import torch

import tree_verify_mla_ddt_amd as ddt


def c(shape, dtype=torch.int32):
    return torch.zeros(shape, dtype=dtype)


def test_entry_points_reject_host_tensors():
    B, Q, D, K, H, dl, dr, L = 2, 9, 4, 4, 4, 64, 16, 40
    S = B * (L + Q)
    f = torch.float32
    with pytest.raises(ValueError, match="GPU tensor"):
        ddt.tree_build(c((B, D, K), f), c((B, D, K)), c((B,)), c((B,)), Q - 1)
    with pytest.raises(ValueError, match="GPU tensor"):
        ddt.verify_attn(c((B, Q, H, dl), f), c((B, Q, H, dr), f), c((S, dl), f), c((S, dr), f),
                        c((B, L + Q)), c((B,)), c((B,)), c((B, Q, 1), torch.int64), 0.1)
    with pytest.raises(ValueError, match="GPU tensor"):
        ddt.verify_attn_noalloc(c((B, Q, H, dl), f), c((B, Q, H, dr), f), c((S, dl), f),
                                c((S, dr), f), c((B, L + Q)), c((B,)), c((B,)),
                                c((B, Q, 1), torch.int64), 0.1)
    with pytest.raises(ValueError, match="GPU tensor"):
        ddt.verify_attn_kernel_times(c((B, Q, H, dl), f), c((B, Q, H, dr), f), c((S, dl), f),
                                     c((S, dr), f), c((B, L + Q)), c((B,)), c((B,)),
                                     c((B, Q, 1), torch.int64), 0.1, reps=1)
    with pytest.raises(ValueError, match="GPU tensor"):
        ddt.tree_accept(c((B, Q)), c((B, Q)), c((B,)), c((B, Q)))
    with pytest.raises(ValueError, match="GPU tensor"):
        ddt.kv_commit(c((B, L + Q)), c((B,)), c((B,)), c((B,)), c((B, Q)))
    with pytest.raises(ValueError, match="GPU tensor"):
        ddt.draft_topk(c((B, D, 512), f), K)
    with pytest.raises(ValueError, match="GPU tensor"):
        ddt.tree_accept_sampling(c((B, Q, 512), f), c((B,), f), c((B, Q)), c((B, Q)), c((B,)),
                                 c((B, Q), f), c((B,), f))


def test_wrong_types_rejected_first():
    with pytest.raises(TypeError):
        ddt.tree_accept([0], c((1, 1)), c((1,)), c((1, 1)))
    with pytest.raises(TypeError):
        ddt.verify_attn(c((1, 1, 1, 64), torch.float16), *[None] * 7, 0.1)
