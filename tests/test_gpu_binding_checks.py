"""The Python binding rejects ill-shaped, mistyped or misplaced tensors before
any kernel is launched: caller-supplied outputs, out-dict entries, workspaces
and per-request arrays are checked against the shapes the call implies."""
import pytest
import torch

import tree_verify_mla_ddt_amd as ddt

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ddt.load_library()
    yield


def z(shape, dtype=torch.int32):
    return torch.zeros(shape, dtype=dtype, device="cuda")


def test_tree_build_rejects():
    B, D, K, budget = 3, 4, 4, 8
    args = [z((B, D, K), torch.float32), z((B, D, K)), z((B,)), z((B,))]
    ddt.tree_build(*args, budget)
    with pytest.raises(ValueError):
        ddt.tree_build(args[0], args[1], args[2], z((B + 1,)), budget)
    with pytest.raises(ValueError):
        ddt.tree_build(args[0], z((B, D, K + 1)), args[2], args[3], budget)
    out = ddt.tree_build(*args, budget)
    out["vis"] = z((B, budget + 1, 2), torch.int64)       # wrong bitset width
    with pytest.raises(ValueError):
        ddt.tree_build(*args, budget, out=out)
    out = ddt.tree_build(*args, budget)
    out["score"] = z((B, budget + 1), torch.int32)         # wrong dtype
    with pytest.raises(TypeError):
        ddt.tree_build(*args, budget, out=out)
    with pytest.raises(KeyError):
        ddt.tree_build(*args, budget, out={"node_token": z((B, budget + 1))})
    with pytest.raises(ValueError):
        ddt.tree_build(args[0].cpu(), *args[1:], budget)


def test_verify_attn_rejects():
    B, Q, H, dl, dr, L = 2, 9, 4, 64, 16, 40
    S = B * (L + Q)
    f = torch.float32
    base = dict(q_lat=z((B, Q, H, dl), f), q_pe=z((B, Q, H, dr), f), c_kv=z((S, dl), f),
                k_pe=z((S, dr), f), req_to_slot=z((B, L + Q)), prefix_len=z((B,)),
                n_nodes=z((B,)), vis=z((B, Q, 1), torch.int64), sm_scale=0.1)

    def call(**kw):
        a = dict(base)
        a.update(kw)
        return ddt.verify_attn(**a)

    call()
    for k, bad in (("prefix_len", z((B + 1,))), ("n_nodes", z((1,))),
                   ("vis", z((B, Q, 2), torch.int64)), ("k_pe", z((S + 1, dr), f)),
                   ("out", z((B, Q, H, dl + 1), f)), ("lse", z((B, Q), f)),
                   ("req_to_slot", z((B + 1, L + Q)))):
        with pytest.raises(ValueError):
            call(**{k: bad})
    with pytest.raises(TypeError):
        call(out=z((B, Q, H, dl), torch.bfloat16))
    need = ddt.workspace_size(B, Q, H, L + Q, dl)
    call(workspace=z((need,), torch.uint8))
    with pytest.raises(ValueError):
        call(workspace=z((max(1, need - 1),), torch.uint8))
    with pytest.raises(TypeError):
        call(workspace=z((need,), torch.int32))


def test_accept_and_commit_reject():
    B, Q = 3, 9
    ddt.tree_accept(z((B, Q)), z((B, Q)), z((B,)), z((B, Q)))
    with pytest.raises(ValueError):
        ddt.tree_accept(z((B, Q)), z((B, Q)), z((B + 1,)), z((B, Q)))
    with pytest.raises(ValueError):
        ddt.tree_accept(z((B, Q)), z((B, Q + 1)), z((B,)), z((B, Q)))
    with pytest.raises(ValueError):
        ddt.tree_accept(z((B, Q)), z((B, Q)), z((B,)), z((B, Q)),
                        out={"accept_len": z((B,)), "accept_nodes": z((B, Q - 1)),
                             "out_tokens": z((B, Q)), "next_root": z((B,))})
    r2s = z((B, 40))
    with pytest.raises(ValueError):
        ddt.kv_commit(r2s, z((B,)), z((B,)), z((B + 1,)), z((B, Q)))
    with pytest.raises(ValueError):
        ddt.kv_commit(r2s, z((B,)), z((B,)), z((B,)), z((B, Q)),
                      out={"freed_slots": z((B, Q)), "n_freed": z((B + 2,))})
