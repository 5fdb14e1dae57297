"""Python binding of libddt.so, the MI355X DDTree tree-verify step.

The functions below only marshal arguments: they check shapes, dtypes and
devices of torch tensors, allocate outputs/workspace with torch (device memory
and streams are all PyTorch is used for) and call the C entry points declared in
include/ddt.h through ctypes on the current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no other code path, and
every call raises if the library is missing or returns an error.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# DDT_LIB names another build of the same library (the host-sanitized one).
LIB_PATH = os.environ.get("DDT_LIB") or os.path.join(_HERE, "libddt.so")

DDT_OK, DDT_EINVAL, DDT_EUNSUPPORTED, DDT_ELAUNCH = 0, -1, -2, -3
DDT_F32, DDT_BF16 = 0, 1
MAX_Q = 128

EXPORTED = ("ddt_version", "ddt_last_error", "ddt_tree_build",
            "ddt_verify_attn_workspace_size", "ddt_verify_attn", "ddt_verify_attn_kernel_times",
            "ddt_verify_attn_noalloc_max_bytes", "ddt_verify_attn_noalloc", "ddt_tree_accept",
            "ddt_kv_commit", "ddt_draft_topk_workspace_size", "ddt_draft_topk",
            "ddt_tree_accept_sampling_workspace_size", "ddt_tree_accept_sampling")


class DDTError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (code {code})")
        self.code = code


_lib = None


def load_library(path: str | None = None):
    """Load libddt.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m tree_verify_mla_ddt_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.ddt_version.argtypes, lib.ddt_version.restype = [], ctypes.c_char_p
    lib.ddt_last_error.argtypes, lib.ddt_last_error.restype = [], ctypes.c_char_p
    lib.ddt_tree_build.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32] + [vp] * 9 + [vp]
    lib.ddt_tree_build.restype = i32
    lib.ddt_verify_attn_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.ddt_verify_attn_workspace_size.restype = sz
    lib.ddt_verify_attn.argtypes = ([vp, vp, vp, vp, i64, vp, i32, vp, vp, vp, i32, i32, i32, i32,
                                     i32, i32, f32, vp, vp, vp, sz, vp])
    lib.ddt_verify_attn.restype = i32
    lib.ddt_verify_attn_kernel_times.argtypes = list(lib.ddt_verify_attn.argtypes) + [i32, vp]
    lib.ddt_verify_attn_kernel_times.restype = i32
    lib.ddt_verify_attn_noalloc_max_bytes.argtypes = []
    lib.ddt_verify_attn_noalloc_max_bytes.restype = sz
    lib.ddt_verify_attn_noalloc.argtypes = list(lib.ddt_verify_attn.argtypes[:19]) + [vp]
    lib.ddt_verify_attn_noalloc.restype = i32
    lib.ddt_tree_accept.argtypes = [vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp]
    lib.ddt_tree_accept.restype = i32
    lib.ddt_kv_commit.argtypes = [vp, i32, vp, vp, vp, vp, i32, i32, vp, vp, vp]
    lib.ddt_kv_commit.restype = i32
    lib.ddt_draft_topk_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.ddt_draft_topk_workspace_size.restype = sz
    lib.ddt_draft_topk.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, sz, vp]
    lib.ddt_draft_topk.restype = i32
    lib.ddt_tree_accept_sampling_workspace_size.argtypes = [i32, i32, i32]
    lib.ddt_tree_accept_sampling_workspace_size.restype = sz
    lib.ddt_tree_accept_sampling.argtypes = ([vp, i32, i32] + [vp] * 6 + [i32, i32] + [vp] * 5
                                             + [sz, vp])
    lib.ddt_tree_accept_sampling.restype = i32
    if path is None:
        _lib = lib
    return lib


def version() -> str:
    return load_library().ddt_version().decode()


def last_error() -> str:
    return load_library().ddt_last_error().decode()


def _check(rc: int):
    if rc != DDT_OK:
        raise DDTError(rc, last_error())


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype, ndim: int | None = None, shape=None, device=None):
    """A contiguous GPU tensor of `dtype`; with `shape`, exactly that shape, and
    with `device`, on that device (every array of a call is on one GPU)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other arrays on {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _workspace(ws: torch.Tensor | None, need: int, device) -> torch.Tensor:
    """The caller's workspace (a contiguous uint8 GPU tensor on `device`, at least
    `need` bytes), or a new one."""
    if ws is None:
        return torch.empty((max(1, need),), dtype=torch.uint8, device=device)
    _dev(ws, "workspace", torch.uint8, 1, device=device)
    if ws.numel() < need:
        raise ValueError(f"workspace of {ws.numel()} bytes given, {need} needed")
    return ws


def _out_dict(out: dict | None, spec: dict, device) -> dict:
    """Output arrays: the caller's (each checked against its dtype and shape)
    or new ones.  spec: name -> (dtype, shape)."""
    if out is None:
        return {k: torch.empty(shp, dtype=dt, device=device) for k, (dt, shp) in spec.items()}
    for k, (dt, shp) in spec.items():
        if k not in out:
            raise KeyError(f"out is missing {k!r}")
        _dev(out[k], k, dt, shape=shp, device=device)
    return out


def tree_build(topk_logp: torch.Tensor, topk_ids: torch.Tensor, root_token: torch.Tensor,
               prefix_len: torch.Tensor, budget: int, out: dict | None = None) -> dict:
    """Best-first draft tree on the GPU (ddt_tree_build).

    topk_logp [B,D,K] f32, topk_ids [B,D,K] i32, root_token [B] i32, prefix_len [B] i32.
    Returns node_token/parent/depth/position/first_child/next_sibling [B,Q] i32,
    score [B,Q] f32, vis [B,Q,W] int64 (bit pattern of the u64 bitsets), n_nodes [B] i32.
    """
    _dev(topk_logp, "topk_logp", torch.float32, 3)
    dev = topk_logp.device
    B, D, K = topk_logp.shape
    _dev(topk_ids, "topk_ids", torch.int32, shape=(B, D, K), device=dev)
    _dev(root_token, "root_token", torch.int32, shape=(B,), device=dev)
    _dev(prefix_len, "prefix_len", torch.int32, shape=(B,), device=dev)
    Q = budget + 1
    W = (Q + 63) // 64
    spec = {k: (torch.int32, (B, Q)) for k in
            ("node_token", "parent", "depth", "position", "first_child", "next_sibling")}
    spec["score"] = (torch.float32, (B, Q))
    spec["vis"] = (torch.int64, (B, Q, W))
    spec["n_nodes"] = (torch.int32, (B,))
    out = _out_dict(out, spec, dev)
    rc = load_library().ddt_tree_build(
        _ptr(topk_logp), _ptr(topk_ids), _ptr(root_token), _ptr(prefix_len), B, D, K, budget,
        _ptr(out["node_token"]), _ptr(out["parent"]), _ptr(out["depth"]), _ptr(out["position"]),
        _ptr(out["first_child"]), _ptr(out["next_sibling"]), _ptr(out["score"]),
        _ptr(out["vis"]), _ptr(out["n_nodes"]), _stream())
    _check(rc)
    return out


def workspace_size(B: int, Q: int, H: int, max_kv: int, d_lat: int) -> int:
    return int(load_library().ddt_verify_attn_workspace_size(B, Q, H, max_kv, d_lat))


def _attn_args(q_lat, q_pe, c_kv, k_pe, req_to_slot, prefix_len, n_nodes, vis, sm_scale,
               out, lse, workspace, want_lse, with_workspace=True):
    """Checked C arguments of ddt_verify_attn (everything but the stream; without
    the two workspace arguments when with_workspace is false) and the output
    tensors."""
    dt = q_lat.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise TypeError("q_lat must be bf16 or f32")
    _dev(q_lat, "q_lat", dt, 4)
    dev = q_lat.device
    B, Q, H, d_lat = q_lat.shape
    _dev(q_pe, "q_pe", dt, 4, device=dev)
    d_rope = q_pe.shape[-1]
    _dev(q_pe, "q_pe", dt, shape=(B, Q, H, d_rope))
    _dev(c_kv, "c_kv", dt, 2, device=dev)
    S = c_kv.shape[0]
    _dev(c_kv, "c_kv", dt, shape=(S, d_lat))
    _dev(k_pe, "k_pe", dt, shape=(S, d_rope), device=dev)
    _dev(req_to_slot, "req_to_slot", torch.int32, 2, device=dev)
    max_kv = req_to_slot.shape[1]
    _dev(req_to_slot, "req_to_slot", torch.int32, shape=(B, max_kv))
    _dev(prefix_len, "prefix_len", torch.int32, shape=(B,), device=dev)
    _dev(n_nodes, "n_nodes", torch.int32, shape=(B,), device=dev)
    _dev(vis, "vis", torch.int64, shape=(B, Q, (Q + 63) // 64), device=dev)
    if out is None:
        out = torch.empty((B, Q, H, d_lat), dtype=torch.float32, device=dev)
    _dev(out, "out", torch.float32, shape=(B, Q, H, d_lat), device=dev)
    if lse is None and want_lse:
        lse = torch.empty((B, Q, H), dtype=torch.float32, device=dev)
    if lse is not None:
        _dev(lse, "lse", torch.float32, shape=(B, Q, H), device=dev)
    lib = load_library()
    args = (_ptr(q_lat), _ptr(q_pe), _ptr(c_kv), _ptr(k_pe), S, _ptr(req_to_slot), max_kv,
            _ptr(prefix_len), _ptr(n_nodes), _ptr(vis), B, Q, H, d_lat, d_rope,
            DDT_BF16 if dt == torch.bfloat16 else DDT_F32, float(sm_scale), _ptr(out),
            _ptr(lse))
    if with_workspace:
        need = int(lib.ddt_verify_attn_workspace_size(B, Q, H, max_kv, d_lat))
        workspace = _workspace(workspace, need, dev)
        args += (_ptr(workspace), workspace.numel() * workspace.element_size())
    return lib, args, out, lse


def verify_attn(q_lat: torch.Tensor, q_pe: torch.Tensor, c_kv: torch.Tensor, k_pe: torch.Tensor,
                req_to_slot: torch.Tensor, prefix_len: torch.Tensor, n_nodes: torch.Tensor,
                vis: torch.Tensor, sm_scale: float, out: torch.Tensor | None = None,
                lse: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                want_lse: bool = True):
    """Tree-verify MLA-absorb attention (ddt_verify_attn).

    q_lat [B,Q,H,d_lat], q_pe [B,Q,H,d_rope], c_kv [S,d_lat], k_pe [S,d_rope] (all bf16 or
    all f32), req_to_slot [B,max_kv] i32, prefix_len [B] i32, n_nodes [B] i32,
    vis [B,Q,W] int64.  Returns (out [B,Q,H,d_lat] f32, lse [B,Q,H] f32 or None)."""
    lib, args, out, lse = _attn_args(q_lat, q_pe, c_kv, k_pe, req_to_slot, prefix_len, n_nodes,
                                     vis, sm_scale, out, lse, workspace, want_lse)
    _check(lib.ddt_verify_attn(*args, _stream()))
    return out, lse


def verify_attn_noalloc(q_lat: torch.Tensor, q_pe: torch.Tensor, c_kv: torch.Tensor,
                        k_pe: torch.Tensor, req_to_slot: torch.Tensor, prefix_len: torch.Tensor,
                        n_nodes: torch.Tensor, vis: torch.Tensor, sm_scale: float,
                        out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                        want_lse: bool = True):
    """ddt_verify_attn_noalloc: verify_attn with the library's static scratch array
    as workspace.  Pass `out` (and `lse`, or want_lse=False) to allocate nothing."""
    lib, args, out, lse = _attn_args(q_lat, q_pe, c_kv, k_pe, req_to_slot, prefix_len, n_nodes,
                                     vis, sm_scale, out, lse, None, want_lse,
                                     with_workspace=False)
    _check(lib.ddt_verify_attn_noalloc(*args, _stream()))
    return out, lse


def verify_attn_kernel_times(q_lat, q_pe, c_kv, k_pe, req_to_slot, prefix_len, n_nodes, vis,
                             sm_scale: float, reps: int, out=None, lse=None, workspace=None,
                             want_lse: bool = True):
    """Mean per-launch milliseconds of the attention kernel and of the merge kernel
    of one ddt_verify_attn call, each launched `reps` times back to back between
    HIP events on the current stream (ddt_verify_attn_kernel_times; synchronizes).
    Returns (attention_ms, merge_ms, out, lse)."""
    lib, args, out, lse = _attn_args(q_lat, q_pe, c_kv, k_pe, req_to_slot, prefix_len, n_nodes,
                                     vis, sm_scale, out, lse, workspace, want_lse)
    ms = (ctypes.c_float * 2)()
    _check(lib.ddt_verify_attn_kernel_times(*args, _stream(), int(reps), ms))
    return float(ms[0]), float(ms[1]), out, lse


def tree_accept(node_token: torch.Tensor, parent: torch.Tensor, n_nodes: torch.Tensor,
                target_argmax: torch.Tensor, out: dict | None = None) -> dict:
    """Greedy follow-the-verified-tree acceptance (ddt_tree_accept)."""
    _dev(node_token, "node_token", torch.int32, 2)
    dev = node_token.device
    B, Q = node_token.shape
    _dev(parent, "parent", torch.int32, shape=(B, Q), device=dev)
    _dev(n_nodes, "n_nodes", torch.int32, shape=(B,), device=dev)
    _dev(target_argmax, "target_argmax", torch.int32, shape=(B, Q), device=dev)
    out = _out_dict(out, {"accept_len": (torch.int32, (B,)),
                          "accept_nodes": (torch.int32, (B, Q)),
                          "out_tokens": (torch.int32, (B, Q)),
                          "next_root": (torch.int32, (B,))}, dev)
    rc = load_library().ddt_tree_accept(
        _ptr(node_token), _ptr(parent), _ptr(n_nodes), _ptr(target_argmax), B, Q,
        _ptr(out["accept_len"]), _ptr(out["accept_nodes"]), _ptr(out["out_tokens"]),
        _ptr(out["next_root"]), _stream())
    _check(rc)
    return out


def tree_accept_sampling(target_logits: torch.Tensor, temperature: torch.Tensor,
                         node_token: torch.Tensor, parent: torch.Tensor, n_nodes: torch.Tensor,
                         coins: torch.Tensor, coin_final: torch.Tensor, out: dict | None = None,
                         workspace: torch.Tensor | None = None) -> dict:
    """Acceptance under temperature sampling from the target's logits [B,Q,V]
    (bf16 or f32) at every tree node (ddt_tree_accept_sampling).  Outputs as
    for tree_accept; coins [B,Q] and coin_final [B] are the caller's U[0,1)
    draws."""
    dt = target_logits.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise TypeError("target_logits must be bf16 or f32")
    _dev(target_logits, "target_logits", dt, 3)
    dev = target_logits.device
    B, Q, V = target_logits.shape
    _dev(temperature, "temperature", torch.float32, shape=(B,), device=dev)
    _dev(node_token, "node_token", torch.int32, shape=(B, Q), device=dev)
    _dev(parent, "parent", torch.int32, shape=(B, Q), device=dev)
    _dev(n_nodes, "n_nodes", torch.int32, shape=(B,), device=dev)
    _dev(coins, "coins", torch.float32, shape=(B, Q), device=dev)
    _dev(coin_final, "coin_final", torch.float32, shape=(B,), device=dev)
    lib = load_library()
    out = _out_dict(out, {"accept_len": (torch.int32, (B,)),
                          "accept_nodes": (torch.int32, (B, Q)),
                          "out_tokens": (torch.int32, (B, Q)),
                          "next_root": (torch.int32, (B,))}, dev)
    need = int(lib.ddt_tree_accept_sampling_workspace_size(B, Q, V))
    workspace = _workspace(workspace, need, dev)
    rc = lib.ddt_tree_accept_sampling(
        _ptr(target_logits), DDT_BF16 if dt == torch.bfloat16 else DDT_F32, V, _ptr(temperature),
        _ptr(node_token), _ptr(parent), _ptr(n_nodes), _ptr(coins), _ptr(coin_final), B, Q,
        _ptr(out["accept_len"]), _ptr(out["accept_nodes"]), _ptr(out["out_tokens"]),
        _ptr(out["next_root"]), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream())
    _check(rc)
    return out


def draft_topk(logits: torch.Tensor, K: int, out: dict | None = None,
               workspace: torch.Tensor | None = None) -> dict:
    """Per-depth top-K log-probs and ids of drafter logits [B,D,V] (bf16 or f32),
    in the layout tree_build takes (ddt_draft_topk)."""
    dt = logits.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise TypeError("logits must be bf16 or f32")
    _dev(logits, "logits", dt, 3)
    dev = logits.device
    B, D, V = logits.shape
    lib = load_library()
    out = _out_dict(out, {"topk_logp": (torch.float32, (B, D, K)),
                          "topk_ids": (torch.int32, (B, D, K))}, dev)
    need = int(lib.ddt_draft_topk_workspace_size(B, D, V, K))
    workspace = _workspace(workspace, need, dev)
    rc = lib.ddt_draft_topk(_ptr(logits), DDT_BF16 if dt == torch.bfloat16 else DDT_F32, B, D, V,
                            K, _ptr(out["topk_logp"]), _ptr(out["topk_ids"]), _ptr(workspace),
                            workspace.numel() * workspace.element_size(), _stream())
    _check(rc)
    return out


def kv_commit(req_to_slot: torch.Tensor, prefix_len: torch.Tensor, n_nodes: torch.Tensor,
              accept_len: torch.Tensor, accept_nodes: torch.Tensor,
              out: dict | None = None) -> dict:
    """Append the accepted path to the committed prefix (ddt_kv_commit).

    Rewrites `req_to_slot` and `prefix_len` in place; returns the released
    slots ("freed_slots" [B][Q], -1 padded) and their count ("n_freed" [B])."""
    _dev(req_to_slot, "req_to_slot", torch.int32, 2)
    dev = req_to_slot.device
    B, max_kv = req_to_slot.shape
    _dev(accept_nodes, "accept_nodes", torch.int32, 2, device=dev)
    Q = accept_nodes.shape[1]
    _dev(accept_nodes, "accept_nodes", torch.int32, shape=(B, Q))
    _dev(prefix_len, "prefix_len", torch.int32, shape=(B,), device=dev)
    _dev(n_nodes, "n_nodes", torch.int32, shape=(B,), device=dev)
    _dev(accept_len, "accept_len", torch.int32, shape=(B,), device=dev)
    out = _out_dict(out, {"freed_slots": (torch.int32, (B, Q)),
                          "n_freed": (torch.int32, (B,))}, dev)
    rc = load_library().ddt_kv_commit(
        _ptr(req_to_slot), max_kv, _ptr(prefix_len), _ptr(n_nodes), _ptr(accept_len),
        _ptr(accept_nodes), B, Q, _ptr(out["freed_slots"]), _ptr(out["n_freed"]), _stream())
    _check(rc)
    return out


def default_sm_scale(d_qk_nope: int = 128, d_rope: int = 64) -> float:
    return 1.0 / math.sqrt(d_qk_nope + d_rope)
