"""Plain CPU oracle for the DDTree tree-verify step (ctypes over ddt_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it to produce expected values.  Nothing in the library's
product path imports it, and it shares no code with the HIP library.

Functions take and return numpy arrays (host memory).  Attention results are
float64.  See ddt_oracle.h for the definitions and the passages they follow.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ddt_oracle.c")
LIB_PATH = os.path.join(_HERE, "libddt_oracle.so")
# AddressSanitizer + UndefinedBehaviorSanitizer build (host code only), loaded
# instead of LIB_PATH when DDT_ORACLE_LIB names it.
SAN_PATH = os.path.join(_HERE, "libddt_oracle_san.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile ddt_oracle.c with gcc (OpenMP, no fast-math) into LIB_PATH."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def build_sanitized() -> str:
    """ddt_oracle.c with -fsanitize=address,undefined (any finding aborts)."""
    tmp = SAN_PATH + ".tmp"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-fno-fast-math",
           "-ffp-contract=off", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, SAN_PATH)
    return SAN_PATH


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("DDT_ORACLE_LIB") or LIB_PATH
        if path == LIB_PATH and not os.path.exists(LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(path)
        p = ctypes.c_void_p
        i32, i64, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_float
        lib.ddt_oracle_tree_build.argtypes = [p, p, p, p, i32, i32, i32, i32] + [p] * 9
        lib.ddt_oracle_verify_attn_rows.argtypes = (
            [p, p, p, p, i64, p, i32, p, p, p, i32, i32, i32, i32, i32, f32, i64, p, p, p])
        lib.ddt_oracle_tree_accept.argtypes = [p, p, p, p, i32, i32, p, p, p, p]
        lib.ddt_oracle_kv_commit.argtypes = [p, i32, p, p, p, p, i32, i32, p, p]
        lib.ddt_oracle_draft_topk.argtypes = [p, i32, i32, i32, i32, p, p]
        lib.ddt_oracle_tree_accept_sampling.argtypes = (
            [p, i32, p, p, p, p, p, p, i32, i32, ctypes.c_double] + [p] * 7)
        lib.ddt_oracle_num_threads.argtypes = []
        lib.ddt_oracle_set_num_threads.argtypes = [i32]
        for f in (lib.ddt_oracle_tree_build, lib.ddt_oracle_verify_attn_rows,
                  lib.ddt_oracle_tree_accept, lib.ddt_oracle_kv_commit,
                  lib.ddt_oracle_draft_topk, lib.ddt_oracle_tree_accept_sampling,
                  lib.ddt_oracle_num_threads, lib.ddt_oracle_set_num_threads):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().ddt_oracle_num_threads())


def set_num_threads(n: int) -> int:
    """Threads the oracle's parallel loops use from now on; returns the count."""
    return int(_load().ddt_oracle_set_num_threads(int(n)))


def tree_build(topk_logp, topk_ids, root_token, prefix_len, budget: int) -> dict:
    """Best-first draft tree; returns a dict of numpy arrays (see ddt_oracle.h)."""
    lib = _load()
    logp, p_logp = _c(topk_logp, np.float32)
    ids, p_ids = _c(topk_ids, np.int32)
    root, p_root = _c(root_token, np.int32)
    plen, p_plen = _c(prefix_len, np.int32)
    B, D, K = logp.shape
    Q = budget + 1
    W = (Q + 63) // 64
    out = {k: np.empty((B, Q), np.int32) for k in
           ("node_token", "parent", "depth", "position", "first_child", "next_sibling")}
    out["score"] = np.empty((B, Q), np.float32)
    out["vis"] = np.empty((B, Q, W), np.uint64)
    out["n_nodes"] = np.empty((B,), np.int32)
    ptr = {k: v.ctypes.data_as(ctypes.c_void_p) for k, v in out.items()}
    rc = lib.ddt_oracle_tree_build(
        p_logp, p_ids, p_root, p_plen, B, D, K, budget,
        ptr["node_token"], ptr["parent"], ptr["depth"], ptr["position"],
        ptr["first_child"], ptr["next_sibling"], ptr["score"], ptr["vis"], ptr["n_nodes"])
    if rc != 0:
        raise ValueError("oracle tree_build rejected its arguments")
    return out


def verify_attn(q_lat, q_pe, c_kv, k_pe, req_to_slot, prefix_len, n_nodes, vis,
                sm_scale: float, rows=None):
    """Double-precision tree-verify attention.

    Float inputs may be any dtype that upcasts exactly to float32 (float32, or a
    bf16 tensor already converted with .float()).  Without `rows` every row is
    evaluated and out has shape [B,Q,H,d_lat], lse [B,Q,H]; with `rows` (an
    [n,3] array of (b, i, h)) out is [n, d_lat] and lse [n].
    """
    lib = _load()
    ql, p_ql = _c(q_lat, np.float32)
    qp, p_qp = _c(q_pe, np.float32)
    ckv, p_ckv = _c(c_kv, np.float32)
    kpe, p_kpe = _c(k_pe, np.float32)
    r2s, p_r2s = _c(req_to_slot, np.int32)
    plen, p_plen = _c(prefix_len, np.int32)
    nn, p_nn = _c(n_nodes, np.int32)
    vv, p_vis = _c(vis, np.uint64)
    B, Q, H, d_lat = ql.shape
    d_rope = qp.shape[-1]
    num_slots = ckv.shape[0]
    max_kv = r2s.shape[1]
    if rows is None:
        b, i, h = np.meshgrid(np.arange(B), np.arange(Q), np.arange(H), indexing="ij")
        rows_arr = np.stack([b.ravel(), i.ravel(), h.ravel()], axis=1)
        shape_out, shape_lse = (B, Q, H, d_lat), (B, Q, H)
    else:
        rows_arr = np.asarray(rows).reshape(-1, 3)
        shape_out, shape_lse = (rows_arr.shape[0], d_lat), (rows_arr.shape[0],)
    rr, p_rows = _c(rows_arr, np.int32)
    n_rows = rr.shape[0]
    out = np.empty((n_rows, d_lat), np.float64)
    lse = np.empty((n_rows,), np.float64)
    rc = lib.ddt_oracle_verify_attn_rows(
        p_ql, p_qp, p_ckv, p_kpe, num_slots, p_r2s, max_kv, p_plen, p_nn, p_vis,
        B, Q, H, d_lat, d_rope, float(np.float32(sm_scale)), n_rows, p_rows,
        out.ctypes.data_as(ctypes.c_void_p), lse.ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError("oracle verify_attn rejected its arguments")
    return out.reshape(shape_out), lse.reshape(shape_lse)


def tree_accept(node_token, parent, n_nodes, target_argmax) -> dict:
    """Greedy follow-the-verified-tree acceptance; returns a dict of arrays."""
    lib = _load()
    tok, p_tok = _c(node_token, np.int32)
    par, p_par = _c(parent, np.int32)
    nn, p_nn = _c(n_nodes, np.int32)
    tgt, p_tgt = _c(target_argmax, np.int32)
    B, Q = tok.shape
    out = {"accept_len": np.empty((B,), np.int32),
           "accept_nodes": np.empty((B, Q), np.int32),
           "out_tokens": np.empty((B, Q), np.int32),
           "next_root": np.empty((B,), np.int32)}
    ptr = {k: v.ctypes.data_as(ctypes.c_void_p) for k, v in out.items()}
    rc = lib.ddt_oracle_tree_accept(p_tok, p_par, p_nn, p_tgt, B, Q,
                                    ptr["accept_len"], ptr["accept_nodes"],
                                    ptr["out_tokens"], ptr["next_root"])
    if rc != 0:
        raise ValueError("oracle tree_accept rejected its arguments")
    return out


def kv_commit(req_to_slot, prefix_len, n_nodes, accept_len, accept_nodes) -> dict:
    """Append the accepted path to the committed prefix.  Returns new copies of
    req_to_slot and prefix_len and the released slots (inputs untouched)."""
    lib = _load()
    r2s = np.array(req_to_slot, dtype=np.int32, order="C", copy=True)
    plen = np.array(prefix_len, dtype=np.int32, order="C", copy=True)
    nn, p_nn = _c(n_nodes, np.int32)
    al, p_al = _c(accept_len, np.int32)
    an, p_an = _c(accept_nodes, np.int32)
    B, max_kv = r2s.shape
    Q = an.shape[1]
    out = {"req_to_slot": r2s, "prefix_len": plen,
           "freed_slots": np.empty((B, Q), np.int32), "n_freed": np.empty((B,), np.int32)}
    rc = lib.ddt_oracle_kv_commit(
        r2s.ctypes.data_as(ctypes.c_void_p), max_kv, plen.ctypes.data_as(ctypes.c_void_p),
        p_nn, p_al, p_an, B, Q, out["freed_slots"].ctypes.data_as(ctypes.c_void_p),
        out["n_freed"].ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError("oracle kv_commit rejected its arguments")
    return out


def draft_topk(logits, K: int) -> dict:
    """Per-depth top-K log-probs and ids of logits [B][D][V] (f32 or bf16 as a
    torch tensor / numpy array; bf16 is upcast exactly).  logp is float64."""
    import torch
    if isinstance(logits, torch.Tensor):
        logits = logits.float().numpy()
    lg, p_lg = _c(logits, np.float32)
    B, D, V = lg.shape
    out = {"topk_logp": np.empty((B, D, K), np.float64), "topk_ids": np.empty((B, D, K), np.int32)}
    rc = _load().ddt_oracle_draft_topk(p_lg, B, D, V, K,
                                       out["topk_logp"].ctypes.data_as(ctypes.c_void_p),
                                       out["topk_ids"].ctypes.data_as(ctypes.c_void_p))
    if rc != 0:
        raise ValueError("oracle draft_topk rejected its arguments")
    return out


def tree_accept_sampling(logits, temperature, node_token, parent, n_nodes, coins, coin_final,
                         band_eps: float = 0.0) -> dict:
    """Sampling acceptance over target logits [B][Q][V] (f32 or bf16 as a torch
    tensor / numpy array; bf16 is upcast exactly).  Returns the greedy
    acceptance outputs plus the diagnostics margin, bonus_lo and bonus_hi."""
    import torch
    if isinstance(logits, torch.Tensor):
        logits = logits.float().numpy()
    lg, p_lg = _c(logits, np.float32)
    B, Q, V = lg.shape
    tmp, p_tmp = _c(temperature, np.float32)
    tok, p_tok = _c(node_token, np.int32)
    par, p_par = _c(parent, np.int32)
    nn, p_nn = _c(n_nodes, np.int32)
    cn, p_cn = _c(coins, np.float32)
    cf, p_cf = _c(coin_final, np.float32)
    assert tmp.shape == (B,) and tok.shape == (B, Q) and par.shape == (B, Q)
    assert nn.shape == (B,) and cn.shape == (B, Q) and cf.shape == (B,)
    out = {"accept_len": np.empty((B,), np.int32),
           "accept_nodes": np.empty((B, Q), np.int32),
           "out_tokens": np.empty((B, Q), np.int32),
           "next_root": np.empty((B,), np.int32),
           "margin": np.empty((B,), np.float64),
           "bonus_lo": np.empty((B,), np.int32),
           "bonus_hi": np.empty((B,), np.int32)}
    ptr = {k: v.ctypes.data_as(ctypes.c_void_p) for k, v in out.items()}
    rc = _load().ddt_oracle_tree_accept_sampling(
        p_lg, V, p_tmp, p_tok, p_par, p_nn, p_cn, p_cf, B, Q, float(band_eps),
        ptr["accept_len"], ptr["accept_nodes"], ptr["out_tokens"], ptr["next_root"],
        ptr["margin"], ptr["bonus_lo"], ptr["bonus_hi"])
    if rc != 0:
        raise ValueError("oracle tree_accept_sampling rejected its arguments")
    return out
