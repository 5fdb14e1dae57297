"""The C ABI of libddt.so, checked without a GPU: the library loads, exports every
entry point include/ddt.h declares, and rejects invalid scalar arguments on the
host (before any device work) with the documented codes and messages."""
import ctypes
import os
import re

import pytest

import tree_verify_mla_ddt_amd as ddt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ddt.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ddt.LIB_PATH):
        pytest.skip("libddt.so not built (run __graft_entry__.build())")
    return ddt.load_library()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:const char\*|int|size_t)\s+(ddt_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    assert header_functions() == sorted(ddt.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    assert ddt.version().startswith("ddt ")
    assert "gfx950" in ddt.version()


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "ddt.h"\nint main(void){return DDT_OK + DDT_BF16 + DDT_MAX_Q * 0;}\n')
    import subprocess
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                        "-c", str(src), "-o", str(tmp_path / "use.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


NULL = None


def call_build(lib, B=1, D=4, K=4, budget=8, null_out=False):
    p = ctypes.c_void_p(16)  # never dereferenced: validation fails first
    outs = [NULL if null_out else p] + [p] * 8
    return lib.ddt_tree_build(p, p, p, p, B, D, K, budget, *outs, NULL)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(B=0), ddt.DDT_EINVAL, "B=0"),
    (dict(D=-1), ddt.DDT_EINVAL, "D=-1"),
    (dict(D=65), ddt.DDT_EINVAL, "D=65"),
    (dict(K=65), ddt.DDT_EINVAL, "K=65"),
    (dict(budget=128), ddt.DDT_EINVAL, "budget=128"),
    (dict(budget=-1), ddt.DDT_EINVAL, "budget=-1"),
    (dict(null_out=True), ddt.DDT_EINVAL, "NULL"),
])
def test_tree_build_rejects(lib, kw, code, needle):
    assert call_build(lib, **kw) == code
    assert needle in ddt.last_error()


def call_attn(lib, B=1, Q=9, H=64, d_lat=512, d_rope=64, dtype=ddt.DDT_BF16, scale=0.07,
              max_kv=100, num_slots=100, ws_bytes=1 << 40, null_q=False):
    p = ctypes.c_void_p(16)
    return lib.ddt_verify_attn(NULL if null_q else p, p, p, p, num_slots, p, max_kv, p, p, p, B, Q,
                               H, d_lat, d_rope, dtype, ctypes.c_float(scale), p, p, p, ws_bytes,
                               NULL)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(B=0), ddt.DDT_EINVAL, "B=0"),
    (dict(B=513), ddt.DDT_EINVAL, "B=513"),
    (dict(Q=0), ddt.DDT_EINVAL, "Q=0"),
    (dict(Q=129), ddt.DDT_EINVAL, "Q=129"),
    (dict(H=0), ddt.DDT_EINVAL, "H=0"),
    (dict(max_kv=0), ddt.DDT_EINVAL, "max_kv=0"),
    (dict(num_slots=0), ddt.DDT_EINVAL, "num_slots=0"),
    (dict(dtype=7), ddt.DDT_EINVAL, "dtype=7"),
    (dict(scale=float("nan")), ddt.DDT_EINVAL, "sm_scale"),
    (dict(scale=float("inf")), ddt.DDT_EINVAL, "sm_scale"),
    (dict(scale=0.0), ddt.DDT_EINVAL, "sm_scale"),
    (dict(scale=-0.1), ddt.DDT_EINVAL, "sm_scale"),
    (dict(d_lat=256), ddt.DDT_EUNSUPPORTED, "not compiled in"),
    (dict(dtype=ddt.DDT_F32), ddt.DDT_EUNSUPPORTED, "not compiled in"),
    (dict(null_q=True), ddt.DDT_EINVAL, "NULL"),
    (dict(ws_bytes=16), ddt.DDT_EINVAL, "workspace"),
])
def test_verify_attn_rejects(lib, kw, code, needle):
    assert call_attn(lib, **kw) == code
    assert needle in ddt.last_error()


def call_attn_times(lib, reps=10, null_ms=False, **kw):
    p = ctypes.c_void_p(16)
    ms = (ctypes.c_float * 2)()
    B, Q = kw.get("B", 1), kw.get("Q", 9)
    return lib.ddt_verify_attn_kernel_times(p, p, p, p, 100, p, 100, p, p, p, B, Q, 64, 512, 64,
                                            ddt.DDT_BF16, ctypes.c_float(0.07), p, p, p, 1 << 40,
                                            NULL, reps, NULL if null_ms else ms)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(reps=0), ddt.DDT_EINVAL, "reps=0"),
    (dict(reps=100001), ddt.DDT_EINVAL, "reps=100001"),
    (dict(null_ms=True), ddt.DDT_EINVAL, "NULL kernel_ms"),
    (dict(B=0), ddt.DDT_EINVAL, "ddt_verify_attn_kernel_times: B=0"),
    (dict(Q=129), ddt.DDT_EINVAL, "ddt_verify_attn_kernel_times: Q=129"),
])
def test_verify_attn_kernel_times_rejects(lib, kw, code, needle):
    assert call_attn_times(lib, **kw) == code
    assert needle in ddt.last_error()


def call_attn_noalloc(lib, B=1, Q=9, H=64, d_lat=512, d_rope=64, dtype=ddt.DDT_BF16,
                      null_out=False):
    p = ctypes.c_void_p(16)
    return lib.ddt_verify_attn_noalloc(p, p, p, p, 100, p, 100, p, p, p, B, Q, H, d_lat, d_rope,
                                       dtype, ctypes.c_float(0.07), NULL if null_out else p, p,
                                       NULL)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(B=0), ddt.DDT_EINVAL, "ddt_verify_attn_noalloc: B=0"),
    (dict(Q=129), ddt.DDT_EINVAL, "ddt_verify_attn_noalloc: Q=129"),
    (dict(d_lat=256), ddt.DDT_EUNSUPPORTED, "not compiled in"),
    (dict(null_out=True), ddt.DDT_EINVAL, "NULL"),
])
def test_verify_attn_noalloc_rejects(lib, kw, code, needle):
    assert call_attn_noalloc(lib, **kw) == code
    assert needle in ddt.last_error()


def test_noalloc_scratch_size(lib):
    # two partial 128-row tiles of 513 floats for each of 256 workgroups, and the
    # stream prefix of 512 requests, the split mode and the start cost (rounded up
    # to 16 bytes)
    assert lib.ddt_verify_attn_noalloc_max_bytes() == 2 * 256 * 128 * 513 * 4 + 516 * 8


def test_workspace_size_query(lib):
    n = lib.ddt_verify_attn_workspace_size(8, 65, 64, 32833, 512)
    assert n > 0
    assert lib.ddt_verify_attn_workspace_size(0, 65, 64, 32833, 512) == 0
    # covers at least one partial 128-row tile of fp32 outputs
    assert n >= 128 * 513 * 4


@pytest.mark.parametrize("B,Q,code,needle", [(0, 9, ddt.DDT_EINVAL, "B=0"),
                                             (1, 0, ddt.DDT_EINVAL, "Q=0"),
                                             (1, 129, ddt.DDT_EINVAL, "Q=129")])
def test_tree_accept_rejects(lib, B, Q, code, needle):
    p = ctypes.c_void_p(16)
    assert lib.ddt_tree_accept(p, p, p, p, B, Q, p, p, p, p, NULL) == code
    assert needle in ddt.last_error()


@pytest.mark.parametrize("B,Q,max_kv,null,needle", [(0, 9, 10, False, "B=0"),
                                                     (1, 0, 10, False, "Q=0"),
                                                     (1, 129, 10, False, "Q=129"),
                                                     (1, 9, 0, False, "max_kv=0"),
                                                     (1, 9, 10, True, "NULL")])
def test_kv_commit_rejects(lib, B, Q, max_kv, null, needle):
    p = ctypes.c_void_p(16)
    assert lib.ddt_kv_commit(p, max_kv, p, p, p, NULL if null else p, B, Q, p, p,
                             NULL) == ddt.DDT_EINVAL
    assert needle in ddt.last_error()


@pytest.mark.parametrize("kw,needle", [(dict(B=0), "B=0"), (dict(D=0), "D=0"),
                                       (dict(B=300, D=300), "65535"), (dict(K=0), "K=0"),
                                       (dict(K=65), "K=65"), (dict(V=3, K=4), "V=3"),
                                       (dict(V=1048577), "V=1048577"), (dict(dtype=5), "dtype=5"),
                                       (dict(ws=8), "workspace")])
def test_draft_topk_rejects(lib, kw, needle):
    a = dict(B=1, D=8, V=160000, K=8, dtype=ddt.DDT_BF16, ws=1 << 40)
    a.update(kw)
    p = ctypes.c_void_p(16)
    assert lib.ddt_draft_topk(p, a["dtype"], a["B"], a["D"], a["V"], a["K"], p, p, p, a["ws"],
                              NULL) == ddt.DDT_EINVAL
    assert needle in ddt.last_error()


def test_draft_topk_workspace_size(lib):
    n = lib.ddt_draft_topk_workspace_size(8, 15, 160000, 16)
    assert n >= 8 * 15 * (16 * 8 + 8)
    assert lib.ddt_draft_topk_workspace_size(8, 15, 10, 16) == 0


@pytest.mark.parametrize("kw,needle", [(dict(B=0), "B=0"), (dict(Q=0), "Q=0"),
                                       (dict(Q=129), "Q=129"), (dict(B=(1 << 17) + 1, Q=128), "2^24"),
                                       (dict(V=0), "V=0"), (dict(V=1048577), "V=1048577"),
                                       (dict(dtype=7), "dtype=7"), (dict(null=True), "NULL"),
                                       (dict(ws=16), "workspace")])
def test_tree_accept_sampling_rejects(lib, kw, needle):
    a = dict(B=8, Q=65, V=160000, dtype=ddt.DDT_BF16, ws=1 << 40, null=False)
    a.update(kw)
    p = ctypes.c_void_p(16)
    coins = NULL if a["null"] else p
    assert lib.ddt_tree_accept_sampling(p, a["dtype"], a["V"], p, p, p, p, coins, p, a["B"],
                                        a["Q"], p, p, p, p, p, a["ws"], NULL) == ddt.DDT_EINVAL
    assert needle in ddt.last_error()


def test_tree_accept_sampling_workspace_size(lib):
    n = lib.ddt_tree_accept_sampling_workspace_size(8, 65, 160000)
    assert n >= 8 * 65 * 14 * 16  # at least 14 chunks of <= 12288 entries per row
    assert lib.ddt_tree_accept_sampling_workspace_size(8, 129, 160000) == 0
    assert lib.ddt_tree_accept_sampling_workspace_size(8, 65, 0) == 0


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        ddt.load_library(str(tmp_path / "nope.so"))


def test_product_path_does_not_reference_the_oracle():
    pkg = os.path.join(ROOT, "tree_verify_mla_ddt_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "ddt_oracle" not in text, f
