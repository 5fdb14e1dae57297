"""Compile the HIP sources under csrc/ into libddt.so (gfx950) next to this file.

Usage: python -m tree_verify_mla_ddt_amd.build [--verbose]
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_PATH = os.path.join(HERE, "libddt.so")
# Host-side checker of the attention work split (CPU tests only).
CHECK_PATH = os.environ.get("DDT_SPLIT_CHECK_LIB") or os.path.join(HERE, "libddt_split_check.so")
# Measured ceilings of the attention tile (bench.py --ceiling).
CEILING_PATH = os.path.join(HERE, "libddt_ceiling.so")
SOURCES = ["api.hip", "draft_topk.hip", "tree_build.hip", "tree_accept.hip",
           "tree_accept_sampling.hip", "kv_commit.hip", "verify_attn.hip", "noalloc.hip"]
ARCH = os.environ.get("DDT_OFFLOAD_ARCH", "gfx950")


def hipcc_command(out_path: str, resource_report: bool = False) -> list[str]:
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-fno-gpu-flush-denormals-to-zero",
           # no packed fp32 VALU instructions (v_pk_*_f32) anywhere in the library
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-I", os.path.join(HERE, "..", "include")]
    if resource_report:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    cmd += [os.path.join(CSRC, s) for s in SOURCES] + ["-o", out_path]
    return cmd


def split_check_command(out_path: str) -> list[str]:
    return ["hipcc", f"--offload-arch={ARCH}", "-O2", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            os.path.join(CSRC, "split_check.hip"), "-o", out_path]


def build_split_check() -> str:
    """The host-only split checker (csrc/split_check.hip) as its own library."""
    tmp = CHECK_PATH + ".tmp"
    res = subprocess.run(split_check_command(tmp), capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}{res.stderr}")
    os.replace(tmp, CHECK_PATH)
    return CHECK_PATH


# AddressSanitizer + UndefinedBehaviorSanitizer for the host pass only (each
# option behind -Xarch_host); the device code is compiled as usual.  The host
# code is the argument validation of every entry point, the launch planning and
# the split checker.  Such a build needs clang's ASan runtime loaded first
# (LD_PRELOAD) and is for CPU tests only.
SAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g", "-Xarch_host", "-O1"]


def build_sanitized(out_dir: str) -> tuple[str, str]:
    """libddt.so and the split checker with sanitized host code, into out_dir."""
    os.makedirs(out_dir, exist_ok=True)
    lib = os.path.join(out_dir, "libddt_san.so")
    check = os.path.join(out_dir, "libddt_split_check_san.so")
    for cmd in (hipcc_command(lib), split_check_command(check)):
        cmd = cmd[:-2] + SAN_HOST_FLAGS + cmd[-2:]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}{res.stderr}")
    return lib, check


def build_ceiling() -> str:
    """The ceiling microbenchmark (csrc/ceiling.hip) as its own library."""
    tmp = CEILING_PATH + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           os.path.join(CSRC, "ceiling.hip"), "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}{res.stderr}")
    os.replace(tmp, CEILING_PATH)
    return CEILING_PATH


def build(verbose: bool = False, resource_report: bool = False) -> str:
    tmp = LIB_PATH + ".tmp"
    res = subprocess.run(hipcc_command(tmp, resource_report), capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    log = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{log}")
    if verbose and log.strip():
        print(log)
    os.replace(tmp, LIB_PATH)
    build_split_check()
    build_ceiling()
    return LIB_PATH


if __name__ == "__main__":
    v = "--verbose" in sys.argv
    print(build(verbose=v, resource_report="--resources" in sys.argv))
