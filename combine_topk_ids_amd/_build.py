"""Build libmoe.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoe.so")
SOURCES = ["host_checks.cpp", "api.hip", "plan.hip", "dispatch.hip", "combine.hip", "exchange.hip",
           "routing_map.hip"]
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")


def hipcc_command(out: str) -> list[str]:
    return [
        "hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-fvisibility=hidden",
        # keep the compiler from emitting packed-fp32 VALU forms
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", os.path.join(ROOT, "include"),
        "-o", out,
    ] + [os.path.join(CSRC, s) for s in SOURCES]


TEST_KERNELS = os.path.join(ROOT, "tests", "kernels")
TEST_LIB = os.path.join(TEST_KERNELS, "libfp8_path_check.so")


def build_test_kernels(force: bool = True) -> str:
    """Compile the test-support kernels that check libmoe's device code paths
    exhaustively (tests/kernels/*.hip) into tests/kernels/libfp8_path_check.so."""
    if not force and os.path.exists(TEST_LIB):
        return TEST_LIB
    tmp = TEST_LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wno-unused-command-line-argument", "-I", CSRC, "-I", os.path.join(ROOT, "include"),
           "-o", tmp, os.path.join(TEST_KERNELS, "fp8_path_check.hip")]
    subprocess.run(cmd, check=True, stdout=subprocess.DEVNULL, stderr=subprocess.PIPE)
    os.replace(tmp, TEST_LIB)
    return TEST_LIB


def build(force: bool = True, verbose: bool = False) -> str:
    """Compile every HIP source into combine_topk_ids_amd/libmoe.so."""
    if not force and os.path.exists(LIB):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=PKG, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(force=True, verbose=True))
    print(build_test_kernels(force=True))
