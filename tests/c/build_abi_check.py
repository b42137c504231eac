"""Builds tests/c/abi_check (a plain-C caller of libattnres checked against
the C oracle) with gcc against the built libattnres.so and liboracle_attnres.so.

    python tests/c/build_abi_check.py
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_check.c")
EXE = os.path.join(HERE, "abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    tmp = EXE + ".tmp"
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           SRC, "-o", tmp,
           "-L", os.path.join(ROOT, "kimi_k3_attention_amd"), "-lattnres",
           "-L", os.path.join(ROOT, "oracle"), "-loracle_attnres",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../kimi_k3_attention_amd:$ORIGIN/../../oracle:"
           + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("building abi_check failed:\n" + res.stderr[-4000:])
    if verbose and res.stderr.strip():
        print(res.stderr, file=sys.stderr)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
