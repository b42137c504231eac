"""The library from plain C on the GPU: tests/c/abi_check allocates device
buffers with the HIP runtime, calls attnres_fwd_path on every kernel path
and compares with the C oracle; it exits 0 only when every case passes."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "abi_check")


def test_plain_c_caller_matches_oracle():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(EXE):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "build_abi_check", os.path.join(ROOT, "tests", "c", "build_abi_check.py"))
        cbuild = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(cbuild)
        cbuild.build()
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ALL PASS" in res.stdout
