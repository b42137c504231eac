"""A call whose kernel needs more dynamic LDS than the runtime's default
limit (the any-H kernel with staged rows at four segments per lane) made
first inside hipGraph capture, in a fresh process that never called
attnres_init: the library sets the kernel's limit then, during capture.
Every replay must match the same call made eagerly, and the library's
status must stay clean.  Runs in a child process, since the library sets
each kernel's limit once per process."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
from kimi_k3_attention_amd import attnres as A
from kimi_k3_attention_amd import workloads as W
from tests import gpu_harness as G

# H = 12288: 6 waves of four segments per lane; T = 300 stages three bank rows
# (72 KB of LDS per workgroup).
# No delta and no bank write, so that every replay computes the same thing.
case = W.Case("first_call_in_capture", T=300, nb=8, H=12288, widx=-1, has_delta=False, seed=5)
inp = W.make_inputs(case)
print("case", case.name, flush=True)
d = G.upload(inp)
s = torch.cuda.Stream()
g = torch.cuda.CUDAGraph()
s.wait_stream(torch.cuda.current_stream())
with torch.cuda.stream(s):
    with torch.cuda.graph(g, stream=s):
        G.run(d, stream=s)
torch.cuda.synchronize()
print("captured", flush=True)
e = G.upload(inp)
G.run(e)
torch.cuda.synchronize()
ref = G.download(e)
for rep in range(3):
    d.out.fill_(0x7F81)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    got = G.download(d)
    assert (got.out == ref.out).all(), "replay %d differs from the eager call" % rep
    print("replay", rep, "ok", flush=True)
assert A.attnres_device_status() == 0
print("ok", flush=True)
"""


def test_first_staged_call_inside_capture():
    if "torch" in sys.modules:
        import torch
        if not torch.cuda.is_available():
            pytest.skip("no GPU")
    res = subprocess.run([sys.executable, "-u", "-c", CHILD, ROOT], capture_output=True,
                         text=True, timeout=300, cwd=ROOT)
    out = res.stdout + res.stderr
    assert res.returncode == 0 and res.stdout.rstrip().endswith("ok"), out[-3000:]
