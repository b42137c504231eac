"""Calls from several host threads at once, each on a stream of its own, over
every kernel path: the tuned row kernel, the split kernel (which orders its
calls on one device through a stream hand-off), the any-H kernel with staged
rows (whose dynamic-LDS limit is set at first use) and the masked any-H
kernel.  The binding's calls release the interpreter lock, so the host side
of the library runs concurrently.  Every result must equal, bit for bit,
the same call made alone: the kernels reduce in a fixed order."""
import threading

import numpy as np
import pytest
import torch

from kimi_k3_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

CASES = [
    dict(T=64, nb=8, widx=3),                 # tuned row kernel
    dict(T=4, nb=8, widx=-1),                 # split kernel
    dict(T=900, nb=6, H=5632, widx=5),        # any-H, three bank rows staged in LDS
    dict(T=100, nb=4, H=2880, widx=-1),       # any-H, masked rows
]
ROUNDS = 4


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_harness
    return gpu_harness


def test_concurrent_calls_from_threads(G):
    cases = [W.Case(f"threads_{k}", seed=90 + k, **kw) for k, kw in enumerate(CASES)]
    inputs = [W.make_inputs(c) for c in cases]
    # Each call alone, one after another: the expected results.
    want = []
    for c, inp in zip(cases, inputs):
        G.say(c.name, "alone")
        d = G.upload(inp)
        G.run(d)
        want.append(G.download(d))

    errors = []
    got = {}
    # Created here and kept until the end: the split path waits on the stream
    # of the previous split call, which must therefore outlive the threads.
    streams = [torch.cuda.Stream() for _ in cases]

    def worker(k):
        try:
            s = streams[k]
            for r in range(ROUNDS):
                with torch.cuda.stream(s):
                    d = G.upload(inputs[k])
                    s.synchronize()
                    G.run(d, stream=s)
                    s.synchronize()
                    got[(k, r)] = G.download(d)
        except Exception as e:  # reported by the main thread
            errors.append((k, repr(e)))

    G.say("threads: start")
    threads = [threading.Thread(target=worker, args=(k,)) for k in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    # A last split call on the current stream, so that the next split call
    # does not wait on a thread's stream once it is gone.
    G.run(G.upload(inputs[1]))
    torch.cuda.synchronize()
    from kimi_k3_attention_amd import attnres as A
    assert A.attnres_device_status() == 0
    for (k, r), res in sorted(got.items()):
        w = want[k]
        assert np.array_equal(res.out, w.out), f"{cases[k].name} round {r}: out"
        assert np.array_equal(res.prefix, w.prefix), f"{cases[k].name} round {r}: prefix"
        assert np.array_equal(res.bank, w.bank), f"{cases[k].name} round {r}: bank"
    assert len(got) == len(cases) * ROUNDS
