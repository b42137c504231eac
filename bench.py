#!/usr/bin/env python3
"""Benchmark of the Kimi-K3 attention-residual forward (libattnres) on one
MI355X.

A step is one attnres_fwd call over one batch of synthetic input.  The
headline workload is the mid prefill: T=1024 tokens, 8 block rows, H=7168,
delta and output norm on, block_write_idx=3.  A hipGraph holds exactly
--steps calls, cycling over input sets whose total footprint exceeds the
256 MB Infinity Cache, with inputs resident in HBM; a timed sample replays it
back to back until the sample covers at least 600 calls.  `value` is the algorithmic HBM rate (rows read + rows written + weight
rows, bytes per call) divided by the measured time per call.

Also reported: the single-token decode sweep (T=1, 0/1/4/8 block rows; the
pages' single-token latency metric) as microseconds per call, cold (rotating
over ~2400 input sets) and warm (one set), and the fp64 CPU oracle timed on
the host (the CPU baseline).

    python bench.py [--steps K] [--warmup W] [--gpus 1]
    python bench.py --eager --only mid --steps 20   # plain launches, for counters
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from kimi_k3_attention_amd import attnres as A  # noqa: E402
from kimi_k3_attention_amd import workloads as W  # noqa: E402

METRIC = "AttnRes µs/call (T=1, 0/4/8 blk) + achieved HBM GB/s at T=1024, 8 blk, H=7168"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
# The mid-prefill call's kernel: 8 block rows, delta, output norm, and the
# two rewritten rows read through the cache (T >= 1024, written slot 3 < 8).
DOMINANT_KERNEL = "attnres_row_kernel<8, true, true, true, false>"
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "attnres_row_kernel_mid_prefill_T1024_traffic.json")
CALIBRATION_BYTES = 512 << 20
# Calls per timed sample of the headline and of the traffic probe: enough
# that the fixed start-up cost of a graph replay (~50 us) is under 0.3 % of
# the sample at any --steps.
MIN_TIMED_CALLS = 600
KERNEL_SOURCES = [os.path.join(ROOT, "kimi_k3_attention_amd", "csrc", f)
                  for f in ("attnres_kernels.hip", "attnres_internal.h")]


def log(*msg):
    print("[bench]", *msg, file=sys.stderr, flush=True)


# The kernels' device code ends where the launch layer begins; host-only
# changes below this line (entry points, workspace handling) leave the
# measured kernels, hence their committed counters, valid.
DEVICE_CODE_END = b"// specialisation tables"


def code_only(text: bytes) -> bytes:
    """C++ source without its comments and layout: // and /* */ comments
    (outside string and character literals) removed, runs of spaces and tabs
    made one space, lines stripped and blank lines dropped.  Line breaks
    stay, since preprocessor lines end at them."""
    out = bytearray()
    i, n = 0, len(text)
    quote = None
    while i < n:
        c = text[i:i + 1]
        if quote:
            out += c
            if c == b"\\" and i + 1 < n:
                out += text[i + 1:i + 2]
                i += 2
                continue
            if c == quote:
                quote = None
            i += 1
        elif c in (b'"', b"'"):
            quote = c
            out += c
            i += 1
        elif text.startswith(b"//", i):
            j = text.find(b"\n", i)
            i = n if j < 0 else j
        elif text.startswith(b"/*", i):
            j = text.find(b"*/", i + 2)
            i = n if j < 0 else j + 2
            out += b" "
        else:
            out += c
            i += 1
    lines = (b" ".join(l.split()) for l in bytes(out).split(b"\n"))
    return b"\n".join(l for l in lines if l)


def kernel_source_hash() -> str:
    """Hash of the kernels' device code: the kernel source up to the launch
    layer, and the internal header, without comments or layout (an edit of a
    comment leaves the measured kernels, hence their profiles, valid)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            text = fh.read()
        if f.endswith(".hip"):
            end = text.find(DEVICE_CODE_END)
            if end < 0:
                raise RuntimeError(f"{f}: no '{DEVICE_CODE_END.decode()}' marker")
            text = text[:end]
        h.update(code_only(text))
    return h.hexdigest()[:16]


def to_dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


class Set:
    """One resident input set of a workload."""

    def __init__(self, inp: W.Inputs):
        c = inp.case
        self.case = c
        self.prefix = to_dev(inp.prefix)
        self.delta = to_dev(inp.delta)
        self.bank = to_dev(inp.bank)
        self.bank3 = self.bank.as_strided((c.T, c.cap, c.H), (c.token_stride, c.slot_stride, 1))
        self.res_w = to_dev(inp.res_w)
        self.rms_w = to_dev(inp.rms_w)
        self.onw = to_dev(inp.onw)
        self.out = to_dev(inp.out_init)
        if self.delta is not None:
            self.delta.zero_()  # repeated in-place calls stay a fixed point

    def call(self, nb=None, token=None, path=None, ntok=1):
        """The whole set, or the ntok tokens from `token` on."""
        c = self.case
        nb = c.nb if nb is None else nb
        if token is None:
            A.attnres_fwd(self.prefix, self.delta, self.bank3, nb, self.res_w, self.rms_w, c.eps,
                          self.onw, c.oeps, c.widx, self.out, path=path)
        else:
            sl = slice(token, token + ntok)
            A.attnres_fwd(self.prefix[sl], None if self.delta is None else self.delta[sl],
                          self.bank3[sl], nb, self.res_w, self.rms_w, c.eps, self.onw, c.oeps,
                          c.widx, self.out[sl], path=path)


def time_graph(calls, steps: int, replays: int = 1, warm: int = 1, min_calls: int = 0,
               stream=None):
    """Captures `steps` calls (cycling over `calls`) into one hipGraph and
    returns, for each of `replays` timed samples, the elapsed ms per graph
    replay, after `warm` untimed replays (graph upload, first touch of the
    buffers).  A sample replays the graph R = ceil(min_calls / steps) times
    back to back between one pair of hipEvents on the launch stream, with no
    host synchronisation inside, so the graph's fixed start-up cost is spread
    over at least `min_calls` calls whatever `steps` is; the sample's time is
    divided by R.  `stream`: the stream to capture on (torch's own by
    default)."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=stream):
        for i in range(steps):
            calls[i % len(calls)]()
    torch.cuda.synchronize()
    for _ in range(warm):
        g.replay()
    torch.cuda.synchronize()
    reps = graph_repeats(steps, min_calls)
    times = []
    stream = torch.cuda.current_stream()
    for _ in range(replays):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / reps)
    del g
    return times


def graph_repeats(steps: int, min_calls: int) -> int:
    """The R that time_graph uses: graph replays per timed sample."""
    return max(1, -(-min_calls // steps))


def time_eager(calls, steps: int):
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        calls[i % len(calls)]()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def pct(xs, q):
    return float(np.percentile(np.asarray(xs), q))


def calibration_copy(nbytes: int = CALIBRATION_BYTES, reps: int = 3):
    """A plain device copy of known size, for scaling the memory-traffic
    counters (FETCH_SIZE / WRITE_SIZE) of the same profiling run."""
    src = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration copy: {reps} x {nbytes} bytes read + written")


def bench_mid(steps: int, warmup: int, eager: bool):
    case = W.mid_prefill()
    per_call_bytes = case.algorithmic_bytes()
    footprint = 2 * case.T * case.H * (case.cap + 3)
    nsets = max(1, -(-2 * MALL_BYTES // footprint))
    log(f"mid prefill: {nsets} input sets of {footprint / 1e6:.0f} MB, {per_call_bytes} B/call")
    sets = [Set(W.make_inputs(W.with_(case, seed=case.seed + 100 * r))) for r in range(nsets)]
    calls = [s.call for s in sets]
    for i in range(warmup):
        calls[i % len(calls)]()
    torch.cuda.synchronize()
    if eager:
        ms = time_eager(calls, steps)
        reps = [ms]
    else:
        # Six timed samples after three untimed replays (the first ~20 ms
        # after building the inputs run a few percent slow).  The graph holds
        # exactly `steps` calls; each sample replays it back to back until it
        # covers at least MIN_TIMED_CALLS calls, so the graph's start-up cost
        # does not depend on `steps`.  The median sample is reported.
        reps = time_graph(calls, steps, replays=6, warm=3, min_calls=MIN_TIMED_CALLS)
        ms = pct(reps, 50)
    repeats = 1 if eager else graph_repeats(steps, MIN_TIMED_CALLS)
    per_call_ms = ms / steps
    per_call = [r / steps * 1e3 for r in reps]
    gbps = per_call_bytes / (per_call_ms * 1e-3) / 1e9
    log(f"mid prefill: {per_call_ms * 1e3:.2f} us/call, {gbps:.0f} GB/s "
        f"({repeats} x {steps} calls per timed sample)")
    return dict(case=case, sets=sets, per_call_ms=per_call_ms, gbps=gbps, bytes=per_call_bytes,
                us=dict(p20=pct(per_call, 20), p50=pct(per_call, 50), p80=pct(per_call, 80)),
                nsets=nsets, calls_timed=repeats * steps, graph_repeats=repeats)


def bench_decode(steps: int):
    """T=1: cold (a different input set per call, ~2400 sets > MALL) and warm
    (one set), for 0/1/4/8 block rows."""
    n = 2400
    case = W.Case("decode_sets", T=n, nb=8, recipe="decode", seed=1)
    s = Set(W.make_inputs(case))
    res = {}
    for nb in (0, 1, 4, 8):
        cold = [lambda t=t, nb=nb: s.call(nb=nb, token=t) for t in range(n)]
        warm = [lambda nb=nb: s.call(nb=nb, token=0)]
        for fn in cold[:50]:
            fn()
        k = max(steps, n)
        tc = time_graph(cold, k, replays=5)
        tw = time_graph(warm, k, replays=5)
        res[f"nb{nb}"] = dict(cold_us=pct([t / k * 1e3 for t in tc], 50),
                              warm_us=pct([t / k * 1e3 for t in tw], 50),
                              bytes=W.Case("x", T=1, nb=nb).algorithmic_bytes())
        log(f"decode nb={nb}: cold {res[f'nb{nb}']['cold_us']:.2f} us, warm {res[f'nb{nb}']['warm_us']:.2f} us")
    return res


LATENCY_TOKENS = (1, 8, 16, 24, 32, 40, 48, 56, 64, 80, 96, 128)


def bench_latency_grid(n: int = 4096):
    """Small batches: us per call of T tokens through the row kernel and the
    split kernel (both forced), num_blocks 0..8, delta and output norm on.
    Consecutive calls take consecutive T-token windows of one resident
    4096-token input (decode recipe, ~650 MB, above the Infinity Cache), so
    every call reads cold rows; hipGraph replay of at least 512 calls."""
    case = W.Case("latency_grid", T=n, nb=8, recipe="decode", seed=1)
    s = Set(W.make_inputs(case))
    grid = {}
    for T in LATENCY_TOKENS:
        windows = n // T
        steps = max(windows, 512)
        row = {}
        for nb in range(9):
            cell = {}
            for name, path in (("row", A.ATTNRES_PATH_ROW), ("split", A.ATTNRES_PATH_SPLIT)):
                calls = [lambda w=w, nb=nb, path=path: s.call(nb=nb, token=w * T, path=path, ntok=T)
                         for w in range(windows)]
                t = time_graph(calls, steps, replays=3)
                cell[name] = round(pct([x / steps * 1e3 for x in t], 50), 3)
            row[f"nb{nb}"] = cell
        grid[f"T{T}"] = row
        log(f"latency grid T={T}: " + " ".join(
            f"nb{k}:{row[f'nb{k}']['row']:.2f}/{row[f'nb{k}']['split']:.2f}" for k in range(9)))
    return grid


def bench_long(steps: int = 20):
    """Long prefill (T=8192 and 4096, padded bank, heavy-tailed rows, no delta,
    no norm): reported as extra information, one resident set each (the 1.2 GB
    and 0.6 GB footprints exceed the Infinity Cache)."""
    res = {}
    for T in (8192, 4096):
        case = W.long_prefill(T)
        s = Set(W.make_inputs(case))
        s.call()
        torch.cuda.synchronize()
        # Right after the input is built, the first ~20 ms of calls run a few
        # percent slow; five untimed replays cover that.
        t = time_graph([s.call], steps, replays=5, warm=5)
        us = pct([x / steps * 1e3 for x in t], 50)
        res[f"T{T}"] = dict(us=round(us, 2), GBps=round(case.algorithmic_bytes() / us / 1e3, 1),
                            frac=round(case.algorithmic_bytes() / us / 1e3 / HBM_PEAK_GBPS, 4))
        log(f"long prefill T={T}: {us:.1f} us, {res[f'T{T}']['GBps']:.0f} GB/s")
        del s
        torch.cuda.empty_cache()
    return res


OVERLAP_TOKENS = (1, 4, 16, 64)


def bench_overlap(n: int = 4096, steps: int = 1200):
    """The two-kernel form beside a producer of delta, against the one-kernel
    call after it.  A step is the producer (delta = x W, a [T, 7168] x
    [7168, 7168] bf16 product, the shape of a projection that produces the
    residual update) followed by the attention-residual call of the same T
    tokens (8 or 4 block rows, delta and output norm).  Three graphs of `steps`
    steps are timed: the producer alone; producer -> attnres_fwd; and, per
    step, a fork: attnres_fwd_bank on a side branch while the producer runs,
    joined before attnres_fwd_cur.  The exposed attention-residual time is a
    graph's time per step minus the producer's.  Consecutive steps take
    consecutive T-token windows of one resident input (decode recipe)."""
    case = W.Case("overlap", T=n, nb=8, recipe="decode", seed=1)
    st = Set(W.make_inputs(case))
    H = case.H
    gen = torch.Generator(device="cuda").manual_seed(5)
    x = (0.01 * torch.randn(n, H, device="cuda", generator=gen)).to(torch.bfloat16)
    wmat = (torch.randn(H, H, device="cuda", generator=gen) / H ** 0.5).to(torch.bfloat16)
    delta = st.delta.view(torch.bfloat16)
    # The matrix product's library sets itself up on first use on a stream,
    # which graph capture does not allow: run it once on the capture stream.
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        for T in OVERLAP_TOKENS:
            torch.mm(x[:T], wmat, out=delta[:T])
    torch.cuda.synchronize()
    res = {}
    for T in OVERLAP_TOKENS:
        windows = n // T
        nbytes = A.attnres_partial_bytes(T, H)
        # one partial-state buffer per window, each 256-byte aligned
        parts = torch.empty(windows, -(-nbytes // 256) * 64, dtype=torch.float32, device="cuda")
        side = torch.cuda.Stream()
        for nb in (8, 4):
            def args(w, nb=nb):
                sl = slice(w * T, (w + 1) * T)
                return (st.prefix[sl], st.delta[sl], st.bank3[sl], nb, st.res_w, st.rms_w,
                        case.eps, st.onw, case.oeps, -1, st.out[sl])

            def produce(w):
                sl = slice(w * T, (w + 1) * T)
                torch.mm(x[sl], wmat, out=delta[sl])

            def chain(w):
                produce(w)
                A.attnres_fwd(*args(w))

            def fork(w):
                main = torch.cuda.current_stream()
                side.wait_stream(main)
                with torch.cuda.stream(side):
                    A.attnres_fwd_bank(*args(w), parts[w], stream=side)
                produce(w)
                main.wait_stream(side)
                A.attnres_fwd_cur(*args(w), parts[w], stream=main)

            cell = {}
            for name, fn in (("producer", produce), ("chain", chain), ("two_kernel", fork)):
                calls = [lambda w=w, fn=fn: fn(w) for w in range(windows)]
                with torch.cuda.stream(cap):
                    for c in calls[:4]:
                        c()
                torch.cuda.synchronize()
                t = time_graph(calls, min(steps, max(windows, 300)), replays=3, warm=2,
                               stream=cap)
                k = min(steps, max(windows, 300))
                cell[name] = round(pct([v / k * 1e3 for v in t], 50), 3)
            cell["exposed_chain"] = round(cell["chain"] - cell["producer"], 3)
            cell["exposed_two_kernel"] = round(cell["two_kernel"] - cell["producer"], 3)
            cell["saved_per_step"] = round(cell["chain"] - cell["two_kernel"], 3)
            res[f"T{T}_nb{nb}"] = cell
            log(f"overlap T={T} nb={nb}: " + ", ".join(f"{k} {v}" for k, v in cell.items()))
        del parts
    res["extra_bytes_per_token"] = 2 * 4 * H + 8  # u written and read back, (m, s)
    return res


def _host_threads() -> int:
    """Host threads for the multi-threaded oracle leg: the CPUs this process
    may run on, at most 16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


HIDDEN_SWEEP = (2048, 2880, 4096, 5120, 7168, 8192, 9216, 11264, 12288, 16384)


def anyh_threads(H: int) -> int:
    """Lanes per workgroup of the library's any-H kernel at hidden size H:
    whole waves of two segments per lane up to 1024 segments, else four."""
    nseg = H // 8
    spl = 2 if nseg <= 1024 else 4
    return -(-nseg // (64 * spl)) * 64


def probe_mid_h(H: int, T: int, cached: bool, steps: int = 120):
    """The traffic probe of the mid-prefill pattern at hidden size H in the
    any-H kernel's launch shape: us per call (graph replay over enough
    buffers to exceed the Infinity Cache)."""
    lib = load_ceiling_probe()
    per_set = 2 * H * T * 11
    sets = []
    for _ in range(max(2, -(-2 * MALL_BYTES // per_set))):
        sets.append(tuple(torch.randint(-30000, 30000, (n * H,), dtype=torch.int16, device="cuda")
                          for n in (T * 8, T, T)) + (torch.empty(T * H, dtype=torch.int16,
                                                                 device="cuda"),))

    def call(st):
        rc = lib.ceiling_mid_h(st[0].data_ptr(), st[1].data_ptr(), st[2].data_ptr(),
                               st[3].data_ptr(), T, H, anyh_threads(H), int(cached),
                               torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"ceiling_mid_h failed ({rc})")

    calls = [lambda st=st: call(st) for st in sets]
    for fn in calls:
        fn()
    torch.cuda.synchronize()
    t = time_graph(calls, steps, replays=3, min_calls=MIN_TIMED_CALLS)
    del sets
    torch.cuda.empty_cache()
    return pct([x / steps * 1e3 for x in t], 50)


def bench_hidden_sweep(Hs=HIDDEN_SWEEP, T: int = 1024, steps: int = 120):
    """The mid-prefill recipe (T=1024, 8 block rows, delta, output norm,
    block_write_idx=3) at other hidden sizes, run by the any-H row kernel
    (and, at 7168, also by the tuned row kernel): per-call time from graph
    replay over enough resident input sets to exceed the Infinity Cache."""
    res = {}
    for H in Hs:
        case = W.Case(f"hidden{H}_T{T}_nb8", T=T, nb=8, H=H, widx=3, seed=2)
        footprint = 2 * T * H * (case.cap + 3)
        nsets = max(1, -(-2 * MALL_BYTES // footprint))
        sets = [Set(W.make_inputs(W.with_(case, seed=case.seed + 100 * r))) for r in range(nsets)]
        nbytes = case.algorithmic_bytes()
        paths = {"any_h": A.ATTNRES_PATH_ANY_H}
        if H == 7168:
            paths["tuned_row"] = A.ATTNRES_PATH_ROW
        entry = {"bytes_per_call": nbytes, "input_sets": nsets}
        for name, path in paths.items():
            calls = [lambda st=st, path=path: st.call(path=path) for st in sets]
            for fn in calls:
                fn()
            torch.cuda.synchronize()
            t = time_graph(calls, steps, replays=3)
            us = pct([x / steps * 1e3 for x in t], 50)
            gbps = nbytes / us / 1e3
            entry[name] = dict(us=round(us, 2), GBps=round(gbps, 1),
                               frac=round(gbps / HBM_PEAK_GBPS, 4))
            log(f"hidden sweep H={H} {name}: {us:.2f} us, {gbps:.0f} GB/s")
        del sets
        torch.cuda.empty_cache()
        # The same rows moved with no arithmetic, in the any-H launch shape and
        # the cache policy the kernel uses for this size.
        cached = T * H >= 1024 * 7168
        pus = probe_mid_h(H, T, cached)
        entry["traffic_probe"] = dict(us=round(pus, 2), cached_rewritten_rows=cached,
                                      frac=round(nbytes / pus / 1e3 / HBM_PEAK_GBPS, 4),
                                      any_h_fraction_of_probe=round(pus / entry["any_h"]["us"], 4))
        log(f"hidden sweep H={H} probe: {pus:.2f} us")
        res[str(H)] = entry
    return res


def bench_variant_sweep(T: int = 1024, windows: int = 4, steps: int = 120):
    """T=1024 calls for every num_blocks 0..8 x delta x output norm (write slot
    nb-1, or none at nb=0), each rotating over `windows` token windows of one
    resident 4096-token input (footprint above the Infinity Cache)."""
    case = W.Case("variant_sweep", T=T * windows, nb=8, widx=-1, seed=11)
    s_all = Set(W.make_inputs(case))
    H = case.H
    res = {}
    for nb in range(9):
        for d in (False, True):
            for o in (False, True):
                widx = nb - 1 if nb > 0 else -1
                c = W.Case("v", T=T, nb=nb, has_delta=d, has_onorm=o, widx=widx)
                nbytes = c.algorithmic_bytes()

                def call(w, nb=nb, d=d, o=o, widx=widx):
                    sl = slice(w * T, (w + 1) * T)
                    A.attnres_fwd(s_all.prefix[sl], s_all.delta[sl] if d else None,
                                  s_all.bank3[sl], nb, s_all.res_w, s_all.rms_w, case.eps,
                                  s_all.onw if o else None, case.oeps, widx, s_all.out[sl])

                calls = [lambda w=w: call(w) for w in range(windows)]
                for fn in calls:
                    fn()
                torch.cuda.synchronize()
                t = time_graph(calls, steps, replays=3)
                us = pct([x / steps * 1e3 for x in t], 50)
                gbps = nbytes / us / 1e3
                key = f"nb{nb}_d{int(d)}_o{int(o)}"
                res[key] = dict(us=round(us, 2), GBps=round(gbps, 1),
                                frac=round(gbps / HBM_PEAK_GBPS, 4))
                log(f"variant {key}: {us:.2f} us, {gbps:.0f} GB/s")
    return res


def bench_configs(steps_min: int = 200):
    """The reference case (T=4, nb=4, delta and output norm) and the 80-case
    variant matrix (T in 1/16/256/2048 x nb in 0/4/8 x delta x output norm x
    write slot in -1/nb-1), each as µs per call and algorithmic GB/s: one
    resident input per T, its tokens split into windows of T that the graph
    replay rotates over, enough of them to exceed the Infinity Cache."""
    H = W.HIDDEN
    res = {}
    for T in (1, 4, 16, 256, 2048):
        per_window = 2 * T * H * 11  # 8 bank slots, prefix, delta, out
        windows = max(4, -(-2 * MALL_BYTES // per_window))
        big = W.Case(f"configs_T{T}", T=T * windows, nb=8, widx=-1, seed=12)
        s_all = Set(W.make_inputs(big))
        cases = [W.pr1_ref()] if T == 4 else [c for c in W.variant_matrix() if c.T == T]
        for c in cases:
            def call(w, c=c):
                sl = slice(w * T, (w + 1) * T)
                A.attnres_fwd(s_all.prefix[sl], s_all.delta[sl] if c.has_delta else None,
                              s_all.bank3[sl], c.nb, s_all.res_w, s_all.rms_w, c.eps,
                              s_all.onw if c.has_onorm else None, c.oeps, c.widx, s_all.out[sl])

            calls = [lambda w=w: call(w) for w in range(windows)]
            for fn in calls[:8]:
                fn()
            torch.cuda.synchronize()
            steps = max(steps_min, windows)
            t = time_graph(calls, steps, replays=3, warm=2)
            us = pct([x / steps * 1e3 for x in t], 50)
            gbps = c.algorithmic_bytes() / us / 1e3
            res[c.name] = dict(T=T, nb=c.nb, delta=c.has_delta, onorm=c.has_onorm, widx=c.widx,
                               us=round(us, 3), GBps=round(gbps, 1),
                               frac=round(gbps / HBM_PEAK_GBPS, 4))
            log(f"config {c.name}: {us:.3f} us, {gbps:.0f} GB/s")
        del s_all
        torch.cuda.empty_cache()
    return res


CEILING_SRC = os.path.join(ROOT, "bench_ceiling.hip")
CEILING_LIB = os.path.join(ROOT, "bench_ceiling.so")
# The mid-prefill call's own buffers and row roles (ceiling_mid): 8 bank rows,
# prefix and delta read; out, prefix and bank slot 3 written; the two
# rewritten rows read through the cache (as the library's row kernel does for
# this call) or streamed.
CEILING_MID_CONFIGS = (("mid_prefill_cached", 1), ("mid_prefill_streamed", 0))
# (name, row reads, row writes to a separate buffer, row writes in place) per
# token, every row of a token in one buffer, every row streamed.
CEILING_CONFIGS = (("one_buffer_10r_1w_2inplace", 10, 1, 2), ("10r_3w", 10, 3, 0),
                   ("long_prefill_9r_1w", 9, 1, 0), ("read_only_10r", 10, 0, 0),
                   ("copy_1r_1w", 1, 1, 0))


def build_ceiling_probe(verbose: bool = False) -> str:
    """Compiles bench_ceiling.hip (the memory-traffic probe) in-tree."""
    import subprocess
    from kimi_k3_attention_amd import build as kbuild
    tmp = CEILING_LIB + ".tmp"
    cmd = [kbuild.HIPCC] + kbuild.FLAGS + ["-o", tmp, CEILING_SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on the ceiling probe:\n" + res.stderr[-4000:])
    os.replace(tmp, CEILING_LIB)
    return CEILING_LIB


def load_ceiling_probe():
    import ctypes
    if not os.path.exists(CEILING_LIB):
        build_ceiling_probe()
    lib = ctypes.CDLL(CEILING_LIB)
    vp, i64, ci, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_uint32
    lib.ceiling_stream.argtypes = [vp, i64, vp, i64, ci, ci, ci, i64, u32, vp]
    lib.ceiling_mid.argtypes = [vp, vp, vp, vp, i64, ci, vp]
    lib.ceiling_mid.restype = ci
    lib.ceiling_mid_h.argtypes = [vp, vp, vp, vp, i64, i64, ci, ci, vp]
    lib.ceiling_mid_h.restype = ci
    lib.ceiling_stream.restype = ci
    return lib


def bench_ceiling(steps: int = 300, call_bytes: int = 190883840, H: int = 7168,
                  eager: bool = False):
    """The traffic of a call without its arithmetic (bench_ceiling.hip), in the
    row kernel's launch shape, over enough input sets to exceed the Infinity
    Cache: the rate this access pattern reaches on the device.  Each
    configuration moves about `call_bytes` per launch (the mid-prefill call's
    bytes), so the token count differs between configurations."""
    lib = load_ceiling_probe()
    res = {}
    T = round(call_bytes / (2 * H * 13))
    for name, cached in CEILING_MID_CONFIGS:
        per_set = 2 * H * T * 11  # bank 8 rows + prefix + delta + out
        sets = []
        for _ in range(max(2, -(-2 * MALL_BYTES // per_set))):
            bank = torch.randint(-30000, 30000, (T * 8 * H,), dtype=torch.int16, device="cuda")
            pf = torch.randint(-30000, 30000, (T * H,), dtype=torch.int16, device="cuda")
            dl = torch.randint(-30000, 30000, (T * H,), dtype=torch.int16, device="cuda")
            out = torch.empty(T * H, dtype=torch.int16, device="cuda")
            sets.append((bank, pf, dl, out))

        def call_mid(st, cached=cached, name=name):
            rc = lib.ceiling_mid(st[0].data_ptr(), st[1].data_ptr(), st[2].data_ptr(),
                                 st[3].data_ptr(), T, cached, torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"ceiling probe {name} failed ({rc})")

        calls = [lambda st=st: call_mid(st) for st in sets]
        for fn in calls:
            fn()
        torch.cuda.synchronize()
        if eager:  # plain launches, one dispatch per call (for counter runs)
            t = [time_eager(calls, steps)]
        else:
            t = time_graph(calls, steps, replays=3, min_calls=MIN_TIMED_CALLS)
        us = pct([x / steps * 1e3 for x in t], 50)
        nbytes = 2 * H * T * 13
        res[name] = dict(T=T, us=round(us, 2), GBps=round(nbytes / us / 1e3, 1),
                         frac=round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4))
        log(f"ceiling probe {name}: {us:.2f} us, {nbytes / us / 1e3:.0f} GB/s")
        del sets
        torch.cuda.empty_cache()
    for name, reads, wd, wi in ([] if eager else CEILING_CONFIGS):
        T = max(1, round(call_bytes / (2 * H * (reads + wd + wi))))
        footprint = 2 * H * T * (reads + wd)
        nsets = max(1, -(-2 * MALL_BYTES // footprint))
        sets = []
        for _ in range(nsets):
            src = torch.randint(-30000, 30000, (T * reads * H,), dtype=torch.int16, device="cuda")
            dst = torch.empty(max(T * wd * H, 8), dtype=torch.int16, device="cuda")
            sets.append((src, dst))

        def call(st):
            rc = lib.ceiling_stream(st[0].data_ptr(), reads * H, st[1].data_ptr(), max(wd, 1) * H,
                                    reads, wd, wi, T, 0x9E3779B9,
                                    torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"ceiling probe {name} failed ({rc})")

        calls = [lambda st=st: call(st) for st in sets]
        for fn in calls:
            fn()
        torch.cuda.synchronize()
        t = time_graph(calls, steps, replays=3, min_calls=MIN_TIMED_CALLS)
        us = pct([x / steps * 1e3 for x in t], 50)
        nbytes = 2 * H * T * (reads + wd + wi)
        res[name] = dict(T=T, us=round(us, 2), GBps=round(nbytes / us / 1e3, 1),
                         frac=round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4))
        log(f"ceiling probe {name}: {us:.2f} us, {nbytes / us / 1e3:.0f} GB/s")
        del sets
        torch.cuda.empty_cache()
    return res


def _host_cpu() -> dict:
    """The host's CPU model and logical CPU counts (reported with the CPU leg)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = None
    return {"model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


def cpu_baseline(single_s: float = 8.0, multi_s: float = 1.5):
    """The fp64 oracle, as it stands, on the host, on whole mid-prefill calls
    (T=1024, 8 block rows): single-threaded for about single_s, then with the
    call's tokens split into contiguous ranges run by a pool of threads (the
    C oracle runs without the GIL) for about multi_s of wall time."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    case = W.mid_prefill()
    inp = W.make_inputs(case)
    ts = case.token_stride

    def run(a, b):
        oracle.attnres_oracle(inp.prefix[a:b], None if inp.delta is None else inp.delta[a:b],
                              inp.bank[a * ts:b * ts], ts, case.slot_stride, case.cap, case.nb,
                              inp.res_w, inp.rms_w, case.eps, inp.onw, case.oeps, case.widx)

    run(0, case.T)  # load / build
    t0 = time.perf_counter()
    calls = 0
    while True:
        run(0, case.T)
        calls += 1
        if time.perf_counter() - t0 >= single_s:
            break
    dt1 = (time.perf_counter() - t0) / calls
    gbps1 = case.algorithmic_bytes() / dt1 / 1e9
    log(f"cpu oracle, 1 thread: {dt1 * 1e3:.0f} ms/call, {gbps1:.3f} GB/s")

    n = _host_threads()
    bounds = [(case.T * k // n, case.T * (k + 1) // n) for k in range(n)]
    with ThreadPoolExecutor(max_workers=n) as pool:
        list(pool.map(lambda ab: run(*ab), bounds))
        t0 = time.perf_counter()
        mcalls = 0
        while True:
            list(pool.map(lambda ab: run(*ab), bounds))
            mcalls += 1
            if time.perf_counter() - t0 >= multi_s:
                break
        dtn = (time.perf_counter() - t0) / mcalls
    gbpsn = case.algorithmic_bytes() / dtn / 1e9
    log(f"cpu oracle, {n} threads: {dtn * 1e3:.0f} ms/call, {gbpsn:.3f} GB/s")
    return dict(value=round(gbpsn, 4), unit="GB/s", cores=n, kind="oracle",
                sample=f"{mcalls} whole calls of the T=1024 nb=8 workload, tokens split over {n} "
                       f"threads (C, fp64), {dtn * 1e3:.0f} ms/call; single-threaded: {calls} "
                       f"calls, {dt1 * 1e3:.0f} ms/call",
                single_thread=dict(value=round(gbps1, 4), unit="GB/s", cores=1,
                                   ms_per_call=round(dt1 * 1e3, 1)),
                ms_per_call=round(dtn * 1e3, 1), host=_host_cpu())


def kernel_trace_entry(nbytes: int):
    """The kernel-only figure from the committed rocprofv3 trace, labelled."""
    us = load_kernel_trace_us()
    if us is None:
        return None
    gbps = nbytes / us / 1e3
    return {"source": os.path.relpath(KERNEL_STATS_FILE, ROOT), "average_us": us,
            "GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4)}


def load_traffic():
    """HBM bytes per launch from the committed counter runs, if they were taken
    on the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


KERNEL_STATS_FILE = os.path.join(PROFILES, "attnres_row_kernel_mid_prefill_T1024_kernel_stats.txt")


def load_kernel_trace_us():
    """The dominant kernel's average duration (us) in the committed rocprofv3
    kernel-trace summary of the headline command, if that summary was taken
    on the current kernel source."""
    if not os.path.exists(KERNEL_STATS_FILE):
        return None
    with open(KERNEL_STATS_FILE) as f:
        lines = f.read().splitlines()
    if not any(l.startswith("# kernel source hash: " + kernel_source_hash()) for l in lines):
        return None
    for l in lines:
        parts = [x.strip() for x in l.split("|")]
        if len(parts) == 7 and parts[0] == DOMINANT_KERNEL:
            return float(parts[5])  # the per-dispatch trace's average
    return None


# ---------------------------------------------------------------------------
# rocprofv3 summaries (run on the CSV output of the profiling commands)
# ---------------------------------------------------------------------------

def _csv_rows(directory, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True)):
        with open(f, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _col(row, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(names)


def write_kernel_stats(trace_dir, out_name, title, command):
    """profiles/<out_name>: the kernel-trace statistics of one profiling run,
    then the libattnres dispatches grouped by kernel and workgroup size (one
    group per launch shape, e.g. per hidden size of the any-H kernel)."""
    os.makedirs(PROFILES, exist_ok=True)
    lines = [f"# rocprofv3 kernel statistics, {title}", f"# command: {command}",
             f"# kernel source hash: {kernel_source_hash()}",
             "# name | calls | average us | min us | max us | share %"]
    for r in _csv_rows(trace_dir, "kernel_stats.csv"):
        lines.append(" | ".join([_col(r, "Name", "KernelName")[:90], _col(r, "Calls"),
                                 f"{float(_col(r, 'AverageNs')) / 1e3:.3f}",
                                 f"{float(_col(r, 'MinNs')) / 1e3:.3f}", f"{float(_col(r, 'MaxNs')) / 1e3:.3f}",
                                 f"{float(_col(r, 'Percentage')):.2f}"]))
    groups = {}
    for r in _csv_rows(trace_dir, "kernel_trace.csv"):
        name = _col(r, "Kernel_Name")
        if "attnres" not in name:
            continue
        m = re.search(r"(attnres_\w+_kernel<[^>]*>)", name)
        short = m.group(1) if m else name[:60]
        key = (short, int(_col(r, "Workgroup_Size_X")), int(_col(r, "Grid_Size_X")),
               int(_col(r, "Scratch_Size")))
        groups.setdefault(key, []).append(
            (int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))) / 1e3)
    if groups:
        lines += ["#", "# libattnres dispatches by launch shape (from the per-dispatch trace)",
                  "# kernel | workgroup size | grid size (lanes) | scratch B/lane | "
                  "dispatches | average us | median us"]
        for (short, wg, grid, scr), ds in sorted(groups.items()):
            lines.append(" | ".join([short, str(wg), str(grid), str(scr), str(len(ds)),
                                     f"{float(np.mean(ds)):.3f}", f"{float(np.median(ds)):.3f}"]))
    with open(os.path.join(PROFILES, out_name), "w") as f:
        f.write("\n".join(lines) + "\n")


def summarize_profile(trace_dir, fetch_dir, write_dir, commands):
    """Writes the committed profiles/ summaries: the kernel-trace statistics
    and the HBM traffic per launch of the dominant kernel, scaled by what the
    same counters read for the plain copy of known size in the same run."""
    os.makedirs(PROFILES, exist_ok=True)
    src_hash = kernel_source_hash()
    write_kernel_stats(trace_dir, "attnres_row_kernel_mid_prefill_T1024_kernel_stats.txt",
                       "mid prefill T=1024 nb=8 (hipGraph replay)", commands.get("trace", "?"))

    def per_kernel(rows):
        out = {}
        for r in rows:
            name = _col(r, "Kernel_Name", "Kernel-Name", "KernelName")
            grid = int(float(_col(r, "Grid_Size", "Grid-Size", "GridSize")))
            val = float(_col(r, "Counter_Value", "Counter-Value", "CounterValue"))
            out.setdefault((name, grid), []).append(val)
        return out

    res = {}
    for tag, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        pk = per_kernel(_csv_rows(d, "counter_collection.csv"))
        ours = [v for (n, g), vals in pk.items() if DOMINANT_KERNEL in n for v in vals]
        # the calibration copy: the kernel whose counter reads about the copy size
        calib = [(n, g, float(np.median(v))) for (n, g), v in pk.items()
                 if "attnres" not in n and len(v) >= 3]
        calib = max(calib, key=lambda x: x[2])
        factor = (CALIBRATION_BYTES / 1024) / calib[2]
        res[tag] = dict(kernel_kib_median=float(np.median(ours)), dispatches=len(ours),
                        calibration_kernel=calib[0][:60], calibration_kib=calib[2],
                        calibration_known_kib=CALIBRATION_BYTES / 1024, scale=factor,
                        bytes_per_launch=float(np.median(ours)) * 1024 * factor)
    case = W.mid_prefill()
    total = res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"]
    out = dict(workload="mid prefill T=1024 nb=8 H=7168 delta+onorm widx=3", kernel=DOMINANT_KERNEL,
               kernel_source_hash=src_hash, commands=commands, counters=res,
               bytes_per_launch=round(total), algorithmic_bytes_per_launch=case.algorithmic_bytes(),
               ratio_to_algorithmic=round(total / case.algorithmic_bytes(), 4))
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def write_counter_summary(out_name, title, commands, runs):
    """profiles/<out_name>: the per-dispatch median of every counter of each
    counter run (rocprofv3 --pmc, counter_collection.csv), by kernel, for the
    libattnres kernels and the traffic probes, plus ratios derived from them.
    `runs` maps a run label to its output directory; a label "tag/name"
    puts "tag" before the kernel names of that run (e.g. two versions of one
    kernel side by side)."""
    os.makedirs(PROFILES, exist_ok=True)
    table = {}   # kernel -> counter -> [values]
    durations = {}
    for label, d in runs.items():
        for r in _csv_rows(d, "counter_collection.csv"):
            name = _col(r, "Kernel_Name", "Kernel-Name", "KernelName")
            m = re.search(r"((?:attnres_\w+_kernel|mid_kernel|ceiling_kernel)<[^>]*>)", name)
            if not m:
                continue
            k = m.group(1)
            if "/" in label:
                k = label.split("/", 1)[0] + " " + k
            ctr = _col(r, "Counter_Name", "Counter-Name", "CounterName")
            table.setdefault(k, {}).setdefault(ctr, []).append(
                float(_col(r, "Counter_Value", "Counter-Value", "CounterValue")))
            try:
                dur = (int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))) / 1e3
                durations.setdefault(k, {}).setdefault(
                    int(_col(r, "Dispatch_Id", "Dispatch-Id", "DispatchId")), dur)
            except (KeyError, ValueError):
                pass
    kernels = sorted(table)
    ctrs = sorted({c for k in kernels for c in table[k]})
    med = {k: {c: float(np.median(table[k][c])) for c in table[k]} for k in kernels}
    lines = [f"# rocprofv3 counters, {title}", f"# kernel source hash: {kernel_source_hash()}"]
    lines += [f"# command: {c}" for c in commands]
    lines += ["# per-dispatch medians; counter | " + " | ".join(kernels)]
    for c in ctrs:
        lines.append(" | ".join([c] + [f"{med[k][c]:.6g}" if c in med[k] else "-" for k in kernels]))

    def ratio(k, a, b):
        x, y = med[k].get(a), med[k].get(b)
        return None if x is None or not y else x / y

    derived = [
        ("wave lifetime, cycles (SQ_WAVE_CYCLES / SQ_WAVES)", "SQ_WAVE_CYCLES", "SQ_WAVES"),
        ("waves resident per busy cycle (SQ_LEVEL_WAVES / SQ_BUSY_CYCLES)", "SQ_LEVEL_WAVES",
         "SQ_BUSY_CYCLES"),
        ("share of wave time waiting on memory or a barrier (SQ_WAIT_ANY / SQ_WAVE_CYCLES)",
         "SQ_WAIT_ANY", "SQ_WAVE_CYCLES"),
        ("share of wave time waiting to issue (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES)",
         "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
        ("share of wave time issuing (SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES)", "SQ_ACTIVE_INST_ANY",
         "SQ_WAVE_CYCLES"),
        ("VALU issue per wave-cycle (SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES)", "SQ_ACTIVE_INST_VALU",
         "SQ_WAVE_CYCLES"),
        ("VALU instructions per wave (SQ_INSTS_VALU / SQ_WAVES)", "SQ_INSTS_VALU", "SQ_WAVES"),
        ("vector loads per wave (SQ_INSTS_VMEM_RD / SQ_WAVES)", "SQ_INSTS_VMEM_RD", "SQ_WAVES"),
        ("vector stores per wave (SQ_INSTS_VMEM_WR / SQ_WAVES)", "SQ_INSTS_VMEM_WR", "SQ_WAVES"),
        ("LDS instructions per wave (SQ_INSTS_LDS / SQ_WAVES)", "SQ_INSTS_LDS", "SQ_WAVES"),
        ("mean L2 read latency, cycles (TCP_TCC_READ_REQ_LATENCY_sum / TCP_TCC_READ_REQ_sum)",
         "TCP_TCC_READ_REQ_LATENCY_sum", "TCP_TCC_READ_REQ_sum"),
        ("mean L2 write latency, cycles (TCP_TCC_WRITE_REQ_LATENCY_sum / TCP_TCC_WRITE_REQ_sum)",
         "TCP_TCC_WRITE_REQ_LATENCY_sum", "TCP_TCC_WRITE_REQ_sum"),
        ("GPU busy cycles per dispatch (GRBM_GUI_ACTIVE)", "GRBM_GUI_ACTIVE", None),
    ]
    lines += ["#", "# derived (same dispatches' medians); quantity | " + " | ".join(kernels)]
    for label, a, b in derived:
        vals = [med[k].get(a) if b is None else ratio(k, a, b) for k in kernels]
        if all(v is None for v in vals):
            continue
        lines.append(" | ".join([label] + ["-" if v is None else f"{v:.4g}" for v in vals]))
    if durations:
        lines += ["#", "# dispatch duration under counter collection, median us | " +
                  " | ".join(kernels)]
        lines.append(" | ".join(["duration"] + [
            f"{float(np.median(list(durations[k].values()))):.3f}" if k in durations else "-"
            for k in kernels]))
    with open(os.path.join(PROFILES, out_name), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--eager", action="store_true", help="plain launches instead of a hipGraph")
    ap.add_argument("--only", choices=["mid", "decode", "ceiling"], default=None)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--calibrate", action="store_true", help="run the known-size copy for counters")
    ap.add_argument("--hidden-sweep", action="store_true",
                    help="only the T=1024 mid-prefill recipe at other hidden sizes (any-H kernel)")
    ap.add_argument("--latency-grid", action="store_true",
                    help="small batches: row vs split kernel over T and num_blocks")
    ap.add_argument("--variant-sweep", action="store_true",
                    help="only T=1024 calls over num_blocks x delta x output norm")
    ap.add_argument("--overlap", action="store_true",
                    help="only the two-kernel form beside a producer of delta, against the "
                         "one-kernel call after it")
    ap.add_argument("--configs", action="store_true",
                    help="only the reference case (T=4, nb=4) and the 80-case variant matrix")
    ap.add_argument("--summarize-profile", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/ summaries from rocprofv3 CSV output directories")
    ap.add_argument("--profile-commands", default=None, help="JSON of the commands that made them")
    ap.add_argument("--summarize-trace", nargs=4, metavar=("TRACE_DIR", "OUT_NAME", "TITLE", "COMMAND"),
                    help="write one kernel-statistics summary into profiles/")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("OUT_NAME", "TITLE"),
                    help="write a counter summary into profiles/ from --counter-run LABEL=DIR "
                         "directories (rocprofv3 --pmc CSV output)")
    ap.add_argument("--counter-run", action="append", default=[], metavar="LABEL=DIR")
    ap.add_argument("--counter-command", action="append", default=[], metavar="CMD")
    args = ap.parse_args()
    if args.summarize_counters:
        write_counter_summary(*args.summarize_counters, args.counter_command,
                              dict(r.split("=", 1) for r in args.counter_run))
        return
    if args.summarize_trace:
        write_kernel_stats(*args.summarize_trace)
        return
    if args.summarize_profile:
        summarize_profile(*args.summarize_profile, commands=json.loads(args.profile_commands or "{}"))
        return
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "the attention-residual op shards by tokens with no exchange, so the "
              "single-GPU figure is the per-GPU rate", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} ({getattr(props, 'gcnArchName', '?')}), {props.multi_processor_count} CUs")
    device = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
              "compute_units": props.multi_processor_count,
              "memory_bytes": props.total_memory, "hip": getattr(torch.version, "hip", None),
              "torch": torch.__version__}
    A.attnres_init()
    if args.calibrate:
        calibration_copy()
    if args.overlap:
        table = bench_overlap()
        print(json.dumps({"metric": "exposed attention-residual time per decode step beside "
                                    "the producer of delta", "unit": "us/step",
                          "higher_is_better": False, "data": "synthetic",
                          "config": {"workload": "T tokens (1/4/16/64), H=7168, 8 or 4 block "
                                                 "rows, delta and output norm, no bank write; "
                                                 "producer delta = x W, [T,7168]x[7168,7168] "
                                                 "bf16",
                                     "timing": "hipGraph replay"},
                          "steps": table, "kernel_source_hash": kernel_source_hash()}),
              flush=True)
        return
    if args.configs:
        table = bench_configs()
        # The rows of the (nb=8, delta, norm, write slot 7) cases moved with no
        # arithmetic, in the row kernel's launch shape and cache policy.
        probes = {}
        for T in (256, 2048):
            pus = probe_mid_h(W.HIDDEN, T, T * W.HIDDEN >= 1024 * 7168)
            nbytes = W.Case("p", T=T, nb=8, widx=7).algorithmic_bytes()
            probes[f"T{T}"] = dict(us=round(pus, 3), frac=round(nbytes / pus / 1e3 / HBM_PEAK_GBPS, 4))
            log(f"configs: traffic probe T={T}: {pus:.2f} us")
        print(json.dumps({"metric": "attention-residual forward latency and throughput per case",
                          "unit": "us/call", "higher_is_better": False, "data": "synthetic",
                          "config": {"workload": "the reference case (T=4, nb=4, delta, output "
                                                 "norm) and the variant matrix (T 1/16/256/2048 x "
                                                 "nb 0/4/8 x delta x output norm x write slot "
                                                 "-1/nb-1), H=7168, bf16",
                                     "timing": "hipGraph replay, rotating token windows"},
                          "cases": table, "traffic_probe_nb8_delta_norm_w7": probes,
                          "kernel_source_hash": kernel_source_hash()}),
              flush=True)
        return
    if args.variant_sweep:
        sweep = bench_variant_sweep()
        print(json.dumps({"metric": "attention-residual forward throughput per variant",
                          "unit": "GB/s", "higher_is_better": True, "data": "synthetic",
                          "config": {"workload": "T=1024 tokens, H=7168, num_blocks 0..8 x delta "
                                                 "x output norm, block_write_idx=nb-1, bf16",
                                     "timing": "hipGraph replay"},
                          "variants": sweep, "kernel_source_hash": kernel_source_hash()}),
              flush=True)
        return
    if args.latency_grid:
        grid = bench_latency_grid()
        print(json.dumps({"metric": "attention-residual forward latency, small batches",
                          "unit": "us/call", "higher_is_better": False, "data": "synthetic",
                          "config": {"workload": "T tokens (cold rows), H=7168, num_blocks 0..8, "
                                                 "delta and output norm on, no bank write, bf16; "
                                                 "row and split kernels forced",
                                     "timing": "hipGraph replay"},
                          "grid": grid, "kernel_source_hash": kernel_source_hash()}), flush=True)
        return
    if args.hidden_sweep:
        sweep = bench_hidden_sweep()
        print(json.dumps({"metric": "attention-residual forward throughput at other hidden sizes",
                          "unit": "GB/s", "higher_is_better": True, "data": "synthetic",
                          "config": {"workload": "T=1024 tokens, 8 block rows, delta and output "
                                                 "norm on, block_write_idx=3, bf16, dense bank",
                                     "timing": "hipGraph replay"},
                          "hidden_sizes": sweep, "kernel_source_hash": kernel_source_hash()}),
              flush=True)
        return

    mid = None if args.only in ("decode", "ceiling") else bench_mid(args.steps, args.warmup,
                                                                     args.eager)
    decode = None if (args.only in ("mid", "ceiling") or args.eager) else bench_decode(args.steps)
    longp = None if (args.only or args.eager) else bench_long()
    ceiling = (bench_ceiling(steps=args.steps if args.eager else 300, eager=args.eager)
               if (args.only == "ceiling" or (args.only is None and not args.eager)) else None)
    if A.attnres_device_status() != A.ATTNRES_OK:
        raise SystemExit("device wait flag raised during the benchmark")
    cpu = None if (args.no_cpu or args.only) else cpu_baseline()

    line = {"metric": METRIC}
    if mid is not None:
        achieved = mid["gbps"]
        line.update({
            "value": round(achieved, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(mid["per_call_ms"], 6),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
            "storage_dtype": "bf16", "data": "synthetic",
            "config": {"workload": "mid prefill: T=1024 tokens, 8 block rows, H=7168, delta and "
                                   "output norm on, block_write_idx=3, bf16, dense bank",
                       "T": 1024, "num_blocks": 8, "H": 7168, "input_sets": mid["nsets"],
                       "timing": "eager" if args.eager else "hipGraph replay",
                       "parallelism": "single GPU"},
            "roofline": {"bound": "hbm", "kernel": DOMINANT_KERNEL, "achieved": round(achieved, 1),
                         "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": round(achieved / HBM_PEAK_GBPS, 4),
                         "traffic": load_traffic(),
                         "algorithmic_bytes_per_launch": mid["bytes"],
                         "achieved_from": "per-call time of back-to-back graph replays on the "
                                          "launch stream (hipEvents), kernels plus the gaps "
                                          "between them",
                         "kernel_trace": kernel_trace_entry(mid["bytes"])},
            "mid_prefill_us_per_call": {k: round(v, 3) for k, v in mid["us"].items()},
            "calls_timed": mid["calls_timed"],
            "graph_repeats": mid["graph_repeats"],
        })
    if decode is not None:
        line["decode_T1_us_per_call"] = {k: round(v["cold_us"], 3) for k, v in decode.items()}
        line["decode_T1_warm_us_per_call"] = {k: round(v["warm_us"], 3) for k, v in decode.items()}
        if mid is None:
            line.update({"value": round(decode["nb8"]["cold_us"], 3), "unit": "us/call",
                         "higher_is_better": False})
    if longp is not None:
        line["long_prefill"] = longp
    if ceiling is not None:
        probe = ceiling["mid_prefill_cached"]
        line["traffic_ceiling"] = {
            "probe": "the mid-prefill call's buffers, row roles, launch shape and cache policy "
                     "(8 bank rows, prefix and delta read, the 2 rewritten rows through the "
                     "cache; out, prefix and bank slot 3 written), no arithmetic",
            "GBps": probe["GBps"],
            # both medians over their graph replays
            "kernel_fraction": None if mid is None else round(
                mid["bytes"] / mid["us"]["p50"] / 1e3 / probe["GBps"], 4),
            "configs": ceiling}
    if cpu is not None:
        line["cpu_baseline"] = cpu
    line["device"] = device
    line["kernel_source_hash"] = kernel_source_hash()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
