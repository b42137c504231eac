"""GPU parity: the HIP path (through the C-ABI binding) against the fp64 oracle
on seeded inputs.

Bar: out within atol 1e-2 + rtol 1.6e-2 of the oracle rounded to bf16; the
written prefix and bank rows, every untouched bank slot, the token padding,
delta and the weights bit-exact.  Both kernels (row and split) are exercised
on the same inputs wherever the split path accepts the size.
"""
import numpy as np
import pytest
import torch

from kimi_k3_attention_amd import workloads as W

pytestmark = pytest.mark.gpu
A_PATH_ANY_H = 3  # ATTNRES_PATH_ANY_H (checked against the header by the boundary tests)


@pytest.fixture(scope="module")
def G():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests import gpu_harness
    return gpu_harness


def _paths(T, H=7168):
    """Every kernel that can run a call of T tokens at hidden size H: at 7168
    the tuned row kernel, the split kernel (T <= 256) and the any-H kernel;
    at other sizes the any-H kernel (through the automatic choice, the row
    selector and its own) and the split kernel with 1 (below 7168), 2 or 3
    segments per lane, masked (T <= 256)."""
    from kimi_k3_attention_amd import attnres as A
    ps = [None, A.ATTNRES_PATH_ROW, A.ATTNRES_PATH_ANY_H]
    if T <= A.ATTNRES_SPLIT_MAX_TOKENS:
        ps.append(A.ATTNRES_PATH_SPLIT)
    return ps


def _path_of(name):
    from kimi_k3_attention_amd import attnres as A
    return {"row": A.ATTNRES_PATH_ROW, "split": A.ATTNRES_PATH_SPLIT,
            "any_h": A.ATTNRES_PATH_ANY_H, "any_h_large": A.ATTNRES_PATH_ANY_H,
            "split_wide": A.ATTNRES_PATH_SPLIT}[name]


# Rows over 8192 elements (four segments per lane, one workgroup per CU) at
# token counts that fill the device several times over.
LARGE_ROW_CASES = [
    dict(H=16384, T=700, nb=8),
    dict(H=12288, T=1100, nb=5, has_onorm=False),
    dict(H=8200, T=600, nb=3, widx=-1),          # 1025 segments: halves of 513 and 512
    dict(H=16376, T=530, nb=0),                  # masked halves, a single source
    dict(H=10240, T=333, nb=7, has_delta=False),
]


def _run_and_check_all_paths(G, case, ref=None, inp=None):
    if inp is None:
        inp = W.make_inputs(case)
    if ref is None:
        ref = G.oracle_full(inp)
    for path in _paths(case.T, case.H):
        G.say(case.name, "path", path)
        d = G.upload(inp)
        G.run(d, path=path)
        G.check_full(inp, G.download(d), ref)
    return inp, ref


def test_pr1_reference_case(G):
    _run_and_check_all_paths(G, W.pr1_ref())


@pytest.mark.parametrize("case", W.decode_sweep(), ids=lambda c: c.name)
def test_single_token_decode(G, case):
    _run_and_check_all_paths(G, case)


@pytest.mark.parametrize("nb", [0, 1, 4, 8])
def test_five_tokens_seed0(G, nb):
    """The validation shape of the benchmark on the vLLM PR #54261 digest
    ("Implementation breakdown" item 4 and the benchmark script under "Key
    source snippets": 0, 1, 4 and 8 blocks on 5 tokens, seed 0), every
    kernel, each flag combination."""
    for d in (False, True):
        for o in (False, True):
            case = W.Case(f"five_nb{nb}_d{int(d)}_o{int(o)}", T=5, nb=nb, has_delta=d,
                          has_onorm=o, widx=nb - 1 if nb else -1, seed=0)
            _run_and_check_all_paths(G, case)


def test_benchmarked_configuration_replayed(G):
    """The configuration the benchmark times: mid prefill (T=1024, 8 block
    rows, delta, output norm, block_write_idx=3) over 4 resident input sets
    with delta zeroed, calls captured in one hipGraph and replayed.  After the
    first call each set is a fixed point (its bank slot 3 holds the prefix
    row), so every replay must reproduce the oracle run on that state."""
    from kimi_k3_attention_amd import attnres as A
    base = W.mid_prefill()
    devs, refs = [], []
    for r in range(4):
        case = W.with_(base, seed=base.seed + 100 * r)
        inp = W.make_inputs(case)
        inp.delta[:] = 0
        # the state after one call: slot 3 = cur = prefix (delta is zero)
        H, ts, ss = case.H, case.token_stride, case.slot_stride
        bank = inp.bank.reshape(case.T, ts)
        bank[:, case.widx * ss:case.widx * ss + H] = inp.prefix
        refs.append((inp, G.oracle_full(inp)))
        devs.append(G.upload(inp))
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(2):
            for d in devs:
                G.run(d)
    for rep in range(3):
        for d in devs:
            d.out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, d in enumerate(devs):
            inp, ref = refs[k]
            G.say("benchmarked configuration, replay", rep, "set", k)
            G.check_full(inp, G.download(d), ref)
    assert A.attnres_device_status() == A.ATTNRES_OK


def test_mid_prefill_full(G):
    case = W.mid_prefill()
    inp = W.make_inputs(case)
    ref = G.oracle_full(inp)
    G.say(case.name)
    d = G.upload(inp)
    G.run(d)
    G.check_full(inp, G.download(d), ref)


@pytest.mark.parametrize("T", [4096, 8192])
def test_long_prefill_full(G, T):
    """Full size in the benchmark's launch shape, every token against the
    oracle (run over token ranges on a thread pool); the whole bank (with its
    padding) and prefix bit-identical (no delta, no write in this workload)."""
    case = W.long_prefill(T)
    inp = W.make_inputs(case)
    assert len(inp.bank) == T * case.token_stride, "bank slices must tile the buffer"
    G.say(case.name, "oracle over", T, "tokens")
    ref = G.oracle_full_threaded(inp)
    G.say(case.name)
    d = G.upload(inp)
    G.run(d)
    got = G.download(d)
    G.check_full(inp, got, ref)
    assert (got.prefix == inp.prefix).all()
    assert (got.bank == inp.bank).all(), "bank (or its padding) modified"


# The any-H kernel with three bank rows staged in LDS, two segments per lane:
# 5-wave workgroups (H 4104..5120) and 6-wave ones (H 5128..6144), 4..8 bank
# rows, more tokens than three per compute unit (T > 768 on 256 CUs); masked
# rows, and the cached-read form (T * H >= 1024 * 7168 with a delta and a
# written source slot).
LDS_ROW_CASES = [
    dict(H=5120, T=900, nb=8, widx=3, slot_major=True),          # slot-major bank
    dict(H=5632, T=800, nb=6, widx=5, row_pad=40, cap=7),        # strided rows, 6 waves
    dict(H=6144, T=1024, nb=8, widx=3),                          # 6 waves
    dict(H=6144, T=1300, nb=4, has_onorm=False, widx=1),         # 6 waves, cached
    dict(H=5632, T=1024, nb=8, widx=3),                          # 6 waves, masked
    dict(H=5128, T=800, nb=5, has_delta=False, widx=4),         # 6 waves, one segment over
    dict(H=6136, T=1300, nb=8, widx=7, recipe="soft"),           # 6 waves, masked and cached
    dict(H=5120, T=1024, nb=8, widx=3),
    dict(H=5120, T=1000, nb=4, has_onorm=False, widx=-1),
    dict(H=5120, T=900, nb=6, has_delta=False, widx=5),
    dict(H=4608, T=1100, nb=7, widx=0),                          # masked
    dict(H=4104, T=800, nb=5, has_delta=False, has_onorm=False),  # masked, one segment over
    dict(H=5120, T=1500, nb=8, widx=2, token_pad=64),            # cached rewritten rows
    dict(H=4616, T=1700, nb=5, widx=4, recipe="soft"),           # masked and cached
]


@pytest.mark.parametrize("kw", LDS_ROW_CASES, ids=lambda kw: "_".join(f"{k}{v}" for k, v in kw.items()))
def test_any_h_rows_in_lds(G, kw):
    case = W.Case("lds_rows_" + "_".join(f"{k}{v}" for k, v in kw.items()), seed=77, **kw)
    inp = W.make_inputs(case)
    ref = G.oracle_full_threaded(inp)
    for path in (None, A_PATH_ANY_H):
        G.say(case.name, "path", path)
        d = G.upload(inp)
        G.run(d, path=path)
        G.check_full(inp, G.download(d), ref)


# The same with four segments per lane: 4..8 bank rows, in 5 waves (H =
# 8200..10240) for more tokens than compute units (T > 256 on 256 CUs), in 6
# waves (H = 10248..12288) for up to two per CU (T = 257..512); masked rows,
# and the cached-read form (T * H >= 1024 * 7168 with a delta and a written
# slot).
STAGED_CASES = [
    dict(H=9216, T=300, nb=8, widx=2, slot_major=True, row_pad=24),  # slot-major, strided
    dict(H=10240, T=800, nb=8, widx=3),                          # cached rewritten rows
    dict(H=12288, T=300, nb=4, has_onorm=False, widx=-1),       # 6 waves
    dict(H=10240, T=400, nb=6, has_delta=False, widx=5),
    dict(H=9000, T=500, nb=7, widx=0),                           # masked
    dict(H=12280, T=260, nb=5, has_delta=False, has_onorm=False),  # 6 waves, masked
    dict(H=9992, T=800, nb=8, widx=7, recipe="soft", token_pad=64),  # masked and cached
    dict(H=11264, T=512, nb=6, has_delta=False, widx=-1),       # 6 waves, masked, two per CU
    dict(H=8200, T=257, nb=4),                                   # first four-segment size
]


@pytest.mark.parametrize("kw", STAGED_CASES, ids=lambda kw: "_".join(f"{k}{v}" for k, v in kw.items()))
def test_any_h_rows_staged_in_lds(G, kw):
    case = W.Case("staged_rows_" + "_".join(f"{k}{v}" for k, v in kw.items()), seed=78, **kw)
    inp = W.make_inputs(case)
    ref = G.oracle_full_threaded(inp)
    for path in (None, A_PATH_ANY_H):
        G.say(case.name, "path", path)
        d = G.upload(inp)
        G.run(d, path=path)
        G.check_full(inp, G.download(d), ref)


@pytest.mark.parametrize("case", W.variant_matrix(), ids=lambda c: c.name)
def test_variant_matrix(G, case):
    inp = W.make_inputs(case)
    ref = G.oracle_full(inp)
    paths = _paths(case.T) if case.T <= 256 else [None, A_PATH_ANY_H]
    for path in paths:
        G.say(case.name, "path", path)
        d = G.upload(inp)
        G.run(d, path=path)
        G.check_full(inp, G.download(d), ref)


# Hidden sizes other than 7168, run by the any-H kernel: two or four segments
# per lane, rows that fill whole waves exactly and rows that need masking.
HIDDEN_CASES = [
    dict(H=8, T=9, nb=3),                 # one segment per row: 63 masked lanes
    dict(H=64, T=3, nb=8),                # split: 13 of 14 parts wholly masked
    dict(H=1024, T=33, nb=8),
    dict(H=2048, T=300, nb=4, has_onorm=False),
    dict(H=2880, T=40, nb=7),             # 360 segments: masked, 3 waves
    dict(H=4096, T=129, nb=8, widx=-1),
    dict(H=4096, T=32, nb=8, has_delta=False),  # automatic choice: split below 7168
    dict(H=4608, T=48, nb=2),
    dict(H=3584, T=16, nb=1),
    dict(H=5120, T=17, nb=0),
    dict(H=6144, T=48, nb=5),
    dict(H=7160, T=20, nb=5),             # one segment short of 7168
    dict(H=8192, T=64, nb=8, has_delta=False),
    dict(H=8200, T=12, nb=2),             # first size with four segments per lane
    dict(H=9216, T=72, nb=3),             # largest T the automatic choice splits
    dict(H=12288, T=48, nb=6),
    dict(H=16384, T=73, nb=8, has_onorm=False),  # first T past it: any-H
    dict(H=16376, T=10, nb=8),            # 2047 segments: masked, 8 waves
    dict(H=16384, T=24, nb=8, widx=0),
]


@pytest.mark.parametrize("kw", HIDDEN_CASES, ids=lambda kw: f"H{kw['H']}_T{kw['T']}_nb{kw['nb']}")
def test_other_hidden_sizes(G, kw):
    kw = dict(kw)
    case = W.other_hidden(kw.pop("H"), kw.pop("T"), kw.pop("nb"), **kw)
    _run_and_check_all_paths(G, case)


@pytest.mark.parametrize("kw", LARGE_ROW_CASES, ids=lambda kw: f"H{kw['H']}_T{kw['T']}_nb{kw['nb']}")
def test_large_rows_many_tokens(G, kw):
    kw = dict(kw)
    case = W.other_hidden(kw.pop("H"), kw.pop("T"), kw.pop("nb"), **kw)
    _run_and_check_all_paths(G, case)


def test_large_rows_back_to_back(G):
    """Calls with 16384-element rows and very different token counts enqueued
    back to back without synchronisation: every result matches the oracle."""
    from kimi_k3_attention_amd import attnres as A
    cases = [W.other_hidden(16384, T, nb, seed=900 + T) for T, nb in
             ((900, 8), (3, 2), (520, 8), (1, 0), (777, 4), (260, 1))]
    inps = [W.make_inputs(c) for c in cases]
    refs = [G.oracle_full(i) for i in inps]
    devs = [G.upload(i) for i in inps]
    torch.cuda.synchronize()
    for rep in range(2):
        if rep:
            devs = [G.upload(i) for i in inps]
            torch.cuda.synchronize()
        for d in devs:
            G.run(d, path=A.ATTNRES_PATH_ANY_H)
        torch.cuda.synchronize()
        for k, d in enumerate(devs):
            G.say("large rows back to back, repetition", rep, "call", k)
            G.check_full(inps[k], G.download(d), refs[k])
    assert A.attnres_device_status() == A.ATTNRES_OK


@pytest.mark.parametrize("H,T,nb", [(7168, 37, 5), (7168, 200, 8), (7168, 1, 8), (2880, 50, 4),
                                    (16384, 9, 3)])
def test_strided_rows(G, H, T, nb):
    """prefix, delta and out rows placed row_pad elements apart (views into
    wider buffers): every kernel reads and writes only the rows; the gaps keep
    their sentinel."""
    case = W.other_hidden(H, T, nb, row_pad=136, seed=300 + T)
    _run_and_check_all_paths(G, case)


def test_interleaved_prefix_delta_and_out(G):
    """prefix and delta as the two halves of one [T, 2H] buffer (prefix is
    written in place), out as every third row of a [3T, H] buffer."""
    from kimi_k3_attention_amd import attnres as A
    case = W.Case("interleaved_T45_nb6", T=45, nb=6, widx=2, seed=310)
    inp = W.make_inputs(case)
    ref = G.oracle_full(inp)
    T, H = case.T, case.H
    for path in _paths(T):
        G.say(case.name, "path", path)
        d = G.upload(inp)
        pd = torch.cat([d.prefix, d.delta], dim=1).contiguous()     # [T, 2H]
        outbuf = torch.full((3 * T, H), G.ROW_GAP_BITS, dtype=torch.int16, device="cuda")
        out = outbuf[::3]
        A.attnres_fwd(pd[:, :H], pd[:, H:], d.bank3, case.nb, d.res_w, d.rms_w, case.eps, d.onw,
                      case.oeps, case.widx, out, path=path)
        torch.cuda.synchronize()
        G.assert_out_close(G.from_dev(out), ref.out_bits, case.name + " out")
        assert (G.from_dev(pd[:, :H]) == ref.prefix_after).all(), "prefix after the call"
        assert (G.from_dev(pd[:, H:]) == inp.delta).all(), "delta modified"
        rest = torch.cat([outbuf[1::3], outbuf[2::3]])
        assert (rest == G.ROW_GAP_BITS).all().item(), "out rows between the strided rows written"
        assert (G.from_dev(d.bank) == ref.bank_after).all(), "bank after the call"


@pytest.mark.parametrize("T,nb,onorm", [(64, 8, True), (200, 5, True), (3, 8, False)])
def test_wide_dynamic_range(G, T, nb, onorm):
    """Every bank, prefix and delta row scaled by its own power of two 2^k,
    k uniform in [-40, 40] (exact in bf16): logits depend only on direction,
    the mixture spans ~24 decades and the fp32 sums of squares stay in range.
    All kernels against the fp64 oracle, eps as in the workloads."""
    case = W.Case(f"range_T{T}_nb{nb}", T=T, nb=nb, has_onorm=onorm, widx=nb - 1,
                  recipe="soft", seed=400 + T)
    inp = W.make_inputs(case)
    rng = np.random.default_rng(case.seed)
    H, ts, ss = case.H, case.token_stride, case.slot_stride

    def scale(bits, k):
        # multiply bf16 values by 2^k by moving the exponent field (no value is
        # zero or subnormal for these draws, and none leaves the normal range)
        e = ((bits >> 7) & 0xFF).astype(np.int64) + k
        assert (e > 0).all() and (e < 255).all()
        return ((bits & 0x807F) | (e.astype(np.uint16) << 7)).astype(np.uint16)

    for t in range(T):
        inp.prefix[t] = scale(inp.prefix[t], int(rng.integers(-40, 41)))
        if inp.delta is not None:
            inp.delta[t] = scale(inp.delta[t], int(rng.integers(-40, 41)))
        for i in range(nb):
            o = t * ts + i * ss
            inp.bank[o:o + H] = scale(inp.bank[o:o + H], int(rng.integers(-40, 41)))
    ref = G.oracle_full(inp)
    assert np.isfinite(ref.out_f64).all()
    for path in _paths(T):
        G.say(case.name, "path", path)
        d = G.upload(inp)
        G.run(d, path=path)
        G.check_full(inp, G.download(d), ref)


def _random_cases(n, seed):
    """Seeded draws over the whole argument space the library accepts."""
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        H = int(rng.choice([7168, 7168, 7168, 8 * int(rng.integers(1, 2049))]))
        T = int(rng.choice([1, 2, 3, int(rng.integers(4, 40)), int(rng.integers(40, 300))]))
        if H > 8192:
            T = min(T, 64)
        nb = int(rng.integers(0, 9))
        cap = int(rng.integers(max(nb, 1), 9))
        widx = int(rng.integers(-1, cap))
        slot_major = bool(rng.random() < 0.2)
        cases.append(W.Case(
            f"rand{seed}_{k}_H{H}_T{T}_nb{nb}", T=T, nb=nb, cap=cap, H=H,
            has_delta=bool(rng.random() < 0.6), has_onorm=bool(rng.random() < 0.6), widx=widx,
            token_pad=0 if slot_major else 8 * int(rng.integers(0, 5)),
            row_pad=8 * int(rng.choice([0, 0, int(rng.integers(1, 40))])),
            slot_major=slot_major, recipe=str(rng.choice(["normal", "soft", "decode"])),
            seed=10_000 + 100 * seed + k))
    return cases


@pytest.mark.parametrize("case", _random_cases(40, 1) + _random_cases(80, 2) + _random_cases(150, 4) + _random_cases(150, 8),
                         ids=lambda c: c.name)
def test_random_configuration(G, case):
    _run_and_check_all_paths(G, case)


def _random_large_cases(n, seed):
    """Seeded draws of calls of 1 to 2 times 1024 * 7168 row elements (T * H),
    where the row kernels read rewritten rows through the cache whenever the
    call has a delta and writes one of its source slots."""
    rng = np.random.default_rng(seed)
    cases = []
    for k in range(n):
        H = int(rng.choice([7168, 7168, 8 * int(rng.integers(256, 2049))]))
        t_min = -(-1024 * 7168 // H)
        T = int(rng.integers(t_min, 2 * t_min + 1))
        nb = int(rng.integers(1, 9))
        cap = int(rng.integers(nb, 9))
        widx = int(rng.choice([-1, int(rng.integers(0, nb)), int(rng.integers(0, nb)), int(rng.integers(0, cap))]))
        slot_major = bool(rng.random() < 0.2)
        cases.append(W.Case(
            f"randlarge{seed}_{k}_H{H}_T{T}_nb{nb}_w{widx}", T=T, nb=nb, cap=cap, H=H,
            has_delta=bool(rng.random() < 0.8), has_onorm=bool(rng.random() < 0.6), widx=widx,
            token_pad=0 if slot_major else 8 * int(rng.integers(0, 5)),
            row_pad=8 * int(rng.choice([0, 0, int(rng.integers(1, 40))])),
            slot_major=slot_major, recipe=str(rng.choice(["normal", "soft"])),
            seed=20_000 + 100 * seed + k))
    return cases


@pytest.mark.parametrize("case", _random_large_cases(10, 5) + _random_large_cases(10, 6),
                         ids=lambda c: c.name)
def test_random_large_configuration(G, case):
    _run_and_check_all_paths(G, case)


def test_soft_logits_mix(G):
    """O(1) logits so the mixture really mixes (the named workloads are nearly
    one-hot)."""
    case = W.soft_logits()
    inp, ref = _run_and_check_all_paths(G, case)
    assert ref.probs.max(axis=1).mean() < 0.9


@pytest.mark.parametrize("T,nb,widx", [(3, 3, 2), (33, 5, 0), (257, 7, 6), (1000, 8, 7), (97, 2, -1)])
def test_ragged_sizes(G, T, nb, widx):
    case = W.Case(f"ragged_T{T}_nb{nb}", T=T, nb=nb, widx=widx, cap=nb + 1, token_pad=8, seed=40 + T)
    _run_and_check_all_paths(G, case)


# The row kernel at H = 7168 reads rows with range-checked loads in calls of
# up to 192 tokens with three or more bank rows (256 with two), and with
# plain loads above.
RANGED_ROW_MAX_T = {2: 256}   # else 192
RANGED_ROW_CASES = [
    dict(nb=2),
    dict(nb=3, has_delta=False),
    dict(nb=4, widx=3),
    dict(nb=5, has_onorm=False, widx=1),
    dict(nb=6, widx=0, recipe="student_t"),
    dict(nb=7, widx=6),
    dict(nb=8, widx=7, has_delta=False, has_onorm=False),
]


@pytest.mark.parametrize("kw", RANGED_ROW_CASES, ids=lambda kw: f"nb{kw['nb']}")
def test_row_kernel_small_call_form(G, kw):
    """The two load forms do the same arithmetic: a call one token past the
    limit (plain loads) matches the oracle, and a call at the limit
    (range-checked loads) on its first tokens gives bit-identical outputs
    and writes."""
    from kimi_k3_attention_amd import attnres as A
    n = RANGED_ROW_MAX_T.get(kw["nb"], 192)
    case = W.Case(f"ranged_nb{kw['nb']}", T=n + 1, seed=70 + kw["nb"], **kw)
    inp = W.make_inputs(case)
    G.say(case.name, f"T={n + 1}")
    d = G.upload(inp)
    G.run(d, path=A.ATTNRES_PATH_ROW)
    full = G.download(d)
    G.check_full(inp, full, G.oracle_full(inp))
    sub = W.with_(case, T=n)
    part_in = W.Inputs(case=sub, prefix=inp.prefix[:n].copy(),
                       delta=None if inp.delta is None else inp.delta[:n].copy(),
                       bank=inp.bank[:sub.bank_elems].copy(), res_w=inp.res_w, rms_w=inp.rms_w,
                       onw=inp.onw, out_init=inp.out_init[:n].copy())
    G.say(case.name, f"T={n}")
    d = G.upload(part_in)
    G.run(d, path=A.ATTNRES_PATH_ROW)
    part = G.download(d)
    assert np.array_equal(part.out, full.out[:n]), "out"
    assert np.array_equal(part.prefix, full.prefix[:n]), "prefix"
    assert np.array_equal(part.bank, full.bank[:sub.bank_elems]), "bank"


@pytest.mark.parametrize("T,nb,widx", [(2500, 1, 0), (1537, 0, -1), (4099, 1, -1)])
def test_persistent_grid_few_blocks(G, T, nb, widx):
    """Few source rows run a persistent grid (a few workgroups per CU, each
    looping over tokens): token counts well above the grid, ragged against
    it, every token checked."""
    case = W.Case(f"persist_T{T}_nb{nb}", T=T, nb=nb, widx=widx, cap=2, seed=500 + T)
    _run_and_check_all_paths(G, case)


@pytest.mark.parametrize("T,has_onorm", [(4, False), (4, True), (40, True), (300, False)])
def test_single_source_zero_row_eps0(G, T, has_onorm):
    """nb = 0 with eps = 0 and an all-zero current row: the logit is 0/0, the
    single source still has weight 1, so out is the zero row (finite) on
    every path, as in the oracle."""
    case = W.Case(f"zero_row_T{T}", T=T, nb=0, has_delta=False, has_onorm=has_onorm, eps=0.0,
                  seed=40 + T)
    inp = W.make_inputs(case)
    inp.prefix[1] = 0
    inp.prefix[T - 1] = 0
    _run_and_check_all_paths(G, case, inp=inp)


# Calls of at least 1024 tokens whose written slot is also a source, with a
# delta: the row kernel then reads prefix and that slot through the cache.
CACHED_REWRITE_CASES = [
    dict(T=1024, nb=8, widx=0, slot_major=True),
    dict(T=1100, nb=5, widx=4, token_pad=64, row_pad=16),
    dict(T=1536, nb=2, widx=1, has_onorm=False),
    dict(T=4099, nb=1, widx=0),
    dict(T=2048, nb=7, widx=3, cap=7),
    # the any-H kernel's cached variant (T * H at or above 1024 * 7168)
    dict(H=8192, T=1024, nb=8, widx=3),
    dict(H=2880, T=2560, nb=4, widx=2),                       # masked rows
    dict(H=16376, T=449, nb=2, widx=1, has_onorm=False),      # four segments per lane, masked
    dict(H=12288, T=600, nb=6, widx=5, token_pad=64),
    # no delta: only the written slot is read through the cache (T * H at or
    # above 2 * 1024 * 7168)
    dict(T=2048, nb=4, widx=3, has_delta=False),
    dict(T=2100, nb=8, widx=7, has_delta=False, has_onorm=False, token_pad=64),
    dict(H=8192, T=1800, nb=6, widx=2, has_delta=False),
    dict(H=2880, T=5200, nb=3, widx=0, has_delta=False),             # masked rows
]


@pytest.mark.parametrize("kw", CACHED_REWRITE_CASES,
                         ids=lambda kw: f"H{kw.get('H', 7168)}_T{kw['T']}_nb{kw['nb']}_w{kw['widx']}")
def test_cached_rewritten_rows(G, kw):
    kw = dict(kw)
    case = W.Case(f"cached_rw_T{kw['T']}", seed=60 + kw["T"] % 97, **kw)
    _run_and_check_all_paths(G, case)


WIDE_SPLIT_CASES = [
    dict(H=7176, T=3, nb=8),                          # one segment past 7168: two per lane, masked
    dict(H=8192, T=1, nb=7),
    dict(H=9000, T=5, nb=1, has_onorm=False),
    dict(H=12288, T=40, nb=4, widx=-1),
    dict(H=14336, T=2, nb=8),                         # two segments per lane, every lane full
    dict(H=14344, T=3, nb=7),                         # three per lane
    dict(H=16384, T=16, nb=8, has_delta=False),
    dict(H=16376, T=1, nb=0),
]


@pytest.mark.parametrize("kw", WIDE_SPLIT_CASES, ids=lambda kw: f"H{kw['H']}_T{kw['T']}_nb{kw['nb']}")
def test_wide_split(G, kw):
    """The split path above 7168 (2 or 3 segments per lane per part, masked at
    the row end), every word path, against the oracle with every kernel."""
    kw = dict(kw)
    case = W.other_hidden(kw.pop("H"), kw.pop("T"), kw.pop("nb"), **kw)
    _run_and_check_all_paths(G, case)


@pytest.mark.parametrize("nb", range(1, 9))
@pytest.mark.parametrize("onorm", [False, True])
def test_split_word_paths(G, nb, onorm):
    """Every way the split path sums its per-part words: DPP wave sums (few
    words), the LDS transposition, and the matrix-core Gram product (an
    output norm at nb >= 7), on a few tokens, against the oracle."""
    case = W.Case(f"split_words_nb{nb}_o{int(onorm)}", T=3, nb=nb, has_onorm=onorm,
                  widx=nb - 1, recipe="soft", seed=70 + nb + 10 * onorm)
    _run_and_check_all_paths(G, case)


def test_slot_major_bank(G):
    case = W.Case("slot_major_T40_nb6", T=40, nb=6, widx=6, slot_major=True, seed=51)
    _run_and_check_all_paths(G, case)


def test_capacity_one_and_write_only(G):
    """nb = 0 with a write: the bank is only written, never read."""
    case = W.Case("write_only_T20", T=20, nb=0, cap=1, widx=0, seed=52)
    _run_and_check_all_paths(G, case)


def test_empty_call_is_a_noop(G):
    case = W.Case("empty", T=0, nb=4, seed=53)
    inp = W.make_inputs(case)
    d = G.upload(inp)
    G.run(d)
    torch.cuda.synchronize()


def test_bitwise_repeatable(G):
    case = W.Case("repeat_T64_nb8", T=64, nb=8, widx=-1, has_delta=False, seed=54)
    inp = W.make_inputs(case)
    for path in _paths(case.T):
        outs = []
        for _ in range(3):
            d = G.upload(inp)
            G.run(d, path=path)
            outs.append(G.download(d).out)
        assert all((o == outs[0]).all() for o in outs), f"path {path} not repeatable"


def test_cancelling_sources(G):
    """Sources that cancel: a zero projection weight makes every weight 1/3,
    slot 1 is the negation of slot 0 and the current residual is small, so
    ||y|| is far below sum_j p_j ||x_j||.  The split path must notice that the
    Gram form of ||y||^2 would lose accuracy and exchange it directly."""
    case = W.Case("cancel_T4_nb2", T=4, nb=2, cap=2, widx=-1, seed=90)
    inp = W.make_inputs(case)
    inp.res_w[:] = 0
    H, ts = case.H, case.token_stride
    for t in range(case.T):
        inp.bank[t * ts + H: t * ts + 2 * H] = inp.bank[t * ts: t * ts + H] ^ np.uint16(0x8000)
    small = (G.widen(inp.prefix) * 0.01).astype(np.float32)
    inp.prefix[:] = torch.from_numpy(small).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ref = G.oracle_full(inp)
    y_norm = np.linalg.norm(ref.out_f64, axis=1)
    assert np.all(ref.probs == ref.probs[:, :1])  # uniform weights
    for path in _paths(case.T):
        G.say(case.name, "path", path)
        d = G.upload(inp)
        G.run(d, path=path)
        G.check_full(inp, G.download(d), ref)
    assert np.isfinite(y_norm).all()


@pytest.mark.parametrize("path_name", ["row", "split", "any_h", "row_small"])
def test_bank_offsets_beyond_32_bits(G, path_name):
    """A bank whose element offsets exceed 2^31 (150 tokens 2^24 elements
    apart, about 4.8 GB; the row kernel takes its small-call form there, and
    its plain form at 200 tokens, about 6.4 GB; 100 tokens 2^25 apart, about
    6.7 GB): only the used rows are filled; sampled tokens are checked
    against the oracle and the elements right after each written row keep
    their sentinel."""
    from kimi_k3_attention_amd import attnres as A
    small = path_name == "row_small"
    path = A.ATTNRES_PATH_ROW if small else _path_of(path_name)
    T, nb, cap, H, ts = ((100, 5, 8, 7168, 1 << 25) if small
                         else (200, 5, 8, 7168, 1 << 24) if path_name == "row"
                         else (150, 5, 8, 7168, 1 << 24))
    case = W.Case("small_rows", T=T, nb=nb, cap=cap, widx=6, seed=95)
    inp = W.make_inputs(case)                      # dense bank, used for the values
    bank = torch.full((T * ts,), 0x7F81, dtype=torch.int16, device="cuda")
    bank3 = bank.as_strided((T, cap, H), (ts, H, 1))
    dense = G.to_dev(inp.bank).view(T, cap, H)
    bank3.copy_(dense)
    assert (T - 1) * ts + cap * H > 2 ** 31
    d = G.upload(inp)
    G.say(case.name, "path", path_name)
    A.attnres_fwd(d.prefix, d.delta, bank3, nb, d.res_w, d.rms_w, case.eps, d.onw, case.oeps,
                  case.widx, d.out, path=path)
    torch.cuda.synchronize()
    tokens = [0, 1, 74, T - 2, T - 1]
    ref = G.oracle_sample(inp, tokens)
    out = G.from_dev(d.out)
    G.assert_out_close(out[tokens], ref.out_bits, "large-offset out")
    assert (G.from_dev(d.prefix)[tokens] == ref.prefix_after).all()
    written = G.from_dev(bank3[tokens, case.widx].contiguous())
    assert (written == ref.written_row).all()
    tail = G.from_dev(bank3[:, cap - 1, :].contiguous())    # slot 7: never read or written
    assert (tail == inp.bank.reshape(T, cap, H)[:, cap - 1]).all()
    after = bank.as_strided((T, 64), (ts, 1), storage_offset=cap * H)
    assert (G.from_dev(after.contiguous()) == 0x7F81).all(), "write past a row"
    del bank, bank3
    torch.cuda.empty_cache()


def test_split_exchange_across_many_calls(G):
    """The split path's exchange words carry a generation that advances every
    call and is never reset: run many consecutive calls, alternating calls
    without and with output norm (one or two exchange phases), different
    token counts and block counts, and check every result; the device fault
    flag must stay clear."""
    from kimi_k3_attention_amd import attnres as A
    cases = [W.Case("xa", T=5, nb=4, has_onorm=True, seed=60),
             W.Case("xb", T=7, nb=8, has_onorm=False, seed=61),
             W.Case("xc", T=1, nb=8, has_onorm=True, widx=7, seed=62),
             W.Case("xd", T=64, nb=6, has_onorm=True, widx=0, seed=63)]
    prepared = []
    for c in cases:
        inp = W.make_inputs(c)
        prepared.append((inp, G.oracle_full(inp)))
    for it in range(60):
        inp, ref = prepared[it % len(prepared)]
        d = G.upload(inp)
        G.run(d, path=A.ATTNRES_PATH_SPLIT)
        G.check_full(inp, G.download(d), ref)
    assert A.attnres_device_status() == A.ATTNRES_OK


def test_split_back_to_back_without_sync(G):
    """Consecutive split calls on one stream with no host synchronisation in
    between (each reuses the same workspace words), results checked after."""
    from kimi_k3_attention_amd import attnres as A
    cases = [W.Case(f"bb{k}", T=3, nb=7, widx=2, seed=70 + k) for k in range(8)]
    inps = [W.make_inputs(c) for c in cases]
    refs = [G.oracle_full(i) for i in inps]
    devs = [G.upload(i) for i in inps]
    torch.cuda.synchronize()
    for _ in range(3):
        for dv in devs:
            dv.out.fill_(0)
        for k, dv in enumerate(devs):
            # restore the in-place buffers so every call sees its original inputs
            dv.prefix.copy_(G.to_dev(inps[k].prefix))
            dv.bank.copy_(G.to_dev(inps[k].bank))
        for dv in devs:
            G.run(dv, path=A.ATTNRES_PATH_SPLIT)
        for k, dv in enumerate(devs):
            G.check_full(inps[k], G.download(dv), refs[k])
    assert A.attnres_device_status() == A.ATTNRES_OK


def test_split_calls_on_several_streams(G):
    """Split calls issued round-robin on three streams with no
    synchronisation between the streams: the library orders them (a stream
    switch waits for the previous stream's work), so every call sees its own
    inputs and the shared workspace is never used twice at once."""
    from kimi_k3_attention_amd import attnres as A
    cases = [W.Case(f"streams{k}", T=5 + 3 * k, nb=6, widx=3, seed=600 + k) for k in range(6)]
    inps = [W.make_inputs(c) for c in cases]
    refs = [G.oracle_full(i) for i in inps]
    streams = [torch.cuda.Stream() for _ in range(3)]
    for rep in range(5):
        devs = [G.upload(i) for i in inps]
        torch.cuda.synchronize()
        for k, d in enumerate(devs):
            with torch.cuda.stream(streams[k % 3]):
                G.run(d, path=A.ATTNRES_PATH_SPLIT)
        torch.cuda.synchronize()
        for k, d in enumerate(devs):
            G.say("several streams, repetition", rep, "call", k)
            G.check_full(inps[k], G.download(d), refs[k])
    assert A.attnres_device_status() == A.ATTNRES_OK


def test_split_calls_from_two_threads(G):
    """Two host threads issue split calls at the same time, each on its own
    stream (the library call runs without the GIL): the workspace hand-off
    and the launch happen under one lock, so every result matches the
    oracle."""
    import threading
    from kimi_k3_attention_amd import attnres as A
    # Repeated calls must be idempotent: no delta, and the written slot (7) is
    # not one of the 7 sources.
    cases = [W.Case(f"threads{k}", T=3 + 2 * k, nb=7, widx=7, has_delta=False, seed=700 + k)
             for k in range(8)]
    inps = [W.make_inputs(c) for c in cases]
    refs = [G.oracle_full(i) for i in inps]
    devs = [G.upload(i) for i in inps]
    torch.cuda.synchronize()
    errors = []

    def worker(ks):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                for _ in range(20):
                    for k in ks:
                        G.run(devs[k], path=A.ATTNRES_PATH_SPLIT)
            stream.synchronize()
        except Exception as e:  # reported in the main thread
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(range(j, 8, 2),)) for j in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for k, d in enumerate(devs):
        G.say("two threads, call", k)
        G.check_full(inps[k], G.download(d), refs[k])
    assert A.attnres_device_status() == A.ATTNRES_OK


@pytest.mark.parametrize("path_name", ["row", "split", "any_h", "any_h_large", "split_wide"])
def test_graph_replay_matches_eager(G, path_name):
    """Calls captured in a hipGraph (torch.cuda.CUDAGraph) and replayed several
    times, with eager work and synchronisation in between, match the eager
    result every time.  delta = 0 makes repeated in-place calls a fixed point
    after the first."""
    from kimi_k3_attention_amd import attnres as A
    path = _path_of(path_name)
    A.attnres_init()
    case = W.Case(f"graph_{path_name}", T=24, nb=6, widx=5, seed=70)
    if path_name == "any_h_large":
        case = W.other_hidden(16384, T=600, nb=6, seed=71)
    if path_name == "split_wide":  # three segments per lane, matrix-core words
        case = W.other_hidden(16384, T=5, nb=8, seed=72)
    inp = W.make_inputs(case)
    inp.delta[:] = 0
    d = G.upload(inp)
    G.run(d, path=path)
    G.run(d, path=path)
    eager = G.download(d)
    g = torch.cuda.CUDAGraph()
    d.out.fill_(0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        G.run(d, path=path)
        G.run(d, path=path)
    for rep in range(4):
        d.out.fill_(0)
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = G.download(d)
        assert (got.out == eager.out).all(), f"replay {rep}: out differs from eager"
        assert (got.bank == eager.bank).all() and (got.prefix == eager.prefix).all()
        del junk
    assert A.attnres_device_status() == A.ATTNRES_OK


def test_invalid_call_raises_and_touches_nothing(G):
    from kimi_k3_attention_amd import attnres as A
    case = W.Case("invalid", T=4, nb=4, widx=1, seed=80)
    inp = W.make_inputs(case)
    d = G.upload(inp)
    bad_out = d.prefix  # out aliasing prefix
    with pytest.raises(A.AttnResError) as e:
        A.attnres_fwd(d.prefix, d.delta, d.bank3, case.nb, d.res_w, d.rms_w, case.eps, d.onw,
                      case.oeps, case.widx, bad_out)
    assert e.value.name == "ATTNRES_E_ALIAS"
    with pytest.raises(A.AttnResError) as e:
        A.attnres_fwd(d.prefix, d.delta, d.bank3, 9, d.res_w, d.rms_w, case.eps, d.onw,
                      case.oeps, case.widx, d.out)
    assert e.value.name == "ATTNRES_E_NUM_BLOCKS"
    # A host tensor among device tensors is refused by the binding before any
    # library call (the kernels would dereference a host address).
    for name in ("delta", "res_w", "out"):
        args = dict(delta=d.delta, res_w=d.res_w, out=d.out)
        args[name] = args[name].cpu()
        with pytest.raises(ValueError, match=name):
            A.attnres_fwd(d.prefix, args["delta"], d.bank3, case.nb, args["res_w"], d.rms_w,
                          case.eps, d.onw, case.oeps, case.widx, args["out"])
    got = G.download(d)
    assert (got.prefix == inp.prefix).all() and (got.bank == inp.bank).all()
    assert (got.out == inp.out_init).all()
