"""The C-ABI boundary on the CPU: the library loads, exports every entry point
include/attnres.h declares, and its host-side checks reject every invalid
argument with the documented code before any GPU work (no GPU needed: these
calls never dereference a pointer)."""
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attnres.h")

H = 7168
MB = 1 << 20


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attnres_[a-z_]+)\s*\(", text)))


def _declared_constants():
    text = open(HEADER).read()
    return {m.group(1): int(m.group(2))
            for m in re.finditer(r"#define\s+(ATTNRES_[A-Z0-9_]+)\s+(-?\d+)", text)}


@pytest.fixture(scope="module")
def A():
    from kimi_k3_attention_amd import attnres
    return attnres


def test_library_exports_every_declared_symbol(A):
    names = _declared_functions()
    assert {"attnres_fwd", "attnres_fwd_path", "attnres_validate", "attnres_init",
            "attnres_shutdown", "attnres_strerror"} <= set(names)
    lib = A.lib()
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, f"symbols declared but not exported: {missing}"


def test_automatic_kernel_choice(A):
    """attnres_auto_path, the choice attnres_fwd makes, against the
    documented rule.  At 7168: split up to 40/40/48/56/56/52/60/56 tokens
    for 1..8 block rows, else the tuned row kernel, and row at every T with
    no block rows.  Elsewhere the any-H kernel except: above 8192, split up
    to 72 tokens with block rows; from 7176 to 8192 up to
    16/24/32/40/32/32/32/40 tokens; from 4104 to 7160 up to
    8/16/24/40/40/48/48/48; at 4096 up to 8 with 7 block rows and 16 with
    8; from 3080 to 4088 up to 8 with 8 block rows.  Host only."""
    split_max = [None, 40, 40, 48, 56, 56, 52, 60, 56]
    for nb in range(9):
        for T in (0, 1, 2, 39, 40, 41, 48, 49, 52, 53, 56, 57, 60, 61, 64, 65, 72, 73, 80, 81, 256,
                  1024, 8192):
            want = (A.ATTNRES_PATH_SPLIT if nb > 0 and T <= split_max[nb]
                    else A.ATTNRES_PATH_ROW)
            assert A.attnres_auto_path(T, 7168, nb) == want, (T, nb)
    wide = [0, 16, 24, 32, 40, 32, 32, 32, 40]
    narrow = [0, 8, 16, 24, 40, 40, 48, 48, 48]
    at4096 = [0, 0, 0, 0, 0, 0, 0, 8, 16]

    def limit(H, nb):
        if nb == 0:
            return -1
        if H > 8192:
            return 72
        if H > 7168:
            return wide[nb]
        if H > 4096:
            return narrow[nb]
        if H == 4096:
            return at4096[nb]
        return 8 if (H > 3072 and nb == 8) else -1

    for H in (8, 2048, 2552, 2560, 2880, 3072, 3080, 3584, 4088, 4096, 4104, 5120, 7160,
              7176, 7680, 8192, 8200, 14344, 16384):
        for nb in range(9):
            for T in (1, 8, 9, 16, 17, 24, 25, 32, 33, 40, 41, 48, 49, 72, 73, 1024):
                want = A.ATTNRES_PATH_SPLIT if T <= limit(H, nb) else A.ATTNRES_PATH_ANY_H
                assert A.attnres_auto_path(T, H, nb) == want, (T, H, nb)
    for (T, H, nb), err in (((1, 7170, 8), "ATTNRES_E_UNSUPPORTED"),
                            ((1, 16392, 8), "ATTNRES_E_UNSUPPORTED"),
                            ((1, 7168, 9), "ATTNRES_E_NUM_BLOCKS"),
                            ((-1, 7168, 1), "ATTNRES_E_SHAPE"),
                            ((1, 0, 1), "ATTNRES_E_SHAPE")):
        with pytest.raises(A.AttnResError) as e:
            A.attnres_auto_path(T, H, nb)
        assert e.value.name == err


def test_binding_status_table_matches_header(A):
    consts = _declared_constants()
    for name, code in consts.items():
        if name.startswith("ATTNRES_E_") or name == "ATTNRES_OK":
            assert A.STATUS[code] == name
            assert A.attnres_strerror(code) != "unknown status"
    assert consts["ATTNRES_SPLIT_MAX_TOKENS"] == A.ATTNRES_SPLIT_MAX_TOKENS
    assert consts["ATTNRES_PATH_ROW"] == A.ATTNRES_PATH_ROW
    assert consts["ATTNRES_PATH_SPLIT"] == A.ATTNRES_PATH_SPLIT
    assert consts["ATTNRES_PATH_ANY_H"] == A.ATTNRES_PATH_ANY_H == 3
    assert consts["ATTNRES_MAX_HIDDEN"] == A.ATTNRES_MAX_HIDDEN


def _args(**kw):
    """A valid argument set with fake, 16-byte aligned, disjoint addresses."""
    T = kw.pop("T", 4)
    a = dict(prefix=0x10000000, delta=0x20000000, blocks=0x40000000, ts=8 * H, ss=H, cap=8, nb=4,
             res_w=0x30000000, rms_w=0x30100000, eps=1e-6, onw=0x30200000, oeps=1e-6, widx=-1,
             out=0x50000000, T=T, H=H)
    a.update(kw)
    return a


def _validate(A, a):
    return A.lib().attnres_validate(a["prefix"], a["delta"], a["blocks"], a["ts"], a["ss"], a["cap"],
                                    a["nb"], a["res_w"], a["rms_w"], a["eps"], a["onw"], a["oeps"],
                                    a["widx"], a["out"], a["T"], a["H"])


CASES = [
    ("valid", {}, "ATTNRES_OK"),
    ("valid_no_optional", dict(delta=None, onw=None, widx=-1), "ATTNRES_OK"),
    ("valid_nb0_no_bank", dict(nb=0, blocks=None, widx=-1), "ATTNRES_OK"),
    ("valid_write_last_slot", dict(widx=7), "ATTNRES_OK"),
    ("valid_padded_token_stride", dict(ts=8 * H + 64), "ATTNRES_OK"),
    ("valid_slot_major", dict(ts=H, ss=4 * H), "ATTNRES_OK"),
    ("valid_single_token_any_token_stride", dict(T=1, ts=0), "ATTNRES_OK"),
    ("valid_empty", dict(T=0, prefix=None, out=None), "ATTNRES_OK"),
    ("null_prefix", dict(prefix=None), "ATTNRES_E_NULL"),
    ("null_out", dict(out=None), "ATTNRES_E_NULL"),
    ("null_res_w", dict(res_w=None), "ATTNRES_E_NULL"),
    ("null_rms_w", dict(rms_w=None), "ATTNRES_E_NULL"),
    ("null_bank_with_blocks", dict(blocks=None), "ATTNRES_E_NULL"),
    ("null_bank_with_write", dict(nb=0, blocks=None, widx=0), "ATTNRES_E_NULL"),
    ("negative_T", dict(T=-1), "ATTNRES_E_SHAPE"),
    ("zero_H", dict(H=0), "ATTNRES_E_SHAPE"),
    ("negative_capacity", dict(cap=-1, nb=0), "ATTNRES_E_SHAPE"),
    ("too_many_tokens", dict(T=1 << 31), "ATTNRES_E_SHAPE"),
    ("tokens_past_dispatch_limit", dict(T=8388608, H=8, ts=64, ss=8, blocks=0x80000000,
                                        out=0x200000000), "ATTNRES_E_SHAPE"),
    ("tokens_at_dispatch_limit", dict(T=8388607, H=8, ts=64, ss=8, blocks=0x80000000,
                                      out=0x200000000), "ATTNRES_OK"),
    ("huge_stride", dict(ts=1 << 50), "ATTNRES_E_SHAPE"),
    ("valid_other_hidden_size", dict(H=4096), "ATTNRES_OK"),
    ("valid_smallest_hidden", dict(H=8), "ATTNRES_OK"),
    ("valid_largest_hidden", dict(H=16384, ts=8 * 16384, ss=16384), "ATTNRES_OK"),
    ("hidden_not_multiple_of_8", dict(H=7164), "ATTNRES_E_UNSUPPORTED"),
    ("hidden_above_max", dict(H=16392, ts=8 * 16392, ss=16392), "ATTNRES_E_UNSUPPORTED"),
    ("nb_negative", dict(nb=-1), "ATTNRES_E_NUM_BLOCKS"),
    ("nb_above_8", dict(nb=9, cap=10, ts=10 * H), "ATTNRES_E_NUM_BLOCKS"),
    ("nb_above_capacity", dict(nb=5, cap=4, ts=4 * H), "ATTNRES_E_NUM_BLOCKS"),
    ("widx_below_minus_one", dict(widx=-2), "ATTNRES_E_WRITE_IDX"),
    ("widx_at_capacity", dict(widx=8), "ATTNRES_E_WRITE_IDX"),
    ("eps_negative", dict(eps=-1e-6), "ATTNRES_E_EPS"),
    ("eps_nan", dict(eps=float("nan")), "ATTNRES_E_EPS"),
    ("eps_inf", dict(eps=float("inf")), "ATTNRES_E_EPS"),
    ("out_eps_negative", dict(oeps=-1.0), "ATTNRES_E_EPS"),
    ("misaligned_prefix", dict(prefix=0x10000008), "ATTNRES_E_ALIGN"),
    ("misaligned_delta", dict(delta=0x20000002), "ATTNRES_E_ALIGN"),
    ("misaligned_bank", dict(blocks=0x40000004), "ATTNRES_E_ALIGN"),
    ("misaligned_weight", dict(onw=0x30200008), "ATTNRES_E_ALIGN"),
    ("misaligned_out", dict(out=0x50000002), "ATTNRES_E_ALIGN"),
    ("token_stride_not_multiple_of_8", dict(ts=8 * H + 4), "ATTNRES_E_ALIGN"),
    ("negative_stride", dict(ss=-H), "ATTNRES_E_STRIDE"),
    ("slot_stride_overlaps_rows", dict(ss=H - 8), "ATTNRES_E_STRIDE"),
    ("token_stride_overlaps_slots", dict(ts=7 * H), "ATTNRES_E_STRIDE"),
    ("zero_strides", dict(ts=0, ss=0), "ATTNRES_E_STRIDE"),
    ("out_aliases_prefix", dict(out=0x10000000), "ATTNRES_E_ALIAS"),
    ("out_overlaps_prefix_tail", dict(out=0x10000000 + 2 * H * 3), "ATTNRES_E_ALIAS"),
    ("out_inside_bank", dict(out=0x40000000 + 2 * H * 9), "ATTNRES_E_ALIAS"),
    ("out_on_weight", dict(out=0x30100000), "ATTNRES_E_ALIAS"),
    ("prefix_written_over_delta", dict(delta=0x10000000 + 32), "ATTNRES_E_ALIAS"),
    ("bank_written_over_prefix", dict(widx=2, prefix=0x40000000 + 2 * H * 8), "ATTNRES_E_ALIAS"),
    ("bank_written_over_weight", dict(widx=2, res_w=0x40000000 + 2 * H * 17), "ATTNRES_E_ALIAS"),
]


@pytest.mark.parametrize("name,mod,expect", CASES, ids=[c[0] for c in CASES])
def test_validate(A, name, mod, expect):
    rc = _validate(A, _args(**mod))
    assert A.STATUS[rc] == expect


def _validate_strided(A, a):
    return A.lib().attnres_validate_strided(
        a["prefix"], a.get("ps", a["H"]), a["delta"], a.get("ds", a["H"]), a["blocks"], a["ts"],
        a["ss"], a["cap"], a["nb"], a["res_w"], a["rms_w"], a["eps"], a["onw"], a["oeps"], a["widx"],
        a["out"], a.get("os", a["H"]), a["T"], a["H"])


P0 = 0x10000000
STRIDED_CASES = [
    ("dense_strides", {}, "ATTNRES_OK"),
    ("padded_rows", dict(ps=H + 64, ds=H + 128, os=2 * H), "ATTNRES_OK"),
    # prefix and delta interleaved in one [T, 2H] buffer (prefix is written)
    ("prefix_delta_interleaved", dict(delta=P0 + 2 * H, ps=2 * H, ds=2 * H), "ATTNRES_OK"),
    ("out_interleaved_with_prefix", dict(out=P0 + 2 * H, ps=2 * H, os=2 * H), "ATTNRES_OK"),
    ("out_interleaved_overlapping", dict(out=P0 + 2 * (H - 8), ps=2 * H, os=2 * H), "ATTNRES_E_ALIAS"),
    ("out_other_stride_overlapping", dict(out=P0 + 2 * H, ps=2 * H, os=3 * H), "ATTNRES_E_ALIAS"),
    ("delta_interleaved_overlapping", dict(delta=P0 + 2 * H - 16, ps=2 * H, ds=2 * H), "ATTNRES_E_ALIAS"),
    ("row_stride_below_H", dict(ps=H - 8), "ATTNRES_E_STRIDE"),
    ("row_stride_zero", dict(os=0), "ATTNRES_E_STRIDE"),
    ("row_stride_negative", dict(ds=-H), "ATTNRES_E_STRIDE"),
    ("row_stride_not_multiple_of_8", dict(os=H + 4), "ATTNRES_E_ALIGN"),
    ("row_stride_huge", dict(ps=1 << 50), "ATTNRES_E_SHAPE"),
    ("single_token_ignores_row_strides", dict(T=1, ps=0, ds=-5, os=3), "ATTNRES_OK"),
    ("no_delta_ignores_its_stride", dict(delta=None, ds=3), "ATTNRES_OK"),
]


@pytest.mark.parametrize("name,mod,expect", STRIDED_CASES, ids=[c[0] for c in STRIDED_CASES])
def test_validate_strided(A, name, mod, expect):
    rc = _validate_strided(A, _args(**mod))
    assert A.STATUS[rc] == expect


def test_dense_validate_is_strided_validate_with_stride_H(A):
    for _, mod, _ in CASES:
        a = _args(**mod)
        assert _validate(A, a) == _validate_strided(A, a), mod


def test_row_overlap_check_against_brute_force(A):
    """out (written) against prefix rows, both strided: the library must
    reject every layout where some element is shared, and, when both have the
    same row stride (or one has a single row), accept every layout where none
    is.  Element sets are enumerated on the host."""
    rng = np.random.default_rng(11)
    h = 16
    far = 0x7000000
    checked_equal = 0
    for _ in range(3000):
        T = int(rng.integers(1, 6))
        ps = h * int(rng.integers(1, 5)) if rng.random() < 0.7 else h + 8 * int(rng.integers(0, 6))
        os_ = ps if rng.random() < 0.6 else h + 8 * int(rng.integers(0, 10))
        off = 16 * int(rng.integers(-40, 40))       # byte offset of out from prefix
        prefix, out = 0x1000000, 0x1000000 + off
        pe = {prefix + 2 * (t * ps + k) for t in range(T) for k in range(h)}
        oe = {out + 2 * (t * os_ + k) for t in range(T) for k in range(h)}
        shared = bool(pe & oe)
        a = dict(prefix=prefix, ps=ps, delta=None, ds=h, blocks=None, ts=0, ss=0, cap=0, nb=0,
                 res_w=far, rms_w=far + 0x10000, eps=1e-6, onw=None, oeps=0.0, widx=-1, out=out,
                 os=os_, T=T, H=h)
        rc = _validate_strided(A, a)
        if shared:
            assert A.STATUS[rc] == "ATTNRES_E_ALIAS", (T, ps, os_, off)
        elif ps == os_ or T == 1:
            assert rc == 0, (T, ps, os_, off, A.STATUS[rc])
            checked_equal += 1
    assert checked_equal > 500


def test_accepted_layouts_never_share_a_written_element(A):
    """Every buffer at once, on the host: prefix, delta, a bank with random
    token and slot strides (token- or slot-major, padded or interleaved),
    out and the three weights, placed at random 16-byte offsets in a small
    address range so that they often meet.  Whenever the library accepts a
    layout, no element the call writes (out; prefix with a delta; bank slot
    block_write_idx of every token) is shared with any other element the
    call reads or writes, and distinct bank rows, prefix rows and out rows
    are disjoint.  Element sets are enumerated exactly."""
    rng = np.random.default_rng(23)
    h = 16
    accepted = rejected = 0
    for _ in range(4000):
        T = int(rng.integers(1, 5))
        cap = int(rng.integers(1, 4))
        nb = int(rng.integers(0, cap + 1))
        widx = int(rng.integers(-1, cap))
        has_d, has_o = rng.random() < 0.7, rng.random() < 0.7
        ps = h + 8 * int(rng.integers(0, 5))
        ds = h + 8 * int(rng.integers(0, 5))
        os_ = h + 8 * int(rng.integers(0, 5))
        if rng.random() < 0.5:                       # token-major, maybe padded
            ss = h + 8 * int(rng.integers(0, 3))
            ts = cap * ss + 8 * int(rng.integers(-2, 4))
        else:                                        # slot-major
            ts = h + 8 * int(rng.integers(0, 3))
            ss = T * ts + 8 * int(rng.integers(-2, 4))
        ts, ss = max(ts, 0), max(ss, 0)

        def place():
            return 0x1000000 + 16 * int(rng.integers(0, 64))

        a = dict(prefix=place(), ps=ps, delta=place() if has_d else None, ds=ds,
                 blocks=place(), ts=ts, ss=ss, cap=cap, nb=nb, res_w=place(), rms_w=place(),
                 eps=1e-6, onw=place() if has_o else None, oeps=1e-6, widx=widx, out=place(),
                 os=os_, T=T, H=h)
        rc = _validate_strided(A, a)
        if rc != 0:
            assert A.STATUS[rc] in ("ATTNRES_E_ALIAS", "ATTNRES_E_STRIDE"), A.STATUS[rc]
            rejected += 1
            continue
        accepted += 1

        def row(base, off):
            return {base + 2 * (off + k) for k in range(h)}

        bank_used = nb > 0 or widx >= 0
        reads, writes = [], []                       # (label, element set)
        for t in range(T):
            reads.append((("prefix", t), row(a["prefix"], t * ps)))
            if has_d:
                reads.append((("delta", t), row(a["delta"], t * ds)))
                writes.append((("prefix", t), row(a["prefix"], t * ps)))
            writes.append((("out", t), row(a["out"], t * os_)))
            if bank_used:
                for i in range(cap):
                    reads.append((("bank", t, i), row(a["blocks"], t * ts + i * ss)))
                if widx >= 0:
                    writes.append((("bank", t, widx), row(a["blocks"], t * ts + widx * ss)))
        for name in ("res_w", "rms_w", "onw"):
            if a[name] is not None:
                reads.append(((name,), row(a[name], 0)))
        everything = reads + [w for w in writes if w[0][0] == "out"]
        for wl, we in writes:
            for ol, oe in everything:
                if ol != wl:
                    assert not (we & oe), (a, wl, ol)
        banks = [e for l, e in reads if l[0] == "bank"]
        assert sum(len(e) for e in banks) == len(set().union(*banks)) if banks else True, a
    assert accepted > 300 and rejected > 300, (accepted, rejected)


def test_read_only_overlaps_are_allowed(A):
    # prefix read-only (no delta) may share memory with a read-only bank and
    # with the weights; only written buffers must be exclusive.
    a = _args(delta=None, widx=-1, res_w=0x10000000, rms_w=0x10000000)
    assert _validate(A, a) == 0


def test_fwd_rejects_before_any_gpu_work(A):
    """attnres_fwd runs the same checks first: an invalid call returns its
    code without touching the (fake) pointers or needing a GPU."""
    a = _args(H=7164)
    lib = A.lib()
    for fn, extra in ((lib.attnres_fwd, [None]), (lib.attnres_fwd_path, [None, A.ATTNRES_PATH_ROW])):
        rc = fn(a["prefix"], a["delta"], a["blocks"], a["ts"], a["ss"], a["cap"], a["nb"], a["res_w"],
                a["rms_w"], a["eps"], a["onw"], a["oeps"], a["widx"], a["out"], a["T"], a["H"], *extra)
        assert A.STATUS[rc] == "ATTNRES_E_UNSUPPORTED"
    a = _args()
    rc = lib.attnres_fwd_path(a["prefix"], a["delta"], a["blocks"], a["ts"], a["ss"], a["cap"], a["nb"],
                              a["res_w"], a["rms_w"], a["eps"], a["onw"], a["oeps"], a["widx"], a["out"],
                              a["T"], a["H"], None, 7)
    assert A.STATUS[rc] == "ATTNRES_E_PATH"


def test_product_path_never_touches_the_oracle():
    """The package and its native sources do not import, load or name the
    oracle (only tests, the smoke check and the benchmark's CPU leg may)."""
    pkg = os.path.join(ROOT, "kimi_k3_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"(import\s+oracle|from\s+oracle|liboracle|oracle_attnres|oracle\.)",
                                     text), f"{f} uses the oracle"


def test_plain_c_caller_builds_and_links():
    """tests/c/abi_check, a C program that calls libattnres directly (no
    Python), compiles against include/attnres.h and links the library, the
    oracle and the HIP runtime; without a GPU it stops at the device query
    with status 2."""
    import importlib.util
    import subprocess
    spec = importlib.util.spec_from_file_location(
        "build_abi_check", os.path.join(ROOT, "tests", "c", "build_abi_check.py"))
    cbuild = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(cbuild)
    exe = cbuild.build()
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except ImportError:
        has_gpu = False
    if has_gpu:
        pytest.skip("a GPU is present: the run is covered by the GPU test")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert res.returncode == 2, res.stdout + res.stderr


def test_validation_under_sanitizers(tmp_path):
    """The host-side checks (kimi_k3_attention_amd/csrc/attnres_validate.cpp,
    plain C++), built with g++ under the address and undefined-behaviour
    sanitizers, through tests/c/validate_fuzz.cpp: 600,000 calls with
    plausible and extreme sizes, strides, indices, epsilons and pointers
    return only documented statuses, with no overflow or bad access; and the
    choice of the split path's two workspace frames from set-up timings."""
    import shutil
    import subprocess
    if shutil.which("g++") is None:
        pytest.skip("g++ not installed")
    exe = str(tmp_path / "validate_fuzz")
    src = os.path.join(ROOT, "kimi_k3_attention_amd", "csrc")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"), "-I", src,
           os.path.join(src, "attnres_validate.cpp"),
           os.path.join(ROOT, "tests", "c", "validate_fuzz.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if build.returncode != 0 and "asan" in (build.stderr or "").lower():
        pytest.skip("the sanitizer runtime is not installed: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr
    # (another preloaded library may come before the sanitizer's runtime)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0 and res.stdout.startswith("ok "), res.stdout + res.stderr


def test_partial_bytes(A):
    """The two-kernel form's state: fp32 [T, H] plus two fp32 per token."""
    lib = A.lib()
    assert lib.attnres_partial_bytes(1, H) == 4 * H + 8
    assert lib.attnres_partial_bytes(1024, 5120) == 4 * 1024 * 5120 + 8 * 1024
    assert lib.attnres_partial_bytes(0, H) == 0
    assert A.STATUS[lib.attnres_partial_bytes(-1, H)] == "ATTNRES_E_SHAPE"
    assert A.STATUS[lib.attnres_partial_bytes(4, 7164)] == "ATTNRES_E_UNSUPPORTED"


def _two_part_rc(A, fn_name, a, partial, nbytes):
    return getattr(A.lib(), fn_name)(
        a["prefix"], a["H"], a["delta"], a["H"], a["blocks"], a["ts"], a["ss"], a["cap"], a["nb"],
        a["res_w"], a["rms_w"], a["eps"], a["onw"], a["oeps"], a["widx"], a["out"], a["H"], a["T"],
        a["H"], partial, nbytes, None)


@pytest.mark.parametrize("fn_name", ["attnres_fwd_bank", "attnres_fwd_cur"])
def test_two_kernel_form_rejects_before_any_gpu_work(A, fn_name):
    """Both halves check the whole call as attnres_fwd does, then the partial
    buffer, and return the code without touching the (fake) pointers."""
    a = _args()
    need = A.lib().attnres_partial_bytes(a["T"], H)
    part = 0x60000000
    assert A.STATUS[_two_part_rc(A, fn_name, _args(H=7164), part, need)] == "ATTNRES_E_UNSUPPORTED"
    assert A.STATUS[_two_part_rc(A, fn_name, a, None, need)] == "ATTNRES_E_NULL"
    assert A.STATUS[_two_part_rc(A, fn_name, a, part + 8, need)] == "ATTNRES_E_ALIGN"
    assert A.STATUS[_two_part_rc(A, fn_name, a, part, need - 16)] == "ATTNRES_E_SHAPE"
    # overlapping the output, the bank or a weight
    for other in ("out", "blocks", "res_w"):
        assert A.STATUS[_two_part_rc(A, fn_name, a, a[other], need)] == "ATTNRES_E_ALIAS", other
    # no bank rows: no buffer needed, so these get as far as the launch (only
    # the bank half, which then launches nothing, returns OK without a GPU)
    if fn_name == "attnres_fwd_bank":
        assert A.STATUS[_two_part_rc(A, fn_name, _args(nb=0, blocks=None), None, 0)] == "ATTNRES_OK"
    assert A.STATUS[_two_part_rc(A, fn_name, _args(T=0, prefix=None, out=None), None, 0)] == "ATTNRES_OK"
