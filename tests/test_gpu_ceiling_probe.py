"""The benchmark's memory-traffic probe (bench_ceiling.hip) really reads every
source row and writes every row it is charged for: its outputs are checked
against the same XOR folding done with numpy on the host."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

H = 7168


def _rotl(v: np.ndarray, s: int) -> np.ndarray:
    if s == 0:
        return v
    return ((v << np.uint32(s)) | (v >> np.uint32(32 - s))).astype(np.uint32)


@pytest.mark.parametrize("reads,wd,wi", [(10, 1, 2), (10, 3, 0), (9, 1, 0), (10, 0, 0), (1, 1, 0)])
def test_probe_moves_every_row(reads, wd, wi):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    lib = bench.load_ceiling_probe()
    T, pad = 5, 64
    ss, ds = reads * H + pad, max(wd, 1) * H + pad
    rng = np.random.default_rng(reads * 100 + wd * 10 + wi)
    src_h = rng.integers(0, 1 << 16, size=T * ss, dtype=np.uint16)
    dst_h = np.full(T * ds, 0x7F85, dtype=np.uint16)
    src = torch.from_numpy(src_h.view(np.int16)).cuda()
    dst = torch.from_numpy(dst_h.view(np.int16)).cuda()
    rows_all = src_h.reshape(T, ss)[:, :reads * H].reshape(T, reads, H)
    folds = set()
    for t in range(T):
        acc = np.bitwise_xor.reduce(rows_all[t].view(np.uint32), axis=0).reshape(-1, 4)
        folds |= set(np.bitwise_xor.reduce(acc, axis=1).tolist())
    never = next(v for v in range(1, 1 << 20) if v not in folds)
    rc = lib.ceiling_stream(src.data_ptr(), ss, dst.data_ptr(), ds, reads, wd, wi, T, never,
                            torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    got_src = src.cpu().numpy().view(np.uint16)
    got_dst = dst.cpu().numpy().view(np.uint16)

    want_src = src_h.copy()
    want_dst = dst_h.copy()
    for t in range(T):
        rows = src_h[t * ss:t * ss + reads * H].reshape(reads, H).view(np.uint32)
        acc = np.bitwise_xor.reduce(rows, axis=0)
        for w in range(wd):
            want_dst[t * ds + w * H:t * ds + (w + 1) * H] = _rotl(acc, w).view(np.uint16)
        for k in range(wi):
            want_src[t * ss + k * H:t * ss + (k + 1) * H] = (rows[k] ^ rows[reads - 1]).view(np.uint16)
    assert (got_dst == want_dst).all(), "dst rows (or the padding after them) differ"
    assert (got_src == want_src).all(), "source rows (or the padding after them) differ"


def test_probe_rejects_unknown_shapes():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    lib = bench.load_ceiling_probe()
    assert lib.ceiling_stream(None, 0, None, 0, 7, 1, 0, 4, 0, None) == -1
    assert lib.ceiling_mid(None, None, None, None, 4, 1, None) == -1


@pytest.mark.parametrize("cached", [0, 1])
def test_mid_probe_moves_every_row(cached):
    """The mid-prefill-layout probe reads all 8 bank rows, prefix and delta,
    and writes out, prefix and bank slot 3 (nothing else), whichever cache
    policy its two rewritten rows are read with."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    lib = bench.load_ceiling_probe()
    T = 6
    rng = np.random.default_rng(40 + cached)
    bank_h = rng.integers(0, 1 << 16, size=T * 8 * H, dtype=np.uint16)
    pf_h = rng.integers(0, 1 << 16, size=T * H, dtype=np.uint16)
    dl_h = rng.integers(0, 1 << 16, size=T * H, dtype=np.uint16)
    out_h = np.full(T * H, 0x7F85, dtype=np.uint16)
    dev = [torch.from_numpy(a.view(np.int16)).cuda() for a in (bank_h, pf_h, dl_h, out_h)]
    rc = lib.ceiling_mid(dev[0].data_ptr(), dev[1].data_ptr(), dev[2].data_ptr(), dev[3].data_ptr(),
                         T, cached, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    bank, pf, dl, out = (d.cpu().numpy().view(np.uint16) for d in dev)
    b = bank_h.reshape(T, 8, H).view(np.uint32).reshape(T, 8, H // 2)
    p32 = pf_h.view(np.uint32).reshape(T, H // 2)
    d32 = dl_h.view(np.uint32).reshape(T, H // 2)
    cur = p32 ^ d32
    want_out = np.bitwise_xor.reduce(b, axis=1) ^ p32 ^ d32
    want_bank = b.copy()
    want_bank[:, 3] = cur
    assert (out.view(np.uint32).reshape(T, H // 2) == want_out).all()
    assert (pf.view(np.uint32).reshape(T, H // 2) == cur).all()
    assert (bank.view(np.uint32).reshape(T, 8, H // 2) == want_bank).all()
    assert (dl == dl_h).all()


@pytest.mark.parametrize("Hx,cached", [(5120, 0), (2888, 1), (12288, 0), (16376, 1)])
def test_mid_probe_any_hidden_size(Hx, cached):
    """The any-H mid-prefill probe (the library's any-H launch shape, row ends
    masked) reads every row and writes out, prefix and bank slot 3 only."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bench
    lib = bench.load_ceiling_probe()
    T = 5
    rng = np.random.default_rng(Hx + cached)
    bank_h = rng.integers(0, 1 << 16, size=T * 8 * Hx, dtype=np.uint16)
    pf_h = rng.integers(0, 1 << 16, size=T * Hx, dtype=np.uint16)
    dl_h = rng.integers(0, 1 << 16, size=T * Hx, dtype=np.uint16)
    out_h = np.full(T * Hx, 0x7F85, dtype=np.uint16)
    dev = [torch.from_numpy(a.view(np.int16)).cuda() for a in (bank_h, pf_h, dl_h, out_h)]
    rc = lib.ceiling_mid_h(dev[0].data_ptr(), dev[1].data_ptr(), dev[2].data_ptr(),
                           dev[3].data_ptr(), T, Hx, bench.anyh_threads(Hx), cached,
                           torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    bank, pf, dl, out = (d.cpu().numpy().view(np.uint16) for d in dev)
    n = Hx // 2
    b = bank_h.view(np.uint32).reshape(T, 8, n)
    p32 = pf_h.view(np.uint32).reshape(T, n)
    d32 = dl_h.view(np.uint32).reshape(T, n)
    cur = p32 ^ d32
    want_bank = b.copy()
    want_bank[:, 3] = cur
    assert (out.view(np.uint32).reshape(T, n) == np.bitwise_xor.reduce(b, axis=1) ^ p32 ^ d32).all()
    assert (pf.view(np.uint32).reshape(T, n) == cur).all()
    assert (bank.view(np.uint32).reshape(T, 8, n) == want_bank).all()
    assert (dl == dl_h).all()
    assert lib.ceiling_mid_h(None, None, None, None, 4, Hx, 64, 0, None) == -1
