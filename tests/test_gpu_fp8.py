"""FP8 block records and the geometric screen over them, on the HIP path vs
the fp64 oracle, through the C ABI.

The FP8 centroid is the float64 mean rounded to nearest even in the format
(E4M3 or E5M2), saturating: the codes must match the oracle's exactly. The
radius about it is float32 rounded up on the GPU and float64 in the oracle;
the GPU value must not be below the oracle's and within 2^-20 relative of it.
Sets are compared bit-exactly with thresholds placed 1e-3 away from every
bound, outputs at the usual bar."""
import numpy as np
import pytest
import torch

import bruteforce
import learned_threshold_block_amd as eta
import oracle.eta_oracle as E
import workloads as W
from gpu_util import Dev, check_output, check_sets_and_counts, log, oracle_decode, prepared

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _codes(values, fmt):
    """Oracle values -> format codes, through the brute force's code table
    (magnitude code, plus the sign bit for negative values and -0)."""
    table = {v: c for c, v in bruteforce.fp8_values(fmt).items() if c < 0x80}
    flat = np.asarray(values, dtype=np.float64).ravel()
    out = np.array([table[abs(float(v))] | (0x80 if np.signbit(v) else 0) for v in flat], dtype=np.uint8)
    return out.reshape(np.shape(values))


def _check_fp8(wl, dev, fmt):
    mu, R = E.build_summaries_fp8(wl.k_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, fmt)
    used = np.zeros(mu.shape[:2], dtype=bool)
    for n in range(wl.n_seqs):
        used[wl.block_table[n, :int(wl.seq_lens[n]) // 64]] = True
    codes, r8 = dev.fp8_codes()
    assert np.array_equal(codes[used], _codes(mu[used], fmt))
    ref, got = R[used], r8[used].astype(np.float64)
    inf = np.isinf(ref)
    assert np.array_equal(inf, np.isinf(got))
    assert np.all(got[~inf] >= ref[~inf])
    assert np.all(got[~inf] <= ref[~inf] * (1 + 2.0 ** -20))


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
@pytest.mark.parametrize("name,kw", [
    ("seq_32k", dict(seq_lens=[4096 + 17, 64 * 40], n_seqs=2)),
    ("seq_32k", dict(seq_lens=[3000, 2000], d=64, kv_dtype="f32")),
    ("ragged_16", dict(n_seqs=3, seq_lens=[300, 4097, 640], h_q=8, h_kv=2, d=128)),
])
def test_fp8_records(name, kw, fmt):
    log(f"[fp8] {fmt} {name} {kw}")
    wl = W.make_workload(name, **kw)
    dev = Dev(wl, fp8=fmt)
    dev.build()
    torch.cuda.synchronize()
    _check_fp8(wl, dev, fmt)
    dev2 = Dev(wl)
    dev2.build()
    torch.cuda.synchronize()
    assert np.array_equal(dev.mu_bits(), dev2.mu_bits())
    assert np.array_equal(dev.radius(), dev2.radius())


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_fp8_rounding_edges(fmt):
    """Blocks of one repeated value per column (the mean is that value):
    ties, subnormals, saturation and signed zero, plus non-finite blocks."""
    d = 64
    cols = np.array([1.0625, 1.1875, 460.0, 500.0, -1e6, 2.0 ** -10, 3 * 2.0 ** -11, -0.3, 2.0 ** -17,
                     3 * 2.0 ** -17, 70000.0, -2.0 ** -30, 0.0, 448.0, 57344.0, 1e-3])
    n_pages = 4
    wl = W.make_workload("tiny_4k_f32", seq_len=64 * n_pages, needles=0)
    for i in range(2):
        row = np.resize(np.roll(cols, i), d)
        wl.k_pages[i, 0] = np.tile(row, (64, 1)).astype(np.float32)
    wl.k_pages[2, 0, 3, 7] = np.inf
    wl.k_pages[3, 0, 9, 1] = np.nan
    dev = Dev(wl, fp8=fmt)
    dev.build()
    torch.cuda.synchronize()
    _check_fp8(wl, dev, fmt)


def test_append_and_prefill_build_fp8():
    """FP8 records built token by token through eta_append_kv, and by the
    prompt pass, equal the bulk build."""
    wl = W.make_workload("seq_32k", seq_lens=[64 * 3 + 10], h_q=4, h_kv=2, d=128, needles=0)
    dev = Dev(wl, fp8="e5m2")
    dev.build()
    torch.cuda.synchronize()
    cache2 = eta.Cache.empty(wl.num_pages, wl.h_kv, wl.d, dtype=dev.cache.k_pages.dtype, fp8="e5m2")
    T = int(wl.seq_lens[0])
    for t in range(T):
        lens = torch.tensor([t], dtype=torch.int32, device="cuda")
        page = int(wl.block_table[0, t // 64])
        kn = dev.cache.k_pages[page, :, t % 64][None].contiguous()
        vn = dev.cache.v_pages[page, :, t % 64][None].contiguous()
        eta.append_kv(cache2, lens, dev.bt, kn, vn)
    torch.cuda.synchronize()
    for j in range(T // 64):
        page = int(wl.block_table[0, j])
        assert torch.equal(cache2.mu8[page], dev.cache.mu8[page])
        assert torch.equal(cache2.radius8[page], dev.cache.radius8[page])
    dev3 = Dev(wl, fp8="e5m2")
    q_all = W.trace_queries(wl, seed=3)
    eta.prefill(dev3.cache, dev3.seq_lens, dev3.bt, eta.upload(q_all, wl.kv_dtype, "cuda"), eta.ETA_TAU_LEARNED,
                torch.ones(wl.h_q, dtype=torch.float32, device="cuda"), w=dev3.w)
    torch.cuda.synchronize()
    c3, r3 = dev3.fp8_codes()
    c1, r1 = dev.fp8_codes()
    assert np.array_equal(c3, c1) and np.array_equal(r3, r1)


@pytest.mark.parametrize("fmt,kw", [
    ("e4m3", dict(seq_lens=[64 * 70 + 3, 64 * 64, 129], h_q=8, h_kv=2, d=128)),
    ("e5m2", dict(seq_lens=[5000, 7000], h_q=4, h_kv=4, d=64, kv_dtype="f32", mode="calibrated")),
    ("e4m3", dict(seq_lens=[3000, 64 * 20 + 1], h_q=4, h_kv=2, d=64)),              # two heads per group
    ("e4m3", dict(seq_lens=[64 * 130 + 63, 64 * 5], h_q=16, h_kv=2, d=128, lwb=2, a=0.4)),
    ("e5m2", dict(n_seqs=4, h_q=8, h_kv=2, d=128, paged=True, density=[0.05, 0.3, 0.6, 0.9] * 2,
                  seq_lens=[9000, 300, 64 * 12, 4097])),
])
def test_fp8_decode_parity(fmt, kw):
    log(f"[fp8 decode] {fmt} {kw}")
    wl, summ = prepared("seq_32k", bound="geometric_fp8", fp8=fmt, **kw)
    dev = Dev(wl, fp8=fmt)
    dev.build()
    o = dev.decode(bound="geometric_fp8")
    st = dev.stats()
    res = oracle_decode(wl, summaries=summ, bound="geometric_fp8", fp8=fmt)
    check_sets_and_counts(wl, res, st)
    check_output(wl, res, o)
    log(f"  per-head blocks {int(res.per_head.sum())}, union {int(res.union.sum())}")


def test_fp8_requires_records():
    wl = W.make_workload("seq_32k", seq_lens=[640], h_q=4, h_kv=2, needles=0)
    dev = Dev(wl)
    with pytest.raises(eta.EtaError):
        dev.decode(bound="geometric_fp8", bias=np.zeros(wl.h_q))
