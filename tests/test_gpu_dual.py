"""Dual screen on the HIP path vs the fp64 oracle, through the C ABI.

The dual score (min of the geometric bound and the z-deviation estimate,
Sections 3.1 and F.1) decides the admitted sets; thresholds are placed with a
1e-3 margin from every dual score, so the sets compare bit-exactly. Records:
the coordinate deviation sigma^ is float16 of a float64 value on both sides;
the two float64 values can differ in their last bits (summation order), so a
float16 result may differ by one unit in the last place, rarely."""
import numpy as np
import pytest
import torch

import learned_threshold_block_amd as eta
import oracle.eta_oracle as E
import workloads as W
from gpu_util import Dev, check_output, check_sets_and_counts, log, oracle_decode, prepared

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _ulps(a_bits, b_bits):
    a = a_bits.astype(np.int32)
    b = b_bits.astype(np.int32)
    # float16 bit patterns of non-negative numbers order like integers
    return np.abs(a - b)


@pytest.mark.parametrize("name,kw", [
    ("seq_32k", dict(seq_lens=[4096 + 17, 64 * 40], n_seqs=2)),
    ("seq_32k", dict(seq_lens=[3000, 2000], d=64, kv_dtype="f32")),
    ("ragged_16", dict(n_seqs=3, seq_lens=[300, 4097, 640], h_q=8, h_kv=2, d=128)),
])
def test_sigma_records(name, kw):
    log(f"[sigma] {name} {kw}")
    wl = W.make_workload(name, **kw)
    dev = Dev(wl, with_sigma=True)
    dev.build()
    torch.cuda.synchronize()
    ref = E.build_sigmas(wl.k_pages, wl.kv_dtype, wl.block_table, wl.seq_lens)
    used = ~np.isnan(ref[..., 0])
    ref_bits = ref[used].astype(np.float16).view(np.uint16)
    got = dev.sigma_bits()[used]
    d = _ulps(got, ref_bits)
    log(f"  {int((d > 0).sum())} of {d.size} coordinates differ, max {int(d.max())} ulp")
    assert d.max() <= 1
    assert (d > 0).mean() <= 1e-3
    # records other than sigma are unchanged by building it
    dev2 = Dev(wl)
    dev2.build()
    torch.cuda.synchronize()
    assert np.array_equal(dev.mu_bits(), dev2.mu_bits())
    assert np.array_equal(dev.radius(), dev2.radius())


def test_sigma_rounding_edges():
    """Blocks of keys a +/- b per coordinate: the deviation is b exactly, so
    float16 ties, subnormals and overflow are decided identically on both sides."""
    d = 64
    cases = [(3.0, 1.0 + 2.0 ** -11), (3.0, 1.0 + 3 * 2.0 ** -11), (0.5, 2.0 ** -20), (0.0, 70000.0),
             (-7.25, 0.125), (5.0, 0.0)]
    n_pages = len(cases) + 2
    wl = W.make_workload("tiny_4k_f32", seq_len=64 * n_pages, needles=0)
    for i, (a, b) in enumerate(cases):
        blk = np.full((64, d), a, dtype=np.float64)
        blk[::2] += b
        blk[1::2] -= b
        wl.k_pages[i, 0] = blk.astype(np.float32)
    wl.k_pages[len(cases), 0, 3, 7] = np.inf
    wl.k_pages[len(cases) + 1, 0, 9, 1] = np.nan
    dev = Dev(wl, with_sigma=True)
    dev.build()
    torch.cuda.synchronize()
    ref = E.build_sigmas(wl.k_pages, wl.kv_dtype, wl.block_table, wl.seq_lens)[:n_pages, 0]
    got = dev.sigma_bits()[:n_pages, 0]
    with np.errstate(over="ignore"):
        ref_bits = ref.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref_bits)


def test_append_builds_sigma():
    """Records built token by token through eta_append_kv equal the bulk build,
    deviation included."""
    wl = W.make_workload("seq_32k", seq_lens=[64 * 2 + 10], h_q=4, h_kv=2, d=128, needles=0)
    dev = Dev(wl, with_sigma=True)
    dev.build()
    torch.cuda.synchronize()
    cache2 = eta.Cache.empty(wl.num_pages, wl.h_kv, wl.d, dtype=dev.cache.k_pages.dtype, with_sigma=True)
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
        assert torch.equal(cache2.sigma[page], dev.cache.sigma[page])
        assert torch.equal(cache2.mu[page], dev.cache.mu[page])
        assert torch.equal(cache2.radius[page], dev.cache.radius[page])


@pytest.mark.parametrize("kw", [
    dict(seq_lens=[64 * 70 + 3, 64 * 64, 129], h_q=8, h_kv=2, d=128),
    dict(seq_lens=[5000, 7000], h_q=4, h_kv=4, d=64, kv_dtype="f32", mode="calibrated"),
    dict(seq_lens=[3000, 64 * 20 + 1], h_q=4, h_kv=2, d=64),                        # two heads per group
    dict(seq_lens=[64 * 130 + 63, 64 * 5], h_q=16, h_kv=2, d=128, lwb=2, a=0.4),
    dict(seq_lens=[64 * 200], h_q=8, h_kv=2, d=128, mode="calibrated", density=0.1, z=1.0),
    dict(n_seqs=4, h_q=8, h_kv=2, d=128, paged=True, density=[0.05, 0.3, 0.6, 0.9] * 2,
         seq_lens=[9000, 300, 64 * 12, 4097]),
])
def test_dual_decode_parity(kw):
    kw = dict(kw)
    z = kw.pop("z", 2.0)
    log(f"[dual] z={z} {kw}")
    wl, summ = prepared("seq_32k", bound="dual", z=z, **kw)
    dev = Dev(wl, with_sigma=True)
    dev.build()
    o = dev.decode(bound="dual", z=z)
    st = dev.stats()
    res = oracle_decode(wl, summaries=summ, bound="dual", z=z)
    check_sets_and_counts(wl, res, st)
    check_output(wl, res, o)
    # the dual sets nest in the geometric ones at the same thresholds
    geo = oracle_decode(wl, summaries=summ[:2])
    if not res.rescued.any() and not geo.rescued.any():
        assert np.all(res.admitted <= geo.admitted)
    log(f"  per-head blocks: dual {int(res.per_head.sum())}, geometric {int(geo.per_head.sum())}")


def test_dual_requires_sigma():
    wl = W.make_workload("seq_32k", seq_lens=[640], h_q=4, h_kv=2, needles=0)
    dev = Dev(wl)
    with pytest.raises(eta.EtaError):
        dev.decode(bound="dual", bias=np.zeros(wl.h_q))
