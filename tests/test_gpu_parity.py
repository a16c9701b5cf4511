"""HIP path vs the fp64 oracle, through the C ABI (needs an MI355X).

Bars: admitted-block bitmaps and counts bit-exact (thresholds are placed with a
1e-3 margin from every bound); outputs within max abs error 1e-5 (float32 K/V)
or 2e-3 (bfloat16 K/V)."""
import os

import numpy as np
import pytest
import torch

import workloads as W
from gpu_util import (Dev, check_output, check_sets_and_counts, fp64_radius_about, log, oracle_decode,
                      prepared)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import learned_threshold_block_amd._lib as L
    L.lib()


def run_case(name, **kw):
    log(f"[case] {name} {kw}")
    wl, summ = prepared(name, **kw)
    dev = Dev(wl)
    dev.build()
    o = dev.decode()
    st = dev.stats()
    res = oracle_decode(wl, summaries=summ)
    check_sets_and_counts(wl, res, st)
    check_output(wl, res, o)
    return wl, dev, res, o


# ----------------------------------------------------------------------------- records
@pytest.mark.parametrize("name,kw", [
    ("tiny_4k_f32", {}),
    ("seq_32k", dict(seq_lens=[4096 + 17, 64 * 40], n_seqs=2)),
    ("seq_32k", dict(seq_lens=[1000, 3000], d=64)),
    ("tiny_4k_f32", dict(d=128, seq_lens=[2048 + 5, 640], h_q=4, h_kv=2)),
])
def test_records_match_oracle_and_are_sound(name, kw):
    log(f"[records] {name} {kw}")
    wl = W.make_workload(name, **kw)
    dev = Dev(wl)
    dev.build()
    torch.cuda.synchronize()
    mu_o, R_o = E_summaries(wl)
    bits = dev.mu_bits()
    R_g = dev.radius()
    used = ~np.isnan(R_o)
    mu_ref = mu_o.astype(np.float16).view(np.uint16)
    assert np.array_equal(bits[used], mu_ref[used]), "centroids differ from the oracle's float16 rounding"
    # sound: stored radius covers every key about the stored centroid, and is tight
    R_true = fp64_radius_about(wl, bits)
    assert np.all(R_g[used].astype(np.float64) >= R_true[used])
    assert np.all(R_g[used].astype(np.float64) <= R_true[used] * (1 + 1e-6) + 1e-30)
    assert np.allclose(R_g[used], R_o[used], rtol=1e-6)


def E_summaries(wl):
    import oracle.eta_oracle as E
    return E.build_summaries(wl.k_pages, wl.kv_dtype, wl.block_table, wl.seq_lens)


def test_record_rounding_edges():
    """Centroid rounding ties, float16 subnormals and overflow (zero-centroid
    fallback) and non-finite keys, compared with NumPy's float16 conversion."""
    rng = np.random.default_rng(5)
    d = 64
    vals = [1 + 2 ** -11, 1 + 3 * 2 ** -11, -(2 + 2 ** -10), 2 ** -25, 3 * 2 ** -26, 2 ** -24 * 1.5,
            65504.0, 65519.0, 65520.0, 1e-8, 0.0, -0.0, 1000.3, 6.1e-5]
    n_pages = len(vals) + 4
    wl = W.make_workload("tiny_4k_f32", seq_len=64 * n_pages, needles=0)
    for i, v in enumerate(vals):
        wl.k_pages[i, 0] = np.float32(v) + np.zeros((64, d), np.float32)
    # random values exactly representable, mean on a rounding boundary in random coordinates
    base = rng.integers(-2000, 2000, size=d).astype(np.float32) / 1024.0
    wl.k_pages[len(vals), 0] = base + (2 ** -11) * (rng.integers(0, 2, size=(64, d)).astype(np.float32))
    wl.k_pages[len(vals) + 1, 0, 3, 7] = np.inf
    wl.k_pages[len(vals) + 2, 0, 9, 1] = np.nan
    wl.k_pages[len(vals) + 3, 0] = 1e30
    dev = Dev(wl)
    dev.build()
    torch.cuda.synchronize()
    mu_o, R_o = E_summaries(wl)
    bits = dev.mu_bits()[:, 0]
    ref = mu_o[:, 0].astype(np.float16).view(np.uint16)
    for p in range(n_pages):
        assert np.array_equal(bits[p], ref[p]), (p, bits[p][:4], ref[p][:4])
    R_g = dev.radius()[:, 0]
    assert np.isinf(R_g[len(vals) + 1]) and np.isinf(R_g[len(vals) + 2])
    finite = np.isfinite(R_o[:, 0])
    assert np.all(R_g[finite] >= R_o[finite, 0]) and np.allclose(R_g[finite], R_o[finite, 0], rtol=1e-6)


def test_append_equals_bulk_build():
    """Appending tokens one at a time (records built when a block fills) gives
    the same bytes as building all records at once."""
    import learned_threshold_block_amd as eta
    wl = W.make_workload("seq_32k", seq_lens=[64 * 3 + 10, 64 * 2], h_q=8, h_kv=2, d=128, needles=0)
    dev = Dev(wl)
    dev.build()
    torch.cuda.synchronize()
    mu_bulk, r_bulk = dev.mu_bits().copy(), dev.radius().copy()
    # fresh cache, filled token by token through eta_append_kv
    cache2 = eta.Cache.empty(wl.num_pages, wl.h_kv, wl.d, dtype=dev.cache.k_pages.dtype)
    T_max = int(wl.seq_lens.max())
    for t in range(T_max):
        active = [n for n in range(wl.n_seqs) if t < int(wl.seq_lens[n])]
        if not active:
            break
        lens = torch.tensor([min(t, int(wl.seq_lens[n])) for n in range(wl.n_seqs)], dtype=torch.int32,
                            device="cuda")
        kn = torch.empty(wl.n_seqs, wl.h_kv, wl.d, dtype=dev.cache.k_pages.dtype, device="cuda")
        vn = torch.empty_like(kn)
        for n in range(wl.n_seqs):
            tt = min(t, int(wl.seq_lens[n]) - 1)
            page = int(wl.block_table[n, tt // 64])
            kn[n] = dev.cache.k_pages[page, :, tt % 64]
            vn[n] = dev.cache.v_pages[page, :, tt % 64]
        # sequences that are already complete append into a scratch slot past their length
        for n in range(wl.n_seqs):
            if t >= int(wl.seq_lens[n]):
                lens[n] = 64 * wl.max_blocks  # out of range: skipped by the kernel
        eta.append_kv(cache2, lens, dev.bt, kn, vn)
    torch.cuda.synchronize()
    for n in range(wl.n_seqs):
        T = int(wl.seq_lens[n])
        for j in range(-(-T // 64)):
            page = int(wl.block_table[n, j])
            rows = min(64, T - 64 * j)
            assert torch.equal(cache2.k_pages[page, :, :rows], dev.cache.k_pages[page, :, :rows])
            assert torch.equal(cache2.v_pages[page, :, :rows], dev.cache.v_pages[page, :, :rows])
    mu2 = cache2.mu.cpu().view(torch.int16).numpy().view(np.uint16)
    r2 = cache2.radius.cpu().numpy()
    for n in range(wl.n_seqs):
        for j in range(int(wl.seq_lens[n]) // 64):
            page = int(wl.block_table[n, j])
            assert np.array_equal(mu2[page], mu_bulk[page])
            assert np.array_equal(r2[page], r_bulk[page])


# ----------------------------------------------------------------------------- decode
def test_tiny_4k_f32_parity():
    run_case("tiny_4k_f32")


def test_seq_32k_parity():
    run_case("seq_32k")


@pytest.mark.parametrize("kw", [
    dict(seq_lens=[64 * 70 + 3, 64 * 64, 129, 1], h_q=8, h_kv=2, d=128),              # ragged, tails, T=1
    dict(seq_lens=[64 * 130 + 63, 64 * 5], h_q=16, h_kv=2, d=128, lwb=2, a=0.4),      # G=8, lwb, a
    dict(seq_lens=[5000, 7000], h_q=4, h_kv=4, d=64),                                  # G=1, d=64 bf16
    dict(seq_lens=[3000, 64 * 50], h_q=8, h_kv=4, d=64, kv_dtype="f32", beta=1.0),    # f32 d=64 G=2
    dict(seq_lens=[2500, 64 * 33], h_q=8, h_kv=2, d=128, kv_dtype="f32", mode="calibrated"),  # f32 d=128
    dict(seq_lens=[64 * 300], h_q=8, h_kv=2, d=128, mode="calibrated", density=0.1),  # sparse
    dict(seq_lens=[64 * 300 + 1], h_q=8, h_kv=2, d=128, density=0.9),                 # dense-ish
    dict(n_seqs=5, h_q=8, h_kv=2, d=128, paged=True, density=[0.05, 0.3, 0.6, 0.9] * 2,
         seq_lens=[9000, 300, 64 * 12, 4097, 20000]),                                 # paged, spread
])
def test_decode_variants(kw):
    run_case("seq_32k", **kw)


def test_dense_mode_is_plain_attention():
    """c = -inf admits every block and leaves logits unfiltered."""
    wl, summ = prepared("seq_32k", seq_lens=[64 * 40 + 9, 2000], h_q=8, h_kv=2, mode="calibrated")
    bias = np.full(wl.h_q, -np.inf, dtype=np.float32)
    dev = Dev(wl)
    dev.build()
    o = dev.decode(bias=bias)
    st = dev.stats()
    res = oracle_decode(wl, summaries=summ, bias=bias)
    check_sets_and_counts(wl, res, st)
    check_output(wl, res, o)
    assert st.admitted(wl.max_blocks).sum() == sum(wl.nblk(n) for n in range(wl.n_seqs)) * wl.h_q


def test_rescue_path():
    """Nothing passes and there is no partial block: each head keeps its
    best-bound block only; o is the mean of that block's values."""
    wl, summ = prepared("seq_32k", seq_lens=[64 * 37, 64 * 8], h_q=8, h_kv=2, mode="calibrated")
    bias = np.full(wl.h_q, 1e4, dtype=np.float32)
    dev = Dev(wl)
    dev.build()
    o = dev.decode(bias=bias)
    st = dev.stats()
    res = oracle_decode(wl, summaries=summ, bias=bias)
    assert res.rescued.all()
    check_sets_and_counts(wl, res, st)
    check_output(wl, res, o)


def _same_up_to_rounding(o1, o2):
    """Work is claimed dynamically and split by measured per-die speed, so the
    float32 summation order may differ between calls: equal to a few float32
    ulps of the output scale."""
    scale = float(np.max(np.abs(o1)))
    assert float(np.max(np.abs(o1 - o2))) <= 1e-6 * scale


def test_page_permutation_invariance(monkeypatch):
    wl, summ = prepared("seq_32k", seq_lens=[64 * 90 + 7, 3333], h_q=8, h_kv=2)
    dev = Dev(wl)
    dev.build()
    o1 = dev.decode()
    wl2 = W.permute_pages(wl, seed=11)
    dev2 = Dev(wl2)
    dev2.build()
    o2 = dev2.decode()
    _same_up_to_rounding(o1, o2)
    # with the static assignment the physical page order is invisible bit for bit
    monkeypatch.setenv("ETA_DETERMINISTIC", "1")
    assert np.array_equal(dev.decode(), dev2.decode())


def test_split_count_invariance(monkeypatch):
    wl, summ = prepared("seq_32k", seq_lens=[64 * 200 + 30, 64 * 77], h_q=8, h_kv=2)
    res = oracle_decode(wl, summaries=summ)
    dev = Dev(wl)
    dev.build()
    for wgs in ("1", "2", "7", "64", "4096"):
        monkeypatch.setenv("ETA_ATTEND_WGS", wgs)
        o = dev.decode()
        log(f"  attend workgroups {wgs}")
        check_output(wl, res, o)
    monkeypatch.delenv("ETA_ATTEND_WGS")


@pytest.mark.parametrize("weights", ["512,2048,512,2048,512,2048,512,2048", "2048,512,1024,1024,700,1900,512,2048"])
def test_weighted_split(monkeypatch, weights):
    """Uneven per-die weights of the attend split (the measured ones are
    replaced through ETA_RANGE_WEIGHTS), including grids with more ranges than
    some weights can fill (empty ranges), keep the results."""
    wl, summ = prepared("seq_32k", seq_lens=[64 * 120 + 30, 64 * 33, 500], h_q=8, h_kv=2)
    res = oracle_decode(wl, summaries=summ)
    dev = Dev(wl)
    dev.build()
    monkeypatch.setenv("ETA_RANGE_WEIGHTS", weights)
    for wgs in ("3", "256", "4096"):
        monkeypatch.setenv("ETA_ATTEND_WGS", wgs)
        o = dev.decode()
        log(f"  weights {weights}, attend workgroups {wgs}")
        check_output(wl, res, o)
        check_sets_and_counts(wl, res, dev.stats())


def test_repeatable(monkeypatch):
    """Default mode: repeated calls agree to float32 rounding; ETA_DETERMINISTIC=1:
    bitwise, and within rounding of the default mode."""
    wl, summ = prepared("seq_32k", seq_lens=[64 * 150 + 1, 64 * 40], h_q=8, h_kv=2)
    res = oracle_decode(wl, summaries=summ)
    dev = Dev(wl)
    dev.build()
    o1 = dev.decode()
    o2 = dev.decode()
    _same_up_to_rounding(o1, o2)
    monkeypatch.setenv("ETA_DETERMINISTIC", "1")
    d1 = dev.decode()
    d2 = dev.decode()
    assert np.array_equal(d1, d2)
    _same_up_to_rounding(o1, d1)
    check_output(wl, res, d1)


def test_many_segments_attend_without_lds_tables():
    """400 (sequence, KV head) segments with a 2048-page block table: the
    segments' tile prefixes (400 x 36 ints) do not fit the attend kernel's LDS
    tables, so it locates each segment's entries with per-segment loads (its
    other variant). One long sequence and 99 short ones, paged."""
    lens = [64 * 2048 - 5] + [300 + 37 * i for i in range(99)]
    wl, summ = prepared("seq_32k", seq_lens=lens, h_q=8, h_kv=4, d=64, needles=0, paged=True)
    S = wl.n_seqs * wl.h_kv
    NT = -(-wl.max_blocks // 64)
    assert S * (NT + 4) > 12288
    dev = Dev(wl)
    dev.build()
    o = dev.decode()
    st = dev.stats()
    res = oracle_decode(wl, summaries=summ)
    check_sets_and_counts(wl, res, st)
    check_output(wl, res, o)


def test_junk_tail_rows_do_not_leak(monkeypatch):
    """Rows past the end hold NaN (the generator's fill); results stay finite and
    equal, bit for bit under the static work split, those with zeroed junk."""
    monkeypatch.setenv("ETA_DETERMINISTIC", "1")
    wl, summ = prepared("seq_32k", seq_lens=[64 * 20 + 3, 64 * 9 + 60], h_q=8, h_kv=2)
    dev = Dev(wl)
    dev.build()
    o_nan = dev.decode()
    assert np.all(np.isfinite(o_nan))
    for n in range(wl.n_seqs):
        T = int(wl.seq_lens[n])
        page = int(wl.block_table[n, T // 64])
        dev.cache.k_pages[page, :, T % 64:] = 0
        dev.cache.v_pages[page, :, T % 64:] = 0
    o0 = dev.decode()
    assert np.array_equal(o_nan, o0)


def test_invalid_device_data_is_reported():
    """An out-of-range page id and an out-of-range length are caught on the
    device: no fault, ETA_ERR_DEVICE_DATA from eta_stats, other sequences fine."""
    import learned_threshold_block_amd as eta
    wl, summ = prepared("seq_32k", seq_lens=[64 * 10 + 5, 64 * 6, 64 * 3], h_q=8, h_kv=2)
    dev = Dev(wl)
    dev.build()
    bt_bad = dev.bt.clone()
    bt_bad[0, 3] = wl.num_pages + 100
    lens_bad = dev.seq_lens.clone()
    lens_bad[1] = 64 * wl.max_blocks + 1
    b = torch.from_numpy(wl.bias).cuda()
    eta.decode(dev.cache, lens_bad, bt_bad, dev.q, eta.ETA_TAU_LEARNED, b, w=dev.w, out=dev.out,
               workspace=dev.ws)
    torch.cuda.synchronize()
    st = dev.stats(check=False)
    assert st.status == eta.ETA_ERR_DEVICE_DATA
    res = oracle_decode(wl, summaries=summ)
    o = dev.out.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(o[2], res.o[2], atol=2e-3, rtol=0)
    # a clean call afterwards reports OK again
    dev.decode()
    assert dev.stats().status == eta.ETA_OK


@pytest.mark.parametrize("blocks", [512, 513])
def test_screen_launch_forms_at_their_boundary(blocks):
    """Up to 8 tiles (512 blocks) per sequence the screen and the finalize run
    as one launch (one workgroup per segment); from 513 blocks on, as two. The
    same sets, counts and outputs at the bar either way: a ragged partner
    sequence, and KV head 0's group needing the rescue (its bias is so large
    that nothing passes, and no block is forced: both lengths fill their last
    page) next to a group that admits blocks at the placed thresholds."""
    wl, summ = prepared("seq_32k", seq_lens=[64 * blocks, 64 * 3], h_q=8, h_kv=2, d=128, needles=0)
    bias = np.array(wl.bias, dtype=np.float32).copy()
    bias[:4] = 1e4
    log(f"[screen launch form] {blocks} blocks")
    dev = Dev(wl)
    dev.build()
    o = dev.decode(bias=bias)
    st = dev.stats()
    res = oracle_decode(wl, summaries=summ, bias=bias)
    assert np.asarray(res.rescued)[:, :4].all()
    check_sets_and_counts(wl, res, st)
    check_output(wl, res, o)
