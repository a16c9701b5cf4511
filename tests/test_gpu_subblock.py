"""Screens on 16- and 32-token blocks (the block-size ablation of Appendix
F.3) on the HIP path vs the fp64 oracle, through the C ABI.

Each smaller block has its own record (float16 centroid, float32 radius,
same rule as the page records): centroid bits must match, radii must bound
the oracle's from above within 1e-6. Thresholds are placed 1e-3 away from
every block's bound, so the admitted sets (in the smaller blocks) compare
bit-exactly, and so do the per-head counts, the union counts, the token
counts and the rescue flags; outputs at the usual bar."""
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


def _check_records(wl, dev, block):
    mu, R = E.build_summaries_sub(wl.k_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, block)
    used = ~np.isnan(R)
    mbits, rad = dev.sub_records()
    with np.errstate(over="ignore", invalid="ignore"):
        assert np.array_equal(mbits[used], mu[used].astype(np.float16).view(np.uint16))
    ref, got = R[used], rad[used].astype(np.float64)
    inf = np.isinf(ref)
    assert np.array_equal(inf, np.isinf(got))
    assert np.all(got[~inf] >= ref[~inf])
    assert np.all(got[~inf] <= ref[~inf] * (1 + 1e-6))


@pytest.mark.parametrize("block", [16, 32])
@pytest.mark.parametrize("name,kw", [
    ("seq_32k", dict(seq_lens=[4096 + 17, 64 * 40 + 40], n_seqs=2)),
    ("seq_32k", dict(seq_lens=[3000, 2000], d=64, kv_dtype="f32")),
    ("ragged_16", dict(n_seqs=3, seq_lens=[300, 4097, 640], h_q=8, h_kv=2, d=128)),
])
def test_subblock_records(name, kw, block):
    log(f"[sub records] b={block} {name} {kw}")
    wl = W.make_workload(name, **kw)
    dev = Dev(wl, sub_block=block)
    dev.build()
    torch.cuda.synchronize()
    _check_records(wl, dev, block)
    dev2 = Dev(wl)
    dev2.build()
    torch.cuda.synchronize()
    assert np.array_equal(dev.mu_bits(), dev2.mu_bits())
    assert np.array_equal(dev.radius(), dev2.radius())


@pytest.mark.parametrize("block", [16, 32])
def test_append_and_prefill_build_subblock_records(block):
    """Records built token by token through eta_append_kv, and by the prompt
    pass, equal the bulk build."""
    wl = W.make_workload("seq_32k", seq_lens=[64 * 3 + 40], h_q=4, h_kv=2, d=128, needles=0)
    dev = Dev(wl, sub_block=block)
    dev.build()
    torch.cuda.synchronize()
    cache2 = eta.Cache.empty(wl.num_pages, wl.h_kv, wl.d, dtype=dev.cache.k_pages.dtype, sub_block=block)
    T = int(wl.seq_lens[0])
    for t in range(T):
        lens = torch.tensor([t], dtype=torch.int32, device="cuda")
        page = int(wl.block_table[0, t // 64])
        kn = dev.cache.k_pages[page, :, t % 64][None].contiguous()
        vn = dev.cache.v_pages[page, :, t % 64][None].contiguous()
        eta.append_kv(cache2, lens, dev.bt, kn, vn)
    torch.cuda.synchronize()
    sb = 64 // block
    for j in range(T // block):
        page = int(wl.block_table[0, j // sb])
        assert torch.equal(cache2.mu_sub[page, :, j % sb], dev.cache.mu_sub[page, :, j % sb])
        assert torch.equal(cache2.radius_sub[page, :, j % sb], dev.cache.radius_sub[page, :, j % sb])
    dev3 = Dev(wl, sub_block=block)
    q_all = W.trace_queries(wl, seed=3)
    eta.prefill(dev3.cache, dev3.seq_lens, dev3.bt, eta.upload(q_all, wl.kv_dtype, "cuda"), eta.ETA_TAU_LEARNED,
                torch.ones(wl.h_q, dtype=torch.float32, device="cuda"), w=dev3.w)
    torch.cuda.synchronize()
    m1, r1 = dev.sub_records()
    m3, r3 = dev3.sub_records()
    used = np.zeros(r1.shape, dtype=bool)
    for j in range(T // block):
        used[int(wl.block_table[0, j // sb]), :, j % sb] = True
    assert np.array_equal(m3[used], m1[used]) and np.array_equal(r3[used], r1[used])


@pytest.mark.parametrize("block,kw", [
    (16, dict(seq_lens=[64 * 70 + 3, 64 * 64, 129], h_q=8, h_kv=2, d=128)),
    (32, dict(seq_lens=[5000, 7000], h_q=4, h_kv=4, d=64, kv_dtype="f32", mode="calibrated")),
    (16, dict(seq_lens=[64 * 130 + 63, 64 * 5 + 20], h_q=16, h_kv=2, d=128, lwb=2, a=0.4)),
    (32, dict(n_seqs=4, h_q=8, h_kv=2, d=128, paged=True, density=[0.05, 0.3, 0.6, 0.9] * 2,
              seq_lens=[9000, 300, 64 * 12, 4097])),
    (16, dict(seq_lens=[64 * 40 + 17], h_q=32, h_kv=4, d=128, density=0.02)),
])
def test_subblock_decode_parity(block, kw):
    log(f"[sub decode] b={block} {kw}")
    wl, summ = prepared("seq_32k", bound="geometric_sub", block=block, **kw)
    dev = Dev(wl, sub_block=block)
    dev.build()
    o = dev.decode(bound="geometric_sub")
    st = dev.stats()
    res = oracle_decode(wl, summaries=summ, bound="geometric_sub", block=block)
    check_sets_and_counts(wl, res, st)
    check_output(wl, res, o)
    log(f"  per-head blocks {int(res.per_head.sum())}, union {int(res.union.sum())}, "
        f"rescued {int(res.rescued.sum())}")


def test_subblock_requires_records():
    wl = W.make_workload("seq_32k", seq_lens=[640], h_q=4, h_kv=2, needles=0)
    dev = Dev(wl)
    with pytest.raises(eta.EtaError):
        dev.decode(bound="geometric_sub")


def test_page_screen_after_subblock_decode():
    """A page-granular decode on the same workspace after a smaller-block one
    reads its own counts (the stats follow the last decode's block size)."""
    wl, summ = prepared("seq_32k", seq_lens=[64 * 30 + 5, 64 * 9], h_q=8, h_kv=2, d=128)
    dev = Dev(wl, sub_block=16)
    dev.build()
    dev.decode(bound="geometric_sub")
    o = dev.decode()
    st = dev.stats()
    res = oracle_decode(wl, summaries=summ)
    check_sets_and_counts(wl, res, st)
    check_output(wl, res, o)
