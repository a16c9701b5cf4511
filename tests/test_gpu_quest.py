"""The comparator screen of Section 4.3 (Quest's coordinate-wise box bound) on
the HIP path vs the fp64 oracle, through the C ABI.

The key box (per coordinate the least key value rounded down and the greatest
rounded up to float16) is exact on both sides, so its bits must match; the
box bound decides the admitted sets, with thresholds placed 1e-3 away from
every bound, so the sets compare bit-exactly and outputs to the usual bar."""
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


def _oracle_bits(x):
    with np.errstate(over="ignore", invalid="ignore"):
        return x.astype(np.float16).view(np.uint16)


def _check_boxes(wl, dev):
    lo, hi = E.build_boxes(wl.k_pages, wl.kv_dtype, wl.block_table, wl.seq_lens)
    # pages that hold a complete block
    used = np.zeros(lo.shape[:2], dtype=bool)
    for n in range(wl.n_seqs):
        nfull = int(wl.seq_lens[n]) // 64
        used[wl.block_table[n, :nfull]] = True
    glo, ghi = dev.box_bits()
    assert np.array_equal(glo[used], _oracle_bits(lo[used]))
    assert np.array_equal(ghi[used], _oracle_bits(hi[used]))


@pytest.mark.parametrize("name,kw", [
    ("seq_32k", dict(seq_lens=[4096 + 17, 64 * 40], n_seqs=2)),
    ("seq_32k", dict(seq_lens=[3000, 2000], d=64, kv_dtype="f32")),
    ("ragged_16", dict(n_seqs=3, seq_lens=[300, 4097, 640], h_q=8, h_kv=2, d=128)),
])
def test_box_records(name, kw):
    log(f"[box] {name} {kw}")
    wl = W.make_workload(name, **kw)
    dev = Dev(wl, with_box=True)
    dev.build()
    torch.cuda.synchronize()
    _check_boxes(wl, dev)
    # the other records are unchanged by building the box
    dev2 = Dev(wl)
    dev2.build()
    torch.cuda.synchronize()
    assert np.array_equal(dev.mu_bits(), dev2.mu_bits())
    assert np.array_equal(dev.radius(), dev2.radius())


def test_box_rounding_edges():
    """Columns whose extrema sit between float16 values, at the range's ends,
    below the subnormals, exactly on float16 values, plus non-finite blocks:
    bits identical on both sides."""
    d = 64
    cases = [(1.0001, -1.0001), (70000.0, -70000.0), (2.0 ** -30, -2.0 ** -30), (0.5, -3.25),
             (65504.0, 65519.0), (1e-7, 3e-8)]
    n_pages = len(cases) + 2
    wl = W.make_workload("tiny_4k_f32", seq_len=64 * n_pages, needles=0)
    rng = np.random.default_rng(3)
    for i, (a, b) in enumerate(cases):
        blk = rng.uniform(min(a, b), max(a, b), size=(64, d))
        blk[0] = a
        blk[1] = b
        wl.k_pages[i, 0] = blk.astype(np.float32)
    wl.k_pages[len(cases), 0, 3, 7] = np.inf
    wl.k_pages[len(cases) + 1, 0, 9, 1] = np.nan
    dev = Dev(wl, with_box=True)
    dev.build()
    torch.cuda.synchronize()
    _check_boxes(wl, dev)


def test_append_and_prefill_build_box():
    """Boxes built token by token through eta_append_kv, and by the prompt
    pass, equal the bulk build."""
    wl = W.make_workload("seq_32k", seq_lens=[64 * 3 + 10], h_q=4, h_kv=2, d=128, needles=0)
    dev = Dev(wl, with_box=True)
    dev.build()
    torch.cuda.synchronize()
    cache2 = eta.Cache.empty(wl.num_pages, wl.h_kv, wl.d, dtype=dev.cache.k_pages.dtype, with_box=True)
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
        assert torch.equal(cache2.kmin[page], dev.cache.kmin[page])
        assert torch.equal(cache2.kmax[page], dev.cache.kmax[page])
    dev3 = Dev(wl, with_box=True)
    q_all = W.trace_queries(wl, seed=3)
    eta.prefill(dev3.cache, dev3.seq_lens, dev3.bt, eta.upload(q_all, wl.kv_dtype, "cuda"), eta.ETA_TAU_LEARNED,
                torch.ones(wl.h_q, dtype=torch.float32, device="cuda"), w=dev3.w)
    torch.cuda.synchronize()
    assert np.array_equal(dev3.box_bits()[0], dev.box_bits()[0])
    assert np.array_equal(dev3.box_bits()[1], dev.box_bits()[1])


@pytest.mark.parametrize("kw", [
    dict(seq_lens=[64 * 70 + 3, 64 * 64, 129], h_q=8, h_kv=2, d=128),
    dict(seq_lens=[5000, 7000], h_q=4, h_kv=4, d=64, kv_dtype="f32", mode="calibrated"),
    dict(seq_lens=[3000, 64 * 20 + 1], h_q=4, h_kv=2, d=64),                        # two heads per group
    dict(seq_lens=[64 * 130 + 63, 64 * 5], h_q=16, h_kv=2, d=128, lwb=2, a=0.4),
    dict(n_seqs=4, h_q=8, h_kv=2, d=128, paged=True, density=[0.05, 0.3, 0.6, 0.9] * 2,
         seq_lens=[9000, 300, 64 * 12, 4097]),
])
def test_quest_decode_parity(kw):
    log(f"[quest] {kw}")
    wl, summ = prepared("seq_32k", bound="quest", **kw)
    dev = Dev(wl, with_box=True)
    dev.build()
    o = dev.decode(bound="quest")
    st = dev.stats()
    res = oracle_decode(wl, summaries=summ, bound="quest")
    check_sets_and_counts(wl, res, st)
    check_output(wl, res, o)
    log(f"  per-head blocks {int(res.per_head.sum())}, union {int(res.union.sum())}")


def test_quest_requires_box():
    wl = W.make_workload("seq_32k", seq_lens=[640], h_q=4, h_kv=2, needles=0)
    dev = Dev(wl)
    with pytest.raises(eta.EtaError):
        dev.decode(bound="quest", bias=np.zeros(wl.h_q))
