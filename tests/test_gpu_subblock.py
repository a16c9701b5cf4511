"""Screens on 16-, 32- and 128-token blocks (the block-size ablation of
Appendix F.3) on the HIP path vs the fp64 oracle, through the C ABI.

Each such block has its own record (float16 centroid, float32 radius, same
rule as the page records; a 128-token block spans two block-table entries
and its record sits with the first page): centroid bits must match, radii
must bound the oracle's from above within 1e-6. Thresholds are placed 1e-3
away from every block's bound, so the admitted sets (in the screen's blocks)
compare bit-exactly, and so do the per-head counts, the union counts, the
token counts and the rescue flags; outputs at the usual bar."""
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


@pytest.mark.parametrize("block", [16, 32, 128])
@pytest.mark.parametrize("name,kw", [
    ("seq_32k", dict(seq_lens=[4096 + 17, 64 * 40 + 40], n_seqs=2)),
    ("seq_32k", dict(seq_lens=[3000, 2000], d=64, kv_dtype="f32")),
    ("seq_32k", dict(seq_lens=[2000, 700], d=128, kv_dtype="f32")),
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


def _record_slots(wl, block):
    """(page, slot) of every complete block's record, per sequence 0."""
    T = int(wl.seq_lens[0])
    first = np.arange(T // block) * block
    return [(int(wl.block_table[0, f // 64]), (f % 64) // block) for f in first]


@pytest.mark.parametrize("block", [16, 32, 128])
def test_append_and_prefill_build_subblock_records(block):
    """Records built token by token through eta_append_kv, and by the prompt
    pass, equal the bulk build."""
    wl = W.make_workload("seq_32k", seq_lens=[64 * 5 + 40], h_q=4, h_kv=2, d=128, needles=0, paged=True)
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
    slots = _record_slots(wl, block)
    assert len(slots) >= 2
    for page, q in slots:
        assert torch.equal(cache2.mu_sub[page, :, q], dev.cache.mu_sub[page, :, q])
        assert torch.equal(cache2.radius_sub[page, :, q], dev.cache.radius_sub[page, :, q])
    m1, r1 = dev.sub_records()
    used = np.zeros(r1.shape, dtype=bool)
    for page, q in slots:
        used[page, :, q] = True
    # the prompt pass at three group sizes (positions per workgroup 128, 32, 256)
    for h_q, h_kv in ((4, 2), (8, 1), (2, 2)):
        wl3 = W.make_workload("seq_32k", seq_lens=[64 * 5 + 40], h_q=h_q, h_kv=h_kv, d=128, needles=0, paged=True)
        ref = Dev(wl3, sub_block=block)
        ref.build()
        dev3 = Dev(wl3, sub_block=block)
        q_all = W.trace_queries(wl3, seed=3)
        eta.prefill(dev3.cache, dev3.seq_lens, dev3.bt, eta.upload(q_all, wl3.kv_dtype, "cuda"),
                    eta.ETA_TAU_LEARNED, torch.ones(wl3.h_q, dtype=torch.float32, device="cuda"), w=dev3.w)
        torch.cuda.synchronize()
        ma, ra = ref.sub_records()
        m3, r3 = dev3.sub_records()
        used3 = np.zeros(ra.shape, dtype=bool)
        for page, q in _record_slots(wl3, block):
            used3[page, :, q] = True
        assert np.array_equal(m3[used3], ma[used3]) and np.array_equal(r3[used3], ra[used3]), (h_q, h_kv)


@pytest.mark.parametrize("block,kw", [
    (16, dict(seq_lens=[64 * 70 + 3, 64 * 64, 129], h_q=8, h_kv=2, d=128)),
    (32, dict(seq_lens=[5000, 7000], h_q=4, h_kv=4, d=64, kv_dtype="f32", mode="calibrated")),
    (16, dict(seq_lens=[64 * 130 + 63, 64 * 5 + 20], h_q=16, h_kv=2, d=128, lwb=2, a=0.4)),
    (32, dict(n_seqs=4, h_q=8, h_kv=2, d=128, paged=True, density=[0.05, 0.3, 0.6, 0.9] * 2,
              seq_lens=[9000, 300, 64 * 12, 4097])),
    (16, dict(seq_lens=[64 * 40 + 17], h_q=32, h_kv=4, d=128, density=0.02)),
    (128, dict(seq_lens=[64 * 70 + 3, 64 * 64, 129], h_q=8, h_kv=2, d=128, paged=True)),
    (128, dict(seq_lens=[5000, 7000], h_q=4, h_kv=4, d=64, kv_dtype="f32", mode="calibrated")),
    (128, dict(seq_lens=[64 * 131 + 63, 64 * 5 + 20], h_q=16, h_kv=2, d=128, lwb=2, a=0.4)),
    (128, dict(n_seqs=4, h_q=8, h_kv=2, d=128, paged=True, density=[0.05, 0.3, 0.6, 0.9] * 2,
               seq_lens=[9000, 300, 64 * 12, 4097])),
    (128, dict(seq_lens=[64 * 40 + 17, 64], h_q=32, h_kv=4, d=128, density=0.02)),
    (32, dict(seq_lens=[3000, 1000], h_q=4, h_kv=2, d=128)),                      # two heads per group
    (128, dict(seq_lens=[3000, 1000 + 64], h_q=4, h_kv=2, d=64, paged=True)),
    (16, dict(seq_lens=[2000, 513], h_q=2, h_kv=1, d=64, kv_dtype="f32", lwb=3)),
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
        dev.decode(bound="geometric_sub", bias=np.zeros(wl.h_q))


def test_pairblock_rescue():
    """A head whose threshold lies above every 128-token block's bound gets the
    block with the largest bound, both of its pages."""
    wl, summ = prepared("seq_32k", bound="geometric_sub", block=128, seq_lens=[64 * 36, 64 * 10], h_q=8, h_kv=2,
                        d=128, paged=True)
    wl.bias = wl.bias.copy()
    wl.bias[[0, 5]] = np.float32(1e3)
    dev = Dev(wl, sub_block=128)
    dev.build()
    o = dev.decode(bound="geometric_sub")
    st = dev.stats()
    res = oracle_decode(wl, summaries=summ, bound="geometric_sub", block=128)
    assert res.rescued[:, 0].all() and res.rescued[:, 5].all()
    check_sets_and_counts(wl, res, st)
    check_output(wl, res, o)


@pytest.mark.parametrize("block", [16, 128])
def test_page_screen_after_subblock_decode(block):
    """A page-granular decode on the same workspace after one on other screen
    blocks reads its own counts (the stats follow the last decode's block size)."""
    wl, summ = prepared("seq_32k", seq_lens=[64 * 30 + 5, 64 * 9], h_q=8, h_kv=2, d=128)
    dev = Dev(wl, sub_block=block)
    dev.build()
    dev.decode(bound="geometric_sub")
    o = dev.decode()
    st = dev.stats()
    res = oracle_decode(wl, summaries=summ)
    check_sets_and_counts(wl, res, st)
    check_output(wl, res, o)


def test_invalid_second_page_of_a_128_token_block_is_never_rescued():
    """A 128-token block whose second page id is out of range is not a
    complete block: the screen neither admits nor ranks it, so the top-1
    rescue picks the best block among the valid ones, nothing reads the bad
    page, and eta_stats reports ETA_ERR_DEVICE_DATA. Lengths are multiples of
    128 and lwb = 0, so no block is forced, and every threshold lies above
    every bound, so every head is rescued."""
    block = 128
    wl, summ = prepared("seq_32k", bound="geometric_sub", block=block, seq_lens=[64 * 16, 64 * 10], h_q=8, h_kv=2,
                        d=128, paged=True)
    wl.bias = np.full(wl.h_q, 1e3, dtype=np.float32)
    res = oracle_decode(wl, summaries=summ, bound="geometric_sub", block=block)
    assert res.rescued.all()
    nb0 = int(wl.seq_lens[0]) // block
    jb = int(np.argmax(res.ub[0, 0, :nb0]))  # the block head 0 of sequence 0 would get
    dev = Dev(wl, sub_block=block)
    dev.build()
    bt_bad = dev.bt.clone()
    bt_bad[0, 2 * jb + 1] = wl.num_pages + 100
    dev.decode(bound="geometric_sub")
    eta.decode(dev.cache, dev.seq_lens, bt_bad, dev.q, eta.ETA_TAU_LEARNED, torch.from_numpy(wl.bias).cuda(),
               w=dev.w, out=dev.out, workspace=dev.ws, bound="geometric_sub")
    torch.cuda.synchronize()
    st = dev.stats(check=False)
    assert st.status == eta.ETA_ERR_DEVICE_DATA
    out = dev.out.cpu().numpy().astype(np.float64)
    check_output(wl, res, out, heads=[(1, h) for h in range(wl.h_q)])
    adm = st.admitted(res.admitted.shape[2])
    qf = E.upcast(wl.q, wl.kv_dtype)
    scale = 1.0 / np.sqrt(wl.d)
    for h in range(wl.h_q):
        ub = res.ub[0, h, :nb0].copy()
        ub[jb] = -np.inf
        best = int(np.argmax(ub))
        gap = ub[best] - np.max(np.delete(ub, best))
        assert gap > 1e-4, gap
        want = np.zeros(adm.shape[2], dtype=bool)
        want[best] = True
        assert np.array_equal(adm[0, h], want), (h, np.flatnonzero(adm[0, h]), best)
        g = h // wl.group
        pages = [int(wl.block_table[0, 2 * best]), int(wl.block_table[0, 2 * best + 1])]
        K = np.concatenate([E.upcast(wl.k_pages[p, g], wl.kv_dtype) for p in pages])
        V = np.concatenate([E.upcast(wl.v_pages[p, g], wl.kv_dtype) for p in pages])
        ref = E.filtered_attention(qf[0, h], K, V, res.tau[0, h], wl.beta, scale)
        assert float(np.max(np.abs(out[0, h] - ref))) <= 2e-3
