"""The append path (eta_append_kv) against the fp64 oracle, through the C ABI.

The decode screen's records are built while the cache grows: one token is
appended per sequence and step, and the record of a block is built when its
last token arrives (the ETA page, Section 3.2: metadata kept in a table beside
the paged cache; Section 4.8: built during generation). Two checks:

* records: a cache filled token by token holds the oracle's records of every
  complete block, compared with the oracle directly (not with the bulk
  builder): float16 centroid bits equal to the rounding of the fp64 mean,
  float32 radius at or above the exact fp64 radius about the stored centroid
  (and within 1e-6 of it), the coordinate deviation, the key box, the FP8
  centroid codes with their radius, and the records of 16-, 32- and
  128-token screen blocks;
* append then decode: from a cache built only by appends, every step appends
  one token to every sequence (crossing slots 62 -> 63 -> the next page, and
  the end of 128-token blocks), checks the records of the cache as it stands
  against the oracle, then runs eta_decode on it and compares the admitted
  sets and counts bit for bit and the outputs at the bar (2e-3 bfloat16,
  1e-5 float32) with the oracle's decode at the same lengths.

Thresholds are placed once, at the final lengths, with a 1e-3 margin from
every complete block's bound; a block is complete at an earlier length only
if it is at the final one, with the same keys and so the same record, so the
margin holds at every step."""
import dataclasses

import numpy as np
import pytest
import torch

import bruteforce
import learned_threshold_block_amd as eta
import oracle.eta_oracle as E
import workloads as W
from gpu_util import check_output, check_sets_and_counts, log, oracle_decode, prepared

pytestmark = pytest.mark.gpu

BLOCK = 64


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import learned_threshold_block_amd._lib as L
    L.lib()


# ----------------------------------------------------------------------------- feeding tokens
class Feeder:
    """Appends tokens of a workload's cache (uploaded once as the source) to a
    fresh cache, one token per sequence and call."""

    def __init__(self, wl, cache):
        self.wl = wl
        self.cache = cache
        self.src_k = eta.upload(wl.k_pages, wl.kv_dtype, "cuda")
        self.src_v = eta.upload(wl.v_pages, wl.kv_dtype, "cuda")
        self.bt = torch.from_numpy(wl.block_table.astype(np.int32)).cuda()
        self.skip = BLOCK * wl.max_blocks  # a length the append path skips

    def append(self, tokens):
        """tokens[n]: index of the token sequence n appends (its length before
        the append), or None to leave it alone."""
        wl = self.wl
        lens = np.array([self.skip if t is None else t for t in tokens], dtype=np.int32)
        pages = np.array([0 if t is None else wl.block_table[n, t // BLOCK] for n, t in enumerate(tokens)],
                         dtype=np.int64)
        rows = np.array([0 if t is None else t % BLOCK for t in tokens], dtype=np.int64)
        assert np.all(pages >= 0) and np.all(pages < wl.num_pages)
        pi, ri = torch.from_numpy(pages).cuda(), torch.from_numpy(rows).cuda()
        kn = self.src_k[pi, :, ri].contiguous()  # [N][H_KV][d]
        vn = self.src_v[pi, :, ri].contiguous()
        assert tuple(kn.shape) == (wl.n_seqs, wl.h_kv, wl.d)
        eta.append_kv(self.cache, torch.from_numpy(lens).cuda(), self.bt, kn, vn)


def fresh_cache(wl, **kw):
    dt = torch.bfloat16 if wl.kv_dtype == "bf16" else torch.float32
    c = eta.Cache.empty(wl.num_pages, wl.h_kv, wl.d, dtype=dt, **kw)
    c.k_pages.fill_(float("nan"))  # rows no append wrote show up in any result that reads them
    c.v_pages.fill_(float("nan"))
    return c


def at_lengths(wl, lens):
    return dataclasses.replace(wl, seq_lens=np.asarray(lens, dtype=np.int32))


# ----------------------------------------------------------------------------- record checks against the oracle
def _bits16(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _f16_bits(x):
    with np.errstate(over="ignore", invalid="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def _complete_pages(wl, lens):
    used = np.zeros((wl.num_pages, wl.h_kv), dtype=bool)
    for n in range(wl.n_seqs):
        used[wl.block_table[n, :int(lens[n]) // BLOCK]] = True
    return used


def _radius_about(wl, pages_keys, centre):
    """max over keys of ||k - centre|| in float64; pages_keys [m][rows][d]."""
    dlt = pages_keys - centre[:, None, :]
    return np.sqrt((dlt * dlt).sum(axis=2)).max(axis=1)


def _check_radius(got, exact):
    got = np.asarray(got, dtype=np.float64)
    assert np.all(got >= exact), "a radius lies below the exact fp64 radius"
    assert np.all(got <= exact * (1 + 1e-6) + 1e-30), "a radius is not tight"


def check_page_records(wl, cache, lens):
    """Centroid bits and radius of every complete page against the oracle."""
    mu_o, R_o = E.build_summaries(wl.k_pages, wl.kv_dtype, wl.block_table, lens)
    used = _complete_pages(wl, lens)
    assert np.array_equal(used, ~np.isnan(R_o))
    bits = _bits16(cache.mu)
    assert np.array_equal(bits[used], _f16_bits(mu_o[used])), "centroids differ from the oracle's rounding"
    keys = E.upcast(wl.k_pages, wl.kv_dtype)[used]  # [m][64][d]
    cen = bits[used].view(np.float16).astype(np.float64)
    _check_radius(cache.radius.cpu().numpy()[used], _radius_about(wl, keys, cen))
    return int(used.sum())


def check_sigma(wl, cache, lens):
    """Coordinate deviation: the oracle's float16 rounding, up to one unit in
    the last place in at most 0.1% of the coordinates (the device's float64
    sum of squares may round differently at a float16 tie's edge)."""
    ref = E.build_sigmas(wl.k_pages, wl.kv_dtype, wl.block_table, lens)
    used = _complete_pages(wl, lens)
    d = np.abs(_bits16(cache.sigma)[used].astype(np.int32) - _f16_bits(ref[used]).astype(np.int32))
    assert d.max() <= 1 and (d > 0).sum() <= max(2, int(1e-3 * d.size)), (int(d.max()), int((d > 0).sum()))


def check_box(wl, cache, lens):
    lo, hi = E.build_boxes(wl.k_pages, wl.kv_dtype, wl.block_table, lens)
    used = _complete_pages(wl, lens)
    assert np.array_equal(_bits16(cache.kmin)[used], _f16_bits(lo[used]))
    assert np.array_equal(_bits16(cache.kmax)[used], _f16_bits(hi[used]))


def _fp8_codes(values, fmt):
    """Oracle FP8 values -> codes through the brute force's table of the format."""
    table = {v: c for c, v in bruteforce.fp8_values(fmt).items() if c < 0x80}
    flat = np.asarray(values, dtype=np.float64).ravel()
    out = np.array([table[abs(float(v))] | (0x80 if np.signbit(v) else 0) for v in flat], dtype=np.uint8)
    return out.reshape(np.shape(values))


def check_fp8(wl, cache, lens, fmt):
    mu8, R8 = E.build_summaries_fp8(wl.k_pages, wl.kv_dtype, wl.block_table, lens, fmt)
    used = _complete_pages(wl, lens)
    assert np.array_equal(cache.mu8.cpu().numpy()[used], _fp8_codes(mu8[used], fmt))
    got = cache.radius8.cpu().numpy()[used].astype(np.float64)
    assert np.all(got >= R8[used]) and np.all(got <= R8[used] * (1 + 2.0 ** -20))


def check_sub_records(wl, cache, lens, block):
    """Records of the cache's screen blocks of `block` tokens (16, 32 or 128)."""
    mu_o, R_o = E.build_summaries_sub(wl.k_pages, wl.kv_dtype, wl.block_table, lens, block)
    used = ~np.isnan(R_o)
    bits = _bits16(cache.mu_sub)
    assert np.array_equal(bits[used], _f16_bits(mu_o[used]))
    got = cache.radius_sub.cpu().numpy()[used].astype(np.float64)
    # exact fp64 radius about the stored centroid, over each block's own keys
    keys_all = E.upcast(wl.k_pages, wl.kv_dtype)
    exact = np.empty_like(got)
    slots = mu_o.shape[2]
    idx = np.argwhere(used)
    for m, (page, g, sl) in enumerate(idx):
        if block < BLOCK:
            keys = keys_all[page, g, sl * block:(sl + 1) * block]
        else:  # the second page follows the first in the table of the sequence that holds it
            n, j = np.argwhere(wl.block_table == page)[0]
            keys = np.concatenate([keys_all[page, g], keys_all[wl.block_table[n, j + 1], g]])
        cen = bits[page, g, sl].view(np.float16).astype(np.float64)
        exact[m] = np.sqrt(((keys - cen) ** 2).sum(axis=1)).max()
    assert slots == max(1, BLOCK // block)
    _check_radius(got, exact)
    return int(used.sum())


# ----------------------------------------------------------------------------- records after appends
RECORD_CASES = [
    # (name, workload overrides, cache extras)
    ("bf16_d128_all_records", dict(seq_lens=[64 * 3 + 10, 64 * 2 + 63, 64 * 4], h_q=8, h_kv=2, d=128, paged=True),
     dict(with_sigma=True, with_box=True, fp8="e4m3")),
    ("f32_d64_all_records", dict(seq_lens=[64 * 2 + 1, 64 * 3 + 62], h_q=4, h_kv=2, d=64, kv_dtype="f32"),
     dict(with_sigma=True, with_box=True, fp8="e5m2")),
    ("bf16_d128_sub16", dict(seq_lens=[64 * 2 + 40, 64 + 15], h_q=4, h_kv=2, d=128, paged=True),
     dict(sub_block=16)),
    ("f32_d128_sub32", dict(seq_lens=[64 * 2 + 33, 64 * 3 - 1], h_q=4, h_kv=2, d=128, kv_dtype="f32"),
     dict(sub_block=32)),
    ("bf16_d64_sub128", dict(seq_lens=[64 * 5 + 3, 64 * 4, 64 * 3 + 63], h_q=4, h_kv=2, d=64, paged=True),
     dict(sub_block=128)),
]


@pytest.mark.parametrize("name,kw,extras", RECORD_CASES, ids=[c[0] for c in RECORD_CASES])
def test_append_records_match_oracle(name, kw, extras):
    """A cache filled only through eta_append_kv holds the oracle's records."""
    log(f"[append records] {name}")
    wl = W.make_workload("seq_32k", needles=0, **kw)
    cache = fresh_cache(wl, **extras)
    feed = Feeder(wl, cache)
    T = [int(t) for t in wl.seq_lens]
    for t in range(max(T)):
        feed.append([t if t < T[n] else None for n in range(wl.n_seqs)])
    torch.cuda.synchronize()
    # the rows of every token, bit for bit, and nothing else written
    for n in range(wl.n_seqs):
        for j in range(-(-T[n] // BLOCK)):
            page = int(wl.block_table[n, j])
            rows = min(BLOCK, T[n] - BLOCK * j)
            src = eta.upload(wl.k_pages[page], wl.kv_dtype, "cuda")
            assert torch.equal(cache.k_pages[page, :, :rows], src[:, :rows])
            srcv = eta.upload(wl.v_pages[page], wl.kv_dtype, "cuda")
            assert torch.equal(cache.v_pages[page, :, :rows], srcv[:, :rows])
            assert bool(torch.isnan(cache.k_pages[page, :, rows:].float()).all())
    npages = check_page_records(wl, cache, wl.seq_lens)
    log(f"  {npages} page records match the oracle")
    if extras.get("with_sigma"):
        check_sigma(wl, cache, wl.seq_lens)
    if extras.get("with_box"):
        check_box(wl, cache, wl.seq_lens)
    if extras.get("fp8"):
        check_fp8(wl, cache, wl.seq_lens, extras["fp8"])
    if extras.get("sub_block"):
        nsub = check_sub_records(wl, cache, wl.seq_lens, extras["sub_block"])
        log(f"  {nsub} records of {extras['sub_block']}-token blocks match the oracle")


# ----------------------------------------------------------------------------- append, then decode, every step
LOOP_CASES = [
    # (name, workload overrides, screen block (64 = pages), steps with a decode)
    ("bf16_d128_g4_lwb2", dict(seq_lens=[64 * 3 + 10, 64 * 4 + 1, 64 * 3 + 63], h_q=8, h_kv=2, d=128, lwb=2,
                               paged=True), 64, 140),
    ("f32_d64_g2_calibrated", dict(seq_lens=[64 * 3 + 30, 64 * 2 + 60], h_q=4, h_kv=2, d=64, kv_dtype="f32",
                                   mode="calibrated"), 64, 140),
    ("bf16_d128_pairs128_lwb1", dict(seq_lens=[64 * 6 + 5, 64 * 5 + 62], h_q=8, h_kv=2, d=128, lwb=1, paged=True),
     128, 200),
]


@pytest.mark.parametrize("name,kw,block,steps", LOOP_CASES, ids=[c[0] for c in LOOP_CASES])
def test_append_then_decode_loop(name, kw, block, steps):
    """Append one token to every sequence, then decode, at every step; records,
    sets, counts and outputs against the oracle at the lengths of that step."""
    log(f"[append+decode] {name}")
    bound = "geometric" if block == BLOCK else "geometric_sub"
    wl, _ = prepared("seq_32k", bound=bound, block=block, needles=0, **kw)
    T_final = wl.seq_lens.astype(np.int64)
    T0 = T_final - steps
    assert np.all(T0 >= 1)
    cache = fresh_cache(wl, **({} if block == BLOCK else dict(sub_block=block)))
    feed = Feeder(wl, cache)
    # the prefix, appended without decoding
    for t in range(int(T0.max())):
        feed.append([t if t < T0[n] else None for n in range(wl.n_seqs)])
    ws = eta.alloc_workspace(cache, wl.n_seqs, wl.max_blocks, wl.h_q)
    out = torch.empty(wl.n_seqs, wl.h_q, wl.d, dtype=torch.float32, device="cuda")
    q = eta.upload(wl.q, wl.kv_dtype, "cuda")
    w = torch.from_numpy(wl.w).cuda()
    b = torch.from_numpy(wl.bias.astype(np.float32)).cuda()
    mode = eta.ETA_TAU_LEARNED if wl.tau_mode == "learned" else eta.ETA_TAU_CALIBRATED
    worst = 0.0
    crossed = set()
    for i in range(steps):
        feed.append([int(T0[n]) + i for n in range(wl.n_seqs)])
        lens = (T0 + i + 1).astype(np.int32)
        for n in range(wl.n_seqs):
            if lens[n] % BLOCK == 0:
                crossed.add(("page", n, int(lens[n]) // BLOCK))
            if lens[n] % 128 == 0:
                crossed.add(("pair", n, int(lens[n]) // 128))
        eta.decode(cache, torch.from_numpy(lens).cuda(), feed.bt, q, mode, b, w=w, a=wl.a, beta=wl.beta,
                   lwb=wl.lwb, out=out, workspace=ws, bound=bound)
        torch.cuda.synchronize()
        wlt = at_lengths(wl, lens)
        check_page_records(wl, cache, lens)
        if block != BLOCK:
            check_sub_records(wl, cache, lens, block)
        st = eta.stats(ws, wl.n_seqs, wl.max_blocks, wl.h_q, wl.h_kv)
        res = oracle_decode(wlt, bound=bound, block=block)
        try:
            check_sets_and_counts(wlt, res, st)
            err = check_output(wlt, res, out.cpu().numpy().astype(np.float64))
        except AssertionError:
            log(f"  failed at step {i}, lengths {lens.tolist()}")
            raise
        worst = max(worst, err)
    log(f"  {steps} steps, lengths {T0.tolist()} -> {T_final.tolist()}, block ends crossed {sorted(crossed)}, "
        f"worst abs err {worst:.3g}")
    for n in range(wl.n_seqs):  # every sequence filled at least two pages while decoding
        assert sum(1 for c in crossed if c[0] == "page" and c[1] == n) >= 2
    if block > BLOCK:
        assert any(c[0] == "pair" for c in crossed)
