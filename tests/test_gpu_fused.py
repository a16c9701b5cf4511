"""The one-launch decode of short segments (at most 512 blocks per sequence,
geometric screen on page blocks) against the fp64 oracle and against the two
launches it replaces (screen phase, then attend phase), through the C ABI.

Each (sequence, KV head) gets several workgroups; each screens the whole
segment into its own copy of the screen's results and attends to its share of
the admitted blocks, and the last of them merges. Bars as everywhere: sets and
counts bit-exact, outputs within 1e-5 (float32 K/V) or 2e-3 (bfloat16 K/V)."""
import numpy as np
import pytest
import torch

import learned_threshold_block_amd as eta
from gpu_util import Dev, check_output, check_sets_and_counts, log, oracle_decode, prepared

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import learned_threshold_block_amd._lib as L
    L.lib()


def _launches(dev, bound="geometric"):
    return eta.decode_launches(dev.cache, dev.seq_lens, dev.bt, dev.wl.h_q, bound=bound)


def test_launch_forms(monkeypatch):
    """One launch up to 512 blocks per sequence with the geometric screen on
    page blocks; two from 513 blocks on, for the other screens, or with
    ETA_FUSED=0."""
    wl, _ = prepared("seq_32k", seq_lens=[64 * 512, 64 * 3], h_q=8, h_kv=2, needles=0)
    dev = Dev(wl, with_box=True)
    assert _launches(dev) == 1
    assert _launches(dev, bound="quest") == 2
    monkeypatch.setenv("ETA_FUSED", "0")
    assert _launches(dev) == 2
    monkeypatch.delenv("ETA_FUSED")
    wl2, _ = prepared("seq_32k", seq_lens=[64 * 513, 64 * 3], h_q=8, h_kv=2, needles=0)
    assert _launches(Dev(wl2)) == 2


CASES = [
    dict(seq_lens=[64 * 70 + 3, 64 * 64, 129, 1], h_q=8, h_kv=2, d=128),               # ragged, tails, T=1
    dict(seq_lens=[64 * 130 + 63, 64 * 5], h_q=16, h_kv=2, d=128, lwb=2, a=0.4),       # G=8 (two launches)
    dict(seq_lens=[5000, 7000], h_q=32, h_kv=4, d=64),                                  # G=8, d=64 bf16
    dict(seq_lens=[3000, 64 * 50], h_q=8, h_kv=4, d=64, kv_dtype="f32", beta=1.0),     # f32 d=64 G=2
    dict(seq_lens=[64 * 300], h_q=8, h_kv=2, d=128, mode="calibrated", density=0.1),   # sparse
    dict(n_seqs=5, h_q=8, h_kv=2, d=128, paged=True, density=[0.05, 0.3, 0.6, 0.9] * 2,
         seq_lens=[9000, 300, 64 * 12, 4097, 32768]),                                  # paged, spread, 512 blocks
    dict(seq_lens=[4000, 64 * 90], h_q=4, h_kv=4, d=128),                               # G=1, d=128 bf16
    dict(seq_lens=[64 * 200 + 1, 2500], h_q=8, h_kv=4, d=128, lwb=3),                   # G=2, d=128 bf16, lwb
    dict(seq_lens=[3000, 64 * 45 + 9], h_q=16, h_kv=4, d=64, kv_dtype="f32"),          # f32 d=64 G=4
]


@pytest.mark.parametrize("kw", CASES)
def test_one_launch_matches_oracle_and_two_phases(monkeypatch, kw):
    log(f"[fused] {kw}")
    wl, summ = prepared("seq_32k", **kw)
    dev = Dev(wl)
    dev.build()
    res = oracle_decode(wl, summaries=summ)
    log(f"  launches {_launches(dev)}")
    o1 = dev.decode()
    st1 = dev.stats()
    check_sets_and_counts(wl, res, st1)
    check_output(wl, res, o1)
    monkeypatch.setenv("ETA_FUSED", "0")
    o2 = dev.decode()
    st2 = dev.stats()
    monkeypatch.delenv("ETA_FUSED")
    check_sets_and_counts(wl, res, st2)
    check_output(wl, res, o2)
    scale = float(np.max(np.abs(o1)))
    assert float(np.max(np.abs(o1 - o2))) <= 1e-6 * scale


def test_rescue_in_one_launch():
    """Nothing passes and no block is forced: every workgroup of a segment
    applies the same top-1 rescue to its own copy of the lists."""
    wl, summ = prepared("seq_32k", seq_lens=[64 * 37, 64 * 8], h_q=8, h_kv=2, mode="calibrated")
    bias = np.full(wl.h_q, 1e4, dtype=np.float32)
    dev = Dev(wl)
    dev.build()
    assert _launches(dev) == 1
    o = dev.decode(bias=bias)
    st = dev.stats()
    res = oracle_decode(wl, summaries=summ, bias=bias)
    assert res.rescued.all()
    check_sets_and_counts(wl, res, st)
    check_output(wl, res, o)


@pytest.mark.parametrize("fill", [0x00, 0xFF, "random"])
def test_arrival_words_need_no_clearing(monkeypatch, fill):
    """The arrival words are tagged per call: whatever the workspace held
    before (zeros, all ones, random bytes, a two-phase decode's state, the
    previous call's words) the result is the same."""
    wl, summ = prepared("seq_32k", seq_lens=[64 * 200 + 30, 64 * 77], h_q=8, h_kv=2)
    res = oracle_decode(wl, summaries=summ)
    dev = Dev(wl)
    dev.build()
    if fill == "random":
        g = torch.Generator(device="cpu").manual_seed(5)
        dev.ws.copy_(torch.randint(0, 256, dev.ws.shape, dtype=torch.uint8, generator=g).to(dev.ws.device))
    else:
        dev.ws.fill_(fill)
    for form in ("1", "1", "0", "1"):
        monkeypatch.setenv("ETA_FUSED", form)
        o = dev.decode()
        st = dev.stats()
        check_sets_and_counts(wl, res, st)
        check_output(wl, res, o)


@pytest.mark.parametrize("wgs", ["4", "6", "16", "100", "512", "4096"])
def test_workgroups_per_segment(monkeypatch, wgs):
    """Any number of workgroups per segment from 2 up (grids below two per
    segment run as two launches): same sets, outputs at the bar."""
    wl, summ = prepared("seq_32k", seq_lens=[64 * 300 + 11, 64 * 40], h_q=8, h_kv=2)
    res = oracle_decode(wl, summaries=summ)
    dev = Dev(wl)
    dev.build()
    monkeypatch.setenv("ETA_ATTEND_WGS", wgs)
    log(f"  grid {wgs}: launches {_launches(dev)}")
    o = dev.decode()
    st = dev.stats()
    check_sets_and_counts(wl, res, st)
    check_output(wl, res, o)


def test_deterministic_one_launch_is_bitwise_repeatable(monkeypatch):
    wl, _ = prepared("seq_32k", seq_lens=[64 * 250 + 5, 3000], h_q=8, h_kv=2)
    dev = Dev(wl)
    dev.build()
    monkeypatch.setenv("ETA_DETERMINISTIC", "1")
    assert np.array_equal(dev.decode(), dev.decode())


@pytest.mark.parametrize("value", [1e-6, 0.0])
def test_screen_queries_near_zero(value):
    """Query elements of 1e-6 (below float16's normal range, in case a screen
    ever rounds queries to it) and exact zeros: same sets, counts and outputs
    as the oracle."""
    import placement
    import workloads as W

    wl = W.make_workload("seq_32k", seq_lens=[64 * 100 + 5, 3000], h_q=8, h_kv=2)
    q32 = W.bf16_bits_to_f32(wl.q).copy()
    q32[0, 1, 7] = value
    q32[1, 6, :5] = value
    wl.q = W.to_storage(q32, wl.kv_dtype)
    summ = placement.place(wl)
    dev = Dev(wl)
    dev.build()
    o = dev.decode()
    st = dev.stats()
    res = oracle_decode(wl, summaries=summ)
    check_sets_and_counts(wl, res, st)
    check_output(wl, res, o)
