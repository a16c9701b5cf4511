"""Causal prompt pass on the HIP path vs the fp64 oracle, through the C ABI.

Every output row is compared element by element with the oracle's at the
bfloat16 bar (max abs error 2e-3); the records the pass builds must equal
the bulk builder's bit for bit. Shapes cover every group size (and so every
tile height: 256, 128, 64 and 32 positions per workgroup), both head dims,
ragged ends inside a key block and inside a workgroup's tile, paged block
tables, both threshold modes, thresholds far below and far above every
logit, and the flagged error paths (which read nothing out of range)."""
import numpy as np
import pytest
import torch

import learned_threshold_block_amd as eta
import oracle.eta_oracle as E
import workloads as W
from gpu_util import TOL, Dev, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(wl, q_all, mode, b_or_c, beta, a=0.0, dev=None, check=True):
    dev = Dev(wl) if dev is None else dev
    qd = eta.upload(q_all, wl.kv_dtype, "cuda")
    m = eta.ETA_TAU_LEARNED if mode == "learned" else eta.ETA_TAU_CALIBRATED
    res = eta.prefill(dev.cache, dev.seq_lens, dev.bt, qd, m, torch.from_numpy(np.asarray(b_or_c, np.float32)).cuda(),
                      w=dev.w, a=a, beta=beta)
    torch.cuda.synchronize()
    if check:
        assert int(res.err.item()) == 0
    return dev, res.out.cpu().numpy().astype(np.float64), int(res.err.item())


def _compare(wl, got, ref):
    """Rows < seq_len within the tolerance, rows past it NaN on both sides."""
    worst = 0.0
    for n in range(wl.n_seqs):
        T = int(wl.seq_lens[n])
        g, r = got[n, :T], ref[n, :T]
        assert np.all(np.isfinite(g)), f"non-finite output in sequence {n}"
        err = float(np.max(np.abs(g - r)))
        if err > TOL["bf16"]:
            t, h, d = np.unravel_index(np.argmax(np.abs(g - r)), g.shape)
            raise AssertionError(f"max abs error {err} at (n={n}, t={t}, h={h}, d={d})")
        worst = max(worst, err)
        assert np.all(np.isnan(got[n, T:])), "rows past the sequence end must be NaN"
    log(f"  max abs err {worst:.3g} (tolerance {TOL['bf16']:g})")
    return worst


CASES = [
    # (config overrides, mode, per-head thresholds, beta, a)
    (dict(seq_lens=[1000, 700], h_q=8, h_kv=2, d=128), "learned", np.linspace(-1.0, 2.5, 8), 5.0, 0.0),
    (dict(seq_lens=[300, 64 * 5], h_q=2, h_kv=2, d=64), "calibrated", [0.5, 1.5], 2.0, 0.3),
    (dict(seq_lens=[777], h_q=16, h_kv=2, d=128), "learned", np.linspace(-0.5, 2.0, 16), 5.0, -0.2),
    (dict(seq_lens=[64 * 9 + 1, 129, 64], h_q=4, h_kv=2, d=128, paged=True), "calibrated",
     [-np.inf, 1.0, np.inf, 0.0], 5.0, 0.0),
    (dict(seq_lens=[1, 2, 63, 65], h_q=8, h_kv=8, d=64), "learned", np.linspace(0.0, 1.0, 8), 1.0, 0.0),
]


@pytest.mark.parametrize("kw,mode,b,beta,a", CASES)
def test_prefill_parity(kw, mode, b, beta, a):
    log(f"[prefill] {mode} {kw} beta={beta} a={a}")
    wl = W.make_workload("seq_32k", needles=0, **kw)
    q_all = W.trace_queries(wl, seed=11)
    b = np.asarray(b, np.float32)
    dev, got, _ = _run(wl, q_all, mode, b, beta, a)
    ref = E.prefill(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, q_all, mode, wl.w, b, a, beta)
    _compare(wl, got, ref)
    # the records of every complete block, as the bulk builder makes them
    dev2 = Dev(wl)
    dev2.build()
    torch.cuda.synchronize()
    assert np.array_equal(dev.mu_bits(), dev2.mu_bits())
    assert np.array_equal(dev.radius().view(np.uint32), dev2.radius().view(np.uint32))


def test_prefill_records_with_sigma():
    """With a deviation buffer the pass fills it too, as the bulk builder does."""
    wl = W.make_workload("seq_32k", seq_lens=[64 * 7 + 5, 64 * 3], h_q=8, h_kv=2, d=128, needles=0)
    q_all = W.trace_queries(wl, seed=12)
    dev = Dev(wl, with_sigma=True)
    _run(wl, q_all, "learned", np.ones(8, np.float32), 5.0, dev=dev)
    dev2 = Dev(wl, with_sigma=True)
    dev2.build()
    torch.cuda.synchronize()
    assert np.array_equal(dev.sigma_bits(), dev2.sigma_bits())
    assert np.array_equal(dev.mu_bits(), dev2.mu_bits())


def test_prefill_longer_sampled_heads():
    """A 4113-token prompt (a ragged end, 65 key blocks): all rows of two heads."""
    wl = W.make_workload("seq_32k", seq_lens=[4096 + 17], h_q=8, h_kv=2, d=128, needles=0)
    q_all = W.trace_queries(wl, seed=13)
    b = np.linspace(-1.0, 2.0, 8).astype(np.float32)
    _, got, _ = _run(wl, q_all, "learned", b, 5.0)
    heads = [(0, 1), (0, 6)]
    ref = E.prefill(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, q_all, "learned", wl.w, b,
                    0.0, 5.0, heads=heads)
    for _, h in heads:
        err = float(np.max(np.abs(got[0, :4113, h] - ref[0, :4113, h])))
        log(f"  head {h}: max abs err {err:.3g}")
        assert err <= TOL["bf16"]
    assert np.all(np.isnan(got[0, 4113:]))


def test_prefill_flags_bad_page_and_length():
    """An out-of-range page id and a length past the table are flagged; the
    other sequence is still exact, the bad-length one is NaN."""
    wl = W.make_workload("seq_32k", seq_lens=[200, 300], h_q=4, h_kv=1, d=128, needles=0)
    q_all = W.trace_queries(wl, seed=14)
    b = np.full(4, 1.0, np.float32)
    dev = Dev(wl)
    dev.seq_lens[1] = 64 * wl.max_blocks + 1
    _, got, err = _run(wl, q_all, "learned", b, 5.0, dev=dev, check=False)
    assert err == 1
    assert np.all(np.isnan(got[1]))
    ref = E.prefill(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, q_all, "learned", wl.w, b,
                    0.0, 5.0)
    assert float(np.max(np.abs(got[0, :200] - ref[0, :200]))) <= TOL["bf16"]
    dev = Dev(wl)
    dev.bt[0, 1] = wl.num_pages  # one past the last page
    _, got, err = _run(wl, q_all, "learned", b, 5.0, dev=dev, check=False)
    assert err == 1
    # rows before the bad block only see good keys
    assert float(np.max(np.abs(got[0, :64] - ref[0, :64]))) <= TOL["bf16"]


def test_prefill_empty_sequence():
    """seq_len 0: every row NaN, no flag, the other sequence exact."""
    wl = W.make_workload("seq_32k", seq_lens=[130, 64], h_q=4, h_kv=2, d=64, needles=0)
    q_all = W.trace_queries(wl, seed=15)
    b = np.full(4, 0.5, np.float32)
    dev = Dev(wl)
    dev.seq_lens[1] = 0
    _, got, err = _run(wl, q_all, "learned", b, 5.0, dev=dev, check=False)
    assert err == 0
    assert np.all(np.isnan(got[1]))
    ref = E.prefill(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, q_all, "learned", wl.w, b,
                    0.0, 5.0)
    assert float(np.max(np.abs(got[0, :130] - ref[0, :130]))) <= TOL["bf16"]


def test_prefill_seq32k_sampled():
    """The full 32768-token prompt (32 query heads over 8 KV heads, d = 128),
    as the benchmark runs it: 260 sampled rows (every workgroup tile's first
    and last row among them at a stride of 16 tiles, plus random ones) of
    eight heads, two per KV head, against the oracle; every row finite, and
    every record equal to the bulk builder's."""
    wl = W.make_workload("seq_32k")
    q_all = W.trace_queries(wl, seed=21)
    b = np.linspace(-1.0, 2.5, wl.h_q).astype(np.float32)
    dev, got, _ = _run(wl, q_all, "learned", b, 5.0)
    rng = np.random.default_rng(5)
    edges = [t for j in range(0, 512, 16) for t in (64 * j, 64 * j + 31, 64 * j + 32, 64 * j + 63)]
    rows = sorted(set([0, 1, 4095, 4096, 16383, 32766, 32767] + edges + rng.integers(0, 32768, 128).tolist()))
    heads = [(0, 0), (0, 3), (0, 5), (0, 10), (0, 17), (0, 22), (0, 28), (0, 31)]
    ref = E.prefill(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, q_all, "learned", wl.w, b,
                    0.0, 5.0, heads=heads, positions=rows)
    assert np.all(np.isfinite(got[0]))
    for _, h in heads:
        err = float(np.max(np.abs(got[0, rows, h] - ref[0, rows, h])))
        log(f"  head {h}: max abs err over {len(rows)} rows {err:.3g}")
        assert err <= TOL["bf16"]
    dev2 = Dev(wl)
    dev2.build()
    torch.cuda.synchronize()
    assert np.array_equal(dev.mu_bits(), dev2.mu_bits())
    assert np.array_equal(dev.radius().view(np.uint32), dev2.radius().view(np.uint32))


@pytest.mark.parametrize("wide", [70000.0, -1e30])
def test_prefill_values_beyond_float16(wide):
    """A V element past float16's exact range anywhere in the prompt switches
    the pass to the two-term bfloat16 products: outputs at the bar relative to
    their size, no error reported."""
    wl = W.make_workload("seq_32k", seq_lens=[64 * 3 + 7, 64 * 2], h_q=4, h_kv=2, d=64, needles=0)
    bits = np.float32(wide).view(np.uint32) >> 16
    page = int(wl.block_table[1, 1])
    wl.v_pages[page, 0, 5, 3] = np.uint16(bits)  # sequence 1, KV head 0, token 69, dim 3
    q_all = W.trace_queries(wl, seed=13)
    b = np.linspace(0.5, 1.5, wl.h_q).astype(np.float32)
    _, got, _ = _run(wl, q_all, "learned", b, 5.0)
    ref = E.prefill(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, q_all, "learned", wl.w, b,
                    0.0, 5.0)
    for n in range(wl.n_seqs):
        T = int(wl.seq_lens[n])
        g, r = got[n, :T], ref[n, :T]
        fin = np.isfinite(r)
        assert np.array_equal(fin, np.isfinite(g))
        err = np.abs(g[fin] - r[fin]) / np.maximum(1.0, np.abs(r[fin]))
        assert float(err.max()) <= TOL["bf16"], float(err.max())
    assert np.all(np.isfinite(got[0, :int(wl.seq_lens[0])]))  # the other sequence is untouched


F32_CASES = [
    (dict(seq_lens=[700, 64 * 5], h_q=8, h_kv=2, d=128), "learned", np.linspace(-1.0, 2.5, 8), 5.0, 0.0),
    (dict(seq_lens=[300, 65], h_q=2, h_kv=2, d=64), "calibrated", [0.5, 1.5], 2.0, 0.3),
    (dict(seq_lens=[64 * 4 + 9, 129, 64], h_q=4, h_kv=2, d=128, paged=True), "calibrated",
     [-np.inf, 1.0, np.inf, 0.0], 5.0, 0.0),
    (dict(seq_lens=[1, 63, 200], h_q=8, h_kv=1, d=64), "learned", np.linspace(0.0, 1.0, 8), 1.0, -0.2),
]


@pytest.mark.parametrize("kw,mode,b,beta,a", F32_CASES)
def test_prefill_parity_f32(kw, mode, b, beta, a):
    """float32 caches: every row at the float32 bar, and the records equal to
    the bulk builder's bit for bit (G = 4, 1, 2 and 8; both head dims)."""
    log(f"[prefill f32] {mode} {kw} beta={beta} a={a}")
    wl = W.make_workload("tiny_4k_f32", needles=0, **kw)
    assert wl.kv_dtype == "f32"
    q_all = W.trace_queries(wl, seed=21)
    b = np.asarray(b, np.float32)
    dev, got, _ = _run(wl, q_all, mode, b, beta, a)
    ref = E.prefill(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, q_all, mode, wl.w, b, a, beta)
    worst = 0.0
    for n in range(wl.n_seqs):
        T = int(wl.seq_lens[n])
        assert np.all(np.isfinite(got[n, :T]))
        worst = max(worst, float(np.max(np.abs(got[n, :T] - ref[n, :T]))))
        assert np.all(np.isnan(got[n, T:]))
    log(f"  max abs err {worst:.3g} (tolerance {TOL['f32']:g})")
    assert worst <= TOL["f32"]
    dev2 = Dev(wl)
    dev2.build()
    torch.cuda.synchronize()
    assert np.array_equal(dev.mu_bits(), dev2.mu_bits())
    assert np.array_equal(dev.radius().view(np.uint32), dev2.radius().view(np.uint32))


def test_prefill_f32_nonfinite_v_reaches_only_later_positions():
    """float32 caches skip the keys after a position: an infinite element of V
    at key s makes that element of the outputs non-finite at positions >= s
    only, as in the oracle; the other elements stay at the bar."""
    wl = W.make_workload("tiny_4k_f32", seq_lens=[64 * 3 + 20], h_q=4, h_kv=2, d=64, needles=0)
    q_all = W.trace_queries(wl, seed=22)
    s_key, elem = 64 + 37, 5
    wl.v_pages[wl.block_table[0, s_key // 64], 1, s_key % 64, elem] = np.float32(np.inf)
    b = np.full(4, 0.5, np.float32)
    _, got, _ = _run(wl, q_all, "learned", b, 5.0)
    ref = E.prefill(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, q_all, "learned", wl.w, b,
                    0.0, 5.0)
    T = int(wl.seq_lens[0])
    g, r = got[0, :T], ref[0, :T]
    assert np.array_equal(np.isfinite(g), np.isfinite(r))
    assert not np.isfinite(g[s_key:, 2:4, elem]).any() and np.isfinite(g[:s_key, 2:4, elem]).all()
    fin = np.isfinite(r)
    assert float(np.max(np.abs(g[fin] - r[fin]))) <= TOL["f32"]
