"""Offline calibration on the HIP path vs the fp64 oracle, through the C ABI.

Weights are integers on both sides, so totals agree exactly. A score whose
bin (or whose side of the learned threshold) is decided by less than the
float32 error of the GPU's dot products may land differently; the test
computes those ambiguous scores in float64 and allows exactly their weight as
the difference, per bin and for the target. The constant must then satisfy
the search's definition on the oracle's histogram within that allowance."""
import math

import numpy as np
import pytest
import torch

import learned_threshold_block_amd as eta
import oracle.eta_oracle as E
import workloads as W
from gpu_util import Dev, log

pytestmark = pytest.mark.gpu

BIN_EPS = 0.01   # ambiguous: within 1% of a bin width of an edge
TAU_EPS = 1e-4   # ambiguous: within this of the learned threshold


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _ambiguity(wl, q_all, h, lo, hi, B, w_h=None, b_h=None):
    """Weights of ambiguous scores: per oracle bin (near an edge) and near the threshold."""
    D = wl.d
    g = h // wl.group
    amb_bin = np.zeros(B, dtype=np.int64)
    amb_tau = 0
    for n in range(wl.n_seqs):
        T = int(wl.seq_lens[n])
        nb = -(-T // 64)
        K = E.upcast(wl.k_pages[wl.block_table[n, :nb], g], wl.kv_dtype).reshape(nb * 64, D)[:T]
        Q = E.upcast(q_all[n, :T, h], wl.kv_dtype)
        S = (Q @ K.T) / math.sqrt(D)
        x = (S - lo) * (B / (hi - lo))
        near = np.abs(x - np.round(x)) < BIN_EPS
        tri = np.tril(np.ones((T, T), dtype=bool))
        wts = np.array([E.row_weight(t) for t in range(T)], dtype=np.int64)[:, None] * np.ones((1, T), np.int64)
        bins = E.score_bins(S, lo, hi, B)
        m = near & tri
        np.add.at(amb_bin, bins[m], wts[m])
        if w_h is not None:
            tau = Q @ np.asarray(w_h, np.float64) + float(b_h)
            amb_tau += int(wts[tri & (np.abs(S - tau[:, None]) < TAU_EPS)].sum())
    return amb_bin, amb_tau


def _check_head(got_hist, got_above, got_total, got_c, ref, amb_bin, amb_tau, lo, hi, B, learned):
    assert got_total == ref["total"]
    # a score near edge b can be in bin b-1 or b on either side
    allow = amb_bin + np.roll(amb_bin, 1) + np.roll(amb_bin, -1)
    diff = np.abs(got_hist.astype(np.int64) - ref["hist"])
    assert np.all(diff <= allow), int((diff > allow).sum())
    assert int(got_hist.sum()) == ref["total"]
    if learned:
        assert abs(got_above - ref["above"]) <= amb_tau
    slack = int(amb_bin.sum()) + (amb_tau if learned else 0)
    tail = np.concatenate([np.cumsum(ref["hist"][::-1])[::-1], [0]])
    b = int(round((got_c - lo) * B / (hi - lo)))
    assert abs(got_c - (lo + b * (hi - lo) / B)) <= 1e-5 * max(1.0, abs(got_c))
    assert tail[b] <= ref["target"] + slack
    assert b == 0 or tail[b - 1] > ref["target"] - slack
    return b


@pytest.mark.parametrize("kw,learned", [
    (dict(seq_lens=[1000, 700], h_q=8, h_kv=2, d=128), True),
    (dict(seq_lens=[900, 64 * 5], h_q=4, h_kv=4, d=64, kv_dtype="f32"), False),
    (dict(seq_lens=[777], h_q=16, h_kv=2, d=128), True),
    (dict(seq_lens=[900, 64 * 5], h_q=4, h_kv=4, d=64), False),
    (dict(seq_lens=[500, 130], h_q=4, h_kv=2, d=64), True),
    (dict(seq_lens=[1000, 64], h_q=2, h_kv=1, d=128, paged=True), False),
])
def test_calibration_parity(kw, learned):
    wl = W.make_workload("seq_32k", needles=0, **kw)
    q_all = W.trace_queries(wl, seed=5)
    lo, hi, B = -8.0, 8.0, min(1024, 8192 // wl.group)
    dev = Dev(wl)
    qd = eta.upload(q_all, wl.kv_dtype, "cuda")
    if learned:
        bias = np.linspace(0.5, 2.0, wl.h_q).astype(np.float32)
        cal = eta.calibrate(dev.cache, dev.seq_lens, dev.bt, qd, B, lo, hi, w=dev.w,
                            b=torch.from_numpy(bias).cuda())
        ref = E.calibrate(wl.k_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, q_all, wl.h_kv, lo, hi, B,
                          w=wl.w, b=bias)
    else:
        rho = np.linspace(0.05, 0.6, wl.h_q).astype(np.float32)
        cal = eta.calibrate(dev.cache, dev.seq_lens, dev.bt, qd, B, lo, hi, rho=torch.from_numpy(rho).cuda())
        ref = E.calibrate(wl.k_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, q_all, wl.h_kv, lo, hi, B, rho=rho)
    torch.cuda.synchronize()
    assert int(cal.err.item()) == 0
    hist = cal.hist.cpu().numpy()
    above = cal.above.cpu().numpy()
    total = cal.total.cpu().numpy()
    c = cal.c.cpu().numpy()
    for h in range(wl.h_q):
        amb_bin, amb_tau = _ambiguity(wl, q_all, h, lo, hi, B, wl.w[h] if learned else None,
                                      bias[h] if learned else None)
        b = _check_head(hist[h], int(above[h]), int(total[h]), float(c[h]), ref[h], amb_bin, amb_tau, lo, hi, B,
                        learned)
        log(f"  head {h}: bin {b} (oracle {ref[h]['bin']}), c {c[h]:.4f}, "
            f"ambiguous weight {int(amb_bin.sum()) / ref[h]['total']:.2e}")


def test_calibrated_constant_reproduces_density():
    """Running the calibrated constants back through the oracle's weighted
    tail gives the target density to within one bin's weight."""
    wl = W.make_workload("seq_32k", seq_lens=[1200], h_q=4, h_kv=1, d=128, needles=0)
    q_all = W.trace_queries(wl, seed=9)
    lo, hi, B = -8.0, 8.0, 2048
    dev = Dev(wl)
    rho = np.array([0.1, 0.25, 0.4, 0.7], dtype=np.float32)
    cal = eta.calibrate(dev.cache, dev.seq_lens, dev.bt, eta.upload(q_all, wl.kv_dtype, "cuda"), B, lo, hi,
                        rho=torch.from_numpy(rho).cuda())
    torch.cuda.synchronize()
    hist = cal.hist.cpu().numpy().astype(np.int64)
    total = cal.total.cpu().numpy()
    c = cal.c.cpu().numpy()
    for h in range(4):
        b = int(round((c[h] - lo) * B / (hi - lo)))
        dens = hist[h, b:].sum() / total[h]
        below = hist[h, b - 1:].sum() / total[h]
        assert dens <= rho[h] < below + 1e-12, (h, dens, rho[h], below)


@pytest.mark.parametrize("kv_dtype", ["bf16", "f32"])
def test_out_of_range_page_is_reported(kv_dtype):
    """A block-table entry past the cache sets the error flag; that key tile is
    skipped and nothing else is disturbed (the row totals do not depend on it)."""
    wl = W.make_workload("seq_32k", seq_lens=[64 * 6 + 9], h_q=4, h_kv=2, d=128, needles=0, kv_dtype=kv_dtype)
    q_all = W.trace_queries(wl, seed=4)
    dev = Dev(wl)
    bt = dev.bt.clone()
    bt[0, 2] = wl.num_pages  # one past the last page
    cal = eta.calibrate(dev.cache, dev.seq_lens, bt, eta.upload(q_all, wl.kv_dtype, "cuda"), 256, -8.0, 8.0,
                        rho=torch.full((wl.h_q,), 0.3, device="cuda"))
    torch.cuda.synchronize()
    assert int(cal.err.item()) == 1
    T = int(wl.seq_lens[0])
    want = sum(E.row_weight(t) * (t + 1) for t in range(T))
    assert all(int(x) == want for x in cal.total.cpu().numpy())
    # the skipped tile's scores are missing from the histogram: less weight than the full triangle
    assert all(int(x) < want for x in cal.hist.cpu().numpy().sum(axis=1))


@pytest.mark.parametrize("kv_dtype", ["bf16", "f32"])
def test_nonfinite_keys_follow_the_oracle(kv_dtype):
    """Keys holding NaN, +inf and -inf: a NaN score falls in bin 0 and is never
    at or above the threshold; an infinite score falls in the end bin of its
    sign and counts as above when positive. Histograms, above-counts and
    constants match the oracle under the same allowance as finite scores."""
    wl = W.make_workload("seq_32k", seq_lens=[64 * 7 + 21, 300], h_q=4, h_kv=2, d=128, needles=0,
                         kv_dtype=kv_dtype)
    q_all = W.trace_queries(wl, seed=12)
    plant = [(0, 0, 70, 3, np.nan), (0, 1, 200, 5, np.inf), (0, 0, 411, 7, -np.inf), (1, 1, 299, 0, np.nan)]
    for n, g, s, e, x in plant:
        page = wl.block_table[n, s // 64]
        wl.k_pages[page, g, s % 64, e] = W.to_storage(np.array([x], np.float32), kv_dtype)[0]
    log(f"[calibration non-finite keys] {kv_dtype}: (seq, kv head, position, element, value) {plant}")
    lo, hi, B = -8.0, 8.0, 512
    dev = Dev(wl)
    bias = np.linspace(0.5, 2.0, wl.h_q).astype(np.float32)
    cal = eta.calibrate(dev.cache, dev.seq_lens, dev.bt, eta.upload(q_all, wl.kv_dtype, "cuda"), B, lo, hi,
                        w=dev.w, b=torch.from_numpy(bias).cuda())
    ref = E.calibrate(wl.k_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, q_all, wl.h_kv, lo, hi, B,
                      w=wl.w, b=bias)
    torch.cuda.synchronize()
    assert int(cal.err.item()) == 0
    hist = cal.hist.cpu().numpy()
    above = cal.above.cpu().numpy()
    total = cal.total.cpu().numpy()
    c = cal.c.cpu().numpy()
    with np.errstate(invalid="ignore"):
        for h in range(wl.h_q):
            amb_bin, amb_tau = _ambiguity(wl, q_all, h, lo, hi, B, wl.w[h], bias[h])
            _check_head(hist[h], int(above[h]), int(total[h]), float(c[h]), ref[h], amb_bin, amb_tau, lo, hi, B,
                        True)
