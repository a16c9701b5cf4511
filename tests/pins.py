"""Checks that pin the fp64 oracle to facts outside itself.

Each `pin_*` takes the oracle module (so that the mutation tests can hand in a
deliberately broken copy) and raises AssertionError when the oracle disagrees
with: values printed on the pages, closed forms, a library routine, or the
per-key brute force. Source: "Elastic Threshold Attention: Learned Contextual
Sparsity for Long-Context Decoding" (paperpeel.com/paper/2609.20888).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import bruteforce
import workloads as W

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _decode(E, wl, bias=None, a=None, beta=None, lwb=None, tau_mode=None, **kw):
    return E.decode(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, wl.q,
                    tau_mode or wl.tau_mode, wl.w, wl.bias if bias is None else bias,
                    wl.a if a is None else a, wl.beta if beta is None else beta,
                    wl.lwb if lwb is None else lwb, **kw)


def tiny(seed, n=2, lens=(200, 128), h_q=4, h_kv=2, d=8, dtype="bf16", mode="learned", lwb=0,
         a=0.0, beta=5.0, density=0.4, bias=None, paged=None):
    """A tiny random workload with its threshold constant placed so that about
    `density` of the complete blocks pass (placement uses the module's own
    bound only to choose a number; the checks do not depend on it)."""
    wl = W.make_workload("seq_32k", seed=seed, n_seqs=n, seq_lens=list(lens), h_q=h_q, h_kv=h_kv,
                         d=d, kv_dtype=dtype, mode=mode, needles=0, lwb=lwb, a=a, beta=beta,
                         threads=1, paged=paged)
    if bias is None:
        bias = np.zeros(h_q, dtype=np.float32)
        rng = np.random.default_rng(seed + 99)
        bias[:] = rng.uniform(1.0, 4.0, size=h_q).astype(np.float32)
    wl.bias = np.asarray(bias, dtype=np.float32)
    return wl


# --------------------------------------------------------------------------- B.1 convention
def pin_sigmoid_convention(E):
    """Section 4.1 / B.1: at start-dense init (tau = -8, logits ~ 0) the gate's
    sigmoid derivative is 3.35e-4 at beta = 1 and ~4.3e-18 at beta = 5, and
    every key passes (Section 2.1)."""
    with open(os.path.join(GOLDEN, "sigmoid_convention.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        eps = 1e-3
        ratio = float(E.gate(np.array([eps]), c["tau"], c["beta"])[0]) / eps
        # the gate multiplies the logit by sigmoid(beta (S - tau)): recover the
        # sigmoid's argument from the ratio and check the printed derivative
        sig = float(E.sigmoid(np.array([c["sigmoid_arg"]]))[0])
        assert abs(ratio - sig) < 1e-6, (ratio, sig)
        assert ratio > 0.99, "start-dense init must let every key pass"
        deriv = sig * float(E.sigmoid(np.array([-c["sigmoid_arg"]]))[0])
        assert abs(deriv / c["sigmoid_prime"] - 1.0) < c["rel_tol"], (deriv, c)


def pin_gate_closed_forms(E):
    """sigmoid(0) = 1/2 at the threshold; far above it the logit passes; far
    below it shrinks to 0 (the uniform floor of Section 1)."""
    S = np.array([2.5, 30.0, -30.0, -2.0])
    g = E.gate(S, 2.5, 5.0)
    assert abs(g[0] - 1.25) < 1e-15
    assert abs(g[1] - 30.0) < 1e-12
    assert abs(g[2]) < 1e-60
    assert abs(g[3] - (-2.0) / (1.0 + math.exp(22.5))) < 1e-20
    gd = E.gate(S, -math.inf, 5.0)
    assert np.array_equal(gd, S), "tau = -inf must leave logits unchanged"


# --------------------------------------------------------------------------- block records
def pin_fp16_rne(E):
    """Centroids are stored as float16 with round-to-nearest-even (F.1)."""
    d = 4
    cases = [
        (1.0 + 2.0 ** -11, 1.0),                       # tie -> even (down)
        (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),       # tie -> even (up)
        (1.0 + 2.0 ** -11 + 2.0 ** -20, 1.0 + 2.0 ** -10),
        (-(2.0 + 2.0 ** -10), -2.0),                   # tie at 2 -> even
        (1000.3, 1000.5),                              # spacing 0.5 near 1000
    ]
    for x, want in cases:
        kb = np.full((64, d), x, dtype=np.float64)
        mu, R = E.block_summary(kb)
        assert np.all(mu == want), (x, mu, want)
        assert abs(R - math.sqrt(d) * abs(x - want)) <= 1e-12 * max(1.0, abs(x)), (R, x, want)
    # the mean of distinct rows, not of a single row
    kb = np.zeros((64, d))
    kb[:32] = 1.0
    mu, R = E.block_summary(kb)
    assert np.all(mu == 0.5) and abs(R - 1.0) < 1e-15
    # overflowing centroid falls back to the origin; non-finite keys give R = inf
    kb = np.full((64, d), 70000.0)
    mu, R = E.block_summary(kb)
    assert np.all(mu == 0.0) and abs(R - 140000.0) < 1e-6
    kb = np.zeros((64, d))
    kb[5, 1] = np.inf
    mu, R = E.block_summary(kb)
    assert R == math.inf
    kb[5, 1] = np.nan
    mu, R = E.block_summary(kb)
    assert R == math.inf


def pin_bound_sound_and_tight(E, seed=0, trials=200):
    """For every block and query, s q.k <= UB (Cauchy-Schwarz about the stored
    centroid), with equality for a query pointing from the centroid to the
    farthest key."""
    rng = np.random.default_rng(seed)
    for it in range(trials):
        d = int(rng.choice([4, 8, 64, 128]))
        kind = it % 5
        if kind == 0:
            kb = rng.standard_normal((1, d)) + 0.3 * rng.standard_normal((64, d))
        elif kind == 1:  # coarse float16 spacing: centroid rounding is large
            kb = 1000.0 + rng.uniform(0, 0.49, size=(1, d)) + 1e-3 * rng.standard_normal((64, d))
        elif kind == 2:  # one outlier key
            kb = rng.standard_normal((64, d))
            kb[rng.integers(64)] *= 25.0
        elif kind == 3:  # all keys equal, off the float16 grid
            kb = np.repeat(rng.uniform(-3000, 3000, size=(1, d)), 64, axis=0)
        else:
            kb = rng.standard_normal((64, d)) * rng.uniform(0.01, 10.0)
        s = 1.0 / math.sqrt(d)
        mu, R = E.block_summary(kb)
        qs = [rng.standard_normal(d) * rng.uniform(0.1, 5.0), -(kb[0] - mu) * 3.7]
        far = int(np.argmax(np.linalg.norm(kb - mu, axis=1)))
        tight_q = (kb[far] - mu) * 2.3
        qs.append(tight_q)
        for q in qs:
            if not np.any(q):
                continue
            ub = float(E.block_bound(q, mu[None, :], np.array([R]), s)[0])
            smax = float((s * (kb @ q)).max())
            assert ub >= smax - 1e-9 * (1 + abs(smax)), (it, kind, ub, smax)
        ub = float(E.block_bound(tight_q, mu[None, :], np.array([R]), s)[0])
        smax = float((s * (kb @ tight_q)).max())
        if np.any(tight_q):
            assert abs(ub - smax) <= 1e-9 * (1 + abs(smax)), ("not tight", it, kind, ub, smax)



# --------------------------------------------------------------------------- dual screen
def pin_sigma_rne(E):
    """sigma^ is the population deviation about the exact mean, stored as
    float16 with round to nearest even (F.1)."""
    d = 4
    for a, b, want in [(3.0, 1.0 + 2.0 ** -11, 1.0),               # tie -> even (down)
                       (3.0, 1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),  # tie -> even (up)
                       (-7.25, 0.125, 0.125),
                       (100.0, 2.0 ** -20, 2.0 ** -20)]:              # float16 subnormal range
        kb = np.full((64, d), a)
        kb[::2] += b
        kb[1::2] -= b
        sig = E.block_sigma(kb)
        assert np.all(sig == np.float64(np.float16(want))), (a, b, sig)
    assert np.all(E.block_sigma(np.full((64, d), 5.5)) == 0.0)
    kb = np.zeros((64, d))
    kb[7, 2] = np.inf
    assert np.isinf(E.block_sigma(kb)[2])


def pin_dual_closed_form(E):
    """Keys mu +/- b (every coordinate) around an fp16-exact mu: sigma^ = b,
    R = b sqrt(d); the dual score is s (q.mu + z b ||q||) for z < sqrt(d) and
    the geometric bound s (q.mu + b sqrt(d) ||q||) for z > sqrt(d)."""
    rng = np.random.default_rng(3)
    d = 8
    mu = np.round(rng.standard_normal(d) * 64) / 64
    b = 0.375
    kb = np.repeat(mu[None], 64, axis=0)
    kb[::2] += b
    kb[1::2] -= b
    m, R = E.block_summary(kb)
    sig = E.block_sigma(kb)
    assert np.array_equal(m, mu) and abs(R - b * math.sqrt(d)) < 1e-15 and np.all(sig == b)
    q = rng.standard_normal(d)
    s = 1 / math.sqrt(d)
    qn = math.sqrt(float(q @ q))
    for z, want in [(2.0, s * (q @ mu + 2.0 * b * qn)), (3.0, s * (q @ mu + b * math.sqrt(d) * qn))]:
        got = float(E.dual_score(q, m[None], np.array([R]), sig[None], s, z)[0])
        assert abs(got - want) <= 1e-12 * (1 + abs(want)), (z, got, want)


def pin_dual_within_geometric(E, seeds=range(3)):
    """The dual score never exceeds the geometric bound, so without rescue the
    dual sets nest inside the geometric ones; a huge z gives the geometric sets."""
    for seed in seeds:
        wl = tiny(40 + seed, n=2, lens=(64 * 9 + 3, 64 * 5 + 7), h_q=4, h_kv=2, d=8, mode="calibrated",
                  bias=np.full(4, 1.0, dtype=np.float32))
        geo = _decode(E, wl, with_output=False)
        dual = _decode(E, wl, with_output=False, bound="dual", z=2.0)
        assert not geo.rescued.any() and not dual.rescued.any()
        ok = ~np.isnan(geo.ub)
        assert np.all(dual.ub[ok] <= geo.ub[ok])
        assert np.all(dual.admitted <= geo.admitted)
        huge = _decode(E, wl, with_output=False, bound="dual", z=1e6)
        assert np.array_equal(huge.admitted, geo.admitted)


def pin_dual_bruteforce(E, seeds=range(3)):
    """Dual-screen sets, counts and outputs equal the per-key brute force."""
    variants = [dict(n=2, lens=(200, 128), h_q=4, h_kv=2, d=8, dtype="bf16", mode="learned"),
                dict(n=1, lens=(320,), h_q=2, h_kv=1, d=4, dtype="f32", mode="calibrated"),
                dict(n=2, lens=(130, 256), h_q=2, h_kv=2, d=8, dtype="bf16", mode="calibrated", lwb=1)]
    for seed in seeds:
        wl = tiny(60 + seed, **variants[seed % len(variants)])
        res = _decode(E, wl, bound="dual", z=2.0)
        bf, bf_union = bruteforce.decode(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table,
                                         wl.seq_lens, wl.q, wl.tau_mode, wl.w, wl.bias, wl.a,
                                         wl.beta, wl.lwb, bound="dual", z=2.0)
        for (n, h), r in bf.items():
            got = sorted(np.nonzero(res.admitted[n, h])[0].tolist())
            assert got == r["admitted"], (seed, n, h, got, r["admitted"])
            assert bool(res.rescued[n, h]) == r["rescued"]
            np.testing.assert_allclose(res.ub[n, h, :len(r["ub"])], r["ub"], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(res.o[n, h], r["o"], rtol=1e-10, atol=1e-12)
        for (n, g), u in bf_union.items():
            assert int(res.union[n, g]) == u


# --------------------------------------------------------------------------- Quest comparator
def pin_quest_directed_rounding(E):
    """float16 rounding toward -inf / +inf, by hand: spacing 2^-10 at 1, the
    largest finite 65504, the smallest subnormal 2^-24."""
    x = np.array([1.0001, -1.0001, 1.0, 0.5, -3.25, 65504.0, 70000.0, -70000.0, 2.0 ** -30, -2.0 ** -30, 0.0])
    down = [1.0, -1.0 - 2.0 ** -10, 1.0, 0.5, -3.25, 65504.0, 65504.0, -np.inf, 0.0, -2.0 ** -24, 0.0]
    up = [1.0 + 2.0 ** -10, -1.0, 1.0, 0.5, -3.25, 65504.0, np.inf, -65504.0, 2.0 ** -24, 0.0, 0.0]
    assert np.array_equal(E.f16_round_down(x), np.array(down))
    assert np.array_equal(E.f16_round_up(x), np.array(up))
    assert np.isnan(E.f16_round_down(np.nan)) and np.isnan(E.f16_round_up(np.nan))


def pin_quest_box_corners(E, seed=3, trials=50):
    """The box bound is the best corner of the stored box (all 2^d corners
    enumerated, d = 4), never below any key's logit, equal to it for a block
    of one repeated float16-exact key; the stored box is the independent
    brute force's outward rounding of the coordinate extrema."""
    import itertools
    rng = np.random.default_rng(seed)
    d = 4
    s = 1.0 / math.sqrt(d)
    for _ in range(trials):
        kb = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.normal(0, 2, (64, d)).astype(np.float32))).astype(np.float64)
        q = rng.normal(0, 1, d)
        lo, hi = E.block_box(kb)
        blo, bhi = bruteforce.box([list(map(float, r)) for r in kb])
        assert np.array_equal(lo, blo) and np.array_equal(hi, bhi)
        assert np.all(lo <= kb.min(axis=0)) and np.all(hi >= kb.max(axis=0))
        ub = float(E.quest_bound(q, lo[None], hi[None], s)[0])
        corners = max(s * sum(q[c] * (hi[c] if pick[c] else lo[c]) for c in range(d))
                      for pick in itertools.product((0, 1), repeat=d))
        assert abs(ub - corners) <= 1e-12 * max(1.0, abs(corners))
        assert ub >= s * float((kb @ q).max()) - 1e-12
    k = np.array([0.5, -1.25, 3.0, 0.0])
    lo, hi = E.block_box(np.tile(k, (64, 1)))
    assert np.array_equal(lo, k) and np.array_equal(hi, k)
    assert float(E.quest_bound(np.array([1.0, 2.0, -1.0, 4.0]), lo[None], hi[None], 1.0)[0]) == 0.5 - 2.5 - 3.0
    bad = np.zeros((64, d))
    bad[5, 2] = np.inf
    lo, hi = E.block_box(bad)
    assert np.all(np.isnan(lo)) and np.all(np.isnan(hi))
    assert np.isnan(E.quest_bound(np.ones(d), lo[None], hi[None], s)[0])


def pin_quest_bruteforce(E, seeds=range(3)):
    """Quest-screen sets, bounds and outputs equal the per-key brute force."""
    variants = [dict(n=2, lens=(200, 128), h_q=4, h_kv=2, d=8, dtype="bf16", mode="learned"),
                dict(n=1, lens=(320,), h_q=2, h_kv=1, d=4, dtype="f32", mode="calibrated"),
                dict(n=2, lens=(130, 256), h_q=2, h_kv=2, d=8, dtype="bf16", mode="calibrated", lwb=1)]
    for seed in seeds:
        wl = tiny(80 + seed, **variants[seed % len(variants)])
        # thresholds at the median box bound of each head (a number only)
        zero = _decode(E, wl, bias=np.zeros(wl.h_q, np.float32), bound="quest", with_output=False)
        wl.bias = np.array([np.nanmedian(zero.ub[:, h] - zero.tau[:, h, None]) for h in range(wl.h_q)],
                           dtype=np.float32)
        res = _decode(E, wl, bound="quest")
        assert 0 < res.admitted.sum() < res.admitted.size
        bf, bf_union = bruteforce.decode(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table,
                                         wl.seq_lens, wl.q, wl.tau_mode, wl.w, wl.bias, wl.a,
                                         wl.beta, wl.lwb, bound="quest")
        for (n, h), r in bf.items():
            got = sorted(np.nonzero(res.admitted[n, h])[0].tolist())
            assert got == r["admitted"], (seed, n, h, got, r["admitted"])
            assert bool(res.rescued[n, h]) == r["rescued"]
            np.testing.assert_allclose(res.ub[n, h, :len(r["ub"])], r["ub"], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(res.o[n, h], r["o"], rtol=1e-10, atol=1e-12)
        for (n, g), u in bf_union.items():
            assert int(res.union[n, g]) == u


# --------------------------------------------------------------------------- FP8 records
def pin_fp8_rounding_table(E):
    """OCP FP8 rounding by hand: ties to even, the subnormal steps 2^-9 (E4M3)
    and 2^-16 (E5M2), saturation at 448 and 57344."""
    x = np.array([1.0, 1.0625, 1.1875, 460.0, 500.0, -1e6, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11, 0.3,
                  2.0 ** -7 + 2.0 ** -10, -0.0])
    e4m3 = [1.0, 1.0, 1.25, 448.0, 448.0, -448.0, 2.0 ** -9, 0.0, 2.0 ** -9, 0.3125, 2.0 ** -7, -0.0]
    e5m2 = [1.0, 1.0, 1.25, 448.0, 512.0, -57344.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11, 0.3125,
            2.0 ** -7, -0.0]
    assert np.array_equal(E.fp8_round(x, "e4m3"), np.array(e4m3))
    assert np.array_equal(E.fp8_round(x, "e5m2"), np.array(e5m2))
    assert np.signbit(E.fp8_round(np.array([-0.0]), "e4m3")[0])
    assert np.isnan(E.fp8_round(np.array([np.nan]), "e5m2")[0])
    assert E.fp8_round(np.array([2.0 ** -17]), "e5m2")[0] == 0.0          # half the smallest subnormal: even
    assert E.fp8_round(np.array([3 * 2.0 ** -17]), "e5m2")[0] == 2.0 ** -15


def pin_fp8_matches_code_search(E, seed=5):
    """fp8_round agrees with a search over all 256 codes of each format, on
    random magnitudes over the whole range, exact ties and the saturation edge."""
    rng = np.random.default_rng(seed)
    for fmt in ("e4m3", "e5m2"):
        vals = sorted(set(bruteforce.fp8_values(fmt).values()))
        mids = [(a + b) / 2 for a, b in zip(vals, vals[1:])]
        x = np.concatenate([rng.normal(0, 1, 200) * 2.0 ** rng.integers(-18, 17, 200), np.array(mids[::7]),
                            np.array(vals[::9]), np.array([1e9, -1e9])])
        got = E.fp8_round(x, fmt)
        want = np.array([bruteforce.fp8_nearest(float(v), fmt) for v in x])
        assert np.array_equal(got, want), (fmt, x[got != want][:5], got[got != want][:5], want[got != want][:5])


def pin_fp8_bound_sound(E, seed=9, trials=100):
    """The geometric bound over FP8 records is never below a key's logit, its
    radius is the farthest key's distance to the stored centroid (attained by
    some key), and it is exact for a block of one repeated FP8-exact key."""
    rng = np.random.default_rng(seed)
    d = 16
    s = 1.0 / math.sqrt(d)
    for _ in range(trials):
        kb = rng.normal(0, 1, (64, d)) + rng.normal(0, 2, d)
        q = rng.normal(0, 1, d)
        for fmt in ("e4m3", "e5m2"):
            mu, R = E.block_summary_fp8(kb, fmt)
            assert np.array_equal(mu, E.fp8_round(kb.mean(axis=0), fmt))
            dist = [math.sqrt(math.fsum((float(kb[t, c]) - float(mu[c])) ** 2 for c in range(d))) for t in range(64)]
            assert abs(R - max(dist)) <= 1e-12 * max(dist)
            ub = float(E.block_bound(q, mu[None], np.array([R]), s)[0])
            assert ub >= s * float((kb @ q).max()) - 1e-12
    k = np.array([0.5, -1.25, 3.0, 0.0] * 4)
    mu, R = E.block_summary_fp8(np.tile(k, (64, 1)), "e4m3")
    assert np.array_equal(mu, k) and R == 0.0
    bad = np.zeros((64, d))
    bad[3, 3] = np.nan
    mu, R = E.block_summary_fp8(bad, "e5m2")
    assert np.all(mu == 0.0) and R == math.inf


def pin_fp8_bruteforce(E, seeds=range(2)):
    """Sets, bounds and outputs of the geometric screen over FP8 records equal
    the per-key brute force (its own code-search rounding)."""
    variants = [dict(n=2, lens=(200, 128), h_q=4, h_kv=2, d=8, dtype="bf16", mode="learned"),
                dict(n=1, lens=(320,), h_q=2, h_kv=1, d=4, dtype="f32", mode="calibrated")]
    for seed in seeds:
        fmt = ("e4m3", "e5m2")[seed % 2]
        wl = tiny(90 + seed, **variants[seed % len(variants)])
        zero = _decode(E, wl, bias=np.zeros(wl.h_q, np.float32), bound="geometric_fp8", fp8=fmt,
                       with_output=False)
        wl.bias = np.array([np.nanmedian(zero.ub[:, h] - zero.tau[:, h, None]) for h in range(wl.h_q)],
                           dtype=np.float32)
        res = _decode(E, wl, bound="geometric_fp8", fp8=fmt)
        assert 0 < res.admitted.sum() < res.admitted.size
        bf, bf_union = bruteforce.decode(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table,
                                         wl.seq_lens, wl.q, wl.tau_mode, wl.w, wl.bias, wl.a,
                                         wl.beta, wl.lwb, bound="geometric_fp8", fp8=fmt)
        for (n, h), r in bf.items():
            got = sorted(np.nonzero(res.admitted[n, h])[0].tolist())
            assert got == r["admitted"], (seed, n, h, got, r["admitted"])
            np.testing.assert_allclose(res.ub[n, h, :len(r["ub"])], r["ub"], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(res.o[n, h], r["o"], rtol=1e-10, atol=1e-12)
        for (n, g), u in bf_union.items():
            assert int(res.union[n, g]) == u


# --------------------------------------------------------------------------- smaller screen blocks
def pin_subblock_bruteforce(E, seeds=range(4)):
    """Screens on 16- and 32-token blocks: sets, bounds, rescue, token counts,
    outputs and union counts equal the per-key brute force at that block size."""
    variants = [dict(n=2, lens=(200, 128), h_q=4, h_kv=2, d=8, dtype="bf16", mode="learned"),
                dict(n=1, lens=(150,), h_q=2, h_kv=1, d=4, dtype="f32", mode="calibrated", lwb=2),
                dict(n=2, lens=(77, 96), h_q=2, h_kv=2, d=8, dtype="bf16", mode="learned"),
                dict(n=1, lens=(300,), h_q=4, h_kv=1, d=4, dtype="f32", mode="learned", lwb=1)]
    for seed in seeds:
        block = (16, 32)[seed % 2]
        wl = tiny(110 + seed, **variants[seed % len(variants)])
        zero = E.decode_blocks(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, wl.q, wl.tau_mode,
                               wl.w, np.zeros(wl.h_q, np.float32), wl.a, wl.beta, wl.lwb, block, with_output=False)
        wl.bias = np.array([np.nanmedian(zero.ub[:, h] - zero.tau[:, h, None]) for h in range(wl.h_q)],
                           dtype=np.float32)
        res = E.decode_blocks(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, wl.q, wl.tau_mode,
                              wl.w, wl.bias, wl.a, wl.beta, wl.lwb, block)
        bf, bf_union = bruteforce.decode(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table,
                                         wl.seq_lens, wl.q, wl.tau_mode, wl.w, wl.bias, wl.a,
                                         wl.beta, wl.lwb, block=block)
        for (n, h), r in bf.items():
            got = sorted(np.nonzero(res.admitted[n, h])[0].tolist())
            assert got == r["admitted"], (seed, block, n, h, got, r["admitted"])
            assert bool(res.rescued[n, h]) == r["rescued"]
            assert int(res.tokens[n, h]) == r["tokens"]
            np.testing.assert_allclose(res.ub[n, h, :len(r["ub"])], r["ub"], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(res.o[n, h], r["o"], rtol=1e-10, atol=1e-12)
        for (n, g), u in bf_union.items():
            assert int(res.union[n, g]) == u


def pin_subblock_no_false_negatives(E, seeds=range(3)):
    """Every key whose logit reaches its head's threshold lies in an admitted
    16-token block (the bound is sound at any block size)."""
    for seed in seeds:
        wl = tiny(120 + seed, n=2, lens=(256, 190), h_q=4, h_kv=2, d=8, dtype="bf16", mode="learned")
        res = E.decode_blocks(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, wl.q, wl.tau_mode,
                              wl.w, wl.bias, wl.a, wl.beta, wl.lwb, 16, with_output=False)
        for n in range(wl.n_seqs):
            T = int(wl.seq_lens[n])
            for h in range(wl.h_q):
                g = h // wl.group
                for t in range(T):
                    k = E.upcast(wl.k_pages[wl.block_table[n, t // 64], g, t % 64], wl.kv_dtype)
                    S = float(E.upcast(wl.q[n, h], wl.kv_dtype) @ k) / math.sqrt(wl.d)
                    if S >= res.tau[n, h]:
                        assert res.admitted[n, h, t // 16], (seed, n, h, t)


def pin_pairblock_bruteforce(E, seeds=range(4)):
    """Screens on 128-token blocks (two consecutive block-table entries each,
    pages in a random physical order): sets, bounds, rescue, token counts,
    outputs and union counts equal the per-key brute force at b = 128. One
    head's threshold lies above every bound, so with no partial block its
    rescue decides its set."""
    variants = [dict(n=2, lens=(700, 384), h_q=4, h_kv=2, d=8, dtype="bf16", mode="learned"),
                dict(n=1, lens=(1000,), h_q=2, h_kv=1, d=4, dtype="f32", mode="calibrated", lwb=2),
                dict(n=3, lens=(129, 255, 64), h_q=2, h_kv=2, d=8, dtype="bf16", mode="learned", lwb=1),
                dict(n=2, lens=(256, 640), h_q=4, h_kv=1, d=4, dtype="f32", mode="learned")]
    for seed in seeds:
        v = variants[seed % len(variants)]
        wl = tiny(130 + seed, paged=True, **v)
        zero = E.decode_blocks(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, wl.q, wl.tau_mode,
                               wl.w, np.zeros(wl.h_q, np.float32), wl.a, wl.beta, wl.lwb, 128, with_output=False)
        off = [zero.ub[:, h] - zero.tau[:, h, None] for h in range(wl.h_q)]
        wl.bias = np.array([np.nanmedian(o) if np.isfinite(o).any() else 0.0 for o in off], dtype=np.float32)
        if v["lens"] == (256, 640):
            wl.bias[0] = np.float32(np.nanmax(off[0]) + 5.0)
        res = E.decode_blocks(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, wl.q, wl.tau_mode,
                              wl.w, wl.bias, wl.a, wl.beta, wl.lwb, 128)
        bf, bf_union = bruteforce.decode(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table,
                                         wl.seq_lens, wl.q, wl.tau_mode, wl.w, wl.bias, wl.a,
                                         wl.beta, wl.lwb, block=128)
        for (n, h), r in bf.items():
            got = sorted(np.nonzero(res.admitted[n, h])[0].tolist())
            assert got == r["admitted"], (seed, n, h, got, r["admitted"])
            assert bool(res.rescued[n, h]) == r["rescued"]
            assert int(res.tokens[n, h]) == r["tokens"]
            np.testing.assert_allclose(res.ub[n, h, :len(r["ub"])], r["ub"], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(res.o[n, h], r["o"], rtol=1e-10, atol=1e-12)
        for (n, g), u in bf_union.items():
            assert int(res.union[n, g]) == u
        if v["lens"] == (256, 640):
            assert res.rescued[:, 0].all()


def pin_pairblock_no_false_negatives(E, seeds=range(2)):
    """Every key whose logit reaches its head's threshold lies in an admitted
    128-token block."""
    for seed in seeds:
        wl = tiny(140 + seed, n=2, lens=(900, 450), h_q=4, h_kv=2, d=8, dtype="bf16", mode="learned", paged=True)
        res = E.decode_blocks(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, wl.q, wl.tau_mode,
                              wl.w, wl.bias, wl.a, wl.beta, wl.lwb, 128, with_output=False)
        hits = 0
        for n in range(wl.n_seqs):
            T = int(wl.seq_lens[n])
            for h in range(wl.h_q):
                g = h // wl.group
                for t in range(T):
                    k = E.upcast(wl.k_pages[wl.block_table[n, t // 64], g, t % 64], wl.kv_dtype)
                    S = float(E.upcast(wl.q[n, h], wl.kv_dtype) @ k) / math.sqrt(wl.d)
                    if S >= res.tau[n, h]:
                        hits += 1
                        assert res.admitted[n, h, t // 128], (seed, n, h, t)
        assert hits > 0


# --------------------------------------------------------------------------- offline calibration
def _grid_trace(E, T=8, d=4):
    """One sequence whose scaled scores are S_ts = s exactly: q_t = (sqrt(d), 0, ...)
    and k_s = (s, 0, ...), float32 storage."""
    wl = tiny(5, n=1, lens=(T,), h_q=1, h_kv=1, d=d, dtype="f32", mode="calibrated")
    page = wl.block_table[0, 0]
    wl.k_pages[page, 0] = 0.0
    wl.k_pages[page, 0, :T, 0] = np.arange(T, dtype=np.float32)
    q = np.zeros((1, 64, 1, d), dtype=np.float32)
    q[0, :T, 0, 0] = math.sqrt(d)
    return wl, q


def pin_calibration_grid(E):
    """Scores 0..t in row t, bins of width 1 over [0, T): bin b holds the weight
    of every row t >= b; the tails and the binary search follow by hand."""
    T = 8
    wl, q = _grid_trace(E, T)
    hist, above, total = E.calibration_histogram(wl.k_pages, "f32", wl.block_table, wl.seq_lens, q, 0, 1,
                                                 0.0, float(T), T, w_h=np.zeros(4), b_h=3.5)
    W = [(1 << 31) // (t + 1) for t in range(T)]
    want = [sum(W[t] for t in range(b, T)) for b in range(T)]
    assert hist.tolist() == want
    assert total == sum(W[t] * (t + 1) for t in range(T))
    # threshold 3.5: row t has max(0, t - 3) scores at or above it; so has 4.0
    # (a score equal to the threshold counts)
    assert above == sum(W[t] * max(0, t - 3) for t in range(T))
    _, above4, _ = E.calibration_histogram(wl.k_pages, "f32", wl.block_table, wl.seq_lens, q, 0, 1,
                                           0.0, float(T), T, w_h=np.zeros(4), b_h=4.0)
    assert above4 == above
    tails = [sum(want[b:]) for b in range(T + 1)]
    for target in (0, tails[5], tails[5] + 1, tails[1] - 1, tails[0]):
        b = E.calibrated_bin(hist, target)
        assert tails[b] <= target and (b == 0 or tails[b - 1] > target), (target, b)
    # the constant threshold 3.5 is recovered as the next bin edge, 4
    res = E.calibrate(wl.k_pages, "f32", wl.block_table, wl.seq_lens, q, 1, 0.0, float(T), T,
                      w=np.zeros((1, 4)), b=np.array([3.5]))
    assert res[0]["c"] == 4.0


def pin_calibration_nonfinite_key(E):
    """The grid trace with key 5 not finite (its first coordinate NaN): every
    score against it (rows t >= 5) is NaN. By hand: those scores leave bin 5,
    which held nothing else, and land in bin 0; the total weight is
    unchanged; and a NaN score is never at or above a threshold."""
    T = 8
    wl, q = _grid_trace(E, T)
    wl.k_pages[wl.block_table[0, 0], 0, 5, 0] = np.nan
    hist, above, total = E.calibration_histogram(wl.k_pages, "f32", wl.block_table, wl.seq_lens, q, 0, 1,
                                                 0.0, float(T), T, w_h=np.zeros(4), b_h=3.5)
    W = [(1 << 31) // (t + 1) for t in range(T)]
    clean = [sum(W[t] for t in range(b, T)) for b in range(T)]
    moved = sum(W[t] for t in range(5, T))
    want = list(clean)
    want[5] -= moved
    want[0] += moved
    assert want[5] == 0
    assert hist.tolist() == want
    assert total == sum(W[t] * (t + 1) for t in range(T))
    assert above == sum(W[t] * (max(0, t - 3) - (1 if t >= 5 else 0)) for t in range(T))


def pin_calibration_row_weighting(E):
    """Every row weighs about 2^31 whatever its length: two sequences whose rows
    each have exactly half of their scores at or above 0 give a density of 1/2
    at c = 0, though the long sequence has far more scores."""
    d = 4
    wl = tiny(6, n=2, lens=(4, 64), h_q=1, h_kv=1, d=d, dtype="f32", mode="calibrated")
    q = np.zeros((2, 64, 1, d), dtype=np.float32)
    for n, T in enumerate((4, 64)):
        page = wl.block_table[n, 0]
        wl.k_pages[page, 0] = 0.0
        wl.k_pages[page, 0, :T, 0] = np.where(np.arange(T) % 2 == 0, 1.0, -1.0)
        q[n, :T, 0, 0] = math.sqrt(d)
    hist, _, total = E.calibration_histogram(wl.k_pages, "f32", wl.block_table, wl.seq_lens, q, 0, 1,
                                             -2.0, 2.0, 4)
    W = lambda t: (1 << 31) // (t + 1)  # noqa: E731
    pos = sum(W(t) * (t // 2 + 1) for T in (4, 64) for t in range(T))
    assert int(hist[2:].sum()) == pos and int(hist[:2].sum()) == total - pos
    frac = pos / total
    rows = sum((t // 2 + 1) / (t + 1) for T in (4, 64) for t in range(T)) / 68
    assert abs(frac - rows) < 1e-6  # the row average, not the key count average


def pin_calibration_target_property(E, seed=11):
    """On a random trace the returned edge satisfies the search's definition,
    and a larger density target gives a constant no larger."""
    wl = tiny(seed, n=2, lens=(300, 170), h_q=4, h_kv=2, d=8, dtype="bf16", mode="learned")
    q = W.trace_queries(wl, seed=3)
    prev = None
    for rho in (0.05, 0.2, 0.5, 0.9):
        res = E.calibrate(wl.k_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, q, wl.h_kv, -8.0, 8.0, 256,
                          rho=np.full(wl.h_q, rho))
        for h, r in res.items():
            tail = np.concatenate([np.cumsum(r["hist"][::-1])[::-1], [0]])
            assert tail[r["bin"]] <= r["target"] and (r["bin"] == 0 or tail[r["bin"] - 1] > r["target"])
            if prev is not None:
                assert r["c"] <= prev[h]
        prev = {h: r["c"] for h, r in res.items()}


# --------------------------------------------------------------------------- causal prefill
def _prefill(E, wl, q, bias=None, mode=None, **kw):
    return E.prefill(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, q, mode or wl.tau_mode,
                     wl.w, wl.bias if bias is None else bias, wl.a, wl.beta, **kw)


def pin_prefill_causal_sdpa(E):
    """tau~ = -inf: every position is textbook causal softmax attention (torch
    SDPA with is_causal, fp64, grouped-query heads)."""
    import torch
    wl = tiny(21, n=2, lens=(150, 97), h_q=4, h_kv=2, d=8, dtype="bf16", mode="calibrated",
              bias=np.full(4, -np.inf, dtype=np.float32))
    q = W.trace_queries(wl, seed=2)
    o = _prefill(E, wl, q)
    for n in range(wl.n_seqs):
        T = int(wl.seq_lens[n])
        nb = -(-T // 64)
        pages = wl.block_table[n, :nb]
        f64 = lambda x: W.storage_to_f32(x, wl.kv_dtype).astype(np.float64)  # noqa: E731
        K = f64(wl.k_pages[pages]).transpose(1, 0, 2, 3).reshape(wl.h_kv, nb * 64, wl.d)[:, :T]
        V = f64(wl.v_pages[pages]).transpose(1, 0, 2, 3).reshape(wl.h_kv, nb * 64, wl.d)[:, :T]
        Q = f64(q[n, :T]).transpose(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(np.ascontiguousarray(Q))[None], torch.from_numpy(np.ascontiguousarray(K))[None],
            torch.from_numpy(np.ascontiguousarray(V))[None], is_causal=True, enable_gqa=True)[0].numpy()
        np.testing.assert_allclose(o[n, :T].transpose(1, 0, 2), ref, rtol=1e-10, atol=1e-12)


def pin_prefill_prefix_means(E):
    """tau~ far above every logit: every logit is filtered to 0 and position t
    returns the plain mean of v_0 .. v_t (the uniform floor, prefix by prefix)."""
    wl = tiny(22, n=1, lens=(130,), h_q=2, h_kv=1, d=8, dtype="f32", mode="calibrated",
              bias=np.full(2, 1e4, dtype=np.float32))
    q = W.trace_queries(wl, seed=4)
    o = _prefill(E, wl, q)
    V = wl.v_pages[wl.block_table[0, :3], 0].astype(np.float64).reshape(-1, wl.d)[:130]
    want = np.cumsum(V, axis=0) / np.arange(1, 131)[:, None]
    for h in range(2):
        np.testing.assert_allclose(o[0, :130, h], want, rtol=1e-12, atol=1e-14)


def pin_prefill_last_row_is_decode(E):
    """The last position of a prompt is one decode step with every block
    admitted: the prefill row equals the decode oracle with lwb >= blocks."""
    wl = tiny(23, n=2, lens=(200, 64), h_q=4, h_kv=2, d=8, dtype="bf16", mode="learned")
    q = W.trace_queries(wl, seed=6)
    o = _prefill(E, wl, q)
    for n in range(wl.n_seqs):
        T = int(wl.seq_lens[n])
        qd = q[:, T - 1].copy()
        res = E.decode(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, qd, wl.tau_mode, wl.w,
                       wl.bias, wl.a, wl.beta, lwb=10 ** 6)
        np.testing.assert_allclose(o[n, T - 1], res.o[n], rtol=1e-10, atol=1e-12)


def pin_prefill_bruteforce(E):
    """Every position of a tiny prompt against a per-element pure-Python loop."""
    wl = tiny(24, n=1, lens=(70,), h_q=2, h_kv=1, d=4, dtype="f32", mode="learned", beta=2.0, a=0.3)
    q = W.trace_queries(wl, seed=8)
    o = _prefill(E, wl, q)
    sel = (1, 37, 64)  # the row-selection path computes the chosen rows alone
    o_sel = E.prefill(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, q, wl.tau_mode, wl.w,
                      wl.bias, wl.a, wl.beta, positions=sel + (500,))
    assert np.all(np.isnan(np.delete(o_sel[0], sel, axis=0)))
    s = 1.0 / math.sqrt(wl.d)
    page = [int(x) for x in wl.block_table[0, :2]]
    key = lambda t: [float(x) for x in wl.k_pages[page[t // 64], 0, t % 64]]  # noqa: E731
    val = lambda t: [float(x) for x in wl.v_pages[page[t // 64], 0, t % 64]]  # noqa: E731
    for h in range(2):
        for t in (0, 1, 37, 63, 64, 69):
            qt = [float(x) for x in q[0, t, h]]
            tau = math.fsum(float(wl.w[h][c]) * qt[c] for c in range(wl.d)) + float(wl.bias[h]) - wl.a
            logits = []
            for u in range(t + 1):
                S = s * math.fsum(qt[c] * key(u)[c] for c in range(wl.d))
                logits.append(S / (1.0 + math.exp(-wl.beta * (S - tau))))
            m = max(logits)
            wts = [math.exp(x - m) for x in logits]
            den = math.fsum(wts)
            want = [math.fsum(wts[u] * val(u)[c] for u in range(t + 1)) / den for c in range(wl.d)]
            np.testing.assert_allclose(o[0, t, h], want, rtol=1e-11, atol=1e-13)
            if t in sel:
                np.testing.assert_allclose(o_sel[0, t, h], want, rtol=1e-11, atol=1e-13)

def pin_prefill_future_value_excluded(E):
    """Causality with a non-finite value: row t depends only on the keys s <= t
    (Section 2.2, E.1), so a non-finite element i of v_s leaves every row
    t < s exactly as it is with a finite value there, and makes element i of
    every row t >= s non-finite (its weight is positive) while the other
    elements stay as they were."""
    wl = tiny(25, n=1, lens=(150,), h_q=2, h_kv=1, d=8, dtype="f32", mode="learned")
    q = W.trace_queries(wl, seed=10)
    s_tok, i = 70, 5
    page, row = int(wl.block_table[0, s_tok // 64]), s_tok % 64
    wl.v_pages[page, 0, row, i] = 0.25
    base = _prefill(E, wl, q)
    for bad in (np.inf, -np.inf, np.nan):
        wl.v_pages[page, 0, row, i] = bad
        o = _prefill(E, wl, q)
        assert np.array_equal(o[0, :s_tok], base[0, :s_tok])
        assert not np.isfinite(o[0, s_tok:150, :, i]).any()
        others = [c for c in range(wl.d) if c != i]
        assert np.array_equal(o[0, s_tok:150][..., others], base[0, s_tok:150][..., others])
    wl.v_pages[page, 0, row, i] = 0.25


# --------------------------------------------------------------------------- thresholds
def pin_threshold_closed_form(E):
    """tau~ = w.q + b - a (learned), c - a (calibrated): Sections 1, 4.7, D.1, G.1."""
    q = np.array([2.0, -1.0, 0.5, 0.0])
    w = np.array([3.0, 1.0, 4.0, 7.0])
    assert abs(E.threshold("learned", q, w, 0.25, 0.4) - (6.0 - 1.0 + 2.0 + 0.25 - 0.4)) < 1e-15
    assert abs(E.threshold("calibrated", q, w, 1.5, 0.4) - 1.1) < 1e-15
    assert E.threshold("learned", q, np.zeros(4), -8.0, 0.0) == -8.0


# --------------------------------------------------------------------------- whole step
def pin_bruteforce(E, seeds=range(6)):
    """Sets, counts, rescue flags and outputs equal the per-key brute force."""
    variants = [
        dict(n=2, lens=(200, 128), h_q=4, h_kv=2, d=8, dtype="bf16", mode="learned"),
        dict(n=1, lens=(300,), h_q=2, h_kv=1, d=4, dtype="f32", mode="calibrated", lwb=2),
        dict(n=3, lens=(64, 65, 191), h_q=4, h_kv=1, d=8, dtype="bf16", mode="learned", a=0.4),
        dict(n=1, lens=(256,), h_q=1, h_kv=1, d=64, dtype="f32", mode="calibrated"),
        dict(n=2, lens=(128, 70), h_q=2, h_kv=2, d=8, dtype="f32", mode="learned", beta=1.0, lwb=1),
        dict(n=1, lens=(192,), h_q=4, h_kv=2, d=4, dtype="bf16", mode="calibrated",
             bias=[1e4, 1e4, 1e4, 1e4]),  # forces the rescue path
    ]
    for seed in seeds:
        v = dict(variants[seed % len(variants)])
        wl = tiny(seed, **v)
        res = _decode(E, wl)
        bf, bf_union = bruteforce.decode(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table,
                                         wl.seq_lens, wl.q, wl.tau_mode, wl.w, wl.bias, wl.a,
                                         wl.beta, wl.lwb)
        for (n, h), r in bf.items():
            got = sorted(np.nonzero(res.admitted[n, h])[0].tolist())
            assert got == r["admitted"], (seed, n, h, got, r["admitted"])
            assert bool(res.rescued[n, h]) == r["rescued"], (seed, n, h)
            assert int(res.tokens[n, h]) == r["tokens"]
            assert int(res.per_head[n, h]) == len(r["admitted"])
            assert abs(res.tau[n, h] - r["tau"]) <= 1e-12 * (1 + abs(r["tau"]))
            np.testing.assert_allclose(res.o[n, h], r["o"], rtol=1e-10, atol=1e-12)
        for (n, g), u in bf_union.items():
            assert int(res.union[n, g]) == u


def pin_no_false_negatives(E, seeds=range(4)):
    """Section 3.1: a block holding a key with S >= tau~ is significant; the
    screen must admit every significant block."""
    for seed in seeds:
        wl = tiny(100 + seed, n=2, lens=(640, 300), h_q=4, h_kv=2, d=8, density=0.3)
        # raise a few keys above their head's threshold
        res0 = _decode(E, wl, with_output=False)
        rng = np.random.default_rng(seed)
        for _ in range(6):
            n = int(rng.integers(2))
            h = int(rng.integers(4))
            t = int(rng.integers(int(wl.seq_lens[n])))
            W.plant_needle(wl, n, h, t, logit=float(res0.tau[n, h]) + 0.5)
        res = _decode(E, wl, with_output=False)
        s = 1.0 / math.sqrt(wl.d)
        for n in range(wl.n_seqs):
            T = int(wl.seq_lens[n])
            for h in range(wl.h_q):
                g = h // wl.group
                qh = W.storage_to_f32(wl.q[n, h], wl.kv_dtype).astype(np.float64)
                for t in range(T):
                    page = wl.block_table[n, t // 64]
                    k = W.storage_to_f32(wl.k_pages[page, g, t % 64], wl.kv_dtype).astype(np.float64)
                    if s * float(k @ qh) >= res.tau[n, h]:
                        assert res.admitted[n, h, t // 64], (seed, n, h, t)


def pin_nesting(E, seed=7):
    """Raising the threshold can only remove blocks (no rescue involved)."""
    wl = tiny(seed, n=1, lens=(64 * 12 + 5,), h_q=2, h_kv=1, d=8, mode="calibrated")
    prev = None
    for c in np.linspace(-1.0, 8.0, 19):
        res = _decode(E, wl, bias=np.full(2, c, dtype=np.float32), with_output=False)
        if prev is not None:
            assert np.all(res.admitted <= prev), c
        prev = res.admitted


def pin_dense_sdpa(E):
    """tau~ = -inf: the gate is the identity and the step is textbook softmax
    attention, checked against torch's scaled_dot_product_attention (fp64,
    grouped-query heads)."""
    import torch
    for seed, (lens, h_q, h_kv, d, dtype) in enumerate([((300, 64, 129), 4, 2, 8, "bf16"),
                                                        ((1000,), 8, 2, 64, "f32")]):
        wl = tiny(seed, n=len(lens), lens=lens, h_q=h_q, h_kv=h_kv, d=d, dtype=dtype,
                  mode="calibrated", bias=np.full(h_q, -np.inf, dtype=np.float32))
        res = _decode(E, wl)
        for n in range(wl.n_seqs):
            T = int(wl.seq_lens[n])
            nb = -(-T // 64)
            pages = wl.block_table[n, :nb]
            f64 = lambda x: W.storage_to_f32(x, dtype).astype(np.float64)  # noqa: E731
            K = f64(wl.k_pages[pages]).transpose(1, 0, 2, 3).reshape(h_kv, nb * 64, d)[:, :T]
            V = f64(wl.v_pages[pages]).transpose(1, 0, 2, 3).reshape(h_kv, nb * 64, d)[:, :T]
            q = f64(wl.q[n])[:, None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q)[None], torch.from_numpy(np.ascontiguousarray(K))[None],
                torch.from_numpy(np.ascontiguousarray(V))[None], enable_gqa=True)[0, :, 0].numpy()
            np.testing.assert_allclose(res.o[n], ref, rtol=1e-10, atol=1e-12)
            assert res.admitted[n, :, :nb].all()


def pin_suppressed_mean(E):
    """tau~ far above every logit: each logit is filtered to 0, every weight is
    exp(0) = 1 and o is the plain mean of the retained values (Section 1's
    uniform floor). With every block forced in, that is the mean over all T
    tokens; with nothing admitted and no tail, the rescue keeps one block."""
    wl = tiny(3, n=2, lens=(320, 200), h_q=2, h_kv=1, d=8, dtype="f32", mode="calibrated",
              bias=np.full(2, 1e4, dtype=np.float32), lwb=100)
    res = _decode(E, wl)
    for n in range(2):
        T = int(wl.seq_lens[n])
        nb = -(-T // 64)
        V = wl.v_pages[wl.block_table[n, :nb], 0].astype(np.float64).reshape(-1, 8)[:T]
        for h in range(2):
            np.testing.assert_allclose(res.o[n, h], V.mean(axis=0), rtol=1e-12, atol=1e-14)
    wl = tiny(4, n=1, lens=(320,), h_q=2, h_kv=1, d=8, dtype="f32", mode="calibrated",
              bias=np.full(2, 1e4, dtype=np.float32), lwb=0)
    res = _decode(E, wl)
    for h in range(2):
        assert res.rescued[0, h] and res.per_head[0, h] == 1
        j = int(np.nonzero(res.admitted[0, h])[0][0])
        assert j == int(np.argmax(res.ub[0, h, :5]))
        V = wl.v_pages[wl.block_table[0, j], 0].astype(np.float64)
        np.testing.assert_allclose(res.o[0, h], V.mean(axis=0), rtol=1e-12, atol=1e-14)


def pin_equal_logits(E):
    """All keys equal: every logit is equal, o is the mean of the retained
    values whatever tau and beta are; all bounds tie, so with nothing admitted
    the rescue takes block 0 (lowest index)."""
    d = 8
    wl = tiny(5, n=1, lens=(64 * 6,), h_q=1, h_kv=1, d=d, dtype="f32", mode="calibrated")
    key = np.linspace(-1, 1, d).astype(np.float32)
    wl.k_pages[:] = key
    for c, expect_all in ((-50.0, True), (50.0, False)):
        res = _decode(E, wl, bias=np.array([c], dtype=np.float32))
        if expect_all:
            assert res.per_head[0, 0] == 6
            V = wl.v_pages[wl.block_table[0, :6], 0].astype(np.float64).reshape(-1, d)
        else:
            assert res.rescued[0, 0] and res.admitted[0, 0, 0] and res.per_head[0, 0] == 1
            V = wl.v_pages[wl.block_table[0, 0], 0].astype(np.float64)
        np.testing.assert_allclose(res.o[0, 0], V.mean(axis=0), rtol=1e-12, atol=1e-14)


def pin_two_keys_closed_form(E):
    """A hand-built block: one key exactly at the threshold (S = tau, gate 1/2),
    63 keys at logit 0 (weight 1). o = (e^{tau/2} v0 + sum v_t) / (e^{tau/2} + 63)."""
    d = 4
    tau = 3.0
    wl = tiny(6, n=1, lens=(64,), h_q=1, h_kv=1, d=d, dtype="f32", mode="calibrated",
              bias=np.array([tau], dtype=np.float32), lwb=1)
    wl.q[0, 0] = np.array([2.0, 0.0, 0.0, 0.0], dtype=np.float32)  # s = 1/2: S = k[0]
    page = wl.block_table[0, 0]
    wl.k_pages[page, 0] = 0.0
    wl.k_pages[page, 0, 17, 0] = tau
    wl.k_pages[page, 0, :, 1:] = 5.0  # orthogonal to q: logits unaffected
    res = _decode(E, wl)
    V = wl.v_pages[page, 0].astype(np.float64)
    e = math.exp(tau / 2)
    want = (e * V[17] + V.sum(axis=0) - V[17]) / (e + 63.0)
    np.testing.assert_allclose(res.o[0, 0], want, rtol=1e-13, atol=1e-15)


def pin_tail_masking(E):
    """Rows of the last page past the sequence end are not tokens (F.4): junk
    there (NaN) changes nothing."""
    wl = tiny(8, n=2, lens=(130, 77), h_q=2, h_kv=1, d=8, dtype="f32", mode="calibrated")
    res_nan = _decode(E, wl)
    for n in range(2):
        T = int(wl.seq_lens[n])
        page = wl.block_table[n, T // 64]
        wl.k_pages[page, :, T % 64:] = 0.0
        wl.v_pages[page, :, T % 64:] = 0.0
    res0 = _decode(E, wl)
    assert np.all(np.isfinite(res_nan.o))
    assert np.array_equal(res_nan.o, res0.o)


def pin_page_permutation(E):
    """The physical page order is invisible: same sets, same outputs."""
    wl = tiny(9, n=2, lens=(400, 333), h_q=4, h_kv=2, d=8)
    wl2 = W.permute_pages(wl, seed=3)
    r1 = _decode(E, wl)
    r2 = _decode(E, wl2)
    assert np.array_equal(r1.admitted, r2.admitted)
    assert np.array_equal(r1.o, r2.o)


def pin_nonfinite_keys(E):
    """A block with a non-finite key has R = inf and is admitted for any
    finite threshold, also for a zero query (bound NaN)."""
    wl = tiny(10, n=1, lens=(256,), h_q=1, h_kv=1, d=8, dtype="f32", mode="calibrated",
              bias=np.array([1e3], dtype=np.float32))
    wl.k_pages[wl.block_table[0, 2], 0, 5, 3] = np.inf
    res = _decode(E, wl, with_output=False)
    assert res.admitted[0, 0, 2] and res.per_head[0, 0] == 1 and not res.rescued[0, 0]
    wl.q[:] = 0.0
    res = _decode(E, wl, with_output=False)
    assert res.admitted[0, 0, 2]


def pin_threshold_tie_admitted(E):
    """Section 3.1 counts a key with S >= tau as significant, so a block whose
    bound equals tau~ exactly is admitted. Exact construction: keys equal to a
    float16-representable vector (centroid exact, R = 0), s = 1/2."""
    wl = tiny(11, n=1, lens=(128,), h_q=1, h_kv=1, d=4, dtype="f32", mode="calibrated",
              bias=np.array([1.5], dtype=np.float32))
    wl.q[0, 0] = np.array([2.0, 0.0, 0.0, 0.0], dtype=np.float32)
    wl.k_pages[:] = 0.0
    wl.k_pages[wl.block_table[0, 1], 0, :, 0] = 1.5   # UB = 0.5 * 2 * 1.5 = 1.5 = tau
    wl.k_pages[wl.block_table[0, 0], 0, :, 0] = 1.0   # UB = 1.0 < tau
    res = _decode(E, wl, with_output=False)
    assert res.ub[0, 0, 1] == 1.5 and res.tau[0, 0] == 1.5
    assert res.admitted[0, 0, 1] and not res.admitted[0, 0, 0] and not res.rescued[0, 0]


ALL_PINS = [
    pin_sigmoid_convention, pin_gate_closed_forms, pin_fp16_rne, pin_bound_sound_and_tight,
    pin_threshold_closed_form, pin_bruteforce, pin_no_false_negatives, pin_nesting,
    pin_dense_sdpa, pin_suppressed_mean, pin_equal_logits, pin_two_keys_closed_form,
    pin_tail_masking, pin_page_permutation, pin_nonfinite_keys, pin_threshold_tie_admitted,
    pin_sigma_rne, pin_dual_closed_form, pin_dual_within_geometric, pin_dual_bruteforce,
    pin_calibration_grid, pin_calibration_row_weighting, pin_calibration_target_property,
    pin_calibration_nonfinite_key,
    pin_prefill_causal_sdpa, pin_prefill_prefix_means, pin_prefill_last_row_is_decode, pin_prefill_bruteforce,
    pin_prefill_future_value_excluded,
    pin_quest_directed_rounding, pin_quest_box_corners, pin_quest_bruteforce,
    pin_fp8_rounding_table, pin_fp8_matches_code_search, pin_fp8_bound_sound, pin_fp8_bruteforce,
    pin_subblock_bruteforce, pin_subblock_no_false_negatives, pin_pairblock_bruteforce,
    pin_pairblock_no_false_negatives,
]
