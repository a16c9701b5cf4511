"""fp64 CPU oracle of the Elastic Threshold Attention (ETA) decode step.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product path. It shares no code with
the HIP library.

Source: "Elastic Threshold Attention: Learned Contextual Sparsity for
Long-Context Decoding" (paperpeel.com/paper/2609.20888). Section numbers below
refer to that page. The page lost its display equations (the dual bound,
Eq. 7) and the body of the decode algorithm (Algorithm 4); where a step is not
fixed by the surviving text, the reading taken is stated at that step.

What one decode step computes, for sequence n of length T and query head h
served by KV head g = floor(h / G), G = H_Q / H_KV:

  1. threshold      tau~ = w_h . q + b_h - a   (learned)   or   c_h - a
                    (calibrated)  -- Sections 1, 4.7, D.1, G.1.
  2. block record   for each complete 64-token block: centroid mu^ = fp16(mean k)
                    (round to nearest even) and radius R = max_s ||k_s - mu^||_2
                    -- Section 3.2 and F.1 (per-KV-head record of an fp16 centroid
                    and an fp32 scalar norm). Reading: the scalar is the radius of
                    the block's keys about the stored centroid, so that
                    q.k <= q.mu^ + ||q|| R holds for every key (Cauchy-Schwarz).
  3. screen         UB = s (q . mu^ + ||q|| R), s = 1/sqrt(d); a complete block is
                    admitted unless UB < tau~ -- Section 3, 3.1, F.1. The partial
                    last block is always loaded (Section 4.8, F.4) and so are the
                    `lwb` most recent complete blocks (Section 4.8).
  4. rescue         if nothing is admitted, the block with the largest UB (lowest
                    index on ties) is admitted -- Section 3.2, F.4 (read globally,
                    not per chunk).
  5. attention      over every token t < T of the admitted blocks:
                    S = s q . k_t,  S~ = S * sigmoid(beta (S - tau~)),
                    o = sum_t exp(S~_t) v_t / sum_t exp(S~_t)  -- Sections 1, 2.2,
                    E.3, G.1. The sign of the sigmoid argument is the one that
                    reproduces sigma'(8) = 3.35e-4 and sigma'(40) ~ 4.3e-18 of B.1.

All arithmetic is float64 on the stored values (bfloat16 or float32 K/V/q,
upcast exactly); only mu^ is rounded, to float16, because that rounding is
part of the stored record.

Pins (tests, CPU): brute-force per-key enumeration on tiny inputs (sets, counts
and outputs), exact bound soundness, no-false-negative and nesting properties,
dense mode against torch's scaled_dot_product_attention, closed forms for the
all-suppressed, equal-logit and single-key cases, the fp16 rounding mode of
mu^, page-permutation invariance, and the sigmoid convention values of B.1.
Optional dual screen (Sections 3.1 and F.1; Eq. 7 did not survive): each
record also carries the coordinate standard deviation sigma^ (float16), and a
block's score is the smaller of the geometric bound and the probabilistic
estimate s (q . mu^ + z ||q * sigma^||), z = 2 by default (B.1 tables). This
reading is not sound (it can miss a block whose best key lies more than z
deviations out), so its sets are pinned against a per-key brute force and
measured for recall, not checked for soundness.

Offline calibration (Section 4.7, D.2, Algorithm 1): calibration_histogram,
calibrated_bin and calibrate below; the reading taken is stated there.

Causal prefill (prefill below): the same gated rule at every position of a
prompt over the keys up to it, dense (no block pruning), thresholds per
position.

FP8 records (Section 5 lists FP8 metadata quantization as future work; the
reading taken): the block centroid stored in an OCP FP8 format (E4M3, 3
mantissa bits, largest 448; or E5M2, 2 mantissa bits, largest 57344), rounded
to nearest even and saturated at the largest finite value, with the radius
measured about that stored centroid, so the geometric bound stays an upper
bound (fp8_round, block_summary_fp8, decode(bound="geometric_fp8")).

Other screen block sizes (Appendix F.3, Table 10 ablates the block size; the
reading taken): with b = 16 or 32 every 64-token page holds 64/b screen
blocks, each with its own record (centroid and radius of its b keys); with
b = 128 a screen block spans two consecutive entries 2j and 2j + 1 of the
block table and its record (over its 128 keys) is kept with the first of the
two pages. The screen, the forced and rescued blocks, the counts and the
attention all work on b-token blocks (build_summaries_sub, decode_blocks).

Comparator screen (Section 4.3, "Comparison with Quest"): per block and KV
head the coordinate-wise minimum and maximum of the keys, rounded outward to
float16, and the box bound s sum_i max(q_i kmax_i, q_i kmin_i) in place of the
geometric one (block_box, quest_bound, decode(bound="quest")).

Parity unpinned: the pages' exact Eq. 7, the body of Algorithm 1 and their
chunk-local rescue rule are not reproducible from the text; the first two are
implemented as readings, the last is not implemented.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterable, Optional

import numpy as np

BLOCK = 64
_CHUNK_BLOCKS = 256


# --------------------------------------------------------------------------- values
def upcast(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Stored K/V/q values -> float64, exactly."""
    if kv_dtype == "bf16":
        bits = np.asarray(x, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if kv_dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


def sigmoid(x):
    """Logistic function 1/(1+e^-x), evaluated without overflow."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    with np.errstate(over="ignore", invalid="ignore"):
        out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
        ex = np.exp(x[~pos])
        out[~pos] = ex / (1.0 + ex)
    return out


def gate(S, tau: float, beta: float):
    """Centered-SiLU filter of a logit: S * sigmoid(beta (S - tau)).

    Sections 1 and E.3 (multiplicative masking S~ = S . sigma) and G.1 (the
    tempered logit with the effective threshold). Logits well above tau pass
    unchanged; logits well below shrink to 0, i.e. weight exp(0) = 1: the
    uniform floor of Section 1."""
    S = np.asarray(S, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        return S * sigmoid(beta * (S - tau))


# --------------------------------------------------------------------------- block records
def block_summary(kb: np.ndarray):
    """Record of complete blocks: kb is float64 [nb, 64, d] (or [64, d]).

    Returns (mu^, R): mu^ float64 [nb, d] holding float16 values, R float64 [nb].
    mu^ is the fp64 mean rounded to float16 (nearest even); if any coordinate is
    not finite in float16 the centroid is the zero vector. R is the largest
    Euclidean distance of a key to mu^, +inf when it is not finite.
    Section 3.2 and F.1 (fp16 centroid, scalar fp32 norm per block per KV head)."""
    single = kb.ndim == 2
    if single:
        kb = kb[None]
    mean = kb.mean(axis=1)
    with np.errstate(over="ignore", invalid="ignore"):
        mu16 = mean.astype(np.float16).astype(np.float64)
    ok = np.isfinite(mu16).all(axis=1)
    mu = np.where(ok[:, None], mu16, 0.0)
    with np.errstate(over="ignore", invalid="ignore"):
        diff = kb - mu[:, None, :]
        r = np.sqrt((diff * diff).sum(axis=2)).max(axis=1)
    r = np.where(np.isnan(r) | np.isinf(r), np.inf, r)
    if single:
        return mu[0], float(r[0])
    return mu, r


FP8_FORMATS = {
    # mantissa bits, smallest normal exponent, largest finite value (OCP 8-bit formats)
    "e4m3": (3, -6, 448.0),
    "e5m2": (2, -14, 57344.0),
}


def fp8_round(x, fmt: str):
    """Nearest value of the FP8 format (ties to even), saturating at the largest
    finite magnitude; zeros keep their sign, NaN stays NaN. float64 in and out."""
    mbits, emin, vmax = FP8_FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    with np.errstate(invalid="ignore", over="ignore"):
        _, e2 = np.frexp(a)                       # a = f 2^e2, f in [0.5, 1): floor(log2 a) = e2 - 1
        e = np.maximum(e2 - 1, emin)              # binade, the subnormal range sharing the smallest
        quantum = np.ldexp(1.0, (e - mbits).astype(np.int64))
        r = np.minimum(np.round(a / quantum) * quantum, vmax)
        out = np.where(a == 0, x, np.copysign(r, x))
    return out


def block_summary_fp8(kb: np.ndarray, fmt: str):
    """Geometric record with an FP8 centroid: mu8 = fp8_round(mean k) and R8 the
    largest distance of a key to mu8 (+inf when not finite); a block holding a
    non-finite key gets the zero centroid and R8 = +inf. kb float64 [nb, 64, d]
    or [64, d]; returns (mu8 float64 holding FP8 values, R8 float64)."""
    single = kb.ndim == 2
    if single:
        kb = kb[None]
    ok = np.isfinite(kb).all(axis=(1, 2))
    with np.errstate(over="ignore", invalid="ignore"):
        mu8 = np.where(ok[:, None], fp8_round(kb.mean(axis=1), fmt), 0.0)
        off8 = kb - mu8[:, None, :]
        r = np.sqrt((off8 * off8).sum(axis=2)).max(axis=1)
    r = np.where(ok & np.isfinite(r), r, np.inf)
    mu = mu8
    return (mu[0], r[0]) if single else (mu, r)


def build_summaries_fp8(k_pages: np.ndarray, kv_dtype: str, block_table: np.ndarray, seq_lens: np.ndarray,
                        fmt: str):
    """(mu8, R8) for every complete block of every (sequence, KV head); NaN where
    there is none."""
    P, HKV, B, D = k_pages.shape
    mu = np.full((P, HKV, D), np.nan)
    R = np.full((P, HKV), np.nan)
    for n in range(len(seq_lens)):
        nfull = int(seq_lens[n]) // BLOCK
        pages = np.asarray(block_table[n, :nfull], dtype=np.int64)
        for g in range(HKV):
            for j0 in range(0, nfull, _CHUNK_BLOCKS):
                pg = pages[j0:j0 + _CHUNK_BLOCKS]
                mu[pg, g], R[pg, g] = block_summary_fp8(upcast(k_pages[pg, g], kv_dtype), fmt)
    return mu, R


def build_summaries(k_pages: np.ndarray, kv_dtype: str, block_table: np.ndarray,
                    seq_lens: np.ndarray, segments: Optional[Iterable] = None):
    """Records for every complete block of every (sequence, KV head).

    Returns mu float64 [num_pages][H_KV][d] and R float64 [num_pages][H_KV];
    entries of pages that hold no complete block are NaN."""
    P, HKV, B, D = k_pages.shape
    assert B == BLOCK
    mu = np.full((P, HKV, D), np.nan)
    R = np.full((P, HKV), np.nan)
    N = len(seq_lens)
    segs = [(n, g) for n in range(N) for g in range(HKV)] if segments is None else list(segments)
    for (n, g) in segs:
        nfull = int(seq_lens[n]) // BLOCK
        pages = np.asarray(block_table[n, :nfull], dtype=np.int64)
        for j0 in range(0, nfull, _CHUNK_BLOCKS):
            pg = pages[j0:j0 + _CHUNK_BLOCKS]
            kb = upcast(k_pages[pg, g], kv_dtype)
            m, r = block_summary(kb)
            mu[pg, g] = m
            R[pg, g] = r
    return mu, R


# --------------------------------------------------------------------------- screen
def block_sigma(kb: np.ndarray) -> np.ndarray:
    """Coordinate standard deviation of complete blocks (kb float64 [nb, 64, d]):
    population deviation (divide by 64) about the float64 mean, stored as
    float16 with round to nearest even; +inf where it is not finite. Section
    F.1: 64-dimensional coordinate standard deviation in float16 (the deviation
    rather than the variance, which would underflow in half precision)."""
    single = kb.ndim == 2
    if single:
        kb = kb[None]
    with np.errstate(over="ignore", invalid="ignore"):
        mean = kb.mean(axis=1)
        dev = kb - mean[:, None, :]
        sd = np.sqrt((dev * dev).mean(axis=1))
        sd16 = sd.astype(np.float16).astype(np.float64)
    sd16 = np.where(np.isfinite(sd16), sd16, np.inf)
    return sd16[0] if single else sd16


def build_sigmas(k_pages: np.ndarray, kv_dtype: str, block_table: np.ndarray, seq_lens: np.ndarray):
    """sigma^ for every complete block of every (sequence, KV head): float64
    [num_pages][H_KV][d] holding float16 values, NaN where there is none."""
    P, HKV, B, D = k_pages.shape
    sig = np.full((P, HKV, D), np.nan)
    for n in range(len(seq_lens)):
        nfull = int(seq_lens[n]) // BLOCK
        pages = np.asarray(block_table[n, :nfull], dtype=np.int64)
        for g in range(HKV):
            for j0 in range(0, nfull, _CHUNK_BLOCKS):
                pg = pages[j0:j0 + _CHUNK_BLOCKS]
                sig[pg, g] = block_sigma(upcast(k_pages[pg, g], kv_dtype))
    return sig


def f16_round_down(x):
    """Largest float16 value <= x (float64 in, float64 out; -inf below the
    range, NaN stays NaN)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        y = x.astype(np.float16)
        fix = y.astype(np.float64) > x
        y = np.where(fix, np.nextafter(y, np.float16(-np.inf)), y)
    return y.astype(np.float64)


def f16_round_up(x):
    """Smallest float16 value >= x (float64 in, float64 out; +inf above the
    range, NaN stays NaN)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        y = x.astype(np.float16)
        fix = y.astype(np.float64) < x
        y = np.where(fix, np.nextafter(y, np.float16(np.inf)), y)
    return y.astype(np.float64)


def block_box(kb: np.ndarray):
    """Coordinate-wise bounding box of complete blocks (kb float64 [nb, 64, d]
    or [64, d]): kmin rounded down and kmax rounded up to float16, so that every
    key lies inside the stored box (Section 4.3: the per-block minimum and
    maximum of each coordinate that the Quest comparator keeps). A block with a
    non-finite key gets NaN in both, which no threshold excludes."""
    single = kb.ndim == 2
    if single:
        kb = kb[None]
    lo = f16_round_down(kb.min(axis=1))
    hi = f16_round_up(kb.max(axis=1))
    bad = ~np.isfinite(kb).all(axis=(1, 2))
    lo[bad] = np.nan
    hi[bad] = np.nan
    return (lo[0], hi[0]) if single else (lo, hi)


def build_boxes(k_pages: np.ndarray, kv_dtype: str, block_table: np.ndarray, seq_lens: np.ndarray):
    """(kmin, kmax) for every complete block of every (sequence, KV head): float64
    [num_pages][H_KV][d] each, holding float16 values; NaN where there is none."""
    P, HKV, B, D = k_pages.shape
    lo = np.full((P, HKV, D), np.nan)
    hi = np.full((P, HKV, D), np.nan)
    for n in range(len(seq_lens)):
        nfull = int(seq_lens[n]) // BLOCK
        pages = np.asarray(block_table[n, :nfull], dtype=np.int64)
        for g in range(HKV):
            for j0 in range(0, nfull, _CHUNK_BLOCKS):
                pg = pages[j0:j0 + _CHUNK_BLOCKS]
                lo[pg, g], hi[pg, g] = block_box(upcast(k_pages[pg, g], kv_dtype))
    return lo, hi


def quest_bound(q: np.ndarray, kmin: np.ndarray, kmax: np.ndarray, scale: float) -> np.ndarray:
    """Box bound of each block: s sum_i max(q_i kmax_i, q_i kmin_i), the largest
    q.k over the box's corners (Section 4.3). Each term takes the IEEE maximum
    in which a NaN product (0 times an infinite edge) yields to the other; a
    NaN record gives a NaN bound."""
    q = np.asarray(q, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        terms = np.fmax(kmax * q[None, :], kmin * q[None, :])
        return scale * terms.sum(axis=1)


def threshold(mode: str, q_h: np.ndarray, w_h, b_h: float, a: float) -> float:
    """Effective threshold tau~ = tau - a.

    learned:    tau = w_h . q + b_h   (Section 1; D.1: per-head linear predictor)
    calibrated: tau = c_h             (Section 4.7: frozen per-head constant)
    a: threshold adjustment (B.1 tables; G.1 writes tau~ = tau - a)."""
    if mode == "learned":
        return float(np.dot(np.asarray(w_h, dtype=np.float64), np.asarray(q_h, dtype=np.float64))) \
            + float(b_h) - float(a)
    if mode == "calibrated":
        return float(b_h) - float(a)
    raise ValueError(f"unknown threshold mode {mode!r}")


def block_bound(q: np.ndarray, mu: np.ndarray, R: np.ndarray, scale: float) -> np.ndarray:
    """Upper bound on the scaled logit s q.k of every key of each block:
    s (q . mu^ + ||q||_2 R). Reading of the geometric block bound of Section 3
    and F.1 (the display equation did not survive)."""
    q = np.asarray(q, dtype=np.float64)
    nq = math.sqrt(float(np.dot(q, q)))
    with np.errstate(invalid="ignore", over="ignore"):
        return scale * (mu @ q + nq * R)


def dual_score(q: np.ndarray, mu: np.ndarray, R: np.ndarray, sigma: np.ndarray, scale: float,
               z: float) -> np.ndarray:
    """Dual screen score of each block: the smaller of the geometric bound
    s (q . mu^ + ||q|| R) and the probabilistic estimate
    s (q . mu^ + z ||q * sigma^||_2) (Sections 3.1 and F.1, reading of the lost
    Eq. 7). A NaN on one side leaves the other (np.fmin)."""
    q = np.asarray(q, dtype=np.float64)
    geo = block_bound(q, mu, R, scale)
    with np.errstate(invalid="ignore", over="ignore"):
        spread = np.sqrt(((sigma * q[None, :]) ** 2).sum(axis=1))
        prob = scale * (mu @ q + z * spread)
    return np.fmin(geo, prob)


def admitted_blocks(ub: np.ndarray, tau: float, seq_len: int, lwb: int, block: int = BLOCK):
    """Blocks loaded for one (sequence, query head) (blocks of `block` tokens).

    ub: bounds of the complete blocks (length floor(T/64)). A complete block is
    admitted unless its bound is below tau~ (Section 3.1: a block matters when
    one of its keys reaches the threshold; a NaN bound cannot exclude it). The
    partial last block and the lwb most recent complete blocks are always
    admitted (Section 4.8, F.4). If nothing is admitted, the block with the
    largest bound is (Top-1 rescue, Section 3.2 and F.4, taken over the whole
    sequence; ties go to the lowest index).
    Returns (bool mask over ceil(T/64) blocks, rescued flag)."""
    nfull = seq_len // block
    nblk = -(-seq_len // block)
    adm = np.zeros(nblk, dtype=bool)
    ub = np.asarray(ub, dtype=np.float64)[:nfull]
    adm[:nfull] = ~(ub < tau)
    if seq_len % block:
        adm[nfull] = True
    if lwb > 0 and nfull > 0:
        adm[max(0, nfull - lwb):nfull] = True
    rescued = False
    if not adm.any():
        adm[int(np.argmax(ub))] = True
        rescued = True
    return adm, rescued


# --------------------------------------------------------------------------- attention
def filtered_attention(q: np.ndarray, keys: np.ndarray, values: np.ndarray,
                       tau: float, beta: float, scale: float) -> np.ndarray:
    """o = sum_t exp(S~_t) v_t / sum_t exp(S~_t) over the retained tokens, with
    S_t = s q.k_t and S~ = gate(S) (Section 2.2: weights w_s = exp(S~) on every
    retained token, normalised over the retained set; G.1)."""
    S = scale * (keys @ np.asarray(q, dtype=np.float64))
    St = gate(S, tau, beta)
    m = St.max()
    w = np.exp(St - m)
    return (w @ values) / w.sum()


@dataclasses.dataclass
class DecodeResult:
    o: np.ndarray            # float64 [N][H_Q][d]  (NaN for heads not evaluated)
    admitted: np.ndarray     # bool [N][H_Q][max_blocks]
    rescued: np.ndarray      # bool [N][H_Q]
    tau: np.ndarray          # float64 [N][H_Q]
    ub: np.ndarray           # float64 [N][H_Q][max_blocks] (NaN where no record)
    per_head: np.ndarray     # int64 [N][H_Q]   admitted blocks
    union: np.ndarray        # int64 [N][H_KV]  blocks loaded for the group
    tokens: np.ndarray       # int64 [N][H_Q]   attended tokens


def decode(k_pages, v_pages, kv_dtype: str, block_table, seq_lens, q, tau_mode: str,
           w, b_or_c, a: float, beta: float, lwb: int, summaries=None,
           heads: Optional[Iterable] = None, with_output: bool = True,
           bound: str = "geometric", z: float = 2.0, sigmas=None, boxes=None,
           fp8: str = "e4m3", summaries8=None) -> DecodeResult:
    """One ETA decode step for every sequence and query head.

    q: [N][H_Q][d] stored values; w: [H_Q][d] (learned mode); b_or_c: [H_Q].
    summaries: (mu, R) from build_summaries, built here if omitted.
    heads: iterable of (n, h) whose output is evaluated (default: all).
    bound: "geometric" (the sound bound), "dual" (dual_score with z and the
    sigma^ records from build_sigmas, built here if omitted), "quest" (the
    comparator's box bound with the (kmin, kmax) records from build_boxes) or
    "geometric_fp8" (the geometric bound over the FP8 records of format `fp8`,
    summaries8 = (mu8, R8) from build_summaries_fp8, built here if omitted)."""
    N, HQ, D = q.shape
    P, HKV, B, D2 = k_pages.shape
    assert D2 == D and B == BLOCK and HQ % HKV == 0
    G = HQ // HKV
    MB = block_table.shape[1]
    scale = 1.0 / math.sqrt(D)
    if summaries is None:
        summaries = build_summaries(k_pages, kv_dtype, block_table, seq_lens)
    mu_all, R_all = summaries
    if bound not in ("geometric", "dual", "quest", "geometric_fp8"):
        raise ValueError(f"unknown bound {bound!r}")
    if bound == "geometric_fp8" and summaries8 is None:
        summaries8 = build_summaries_fp8(k_pages, kv_dtype, block_table, seq_lens, fp8)
    if bound == "dual" and sigmas is None:
        sigmas = build_sigmas(k_pages, kv_dtype, block_table, seq_lens)
    if bound == "quest" and boxes is None:
        boxes = build_boxes(k_pages, kv_dtype, block_table, seq_lens)
    qf = upcast(q, kv_dtype)
    want = None if heads is None else set((int(n), int(h)) for n, h in heads)

    o = np.full((N, HQ, D), np.nan)
    admitted = np.zeros((N, HQ, MB), dtype=bool)
    rescued = np.zeros((N, HQ), dtype=bool)
    taus = np.zeros((N, HQ))
    ubs = np.full((N, HQ, MB), np.nan)
    for n in range(N):
        T = int(seq_lens[n])
        nfull = T // BLOCK
        pages = np.asarray(block_table[n], dtype=np.int64)
        for h in range(HQ):
            g = h // G
            tau = threshold(tau_mode, qf[n, h], None if w is None else w[h], b_or_c[h], a)
            taus[n, h] = tau
            if bound == "dual":
                ub = dual_score(qf[n, h], mu_all[pages[:nfull], g], R_all[pages[:nfull], g],
                                sigmas[pages[:nfull], g], scale, z)
            elif bound == "quest":
                ub = quest_bound(qf[n, h], boxes[0][pages[:nfull], g], boxes[1][pages[:nfull], g], scale)
            elif bound == "geometric_fp8":
                ub = block_bound(qf[n, h], summaries8[0][pages[:nfull], g], summaries8[1][pages[:nfull], g], scale)
            else:
                ub = block_bound(qf[n, h], mu_all[pages[:nfull], g], R_all[pages[:nfull], g], scale)
            ubs[n, h, :nfull] = ub
            adm, resc = admitted_blocks(ub, tau, T, lwb)
            admitted[n, h, :len(adm)] = adm
            rescued[n, h] = resc
            if not with_output or (want is not None and (n, h) not in want):
                continue
            o[n, h] = _attend(qf[n, h], k_pages, v_pages, kv_dtype, pages, g, np.nonzero(adm)[0],
                              T, tau, beta, scale)

    per_head = admitted.sum(axis=2).astype(np.int64)
    union = np.zeros((N, HKV), dtype=np.int64)
    tokens = np.zeros((N, HQ), dtype=np.int64)
    for n in range(N):
        T = int(seq_lens[n])
        nblk = -(-T // BLOCK)
        width = np.minimum(BLOCK, T - BLOCK * np.arange(nblk))
        for g in range(HKV):
            union[n, g] = admitted[n, g * G:(g + 1) * G, :nblk].any(axis=0).sum()
        tokens[n] = admitted[n, :, :nblk] @ width
    return DecodeResult(o=o, admitted=admitted, rescued=rescued, tau=taus, ub=ubs,
                        per_head=per_head, union=union, tokens=tokens)


def _attend(qh, k_pages, v_pages, kv_dtype, pages, g, blocks, T, tau, beta, scale):
    """filtered_attention over the tokens t < T of the given blocks, gathering
    the cache in slices of blocks so that long contexts fit in memory. The max
    is taken over all retained tokens first, then the weighted sums."""
    St_parts = []
    for b0 in range(0, len(blocks), _CHUNK_BLOCKS):
        bl = blocks[b0:b0 + _CHUNK_BLOCKS]
        kb = upcast(k_pages[pages[bl], g], kv_dtype).reshape(-1, qh.shape[0])
        tok = (bl[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
        keep = tok < T
        S = scale * (kb[keep] @ qh)
        St_parts.append(gate(S, tau, beta))
    St = np.concatenate(St_parts)
    m = St.max()
    num = np.zeros(qh.shape[0])
    den = 0.0
    pos = 0
    for b0 in range(0, len(blocks), _CHUNK_BLOCKS):
        bl = blocks[b0:b0 + _CHUNK_BLOCKS]
        vb = upcast(v_pages[pages[bl], g], kv_dtype).reshape(-1, qh.shape[0])
        tok = (bl[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)
        keep = tok < T
        wts = np.exp(St[pos:pos + int(keep.sum())] - m)
        pos += int(keep.sum())
        num += wts @ vb[keep]
        den += wts.sum()
    return num / den


# --------------------------------------------------------------------------- smaller screen blocks
def build_summaries_sub(k_pages: np.ndarray, kv_dtype: str, block_table: np.ndarray, seq_lens: np.ndarray,
                        block: int):
    """Records of every complete screen block of `block` tokens (16, 32 or
    128). Block j of a sequence holds its tokens j b .. j b + b - 1; its record
    lives with the page of its first token, in slot (j b mod 64) / b of that
    page: a page holds 64/b blocks of 16 or 32 tokens, while a 128-token block
    spans the pages 2j and 2j + 1 of the block table and its record sits in
    the single slot of page 2j. mu float64 [num_pages][H_KV][slots][d] holding
    float16 values and R float64 [num_pages][H_KV][slots] (slots = 64/b, or 1),
    NaN where there is none. Same record rule as build_summaries (block_summary
    on the block's b keys)."""
    assert block in (16, 32, 128)
    SB = max(1, BLOCK // block)
    P, HKV, B, D = k_pages.shape
    mu = np.full((P, HKV, SB, D), np.nan)
    R = np.full((P, HKV, SB), np.nan)
    chunk = max(1, _CHUNK_BLOCKS * BLOCK // block)
    for n in range(len(seq_lens)):
        nsub = int(seq_lens[n]) // block
        if nsub == 0:
            continue
        bt = np.asarray(block_table[n], dtype=np.int64)
        first = np.arange(nsub) * block
        pg = bt[first // BLOCK]
        sub = (first % BLOCK) // block
        for g in range(HKV):
            for j0 in range(0, nsub, chunk):
                sl = slice(j0, j0 + chunk)
                tok = first[sl, None] + np.arange(block)[None, :]
                rows = upcast(k_pages[bt[tok // BLOCK], g, tok % BLOCK], kv_dtype)
                m, r = block_summary(rows)
                mu[pg[sl], g, sub[sl]] = m
                R[pg[sl], g, sub[sl]] = r
    return mu, R


def decode_blocks(k_pages, v_pages, kv_dtype: str, block_table, seq_lens, q, tau_mode: str, w, b_or_c, a: float,
                  beta: float, lwb: int, block: int, summaries=None, heads: Optional[Iterable] = None,
                  with_output: bool = True) -> DecodeResult:
    """decode with the geometric screen on blocks of `block` tokens (16, 32 or
    128): block j of sequence n is its tokens j b .. j b + b - 1 (token t lies in
    page block_table[n][t / 64], row t mod 64), with the record that
    build_summaries_sub keeps for it. Admitted sets, bounds, forced blocks (the
    partial last block, the lwb most recent complete blocks), the rescue and
    the counts are per b-token block; admitted is
    [N][H_Q][ceil(64 max_blocks / b)]; union counts b-token blocks admitted by
    any head of the group; attention runs over the tokens t < T of the
    admitted blocks."""
    N, HQ, D = q.shape
    P, HKV, B, D2 = k_pages.shape
    assert D2 == D and B == BLOCK and HQ % HKV == 0 and block in (16, 32, 128)
    G = HQ // HKV
    MB = -(-block_table.shape[1] * BLOCK // block)
    scale = 1.0 / math.sqrt(D)
    mu_all, R_all = build_summaries_sub(k_pages, kv_dtype, block_table, seq_lens, block) \
        if summaries is None else summaries
    qf = upcast(q, kv_dtype)
    want = None if heads is None else set((int(n), int(h)) for n, h in heads)
    o = np.full((N, HQ, D), np.nan)
    admitted = np.zeros((N, HQ, MB), dtype=bool)
    rescued = np.zeros((N, HQ), dtype=bool)
    taus = np.zeros((N, HQ))
    ubs = np.full((N, HQ, MB), np.nan)
    for n in range(N):
        T = int(seq_lens[n])
        nfull = T // block
        pages = np.asarray(block_table[n], dtype=np.int64)
        first = np.arange(nfull) * block
        rp, rs = pages[first // BLOCK], (first % BLOCK) // block  # where each block's record lives
        for h in range(HQ):
            g = h // G
            tau = threshold(tau_mode, qf[n, h], None if w is None else w[h], b_or_c[h], a)
            taus[n, h] = tau
            ub = block_bound(qf[n, h], mu_all[rp, g, rs], R_all[rp, g, rs], scale)
            ubs[n, h, :nfull] = ub
            adm, resc = admitted_blocks(ub, tau, T, lwb, block)
            admitted[n, h, :len(adm)] = adm
            rescued[n, h] = resc
            if not with_output or (want is not None and (n, h) not in want):
                continue
            tok = (np.nonzero(adm)[0][:, None] * block + np.arange(block)[None, :]).reshape(-1)
            tok = tok[tok < T]
            K = upcast(k_pages[pages[tok // BLOCK], g, tok % BLOCK], kv_dtype)
            V = upcast(v_pages[pages[tok // BLOCK], g, tok % BLOCK], kv_dtype)
            o[n, h] = filtered_attention(qf[n, h], K, V, tau, beta, scale)
    per_head = admitted.sum(axis=2).astype(np.int64)
    union = np.zeros((N, HKV), dtype=np.int64)
    tokens = np.zeros((N, HQ), dtype=np.int64)
    for n in range(N):
        T = int(seq_lens[n])
        nblk = -(-T // block)
        width = np.minimum(block, T - block * np.arange(nblk))
        for g in range(HKV):
            union[n, g] = admitted[n, g * G:(g + 1) * G, :nblk].any(axis=0).sum()
        tokens[n] = admitted[n, :, :nblk] @ width
    return DecodeResult(o=o, admitted=admitted, rescued=rescued, tau=taus, ub=ubs,
                        per_head=per_head, union=union, tokens=tokens)


# --------------------------------------------------------------------------- offline calibration
# Section 4.7 and Appendix D.2 (Algorithm 1, whose body did not survive): the
# learned predictor of a head is replaced by a frozen constant c_h found from a
# 1/t-weighted histogram of attention scores over calibration sequences and a
# binary search for the head's training density. Reading taken here:
#   * every position t (0-based) of a calibration sequence is a query row over
#     the keys s <= t (causal), with scaled scores S = s_scale q_t . k_s;
#   * each key of row t carries the integer weight floor(2^31 / (t + 1)), so
#     every row weighs about the same whatever its length (the 1/t weighting);
#   * the histogram has num_bins equal bins over [lo, hi); scores outside fall
#     in the end bins;
#   * the target is the head's training density: the weighted count of scores
#     at or above the learned threshold w_h . q_t + b_h (or a given fraction
#     rho_h of the total weight);
#   * the binary search returns the lowest bin edge whose weighted tail (the
#     weight of the bins at or above it) does not exceed the target; c_h is
#     that edge.
CALIB_WEIGHT_ONE = 1 << 31


def row_weight(t: int) -> int:
    """Integer weight of every key of query row t (0-based, t + 1 keys)."""
    return CALIB_WEIGHT_ONE // (t + 1)


def score_bins(S: np.ndarray, lo: float, hi: float, num_bins: int) -> np.ndarray:
    """Bin index of each score: floor((S - lo) num_bins / (hi - lo)), clamped to the
    end bins; a NaN score (non-finite key) falls in bin 0."""
    with np.errstate(invalid="ignore"):
        x = np.floor((np.asarray(S, dtype=np.float64) - lo) * (num_bins / (hi - lo)))
    x = np.where(np.isnan(x), 0.0, x)
    return np.clip(x, 0, num_bins - 1).astype(np.int64)


def calibration_histogram(k_pages, kv_dtype: str, block_table, seq_lens, q_all, h: int, G: int,
                          lo: float, hi: float, num_bins: int, w_h=None, b_h=None, chunk: int = 256):
    """Weighted histogram of one query head's scores over the calibration
    sequences. q_all: [N][positions][H_Q][d] stored values (a query at every
    position). Returns (hist int64 [num_bins], above, total): above is the
    weighted count of scores at or above the learned threshold w_h . q_t + b_h
    (None without a predictor), total the weight of all scores."""
    D = q_all.shape[-1]
    scale = 1.0 / math.sqrt(D)
    g = h // G
    hist = np.zeros(num_bins, dtype=np.int64)
    above = 0 if w_h is not None else None
    total = 0
    for n in range(len(seq_lens)):
        T = int(seq_lens[n])
        nb = -(-T // BLOCK)
        pages = np.asarray(block_table[n, :nb], dtype=np.int64)
        K = upcast(k_pages[pages, g], kv_dtype).reshape(nb * BLOCK, D)[:T]
        Q = upcast(q_all[n, :T, h], kv_dtype)
        for t0 in range(0, T, chunk):
            t1 = min(T, t0 + chunk)
            S = scale * (Q[t0:t1] @ K[:t1].T)               # rows t0..t1-1, keys 0..t1-1
            bins = score_bins(S, lo, hi, num_bins)
            if w_h is not None:
                tau = Q[t0:t1] @ np.asarray(w_h, dtype=np.float64) + float(b_h)
            for i in range(t1 - t0):
                t = t0 + i
                wt = row_weight(t)
                hist += wt * np.bincount(bins[i, :t + 1], minlength=num_bins)
                total += wt * (t + 1)
                if w_h is not None:
                    above += wt * int(np.count_nonzero(S[i, :t + 1] >= tau[i]))
    return hist, above, total


def calibrated_bin(hist: np.ndarray, target: int) -> int:
    """Binary search for the lowest bin edge b (0..num_bins) whose weighted tail
    sum(hist[b:]) does not exceed target."""
    tail = np.concatenate([np.cumsum(hist[::-1])[::-1], [0]])  # tail[b] = sum(hist[b:])
    lo_b, hi_b = 0, len(hist)
    while lo_b < hi_b:
        mid = (lo_b + hi_b) // 2
        if tail[mid] <= target:
            hi_b = mid
        else:
            lo_b = mid + 1
    return lo_b


def calibrate(k_pages, kv_dtype: str, block_table, seq_lens, q_all, num_kv_heads: int, lo: float, hi: float,
              num_bins: int, w=None, b=None, rho=None, heads: Optional[Iterable] = None):
    """Calibrated constants c_h for the given query heads (default: all).
    Target from the learned predictor (w, b) or from densities rho [H_Q]
    (target = floor(rho_h * total)). Returns {h: dict(hist, above, total, target, bin, c)}."""
    HQ = q_all.shape[2]
    G = HQ // num_kv_heads
    out = {}
    for h in (range(HQ) if heads is None else heads):
        hist, above, total = calibration_histogram(k_pages, kv_dtype, block_table, seq_lens, q_all, h, G, lo, hi,
                                                   num_bins, None if w is None else w[h],
                                                   None if b is None else b[h])
        target = above if rho is None else int(math.floor(float(rho[h]) * total))
        bstar = calibrated_bin(hist, target)
        out[h] = dict(hist=hist, above=above, total=total, target=target, bin=bstar,
                      c=lo + bstar * (hi - lo) / num_bins)
    return out


# --------------------------------------------------------------------------- causal prefill
def prefill(k_pages, v_pages, kv_dtype: str, block_table, seq_lens, q_all, tau_mode: str, w, b_or_c,
            a: float, beta: float, heads: Optional[Iterable] = None, chunk: int = 512,
            positions: Optional[Iterable] = None) -> np.ndarray:
    """Causal ETA attention over a whole prompt (the training-time rule of
    Sections 2.2, E.3 and G.1 applied at every position): for position t of
    sequence n and query head h, over the keys s <= t,
        S = s_scale q_t . k_s,  S~ = S sigmoid(beta (S - tau~_t)),
        o_t = sum_s exp(S~) v_s / sum_s exp(S~),
    with tau~_t the learned (w_h . q_t + b_h - a) or calibrated (c_h - a)
    threshold of that position. No block is pruned: the prompt pass is dense
    and the gate alone filters (the blocks' records are built alongside, by
    build_summaries). q_all: [N][positions][H_Q][d]; returns float64
    [N][positions][H_Q][d], NaN at positions >= seq_len, for heads not in
    `heads` and, if `positions` is given, at positions not in it (each row
    depends only on its own query and the keys up to it)."""
    N, Lq, HQ, D = q_all.shape
    HKV = k_pages.shape[1]
    G = HQ // HKV
    scale = 1.0 / math.sqrt(D)
    want = None if heads is None else set((int(n), int(h)) for n, h in heads)
    pick = None if positions is None else np.unique(np.asarray(list(positions), dtype=np.int64))
    o = np.full((N, Lq, HQ, D), np.nan)
    for n in range(N):
        T = int(seq_lens[n])
        rows = np.arange(T) if pick is None else pick[(pick >= 0) & (pick < T)]
        if rows.size == 0:
            continue
        nb = -(-T // BLOCK)
        pages = np.asarray(block_table[n, :nb], dtype=np.int64)
        for h in range(HQ):
            if want is not None and (n, h) not in want:
                continue
            g = h // G
            K = upcast(k_pages[pages, g], kv_dtype).reshape(nb * BLOCK, D)[:T]
            V = upcast(v_pages[pages, g], kv_dtype).reshape(nb * BLOCK, D)[:T]
            Q = upcast(q_all[n, :T, h], kv_dtype)
            for c0 in range(0, rows.size, chunk):
                r = rows[c0:c0 + chunk]
                t1 = int(r[-1]) + 1
                tau = np.array([threshold(tau_mode, Q[t], None if w is None else w[h], b_or_c[h], a) for t in r])
                S = scale * (Q[r] @ K[:t1].T)
                St = gate(S, tau[:, None], beta)
                causal = np.arange(t1)[None, :] <= r[:, None]
                St = np.where(causal, St, -np.inf)
                m = St.max(axis=1, keepdims=True)
                wts = np.exp(St - m)
                o[n, r, h] = causal_weighted_sum(wts, V[:t1], causal) / wts.sum(axis=1, keepdims=True)
    return o


def causal_weighted_sum(wts: np.ndarray, V: np.ndarray, causal: np.ndarray) -> np.ndarray:
    """Row t of the result is the sum over the keys s <= t (causal[t, s]) of
    wts[t, s] v_s. The keys after t take no part in row t's sum, not even as
    0 * v_s, which a non-finite v_s would turn into NaN (the causal sum of
    Section 2.2 and E.1 runs over the keys up to t only). Elements of V that
    are not finite are therefore added one by one to the rows that see them."""
    bad = ~np.isfinite(V)
    if not bad.any():
        return wts @ V
    with np.errstate(invalid="ignore", over="ignore"):
        num = wts @ np.where(bad, 0.0, V)
        for s, i in zip(*np.nonzero(bad)):
            rows = causal[:, s]
            num[rows, i] += wts[rows, s] * V[s, i]
    return num
