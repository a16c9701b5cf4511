"""Per-key brute force of the ETA decode step, for tiny inputs only.

An independent second implementation used to pin the oracle: pure-Python loops
over every key with the `math` module (fsum, exact float16 rounding through
`struct`), no NumPy vector arithmetic and no code shared with `oracle/`.
Screen blocks of 16 or 32 tokens are taken through the `block` argument.
It follows "Elastic Threshold Attention" (paperpeel.com/paper/2609.20888),
Sections 2.2, 3.1, 3.2, 4.8, F.1, F.4 and G.1, with the same readings as the
oracle (geometric bound about the fp16 centroid, global top-1 rescue; the
optional dual score as the smaller of that bound and s (q . mu^ + z ||q * sigma^||);
the Quest comparator's box bound of Section 4.3 over outward-rounded float16
coordinate extrema).
"""
from __future__ import annotations

import math
import struct

BLOCK = 64


def _f16(x: float) -> float:
    try:
        return struct.unpack("<e", struct.pack("<e", x))[0]
    except OverflowError:
        return math.inf


def _sig(x: float) -> float:
    if math.isnan(x):
        return math.nan
    if x >= 0:
        return 1.0 / (1.0 + math.exp(-x))
    try:
        e = math.exp(x)
    except OverflowError:  # pragma: no cover - x < 0 cannot overflow
        return 0.0
    return e / (1.0 + e)


def value(stored, kv_dtype: str) -> float:
    if kv_dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", int(stored) << 16))[0]
    return float(stored)


def record(rows):
    """(centroid, radius) of one complete block given its key rows."""
    d = len(rows[0])
    mean = [math.fsum(r[c] for r in rows) / len(rows) for c in range(d)]
    mu = [_f16(x) for x in mean]
    if not all(math.isfinite(x) for x in mu):
        mu = [0.0] * d
    best = 0.0
    for r in rows:
        try:
            dist = math.sqrt(math.fsum((r[c] - mu[c]) ** 2 for c in range(d)))
        except (OverflowError, ValueError):
            dist = math.inf
        if math.isnan(dist) or math.isinf(dist):
            return mu, math.inf
        best = max(best, dist)
    return mu, best


def deviation(rows):
    """Coordinate standard deviation (population) of one block about its exact
    mean, rounded to float16; inf where not finite."""
    d = len(rows[0])
    out = []
    for c in range(d):
        col = [r[c] for r in rows]
        try:
            m = math.fsum(col) / len(col)
            sd = math.sqrt(math.fsum((x - m) ** 2 for x in col) / len(col))
        except (OverflowError, ValueError):
            sd = math.inf
        sd = _f16(sd) if math.isfinite(sd) else math.inf
        out.append(sd)
    return out


def _f16_directed(x: float, up: bool) -> float:
    """float16 value nearest to x on the requested side, through the bit
    pattern: struct rounds to nearest, then one step of the pattern fixes the
    side (patterns of one sign order like their magnitudes)."""
    if math.isnan(x):
        return math.nan
    try:
        bits = struct.unpack("<H", struct.pack("<e", x))[0]
    except OverflowError:
        bits = 0x7C00 if x > 0 else 0xFC00
    y = struct.unpack("<e", struct.pack("<H", bits))[0]
    if (up and y < x) or (not up and y > x):
        if bits & 0x7FFF == 0:
            bits = 0x0001 if up else 0x8001
        elif (bits & 0x8000 != 0) == up:
            bits -= 1
        else:
            bits += 1
        y = struct.unpack("<e", struct.pack("<H", bits))[0]
    return y


def box(rows):
    """(kmin, kmax) of one block: per coordinate the least and greatest key
    value, rounded outward to float16; NaN for a block with a non-finite key."""
    d = len(rows[0])
    if not all(math.isfinite(x) for r in rows for x in r):
        return [math.nan] * d, [math.nan] * d
    lo = [_f16_directed(min(r[c] for r in rows), up=False) for c in range(d)]
    hi = [_f16_directed(max(r[c] for r in rows), up=True) for c in range(d)]
    return lo, hi


def fp8_values(fmt: str):
    """Every finite value of an OCP 8-bit format, by code (sign, exponent,
    mantissa fields decoded from the definition): {code: value}."""
    eb, mb = (4, 3) if fmt == "e4m3" else (5, 2)
    bias = (1 << (eb - 1)) - 1
    vals = {}
    for code in range(256):
        sgn = -1.0 if code & 0x80 else 1.0
        e = (code >> mb) & ((1 << eb) - 1)
        m = code & ((1 << mb) - 1)
        if fmt == "e4m3" and e == 15 and m == 7:
            continue  # NaN
        if fmt == "e5m2" and e == 31:
            continue  # infinities and NaN
        v = m * 2.0 ** (1 - bias - mb) if e == 0 else (1.0 + m / 2.0 ** mb) * 2.0 ** (e - bias)
        vals[code] = sgn * v
    return vals


def fp8_nearest(x: float, fmt: str) -> float:
    """The format's value nearest to x by search over all codes; a tie goes to
    the code with an even mantissa; beyond the largest finite magnitude, that
    magnitude (saturation)."""
    if math.isnan(x):
        return math.nan
    vals = fp8_values(fmt)
    top = max(vals.values())
    if abs(x) >= top:
        return math.copysign(top, x)
    best = None
    for code, v in vals.items():
        dist = abs(v - x)
        if best is None or dist < best[0] or (dist == best[0] and code % 2 == 0 and best[1] % 2 == 1):
            best = (dist, code, v)
    return best[2] if best[2] != 0 else math.copysign(0.0, x)


def record_fp8(rows, fmt: str):
    """(FP8 centroid, radius about it) of one block; zero centroid and an
    infinite radius for a block with a non-finite key."""
    d = len(rows[0])
    if not all(math.isfinite(x) for r in rows for x in r):
        return [0.0] * d, math.inf
    mean = [math.fsum(r[c] for r in rows) / len(rows) for c in range(d)]
    mu = [fp8_nearest(x, fmt) for x in mean]
    best = 0.0
    for r in rows:
        best = max(best, math.sqrt(math.fsum((r[c] - mu[c]) ** 2 for c in range(d))))
    return mu, best


def _greater(a: float, b: float) -> float:
    if math.isnan(a):
        return b
    if math.isnan(b):
        return a
    return max(a, b)


def _smaller(a: float, b: float) -> float:
    if math.isnan(a):
        return b
    if math.isnan(b):
        return a
    return min(a, b)


def decode(wl_k, wl_v, kv_dtype, block_table, seq_lens, q, tau_mode, w, b_or_c, a, beta, lwb,
           bound="geometric", z=2.0, fp8="e4m3", block=BLOCK):
    """Returns dict with per (n, h): admitted block list, rescued flag, output
    list, plus union counts per (n, g). Inputs are NumPy arrays of stored values
    but are read element by element."""
    N, HQ, D = q.shape
    HKV = wl_k.shape[1]
    G = HQ // HKV
    s = 1.0 / math.sqrt(D)
    out = {}
    union = {}
    for n in range(N):
        T = int(seq_lens[n])
        nfull = T // block
        nblk = -(-T // block)

        def key(g, t):
            page = int(block_table[n][t // BLOCK])
            return [value(x, kv_dtype) for x in wl_k[page][g][t % BLOCK]]

        def val(g, t):
            page = int(block_table[n][t // BLOCK])
            return [value(x, kv_dtype) for x in wl_v[page][g][t % BLOCK]]

        for g in range(HKV):
            if bound == "geometric_fp8":
                recs = [record_fp8([key(g, j * block + r) for r in range(block)], fp8) for j in range(nfull)]
            else:
                recs = [record([key(g, j * block + r) for r in range(block)]) for j in range(nfull)]
            devs = [deviation([key(g, j * block + r) for r in range(block)]) for j in range(nfull)] \
                if bound == "dual" else None
            boxes = [box([key(g, j * block + r) for r in range(block)]) for j in range(nfull)] \
                if bound == "quest" else None
            loaded = set()
            for hh in range(G):
                h = g * G + hh
                qh = [value(x, kv_dtype) for x in q[n][h]]
                if tau_mode == "learned":
                    tau = math.fsum(float(w[h][c]) * qh[c] for c in range(D)) + float(b_or_c[h]) - a
                else:
                    tau = float(b_or_c[h]) - a
                qn = math.sqrt(math.fsum(x * x for x in qh))
                adm = []
                ubs = []
                for j in range(nfull):
                    mu, R = recs[j]
                    dot = math.fsum(qh[c] * mu[c] for c in range(D))
                    ub = s * (dot + qn * R)
                    if bound == "quest":
                        lo, hi = boxes[j]
                        terms = []
                        for c in range(D):
                            with_nan = [qh[c] * hi[c] if not (qh[c] == 0 and math.isinf(hi[c])) else math.nan,
                                        qh[c] * lo[c] if not (qh[c] == 0 and math.isinf(lo[c])) else math.nan]
                            terms.append(_greater(*with_nan))
                        try:
                            ub = math.nan if any(math.isnan(x) for x in terms) else s * math.fsum(terms)
                        except ValueError:  # +inf and -inf terms
                            ub = math.nan
                    if bound == "dual":
                        try:
                            spread = math.sqrt(math.fsum((qh[c] * devs[j][c]) ** 2 for c in range(D)))
                            est = s * (dot + z * spread)
                        except (OverflowError, ValueError):
                            est = math.inf
                        ub = _smaller(ub, est)
                    ubs.append(ub)
                    forced = j >= nfull - lwb
                    if forced or not (ub < tau):
                        adm.append(j)
                if T % block:
                    adm.append(nfull)
                rescued = False
                if not adm:
                    best = 0
                    for j in range(1, nfull):
                        if ubs[j] > ubs[best]:
                            best = j
                    adm = [best]
                    rescued = True
                loaded.update(adm)
                # attention over every retained token
                logits = []
                vals = []
                for j in adm:
                    for r in range(block):
                        t = j * block + r
                        if t >= T:
                            break
                        S = s * math.fsum(qh[c] * x for c, x in enumerate(key(g, t)))
                        arg = beta * (S - tau)
                        logits.append(S * _sig(arg))
                        vals.append(val(g, t))
                m = max(logits)
                wts = [math.exp(x - m) for x in logits]
                den = math.fsum(wts)
                o = [math.fsum(wts[i] * vals[i][c] for i in range(len(wts))) / den for c in range(D)]
                tokens = sum(min(block, T - j * block) for j in adm)
                out[(n, h)] = dict(admitted=sorted(adm), rescued=rescued, o=o, tau=tau, ub=ubs,
                                   tokens=tokens)
            union[(n, g)] = len(loaded)
    return out, union
