"""Seeded synthetic workloads for the ETA decode step.

This module only draws random numbers and lays them out the way the KV cache
is stored. It holds none of the method's arithmetic: no block summaries, no
bounds, no thresholds, no gate, no softmax. Both the HIP path (through the
Python binding) and the fp64 oracle consume what it produces.

Shapes and distributions follow the decode benchmark described in
"Elastic Threshold Attention: Learned Contextual Sparsity for Long-Context
Decoding" (paperpeel.com/paper/2609.20888), Section 4.8 and Appendix F:
GQA with 64-token KV blocks, long contexts, block-sparse decoding. The key
distribution (per-block cluster centre plus small per-token noise) gives
blocks a spread of bound values so that thresholds can select a fraction of
them; planted "needle" keys aligned with a query stand in for the retrieval
structure of the needle tests in Section 4.4 (no benchmark items are used).

Storage conventions (shared with the C ABI):
  k_pages, v_pages : [num_pages][H_KV][64][d]; float32, or uint16 holding
                     bfloat16 bit patterns (round-to-nearest-even from fp32).
  q                : [N][H_Q][d], same storage type as K/V.
  w                : float32 [H_Q][d] (threshold predictor weights).
  block_table      : int32 [N][max_blocks]; -1 marks unused slots.
  seq_lens         : int32 [N].
Rows of a sequence's last page beyond its length are filled with `tail_fill`
(NaN by default) so that any read of them shows up in the result.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

BLOCK = 64
NEEDLE_LOGIT = 12.0  # scaled logit s*q.k of a planted needle key (before bf16 rounding)


# --------------------------------------------------------------------------- dtype plumbing
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (NaN stays NaN)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    r = ((u.astype(np.uint64) + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x32: np.ndarray, kv_dtype: str) -> np.ndarray:
    if kv_dtype == "bf16":
        return f32_to_bf16_bits(x32)
    if kv_dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    raise ValueError(kv_dtype)


def storage_to_f32(x: np.ndarray, kv_dtype: str) -> np.ndarray:
    return bf16_bits_to_f32(x) if kv_dtype == "bf16" else np.asarray(x, dtype=np.float32)


# --------------------------------------------------------------------------- workload record
@dataclasses.dataclass
class Workload:
    name: str
    kv_dtype: str
    n_seqs: int
    h_q: int
    h_kv: int
    d: int
    seq_lens: np.ndarray
    block_table: np.ndarray
    num_pages: int
    k_pages: np.ndarray
    v_pages: np.ndarray
    q: np.ndarray
    w: np.ndarray
    tau_mode: str               # "learned" | "calibrated"
    target_density: np.ndarray  # float64 [H_Q] per-head target fraction of blocks
    a: float = 0.0
    beta: float = 5.0
    lwb: int = 0
    bias: Optional[np.ndarray] = None  # float32 [H_Q]: b_h (learned) or c_h (calibrated)
    needles: list = dataclasses.field(default_factory=list)  # (n, h, token)
    seed: int = 0
    center_scale: float = 1.0
    noise_scale: float = 0.3
    redraw_round: int = 0

    @property
    def max_blocks(self) -> int:
        return self.block_table.shape[1]

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    def nblk(self, n: int) -> int:
        return -(-int(self.seq_lens[n]) // BLOCK)

    def kv_bytes(self) -> int:
        return self.k_pages.nbytes + self.v_pages.nbytes


# --------------------------------------------------------------------------- generators
_RECIPES = {
    # name: sizes, storage dtype, threshold mode, target per-head density, planted needles, default seed
    "tiny_4k_f32": dict(seed=1000, n=1, h_q=1, h_kv=1, d=64, T=4096, dtype="f32", mode="learned",
                        density=0.40, needles=3),
    "seq_32k": dict(seed=1001, n=1, h_q=32, h_kv=8, d=128, T=32768, dtype="bf16", mode="learned",
                    density=0.38, needles=0),
    "batch_4x128k": dict(seed=1002, n=4, h_q=32, h_kv=8, d=128, T=131072, dtype="bf16", mode="calibrated",
                         density=0.38, needles=0),
    "seq_512k": dict(seed=1003, n=1, h_q=32, h_kv=8, d=128, T=524288, dtype="bf16", mode="learned",
                     density=0.38, needles=16),
    # lengths log-uniform in [t_lo, t_hi], pages in a seeded random physical order, per-head density U[0.05, 0.90]
    "ragged_16": dict(seed=1004, n=16, h_q=32, h_kv=8, d=128, T=None, dtype="bf16", mode="learned",
                      density=None, needles=0, t_lo=4096, t_hi=262144, paged=True),
    # the head shape of the pages' decode benchmark (32 query heads over 4 KV heads, G = 8, d = 64) at
    # 512K tokens per sequence and a batch of 64 (a 32 GiB cache); frozen per-head constants (the
    # calibrated mode) and queries correlated within a group (rho), so that the group's union of admitted
    # blocks is about half the blocks at 38% per head
    "table5_512k": dict(seed=1005, n=64, h_q=32, h_kv=4, d=64, T=524288, dtype="bf16", mode="calibrated",
                        density=0.38, needles=0, rho=0.97),
}

WORKLOAD_NAMES = tuple(_RECIPES)


def recipe(name: str) -> dict:
    return dict(_RECIPES[name])


def _streams(seed: int, k: int):
    return np.random.SeedSequence(seed).spawn(k)


def make_workload(name: str, seed: Optional[int] = None, *, n_seqs: Optional[int] = None,
                  seq_len: Optional[int] = None, seq_lens=None, h_q: Optional[int] = None,
                  h_kv: Optional[int] = None, d: Optional[int] = None, kv_dtype: Optional[str] = None,
                  mode: Optional[str] = None, density=None, needles: Optional[int] = None,
                  paged: Optional[bool] = None, lwb: int = 0, a: float = 0.0, beta: float = 5.0,
                  tail_fill: float = float("nan"), threads: int = 8, rho: Optional[float] = None) -> Workload:
    """Draw one seeded workload. `name` picks the base recipe (one of WORKLOAD_NAMES);
    keyword overrides shrink or reshape it for parity-size cases.

    rho: correlation of the queries within a KV head's group. Query head h of
    group g is q_h = rho c_g + sqrt(1 - rho^2) e_h, with c_g and e_h independent
    N(0, I_d) draws (e_h is the uncorrelated workloads' query), so every pair of
    heads of a group has correlation rho^2 per coordinate. None (the default
    of most recipes) or 0 gives independent queries."""
    spec = recipe(name)
    seed = spec["seed"] if seed is None else int(seed)
    N = spec["n"] if n_seqs is None else int(n_seqs)
    HQ = spec["h_q"] if h_q is None else int(h_q)
    HKV = spec["h_kv"] if h_kv is None else int(h_kv)
    D = spec["d"] if d is None else int(d)
    dt = spec["dtype"] if kv_dtype is None else kv_dtype
    md = spec["mode"] if mode is None else mode
    n_needles = spec["needles"] if needles is None else int(needles)
    is_paged = bool(spec.get("paged", False)) if paged is None else bool(paged)
    if HQ % HKV:
        raise ValueError("H_Q must be a multiple of H_KV")

    (ss_len, ss_ctr, ss_noise, ss_v, ss_q, ss_w, ss_dens, ss_needle, ss_perm, ss_qgroup) = _streams(seed, 10)
    rho = spec.get("rho") if rho is None else float(rho)
    if rho is not None and not 0.0 <= rho <= 1.0:
        raise ValueError("rho must lie in [0, 1]")

    # sequence lengths
    if seq_lens is not None:
        lens = np.asarray(seq_lens, dtype=np.int64)
        N = len(lens)
    elif seq_len is not None:
        lens = np.full(N, int(seq_len), dtype=np.int64)
    elif spec["T"] is not None:
        lens = np.full(N, spec["T"], dtype=np.int64)
    else:  # log-uniform lengths
        rng = np.random.default_rng(ss_len)
        lo, hi = math.log(spec["t_lo"]), math.log(spec["t_hi"])
        lens = np.exp(rng.uniform(lo, hi, size=N)).astype(np.int64)
        lens = np.clip(lens, spec["t_lo"], spec["t_hi"])
    if (lens < 1).any():
        raise ValueError("sequence lengths must be >= 1")
    nblks = -(-lens // BLOCK)
    max_blocks = int(nblks.max())

    # page assignment
    total_pages = int(nblks.sum())
    if is_paged:
        perm = np.random.default_rng(ss_perm).permutation(total_pages).astype(np.int32)
        num_pages = total_pages
    else:
        perm = None
        num_pages = N * max_blocks
    bt = np.full((N, max_blocks), -1, dtype=np.int32)
    off = 0
    for n in range(N):
        nb = int(nblks[n])
        if is_paged:
            bt[n, :nb] = perm[off:off + nb]
        else:
            bt[n, :nb] = n * max_blocks + np.arange(nb, dtype=np.int32)
        off += nb

    store_t = np.uint16 if dt == "bf16" else np.float32
    k_pages = np.zeros((num_pages, HKV, BLOCK, D), dtype=store_t)
    v_pages = np.zeros((num_pages, HKV, BLOCK, D), dtype=store_t)

    ctr_seqs = ss_ctr.spawn(N * HKV)
    noise_seqs = ss_noise.spawn(N * HKV)
    v_seqs = ss_v.spawn(N * HKV)

    def fill_segment(sidx: int) -> None:
        n, g = divmod(sidx, HKV)
        T = int(lens[n])
        nb = int(nblks[n])
        r_c = np.random.default_rng(ctr_seqs[sidx])
        r_e = np.random.default_rng(noise_seqs[sidx])
        r_v = np.random.default_rng(v_seqs[sidx])
        pages = bt[n, :nb]
        chunk = 512
        for j0 in range(0, nb, chunk):
            j1 = min(nb, j0 + chunk)
            c = r_c.standard_normal((j1 - j0, 1, D), dtype=np.float32)
            e = r_e.standard_normal((j1 - j0, BLOCK, D), dtype=np.float32)
            kk = c + np.float32(0.3) * e
            vv = r_v.standard_normal((j1 - j0, BLOCK, D), dtype=np.float32)
            # rows past the end of the sequence hold junk
            if j1 == nb and T % BLOCK:
                kk[-1, T % BLOCK:, :] = tail_fill
                vv[-1, T % BLOCK:, :] = tail_fill
            k_pages[pages[j0:j1], g] = to_storage(kk, dt)
            v_pages[pages[j0:j1], g] = to_storage(vv, dt)

    nseg = N * HKV
    if threads > 1 and nseg > 1:
        with ThreadPoolExecutor(max_workers=min(threads, nseg)) as ex:
            list(ex.map(fill_segment, range(nseg)))
    else:
        for s in range(nseg):
            fill_segment(s)

    q32 = np.random.default_rng(ss_q).standard_normal((N, HQ, D), dtype=np.float32)
    if rho:  # a component shared by the heads of each group
        c = np.random.default_rng(ss_qgroup).standard_normal((N, HKV, D), dtype=np.float32)
        q32 = (np.float32(rho) * np.repeat(c, HQ // HKV, axis=1)
               + np.float32(math.sqrt(1.0 - rho * rho)) * q32).astype(np.float32)
    q = to_storage(q32, dt)
    w = (np.random.default_rng(ss_w).standard_normal((HQ, D), dtype=np.float32)
         / np.float32(math.sqrt(D))).astype(np.float32)

    # target densities
    if density is None:
        if spec["density"] is None:  # per-head spread
            dens = np.random.default_rng(ss_dens).uniform(0.05, 0.90, size=HQ)
        else:
            dens = np.full(HQ, spec["density"])
    else:
        dens = np.broadcast_to(np.asarray(density, dtype=np.float64), (HQ,)).copy()

    wl = Workload(name=name, kv_dtype=dt, n_seqs=N, h_q=HQ, h_kv=HKV, d=D,
                  seq_lens=lens.astype(np.int32), block_table=bt, num_pages=num_pages,
                  k_pages=k_pages, v_pages=v_pages, q=q, w=w, tau_mode=md,
                  target_density=dens, a=float(a), beta=float(beta), lwb=int(lwb), seed=seed)

    # needles: key rows aligned with one query head of the group, at seeded positions
    if n_needles:
        rng = np.random.default_rng(ss_needle)
        for _ in range(n_needles):
            n = int(rng.integers(N))
            t = int(rng.integers(int(lens[n])))
            h = int(rng.integers(HQ))
            wl.needles.append((n, h, t))
            plant_needle(wl, n, h, t)
    return wl


def plant_needle(wl: Workload, n: int, h: int, t: int, logit: float = NEEDLE_LOGIT) -> None:
    """Overwrite key t of sequence n in KV head h//G with a vector parallel to
    query head h, scaled so that its scaled dot product with that query is
    about `logit`."""
    qh = storage_to_f32(wl.q[n, h], wl.kv_dtype).astype(np.float64)
    nq = float(np.sqrt(np.dot(qh, qh)))
    alpha = logit * math.sqrt(wl.d) / max(nq, 1e-30)
    key = (alpha * qh / max(nq, 1e-30)).astype(np.float32)
    g = h // wl.group
    page = int(wl.block_table[n, t // BLOCK])
    wl.k_pages[page, g, t % BLOCK] = to_storage(key, wl.kv_dtype)


def _segment_centres(wl: Workload, n: int, g: int) -> np.ndarray:
    """Re-draw the block centres of segment (n, g) exactly as make_workload did."""
    ss_ctr = _streams(wl.seed, 9)[1]
    r_c = np.random.default_rng(ss_ctr.spawn(wl.n_seqs * wl.h_kv)[n * wl.h_kv + g])
    nb = wl.nblk(n)
    out = []
    for j0 in range(0, nb, 512):
        j1 = min(nb, j0 + 512)
        out.append(r_c.standard_normal((j1 - j0, 1, wl.d), dtype=np.float32))
    return np.concatenate(out, axis=0)


def redraw_blocks(wl: Workload, blocks) -> None:
    """Re-draw the per-token noise of the given complete blocks, each listed as
    (n, g, j), from a fresh sub-stream; needles inside them are re-planted."""
    blocks = sorted(set((int(n), int(g), int(j)) for n, g, j in blocks))
    if not blocks:
        return
    wl.redraw_round += 1
    rng = np.random.default_rng(np.random.SeedSequence([wl.seed, 7919, wl.redraw_round]))
    needle_at = {}
    for (n, h, t) in wl.needles:
        needle_at.setdefault((n, h // wl.group, t // BLOCK), []).append((h, t))
    centres = {}
    for (n, g, j) in blocks:
        if (n, g) not in centres:
            centres[(n, g)] = _segment_centres(wl, n, g)
        page = int(wl.block_table[n, j])
        e = rng.standard_normal((BLOCK, wl.d), dtype=np.float32)
        kk = centres[(n, g)][j] + np.float32(0.3) * e
        T = int(wl.seq_lens[n])
        valid = min(BLOCK, T - j * BLOCK)
        new = storage_to_f32(wl.k_pages[page, g], wl.kv_dtype).copy()
        new[:valid] = kk[:valid]
        wl.k_pages[page, g] = to_storage(new, wl.kv_dtype)
        for (h, t) in needle_at.get((n, g, j), []):
            plant_needle(wl, n, h, t)


def permute_pages(wl: Workload, seed: int) -> Workload:
    """Same logical cache stored in a different physical page order."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(wl.num_pages).astype(np.int32)  # old page p -> new page perm[p]
    k_new = np.empty_like(wl.k_pages)
    v_new = np.empty_like(wl.v_pages)
    k_new[perm] = wl.k_pages
    v_new[perm] = wl.v_pages
    bt = wl.block_table.copy()
    used = bt >= 0
    bt[used] = perm[bt[used]]
    return dataclasses.replace(wl, k_pages=k_new, v_pages=v_new, block_table=bt,
                               needles=list(wl.needles))


def trace_queries(wl: Workload, seed: int = 77) -> np.ndarray:
    """A query for every position of every sequence (calibration traces):
    [N][64 * max_blocks][H_Q][d] in the workload's storage type, N(0, 1)
    entries; positions past a sequence's length hold zeros."""
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(1)[0])
    L = BLOCK * wl.max_blocks
    q = np.zeros((wl.n_seqs, L, wl.h_q, wl.d), dtype=np.float32)
    for n in range(wl.n_seqs):
        T = int(wl.seq_lens[n])
        q[n, :T] = rng.standard_normal((T, wl.h_q, wl.d)).astype(np.float32)
    return to_storage(q, wl.kv_dtype)
