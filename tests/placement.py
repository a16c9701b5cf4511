"""Threshold placement for the test workloads (uses the oracle; test side only).

Chooses each head's bias b_h (learned mode) or constant c_h (calibrated mode)
so that about the target fraction of complete blocks passes the oracle's
screen, then re-draws the noise of any block whose bound lies within `margin`
of a threshold of its group, until none does. With that margin, the admitted
sets are decided identically by any implementation whose bound and threshold
agree with the oracle's to better than `margin`.
"""
from __future__ import annotations

import math

import numpy as np

import oracle.eta_oracle as E
import workloads as W

BLOCK = 64


def _bounds(wl, mu, R, sigma=None, z=2.0, boxes=None, block=64):
    """ub[n][h][j] for complete blocks (NaN elsewhere), tau offsets per (n, h).
    With sigma, the dual screen score instead of the geometric bound; with
    boxes (kmin, kmax), the comparator's box bound."""
    N, HQ, D = wl.q.shape
    G = wl.group
    s = 1.0 / math.sqrt(D)
    qf = E.upcast(wl.q, wl.kv_dtype)
    ub = np.full((N, HQ, -(-wl.max_blocks * BLOCK // block)), np.nan)
    for n in range(N):
        if block != BLOCK:  # records of other screen blocks: mu [P][HKV][slots][d], kept with the first page
            nsub = int(wl.seq_lens[n]) // block
            first = np.arange(nsub) * block
            pg, sl = wl.block_table[n][first // BLOCK], (first % BLOCK) // block
            for h in range(HQ):
                ub[n, h, :nsub] = E.block_bound(qf[n, h], mu[pg, h // G, sl], R[pg, h // G, sl], s)
            continue
        nfull = int(wl.seq_lens[n]) // BLOCK
        pages = wl.block_table[n, :nfull]
        for h in range(HQ):
            g = h // G
            if boxes is not None:
                ub[n, h, :nfull] = E.quest_bound(qf[n, h], boxes[0][pages, g], boxes[1][pages, g], s)
            elif sigma is None:
                ub[n, h, :nfull] = E.block_bound(qf[n, h], mu[pages, g], R[pages, g], s)
            else:
                ub[n, h, :nfull] = E.dual_score(qf[n, h], mu[pages, g], R[pages, g], sigma[pages, g], s, z)
    if wl.tau_mode == "learned":
        off = np.einsum("nhd,hd->nh", qf, wl.w.astype(np.float64)) - wl.a
    else:
        off = np.full((N, HQ), -wl.a)
    return ub, off


def place(wl, margin: float = 1e-3, max_rounds: int = 50, summaries=None, bound: str = "geometric",
          z: float = 2.0, fp8: str = "e4m3", block: int = 64):
    """Set wl.bias in place; returns the oracle summaries of the final cache
    ((mu, R), (mu, R, sigma) for the dual screen, (mu, R, kmin, kmax) for the
    comparator's box bound; the FP8 records (mu8, R8) for "geometric_fp8"; the
    records of `block`-token blocks (mu_sub, R_sub) for "geometric_sub")."""
    if bound == "geometric_sub":
        mu, R = E.build_summaries_sub(wl.k_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, block)
    elif bound == "geometric_fp8":
        mu, R = E.build_summaries_fp8(wl.k_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, fp8)
    else:
        mu, R = E.build_summaries(wl.k_pages, wl.kv_dtype, wl.block_table, wl.seq_lens) \
            if summaries is None else summaries[:2]
    sigma = None
    boxes = None
    if bound == "dual":
        sigma = E.build_sigmas(wl.k_pages, wl.kv_dtype, wl.block_table, wl.seq_lens)
    if bound == "quest":
        boxes = E.build_boxes(wl.k_pages, wl.kv_dtype, wl.block_table, wl.seq_lens)
    blk = block if bound == "geometric_sub" else 64
    ub, off = _bounds(wl, mu, R, sigma, z, boxes, blk)
    HQ = wl.h_q
    bias = np.zeros(HQ, dtype=np.float32)
    for h in range(HQ):
        t = float(wl.target_density[h])
        x = (ub[:, h, :] - off[:, h, None]).ravel()  # admitted iff x >= bias
        x = np.sort(x[~np.isnan(x)])[::-1]
        if t >= 1.0:
            bias[h] = -np.inf
            continue
        k = int(round(t * len(x)))
        k = min(max(k, 1), len(x) - 1)
        bias[h] = np.float32(0.5 * (x[k - 1] + x[k]))
    wl.bias = bias
    for _ in range(max_rounds):
        tau = off + bias.astype(np.float64)[None, :]
        close = np.abs(ub - tau[:, :, None]) < margin
        bad = set()
        G = wl.group
        for n, h, j in zip(*np.nonzero(close)):
            bad.add((int(n), int(h) // G, int(j) * blk // 64))  # the page holding the block
        if not bad:
            if boxes is not None:
                return mu, R, boxes[0], boxes[1]
            return (mu, R) if sigma is None else (mu, R, sigma)
        W.redraw_blocks(wl, bad)
        for (n, g, j) in bad:
            page = int(wl.block_table[n, j])
            kb = E.upcast(wl.k_pages[page, g], wl.kv_dtype)
            if bound == "geometric_sub" and blk > 64:  # a 128-token block: pages j and j + 1
                kb2 = E.upcast(wl.k_pages[int(wl.block_table[n, j + 1]), g], wl.kv_dtype)
                m, r = E.block_summary(np.concatenate([kb, kb2]))
            elif bound == "geometric_sub":
                m, r = E.block_summary(kb.reshape(64 // blk, blk, -1))
            else:
                m, r = E.block_summary_fp8(kb, fp8) if bound == "geometric_fp8" else E.block_summary(kb)
            mu[page, g] = m
            R[page, g] = r
            if sigma is not None:
                sigma[page, g] = E.block_sigma(kb)
            if boxes is not None:
                boxes[0][page, g], boxes[1][page, g] = E.block_box(kb)
        ub, off = _bounds(wl, mu, R, sigma, z, boxes, blk)
    raise RuntimeError("margin enforcement did not converge")


def densities(res, wl):
    """Per-head admitted fraction of blocks, and per-(n,g) union fraction."""
    nblk = np.array([wl.nblk(n) for n in range(wl.n_seqs)], dtype=np.float64)
    per_head = res.per_head / nblk[:, None]
    union = res.union / nblk[:, None]
    return per_head, union
