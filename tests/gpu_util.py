"""Helpers for the GPU parity tests: upload a workload, run the HIP path
through the C ABI, and compare with the oracle."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import learned_threshold_block_amd as eta
import oracle.eta_oracle as E
import placement
import workloads as W

TOL = {"f32": 1e-5, "bf16": 2e-3}   # max abs error on o, per K/V storage type


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


class Dev:
    """A workload's inputs on the GPU."""

    def __init__(self, wl: W.Workload, device="cuda", with_sigma=False, with_box=False, fp8=None, sub_block=0):
        self.wl = wl
        self.device = torch.device(device)
        z16 = lambda: torch.zeros(wl.num_pages, wl.h_kv, wl.d, dtype=torch.float16, device=device)  # noqa: E731
        sig = z16() if with_sigma else None
        lo, hi = (z16(), z16()) if with_box else (None, None)
        self.cache = eta.Cache(eta.upload(wl.k_pages, wl.kv_dtype, device),
                               eta.upload(wl.v_pages, wl.kv_dtype, device),
                               torch.zeros(wl.num_pages, wl.h_kv, wl.d, dtype=torch.float16, device=device),
                               torch.zeros(wl.num_pages, wl.h_kv, dtype=torch.float32, device=device), sig,
                               lo, hi,
                               torch.zeros(wl.num_pages, wl.h_kv, wl.d, dtype=torch.uint8, device=device)
                               if fp8 else None,
                               torch.zeros(wl.num_pages, wl.h_kv, dtype=torch.float32, device=device)
                               if fp8 else None, fp8 or "e4m3", sub_block,
                               torch.zeros(wl.num_pages, wl.h_kv, max(1, 64 // sub_block), wl.d,
                                           dtype=torch.float16, device=device) if sub_block else None,
                               torch.zeros(wl.num_pages, wl.h_kv, max(1, 64 // sub_block), dtype=torch.float32,
                                           device=device) if sub_block else None)
        self.seq_lens = torch.from_numpy(wl.seq_lens.astype(np.int32)).to(device)
        self.bt = torch.from_numpy(wl.block_table.astype(np.int32)).to(device)
        self.q = eta.upload(wl.q, wl.kv_dtype, device)
        self.w = torch.from_numpy(wl.w).to(device)
        self.ws = eta.alloc_workspace(self.cache, wl.n_seqs, wl.max_blocks, wl.h_q)
        self.out = torch.empty(wl.n_seqs, wl.h_q, wl.d, dtype=torch.float32, device=device)

    def build(self):
        eta.build_block_summaries(self.cache, self.seq_lens, self.bt)

    def decode(self, bias=None, tau_mode=None, a=None, beta=None, lwb=None, bound="geometric", z=2.0):
        wl = self.wl
        b = torch.from_numpy(np.asarray(wl.bias if bias is None else bias, dtype=np.float32)).to(self.device)
        mode = wl.tau_mode if tau_mode is None else tau_mode
        m = eta.ETA_TAU_LEARNED if mode == "learned" else eta.ETA_TAU_CALIBRATED
        eta.decode(self.cache, self.seq_lens, self.bt, self.q, m, b, w=self.w,
                   a=wl.a if a is None else a, beta=wl.beta if beta is None else beta,
                   lwb=wl.lwb if lwb is None else lwb, out=self.out, workspace=self.ws, bound=bound, z=z)
        torch.cuda.synchronize()
        return self.out.cpu().numpy().astype(np.float64)

    def stats(self, check=True):
        wl = self.wl
        return eta.stats(self.ws, wl.n_seqs, wl.max_blocks, wl.h_q, wl.h_kv, check=check)

    def sub_records(self):
        return (self.cache.mu_sub.cpu().view(torch.int16).numpy().view(np.uint16),
                self.cache.radius_sub.cpu().numpy())

    def mu_bits(self):
        return self.cache.mu.cpu().view(torch.int16).numpy().view(np.uint16)

    def radius(self):
        return self.cache.radius.cpu().numpy()

    def sigma_bits(self):
        return self.cache.sigma.cpu().view(torch.int16).numpy().view(np.uint16)

    def fp8_codes(self):
        return self.cache.mu8.cpu().numpy(), self.cache.radius8.cpu().numpy()

    def box_bits(self):
        f = lambda t: t.cpu().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
        return f(self.cache.kmin), f(self.cache.kmax)


def oracle_decode(wl, summaries=None, heads=None, bias=None, tau_mode=None, a=None, beta=None, lwb=None,
                  bound="geometric", z=2.0, fp8="e4m3", block=64):
    """summaries: (mu, R); for the dual screen (mu, R, sigma); for the
    comparator's box bound (mu, R, kmin, kmax); for "geometric_fp8" the FP8
    records (mu8, R8); for "geometric_sub" the records of `block`-token
    blocks."""
    if bound == "geometric_sub":
        return E.decode_blocks(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, wl.q,
                               wl.tau_mode if tau_mode is None else tau_mode, wl.w,
                               wl.bias if bias is None else bias, wl.a if a is None else a,
                               wl.beta if beta is None else beta, wl.lwb if lwb is None else lwb, block,
                               summaries=summaries, heads=heads)
    if bound == "geometric_fp8":
        return E.decode(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, wl.q,
                        wl.tau_mode if tau_mode is None else tau_mode, wl.w,
                        wl.bias if bias is None else bias, wl.a if a is None else a,
                        wl.beta if beta is None else beta, wl.lwb if lwb is None else lwb,
                        heads=heads, bound=bound, fp8=fp8, summaries8=summaries)
    sig = None
    boxes = None
    if summaries is not None and len(summaries) == 3:
        sig = summaries[2]
        summaries = summaries[:2]
    if summaries is not None and len(summaries) == 4:
        boxes = summaries[2:]
        summaries = summaries[:2]
    return E.decode(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, wl.q,
                    wl.tau_mode if tau_mode is None else tau_mode, wl.w,
                    wl.bias if bias is None else bias, wl.a if a is None else a,
                    wl.beta if beta is None else beta, wl.lwb if lwb is None else lwb,
                    summaries=summaries, heads=heads, bound=bound, z=z, sigmas=sig, boxes=boxes)


def check_sets_and_counts(wl, res, st):
    """Admitted bitmaps bit-exact, counts exact (in the screen's blocks)."""
    adm = st.admitted(res.admitted.shape[2])
    if not np.array_equal(adm, res.admitted):
        bad = np.argwhere(adm != res.admitted)
        n, h, j = bad[0]
        raise AssertionError(f"admitted sets differ at {len(bad)} places; first (n={n}, h={h}, j={j}): "
                             f"gpu={adm[n, h, j]} oracle={res.admitted[n, h, j]} "
                             f"ub={res.ub[n, h, j]} tau={res.tau[n, h]}")
    np.testing.assert_array_equal(st.admitted_per_head, res.per_head)
    np.testing.assert_array_equal(st.union_per_kv, res.union)
    np.testing.assert_array_equal(st.tokens_per_head, res.tokens)
    np.testing.assert_array_equal(st.rescued.astype(bool), res.rescued)


def check_output(wl, res, o_gpu, heads=None, tol=None):
    tol = TOL[wl.kv_dtype] if tol is None else tol
    if heads is None:
        ref, got = res.o, o_gpu
    else:
        idx = tuple(np.array(list(heads)).T)
        ref, got = res.o[idx], o_gpu[idx]
    assert np.all(np.isfinite(got)), "non-finite output"
    err = float(np.max(np.abs(got - ref)))
    scale = float(np.max(np.abs(ref)))
    log(f"  max|o| = {scale:.4g}, max abs err = {err:.3g} (tolerance {tol:g})")
    assert err <= tol, f"max abs error {err} > {tol}"
    return err


def prepared(name, bound="geometric", z=2.0, fp8="e4m3", block=64, **kw):
    """Workload with thresholds placed and margins enforced (oracle side) for
    the given screen."""
    wl = W.make_workload(name, **kw)
    summ = placement.place(wl, bound=bound, z=z, fp8=fp8, block=block)
    return wl, summ


def fp64_radius_about(wl, mu_bits):
    """max_s ||k_s - mu^|| in float64 for every page/kv head of complete blocks,
    about the given float16 centroids; NaN where no complete block."""
    mu = mu_bits.view(np.float16).astype(np.float64)
    R = np.full(mu.shape[:2], np.nan)
    for n in range(wl.n_seqs):
        nfull = int(wl.seq_lens[n]) // 64
        pages = wl.block_table[n, :nfull]
        for g in range(wl.h_kv):
            k = E.upcast(wl.k_pages[pages, g], wl.kv_dtype)
            d = k - mu[pages, g][:, None, :]
            R[pages, g] = np.sqrt((d * d).sum(axis=2)).max(axis=1)
    return R


__all__ = ["Dev", "oracle_decode", "check_sets_and_counts", "check_output", "prepared", "log", "TOL",
           "fp64_radius_about", "math"]
