#!/usr/bin/env python3
"""ETA decode-step benchmark on one MI355X.

Workload (default): one sequence of 524,288 tokens, GQA 32 query / 8 KV heads,
d = 128, bfloat16 paged KV cache (64-token pages), learned thresholds placed
for ~38% per-head block density, 16 planted needle keys. A step is one full
ETA decode (threshold + bound screen + compaction, split flash-decode over the
admitted blocks with the merge of the splits) for every query head, with the
cache resident in HBM.

Prints one JSON line: decode latency (us/step), achieved HBM bandwidth on the
bytes the step must read, the roofline of the dominant (attend) kernel from HIP
events, a dense comparator (every block admitted, unfiltered softmax) on the
same cache, and the fp64 CPU oracle timed on a bounded sample.

Thresholds are calibrated on the GPU through the library itself (bisection
on each head's bias until its admitted-block count hits the target), so the
timed path never touches the oracle.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
# sources whose change invalidates a stored counter measurement of the attend kernel
ATTEND_SOURCES = ("learned_threshold_block_amd/csrc/eta_attend.hip", "learned_threshold_block_amd/csrc/eta_device.h",
                  "learned_threshold_block_amd/csrc/eta_internal.h", "learned_threshold_block_amd/csrc/eta_screen_dev.h")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="seq_512k", choices=["seq_32k", "batch_4x128k", "seq_512k", "ragged_16"])
    p.add_argument("--density", type=float, default=None, help="per-head target density override")
    p.add_argument("--seq-len", type=int, default=None,
                   help="override the length of every sequence of the workload (the line then names the length "
                        "and carries no stored traffic)")
    p.add_argument("--no-dense", action="store_true", help="skip the dense comparator")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--no-others", action="store_true",
                   help="time only the chosen workload (by default the 512K headline run also times "
                        + ", ".join(OTHER_WORKLOADS) + ")")
    p.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work to time")
    p.add_argument("--sweep", action="store_true", help="also time batch_4x128k at 10/38/70/100%% density")
    p.add_argument("--bound", default="geometric",
                   choices=["geometric", "dual", "quest", "geometric_fp8", "geometric_sub"],
                   help="block screen: the geometric bound, the dual screen (z deviations) or the comparator box bound")
    p.add_argument("--z", type=float, default=2.0, help="deviations of the dual screen")
    p.add_argument("--sub-block", type=int, default=16, choices=[16, 32, 128],
                   help="tokens per screen block for --bound geometric_sub")
    p.add_argument("--calibration", action="store_true",
                   help="only time the offline calibration (16 sequences x 4096 positions, GQA 32/8, d=128, bf16) "
                        "and print its own JSON line")
    p.add_argument("--compare-screens", action="store_true",
                   help="geometric, dual, box-bound and FP8 screens at the same thresholds")
    p.add_argument("--prefill", action="store_true",
                   help="time the causal prompt pass over the seq_32k prompt instead of the decode step")
    p.add_argument("--regime", type=int, default=0, metavar="BATCH",
                   help="only run the block-size ablation at the pages' head shape (G = 8, d = 64, 512K tokens) "
                        "with BATCH sequences and print its own JSON line")
    p.add_argument("--append", action="store_true",
                   help="only time eta_append_kv on the workload's last pages and print its own JSON line")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run a plain device-to-device copy of MIB MiB `steps` times (calibrates the "
                        "HBM byte counters) and exit")
    return p.parse_args()


def attend_sources_sha256():
    import hashlib

    h = hashlib.sha256()
    for rel in ATTEND_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_key(workload, density, bound="geometric", seq_len=None):
    """Name of a decode workload in the committed counter summaries: the
    recipe, the mean per-head target density, and any length or screen that
    differs from the recipe's defaults."""
    return f"{workload}@{density:.2f}" + ("" if seq_len is None else f"-T{seq_len}") + \
        ("" if bound == "geometric" else "-" + bound)


def stored_traffic(workload_key):
    """HBM bytes per attend launch from the committed counter summary (FETCH_SIZE
    + WRITE_SIZE, scaled by the copy-kernel calibration), or None when there is
    none for this workload or the attend kernel's sources changed since."""
    import glob
    import re

    for path in sorted(glob.glob(os.path.join(PROFILES, "*traffic*.md"))):
        with open(path) as f:
            text = f.read()
        fields = dict(re.findall(r"^- (\w+): `([^`]*)`", text, flags=re.M))
        if fields.get("workload_key") != workload_key:
            continue
        if fields.get("attend_sources_sha256") != attend_sources_sha256():
            return None
        return int(fields["traffic_bytes_per_launch"])
    return None


def calibration_bench(steps):
    """Offline calibration (eta_calibrate): 1/t-weighted score histograms over
    16 synthetic sequences of 4096 positions, a query at every position, and
    the per-head search. Times the GPU call with HIP events; the fp64 oracle
    on one (sequence, head) pair, scaled to the whole job."""
    import torch

    import learned_threshold_block_amd as eta
    import workloads as W

    wl = W.make_workload("seq_32k", n_seqs=16, seq_len=4096, needles=0)
    q_all = W.trace_queries(wl, seed=5)
    dev = torch.device("cuda")
    cache = eta.Cache(eta.upload(wl.k_pages, wl.kv_dtype, dev), eta.upload(wl.v_pages, wl.kv_dtype, dev),
                      torch.zeros(wl.num_pages, wl.h_kv, wl.d, dtype=torch.float16, device=dev),
                      torch.zeros(wl.num_pages, wl.h_kv, dtype=torch.float32, device=dev))
    lens = torch.from_numpy(wl.seq_lens.astype(np.int32)).to(dev)
    bt = torch.from_numpy(wl.block_table.astype(np.int32)).to(dev)
    qd = eta.upload(q_all, wl.kv_dtype, dev)
    w = torch.from_numpy(wl.w).to(dev)
    b = torch.full((wl.h_q,), 1.0, dtype=torch.float32, device=dev)
    B, lo, hi = 1024, -8.0, 8.0
    cal = eta.calibrate(cache, lens, bt, qd, B, lo, hi, w=w, b=b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        eta.calibrate(cache, lens, bt, qd, B, lo, hi, w=w, b=b)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    scores = sum(int(T) * (int(T) + 1) // 2 for T in wl.seq_lens) * wl.h_q
    tflops = 2.0 * wl.d * scores / (ms * 1e-3) / 1e12
    dens = (cal.above.double() / cal.total.double()).cpu().numpy()
    # oracle on one (sequence, head): the same histogram in fp64
    import oracle.eta_oracle as E
    from threadpoolctl import threadpool_limits

    one = dict(k_pages=wl.k_pages, kv_dtype=wl.kv_dtype, block_table=wl.block_table[:1], seq_lens=wl.seq_lens[:1],
               q_all=q_all[:1])
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        E.calibration_histogram(one["k_pages"], one["kv_dtype"], one["block_table"], one["seq_lens"], one["q_all"],
                                0, wl.group, lo, hi, B, w_h=wl.w[0], b_h=1.0)
        cpu_s = (time.perf_counter() - t0) * wl.n_seqs * wl.h_q
    print(json.dumps({
        "metric": "ETA offline calibration (1/t-weighted score histograms + per-head search), ms per job",
        "value": round(ms, 3), "unit": "ms", "higher_is_better": False, "steps": steps, "data": "synthetic",
        "config": {"workload": "16 seqs x 4096 positions, a query at every position, GQA 32/8, d=128, bf16 keys, "
                               "learned predictor w ~ N(0, 1/d), b = 1.0, 1024 bins over [-8, 8)",
                   "scores": scores},
        "dtype": "f32",
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4), "traffic": None,
                     "note": "2*d flops per scored (query, key) pair on bf16 matrix cores; each score is then "
                             "binned with one 64-bit LDS atomic add, which is what the kernel waits on"},
        "training_density_mean": round(float(dens.mean()), 4),
        "calibrated_c_mean": round(float(cal.c.mean().item()), 4),
        "cpu_baseline": {"value": round(cpu_s * 1e3, 1), "unit": "ms", "cores": 1, "kind": "oracle",
                         "sample": "one (sequence, head) pair of fp64 NumPy histogramming, scaled by 16 x 32"},
    }), flush=True)


def compare_screens(workload, density, steps, warmup, z):
    """The screens at the same thresholds (placed for the geometric bound at
    the workload's target density): admitted fraction per head and per KV head,
    and the decode step time, for the geometric bound, the dual score, the
    comparator's box bound (Section 4.3), the geometric bound over E4M3
    records, and the geometric bound on 16-, 32- and 128-token screen blocks
    (Appendix F.3's block size; densities in those blocks)."""
    S = Setup(workload, density, "all", z)
    S.calibrate()
    rows = {}
    for b in ("geometric", "dual", "quest", "geometric_fp8", "geometric_sub", "geometric_sub32", "geometric_sub128"):
        if b in ("geometric_sub32", "geometric_sub128"):
            S.use_sub_block(int(b[len("geometric_sub"):]))
        S.bound = "geometric_sub" if b.startswith("geometric_sub") else b
        S.run()
        S.torch.cuda.synchronize()
        st, dh, du = S.densities()
        us = time_steps(S, steps, warmup)
        ph = time_phases(S, steps)
        key = {"geometric_sub": "geometric_b16", "geometric_sub32": "geometric_b32",
               "geometric_sub128": "geometric_b128"}.get(b, b)
        rows[key] = {"density_per_head": round(dh, 4), "density_union": round(du, 4), "us_per_step": round(us, 2),
                   "screen_us": round(float(ph[0]), 2), "attend_and_merge_us": round(float(ph[1]), 2)}
        log(f"{key}: per-head {dh:.4f} union {du:.4f} step {us:.1f} us")
    wl = S.wl
    print(json.dumps({
        "metric": "block screens at equal thresholds: admitted density and decode step time",
        "unit": "us/step", "higher_is_better": False, "steps": steps, "warmup": warmup, "data": "synthetic",
        "dtype": wl.kv_dtype,
        "config": {"workload": f"{workload}: {wl.n_seqs} x {int(wl.seq_lens.max())} tokens, GQA {wl.h_q}/{wl.h_kv}, "
                               f"d={wl.d}; thresholds placed for the geometric bound at per-head density "
                               f"{float(np.mean(wl.target_density)):.2f}; dual z={z:g}"},
        "screens": rows,
    }), flush=True)


def regime_bench(batch, steps, warmup):
    """The head shape of the pages' decode benchmark (Table 5 and Table 10 of
    the ETA page): 32 query heads over 4 KV heads (G = 8), d = 64, 64-token
    pages, `batch` sequences of 524,288 tokens (batch 64: a 32 GiB cache, the
    size Table 10 names), frozen per-head constants (the calibrated mode),
    queries correlated within each group. Two settings:
    per-head density 0.38 with rho = 0.97 (about half the blocks in each
    group's union) and per-head density 0.10 with rho = 0.98 (about a sixth).
    For each: thresholds bisected for the per-head density on 64-token blocks;
    then the geometric screen on 16-, 32-, 64- and 128-token blocks at those
    thresholds (densities counted in each size's blocks), and the dense
    comparator (every block, plain softmax) on the same cache."""
    import torch

    import workloads as W

    S = Setup("table5_512k", 0.38, "geometric_sub", 2.0, 16, None, n_seqs=batch)
    wl = S.wl
    settings = {}
    for dens, rho in ((0.38, 0.97), (0.10, 0.98)):
        if rho != W.recipe("table5_512k")["rho"] or dens != 0.38:
            # same keys and values; only the queries (a function of rho) and the targets change
            wq = W.make_workload("table5_512k", n_seqs=batch, seq_len=64, rho=rho)
            wl.q = wq.q
            S.q.copy_(S.eta.upload(wq.q, wl.kv_dtype, "cuda"))
        wl.target_density = np.full(wl.h_q, dens)
        S.bound = "geometric"
        S.calibrate()
        rows = {}
        dense_us = None
        for b in (64, 16, 32, 128, "dense"):
            if b == "dense":
                saved, mode = S.bias.clone(), S.mode
                S.bias.fill_(-math.inf)
                S.mode = S.eta.ETA_TAU_CALIBRATED
                S.bound = "geometric"
            elif b == 64:
                S.bound = "geometric"
            else:
                if S.sub_block != b:
                    S.use_sub_block(b)
                S.bound = "geometric_sub"
            st, dh, du = S.densities()
            kv, _ = S.step_bytes(st)
            us = time_steps(S, steps, warmup)
            ph = time_phases(S, steps)
            row = {"density_per_head": round(dh, 4), "density_union": round(du, 4), "us_per_step": round(us, 2),
                   "screen_us": round(float(ph[0]), 2), "attend_and_merge_us": round(float(ph[1]), 2),
                   "attend_gbs_union_kv": round(kv / (ph[1] * 1e-6) / 1e9, 1),
                   "attend_frac_of_peak": round(kv / (ph[1] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
            if b == "dense":
                S.bias.copy_(saved)
                S.mode = mode
                dense_us = us
            rows["dense" if b == "dense" else f"b{b}"] = row
            log(f"regime per-head {dens} rho {rho}: {b}: per-head {dh:.3f} union {du:.3f} step {us:.1f} us "
                f"attend {ph[1]:.1f} us")
        for key, row in rows.items():
            if key != "dense":
                row["speedup_vs_dense"] = round(dense_us / row["us_per_step"], 3)
        settings[f"per_head_{dens:.2f}_rho_{rho:.2f}"] = {"rho": rho, "target_density_per_head": dens,
                                                          "screens": rows}
    print(json.dumps({
        "metric": "block-size ablation at the pages' decode head shape: step time, densities, attend bandwidth",
        "unit": "us/step", "higher_is_better": False, "steps": steps, "warmup": warmup, "data": "synthetic",
        "dtype": wl.kv_dtype, "n_gpus": 1,
        "config": {"workload": f"table5_512k: {wl.n_seqs} x {int(wl.seq_lens.max())} tokens, GQA {wl.h_q}/{wl.h_kv} "
                               f"(G = {wl.group}), d={wl.d}, {wl.kv_dtype} paged KV, {wl.kv_bytes() / 2**30:.1f} GiB; "
                               "calibrated per-head constants bisected on 64-token blocks, the other block sizes at the same "
                               "thresholds"},
        "settings": settings,
    }), flush=True)
    del S
    torch.cuda.empty_cache()


def prefill_bench(steps, warmup, cpu_budget, no_cpu):
    """Causal prompt pass (eta_prefill) over the 32768-token prompt of the
    seq_32k workload (1 sequence, GQA 32/8, d=128, bf16): the gated rule at
    every position plus the records of every block. Times the entry point
    with HIP events on the launch stream; the roofline counts the method's
    flops (4 d per causal (query, key) pair and head). Context: torch's fused
    causal attention (no gate) on the same shapes, and the fp64 oracle on a
    sample of rows of one head, scaled to the whole job."""
    import torch

    import learned_threshold_block_amd as eta
    import workloads as W

    wl = W.make_workload("seq_32k")
    q_all = W.trace_queries(wl, seed=21)
    dev = torch.device("cuda")
    cache = eta.Cache(eta.upload(wl.k_pages, wl.kv_dtype, dev), eta.upload(wl.v_pages, wl.kv_dtype, dev),
                      torch.zeros(wl.num_pages, wl.h_kv, wl.d, dtype=torch.float16, device=dev),
                      torch.zeros(wl.num_pages, wl.h_kv, dtype=torch.float32, device=dev))
    lens = torch.from_numpy(wl.seq_lens.astype(np.int32)).to(dev)
    bt = torch.from_numpy(wl.block_table.astype(np.int32)).to(dev)
    qd = eta.upload(q_all, wl.kv_dtype, dev)
    w = torch.from_numpy(wl.w).to(dev)
    bias = np.linspace(-1.0, 2.5, wl.h_q).astype(np.float32)
    b = torch.from_numpy(bias).to(dev)
    out = torch.empty(wl.n_seqs, q_all.shape[1], wl.h_q, wl.d, dtype=torch.float32, device=dev)
    for _ in range(warmup):
        eta.prefill(cache, lens, bt, qd, eta.ETA_TAU_LEARNED, b, w=w, beta=5.0, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        res = eta.prefill(cache, lens, bt, qd, eta.ETA_TAU_LEARNED, b, w=w, beta=5.0, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    assert int(res.err.item()) == 0
    T = int(wl.seq_lens[0])
    pairs = T * (T + 1) // 2
    flops = 4.0 * wl.d * pairs * wl.h_q
    tflops = flops / (ms * 1e-3) / 1e12
    tokens_s = T / (ms * 1e-3)
    # context: torch's fused causal attention on the same shapes, without the gate
    qt = qd[0].transpose(0, 1).contiguous()[None]                   # [1][HQ][T][d]
    pages = torch.from_numpy(wl.block_table[0].astype(np.int64)).to(dev)
    kt = cache.k_pages[pages].transpose(0, 1).reshape(wl.h_kv, T, wl.d)[None].contiguous()
    vt = cache.v_pages[pages].transpose(0, 1).reshape(wl.h_kv, T, wl.d)[None].contiguous()
    sdpa = lambda: torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,  # noqa: E731
                                                                    enable_gqa=True)
    try:
        for _ in range(2):
            sdpa()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            sdpa()
        e1.record()
        torch.cuda.synchronize()
        sdpa_ms = round(e0.elapsed_time(e1) / steps, 3)
    except RuntimeError as ex:  # a backend without grouped heads or this size
        sdpa_ms = f"unavailable: {ex}"[:120]
    cpu = None
    if not no_cpu:
        import oracle.eta_oracle as E
        from threadpoolctl import threadpool_limits

        rows = np.random.default_rng(3).choice(T, size=256, replace=False)
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            reps = 0
            while True:
                E.prefill(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, q_all, "learned", wl.w,
                          bias, 0.0, 5.0, heads=[(0, reps % wl.h_q)], positions=rows)
                reps += 1
                if time.perf_counter() - t0 > cpu_budget / 2:
                    break
            el = time.perf_counter() - t0
        sample_pairs = int((rows + 1).sum()) * reps
        cpu_s = el * (pairs * wl.h_q) / sample_pairs
        cpu = {"value": round(T / cpu_s, 2), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"{reps} x (256 random rows of one head) of the fp64 oracle, scaled by causal pairs "
                         f"to all {T} rows x {wl.h_q} heads"}
    print(json.dumps({
        "metric": "ETA causal prefill throughput (gated attention at every prompt position + block records)",
        "value": round(tokens_s, 1), "unit": "tokens/s", "higher_is_better": True, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 3), "data": "synthetic", "dtype": "bf16",
        "config": {"workload": "seq_32k prompt: 1 x 32768 tokens, GQA 32/8, d=128, bf16 K/V/q, learned threshold "
                               "(w ~ N(0, 1/d), b_h linearly spaced in [-1, 2.5]), beta 5",
                   "causal_pairs_per_head": pairs},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(tflops / 2500.0, 4), "traffic": None,
                     "note": "4*d flops per causal (query, key) pair and head, P times V in float16 (V within "
                             "float16's exact range); bound by vector issue, not the matrix cores: the gate and the "
                             "softmax take about 11.6 vector instructions per logit, 3 of them transcendental"},
        "torch_sdpa_causal_ungated_ms": sdpa_ms,
        "cpu_baseline": cpu,
    }), flush=True)


def append_bench(workload, steps, warmup):
    """eta_append_kv: one new token per (sequence, KV head) written into its
    page slot, with the record of the page built when the token fills slot 63.
    Times both kinds of call on the last page of every sequence of the
    workload (the sequence lengths set just below that page's slot 5 and slot
    63), with HIP events on the launch stream and the calls back to back on
    the GPU (the host's enqueue time per call is reported beside). The bytes
    counted are the new K and V rows, plus the filled page's K rows read and
    its record written; a call moves kilobytes, so it is bound by launch
    latency, not by HBM."""
    import torch

    import learned_threshold_block_amd as eta
    import workloads as W

    wl = W.make_workload(workload)
    dev = torch.device("cuda")
    cache = eta.Cache(eta.upload(wl.k_pages, wl.kv_dtype, dev), eta.upload(wl.v_pages, wl.kv_dtype, dev),
                      torch.zeros(wl.num_pages, wl.h_kv, wl.d, dtype=torch.float16, device=dev),
                      torch.zeros(wl.num_pages, wl.h_kv, dtype=torch.float32, device=dev))
    bt = torch.from_numpy(wl.block_table.astype(np.int32)).to(dev)
    rng = np.random.default_rng(11)
    shape = (wl.n_seqs, wl.h_kv, wl.d)
    kvt = torch.bfloat16 if wl.kv_dtype == "bf16" else torch.float32
    k_new = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(dev).to(kvt)
    v_new = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(dev).to(kvt)
    last = (wl.seq_lens.astype(np.int64) - 1) // 64 * 64  # first token of each sequence's last page
    esz = 2 if wl.kv_dtype == "bf16" else 4
    rows = wl.n_seqs * wl.h_kv
    host_us = {}
    # A call costs the host more than the kernel takes, so the calls are
    # enqueued behind copies of the V pages that keep the GPU busy until the
    # last call is queued: the events then time the kernels back to back.
    ahead = torch.empty_like(cache.v_pages)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    v_bytes = cache.v_pages.numel() * esz
    n_ahead = max(2, math.ceil(steps * 120e-6 / (2 * v_bytes / 4e12)))  # ~120 us of GPU work per call queued
    res = {}
    for name, slot in (("row", 5), ("row_and_record", 63)):
        lens = torch.from_numpy((last + slot).astype(np.int32)).to(dev)
        for _ in range(warmup):
            eta.append_kv(cache, lens, bt, k_new, v_new)
        torch.cuda.synchronize()
        c0, e0, e1 = ev(), ev(), ev()
        c0.record()
        for _ in range(n_ahead):
            ahead.copy_(cache.v_pages)
        e0.record()
        h0 = time.perf_counter()
        for _ in range(steps):
            eta.append_kv(cache, lens, bt, k_new, v_new)
        host_s = time.perf_counter() - h0
        e1.record()
        torch.cuda.synchronize()
        if host_s * 1e3 >= c0.elapsed_time(e0):
            raise RuntimeError("the copies ahead ran out before the last call was queued")
        us = e0.elapsed_time(e1) / steps * 1e3
        host_us[name] = host_s / steps * 1e6
        nbytes = rows * 2 * wl.d * esz * 2  # new K and V rows: read, then written into the page
        if slot == 63:
            nbytes += rows * (64 * wl.d * esz + wl.d * 2 + 4)  # the page's K rows read, its record written
        res[name] = (us, nbytes)
    us, nbytes = res["row_and_record"]
    gbs = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "ETA append latency (one token per sequence and KV head; the call that fills a page also "
                  "builds its record)",
        "value": round(us, 2), "unit": "us/call", "higher_is_better": False, "steps": steps, "warmup": warmup,
        "data": "synthetic", "dtype": wl.kv_dtype,
        "config": {"workload": f"{workload}: {wl.n_seqs} sequences x {wl.h_kv} KV heads, d={wl.d}, "
                               f"{wl.kv_dtype} K/V, the last page of every sequence"},
        "row_only_us": round(res["row"][0], 2),
        "host_enqueue_us": round(host_us["row_and_record"], 2),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": 8000.0, "unit": "GB/s",
                     "frac": round(gbs / 8000.0, 5), "traffic": None,
                     "note": f"{nbytes} bytes per call (new K and V rows read and written, the filled page's K "
                             "rows read, its record written): launch latency bound"},
        "cpu_baseline": None,
    }), flush=True)


def copy_probe(mib, steps):
    """A plain copy of a known size, for the counter calibration."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) / steps * 1e6
    print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4, "steps": steps,
                      "us_per_copy": round(us, 2), "gbs_read_plus_write": round(2 * n * 4 / (us * 1e-6) / 1e9, 1)}),
          flush=True)


class Setup:
    """One workload resident on the GPU."""

    def __init__(self, name, density=None, bound="geometric", z=2.0, sub_block=16, seq_len=None, **gen):
        import torch

        import learned_threshold_block_amd as eta
        import workloads as W

        t0 = time.time()
        kw = dict(gen) if density is None else dict(gen, density=density)
        if seq_len is not None:
            kw["seq_len"] = seq_len
        self.wl = wl = W.make_workload(name, **kw)
        log(f"{name}: generated {wl.kv_bytes() / 1e9:.2f} GB of K/V in {time.time() - t0:.1f}s")
        self.eta, self.torch = eta, torch
        dev = torch.device("cuda")
        self.bound, self.z = bound, z
        z16 = lambda: torch.zeros(wl.num_pages, wl.h_kv, wl.d, dtype=torch.float16, device=dev)  # noqa: E731
        sig = z16() if bound in ("dual", "all") else None
        lo, hi = (z16(), z16()) if bound in ("quest", "all") else (None, None)
        fp8 = bound in ("geometric_fp8", "all")
        mu8 = torch.zeros(wl.num_pages, wl.h_kv, wl.d, dtype=torch.uint8, device=dev) if fp8 else None
        r8 = torch.zeros(wl.num_pages, wl.h_kv, dtype=torch.float32, device=dev) if fp8 else None
        self.sub_block = sub_block if bound in ("geometric_sub", "all") else 0
        sb = eta.sub_slots(self.sub_block) if self.sub_block else 0
        mus = torch.zeros(wl.num_pages, wl.h_kv, sb, wl.d, dtype=torch.float16, device=dev) if sb else None
        rs = torch.zeros(wl.num_pages, wl.h_kv, sb, dtype=torch.float32, device=dev) if sb else None
        if bound == "all":  # every record, for comparisons at equal thresholds
            self.bound = "geometric"
        self.cache = eta.Cache(eta.upload(wl.k_pages, wl.kv_dtype, dev), eta.upload(wl.v_pages, wl.kv_dtype, dev),
                               torch.zeros(wl.num_pages, wl.h_kv, wl.d, dtype=torch.float16, device=dev),
                               torch.zeros(wl.num_pages, wl.h_kv, dtype=torch.float32, device=dev), sig, lo, hi,
                               mu8, r8, "e4m3", self.sub_block, mus, rs)
        self.seq_lens = torch.from_numpy(wl.seq_lens.astype(np.int32)).to(dev)
        self.bt = torch.from_numpy(wl.block_table.astype(np.int32)).to(dev)
        self.q = eta.upload(wl.q, wl.kv_dtype, dev)
        self.w = torch.from_numpy(wl.w).to(dev)
        self.ws = eta.alloc_workspace(self.cache, wl.n_seqs, wl.max_blocks, wl.h_q)
        self.out = torch.empty(wl.n_seqs, wl.h_q, wl.d, dtype=torch.float32, device=dev)
        self.mode = eta.ETA_TAU_LEARNED if wl.tau_mode == "learned" else eta.ETA_TAU_CALIBRATED
        eta.build_block_summaries(self.cache, self.seq_lens, self.bt)
        torch.cuda.synchronize()
        self._rotation()
        self.nblk = np.array([wl.nblk(n) for n in range(wl.n_seqs)], dtype=np.float64)
        self.bias = torch.zeros(wl.h_q, dtype=torch.float32, device=dev)

    def _rotation(self):
        """A K/V cache small enough to stay in the 256 MB last-level cache
        (MALL) between steps would be timed from there: keep identical copies
        (same pages, same records) of at least 600 MB in all and let each call
        use the next one, so every step reads cold data."""
        import dataclasses
        ncopy = max(1, -(-600_000_000 // self.wl.kv_bytes()))
        c = self.cache
        clone = lambda: dataclasses.replace(c, **{f.name: getattr(c, f.name).clone()  # noqa: E731
                                                  for f in dataclasses.fields(c)
                                                  if isinstance(getattr(c, f.name), self.torch.Tensor)})
        self.caches = [c] + [clone() for _ in range(ncopy - 1)]
        self.rot = 0

    def run(self, phase=None, bias=None, mode=None):
        cache = self.caches[self.rot]
        self.rot = (self.rot + 1) % len(self.caches)
        self.eta.decode(cache, self.seq_lens, self.bt, self.q, self.mode if mode is None else mode,
                        self.bias if bias is None else bias, w=self.w, a=self.wl.a, beta=self.wl.beta,
                        lwb=self.wl.lwb, out=self.out, workspace=self.ws, phase=phase, bound=self.bound, z=self.z)

    def stats(self):
        wl = self.wl
        return self.eta.stats(self.ws, wl.n_seqs, wl.max_blocks, wl.h_q, wl.h_kv, bitmap=False)

    def launches(self):
        """1 when a step of this setup runs as one launch (short segments), 2
        when it runs as the screen phase and the attend phase."""
        return self.eta.decode_launches(self.cache, self.seq_lens, self.bt, self.wl.h_q, bound=self.bound)

    def calibrate(self, iters=40):
        """Bisect each head's bias/constant so that its admitted fraction of
        blocks (averaged over sequences) reaches the workload's target."""
        wl, torch = self.wl, self.torch
        target = wl.target_density
        if np.all(target >= 1.0):
            self.bias.fill_(-math.inf)
            return
        lo = np.full(wl.h_q, -64.0)
        hi = np.full(wl.h_q, 64.0)
        for _ in range(iters):
            mid = 0.5 * (lo + hi)
            self.bias.copy_(torch.from_numpy(mid.astype(np.float32)))
            self.run(phase=self.eta.ETA_PHASE_SCREEN)
            b = self.block_tokens()
            nb = np.array([-(-int(T) // b) for T in wl.seq_lens], dtype=np.float64)
            dens = (self.stats().admitted_per_head / nb[:, None]).mean(axis=0)
            lo = np.where(dens > target, mid, lo)
            hi = np.where(dens > target, hi, mid)
        self.bias.copy_(torch.from_numpy((0.5 * (lo + hi)).astype(np.float32)))
        self.bias[target >= 1.0] = -math.inf

    def block_tokens(self):
        """Tokens per screen block of the current screen."""
        return self.sub_block if self.bound == "geometric_sub" else 64

    def densities(self):
        """Per-head and union admitted fractions of the current thresholds
        (one decode first, so the counts are those of this setup)."""
        self.run()
        st = self.stats()
        b = self.block_tokens()
        nb = np.array([-(-int(T) // b) for T in self.wl.seq_lens], dtype=np.float64)
        per_head = float((st.admitted_per_head / nb[:, None]).mean())
        union = float((st.union_per_kv / nb[:, None]).mean())
        return st, per_head, union

    def use_sub_block(self, sub_block):
        """Records of another screen block size (same K/V and thresholds)."""
        eta, torch, wl = self.eta, self.torch, self.wl
        sb = eta.sub_slots(sub_block)
        c = self.cache
        self.cache = eta.Cache(c.k_pages, c.v_pages, c.mu, c.radius, c.sigma, c.kmin, c.kmax, c.mu8, c.radius8,
                               c.mu8_format, sub_block,
                               torch.zeros(wl.num_pages, wl.h_kv, sb, wl.d, dtype=torch.float16, device=c.mu.device),
                               torch.zeros(wl.num_pages, wl.h_kv, sb, dtype=torch.float32, device=c.mu.device))
        self.sub_block = sub_block
        self.ws = eta.alloc_workspace(self.cache, wl.n_seqs, wl.max_blocks, wl.h_q)
        eta.build_block_summaries(self.cache, self.seq_lens, self.bt)
        torch.cuda.synchronize()
        self._rotation()

    def step_bytes(self, st):
        """Bytes one step must move: admitted K/V tiles once per union block,
        the records the screen reads for every complete block, the block
        table, the queries/thresholds and the output."""
        wl = self.wl
        esz = 2 if wl.kv_dtype == "bf16" else 4
        b = self.block_tokens()
        union = int(st.union_per_kv.sum())
        if b > 64:  # a block's pages: a partial last block (always loaded) may have only its first page
            one_page = sum(1 for T in wl.seq_lens if 0 < int(T) % b <= 64)
            kv = (union * (b // 64) - one_page * wl.h_kv) * 2 * 64 * wl.d * esz
        else:
            kv = union * 2 * b * wl.d * esz
        nfull = int(sum(int(wl.seq_lens[n]) // 64 for n in range(wl.n_seqs)))
        # records the screen reads per complete page: centroid and radius (and
        # the deviation), or the key box; 64/b records of b-token blocks
        rec = {"geometric": 2 * wl.d + 4, "dual": 4 * wl.d + 4, "quest": 4 * wl.d,
               "geometric_fp8": wl.d + 4, "geometric_sub": (2 * wl.d + 4) * 64 / max(b, 1)}[self.bound]
        meta = int(nfull * wl.h_kv * rec) + int(self.nblk.sum()) * 4
        small = wl.n_seqs * wl.h_q * wl.d * (esz + 4) + wl.h_q * wl.d * 4
        return kv, kv + meta + small


def time_steps(S, steps, warmup):
    """Wall-clock time per decode step over `steps` back-to-back eta_decode
    calls (after `warmup`), bracketed by device synchronisation."""
    torch = S.torch
    for _ in range(warmup):
        S.run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        S.run()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e6


def time_phases(S, steps):
    """Average duration (us) of each phase's launches: HIP events on the launch
    stream around `steps` back-to-back launches of that phase alone (screen +
    finalize; attend with the merge of the splits). Each phase is idempotent
    given the previous phase's workspace contents, so repeating it measures
    the kernels themselves without the gaps that events between phases would
    add to a step."""
    eta, torch = S.eta, S.torch
    S.run()
    torch.cuda.synchronize()
    out = []
    for phase in (eta.ETA_PHASE_SCREEN, eta.ETA_PHASE_ATTEND):
        S.run(phase=phase)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            S.run(phase=phase)
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / steps * 1e3)
    return np.array(out)


def time_one_launch(S, steps):
    """Average duration (us) of a step that runs as one launch: HIP events on
    the launch stream around `steps` back-to-back eta_decode calls."""
    torch = S.torch
    S.run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        S.run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps * 1e3


def two_launch_step_us(S, steps, warmup):
    """Step time of the same setup forced into its two launches (ETA_FUSED=0)."""
    old = os.environ.get("ETA_FUSED")
    os.environ["ETA_FUSED"] = "0"
    try:
        return time_steps(S, steps, warmup)
    finally:
        if old is None:
            del os.environ["ETA_FUSED"]
        else:
            os.environ["ETA_FUSED"] = old


def cpu_baseline(S, budget_s):
    """The fp64 oracle's decode step on one (sequence, KV head) segment at a
    time, single-threaded, for about `budget_s` seconds; scaled to a full step.
    (Its NumPy products on 16 BLAS threads made the 512K step slower, 3.32 s
    against 1.94 s on one thread: the products per block are too small.)"""
    from threadpoolctl import threadpool_limits

    import oracle.eta_oracle as E

    wl = S.wl
    G = wl.group
    bias = S.bias.cpu().numpy()
    segs = [(n, g) for n in range(wl.n_seqs) for g in range(wl.h_kv)]
    done, elapsed, blocks_done = 0, 0.0, 0
    with threadpool_limits(limits=1):
        for (n, g) in segs:
            sub = dict(k_pages=wl.k_pages[:, g:g + 1], v_pages=wl.v_pages[:, g:g + 1])
            bt = wl.block_table[n:n + 1]
            lens = wl.seq_lens[n:n + 1]
            summ = E.build_summaries(sub["k_pages"], wl.kv_dtype, bt, lens)  # records: built once, not timed
            q = wl.q[n:n + 1, g * G:(g + 1) * G]
            t0 = time.perf_counter()
            E.decode(sub["k_pages"], sub["v_pages"], wl.kv_dtype, bt, lens, q, wl.tau_mode,
                     wl.w[g * G:(g + 1) * G], bias[g * G:(g + 1) * G], wl.a, wl.beta, wl.lwb, summaries=summ)
            elapsed += time.perf_counter() - t0
            done += 1
            blocks_done += wl.nblk(n)
            if elapsed >= budget_s:
                break
    total_blocks = sum(wl.nblk(n) for (n, g) in segs)
    per_step_s = elapsed * total_blocks / blocks_done
    return {"value": per_step_s * 1e6, "unit": "us/step", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {len(segs)} (sequence, KV head) segments ({G} query heads each), "
                      f"{elapsed:.1f}s of single-threaded fp64 NumPy, scaled by blocks to the full step",
            "cpu": host_cpu_model()}


def host_cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def describe(S, workload, seq_len, bound="geometric", z=2.0, sub_block=16):
    """The workload's name for the JSON line: shapes, dtype, thresholds, screen."""
    wl = S.wl
    base = ({"seq_32k": "1 seq x 32768 ctx", "batch_4x128k": "4 seq x 131072 ctx",
             "seq_512k": "1 seq x 524288 ctx", "ragged_16": "16 ragged seqs 4K-256K"}[workload]
            if seq_len is None else f"{wl.n_seqs} seq x {seq_len} ctx")
    dens = "per-head density U[0.05, 0.90]" if workload == "ragged_16" else \
        f"target per-head density {float(np.mean(wl.target_density)):.2f}"
    return (base + f", GQA {wl.h_q}/{wl.h_kv}, d={wl.d}, {wl.kv_dtype} paged KV (64-token pages), "
            + f"{wl.tau_mode} thresholds, {dens}, {len(wl.needles)} needle keys"
            + {"geometric": "", "dual": f", dual screen z={z:g}", "quest": ", comparator box-bound screen",
               "geometric_fp8": ", geometric screen over E4M3 records",
               "geometric_sub": f", geometric screen on {sub_block}-token blocks"}[bound])


def measure(S, workload, steps, warmup, bound="geometric", seq_len=None):
    """Step time, densities, bandwidths, phase times and the attend kernel's
    roofline of one calibrated workload."""
    st, dens_head, dens_union = S.densities()
    kv_bytes, all_bytes = S.step_bytes(st)
    log(f"{workload}: density per-head {dens_head:.3f} union {dens_union:.3f}; union K/V {kv_bytes / 1e9:.3f} GB")
    us = time_steps(S, steps, warmup)
    ph = time_phases(S, steps)
    log(f"{workload}: step {us:.1f} us; phases screen / attend+merge {ph[0]:.1f} / {ph[1]:.1f} us")
    wl = S.wl
    esz = 2 if wl.kv_dtype == "bf16" else 4
    U = int(st.union_per_kv.sum())  # union blocks in the screen's block size
    # K/V rows of the union's blocks (kv_bytes follows the screen's block size),
    # one 8-byte entry per block, the queries
    attend_bytes = kv_bytes + U * 8 + wl.n_seqs * wl.h_q * wl.d * esz
    attend_gbs = attend_bytes / (ph[1] * 1e-6) / 1e9
    key = traffic_key(workload, float(np.mean(wl.target_density)), bound, seq_len)
    kernel, kbytes, kus = "k_attend", attend_bytes, ph[1]
    extra = {}
    if S.launches() == 1:
        # the whole step is one kernel: its algorithmic bytes are the step's
        # (union K/V, every complete block's record read once, the block
        # table, queries, predictor weights and the output)
        kus = time_one_launch(S, steps)
        kbytes = all_bytes
        kernel = "k_attend (one launch: screen, attend, merge)"
        two = two_launch_step_us(S, steps, warmup)
        log(f"{workload}: one launch {kus:.1f} us (events); the same step as two launches {two:.1f} us")
        extra = {"one_launch_us": round(kus, 2), "two_launch_us_per_step": round(two, 2)}
    kgbs = kbytes / (kus * 1e-6) / 1e9
    return {
        **extra,
        "us_per_step": round(us, 2),
        "density_per_head": round(dens_head, 4),
        "density_union": round(dens_union, 4),
        "achieved_gbs_union_kv": round(kv_bytes / (us * 1e-6) / 1e9, 1),
        "achieved_gbs_all_bytes": round(all_bytes / (us * 1e-6) / 1e9, 1),
        "phase_us": {"screen": round(float(ph[0]), 2), "attend_and_merge": round(float(ph[1]), 2)},
        "roofline": {"bound": "hbm", "achieved": round(kgbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(kgbs / PEAK_HBM_GBS, 4), "traffic": stored_traffic(key),
                     "kernel": kernel, "bytes_per_launch": int(kbytes)},
    }


# The other configurations of the benchmark's workload set, timed after the
# headline one in the default run: 4 x 128K (the metric's 128K context, config
# with calibrated per-head constants at 38% per-head density), one 32K
# sequence, and 16 ragged sequences on a paged cache in random page order.
OTHER_WORKLOADS = ("batch_4x128k", "seq_32k", "ragged_16")


def other_workloads(steps, warmup):
    import torch

    out = {}
    for name in OTHER_WORKLOADS:
        S = Setup(name)
        S.calibrate()
        m = measure(S, name, steps, warmup)
        m["config"] = describe(S, name, None)
        m["kv_copies_rotated"] = len(S.caches)
        out[name] = m
        del S
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(args.copy_probe, args.steps)
        return
    if args.calibration:
        calibration_bench(max(3, min(args.steps, 20)))
        return
    if args.compare_screens:
        compare_screens(args.workload, args.density, max(5, min(args.steps, 50)), min(args.warmup, 5), args.z)
        return
    if args.regime:
        regime_bench(args.regime, max(5, min(args.steps, 20)), min(args.warmup, 3))
        return
    if args.append:
        append_bench(args.workload, max(20, min(args.steps * 2, 100)), max(3, args.warmup))
        return
    if args.prefill:
        prefill_bench(max(2, min(args.steps, 20)), min(args.warmup, 3), args.cpu_budget, args.no_cpu)
        return

    S = Setup(args.workload, args.density, args.bound, args.z, args.sub_block, args.seq_len)
    S.calibrate()
    m = measure(S, args.workload, args.steps, args.warmup, args.bound, args.seq_len)
    us = m["us_per_step"]
    wl = S.wl
    result = {
        "metric": "ETA decode us/step + achieved HBM GB/s at 128K/512K ctx, ~38% block density",
        "value": us,
        "unit": "us/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": describe(S, args.workload, args.seq_len, args.bound, args.z, args.sub_block),
            "kv_dtype": wl.kv_dtype,
            "screen": f"dual z={args.z:g}" if args.bound == "dual" else args.bound,
            "seq_lens_total": int(wl.seq_lens.sum()),
            "density_per_head": m["density_per_head"],
            "density_union": m["density_union"],
            "kv_copies_rotated": len(S.caches),
        },
        "achieved_gbs_union_kv": m["achieved_gbs_union_kv"],
        "achieved_gbs_all_bytes": m["achieved_gbs_all_bytes"],
        "phase_us": m["phase_us"],
        **{k: m[k] for k in ("one_launch_us", "two_launch_us_per_step") if k in m},
        "roofline": m["roofline"],
    }
    if not args.no_dense:
        dense_bias = torch.full((wl.h_q,), -math.inf, device="cuda")
        saved = S.bias.clone()
        S.bias.copy_(dense_bias)
        mode_saved = S.mode
        S.mode = S.eta.ETA_TAU_CALIBRATED
        S.run()
        dst, _, dunion = S.densities()
        dkv, dall = S.step_bytes(dst)
        dus = time_steps(S, max(10, args.steps // 2), 3)
        dph = time_phases(S, max(10, args.steps // 2))
        result["dense_comparator"] = {"us_per_step": round(dus, 2), "density_union": round(dunion, 4),
                                      "achieved_gbs_kv": round(dkv / (dus * 1e-6) / 1e9, 1),
                                      "attend_us": round(float(dph[1]), 2),
                                      "speedup_eta_vs_dense": round(dus / us, 3)}
        S.bias.copy_(saved)
        S.mode = mode_saved
        log(f"dense comparator {dus:.1f} us")
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(S, args.cpu_budget)
        log(f"cpu baseline {result['cpu_baseline']['value'] / 1e3:.1f} ms/step")
    if not args.no_others and args.workload == "seq_512k" and args.seq_len is None and args.bound == "geometric" \
            and args.density is None:
        del S
        torch.cuda.empty_cache()
        result["workloads"] = other_workloads(max(10, args.steps // 2), min(args.warmup, 5))
        S = None
    if args.sweep:
        del S
        torch.cuda.empty_cache()
        sw = {}
        for dens in (0.10, 0.38, 0.70, 1.0):
            S2 = Setup("batch_4x128k", dens)
            S2.calibrate()
            st2, dh, du = S2.densities()
            k2, a2 = S2.step_bytes(st2)
            us2 = time_steps(S2, max(10, args.steps // 2), 3)
            ph2 = time_phases(S2, max(10, args.steps // 2))
            sw[f"{int(dens * 100)}%"] = {"us_per_step": round(us2, 2), "density_per_head": round(dh, 4),
                                        "density_union": round(du, 4),
                                        "achieved_gbs_kv": round(k2 / (us2 * 1e-6) / 1e9, 1),
                                        "attend_us": round(float(ph2[1]), 2)}
            log(f"batch_4x128k {dens}: {us2:.1f} us, union {du:.3f}")
            del S2
            torch.cuda.empty_cache()
        result["batch_4x128k_density_sweep"] = sw
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
