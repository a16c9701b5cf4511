"""Generators and test-side threshold placement (CPU)."""
import numpy as np
import pytest
import torch

import oracle.eta_oracle as E
import placement
import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 3.0e38, -3.4e38, 1e-40, np.inf, -np.inf], np.float32),
                        # exact ties between two bf16 values
                        (np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8], np.float64)).astype(np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_deterministic_and_layout():
    a = W.make_workload("ragged_16", n_seqs=3, seq_lens=[300, 4097, 64], h_q=4, h_kv=2, d=64)
    b = W.make_workload("ragged_16", n_seqs=3, seq_lens=[300, 4097, 64], h_q=4, h_kv=2, d=64)
    for f in ("k_pages", "v_pages", "q", "w", "block_table"):
        assert np.array_equal(getattr(a, f), getattr(b, f), equal_nan=True), f
    used = a.block_table[a.block_table >= 0]
    assert len(np.unique(used)) == len(used) == a.num_pages
    for n in range(a.n_seqs):
        nb = a.nblk(n)
        assert (a.block_table[n, :nb] >= 0).all() and (a.block_table[n, nb:] == -1).all()
        T = int(a.seq_lens[n])
        if T % 64:
            tail = a.k_pages[a.block_table[n, nb - 1], :, T % 64:]
            assert np.all(np.isnan(W.bf16_bits_to_f32(tail)))


def test_redraw_keeps_rest():
    wl = W.make_workload("seq_32k", seq_len=64 * 5 + 3, needles=0)
    before = wl.k_pages.copy()
    W.redraw_blocks(wl, [(0, 1, 2)])
    page = wl.block_table[0, 2]
    changed = np.any(wl.k_pages != before, axis=(2, 3))
    assert changed[page, 1] and changed.sum() == 1


def test_placement_hits_density_with_margin():
    wl = W.make_workload("seq_32k")
    mu, R = placement.place(wl)
    res = E.decode(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, wl.q,
                   wl.tau_mode, wl.w, wl.bias, wl.a, wl.beta, wl.lwb, summaries=(mu, R),
                   with_output=False)
    per_head, union = placement.densities(res, wl)
    assert abs(per_head.mean() - 0.38) < 0.01
    assert 0.6 < union.mean() < 1.0
    gap = np.abs(res.ub - res.tau[:, :, None])
    assert np.nanmin(gap) >= 1e-3


def test_query_correlation_within_groups():
    """rho = 0 draws the uncorrelated queries; rho = 1 makes a group's query
    heads equal; in between, two heads of a group correlate by about rho^2 per
    coordinate and heads of different groups not at all."""
    base = W.make_workload("seq_32k", seq_len=640, h_q=8, h_kv=2, d=128)
    zero = W.make_workload("seq_32k", seq_len=640, h_q=8, h_kv=2, d=128, rho=0.0)
    assert np.array_equal(base.q, zero.q)
    one = W.make_workload("seq_32k", seq_len=640, h_q=8, h_kv=2, d=128, rho=1.0)
    for h in range(8):
        assert np.array_equal(one.q[0, h], one.q[0, (h // 4) * 4])
    assert not np.array_equal(one.q[0, 0], one.q[0, 4])
    rho = 0.9
    wl = W.make_workload("seq_32k", seq_len=64, n_seqs=64, h_q=16, h_kv=2, d=128, rho=rho, threads=1)
    qf = W.storage_to_f32(wl.q, "bf16").astype(np.float64)
    same = np.mean([np.corrcoef(qf[n, 0], qf[n, 1 + k])[0, 1] for n in range(64) for k in range(7)])
    other = np.mean([np.corrcoef(qf[n, 0], qf[n, 8 + k])[0, 1] for n in range(64) for k in range(8)])
    assert abs(same - rho * rho) < 0.03, same
    assert abs(other) < 0.03, other
    with pytest.raises(ValueError):
        W.make_workload("seq_32k", seq_len=64, rho=1.5)


def test_table5_recipe_shape():
    wl = W.make_workload("table5_512k", n_seqs=1, seq_len=1000)
    assert (wl.h_q, wl.h_kv, wl.d, wl.kv_dtype, wl.tau_mode) == (32, 4, 64, "bf16", "calibrated")
    assert W.recipe("table5_512k")["n"] == 64 and W.recipe("table5_512k")["T"] == 524288
