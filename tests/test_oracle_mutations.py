"""Planted mistakes in a copy of the oracle must each break at least one pin.

Every mutant is a plausible slip (a dropped term, a flipped sign, a wrong
index or rounding mode). The copy is built from the oracle's source text on
the CPU; the real oracle module is never modified.
"""
import importlib.util
import itertools
import os

import pytest

import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "eta_oracle.py")
_count = itertools.count()

MUTANTS = {
    "bound_drops_radius_term": ("return scale * (mu @ q + nq * R)", "return scale * (mu @ q)"),
    "bound_uses_squared_norm": ("return scale * (mu @ q + nq * R)", "return scale * (mu @ q + nq * nq * R)"),
    "radius_about_unrounded_mean": ("diff = kb - mu[:, None, :]", "diff = kb - mean[:, None, :]"),
    "centroid_rounded_to_fp32": ("mu16 = mean.astype(np.float16).astype(np.float64)",
                                 "mu16 = mean.astype(np.float32).astype(np.float64)"),
    "gate_sign_flipped": ("return S * sigmoid(beta * (S - tau))", "return S * sigmoid(beta * (tau - S))"),
    "gate_additive": ("return S * sigmoid(beta * (S - tau))", "return S + sigmoid(beta * (S - tau)) - 1.0"),
    "threshold_adds_a": ("+ float(b_h) - float(a)", "+ float(b_h) + float(a)"),
    "group_index_modulo": ("g = h // G", "g = h % HKV"),
    "tail_block_dropped": ("    if seq_len % block:\n        adm[nfull] = True\n", ""),
    "lwb_counts_from_start": ("adm[max(0, nfull - lwb):nfull] = True", "adm[:min(lwb, nfull)] = True"),
    "rescue_takes_last_max": ("adm[int(np.argmax(ub))] = True",
                              "adm[len(ub) - 1 - int(np.argmax(ub[::-1]))] = True"),
    "rescue_missing": ("    if not adm.any():\n        adm[int(np.argmax(ub))] = True\n        rescued = True\n", ""),
    "no_logit_scale": ("scale = 1.0 / math.sqrt(D)", "scale = 1.0"),
    "output_not_normalised": ("    return num / den\n", "    return num\n"),
    "tail_mask_off_by_one": ("        keep = tok < T\n        S = scale", "        keep = tok <= T\n        S = scale"),
    "union_counts_heads": ("union[n, g] = admitted[n, g * G:(g + 1) * G, :nblk].any(axis=0).sum()",
                           "union[n, g] = admitted[n, g * G:(g + 1) * G, :nblk].sum()"),
    "token_count_ignores_tail": ("width = np.minimum(BLOCK, T - BLOCK * np.arange(nblk))",
                                 "width = np.full(nblk, BLOCK)"),
    "strict_bound_comparison": ("adm[:nfull] = ~(ub < tau)", "adm[:nfull] = ub > tau + 1e-3"),
    "sigma_is_variance": ("sd = np.sqrt((dev * dev).mean(axis=1))", "sd = (dev * dev).mean(axis=1)"),
    "sigma_sample_deviation": ("sd = np.sqrt((dev * dev).mean(axis=1))",
                               "sd = np.sqrt((dev * dev).sum(axis=1) / (kb.shape[1] - 1))"),
    "dual_takes_larger": ("return np.fmin(geo, prob)", "return np.fmax(geo, prob)"),
    "dual_drops_z": ("prob = scale * (mu @ q + z * spread)", "prob = scale * (mu @ q + spread)"),
    "dual_spread_unsquared": ("spread = np.sqrt(((sigma * q[None, :]) ** 2).sum(axis=1))",
                              "spread = (sigma * np.abs(q[None, :])).sum(axis=1)"),
    "calibration_nan_in_last_bin": ("x = np.where(np.isnan(x), 0.0, x)", "x = np.where(np.isnan(x), num_bins - 1.0, x)"),
    "calibration_unweighted_rows": ("    return CALIB_WEIGHT_ONE // (t + 1)\n", "    return CALIB_WEIGHT_ONE\n"),
    "calibration_drops_diagonal": ("hist += wt * np.bincount(bins[i, :t + 1], minlength=num_bins)",
                                   "hist += wt * np.bincount(bins[i, :t], minlength=num_bins)"),
    "calibration_search_strict": ("        if tail[mid] <= target:\n", "        if tail[mid] < target:\n"),
    "calibration_threshold_strict": ("np.count_nonzero(S[i, :t + 1] >= tau[i])", "np.count_nonzero(S[i, :t + 1] > tau[i])"),
    "prefill_masked_value_enters": ("causal_weighted_sum(wts, V[:t1], causal) / wts.sum", "(wts @ V[:t1]) / wts.sum"),
    "prefill_excludes_diagonal": ("causal = np.arange(t1)[None, :] <= r[:, None]",
                                  "causal = np.arange(t1)[None, :] < r[:, None]"),
    "prefill_threshold_of_first_row": ("threshold(tau_mode, Q[t], None if w is None else w[h], b_or_c[h], a) for t in r",
                                       "threshold(tau_mode, Q[r[0]], None if w is None else w[h], b_or_c[h], a) for t in r"),
    "quest_round_down_to_nearest": ("        fix = y.astype(np.float64) > x\n",
                                    "        fix = np.zeros(np.shape(x), dtype=bool)\n"),
    "quest_box_min_rounded_up": ("lo = f16_round_down(kb.min(axis=1))", "lo = f16_round_up(kb.min(axis=1))"),
    "quest_upper_corner_only": ("terms = np.fmax(kmax * q[None, :], kmin * q[None, :])", "terms = kmax * q[None, :]"),
    "quest_nonfinite_block_kept": ("    lo[bad] = np.nan\n", "    lo[bad] = 0.0\n"),
    "fp8_round_truncates": ("r = np.minimum(np.round(a / quantum) * quantum, vmax)",
                            "r = np.minimum(np.floor(a / quantum) * quantum, vmax)"),
    "fp8_no_subnormal_binade": ("e = np.maximum(e2 - 1, emin)", "e = e2 - 1"),
    "fp8_no_saturation": ("r = np.minimum(np.round(a / quantum) * quantum, vmax)",
                          "r = np.round(a / quantum) * quantum"),
    "fp8_radius_about_mean": ("off8 = kb - mu8[:, None, :]", "off8 = kb - kb.mean(axis=1)[:, None, :]"),
    "subblock_record_slot": ("        sub = (first % BLOCK) // block\n", "        sub = ((first % BLOCK) // block + 1) % SB\n"),
    "pairblock_record_first_page_only": (
        "rows = upcast(k_pages[bt[tok // BLOCK], g, tok % BLOCK], kv_dtype)",
        "rows = upcast(k_pages[bt[tok[:, :BLOCK] // BLOCK], g, tok[:, :BLOCK] % BLOCK], kv_dtype)"),
    "pairblock_record_on_second_page": ("rp, rs = pages[first // BLOCK], (first % BLOCK) // block",
                                        "rp, rs = pages[(first + block - 1) // BLOCK], (first % BLOCK) // block"),
    "subblock_token_width": ("        width = np.minimum(block, T - block * np.arange(nblk))",
                             "        width = np.minimum(BLOCK, T - block * np.arange(nblk))"),
    "subblock_key_page": ("            K = upcast(k_pages[pages[tok // BLOCK], g, tok % BLOCK], kv_dtype)",
                          "            K = upcast(k_pages[pages[tok // BLOCK], g, (tok + 1) % BLOCK], kv_dtype)"),
    "prefill_ungated": ("                St = gate(S, tau[:, None], beta)\n", "                St = S\n"),
}


def load_mutant(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation target for {name} not found"
    src = src.replace(old, new)
    mod_name = f"_oracle_mutant_{next(_count)}"
    spec = importlib.util.spec_from_loader(mod_name, loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(src, f"<{name}>", "exec"), mod.__dict__)
    return mod


def caught(mod):
    for pin in pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            return pin.__name__, repr(e)[:200]
    return None


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    res = caught(load_mutant(name))
    assert res is not None, f"mutant {name} passed every pin"
