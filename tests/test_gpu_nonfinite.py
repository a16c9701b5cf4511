"""Non-finite values of V, on the HIP path and in the oracle, through the C ABI.

Decode (include/eta.h, eta_decode): V of a block a head did not admit never
reaches that head's output; a non-finite element i of V at a token a head
attends to makes element i of that head's output non-finite (the oracle's
weighted sum is then infinite or NaN as well), and leaves every other element
at the usual bar. With 16-token screen blocks this holds per block, also
between the blocks of one page that different heads admitted.

Prompt pass (eta_prefill): a non-finite element i of V at key s makes element
i of the outputs at every position of s's 64-token key block and later
non-finite. That is the oracle's result from position s on; positions of the
block before s are the documented departure (the masked keys enter the
block's products with weight 0, and 0 times a non-finite value is NaN).
Earlier positions and the other elements match the oracle at the bar."""
import numpy as np
import pytest
import torch

import learned_threshold_block_amd as eta
import oracle.eta_oracle as E
import workloads as W
from gpu_util import TOL, Dev, log, oracle_decode, prepared

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bits(x, kv_dtype):
    return W.to_storage(np.array([x], np.float32), kv_dtype)[0]


def _compare_masked(got, ref, tol, what):
    """Finiteness identical element by element; finite elements within tol."""
    fin = np.isfinite(ref)
    assert np.array_equal(fin, np.isfinite(got)), f"{what}: non-finite elements differ"
    if fin.any():
        err = float(np.max(np.abs(got[fin] - ref[fin])))
        assert err <= tol, f"{what}: max abs error {err}"
        return err
    return 0.0


def test_decode_nonfinite_v_page_screen():
    wl, summ = prepared("seq_32k", seq_lens=[64 * 24 + 17], h_q=8, h_kv=2, d=128, needles=0)
    res = oracle_decode(wl, summaries=summ)
    adm = res.admitted[0]  # [H_Q][blocks]
    G = wl.group
    nfull = int(wl.seq_lens[0]) // 64
    grp = adm[0:G, :nfull]
    # a block no head of group 0 admits, and one that some but not all of them admit
    j_none = int(np.flatnonzero(~grp.any(axis=0))[0])
    part = np.flatnonzero(grp.any(axis=0) & ~grp.all(axis=0))
    j_some = int(part[0])
    log(f"[decode inf V] block {j_none} (no head), block {j_some} (heads {np.flatnonzero(grp[:, j_some]).tolist()})")
    wl.v_pages[wl.block_table[0, j_none], 0, 7, 11] = _bits(np.nan, wl.kv_dtype)
    wl.v_pages[wl.block_table[0, j_none], 0, 8, 12] = _bits(np.inf, wl.kv_dtype)
    wl.v_pages[wl.block_table[0, j_some], 0, 5, 3] = _bits(np.inf, wl.kv_dtype)
    dev = Dev(wl)
    dev.build()
    got = dev.decode()
    ref = oracle_decode(wl, summaries=summ).o
    for h in range(wl.h_q):
        sees = h < G and grp[h, j_some]
        _compare_masked(got[0, h], ref[0, h], TOL[wl.kv_dtype], f"head {h}")
        assert bool(np.isfinite(got[0, h, 3])) != bool(sees), h
        assert np.isfinite(got[0, h, 11]) and np.isfinite(got[0, h, 12])


def test_decode_nonfinite_v_16_token_blocks():
    block = 16
    wl, summ = prepared("seq_32k", bound="geometric_sub", block=block, seq_lens=[64 * 24 + 17], h_q=8, h_kv=2,
                        d=128, needles=0)
    res = oracle_decode(wl, summaries=summ, bound="geometric_sub", block=block)
    adm = res.admitted[0]  # [H_Q][16-token blocks]
    G, per = wl.group, 64 // block
    found = None
    for j in range(int(wl.seq_lens[0]) // 64):
        blocks = adm[0:G, j * per:(j + 1) * per]  # [head][block of the page]
        for q in range(per):
            a = np.flatnonzero(blocks[:, q])
            b = np.flatnonzero(~blocks[:, q] & blocks.any(axis=1))  # admits another block of the page only
            if len(a) and len(b):
                found = (j, q, int(a[0]), int(b[0]))
                break
        if found:
            break
    assert found is not None
    j, q, h_in, h_out = found
    log(f"[decode inf V, 16-token blocks] page entry {j}, block {q}: head {h_in} admits it, head {h_out} "
        f"admits another block of the page")
    wl.v_pages[wl.block_table[0, j], 0, q * block + 3, 5] = _bits(np.inf, wl.kv_dtype)
    dev = Dev(wl, sub_block=block)
    dev.build()
    got = dev.decode(bound="geometric_sub")
    ref = oracle_decode(wl, summaries=summ, bound="geometric_sub", block=block).o
    for h in range(wl.h_q):
        _compare_masked(got[0, h], ref[0, h], TOL[wl.kv_dtype], f"head {h}")
    assert not np.isfinite(got[0, h_in, 5])
    assert np.all(np.isfinite(got[0, h_out]))


def test_prefill_nonfinite_v():
    wl = W.make_workload("seq_32k", seq_lens=[64 * 3 + 7, 64 * 2], h_q=4, h_kv=2, d=64, needles=0)
    # sequence 1, KV head 0, token 69 (key block 1, row 5), element 3
    s_tok, elem = 69, 3
    page = int(wl.block_table[1, s_tok // 64])
    wl.v_pages[page, 0, s_tok % 64, elem] = _bits(np.inf, wl.kv_dtype)
    q_all = W.trace_queries(wl, seed=13)
    b = np.linspace(0.5, 1.5, wl.h_q).astype(np.float32)
    dev = Dev(wl)
    qd = eta.upload(q_all, wl.kv_dtype, "cuda")
    res = eta.prefill(dev.cache, dev.seq_lens, dev.bt, qd, eta.ETA_TAU_LEARNED, torch.from_numpy(b).cuda(), w=dev.w,
                      beta=5.0)
    torch.cuda.synchronize()
    assert int(res.err.item()) == 0
    got = res.out.cpu().numpy().astype(np.float64)
    ref = E.prefill(wl.k_pages, wl.v_pages, wl.kv_dtype, wl.block_table, wl.seq_lens, q_all, "learned", wl.w, b,
                    0.0, 5.0)
    G = wl.group
    tol = TOL["bf16"]
    # the other sequence and the other KV head's heads: untouched
    _compare_masked(got[0, :int(wl.seq_lens[0])], ref[0, :int(wl.seq_lens[0])], tol, "sequence 0")
    T1 = int(wl.seq_lens[1])
    _compare_masked(got[1, :T1, G:], ref[1, :T1, G:], tol, "sequence 1, KV head 1")
    blk0 = (s_tok // 64) * 64
    for h in range(G):
        g1, r1 = got[1, :T1, h], ref[1, :T1, h]
        # before the value's key block: exact rule, every element
        _compare_masked(g1[:blk0], r1[:blk0], tol, f"head {h}, positions < {blk0}")
        # from the block on: element 3 non-finite; the oracle from position s on
        assert not np.isfinite(g1[blk0:, elem]).any()
        assert not np.isfinite(r1[s_tok:, elem]).any() and np.isfinite(r1[blk0:s_tok, elem]).all()
        others = [e for e in range(wl.d) if e != elem]
        _compare_masked(g1[blk0:, others], r1[blk0:, others], tol, f"head {h}, other elements")
