"""HIP path vs the fp64 oracle at the benchmark workloads' full sizes, in the
launch configuration the benchmark times (default attend grid, dynamic claims).

Admitted-block bitmaps and every count are compared bit-exactly for all heads;
outputs are compared on a sample of heads that the oracle evaluates one by one
(it screens every head but attends only the sampled ones)."""
import numpy as np
import pytest
import torch

from gpu_util import Dev, check_output, check_sets_and_counts, log, oracle_decode, prepared

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _sample_heads(wl, per_seq, seed):
    rng = np.random.default_rng(seed)
    heads = []
    for n in range(wl.n_seqs):
        for h in rng.choice(wl.h_q, size=min(per_seq, wl.h_q), replace=False):
            heads.append((n, int(h)))
    return heads


def _run_full(name, per_seq, seed=7, bound="geometric", fp8="e4m3", block=64, **kw):
    log(f"[full-size] {name} ({bound} screen): generating and placing thresholds")
    wl, summ = prepared(name, bound=bound, fp8=fp8, block=block, **kw)
    log(f"[full-size] {name}: {wl.n_seqs} seqs, {int(wl.seq_lens.sum())} tokens, "
        f"{wl.kv_bytes() / 1e9:.2f} GB K/V")
    heads = _sample_heads(wl, per_seq, seed)
    dev = Dev(wl, with_sigma=bound == "dual", with_box=bound == "quest",
              fp8=fp8 if bound == "geometric_fp8" else None, sub_block=block if bound == "geometric_sub" else 0)
    dev.build()
    o = dev.decode(bound=bound)
    st = dev.stats()
    log(f"[full-size] {name}: oracle on {len(heads)} heads")
    res = oracle_decode(wl, summaries=summ, heads=heads, bound=bound, fp8=fp8, block=block)
    check_sets_and_counts(wl, res, st)
    check_output(wl, res, o, heads=heads)
    dens = st.admitted_per_head.sum() / (wl.h_q * sum(-(-int(T) // block) for T in wl.seq_lens))
    log(f"[full-size] {name}: per-head density {dens:.3f}, rescued {int(st.rescued.sum())}")
    del dev
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_seq_512k_full():
    """One sequence of 524,288 tokens, GQA 32/8, d = 128, bf16, learned
    thresholds at ~38% per-head density, 16 planted needles: all 32 heads."""
    _run_full("seq_512k", per_seq=32)


@pytest.mark.timeout(600)
def test_batch_4x128k_full():
    """Four sequences of 131,072 tokens, calibrated thresholds: 8 heads each."""
    _run_full("batch_4x128k", per_seq=8)


@pytest.mark.timeout(600)
def test_ragged_16_full():
    """Sixteen log-uniform lengths in [4K, 256K], pages in random order,
    per-head densities spread over [5%, 90%]: 3 heads per sequence."""
    _run_full("ragged_16", per_seq=3)


@pytest.mark.timeout(600)
def test_seq_512k_dual_full():
    """The 512K workload under the dual screen (z = 2): 8 heads."""
    _run_full("seq_512k", per_seq=8, bound="dual")


@pytest.mark.timeout(600)
def test_seq_512k_quest_full():
    """The 512K workload under the comparator's box bound: 8 heads."""
    _run_full("seq_512k", per_seq=8, bound="quest")


@pytest.mark.timeout(600)
def test_seq_512k_fp8_full():
    """The 512K workload under the geometric bound over E4M3 records: 8 heads."""
    _run_full("seq_512k", per_seq=8, bound="geometric_fp8", fp8="e4m3")


@pytest.mark.timeout(600)
def test_seq_512k_subblock16_full():
    """The 512K workload with 16-token screen blocks: 8 heads."""
    _run_full("seq_512k", per_seq=8, bound="geometric_sub", block=16)


@pytest.mark.timeout(600)
def test_seq_512k_pairblock128_full():
    """The 512K workload with 128-token screen blocks: 8 heads."""
    _run_full("seq_512k", per_seq=8, bound="geometric_sub", block=128)


@pytest.mark.timeout(600)
def test_longest_supported_sequence():
    """One sequence at the largest block table the library accepts (65,536
    pages: 4,194,304 tokens), one KV head of four query heads, d = 64: the
    screen's 1,024 tiles, the attend kernel's full tile prefix in LDS. Sets and
    counts bit-exact for all heads, outputs on two of them."""
    _run_full("seq_32k", per_seq=2, seq_lens=[64 * 65536], h_q=4, h_kv=1, d=64, needles=0)


@pytest.mark.timeout(600)
def test_table5_shape_full():
    """The head shape of the pages' decode benchmark (32 query heads over 4 KV
    heads, G = 8, d = 64) at 524,288 tokens, two sequences, queries correlated
    within each group (rho = 0.97): sets and counts bit-exact for all heads,
    outputs on 6 heads per sequence."""
    _run_full("table5_512k", per_seq=6, n_seqs=2)


@pytest.mark.timeout(600)
def test_table5_shape_subblock16_full():
    """The same shape with 16-token screen blocks: 4 heads per sequence."""
    _run_full("table5_512k", per_seq=4, n_seqs=2, bound="geometric_sub", block=16)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("density", [0.10, 0.70, 1.00])
def test_batch_4x128k_densities_full(density):
    """The 4 x 128K workload at the other points of the benchmark's density
    sweep (10%, 70% and 100% per head): every set and count, 4 heads per
    sequence for the outputs."""
    _run_full("batch_4x128k", per_seq=4, seed=11, density=density)
