"""eta_decode_noalloc (the decode step whose workspace is the library's own
fixed device array) against eta_decode with a caller workspace, through the C
ABI: two calls in a row, the second with smaller sizes, each within the
output bar of eta_decode's result on the same inputs (and of the oracle's),
and sizes beyond the array refused before any launch."""
import numpy as np
import pytest
import torch

import learned_threshold_block_amd as eta
from gpu_util import TOL, Dev, check_output, log, oracle_decode, prepared

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(wl, summ):
    dev = Dev(wl)
    dev.build()
    ref = dev.decode()  # eta_decode, caller workspace
    mode = eta.ETA_TAU_LEARNED if wl.tau_mode == "learned" else eta.ETA_TAU_CALIBRATED
    out = torch.full((wl.n_seqs, wl.h_q, wl.d), float("nan"), dtype=torch.float32, device="cuda")
    eta.decode_noalloc(dev.cache, dev.seq_lens, dev.bt, dev.q, mode,
                       torch.from_numpy(wl.bias.astype(np.float32)).cuda(), w=dev.w, a=wl.a, beta=wl.beta,
                       lwb=wl.lwb, out=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got))
    diff = float(np.max(np.abs(got - ref)))
    log(f"  noalloc vs eta_decode: max abs diff {diff:.3g}")
    assert diff <= TOL[wl.kv_dtype]
    check_output(wl, oracle_decode(wl, summaries=summ), got)


def test_noalloc_matches_decode_twice_second_smaller():
    log("[noalloc] call 1: 2 sequences, GQA 16/4, d = 128, bf16")
    wl1, s1 = prepared("seq_32k", seq_lens=[64 * 70 + 17, 64 * 40], h_q=16, h_kv=4, needles=0)
    _both(wl1, s1)
    log("[noalloc] call 2: 1 sequence, GQA 4/2, d = 64, f32 (smaller)")
    wl2, s2 = prepared("tiny_4k_f32", seq_lens=[700], h_q=4, h_kv=2, d=64)
    _both(wl2, s2)


def test_noalloc_refuses_sizes_beyond_its_array():
    """Sizes whose workspace exceeds ETA_NOALLOC_WORKSPACE_BYTES fail with
    ETA_ERR_WORKSPACE_TOO_SMALL before anything is launched."""
    N, MB, HQ, HKV, D = 256, 8192, 4, 2, 64
    cache = eta.Cache.empty(4, HKV, D, dtype=torch.bfloat16)
    need = eta.decode_workspace_size(cache, N, MB, HQ)
    assert need > eta.ETA_NOALLOC_WORKSPACE_BYTES
    lens = torch.ones(N, dtype=torch.int32, device="cuda")
    bt = torch.zeros(N, MB, dtype=torch.int32, device="cuda")
    q = torch.zeros(N, HQ, D, dtype=torch.bfloat16, device="cuda")
    c = torch.zeros(HQ, dtype=torch.float32, device="cuda")
    out = torch.zeros(N, HQ, D, dtype=torch.float32, device="cuda")
    with pytest.raises(eta.EtaError) as ei:
        eta.decode_noalloc(cache, lens, bt, q, eta.ETA_TAU_CALIBRATED, c, out=out)
    assert ei.value.status == eta.ETA_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
