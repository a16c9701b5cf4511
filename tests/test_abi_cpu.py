"""The C ABI library loads, exports what include/eta.h declares, and rejects
bad host-side arguments before any device work (runs without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from learned_threshold_block_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "eta.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(eta_[a-z_]+)\s*\(", text)))


def test_header_declares_the_abi():
    assert declared_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (eta_\w+)", out))
    assert set(declared_functions()) <= exported


def test_struct_layouts_match_header(tmp_path):
    """The ctypes mirrors of eta_cache, eta_seqs and eta_screen_opts have the
    header's fields, offsets and sizes (a C program compiled against eta.h
    prints them): a field added on one side only is caught here."""
    structs = {"eta_cache": _lib.EtaCacheC, "eta_seqs": _lib.EtaSeqsC, "eta_screen_opts": _lib.EtaScreenOptsC,
               "eta_calib_opts": _lib.EtaCalibOptsC}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "eta.h"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("  return 0;\n}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for cname, cls in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert got[(cname, fname)] == getattr(cls, fname).offset, (cname, fname)
    # and the header has no field the mirror lacks
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for cname, cls in structs.items():
        body = re.search(r"typedef struct \{([^}]*)\}\s*" + cname + ";", text).group(1)
        names = re.findall(r"(\w+)\s*;", body)
        assert names == [f for f, _ in cls._fields_], (cname, names)


def test_status_strings():
    L = _lib.lib()
    for code in (0, -1, -2, -3, -4, -5):
        assert L.eta_status_string(code).decode() not in ("", "unknown status")
    assert L.eta_status_string(7).decode() == "unknown status"


FAKE = 1 << 20  # aligned fake device addresses: validation never dereferences them


def cache(**kw):
    c = dict(kv_dtype=_lib.ETA_BF16, head_dim=128, num_kv_heads=8, block_size=64, num_pages=16,
             k_pages=FAKE, v_pages=FAKE * 2, mu=FAKE * 3, radius=FAKE * 4, sigma=None)
    c.update(kw)
    return _lib.EtaCacheC(**c)


def seqs(**kw):
    s = dict(num_seqs=2, max_blocks_per_seq=8, seq_lens=FAKE * 5, block_table=FAKE * 6)
    s.update(kw)
    return _lib.EtaSeqsC(**s)


def ws_size(c, n=2, mb=8, hq=32):
    return _lib.lib().eta_decode_workspace_size(ctypes.byref(c), n, mb, hq)


def test_workspace_size():
    c = cache()
    n1 = ws_size(c)
    assert n1 > 0 and n1 % 256 == 0
    assert ws_size(c, n=4, mb=2048) > n1
    assert ws_size(cache(head_dim=96)) == 0
    assert ws_size(c, hq=31) == 0          # not a multiple of H_KV
    assert ws_size(c, hq=24) == 0          # G = 3 unsupported
    assert ws_size(c, mb=(1 << 16) + 1) == 0
    assert ws_size(cache(k_pages=FAKE + 2)) == 0


def decode(c=None, s=None, **kw):
    c = c or cache()
    s = s or seqs()
    a = dict(q=FAKE * 7, hq=32, mode=_lib.ETA_TAU_LEARNED, w=FAKE * 8, b=FAKE * 9, a=0.0, beta=5.0,
             lwb=0, bs=64, out=FAKE * 10, ws=FAKE * 11, nbytes=None)
    a.update(kw)
    nbytes = ws_size(c) if a["nbytes"] is None else a["nbytes"]
    return _lib.lib().eta_decode(ctypes.byref(c), ctypes.byref(s), a["q"], a["hq"], a["mode"], a["w"],
                                 a["b"], a["a"], a["beta"], a["lwb"], a["bs"], a["out"], a["ws"],
                                 nbytes, None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), _lib.ETA_ERR_INVALID_ARGUMENT),
    (dict(q=FAKE + 4), _lib.ETA_ERR_INVALID_ARGUMENT),
    (dict(out=None), _lib.ETA_ERR_INVALID_ARGUMENT),
    (dict(w=None), _lib.ETA_ERR_INVALID_ARGUMENT),
    (dict(b=None), _lib.ETA_ERR_INVALID_ARGUMENT),
    (dict(mode=5), _lib.ETA_ERR_INVALID_ARGUMENT),
    (dict(beta=0.0), _lib.ETA_ERR_INVALID_ARGUMENT),
    (dict(beta=float("inf")), _lib.ETA_ERR_INVALID_ARGUMENT),
    (dict(a=float("nan")), _lib.ETA_ERR_INVALID_ARGUMENT),
    (dict(lwb=-1), _lib.ETA_ERR_INVALID_ARGUMENT),
    (dict(bs=32), _lib.ETA_ERR_INVALID_ARGUMENT),
    (dict(hq=30), _lib.ETA_ERR_INVALID_ARGUMENT),
    (dict(hq=48), _lib.ETA_ERR_UNSUPPORTED),
    (dict(ws=None), _lib.ETA_ERR_INVALID_ARGUMENT),
    (dict(ws=FAKE + 16), _lib.ETA_ERR_INVALID_ARGUMENT),
    (dict(nbytes=1024), _lib.ETA_ERR_WORKSPACE_TOO_SMALL),
])
def test_decode_rejects(kw, expect):
    assert decode(**kw) == expect


def test_decode_rejects_cache_and_seqs():
    assert decode(c=cache(block_size=32)) == _lib.ETA_ERR_UNSUPPORTED
    assert decode(c=cache(head_dim=80)) == _lib.ETA_ERR_UNSUPPORTED
    assert decode(c=cache(kv_dtype=3)) == _lib.ETA_ERR_INVALID_ARGUMENT
    assert decode(c=cache(mu=0)) == _lib.ETA_ERR_INVALID_ARGUMENT
    assert decode(s=seqs(num_seqs=0)) == _lib.ETA_ERR_INVALID_ARGUMENT
    assert decode(s=seqs(seq_lens=0)) == _lib.ETA_ERR_INVALID_ARGUMENT
    assert decode(s=seqs(block_table=FAKE + 2)) == _lib.ETA_ERR_INVALID_ARGUMENT
    L = _lib.lib()
    c, s = cache(), seqs()
    assert L.eta_build_block_summaries(ctypes.byref(c), None, None) == _lib.ETA_ERR_INVALID_ARGUMENT
    assert L.eta_build_block_summaries(None, ctypes.byref(s), None) == _lib.ETA_ERR_INVALID_ARGUMENT
    assert L.eta_append_kv(ctypes.byref(c), ctypes.byref(s), None, FAKE, None) == _lib.ETA_ERR_INVALID_ARGUMENT
    assert L.eta_decode_phase(9, ctypes.byref(c), ctypes.byref(s), FAKE, 32, 0, FAKE, FAKE, 0.0, 5.0, 0, 64,
                              FAKE, FAKE, 1 << 30, None) == _lib.ETA_ERR_INVALID_ARGUMENT
    assert L.eta_stats(None, 1, 1, 1, 1, None, None, None, None, None, None) == _lib.ETA_ERR_INVALID_ARGUMENT


def decode_ex(phase, bound, z, c=None, nbytes=None):
    c = c or cache()
    s = seqs()
    opts = _lib.EtaScreenOptsC(bound, z)
    return _lib.lib().eta_decode_ex(phase, ctypes.byref(opts), ctypes.byref(c), ctypes.byref(s), FAKE * 7, 32,
                                    _lib.ETA_TAU_LEARNED, FAKE * 8, FAKE * 9, 0.0, 5.0, 0, 64, FAKE * 10,
                                    FAKE * 11, 1024 if nbytes is None else nbytes, None)


def test_decode_ex_rejects_bad_screens():
    """Validation of the screen choice runs before anything else reaches the
    device (a too-small workspace is the first error a valid screen meets)."""
    with_sigma = cache(sigma=FAKE * 12)
    too_small = _lib.ETA_ERR_WORKSPACE_TOO_SMALL
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_DUAL, 2.0) == _lib.ETA_ERR_INVALID_ARGUMENT  # no sigma
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_DUAL, -1.0, c=with_sigma) == _lib.ETA_ERR_INVALID_ARGUMENT
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_DUAL, float("nan"), c=with_sigma) == \
        _lib.ETA_ERR_INVALID_ARGUMENT
    assert decode_ex(_lib.ETA_PHASE_ALL, 7, 2.0, c=with_sigma) == _lib.ETA_ERR_INVALID_ARGUMENT
    assert decode_ex(5, _lib.ETA_BOUND_GEOMETRIC, 0.0) == _lib.ETA_ERR_INVALID_ARGUMENT
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_DUAL, 2.0, c=cache(sigma=FAKE + 2)) == \
        _lib.ETA_ERR_INVALID_ARGUMENT  # misaligned sigma
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_DUAL, 2.0, c=with_sigma) == too_small
    # comparator box bound: needs both corners, aligned
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_QUEST, 0.0) == _lib.ETA_ERR_INVALID_ARGUMENT
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_QUEST, 0.0, c=cache(kmin=FAKE * 13)) == \
        _lib.ETA_ERR_INVALID_ARGUMENT  # one corner only
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_QUEST, 0.0, c=cache(kmin=FAKE * 13, kmax=FAKE + 8)) == \
        _lib.ETA_ERR_INVALID_ARGUMENT  # misaligned
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_QUEST, 0.0, c=cache(kmin=FAKE * 13, kmax=FAKE * 14)) == \
        too_small
    # FP8 records: both buffers, aligned, a known format
    fp8 = dict(mu8=FAKE * 15, radius8=FAKE * 16, mu8_format=_lib.ETA_FP8_E5M2)
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_GEOMETRIC_FP8, 0.0) == _lib.ETA_ERR_INVALID_ARGUMENT
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_GEOMETRIC_FP8, 0.0, c=cache(mu8=FAKE * 15)) == \
        _lib.ETA_ERR_INVALID_ARGUMENT
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_GEOMETRIC_FP8, 0.0, c=cache(**dict(fp8, mu8_format=5))) == \
        _lib.ETA_ERR_INVALID_ARGUMENT
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_GEOMETRIC_FP8, 0.0, c=cache(**dict(fp8, mu8=FAKE + 4))) == \
        _lib.ETA_ERR_INVALID_ARGUMENT
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_GEOMETRIC_FP8, 0.0, c=cache(**fp8)) == too_small
    # smaller screen blocks: 16 or 32 tokens, both buffers
    sub = dict(sub_block=16, mu_sub=FAKE * 17, radius_sub=FAKE * 18)
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_GEOMETRIC_SUB, 0.0) == _lib.ETA_ERR_INVALID_ARGUMENT
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_GEOMETRIC_SUB, 0.0, c=cache(**dict(sub, sub_block=8))) == \
        _lib.ETA_ERR_INVALID_ARGUMENT
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_GEOMETRIC_SUB, 0.0, c=cache(**dict(sub, radius_sub=None))) == \
        _lib.ETA_ERR_INVALID_ARGUMENT
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_GEOMETRIC_SUB, 0.0, c=cache(**sub)) == too_small
    for bad in (64, 48, 256, 0, -16):  # 16, 32 and 128 are the supported sizes
        assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_GEOMETRIC_SUB, 0.0, c=cache(**dict(sub, sub_block=bad))) \
            == _lib.ETA_ERR_INVALID_ARGUMENT, bad
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_GEOMETRIC_SUB, 0.0, c=cache(**dict(sub, sub_block=128))) == \
        too_small
    # the workspace for a cache with smaller-block records covers their tiles;
    # 128-token blocks screen pages and need no more than the page screen
    assert ws_size(cache(**sub)) > ws_size(cache())
    assert ws_size(cache(**dict(sub, sub_block=128))) == ws_size(cache())
    assert decode_ex(_lib.ETA_PHASE_SCREEN, _lib.ETA_BOUND_GEOMETRIC, 0.0) == too_small


def test_calibrate_rejects():
    L = _lib.lib()
    c, s = cache(), seqs()

    def call(w=FAKE * 8, b=FAKE * 9, rho=None, bins=512, lo=-8.0, hi=8.0, hq=32, q=FAKE * 7, hist=FAKE * 10):
        o = _lib.EtaCalibOptsC(bins, lo, hi)
        return L.eta_calibrate(ctypes.byref(c), ctypes.byref(s), q, hq, w, b, rho, ctypes.byref(o), hist,
                               FAKE * 11, FAKE * 12, FAKE * 13, FAKE * 14, None)
    bad = _lib.ETA_ERR_INVALID_ARGUMENT
    assert call(w=None, b=None, rho=None) == bad          # no target
    assert call(rho=FAKE * 15) == bad                     # both targets
    assert call(b=None) == bad                            # half a predictor
    assert call(bins=1) == bad
    assert call(lo=1.0, hi=1.0) == bad
    assert call(hi=float("inf")) == bad
    assert call(q=FAKE + 2) == bad
    assert call(hist=FAKE + 4) == bad
    assert call(hq=30) == bad
    assert call(bins=4096) == _lib.ETA_ERR_UNSUPPORTED    # G = 4: 16384 bins of LDS


def test_prefill_rejects():
    """Host-checkable arguments of eta_prefill fail before any device work."""
    L = _lib.lib()
    s = seqs()

    def call(c=None, mode=_lib.ETA_TAU_LEARNED, w=FAKE * 8, b=FAKE * 9, a=0.0, beta=5.0, hq=32, q=FAKE * 7,
             out=FAKE * 10, err=FAKE * 11, ss=None):
        c = cache() if c is None else c
        ss = s if ss is None else ss
        return L.eta_prefill(ctypes.byref(c), ctypes.byref(ss), q, hq, mode, w, b, a, beta, out, err, None)
    bad = _lib.ETA_ERR_INVALID_ARGUMENT
    assert call(w=None) == bad                              # learned needs w
    assert call(b=None, mode=_lib.ETA_TAU_CALIBRATED) == bad
    assert call(mode=7) == bad
    assert call(beta=0.0) == bad
    assert call(beta=float("inf")) == bad
    assert call(a=float("nan")) == bad
    assert call(q=FAKE + 2) == bad
    assert call(out=FAKE + 4) == bad
    assert call(out=None) == bad
    assert call(err=None) == bad
    assert call(hq=30) == bad
    assert call(ss=seqs(num_seqs=0)) == bad
    assert call(c=cache(kv_dtype=_lib.ETA_F32), w=None) == bad  # float32 caches take the same checks
    assert call(c=cache(head_dim=96)) == _lib.ETA_ERR_UNSUPPORTED
    assert call(hq=8 * 16) == _lib.ETA_ERR_UNSUPPORTED                         # G = 16
    assert call(ss=seqs(num_seqs=65536 // 32 + 1)) == _lib.ETA_ERR_UNSUPPORTED  # grid rows


def test_decode_rejects_records_of_4gib_or_more():
    """The screen addresses the records it reads with 32-bit offsets: a record
    array of 2^32 bytes or more is refused before any launch (it would wrap to
    a small size and read zeros)."""
    # 16-token blocks at d = 128: 524,288 pages x 8 KV heads x 4 slots x 256 B = 4 GiB
    sub = dict(sub_block=16, mu_sub=FAKE * 17, radius_sub=FAKE * 18)
    big = cache(num_pages=524288, **sub)
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_GEOMETRIC_SUB, 0.0, c=big, nbytes=1 << 40) == \
        _lib.ETA_ERR_UNSUPPORTED
    # one page fewer fits (the first error it meets is then the fake workspace size)
    ok = cache(num_pages=524287, **sub)
    assert decode_ex(_lib.ETA_PHASE_ALL, _lib.ETA_BOUND_GEOMETRIC_SUB, 0.0, c=ok, nbytes=16) == \
        _lib.ETA_ERR_WORKSPACE_TOO_SMALL
    # page records at d = 128: 2^24 (page, KV head) pairs are 4 GiB of centroids
    assert decode(c=cache(num_pages=1 << 21), nbytes=1 << 40) == _lib.ETA_ERR_UNSUPPORTED
    assert decode(c=cache(num_pages=(1 << 21) - 1), nbytes=16) == _lib.ETA_ERR_WORKSPACE_TOO_SMALL


def test_binding_shape_checks():
    """decode()'s shape checks (CPU tensors suffice: they run before any
    pointer is taken)."""
    import torch
    from learned_threshold_block_amd import _decode_shapes
    N, HQ, D = 2, 8, 128
    lens = torch.zeros(N, dtype=torch.int32)
    bt = torch.zeros(N, 4, dtype=torch.int32)
    q = torch.zeros(N, HQ, D)
    b = torch.zeros(HQ)
    w = torch.zeros(HQ, D)
    learned = _lib.ETA_TAU_LEARNED
    assert _decode_shapes(D, lens, bt, q, learned, b, w) == (N, HQ, D)
    assert _decode_shapes(D, lens, bt, q, _lib.ETA_TAU_CALIBRATED, b, None) == (N, HQ, D)
    bad = [
        dict(head_dim=64),                          # q's d differs from the cache's
        dict(q=torch.zeros(N, HQ * D)),             # not 3-D
        dict(lens=torch.zeros(N + 1, dtype=torch.int32)),
        dict(lens=torch.zeros(N, 1, dtype=torch.int32)),
        dict(bt=torch.zeros(N + 1, 4, dtype=torch.int32)),
        dict(bt=torch.zeros(N * 4, dtype=torch.int32)),
        dict(b=torch.zeros(HQ - 1)),
        dict(b=torch.zeros(HQ + 1)),
        dict(w=torch.zeros(HQ, D - 1)),
        dict(w=torch.zeros(HQ - 1, D)),
        dict(w=None),                               # learned mode without a predictor
    ]
    for kw in bad:
        a = dict(head_dim=D, lens=lens, bt=bt, q=q, b=b, w=w)
        a.update(kw)
        with pytest.raises(ValueError):
            _decode_shapes(a["head_dim"], a["lens"], a["bt"], a["q"], learned, a["b"], a["w"])


def launches(c=None, s=None, hq=32, bound=_lib.ETA_BOUND_GEOMETRIC):
    c = c or cache()
    s = s or seqs()
    opts = _lib.EtaScreenOptsC(bound, 2.0)
    return _lib.lib().eta_decode_launches(ctypes.byref(opts), ctypes.byref(c), ctypes.byref(s), hq)


def test_launch_form_rule():
    """One launch for sequences of at most 512 blocks with the geometric page
    screen and a group size whose attend runs 8 wavefronts; two otherwise;
    invalid sizes give the same status as eta_decode (host logic only: without
    a device the attend grid defaults to 256 workgroups)."""
    assert launches(s=seqs(max_blocks_per_seq=512)) == 1                       # 32K tokens, G = 4, bf16
    assert launches(s=seqs(max_blocks_per_seq=513)) == 2                       # more than 8 tiles
    assert launches(c=cache(kmin=FAKE * 12, kmax=FAKE * 13), bound=_lib.ETA_BOUND_QUEST) == 2
    assert launches(hq=64) == 2                                                # G = 8 at d = 128: 4 wavefronts
    assert launches(c=cache(head_dim=64), hq=64) == 1                          # G = 8 at d = 64: 8 wavefronts
    assert launches(s=seqs(num_seqs=64)) == 2                                  # 512 segments: under two per segment
    assert launches(hq=31) == _lib.ETA_ERR_INVALID_ARGUMENT
    assert launches(c=cache(head_dim=96)) == _lib.ETA_ERR_UNSUPPORTED


def test_launch_form_can_be_forced_to_two(monkeypatch):
    monkeypatch.setenv("ETA_FUSED", "0")
    assert launches(s=seqs(max_blocks_per_seq=512)) == 2
