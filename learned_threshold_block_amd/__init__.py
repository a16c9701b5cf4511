"""ETA (Elastic Threshold Attention) long-context decode for AMD MI355X.

Thin Python binding over libeta.so (C ABI in include/eta.h). PyTorch tensors
provide device memory and the HIP stream; every step of the decode runs in the
library's HIP kernels. Functions here only check tensor placement/dtypes and
pass pointers.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import numpy as np
import torch

from . import _lib
from ._lib import (  # noqa: F401
    ETA_BF16, ETA_BOUND_DUAL, ETA_BOUND_GEOMETRIC, ETA_BOUND_GEOMETRIC_FP8, ETA_BOUND_GEOMETRIC_SUB, ETA_BOUND_QUEST, ETA_ERR_DEVICE_DATA,
    ETA_FP8_E4M3, ETA_FP8_E5M2, ETA_ERR_HIP, ETA_ERR_INVALID_ARGUMENT, ETA_ERR_UNSUPPORTED,
    ETA_ERR_WORKSPACE_TOO_SMALL, ETA_F32, ETA_OK, ETA_PHASE_ALL, ETA_PHASE_ATTEND, ETA_PHASE_MERGE, ETA_PHASE_SCREEN,
    ETA_NOALLOC_WORKSPACE_BYTES, ETA_TAU_CALIBRATED, ETA_TAU_LEARNED, EtaError, status_string,
)

BLOCK = 64
_WS_GLOB_SB = 7  # int32 slot of the workspace header holding the last decode's screen blocks per page
_WS_GLOB_PB = 8  # and the one holding its pages per screen block
_KV_DTYPES = {torch.bfloat16: ETA_BF16, torch.float32: ETA_F32}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check(status: int, what: str) -> None:
    if status != _lib.ETA_OK:
        raise EtaError(status, what)


def _need(t: torch.Tensor, name: str, dtype=None, device=None) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def sub_slots(sub_block: int) -> int:
    """Record slots per page for screen blocks of sub_block tokens: 64/sub_block
    for blocks inside a page, one (kept by the first page) for 128."""
    return BLOCK // sub_block if sub_block < BLOCK else 1


@dataclasses.dataclass
class Cache:
    """Paged KV cache [num_pages][H_KV][64][d] plus per-block records."""
    k_pages: torch.Tensor
    v_pages: torch.Tensor
    mu: torch.Tensor       # float16 [num_pages][H_KV][d]
    radius: torch.Tensor   # float32 [num_pages][H_KV]
    sigma: Optional[torch.Tensor] = None  # float16 [num_pages][H_KV][d], for the dual screen
    kmin: Optional[torch.Tensor] = None   # float16 [num_pages][H_KV][d], key box (comparator screen)
    kmax: Optional[torch.Tensor] = None
    mu8: Optional[torch.Tensor] = None    # uint8 [num_pages][H_KV][d], FP8 centroid (FP8 screen)
    radius8: Optional[torch.Tensor] = None  # float32 [num_pages][H_KV], radius about it
    mu8_format: str = "e4m3"              # "e4m3" or "e5m2"
    sub_block: int = 0                    # 16, 32 or 128: records of other screen blocks (0: none)
    mu_sub: Optional[torch.Tensor] = None   # float16 [num_pages][H_KV][slots][d], slots = 64/sub_block or 1
    radius_sub: Optional[torch.Tensor] = None  # float32 [num_pages][H_KV][slots]; a 128-token block's record
    #                                            sits with its first page (block-table entry 2j)

    def __post_init__(self):
        _need(self.k_pages, "k_pages")
        dev = self.k_pages.device
        if self.k_pages.dtype not in _KV_DTYPES:
            raise TypeError("k_pages must be bfloat16 or float32")
        _need(self.v_pages, "v_pages", self.k_pages.dtype, dev)
        _need(self.mu, "mu", torch.float16, dev)
        _need(self.radius, "radius", torch.float32, dev)
        if self.k_pages.dim() != 4 or self.k_pages.shape != self.v_pages.shape:
            raise ValueError("k_pages/v_pages must be [num_pages][H_KV][64][d]")
        P, H, B, D = self.k_pages.shape
        if tuple(self.mu.shape) != (P, H, D) or tuple(self.radius.shape) != (P, H):
            raise ValueError("mu must be [num_pages][H_KV][d] and radius [num_pages][H_KV]")
        for name in ("sigma", "kmin", "kmax"):
            t = getattr(self, name)
            if t is not None:
                _need(t, name, torch.float16, dev)
                if tuple(t.shape) != (P, H, D):
                    raise ValueError(f"{name} must be [num_pages][H_KV][d]")
        if (self.kmin is None) != (self.kmax is None):
            raise ValueError("kmin and kmax go together")
        if (self.mu8 is None) != (self.radius8 is None):
            raise ValueError("mu8 and radius8 go together")
        if self.mu8 is not None:
            _need(self.mu8, "mu8", torch.uint8, dev)
            _need(self.radius8, "radius8", torch.float32, dev)
            if tuple(self.mu8.shape) != (P, H, D) or tuple(self.radius8.shape) != (P, H):
                raise ValueError("mu8 must be [num_pages][H_KV][d] and radius8 [num_pages][H_KV]")
        if self.mu8_format not in ("e4m3", "e5m2"):
            raise ValueError("mu8_format must be 'e4m3' or 'e5m2'")
        if (self.mu_sub is None) != (self.radius_sub is None) or (self.mu_sub is None) != (self.sub_block == 0):
            raise ValueError("sub_block, mu_sub and radius_sub go together")
        if self.mu_sub is not None:
            if self.sub_block not in (16, 32, 128):
                raise ValueError("sub_block must be 16, 32 or 128")
            sb = sub_slots(self.sub_block)
            _need(self.mu_sub, "mu_sub", torch.float16, dev)
            _need(self.radius_sub, "radius_sub", torch.float32, dev)
            if tuple(self.mu_sub.shape) != (P, H, sb, D) or tuple(self.radius_sub.shape) != (P, H, sb):
                raise ValueError("mu_sub must be [num_pages][H_KV][slots][d], radius_sub [num_pages][H_KV][slots] "
                                 "(slots = 64/sub_block, or 1 for 128)")

    @classmethod
    def empty(cls, num_pages, num_kv_heads, head_dim, dtype=torch.bfloat16, device="cuda", with_sigma=False,
              with_box=False, fp8: Optional[str] = None, sub_block: int = 0):
        k = torch.zeros(num_pages, num_kv_heads, BLOCK, head_dim, dtype=dtype, device=device)
        v = torch.zeros_like(k)
        mu = torch.zeros(num_pages, num_kv_heads, head_dim, dtype=torch.float16, device=device)
        r = torch.zeros(num_pages, num_kv_heads, dtype=torch.float32, device=device)
        sig = torch.zeros_like(mu) if with_sigma else None
        lo = torch.zeros_like(mu) if with_box else None
        hi = torch.zeros_like(mu) if with_box else None
        mu8 = torch.zeros(num_pages, num_kv_heads, head_dim, dtype=torch.uint8, device=device) if fp8 else None
        r8 = torch.zeros_like(r) if fp8 else None
        sb = sub_slots(sub_block) if sub_block else 0
        mus = torch.zeros(num_pages, num_kv_heads, sb, head_dim, dtype=torch.float16, device=device) if sb else None
        rs = torch.zeros(num_pages, num_kv_heads, sb, dtype=torch.float32, device=device) if sb else None
        return cls(k, v, mu, r, sig, lo, hi, mu8, r8, fp8 or "e4m3", sub_block, mus, rs)

    @property
    def kv_dtype(self) -> int:
        return _KV_DTYPES[self.k_pages.dtype]

    @property
    def num_kv_heads(self) -> int:
        return self.k_pages.shape[1]

    @property
    def head_dim(self) -> int:
        return self.k_pages.shape[3]

    def c_struct(self) -> _lib.EtaCacheC:
        P, H, B, D = self.k_pages.shape
        return _lib.EtaCacheC(self.kv_dtype, D, H, B, P, _ptr(self.k_pages), _ptr(self.v_pages),
                              _ptr(self.mu), _ptr(self.radius), _ptr(self.sigma), _ptr(self.kmin),
                              _ptr(self.kmax), _ptr(self.mu8), _ptr(self.radius8),
                              _lib.ETA_FP8_E4M3 if self.mu8_format == "e4m3" else _lib.ETA_FP8_E5M2,
                              int(self.sub_block), _ptr(self.mu_sub), _ptr(self.radius_sub))


def _seqs(seq_lens: torch.Tensor, block_table: torch.Tensor, device) -> _lib.EtaSeqsC:
    _need(seq_lens, "seq_lens", torch.int32, device)
    _need(block_table, "block_table", torch.int32, device)
    if block_table.dim() != 2 or block_table.shape[0] != seq_lens.shape[0]:
        raise ValueError("block_table must be [num_seqs][max_blocks_per_seq]")
    return _lib.EtaSeqsC(block_table.shape[0], block_table.shape[1], _ptr(seq_lens), _ptr(block_table))


def build_block_summaries(cache: Cache, seq_lens, block_table, stream=None) -> None:
    c, s = cache.c_struct(), _seqs(seq_lens, block_table, cache.k_pages.device)
    _check(_lib.lib().eta_build_block_summaries(ctypes.byref(c), ctypes.byref(s), _stream(stream)),
           "eta_build_block_summaries")


def append_kv(cache: Cache, seq_lens, block_table, k_new, v_new, stream=None) -> None:
    dev = cache.k_pages.device
    _need(k_new, "k_new", cache.k_pages.dtype, dev)
    _need(v_new, "v_new", cache.k_pages.dtype, dev)
    N = seq_lens.shape[0]
    if tuple(k_new.shape) != (N, cache.num_kv_heads, cache.head_dim) or k_new.shape != v_new.shape:
        raise ValueError("k_new/v_new must be [num_seqs][H_KV][d]")
    c, s = cache.c_struct(), _seqs(seq_lens, block_table, dev)
    _check(_lib.lib().eta_append_kv(ctypes.byref(c), ctypes.byref(s), _ptr(k_new), _ptr(v_new),
                                    _stream(stream)), "eta_append_kv")


def decode_workspace_size(cache: Cache, num_seqs: int, max_blocks_per_seq: int, num_q_heads: int) -> int:
    c = cache.c_struct()
    return int(_lib.lib().eta_decode_workspace_size(ctypes.byref(c), num_seqs, max_blocks_per_seq,
                                                    num_q_heads))


def alloc_workspace(cache: Cache, num_seqs: int, max_blocks_per_seq: int, num_q_heads: int) -> torch.Tensor:
    n = decode_workspace_size(cache, num_seqs, max_blocks_per_seq, num_q_heads)
    if n == 0:
        raise EtaError(_lib.ETA_ERR_UNSUPPORTED, "eta_decode_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=cache.k_pages.device)  # 256-byte aligned


def _decode_shapes(head_dim: int, seq_lens, block_table, q, tau_mode: int, b_or_c, w):
    """Shape checks of a decode call's tensors (the C ABI takes raw pointers, so
    a mismatch here would become out-of-bounds device accesses). Returns
    (N, H_Q, d)."""
    if q.dim() != 3:
        raise ValueError("q must be [num_seqs][H_Q][d]")
    N, HQ, D = q.shape
    if D != head_dim:
        raise ValueError(f"q's head dim {D} differs from the cache's {head_dim}")
    if seq_lens.dim() != 1 or seq_lens.shape[0] != N:
        raise ValueError(f"seq_lens must be [num_seqs] = [{N}], got {tuple(seq_lens.shape)}")
    if block_table.dim() != 2 or block_table.shape[0] != N:
        raise ValueError(f"block_table must be [num_seqs][max_blocks_per_seq] with num_seqs = {N}")
    if b_or_c.numel() != HQ:
        raise ValueError(f"b_or_c must hold H_Q = {HQ} values, got {b_or_c.numel()}")
    if int(tau_mode) == ETA_TAU_LEARNED and w is None:
        raise ValueError("the learned threshold mode needs w")
    if w is not None and tuple(w.shape) != (HQ, D):
        raise ValueError(f"w must be [H_Q][d] = {(HQ, D)}, got {tuple(w.shape)}")
    return N, HQ, D


def decode(cache: Cache, seq_lens, block_table, q, tau_mode: int, b_or_c, w=None, a: float = 0.0,
           beta: float = 5.0, lwb: int = 0, out=None, workspace=None, phase: Optional[int] = None,
           stream=None, bound: str = "geometric", z: float = 2.0) -> torch.Tensor:
    """One ETA decode step; returns out [num_seqs][H_Q][d] float32.
    With `phase` set, runs only that phase (screen, attend or merge).
    bound: "geometric", "dual" (needs cache.sigma; z deviations), "quest"
    (the comparator's box bound; needs cache.kmin and cache.kmax),
    "geometric_fp8" (the geometric bound over cache.mu8 / cache.radius8) or
    "geometric_sub" (the geometric bound on cache.sub_block-token blocks)."""
    dev = cache.k_pages.device
    _need(q, "q", cache.k_pages.dtype, dev)
    _need(b_or_c, "b_or_c", torch.float32, dev)
    if w is not None:
        _need(w, "w", torch.float32, dev)
    N, HQ, D = _decode_shapes(cache.head_dim, seq_lens, block_table, q, tau_mode, b_or_c, w)
    if out is None:
        out = torch.empty(N, HQ, D, dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev)
    if tuple(out.shape) != (N, HQ, D):
        raise ValueError(f"out must be [num_seqs][H_Q][d] = {(N, HQ, D)}, got {tuple(out.shape)}")
    if workspace is None:
        workspace = alloc_workspace(cache, N, block_table.shape[1], HQ)
    _need(workspace, "workspace", torch.uint8, dev)
    c, s = cache.c_struct(), _seqs(seq_lens, block_table, dev)
    args = (ctypes.byref(c), ctypes.byref(s), _ptr(q), HQ, int(tau_mode), _ptr(w), _ptr(b_or_c),
            float(a), float(beta), int(lwb), BLOCK, _ptr(out), _ptr(workspace), workspace.numel(),
            _stream(stream))
    if bound == "geometric":
        if phase is None:
            _check(_lib.lib().eta_decode(*args), "eta_decode")
        else:
            _check(_lib.lib().eta_decode_phase(int(phase), *args), "eta_decode_phase")
    elif bound in ("dual", "quest", "geometric_fp8", "geometric_sub"):
        code = {"dual": _lib.ETA_BOUND_DUAL, "quest": _lib.ETA_BOUND_QUEST,
                "geometric_fp8": _lib.ETA_BOUND_GEOMETRIC_FP8, "geometric_sub": _lib.ETA_BOUND_GEOMETRIC_SUB}[bound]
        opts = _lib.EtaScreenOptsC(code, float(z))
        ph = _lib.ETA_PHASE_ALL if phase is None else int(phase)
        _check(_lib.lib().eta_decode_ex(ph, ctypes.byref(opts), *args), "eta_decode_ex")
    else:
        raise ValueError(f"unknown bound {bound!r}")
    return out


def decode_launches(cache: Cache, seq_lens, block_table, num_q_heads: int, bound: str = "geometric",
                    z: float = 2.0) -> int:
    """eta_decode_launches: 1 when a decode step of these sizes runs as one
    launch on the current device (short segments, geometric screen on page
    blocks), 2 when it runs as the screen phase then the attend phase."""
    dev = cache.k_pages.device
    c, s = cache.c_struct(), _seqs(seq_lens, block_table, dev)
    code = {"geometric": _lib.ETA_BOUND_GEOMETRIC, "dual": _lib.ETA_BOUND_DUAL, "quest": _lib.ETA_BOUND_QUEST,
            "geometric_fp8": _lib.ETA_BOUND_GEOMETRIC_FP8, "geometric_sub": _lib.ETA_BOUND_GEOMETRIC_SUB}[bound]
    opts = _lib.EtaScreenOptsC(code, float(z))
    r = int(_lib.lib().eta_decode_launches(ctypes.byref(opts), ctypes.byref(c), ctypes.byref(s), int(num_q_heads)))
    if r < 0:
        _check(r, "eta_decode_launches")
    return r


def decode_noalloc(cache: Cache, seq_lens, block_table, q, tau_mode: int, b_or_c, w=None, a: float = 0.0,
                   beta: float = 5.0, lwb: int = 0, out=None, stream=None) -> torch.Tensor:
    """eta_decode_noalloc: one decode step (geometric screen) whose workspace
    is the library's own fixed device array (ETA_NOALLOC_WORKSPACE_BYTES per
    GPU), so the call allocates nothing; `out` [num_seqs][H_Q][d] float32 must
    then be given. Calls that overlap in time on one GPU race."""
    dev = cache.k_pages.device
    _need(q, "q", cache.k_pages.dtype, dev)
    _need(b_or_c, "b_or_c", torch.float32, dev)
    if w is not None:
        _need(w, "w", torch.float32, dev)
    N, HQ, D = _decode_shapes(cache.head_dim, seq_lens, block_table, q, tau_mode, b_or_c, w)
    if out is None:
        raise ValueError("decode_noalloc needs a preallocated out tensor")
    _need(out, "out", torch.float32, dev)
    if tuple(out.shape) != (N, HQ, D):
        raise ValueError(f"out must be [num_seqs][H_Q][d] = {(N, HQ, D)}, got {tuple(out.shape)}")
    c, s = cache.c_struct(), _seqs(seq_lens, block_table, dev)
    _check(_lib.lib().eta_decode_noalloc(ctypes.byref(c), ctypes.byref(s), _ptr(q), HQ, int(tau_mode), _ptr(w),
                                         _ptr(b_or_c), float(a), float(beta), int(lwb), BLOCK, _ptr(out),
                                         _stream(stream)), "eta_decode_noalloc")
    return out


@dataclasses.dataclass
class Calibration:
    hist: torch.Tensor    # int64 view of uint64 [H_Q][num_bins]
    above: torch.Tensor   # [H_Q]
    total: torch.Tensor   # [H_Q]
    c: torch.Tensor       # float32 [H_Q] calibrated constants
    err: torch.Tensor     # int32 [1]


def calibrate(cache: Cache, seq_lens, block_table, q_all, num_bins: int, lo: float, hi: float, w=None, b=None,
              rho=None, stream=None) -> Calibration:
    """Offline calibration of per-head constants (eta_calibrate): q_all is
    [N][64*max_blocks][H_Q][d] (a query at every position); the target is the
    training density of the learned predictor (w, b) or the densities rho."""
    dev = cache.k_pages.device
    _need(q_all, "q_all", cache.k_pages.dtype, dev)
    N, L, HQ, D = q_all.shape
    if L != BLOCK * block_table.shape[1] or N != block_table.shape[0] or D != cache.head_dim:
        raise ValueError("q_all must be [num_seqs][64 * max_blocks_per_seq][H_Q][d]")
    for t, name in ((w, "w"), (b, "b"), (rho, "rho")):
        if t is not None:
            _need(t, name, torch.float32, dev)
    hist = torch.empty(HQ, num_bins, dtype=torch.int64, device=dev)
    above = torch.empty(HQ, dtype=torch.int64, device=dev)
    total = torch.empty(HQ, dtype=torch.int64, device=dev)
    c = torch.empty(HQ, dtype=torch.float32, device=dev)
    err = torch.empty(1, dtype=torch.int32, device=dev)
    cs, ss = cache.c_struct(), _seqs(seq_lens, block_table, dev)
    opts = _lib.EtaCalibOptsC(int(num_bins), float(lo), float(hi))
    _check(_lib.lib().eta_calibrate(ctypes.byref(cs), ctypes.byref(ss), _ptr(q_all), HQ, _ptr(w), _ptr(b), _ptr(rho),
                                    ctypes.byref(opts), _ptr(hist), _ptr(above), _ptr(total), _ptr(c), _ptr(err),
                                    _stream(stream)), "eta_calibrate")
    return Calibration(hist, above, total, c, err)


@dataclasses.dataclass
class Prefill:
    out: torch.Tensor  # float32 [N][64*max_blocks][H_Q][d]; NaN rows at positions >= seq_len
    err: torch.Tensor  # int32 [1]: 1 if an out-of-range length or page id was met


def prefill(cache: Cache, seq_lens, block_table, q_all, tau_mode: int, b_or_c, w=None, a: float = 0.0,
            beta: float = 5.0, out=None, stream=None) -> Prefill:
    """Causal prompt pass (eta_prefill): gated attention at every position of
    every sequence over the keys up to it, and the records of every complete
    block. q_all is [N][64*max_blocks][H_Q][d] of the cache's element type."""
    dev = cache.k_pages.device
    _need(q_all, "q_all", cache.k_pages.dtype, dev)
    N, L, HQ, D = q_all.shape
    if L != BLOCK * block_table.shape[1] or N != block_table.shape[0] or D != cache.head_dim:
        raise ValueError("q_all must be [num_seqs][64 * max_blocks_per_seq][H_Q][d]")
    _need(b_or_c, "b_or_c", torch.float32, dev)
    if w is not None:
        _need(w, "w", torch.float32, dev)
    if out is None:
        out = torch.empty(N, L, HQ, D, dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev)
    err = torch.empty(1, dtype=torch.int32, device=dev)
    c, s = cache.c_struct(), _seqs(seq_lens, block_table, dev)
    _check(_lib.lib().eta_prefill(ctypes.byref(c), ctypes.byref(s), _ptr(q_all), HQ, int(tau_mode), _ptr(w),
                                  _ptr(b_or_c), float(a), float(beta), _ptr(out), _ptr(err), _stream(stream)),
           "eta_prefill")
    return Prefill(out, err)


@dataclasses.dataclass
class Stats:
    admitted_per_head: np.ndarray   # int32 [N][H_Q]
    union_per_kv: np.ndarray        # int32 [N][H_KV]
    tokens_per_head: np.ndarray     # int64 [N][H_Q]
    rescued: np.ndarray             # uint8 [N][H_Q]
    bitmap: Optional[np.ndarray]    # uint32 [N][H_Q][ceil(MB/32)]
    status: int

    def admitted(self, max_blocks: int) -> np.ndarray:
        """bool [N][H_Q][max_blocks] from the bitmap."""
        b = np.unpackbits(self.bitmap.view(np.uint8), axis=-1, bitorder="little")
        return b[..., :max_blocks].astype(bool)


def stats(workspace: torch.Tensor, num_seqs: int, max_blocks_per_seq: int, num_q_heads: int,
          num_kv_heads: int, bitmap: bool = True, stream=None, check: bool = True,
          block_tokens: Optional[int] = None) -> Stats:
    """Counts of the last decode on this workspace. block_tokens: tokens per
    screen block of that decode (cache.sub_block after a "geometric_sub"
    decode, else 64), which sizes the bitmap (ceil(64 max_blocks_per_seq /
    block_tokens) bits per head); read from the workspace's header when not
    given."""
    if block_tokens is None:
        block_tokens = BLOCK
        if bitmap:
            hdr = workspace[:64].view(torch.int32)
            sb, pb = int(hdr[_WS_GLOB_SB].item()), int(hdr[_WS_GLOB_PB].item())
            block_tokens = BLOCK // sb if sb in (2, 4) else 2 * BLOCK if pb == 2 else BLOCK
    nbits = -(-max_blocks_per_seq * BLOCK // block_tokens)
    a = np.zeros((num_seqs, num_q_heads), np.int32)
    u = np.zeros((num_seqs, num_kv_heads), np.int32)
    t = np.zeros((num_seqs, num_q_heads), np.int64)
    r = np.zeros((num_seqs, num_q_heads), np.uint8)
    bm = np.zeros((num_seqs, num_q_heads, (nbits + 31) // 32), np.uint32) if bitmap else None
    st = _lib.lib().eta_stats(_ptr(workspace), num_seqs, max_blocks_per_seq, num_q_heads, num_kv_heads,
                              a.ctypes.data, u.ctypes.data, t.ctypes.data, r.ctypes.data,
                              None if bm is None else bm.ctypes.data, _stream(stream))
    if check and st not in (_lib.ETA_OK,):
        raise EtaError(st, "eta_stats")
    return Stats(a, u, t, r, bm, st)


# ----------------------------------------------------------------------------- uploads
def bf16_tensor_from_bits(bits: np.ndarray, device) -> torch.Tensor:
    """Upload an array of bfloat16 bit patterns (uint16) as a torch.bfloat16 tensor."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to(device).view(torch.bfloat16)


def upload(arr: np.ndarray, kv_dtype: str, device) -> torch.Tensor:
    if kv_dtype == "bf16":
        return bf16_tensor_from_bits(arr, device)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)
