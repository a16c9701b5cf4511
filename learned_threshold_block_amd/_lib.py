"""ctypes view of libeta.so (the C ABI in include/eta.h).

Argument marshalling only. The shared library must have been built in this
directory (learned_threshold_block_amd/build.py); there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# ETA_LIBRARY names another build of the same library (the host-sanitizer
# build of sanitized_build.py); by default the in-tree libeta.so
LIB_PATH = os.environ.get("ETA_LIBRARY") or os.path.join(HERE, "libeta.so")

ETA_OK = 0
ETA_ERR_INVALID_ARGUMENT = -1
ETA_ERR_UNSUPPORTED = -2
ETA_ERR_WORKSPACE_TOO_SMALL = -3
ETA_ERR_HIP = -4
ETA_ERR_DEVICE_DATA = -5

ETA_F32 = 0
ETA_BF16 = 1
ETA_TAU_LEARNED = 0
ETA_TAU_CALIBRATED = 1
ETA_PHASE_ALL = -1
ETA_PHASE_SCREEN = 0
ETA_PHASE_ATTEND = 1
ETA_PHASE_MERGE = 2
ETA_BOUND_GEOMETRIC = 0
ETA_BOUND_DUAL = 1
ETA_BOUND_QUEST = 2
ETA_BOUND_GEOMETRIC_FP8 = 3
ETA_BOUND_GEOMETRIC_SUB = 4
ETA_FP8_E4M3 = 0
ETA_FP8_E5M2 = 1
ETA_NOALLOC_WORKSPACE_BYTES = 32 << 20

EXPORTS = (
    "eta_build_block_summaries",
    "eta_append_kv",
    "eta_decode_workspace_size",
    "eta_decode",
    "eta_decode_noalloc",
    "eta_decode_phase",
    "eta_decode_ex",
    "eta_decode_launches",
    "eta_calibrate",
    "eta_prefill",
    "eta_stats",
    "eta_status_string",
)


class EtaCacheC(ctypes.Structure):
    _fields_ = [
        ("kv_dtype", ctypes.c_int),
        ("head_dim", ctypes.c_int),
        ("num_kv_heads", ctypes.c_int),
        ("block_size", ctypes.c_int),
        ("num_pages", ctypes.c_int),
        ("k_pages", ctypes.c_void_p),
        ("v_pages", ctypes.c_void_p),
        ("mu", ctypes.c_void_p),
        ("radius", ctypes.c_void_p),
        ("sigma", ctypes.c_void_p),
        ("kmin", ctypes.c_void_p),
        ("kmax", ctypes.c_void_p),
        ("mu8", ctypes.c_void_p),
        ("radius8", ctypes.c_void_p),
        ("mu8_format", ctypes.c_int),
        ("sub_block", ctypes.c_int),
        ("mu_sub", ctypes.c_void_p),
        ("radius_sub", ctypes.c_void_p),
    ]


class EtaScreenOptsC(ctypes.Structure):
    _fields_ = [
        ("bound", ctypes.c_int),
        ("z", ctypes.c_float),
    ]


class EtaCalibOptsC(ctypes.Structure):
    _fields_ = [
        ("num_bins", ctypes.c_int),
        ("lo", ctypes.c_float),
        ("hi", ctypes.c_float),
    ]


class EtaSeqsC(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int),
        ("max_blocks_per_seq", ctypes.c_int),
        ("seq_lens", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
    ]


class EtaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libeta.so once. Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libeta.so not built at {LIB_PATH}; run learned_threshold_block_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    cp, sp = ctypes.POINTER(EtaCacheC), ctypes.POINTER(EtaSeqsC)
    L.eta_build_block_summaries.argtypes = [cp, sp, P]
    L.eta_build_block_summaries.restype = I
    L.eta_append_kv.argtypes = [cp, sp, P, P, P]
    L.eta_append_kv.restype = I
    L.eta_decode_workspace_size.argtypes = [cp, I, I, I]
    L.eta_decode_workspace_size.restype = S
    dec = [cp, sp, P, I, I, P, P, F, F, I, I, P, P, S, P]
    L.eta_decode.argtypes = dec
    L.eta_decode.restype = I
    L.eta_decode_noalloc.argtypes = dec[:12] + [P]
    L.eta_decode_noalloc.restype = I
    L.eta_decode_phase.argtypes = [I] + dec
    L.eta_decode_phase.restype = I
    L.eta_decode_ex.argtypes = [I, ctypes.POINTER(EtaScreenOptsC)] + dec
    L.eta_decode_ex.restype = I
    L.eta_decode_launches.argtypes = [ctypes.POINTER(EtaScreenOptsC), cp, sp, I]
    L.eta_decode_launches.restype = I
    L.eta_calibrate.argtypes = [cp, sp, P, I, P, P, P, ctypes.POINTER(EtaCalibOptsC), P, P, P, P, P, P]
    L.eta_calibrate.restype = I
    L.eta_prefill.argtypes = [cp, sp, P, I, I, P, P, F, F, P, P, P]
    L.eta_prefill.restype = I
    L.eta_stats.argtypes = [P, I, I, I, I, P, P, P, P, P, P]
    L.eta_stats.restype = I
    L.eta_status_string.argtypes = [I]
    L.eta_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def status_string(status: int) -> str:
    try:
        return lib().eta_status_string(int(status)).decode()
    except ImportError:
        return "libeta.so not loaded"
