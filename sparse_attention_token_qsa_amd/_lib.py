"""ctypes binding of libqsa.so (C ABI in include/qsa.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  There is no
CPU fallback: a missing library raises.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqsa.so")

QSA_OK = 0
QSA_ERR_NULL = -1
QSA_ERR_EXTENT = -2
QSA_ERR_BUDGET = -3
QSA_ERR_STRIDE = -4
QSA_ERR_CAPACITY = -5
QSA_ERR_PARAM = -6
QSA_ERR_LAUNCH = -7
STATUS_BAD_POSITION = 1
STATUS_NONFINITE_SCORE = 2
STATUS_BAD_INDEX = 4
STATUS_BAD_GEOMETRY = 8
HEADS = 4
HEAD_DIM = 128
RATIO = 4
MAX_KEEP_BLOCKS = 512
MAX_TOKENS = 262147
NOALLOC_SCRATCH_BYTES = 8 << 20

# Every symbol the header declares.
EXPORTS = ("qsa_pool_keys", "qsa_score_rows", "qsa_prep_queries", "qsa_pool_prep", "qsa_score_prepped",
           "qsa_select_mask", "qsa_select_indices", "qsa_select_workspace_bytes",
           "qsa_select_mask_ws", "qsa_select_mask_noalloc", "qsa_score_select_workspace_bytes",
           "qsa_score_select_flags_offset",
           "qsa_score_select_mask",
           "qsa_gather_kv", "qsa_pool_window", "qsa_prep_queries_dev", "qsa_pool_prep_dev",
           "qsa_score_prepped_dev", "qsa_select_indices_dev", "qsa_select_indices_ws", "qsa_rope_inv_freq", "qsa_strerror",
           "qsa_abi_version")
ABI_VERSION = 10

_lib = None


class QsaError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} (code {code})")
        self.code = code


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libqsa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m sparse_attention_token_qsa_amd.build`")
    lib = ctypes.CDLL(path)
    P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    lib.qsa_pool_keys.argtypes = [P, I64, I64, P, I32, F, F, I64, I64, P, P]
    lib.qsa_pool_keys.restype = ctypes.c_int
    lib.qsa_score_rows.argtypes = [P, I64, P, I64, P, I32, F, F, P, I64, P, I64, I64, P, P]
    lib.qsa_score_rows.restype = ctypes.c_int
    lib.qsa_prep_queries.argtypes = [P, I64, P, I64, P, I32, F, F, I64, P, P, P]
    lib.qsa_prep_queries.restype = ctypes.c_int
    lib.qsa_pool_prep.argtypes = [P, I64, I64, P, I64, I64, P, P, I64, P, I64, P, P, I32, F, F, P, P]
    lib.qsa_pool_prep.restype = ctypes.c_int
    lib.qsa_score_prepped.argtypes = [P, P, I64, P, I64, P, I64, I64, P, P]
    lib.qsa_score_prepped.restype = ctypes.c_int
    lib.qsa_select_mask.argtypes = [P, I64, I64, P, I64, I64, I64, P, P, P]
    lib.qsa_select_mask.restype = ctypes.c_int
    lib.qsa_select_indices.argtypes = [P, I64, I64, P, I64, I64, I64, P, I64, P, P, P]
    lib.qsa_select_indices.restype = ctypes.c_int
    lib.qsa_select_workspace_bytes.argtypes = [I64, I64]
    lib.qsa_select_workspace_bytes.restype = ctypes.c_int64
    lib.qsa_select_mask_ws.argtypes = [P, I64, I64, P, I64, I64, I64, P, P, P, I64, P]
    lib.qsa_select_mask_ws.restype = ctypes.c_int
    lib.qsa_select_mask_noalloc.argtypes = [P, I64, I64, P, I64, I64, I64, P, P, P]
    lib.qsa_select_mask_noalloc.restype = ctypes.c_int
    lib.qsa_score_select_workspace_bytes.argtypes = [I64, I64, I64]
    lib.qsa_score_select_workspace_bytes.restype = ctypes.c_int64
    lib.qsa_score_select_flags_offset.argtypes = [I64, I64, I64]
    lib.qsa_score_select_flags_offset.restype = ctypes.c_int64
    lib.qsa_score_select_mask.argtypes = [P, P, I64, P, I64, I64, P, P, P, I64, P]
    lib.qsa_score_select_mask.restype = ctypes.c_int
    lib.qsa_gather_kv.argtypes = [P, P, I64, ctypes.c_int32, ctypes.c_int32, P, I64, I64, P, I64, P, I64,
                                  I64, P, P, P, P, P]
    lib.qsa_gather_kv.restype = ctypes.c_int
    F32 = ctypes.c_float
    I32 = ctypes.c_int32
    lib.qsa_pool_window.argtypes = [P, I64, I64, P, I32, F32, F32, P, I64, P, P, P]
    lib.qsa_pool_window.restype = ctypes.c_int
    lib.qsa_prep_queries_dev.argtypes = [P, I64, P, I64, P, I32, F32, F32, P, I64, P, P, P]
    lib.qsa_prep_queries_dev.restype = ctypes.c_int
    lib.qsa_pool_prep_dev.argtypes = [P, I64, I64, P, I64, P, P, I64, P, I64, P, P, I32, F32, F32, P, P, P]
    lib.qsa_pool_prep_dev.restype = ctypes.c_int
    lib.qsa_score_prepped_dev.argtypes = [P, P, I64, P, P, I64, P, I64, I64, P, P]
    lib.qsa_score_prepped_dev.restype = ctypes.c_int
    lib.qsa_select_indices_dev.argtypes = [P, I64, I64, P, I64, P, I64, I64, P, I64, P, P, P, I64, P]
    lib.qsa_select_indices_dev.restype = ctypes.c_int
    lib.qsa_select_indices_ws.argtypes = [P, I64, I64, P, I64, I64, I64, P, I64, P, P, P, I64, P]
    lib.qsa_select_indices_ws.restype = ctypes.c_int
    lib.qsa_rope_inv_freq.argtypes = [I32, F, P]
    lib.qsa_rope_inv_freq.restype = ctypes.c_int
    lib.qsa_strerror.argtypes = [ctypes.c_int]
    lib.qsa_strerror.restype = ctypes.c_char_p
    lib.qsa_abi_version.argtypes = []
    lib.qsa_abi_version.restype = ctypes.c_int
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load().qsa_strerror(code).decode()


def abi_version() -> int:
    return load().qsa_abi_version()
