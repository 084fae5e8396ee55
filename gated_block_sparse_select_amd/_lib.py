"""ctypes loader for libsas.so (built in-tree by ``build.py``).

Importing this module loads the library; if it is missing the import fails
loudly - there is no fallback implementation of any step.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsas.so")

SAS_OK, SAS_ERR_ARG, SAS_ERR_DTYPE, SAS_ERR_UNSUPPORTED, SAS_ERR_WORKSPACE, SAS_ERR_HIP = range(6)
SAS_F32, SAS_BF16 = 0, 1
SAS_GATE_SOFTMAX, SAS_GATE_SIGMOID, SAS_GATE_HARD, SAS_GATE_EXTERNAL = range(4)
GATES = {"softmax": SAS_GATE_SOFTMAX, "sigmoid": SAS_GATE_SIGMOID, "hard": SAS_GATE_HARD,
         "external": SAS_GATE_EXTERNAL}
ABI_VERSION = 4
NOALLOC_SCRATCH_BYTES = 16 << 20   # SAS_NOALLOC_SCRATCH_BYTES
BLOCK = 64

EXPORTED = [
    "sas_abi_version", "sas_status_string", "sas_pool_workspace_bytes", "sas_pool_scores",
    "sas_select", "sas_mask_documents", "sas_blocks_from_cu_seqlens", "sas_fwd", "sas_bwd_workspace_bytes",
    "sas_bwd_min_workspace_bytes", "sas_bwd",
    "sas_decode_workspace_bytes", "sas_decode", "sas_decode_noalloc",
    "sas_decode_paged_workspace_bytes",
    "sas_decode_paged", "sas_prof_enable", "sas_prof_collect",
    "sas_last_hip_error",
]


class SasShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("n", ctypes.c_int32), ("d", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32), ("gate", ctypes.c_int32),
                ("nb", ctypes.c_int32), ("blocks", ctypes.c_void_p)]


class SasDecodeShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("cap", ctypes.c_int32), ("d", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32), ("gate", ctypes.c_int32)]


class SasDecodePagedShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("d", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("scale", ctypes.c_float), ("dtype", ctypes.c_int32), ("gate", ctypes.c_int32)]


class SasError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {status_string(status)}"
        if status == SAS_ERR_HIP:
            msg += f" ({lib().sas_last_hip_error().decode()})"
        super().__init__(msg)


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"libsas.so not found at {LIB_PATH}; build it with "
                "`python -m gated_block_sparse_select_amd.build` (needs hipcc)")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p
        sp = ctypes.POINTER(SasShape)
        dp = ctypes.POINTER(SasDecodeShape)
        L.sas_abi_version.restype = i32
        if L.sas_abi_version() != ABI_VERSION:
            raise ImportError(f"{LIB_PATH} implements ABI {L.sas_abi_version()}, this binding "
                              f"needs {ABI_VERSION}: rebuild the library")
        L.sas_status_string.restype = ctypes.c_char_p
        L.sas_status_string.argtypes = [i32]
        L.sas_pool_workspace_bytes.restype = sz
        L.sas_pool_workspace_bytes.argtypes = [sp]
        L.sas_pool_scores.restype = i32
        L.sas_pool_scores.argtypes = [sp, vp, vp, vp, vp, sz, st]
        L.sas_select.restype = i32
        L.sas_select.argtypes = [sp, vp, vp, vp, vp, vp, st]
        L.sas_mask_documents.restype = i32
        L.sas_mask_documents.argtypes = [sp, vp, vp, st]
        ip = ctypes.POINTER(ctypes.c_int32)
        L.sas_blocks_from_cu_seqlens.restype = i32
        L.sas_blocks_from_cu_seqlens.argtypes = [ip, i32, ip, ip, i32]
        L.sas_fwd.restype = i32
        L.sas_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, st]
        L.sas_bwd_workspace_bytes.restype = sz
        L.sas_bwd_workspace_bytes.argtypes = [sp]
        L.sas_bwd_min_workspace_bytes.restype = sz
        L.sas_bwd_min_workspace_bytes.argtypes = [sp]
        L.sas_bwd.restype = i32
        L.sas_bwd.argtypes = [sp] + [vp] * 15 + [vp, sz, st]
        L.sas_decode_workspace_bytes.restype = sz
        L.sas_decode_workspace_bytes.argtypes = [dp]
        L.sas_decode.restype = i32
        L.sas_decode.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, sz, st]
        L.sas_decode_noalloc.restype = i32
        L.sas_decode_noalloc.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, st]
        pp = ctypes.POINTER(SasDecodePagedShape)
        L.sas_decode_paged_workspace_bytes.restype = sz
        L.sas_decode_paged_workspace_bytes.argtypes = [pp]
        L.sas_decode_paged.restype = i32
        L.sas_decode_paged.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, st]
        L.sas_last_hip_error.restype = ctypes.c_char_p
        L.sas_prof_enable.restype = i32
        L.sas_prof_enable.argtypes = [i32]
        L.sas_prof_collect.restype = i32
        L.sas_prof_collect.argtypes = [ctypes.POINTER(ctypes.c_char_p),
                                       ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int32), i32]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().sas_status_string(int(status)).decode()
