"""ctypes declarations of the C ABI in include/retention.h."""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libretention.so")

RET_F32 = 0
RET_BF16 = 1
RET_OK = 0
RET_ERR_INVALID_ARG = -1
RET_ERR_UNSUPPORTED = -2
RET_ERR_HIP = -3
# RETENTION_NOALLOC_MAX_WORKSPACE_BYTES of include/retention.h.
NOALLOC_MAX_WORKSPACE_BYTES = 64 << 20

# Every symbol include/retention.h declares.
EXPORTED = (
    "retention_abi_version",
    "retention_status_string",
    "retention_parallel",
    "retention_chunkwise_workspace_bytes",
    "retention_chunk_stages_workspace_bytes",
    "retention_chunkwise",
    "retention_chunkwise_noalloc",
    "retention_chunk_states",
    "retention_chunk_output",
    "retention_recurrent_step",
    "retention_xpos_rotate",
    "retention_chunkwise_backward_workspace_bytes",
    "retention_chunkwise_backward",
)


# RETENTION_ABI_VERSION of include/retention.h that the structures here mirror.
ABI_VERSION = 4


class GnStruct(ctypes.Structure):
    """retention_gn_t: eps, device weight, bias and gate pointers."""

    _fields_ = [("eps", ctypes.c_float), ("weight", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("gate", ctypes.c_void_p)]


_lib = None


def load():
    """Load libretention.so from the package directory (built in-tree)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m retnet_retention_msr_amd.build` "
            "(there is no fallback path)"
        )
    _lib = open_library(LIB_PATH)
    return _lib


def open_library(path):
    """ctypes handle of a library at ``path`` that implements include/retention.h,
    with every entry point's argument and result types declared."""
    lib = ctypes.CDLL(path)
    vp, i, f_p, gn_p = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(GnStruct)
    lib.retention_abi_version.argtypes = []
    lib.retention_abi_version.restype = i
    lib.retention_status_string.argtypes = [i]
    lib.retention_status_string.restype = ctypes.c_char_p
    lib.retention_parallel.argtypes = [vp, vp, vp, f_p, vp, i, i, i, i, i, i, gn_p, vp]
    lib.retention_parallel.restype = i
    lib.retention_chunkwise_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.retention_chunkwise_workspace_bytes.restype = ctypes.c_size_t
    lib.retention_chunk_stages_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.retention_chunk_stages_workspace_bytes.restype = ctypes.c_size_t
    lib.retention_chunkwise.argtypes = [vp, vp, vp, f_p, vp, i, i, i, i, i, i, i, vp, vp, gn_p, vp,
                                        ctypes.c_size_t, vp]
    lib.retention_chunkwise.restype = i
    lib.retention_chunkwise_noalloc.argtypes = [vp, vp, vp, f_p, vp, i, i, i, i, i, i, i, vp, vp, gn_p, vp]
    lib.retention_chunkwise_noalloc.restype = i
    lib.retention_chunk_states.argtypes = [vp, vp, f_p, i, i, i, i, i, i, i, vp, vp, vp, ctypes.c_size_t, vp]
    lib.retention_chunk_states.restype = i
    lib.retention_chunk_output.argtypes = [vp, vp, vp, f_p, vp, i, i, i, i, i, i, i, i, gn_p, vp,
                                           ctypes.c_size_t, vp]
    lib.retention_chunk_output.restype = i
    lib.retention_recurrent_step.argtypes = [vp, vp, vp, f_p, vp, vp, i, i, i, i, i, gn_p, vp]
    lib.retention_recurrent_step.restype = i
    lib.retention_xpos_rotate.argtypes = [vp, vp, vp, vp, f_p, i, i, i, i, ctypes.c_longlong, i, vp]
    lib.retention_xpos_rotate.restype = i
    lib.retention_chunkwise_backward_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.retention_chunkwise_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.retention_chunkwise_backward.argtypes = [vp, vp, vp, vp, f_p, vp, vp, vp, i, i, i, i, i, i, i, vp, vp, vp,
                                                 vp, ctypes.c_size_t, vp]
    lib.retention_chunkwise_backward.restype = i
    if lib.retention_abi_version() != ABI_VERSION:
        raise RuntimeError(
            f"{path} has ABI version {lib.retention_abi_version()}, this binding expects {ABI_VERSION}: rebuild it"
        )
    return lib


def status_string(code: int) -> str:
    return load().retention_status_string(int(code)).decode()
