"""ctypes view of the C ABI in include/kda.h (libkda.so).

Only argument marshalling lives here.  If the library is missing this module
raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

KDA_DTYPE_BF16 = 0
KDA_DTYPE_FP32 = 1
KDA_FLAG_QK_L2NORM = 1
KDA_FLAG_GATE_SOFTPLUS = 2
KDA_FLAG_SCALAR_GATE = 4

STATUS = {
    0: "KDA_OK", 1: "KDA_ERR_NULL_POINTER", 2: "KDA_ERR_BAD_SHAPE", 3: "KDA_ERR_UNSUPPORTED",
    4: "KDA_ERR_WORKSPACE_TOO_SMALL", 5: "KDA_ERR_BAD_STRUCT", 6: "KDA_ERR_HIP", 7: "KDA_ERR_ALIAS",
}
STATUS_CODE = {v: k for k, v in STATUS.items()}

# Every function declared in include/kda.h.
EXPORTS = ("kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd", "kda_recurrent_fwd", "kda_recurrent_step",
           "kda_recurrent_bwd_workspace_bytes", "kda_recurrent_bwd", "kda_chunk_bwd_workspace_bytes",
           "kda_chunk_bwd", "kda_dplr_recurrent_fwd",
           "kda_status_string", "kda_last_error", "kda_last_hip_error", "kda_abi_version", "kda_version",
           "kda_chunk_fwd_noalloc", "kda_chunk_fwd_noalloc_max_workspace_bytes", "kda_dplr_chunk_fwd",
           "kda_dplr_chunk_fwd_workspace_bytes")

vp = ctypes.c_void_p


class ChunkFwdArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("q", vp), ("k", vp), ("v", vp), ("g", vp), ("beta", vp),
        ("initial_state", vp), ("final_state", vp), ("o", vp), ("cu_seqlens", vp),
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
        ("chunk_size", ctypes.c_int32),
        ("workspace", vp), ("workspace_bytes", ctypes.c_size_t),
        ("stream", vp),
        ("flags", ctypes.c_uint32), ("gate_scale", ctypes.c_float),
    ]


class RecurrentStepArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("q", vp), ("k", vp), ("v", vp), ("g", vp), ("beta", vp),
        ("initial_state", vp), ("final_state", vp), ("o", vp),
        ("N", ctypes.c_int32), ("H", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
        ("stream", vp),
        ("flags", ctypes.c_uint32), ("gate_scale", ctypes.c_float),
    ]


class RecurrentBwdArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("q", vp), ("k", vp), ("v", vp), ("g", vp), ("beta", vp),
        ("initial_state", vp), ("grad_o", vp), ("grad_final_state", vp),
        ("grad_q", vp), ("grad_k", vp), ("grad_v", vp), ("grad_g", vp), ("grad_beta", vp),
        ("grad_initial_state", vp), ("cu_seqlens", vp),
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("in_dtype", ctypes.c_int),
        ("workspace", vp), ("workspace_bytes", ctypes.c_size_t),
        ("stream", vp),
        ("flags", ctypes.c_uint32), ("gate_scale", ctypes.c_float),
    ]


class DplrArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("q", vp), ("k", vp), ("v", vp), ("g", vp), ("a", vp), ("b", vp),
        ("initial_state", vp), ("final_state", vp), ("o", vp), ("cu_seqlens", vp),
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
        ("stream", vp),
    ]


class DplrChunkArgs(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("q", vp), ("k", vp), ("v", vp), ("g", vp), ("a", vp), ("b", vp),
        ("initial_state", vp), ("final_state", vp), ("o", vp), ("cu_seqlens", vp),
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
        ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("in_dtype", ctypes.c_int), ("out_dtype", ctypes.c_int),
        ("workspace", vp), ("workspace_bytes", ctypes.c_size_t),
        ("stream", vp),
    ]


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.name = STATUS.get(status, f"status {status}")
        super().__init__(f"{self.name}: {message}")


_lib = None


def load():
    """Load libkda.so (built by gated_delta_rule_52_amd.build); raise if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m gated_delta_rule_52_amd.build` (there is no fallback)")
        lib = ctypes.CDLL(LIB_PATH)
        lib.kda_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
        lib.kda_chunk_fwd_workspace_bytes.argtypes = [ctypes.POINTER(ChunkFwdArgs)]
        lib.kda_chunk_fwd.restype = ctypes.c_int
        lib.kda_chunk_fwd.argtypes = [ctypes.POINTER(ChunkFwdArgs)]
        lib.kda_recurrent_fwd.restype = ctypes.c_int
        lib.kda_recurrent_fwd.argtypes = [ctypes.POINTER(ChunkFwdArgs)]
        lib.kda_recurrent_step.restype = ctypes.c_int
        lib.kda_recurrent_step.argtypes = [ctypes.POINTER(RecurrentStepArgs)]
        lib.kda_recurrent_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.kda_recurrent_bwd_workspace_bytes.argtypes = [ctypes.POINTER(RecurrentBwdArgs)]
        lib.kda_recurrent_bwd.restype = ctypes.c_int
        lib.kda_recurrent_bwd.argtypes = [ctypes.POINTER(RecurrentBwdArgs)]
        lib.kda_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
        lib.kda_chunk_bwd_workspace_bytes.argtypes = [ctypes.POINTER(RecurrentBwdArgs)]
        lib.kda_chunk_bwd.restype = ctypes.c_int
        lib.kda_chunk_bwd.argtypes = [ctypes.POINTER(RecurrentBwdArgs)]
        lib.kda_dplr_recurrent_fwd.restype = ctypes.c_int
        lib.kda_dplr_recurrent_fwd.argtypes = [ctypes.POINTER(DplrArgs)]
        lib.kda_status_string.restype = ctypes.c_char_p
        lib.kda_status_string.argtypes = [ctypes.c_int]
        lib.kda_last_error.restype = ctypes.c_char_p
        lib.kda_last_error.argtypes = []
        lib.kda_last_hip_error.restype = ctypes.c_char_p
        lib.kda_last_hip_error.argtypes = []
        lib.kda_abi_version.restype = ctypes.c_int
        lib.kda_abi_version.argtypes = []
        lib.kda_version.restype = ctypes.c_int
        lib.kda_version.argtypes = []
        lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
        lib.kda_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(ChunkFwdArgs)]
        lib.kda_chunk_fwd_noalloc_max_workspace_bytes.restype = ctypes.c_size_t
        lib.kda_chunk_fwd_noalloc_max_workspace_bytes.argtypes = []
        lib.kda_dplr_chunk_fwd.restype = ctypes.c_int
        lib.kda_dplr_chunk_fwd.argtypes = [ctypes.POINTER(DplrChunkArgs)]
        lib.kda_dplr_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
        lib.kda_dplr_chunk_fwd_workspace_bytes.argtypes = [ctypes.POINTER(DplrChunkArgs)]
        _lib = lib
    return _lib


def check(status: int):
    if status != 0:
        raise KdaError(status, load().kda_last_error().decode())


def chunk_fwd_raw(args: ChunkFwdArgs) -> int:
    args.struct_size = ctypes.sizeof(ChunkFwdArgs)
    return load().kda_chunk_fwd(ctypes.byref(args))


def dplr_chunk_fwd_raw(args: DplrChunkArgs) -> int:
    args.struct_size = ctypes.sizeof(DplrChunkArgs)
    return load().kda_dplr_chunk_fwd(ctypes.byref(args))


def dplr_chunk_workspace_raw(args: DplrChunkArgs) -> int:
    args.struct_size = ctypes.sizeof(DplrChunkArgs)
    return load().kda_dplr_chunk_fwd_workspace_bytes(ctypes.byref(args))


def chunk_fwd_noalloc_raw(args: ChunkFwdArgs) -> int:
    args.struct_size = ctypes.sizeof(ChunkFwdArgs)
    return load().kda_chunk_fwd_noalloc(ctypes.byref(args))


def chunk_workspace_raw(args: ChunkFwdArgs) -> int:
    args.struct_size = ctypes.sizeof(ChunkFwdArgs)
    return load().kda_chunk_fwd_workspace_bytes(ctypes.byref(args))


def recurrent_fwd_raw(args: ChunkFwdArgs) -> int:
    args.struct_size = ctypes.sizeof(ChunkFwdArgs)
    return load().kda_recurrent_fwd(ctypes.byref(args))


def recurrent_step_raw(args: RecurrentStepArgs) -> int:
    args.struct_size = ctypes.sizeof(RecurrentStepArgs)
    return load().kda_recurrent_step(ctypes.byref(args))


def recurrent_bwd_raw(args: RecurrentBwdArgs) -> int:
    args.struct_size = ctypes.sizeof(RecurrentBwdArgs)
    return load().kda_recurrent_bwd(ctypes.byref(args))


def recurrent_bwd_workspace_raw(args: RecurrentBwdArgs) -> int:
    args.struct_size = ctypes.sizeof(RecurrentBwdArgs)
    return load().kda_recurrent_bwd_workspace_bytes(ctypes.byref(args))


def chunk_bwd_raw(args: RecurrentBwdArgs) -> int:
    args.struct_size = ctypes.sizeof(RecurrentBwdArgs)
    return load().kda_chunk_bwd(ctypes.byref(args))


def chunk_bwd_workspace_raw(args: RecurrentBwdArgs) -> int:
    args.struct_size = ctypes.sizeof(RecurrentBwdArgs)
    return load().kda_chunk_bwd_workspace_bytes(ctypes.byref(args))


def dplr_fwd_raw(args: DplrArgs) -> int:
    args.struct_size = ctypes.sizeof(DplrArgs)
    return load().kda_dplr_recurrent_fwd(ctypes.byref(args))
