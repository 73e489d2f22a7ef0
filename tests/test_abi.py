"""CPU tests of the C ABI: the library loads, exports every function that
include/kda.h declares, and rejects bad arguments with the documented status
codes before anything is launched (no GPU is touched here)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_52_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 1 << 32          # distinct fake device addresses: only compared, never used
S = _lib.STATUS_CODE


def header_functions():
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[\w\s\*]+?\b(kda_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_function_is_exported():
    lib = _lib.load()
    decl = header_functions()
    assert decl == sorted(_lib.EXPORTS)
    for name in decl:
        assert hasattr(lib, name), name
    assert lib.kda_abi_version() == 7
    # the names the boundary's specification gives: the version and the HIP error text
    assert lib.kda_version() == lib.kda_abi_version()
    for name in ("kda_chunk_fwd", "kda_chunk_fwd_workspace_bytes", "kda_recurrent_step", "kda_status_string",
                 "kda_last_hip_error", "kda_version"):
        assert name in decl, name


def test_status_strings():
    lib = _lib.load()
    for code in range(8):
        assert lib.kda_status_string(code).decode() not in ("", "unknown status")
    assert lib.kda_status_string(99).decode() == "unknown status"


def chunk_args(**kw):
    a = _lib.ChunkFwdArgs()
    base = dict(q=FAKE, k=2 * FAKE, v=3 * FAKE, g=4 * FAKE, beta=5 * FAKE, o=6 * FAKE,
                initial_state=None, final_state=7 * FAKE, cu_seqlens=None,
                B=1, T=128, H=2, dk=128, dv=128, num_seqs=1, scale=1.0,
                in_dtype=_lib.KDA_DTYPE_BF16, out_dtype=_lib.KDA_DTYPE_FP32, chunk_size=64)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(dk=96), "KDA_ERR_UNSUPPORTED"),
    (dict(dv=256), "KDA_ERR_UNSUPPORTED"),
    (dict(in_dtype=7), "KDA_ERR_UNSUPPORTED"),
    (dict(chunk_size=48), "KDA_ERR_UNSUPPORTED"),
    (dict(H=0), "KDA_ERR_BAD_SHAPE"),
    (dict(T=-1), "KDA_ERR_BAD_SHAPE"),
    (dict(num_seqs=2), "KDA_ERR_BAD_SHAPE"),
    (dict(B=2, num_seqs=2, cu_seqlens=8 * FAKE), "KDA_ERR_BAD_SHAPE"),
    (dict(scale=float("nan")), "KDA_ERR_BAD_SHAPE"),
    (dict(B=2, num_seqs=2, T=2 ** 30, H=1, dk=64, dv=64), "KDA_ERR_BAD_SHAPE"),  # 2^31 tokens
    (dict(q=None), "KDA_ERR_NULL_POINTER"),
    (dict(o=None), "KDA_ERR_NULL_POINTER"),
    (dict(o=FAKE + 64), "KDA_ERR_ALIAS"),
    (dict(final_state=3 * FAKE + 8), "KDA_ERR_ALIAS"),
    (dict(initial_state=7 * FAKE + 4096), "KDA_ERR_ALIAS"),
    (dict(flags=8), "KDA_ERR_UNSUPPORTED"),
    # o written while other workgroups still read the initial state or the sequence offsets
    (dict(initial_state=8 * FAKE, o=8 * FAKE + 64), "KDA_ERR_ALIAS"),
    (dict(cu_seqlens=9 * FAKE, o=9 * FAKE - 64), "KDA_ERR_ALIAS"),
    (dict(cu_seqlens=7 * FAKE + 16), "KDA_ERR_ALIAS"),
    (dict(cu_seqlens=9 * FAKE + 64, workspace=9 * FAKE, workspace_bytes=1 << 40), "KDA_ERR_ALIAS"),
    (dict(flags=_lib.KDA_FLAG_GATE_SOFTPLUS, gate_scale=-1.0), "KDA_ERR_BAD_SHAPE"),
    (dict(flags=_lib.KDA_FLAG_GATE_SOFTPLUS, gate_scale=float("nan")), "KDA_ERR_BAD_SHAPE"),
])
def test_chunk_fwd_rejects(kw, status):
    rc = _lib.chunk_fwd_raw(chunk_args(**kw))
    assert rc == S[status], (_lib.STATUS.get(rc), _lib.load().kda_last_error())
    assert _lib.load().kda_last_error().decode() != ""


@pytest.mark.parametrize("kw,status", [
    (dict(dk=96), "KDA_ERR_UNSUPPORTED"),
    (dict(out_dtype=7), "KDA_ERR_UNSUPPORTED"),
    (dict(H=0), "KDA_ERR_BAD_SHAPE"),
    (dict(num_seqs=2), "KDA_ERR_BAD_SHAPE"),
    (dict(B=2, num_seqs=2, cu_seqlens=8 * FAKE), "KDA_ERR_BAD_SHAPE"),
    (dict(scale=float("inf")), "KDA_ERR_BAD_SHAPE"),
    (dict(v=None), "KDA_ERR_NULL_POINTER"),
    (dict(o=2 * FAKE + 8), "KDA_ERR_ALIAS"),
    (dict(final_state=6 * FAKE + 8), "KDA_ERR_ALIAS"),
    (dict(initial_state=8 * FAKE, o=8 * FAKE + 64), "KDA_ERR_ALIAS"),
    (dict(cu_seqlens=9 * FAKE, o=9 * FAKE - 64), "KDA_ERR_ALIAS"),
    (dict(flags=16), "KDA_ERR_UNSUPPORTED"),
    (dict(flags=3, gate_scale=float("inf")), "KDA_ERR_BAD_SHAPE"),
])
def test_recurrent_fwd_rejects(kw, status):
    # the same argument rules as kda_chunk_fwd; chunk_size and workspace are ignored
    rc = _lib.recurrent_fwd_raw(chunk_args(chunk_size=48, **kw))
    assert rc == S[status], (_lib.STATUS.get(rc), _lib.load().kda_last_error())
    assert _lib.load().kda_last_error().decode() != ""


def test_chunk_struct_size_is_checked():
    a = chunk_args()
    a.struct_size = ctypes.sizeof(_lib.ChunkFwdArgs) - 4
    assert _lib.load().kda_chunk_fwd(ctypes.byref(a)) == S["KDA_ERR_BAD_STRUCT"]
    assert _lib.load().kda_chunk_fwd(None) == S["KDA_ERR_NULL_POINTER"]


def test_version_1_structs_are_accepted_without_transforms():
    """A struct that ends before `flags` (ABI version 1) is read without the
    fields after it: invalid values there are never looked at."""
    lib = _lib.load()
    v1 = _lib.ChunkFwdArgs.flags.offset
    a = chunk_args(B=0, num_seqs=0, flags=0xff, gate_scale=-1.0)
    a.struct_size = v1
    assert lib.kda_chunk_fwd(ctypes.byref(a)) == 0
    assert lib.kda_recurrent_fwd(ctypes.byref(a)) == 0
    a.struct_size = ctypes.sizeof(_lib.ChunkFwdArgs)
    assert lib.kda_chunk_fwd(ctypes.byref(a)) == S["KDA_ERR_UNSUPPORTED"]
    r = step_args(N=0, flags=0xff, gate_scale=-1.0)
    r.struct_size = _lib.RecurrentStepArgs.flags.offset
    assert lib.kda_recurrent_step(ctypes.byref(r)) == 0
    r.struct_size = ctypes.sizeof(_lib.RecurrentStepArgs)
    assert lib.kda_recurrent_step(ctypes.byref(r)) == S["KDA_ERR_UNSUPPORTED"]
    # the workspace query reads the same way
    w = chunk_args(T=4096, flags=0xff)
    w.struct_size = v1
    assert lib.kda_chunk_fwd_workspace_bytes(ctypes.byref(w)) == _lib.chunk_workspace_raw(chunk_args(T=4096))


def test_workspace_query():
    assert _lib.chunk_workspace_raw(chunk_args(dk=7)) == 2 ** 64 - 1
    n = _lib.chunk_workspace_raw(chunk_args(T=65536, H=16))
    assert 0 <= n < 2 ** 40


def step_args(**kw):
    a = _lib.RecurrentStepArgs()
    base = dict(q=FAKE, k=2 * FAKE, v=3 * FAKE, g=4 * FAKE, beta=5 * FAKE, o=6 * FAKE,
                initial_state=7 * FAKE, final_state=7 * FAKE, N=4, H=2, dk=128, dv=128, scale=1.0,
                in_dtype=_lib.KDA_DTYPE_BF16, out_dtype=_lib.KDA_DTYPE_FP32)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(dk=32), "KDA_ERR_UNSUPPORTED"),
    (dict(out_dtype=5), "KDA_ERR_UNSUPPORTED"),
    (dict(N=-1), "KDA_ERR_BAD_SHAPE"),
    (dict(H=0), "KDA_ERR_BAD_SHAPE"),
    (dict(final_state=None), "KDA_ERR_NULL_POINTER"),
    (dict(beta=None), "KDA_ERR_NULL_POINTER"),
    (dict(o=5 * FAKE), "KDA_ERR_ALIAS"),
    (dict(final_state=FAKE), "KDA_ERR_ALIAS"),
    (dict(initial_state=7 * FAKE + 256), "KDA_ERR_ALIAS"),
    (dict(initial_state=8 * FAKE, o=8 * FAKE + 64), "KDA_ERR_ALIAS"),
    (dict(flags=32), "KDA_ERR_UNSUPPORTED"),
    (dict(flags=_lib.KDA_FLAG_GATE_SOFTPLUS, gate_scale=-0.5), "KDA_ERR_BAD_SHAPE"),
])
def test_recurrent_step_rejects(kw, status):
    rc = _lib.recurrent_step_raw(step_args(**kw))
    assert rc == S[status], (_lib.STATUS.get(rc), _lib.load().kda_last_error())


def test_empty_problems_are_no_ops():
    # nothing to do: returns before any HIP call
    assert _lib.recurrent_step_raw(step_args(N=0)) == 0
    assert _lib.chunk_fwd_raw(chunk_args(B=0, num_seqs=0)) == 0
    assert _lib.recurrent_fwd_raw(chunk_args(B=0, num_seqs=0)) == 0


def bwd_args(**kw):
    a = _lib.RecurrentBwdArgs()
    base = dict(q=FAKE, k=2 * FAKE, v=3 * FAKE, g=4 * FAKE, beta=5 * FAKE, initial_state=6 * FAKE,
                grad_o=7 * FAKE, grad_final_state=8 * FAKE, grad_q=9 * FAKE, grad_k=10 * FAKE,
                grad_v=11 * FAKE, grad_g=12 * FAKE, grad_beta=13 * FAKE, grad_initial_state=14 * FAKE,
                cu_seqlens=None, B=2, T=100, H=2, dk=128, dv=64, num_seqs=2, scale=1.0,
                in_dtype=_lib.KDA_DTYPE_BF16, workspace=15 * FAKE, workspace_bytes=1 << 30)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


def test_backward_workspace_size():
    """At least one stored state (H * dk * dv fp32) per 8 tokens, growing with
    the token count; invalid sizes give (size_t)-1."""
    state = 2 * 128 * 64 * 4
    n1 = _lib.recurrent_bwd_workspace_raw(bwd_args())
    n2 = _lib.recurrent_bwd_workspace_raw(bwd_args(T=1000))
    nv = _lib.recurrent_bwd_workspace_raw(bwd_args(B=1, T=1001, num_seqs=5, cu_seqlens=16 * FAKE))
    assert n1 >= (200 // 8) * state and n2 >= (2000 // 8) * state and n2 > n1
    assert nv >= (1001 // 8) * state
    assert _lib.recurrent_bwd_workspace_raw(bwd_args(dk=32)) == 2 ** 64 - 1
    # the input transforms add fp32 copies of the transformed inputs
    nx = _lib.recurrent_bwd_workspace_raw(bwd_args(flags=_lib.KDA_FLAG_QK_L2NORM))
    assert nx >= n1 + 200 * 2 * (2 * 128 + 128 + 2 * 64 + 3) * 4


@pytest.mark.parametrize("kw,status", [
    (dict(dk=96), "KDA_ERR_UNSUPPORTED"),
    (dict(in_dtype=5), "KDA_ERR_UNSUPPORTED"),
    (dict(H=0), "KDA_ERR_BAD_SHAPE"),
    (dict(num_seqs=3), "KDA_ERR_BAD_SHAPE"),
    (dict(cu_seqlens=16 * FAKE), "KDA_ERR_BAD_SHAPE"),  # packed input needs B = 1
    (dict(scale=float("nan")), "KDA_ERR_BAD_SHAPE"),
    (dict(B=2, num_seqs=2, T=2 ** 30, H=1, dk=64, dv=64), "KDA_ERR_BAD_SHAPE"),
    (dict(grad_o=None), "KDA_ERR_NULL_POINTER"),
    (dict(grad_beta=None), "KDA_ERR_NULL_POINTER"),
    (dict(workspace_bytes=1000), "KDA_ERR_WORKSPACE_TOO_SMALL"),
    (dict(workspace=None), "KDA_ERR_WORKSPACE_TOO_SMALL"),
    (dict(grad_q=FAKE + 256), "KDA_ERR_ALIAS"),              # inside q
    (dict(grad_k=9 * FAKE + 256), "KDA_ERR_ALIAS"),          # inside grad_q
    (dict(grad_v=15 * FAKE + 4096), "KDA_ERR_ALIAS"),        # inside the workspace
    (dict(grad_g=6 * FAKE + 64), "KDA_ERR_ALIAS"),           # inside initial_state
    (dict(workspace=8 * FAKE), "KDA_ERR_ALIAS"),             # the final-state gradient
    (dict(grad_initial_state=6 * FAKE + 64), "KDA_ERR_ALIAS"),  # partly over initial_state
    (dict(grad_initial_state=8 * FAKE + 64), "KDA_ERR_ALIAS"),  # partly over grad_final_state
    (dict(grad_initial_state=5 * FAKE), "KDA_ERR_ALIAS"),       # over beta
    (dict(flags=8), "KDA_ERR_UNSUPPORTED"),
    (dict(flags=_lib.KDA_FLAG_GATE_SOFTPLUS, gate_scale=-1.0), "KDA_ERR_BAD_SHAPE"),
])
def test_backward_rejects(kw, status):
    rc = _lib.recurrent_bwd_raw(bwd_args(**kw))
    assert rc == S[status], (_lib.STATUS.get(rc), _lib.load().kda_last_error())
    assert _lib.load().kda_last_error().decode() != ""


def test_backward_struct_and_empty_calls():
    lib = _lib.load()
    a = bwd_args()
    a.struct_size = ctypes.sizeof(_lib.RecurrentBwdArgs) - 8
    assert lib.kda_recurrent_bwd(ctypes.byref(a)) == S["KDA_ERR_BAD_STRUCT"]
    assert lib.kda_recurrent_bwd(None) == S["KDA_ERR_NULL_POINTER"]
    # nothing to do: no sequence, or no token and no initial-state gradient (no launch)
    assert _lib.recurrent_bwd_raw(bwd_args(B=0, num_seqs=0)) == 0
    assert _lib.recurrent_bwd_raw(bwd_args(T=0, grad_initial_state=None, q=None, grad_q=None)) == 0


def test_chunk_backward_workspace_size():
    """Per chunk of 64 tokens and head: a reverse pack plus the state, V_new,
    the state gradient and dV_new in fp32 (at least 3.2 KiB per token and
    head); other dtypes, head sizes or flags give (size_t)-1."""
    n1 = _lib.chunk_bwd_workspace_raw(bwd_args(dv=128))
    n2 = _lib.chunk_bwd_workspace_raw(bwd_args(dv=128, T=1000))
    assert n1 >= 2 * 128 * 2 * 3200 and n2 >= 2 * 1024 * 2 * 3200 and n2 > n1
    for kw in (dict(), dict(dv=128, in_dtype=_lib.KDA_DTYPE_FP32), dict(dv=128, dk=64),
               dict(dv=128, flags=_lib.KDA_FLAG_QK_L2NORM)):
        assert _lib.chunk_bwd_workspace_raw(bwd_args(**kw)) == 2 ** 64 - 1, kw


@pytest.mark.parametrize("kw,status", [
    (dict(dv=64), "KDA_ERR_UNSUPPORTED"),
    (dict(dk=64), "KDA_ERR_UNSUPPORTED"),
    (dict(in_dtype=_lib.KDA_DTYPE_FP32), "KDA_ERR_UNSUPPORTED"),
    (dict(flags=_lib.KDA_FLAG_SCALAR_GATE), "KDA_ERR_UNSUPPORTED"),
    (dict(flags=_lib.KDA_FLAG_QK_L2NORM), "KDA_ERR_UNSUPPORTED"),
    (dict(H=0), "KDA_ERR_BAD_SHAPE"),
    (dict(num_seqs=3), "KDA_ERR_BAD_SHAPE"),
    (dict(grad_o=None), "KDA_ERR_NULL_POINTER"),
    (dict(workspace_bytes=1000), "KDA_ERR_WORKSPACE_TOO_SMALL"),
    (dict(workspace=None), "KDA_ERR_WORKSPACE_TOO_SMALL"),
    (dict(grad_q=FAKE + 256), "KDA_ERR_ALIAS"),              # inside q
    (dict(grad_v=15 * FAKE + 4096), "KDA_ERR_ALIAS"),        # inside the workspace
    (dict(grad_initial_state=6 * FAKE + 64), "KDA_ERR_ALIAS"),  # partly over initial_state
    (dict(grad_initial_state=5 * FAKE), "KDA_ERR_ALIAS"),       # over beta
])
def test_chunk_backward_rejects(kw, status):
    args = dict(dv=128)
    args.update(kw)
    rc = _lib.chunk_bwd_raw(bwd_args(**args))
    assert rc == S[status], (_lib.STATUS.get(rc), _lib.load().kda_last_error())
    assert _lib.load().kda_last_error().decode() != ""


def test_chunk_backward_struct_and_empty_calls():
    lib = _lib.load()
    a = bwd_args(dv=128)
    a.struct_size = ctypes.sizeof(_lib.RecurrentBwdArgs) - 8
    assert lib.kda_chunk_bwd(ctypes.byref(a)) == S["KDA_ERR_BAD_STRUCT"]
    assert lib.kda_chunk_bwd(None) == S["KDA_ERR_NULL_POINTER"]
    assert _lib.chunk_bwd_raw(bwd_args(dv=128, B=0, num_seqs=0)) == 0
    assert _lib.chunk_bwd_raw(bwd_args(dv=128, T=0, grad_initial_state=None, q=None, grad_q=None)) == 0


def dplr_args(**kw):
    a = _lib.DplrArgs()
    base = dict(q=FAKE, k=2 * FAKE, v=3 * FAKE, g=4 * FAKE, a=5 * FAKE, b=6 * FAKE, initial_state=7 * FAKE,
                final_state=7 * FAKE, o=8 * FAKE, cu_seqlens=None, B=2, T=64, H=2, dk=128, dv=128, num_seqs=2,
                scale=1.0, in_dtype=_lib.KDA_DTYPE_BF16, out_dtype=_lib.KDA_DTYPE_FP32)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(dk=32), "KDA_ERR_UNSUPPORTED"),
    (dict(out_dtype=9), "KDA_ERR_UNSUPPORTED"),
    (dict(H=0), "KDA_ERR_BAD_SHAPE"),
    (dict(num_seqs=3), "KDA_ERR_BAD_SHAPE"),
    (dict(scale=float("nan")), "KDA_ERR_BAD_SHAPE"),
    (dict(b=None), "KDA_ERR_NULL_POINTER"),
    (dict(o=5 * FAKE + 16), "KDA_ERR_ALIAS"),            # inside a
    (dict(final_state=6 * FAKE + 16, initial_state=None), "KDA_ERR_ALIAS"),  # inside b
    (dict(initial_state=7 * FAKE + 64), "KDA_ERR_ALIAS"),  # partial overlap with final_state
])
def test_dplr_rejects(kw, status):
    rc = _lib.dplr_fwd_raw(dplr_args(**kw))
    assert rc == S[status], (_lib.STATUS.get(rc), _lib.load().kda_last_error())
    assert _lib.load().kda_last_error().decode() != ""


def test_dplr_struct_size_and_empty_call():
    lib = _lib.load()
    a = dplr_args()
    a.struct_size = ctypes.sizeof(_lib.DplrArgs) + 8
    assert lib.kda_dplr_recurrent_fwd(ctypes.byref(a)) == S["KDA_ERR_BAD_STRUCT"]
    assert _lib.dplr_fwd_raw(dplr_args(B=0, num_seqs=0)) == 0


def dplr_chunk_args(**kw):
    a = _lib.DplrChunkArgs()
    base = dict(q=FAKE, k=2 * FAKE, v=3 * FAKE, g=4 * FAKE, a=5 * FAKE, b=6 * FAKE, initial_state=7 * FAKE,
                final_state=7 * FAKE, o=8 * FAKE, cu_seqlens=None, B=2, T=64, H=2, dk=128, dv=128, num_seqs=2,
                scale=1.0, in_dtype=_lib.KDA_DTYPE_BF16, out_dtype=_lib.KDA_DTYPE_FP32,
                workspace=9 * FAKE, workspace_bytes=1 << 30)
    base.update(kw)
    for k, v in base.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,status", [
    (dict(dk=32), "KDA_ERR_UNSUPPORTED"),
    (dict(in_dtype=4), "KDA_ERR_UNSUPPORTED"),
    (dict(H=0), "KDA_ERR_BAD_SHAPE"),
    (dict(num_seqs=3), "KDA_ERR_BAD_SHAPE"),
    (dict(a=None), "KDA_ERR_NULL_POINTER"),
    (dict(o=5 * FAKE + 16), "KDA_ERR_ALIAS"),                 # inside a
    (dict(initial_state=7 * FAKE + 64), "KDA_ERR_ALIAS"),     # partial overlap with final_state
    (dict(workspace_bytes=1000), "KDA_ERR_WORKSPACE_TOO_SMALL"),
    (dict(workspace=None), "KDA_ERR_WORKSPACE_TOO_SMALL"),
    (dict(workspace=8 * FAKE + 4096), "KDA_ERR_ALIAS"),       # inside o
    (dict(workspace=7 * FAKE), "KDA_ERR_ALIAS"),              # the states
])
def test_dplr_chunk_rejects(kw, status):
    rc = _lib.dplr_chunk_fwd_raw(dplr_chunk_args(**kw))
    assert rc == S[status], (_lib.STATUS.get(rc), _lib.load().kda_last_error())
    assert _lib.load().kda_last_error().decode() != ""


def test_dplr_chunk_workspace_and_struct():
    lib = _lib.load()
    n1 = _lib.dplr_chunk_workspace_raw(dplr_chunk_args(T=1000))
    n2 = _lib.dplr_chunk_workspace_raw(dplr_chunk_args(T=100000))
    assert 0 < n1 < n2 < 2 ** 64 - 1
    assert _lib.dplr_chunk_workspace_raw(dplr_chunk_args(dk=32)) == 2 ** 64 - 1
    a = dplr_chunk_args()
    a.struct_size = ctypes.sizeof(_lib.DplrChunkArgs) - 8
    assert lib.kda_dplr_chunk_fwd(ctypes.byref(a)) == S["KDA_ERR_BAD_STRUCT"]
    assert _lib.dplr_chunk_fwd_raw(dplr_chunk_args(B=0, num_seqs=0)) == 0
