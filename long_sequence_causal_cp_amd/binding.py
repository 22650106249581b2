"""Thin ctypes binding of ``libcp_attn.so`` (argument marshalling only).

Every function here has the name of the C entry point it wraps and only
turns torch tensors / Python values into pointers and sizes: all computation
runs in the library's HIP kernels.  PyTorch provides device memory and
streams.  If the library is missing, loading raises instead of falling back
to anything else.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcp_attn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "cp_attn.h")

CP_MAX_CHUNKS = 8
CP_MAX_STEPS = 64
CP_OK, CP_ERR_INVALID, CP_ERR_UNSUPPORTED, CP_ERR_WORKSPACE, CP_ERR_HIP = range(5)
CP_STEP_WRITE, CP_STEP_MERGE = 0, 1
CP_BWD_DQ_ACCUMULATE, CP_BWD_DKV_ACCUMULATE = 1, 2
CP_PLAN_MERGE, CP_PLAN_FINALIZE, CP_PLAN_WRITE_O, CP_PLAN_ACTIVE = 1, 2, 4, 8
STATUS_NAMES = {0: "CP_OK", 1: "CP_ERR_INVALID", 2: "CP_ERR_UNSUPPORTED", 3: "CP_ERR_WORKSPACE", 4: "CP_ERR_HIP"}


class CpChunks(ctypes.Structure):
    """cp_chunks_t: n_chunks chunks of chunk_len tokens at absolute starts."""
    _fields_ = [("n_chunks", ctypes.c_int32), ("chunk_len", ctypes.c_int32),
                ("start", ctypes.c_int64 * CP_MAX_CHUNKS)]

    @classmethod
    def make(cls, starts: Sequence[int], chunk_len: int) -> "CpChunks":
        t = cls()
        t.n_chunks = len(starts)
        t.chunk_len = chunk_len
        for i, s in enumerate(starts):
            t.start[i] = int(s)
        return t

    def starts(self):
        return [int(self.start[i]) for i in range(self.n_chunks)]

    def __repr__(self):
        return f"CpChunks(n={self.n_chunks}, len={self.chunk_len}, start={self.starts()})"


class CpError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is not built; run __graft_entry__.build() "
                           "(python -m long_sequence_causal_cp_amd.build)")
    lib = ctypes.CDLL(path)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    pch = ctypes.POINTER(CpChunks)
    sig = {
        "cp_last_error": (ctypes.c_char_p, []),
        "cp_version": (i32, []),
        "cp_zigzag_chunks": (i32, [i32, i32, i32, i32, pch, pch]),
        "cp_attn_step_fwd": (i32, [vp, vp, vp, vp, vp, vp, i32, i32, i32, pch, pch, f32, i32, vp]),
        "cp_attn_step_fwd_fp8": (i32, [vp, vp, vp, vp, vp, vp, i32, i32, i32, pch, pch, f32, f32, f32, f32, i32,
                                       vp]),
        "cp_attn_merge": (i32, [vp, vp, vp, vp, i32, i32, i32, i32, vp, vp]),
        "cp_attn_bwd_delta": (i32, [vp, vp, vp, i32, i32, i32, i32, vp]),
        "cp_attn_step_bwd": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, pch, pch, f32, i32, vp]),
        "cp_ring_attn_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "cp_ring_attn_fwd": (i32, [vp, pch, ctypes.POINTER(vp), ctypes.POINTER(vp), pch, i32, vp, vp,
                                   i32, i32, i32, f32, vp, sz, vp, vp]),
        "cp_ring_attn_fwd_fp8_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "cp_ring_attn_fwd_fp8": (i32, [vp, pch, ctypes.POINTER(vp), ctypes.POINTER(vp), pch, i32, vp, vp,
                                       i32, i32, i32, f32, f32, f32, f32, vp, sz, vp, vp]),
        "cp_ring_attn_bwd_workspace_bytes": (sz, [i32, i32, i32, i32, i32]),
        "cp_ring_attn_bwd": (i32, [vp, pch, vp, vp, vp, ctypes.POINTER(vp), ctypes.POINTER(vp), pch, i32,
                                   ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(i32), vp,
                                   i32, i32, i32, f32, vp, sz, vp, vp]),
        "cp_profile_enable": (i32, [i32]),
        "cp_profile_read": (i32, [ctypes.POINTER(ctypes.c_float), i32, ctypes.POINTER(ctypes.c_int)]),
        "cp_profile_read_named": (i32, [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_char_p), i32,
                                        ctypes.POINTER(ctypes.c_int)]),
        "cp_test_set_delays": (i32, [i32, i32]),
        "cp_ring_attn_fwd_noalloc_max_bytes": (sz, []),
        "cp_ring_attn_fwd_noalloc": (i32, [vp, pch, ctypes.POINTER(vp), ctypes.POINTER(vp), pch, i32, vp, vp,
                                           i32, i32, i32, f32, vp, vp]),
        "cp_ring_attn_fwd_plan": (i32, [pch, pch, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                        ctypes.POINTER(i32), ctypes.POINTER(i32)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions(path: str = HEADER):
    """Names of the functions include/cp_attn.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cp_[a-z0-9_]+)\s*\(", text)))


def _check(status: int):
    if status != CP_OK:
        raise CpError(status, cp_last_error())


def cp_last_error() -> str:
    return load_library().cp_last_error().decode()


def cp_version() -> int:
    return load_library().cp_version()


def cp_zigzag_chunks(cp_size: int, rank: int, chunk_len: int, step: int = 0):
    q, kv = CpChunks(), CpChunks()
    _check(load_library().cp_zigzag_chunks(cp_size, rank, chunk_len, step, ctypes.byref(q), ctypes.byref(kv)))
    return q, kv


# ---- tensor marshalling helpers (no arithmetic) ----
def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(s):
    import torch
    if s is None:
        s = torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name):
    import torch
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or not t.is_contiguous() or t.device.type != "cuda":
        raise TypeError(f"{name} must be a contiguous {dtype} CUDA tensor")


def cp_attn_step_fwd(q, k, v, o, lse, out, q_chunks: CpChunks, kv_chunks: CpChunks,
                     softmax_scale: float, mode: int, stream=None):
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out")):
        _need(t, torch.bfloat16, n)
    _need(o, torch.float32, "o")
    _need(lse, torch.float32, "lse")
    B, H, _, D = q.shape
    _check(load_library().cp_attn_step_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(out),
                                           B, H, D, ctypes.byref(q_chunks), ctypes.byref(kv_chunks),
                                           float(softmax_scale), int(mode), _stream(stream)))


def cp_attn_merge(o_acc, lse_acc, o_part, lse_part, out=None, stream=None):
    import torch
    for t, n in ((o_acc, "o_acc"), (o_part, "o_part"), (lse_acc, "lse_acc"), (lse_part, "lse_part")):
        _need(t, torch.float32, n)
    _need(out, torch.bfloat16, "out")
    B, H, Sq, D = o_acc.shape
    _check(load_library().cp_attn_merge(_ptr(o_acc), _ptr(lse_acc), _ptr(o_part), _ptr(lse_part),
                                        B, H, Sq, D, _ptr(out), _stream(stream)))


def cp_attn_step_fwd_fp8(q, k, vt, o, lse, out, q_chunks: CpChunks, kv_chunks: CpChunks, softmax_scale: float,
                         q_scale: float, k_scale: float, v_scale: float, mode: int = CP_STEP_WRITE, stream=None):
    """q, k: e4m3 [B,H,S,D]; vt: e4m3 [B,H,D,Skv] (V transposed); torch.float8_e4m3fn tensors."""
    import torch
    for t, n in ((q, "q"), (k, "k"), (vt, "vt")):
        _need(t, torch.float8_e4m3fn, n)
    _need(o, torch.float32, "o")
    _need(lse, torch.float32, "lse")
    _need(out, torch.bfloat16, "out")
    B, H, _, D = q.shape
    _check(load_library().cp_attn_step_fwd_fp8(_ptr(q), _ptr(k), _ptr(vt), _ptr(o), _ptr(lse), _ptr(out), B, H, D,
                                               ctypes.byref(q_chunks), ctypes.byref(kv_chunks),
                                               float(softmax_scale), float(q_scale), float(k_scale),
                                               float(v_scale), int(mode), _stream(stream)))


def cp_attn_bwd_delta(out, d_out, delta, stream=None):
    import torch
    _need(out, torch.bfloat16, "out")
    _need(d_out, torch.bfloat16, "d_out")
    _need(delta, torch.float32, "delta")
    B, H, Sq, D = out.shape
    _check(load_library().cp_attn_bwd_delta(_ptr(out), _ptr(d_out), _ptr(delta), B, H, Sq, D, _stream(stream)))


def cp_attn_step_bwd(q, k, v, d_out, lse, delta, dq, dk, dv, q_chunks: CpChunks, kv_chunks: CpChunks,
                     softmax_scale: float, mode: int = 0, stream=None):
    import torch
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (d_out, "d_out")):
        _need(t, torch.bfloat16, n)
    for t, n in ((lse, "lse"), (delta, "delta"), (dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, torch.float32, n)
    B, H, _, D = q.shape
    _check(load_library().cp_attn_step_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(d_out), _ptr(lse), _ptr(delta),
                                           _ptr(dq), _ptr(dk), _ptr(dv), B, H, D, ctypes.byref(q_chunks),
                                           ctypes.byref(kv_chunks), float(softmax_scale), int(mode),
                                           _stream(stream)))


def cp_ring_attn_workspace_bytes(B: int, H: int, Skv: int, D: int, Sq: int) -> int:
    return int(load_library().cp_ring_attn_workspace_bytes(B, H, Skv, D, Sq))


def cp_ring_attn_fwd(q, q_chunks: CpChunks, k_steps, v_steps, kv_chunks_steps, out, lse,
                     softmax_scale: float, workspace, stream=None, copy_stream=None):
    import torch
    _need(q, torch.bfloat16, "q")
    _need(out, torch.bfloat16, "out")
    _need(lse, torch.float32, "lse")
    _need(workspace, torch.uint8, "workspace")
    n = len(k_steps)
    if len(v_steps) != n or len(kv_chunks_steps) != n:
        raise ValueError("k_steps, v_steps and kv_chunks_steps must have the same length")
    for t in list(k_steps) + list(v_steps):
        _need(t, torch.bfloat16, "k/v step")
    kp = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in k_steps])
    vp = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in v_steps])
    tables = (CpChunks * max(n, 1))(*kv_chunks_steps)
    if copy_stream is None:
        raise ValueError("copy_stream is required (a torch.cuda.Stream; stream itself runs the copies in order)")
    B, H, _, D = q.shape
    _check(load_library().cp_ring_attn_fwd(_ptr(q), ctypes.byref(q_chunks), kp, vp, tables, n,
                                           _ptr(out), _ptr(lse), B, H, D, float(softmax_scale),
                                           _ptr(workspace), workspace.numel(), _stream(stream),
                                           _stream(copy_stream)))


def cp_ring_attn_fwd_noalloc(q, q_chunks: CpChunks, k_steps, v_steps, kv_chunks_steps, out, lse,
                             softmax_scale: float, stream=None, copy_stream=None):
    """cp_ring_attn_fwd with the library's static scratch array as its workspace (no allocation)."""
    import torch
    _need(q, torch.bfloat16, "q")
    _need(out, torch.bfloat16, "out")
    _need(lse, torch.float32, "lse")
    n = len(k_steps)
    if len(v_steps) != n or len(kv_chunks_steps) != n:
        raise ValueError("k_steps, v_steps and kv_chunks_steps must have the same length")
    for t in list(k_steps) + list(v_steps):
        _need(t, torch.bfloat16, "k/v step")
    kp = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in k_steps])
    vp = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in v_steps])
    tables = (CpChunks * max(n, 1))(*kv_chunks_steps)
    if copy_stream is None:
        raise ValueError("copy_stream is required (a torch.cuda.Stream; stream itself runs the copies in order)")
    B, H, _, D = q.shape
    _check(load_library().cp_ring_attn_fwd_noalloc(_ptr(q), ctypes.byref(q_chunks), kp, vp, tables, n,
                                                   _ptr(out), _ptr(lse), B, H, D, float(softmax_scale),
                                                   _stream(stream), _stream(copy_stream)))


def cp_ring_attn_fwd_fp8_workspace_bytes(B: int, H: int, Skv: int, D: int, Sq: int) -> int:
    return int(load_library().cp_ring_attn_fwd_fp8_workspace_bytes(B, H, Skv, D, Sq))


def cp_ring_attn_fwd_fp8(q, q_chunks: CpChunks, k_steps, vt_steps, kv_chunks_steps, out, lse, softmax_scale: float,
                         q_scale: float, k_scale: float, v_scale: float, workspace, stream=None, copy_stream=None):
    """q, k_steps: e4m3 [B,H,S,D]; vt_steps: e4m3 [B,H,D,Skv]; torch.float8_e4m3fn tensors."""
    import torch
    _need(q, torch.float8_e4m3fn, "q")
    _need(out, torch.bfloat16, "out")
    _need(lse, torch.float32, "lse")
    _need(workspace, torch.uint8, "workspace")
    n = len(k_steps)
    if len(vt_steps) != n or len(kv_chunks_steps) != n:
        raise ValueError("k_steps, vt_steps and kv_chunks_steps must have the same length")
    for t in list(k_steps) + list(vt_steps):
        _need(t, torch.float8_e4m3fn, "k/vt step")
    kp = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in k_steps])
    vp_ = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in vt_steps])
    tables = (CpChunks * max(n, 1))(*kv_chunks_steps)
    if copy_stream is None:
        raise ValueError("copy_stream is required (a torch.cuda.Stream; stream itself runs the copies in order)")
    B, H, _, D = q.shape
    _check(load_library().cp_ring_attn_fwd_fp8(_ptr(q), ctypes.byref(q_chunks), kp, vp_, tables, n, _ptr(out),
                                               _ptr(lse), B, H, D, float(softmax_scale), float(q_scale),
                                               float(k_scale), float(v_scale), _ptr(workspace), workspace.numel(),
                                               _stream(stream), _stream(copy_stream)))


def cp_ring_attn_bwd_workspace_bytes(B: int, H: int, Skv: int, D: int, Sq: int) -> int:
    return int(load_library().cp_ring_attn_bwd_workspace_bytes(B, H, Skv, D, Sq))


def cp_ring_attn_bwd(q, q_chunks: CpChunks, d_out, out, lse, k_steps, v_steps, kv_chunks_steps, dk_steps, dv_steps,
                     dq, softmax_scale: float, workspace, dkv_accumulate=None, stream=None, copy_stream=None):
    import torch
    for t, n in ((q, "q"), (d_out, "d_out"), (out, "out")):
        _need(t, torch.bfloat16, n)
    _need(lse, torch.float32, "lse")
    _need(dq, torch.float32, "dq")
    _need(workspace, torch.uint8, "workspace")
    n = len(k_steps)
    if not (len(v_steps) == len(kv_chunks_steps) == len(dk_steps) == len(dv_steps) == n):
        raise ValueError("k_steps, v_steps, kv_chunks_steps, dk_steps and dv_steps must have the same length")
    for t in list(k_steps) + list(v_steps):
        _need(t, torch.bfloat16, "k/v step")
    for t in list(dk_steps) + list(dv_steps):
        _need(t, torch.float32, "dk/dv step")
    ptrs = lambda ts: (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in ts])
    tables = (CpChunks * max(n, 1))(*kv_chunks_steps)
    acc = None
    if dkv_accumulate is not None:
        if len(dkv_accumulate) != n:
            raise ValueError("dkv_accumulate must have one entry per step")
        acc = (ctypes.c_int * n)(*[int(bool(x)) for x in dkv_accumulate])
    if copy_stream is None:
        raise ValueError("copy_stream is required (a torch.cuda.Stream; stream itself runs the copies in order)")
    B, H, _, D = q.shape
    _check(load_library().cp_ring_attn_bwd(_ptr(q), ctypes.byref(q_chunks), _ptr(d_out), _ptr(out), _ptr(lse),
                                           ptrs(k_steps), ptrs(v_steps), tables, n, ptrs(dk_steps), ptrs(dv_steps),
                                           acc, _ptr(dq), B, H, D, float(softmax_scale), _ptr(workspace),
                                           workspace.numel(), _stream(stream), _stream(copy_stream)))


def cp_profile_enable(enable: bool):
    _check(load_library().cp_profile_enable(1 if enable else 0))


def cp_profile_read(max_entries: int = 4096):
    buf = (ctypes.c_float * max_entries)()
    n = ctypes.c_int(0)
    _check(load_library().cp_profile_read(buf, max_entries, ctypes.byref(n)))
    return [buf[i] for i in range(n.value)]


def cp_profile_read_named(max_entries: int = 4096):
    """(milliseconds, kernel name) of every timed launch, in launch order."""
    buf = (ctypes.c_float * max_entries)()
    names = (ctypes.c_char_p * max_entries)()
    n = ctypes.c_int(0)
    _check(load_library().cp_profile_read_named(buf, names, max_entries, ctypes.byref(n)))
    return [(buf[i], names[i].decode()) for i in range(n.value)]


def cp_test_set_delays(compute_us: int, copy_us: int):
    _check(load_library().cp_test_set_delays(int(compute_us), int(copy_us)))


def cp_ring_attn_fwd_plan(q_chunks: CpChunks, kv_chunks_steps):
    """Launches of cp_ring_attn_fwd for these tables: a list of (first_step, step_count, {chunk: flags})."""
    n = len(kv_chunks_steps)
    T = CpChunks * n
    cap = CP_MAX_STEPS + 1
    nl = ctypes.c_int(0)
    first = (ctypes.c_int * cap)()
    count = (ctypes.c_int * cap)()
    flags = (ctypes.c_int * (cap * CP_MAX_CHUNKS))()
    _check(load_library().cp_ring_attn_fwd_plan(ctypes.byref(q_chunks), T(*kv_chunks_steps), n, cap,
                                                ctypes.byref(nl), first, count, flags))
    return [(first[l], count[l], {c: flags[l * CP_MAX_CHUNKS + c] for c in range(CP_MAX_CHUNKS)
                                  if flags[l * CP_MAX_CHUNKS + c]}) for l in range(nl.value)]
