"""Thin Python binding of liblaga.so (argument marshalling only).

Every function takes torch tensors that already live on the GPU, passes their
device pointers and the current HIP stream to the C ABI declared in
include/laga.h, and raises LagaError on a non-OK status.  No computation
happens here; there is no fallback when the library is missing.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblaga.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "laga.h")

LAGA_F32, LAGA_BF16 = 0, 1
LAGA_OPERANDS_FP16, LAGA_OPERANDS_SPLIT = 0, 1
LAGA_BWD_STAGES = 7
LAGA_KV_LO_SHIFT = 12  # the #define of laga.h: scale exponent of the e4m3 low plane of split K/V
LAGA_NOALLOC_SCRATCH_BYTES = 256 << 20  # the #define of laga.h: static scratch of laga_attn_bwd_noalloc
BWD_STAGE_NAMES = ("bwd_delta", "attn_bwd_dkdv", "attn_bwd_dq", "dk_pe_head_sum", "fold_dL", "fold_dW",
                   "rmsnorm_bwd")
STATUS = {0: "LAGA_OK", 1: "LAGA_ERR_INVALID", 2: "LAGA_ERR_UNSUPPORTED", 3: "LAGA_ERR_ALIGN",
          4: "LAGA_ERR_HIP", 5: "LAGA_ERR_WORKSPACE"}


class LagaError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: {text}")
        self.status = status


class laga_dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("S", ctypes.c_int64), ("n_h", ctypes.c_int32),
                ("sp_size", ctypes.c_int32), ("sp_rank", ctypes.c_int32), ("d_kv", ctypes.c_int32),
                ("d_nope", ctypes.c_int32), ("d_rope", ctypes.c_int32), ("d_v", ctypes.c_int32),
                ("eps", ctypes.c_float), ("dtype", ctypes.c_int32), ("precision", ctypes.c_int32)]


def make_dims(B, S, n_h, sp_size, sp_rank, d_kv, d_nope, d_rope, d_v, dtype, precision=0, eps=1e-6):
    return laga_dims(B, S, n_h, sp_size, sp_rank, d_kv, d_nope, d_rope, d_v, eps, dtype, precision)


_P = ctypes.c_void_p
_SIGS = {
    "laga_kv_elem_bytes": (ctypes.c_size_t, [ctypes.POINTER(laga_dims)]),
    "laga_latent_norm": (ctypes.c_int, [ctypes.POINTER(laga_dims), _P, _P, _P, _P, _P]),
    "laga_kv_up": (ctypes.c_int, [ctypes.POINTER(laga_dims), _P, _P, _P, _P, _P]),
    "laga_attn_fwd": (ctypes.c_int, [ctypes.POINTER(laga_dims), _P, _P, _P, _P, _P, _P, _P]),
    "laga_absorbed_fwd": (ctypes.c_int, [ctypes.POINTER(laga_dims)] + [_P] * 10),
    "laga_attn_fwd_fused_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(laga_dims)]),
    "laga_absorbed_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(laga_dims)]),
    "laga_absorbed_bwd_min_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(laga_dims)]),
    "laga_absorbed_bwd": (ctypes.c_int, [ctypes.POINTER(laga_dims)] + [_P] * 13 + [ctypes.c_size_t, _P]),
    "laga_attn_fwd_fused": (ctypes.c_int, [ctypes.POINTER(laga_dims)] + [_P] * 8 + [ctypes.c_size_t, _P]),
    "laga_attn_bwd_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(laga_dims)]),
    "laga_attn_bwd": (ctypes.c_int, [ctypes.POINTER(laga_dims)] + [_P] * 17 + [ctypes.c_size_t, _P]),
    "laga_attn_bwd_traced": (ctypes.c_int, [ctypes.POINTER(laga_dims)] + [_P] * 17
                             + [ctypes.c_size_t, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, _P]),
    "laga_attn_bwd_noalloc": (ctypes.c_int, [ctypes.POINTER(laga_dims)] + [_P] * 17),
    "laga_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblaga.so once.  torch is imported first so the library binds to
    the HIP runtime torch already loaded (one runtime per process)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m head_latent_attention_laga_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions(header: str = HEADER) -> list[str]:
    """Names of the functions include/laga.h declares."""
    text = open(header).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(laga_\w+)\s*\(", text, re.M)))


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, status: int):
    if status != 0:
        text = load().laga_status_string(status).decode()
        raise LagaError(fn, status, text)


def kv_elem_bytes(dims: laga_dims) -> int:
    return int(load().laga_kv_elem_bytes(ctypes.byref(dims)))


def latent_norm(dims, latent, gamma, latent_n, rstd, stream=None):
    _check("laga_latent_norm", load().laga_latent_norm(
        ctypes.byref(dims), _ptr(latent), _ptr(gamma), _ptr(latent_n), _ptr(rstd), _stream(stream)))


def kv_up(dims, latent_n, w_kv_b, k_nope, v, stream=None):
    _check("laga_kv_up", load().laga_kv_up(
        ctypes.byref(dims), _ptr(latent_n), _ptr(w_kv_b), _ptr(k_nope), _ptr(v), _stream(stream)))


def attn_fwd(dims, q, k_nope, k_pe, v, o, lse, stream=None):
    _check("laga_attn_fwd", load().laga_attn_fwd(
        ctypes.byref(dims), _ptr(q), _ptr(k_nope), _ptr(k_pe), _ptr(v), _ptr(o), _ptr(lse),
        _stream(stream)))


def absorbed_fwd(dims, q, latent_n, k_pe, w_kv_b, q_abs, kx, acc, o, lse, stream=None):
    _check("laga_absorbed_fwd", load().laga_absorbed_fwd(
        ctypes.byref(dims), _ptr(q), _ptr(latent_n), _ptr(k_pe), _ptr(w_kv_b), _ptr(q_abs), _ptr(kx), _ptr(acc),
        _ptr(o), _ptr(lse), _stream(stream)))


def attn_fwd_fused_workspace_bytes(dims) -> int:
    return int(load().laga_attn_fwd_fused_workspace_bytes(ctypes.byref(dims)))


def attn_fwd_fused(dims, q, latent, gamma, k_pe, w_kv_b, o, lse, workspace, stream=None):
    _check("laga_attn_fwd_fused", load().laga_attn_fwd_fused(
        ctypes.byref(dims), _ptr(q), _ptr(latent), _ptr(gamma), _ptr(k_pe), _ptr(w_kv_b), _ptr(o), _ptr(lse),
        _ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(stream)))


def absorbed_bwd_workspace_bytes(dims) -> int:
    return int(load().laga_absorbed_bwd_workspace_bytes(ctypes.byref(dims)))


def absorbed_bwd_min_workspace_bytes(dims) -> int:
    return int(load().laga_absorbed_bwd_min_workspace_bytes(ctypes.byref(dims)))


def absorbed_bwd(dims, q, latent, gamma, rstd, k_pe, w_kv_b, d_o, dq, d_latent, d_k_pe, d_w_kv_b, d_gamma,
                 workspace, stream=None):
    _check("laga_absorbed_bwd", load().laga_absorbed_bwd(
        ctypes.byref(dims), _ptr(q), _ptr(latent), _ptr(gamma), _ptr(rstd), _ptr(k_pe), _ptr(w_kv_b), _ptr(d_o),
        _ptr(dq), _ptr(d_latent), _ptr(d_k_pe), _ptr(d_w_kv_b), _ptr(d_gamma), _ptr(workspace),
        ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(stream)))


def attn_bwd_workspace_bytes(dims) -> int:
    return int(load().laga_attn_bwd_workspace_bytes(ctypes.byref(dims)))


def attn_bwd(dims, q, latent, gamma, rstd, k_nope, k_pe, v, w_kv_b, o, lse, d_o, dq, d_latent,
             d_k_pe, d_w_kv_b, d_gamma, workspace, stream=None):
    _check("laga_attn_bwd", load().laga_attn_bwd(
        ctypes.byref(dims), _ptr(q), _ptr(latent), _ptr(gamma), _ptr(rstd), _ptr(k_nope), _ptr(k_pe),
        _ptr(v), _ptr(w_kv_b), _ptr(o), _ptr(lse), _ptr(d_o), _ptr(dq), _ptr(d_latent), _ptr(d_k_pe),
        _ptr(d_w_kv_b), _ptr(d_gamma), _ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
        _stream(stream)))


def attn_bwd_noalloc(dims, q, latent, gamma, rstd, k_nope, k_pe, v, w_kv_b, o, lse, d_o, dq, d_latent,
                     d_k_pe, d_w_kv_b, d_gamma, stream=None):
    """laga_attn_bwd on the library's static per-device scratch (no workspace argument, no allocation)."""
    _check("laga_attn_bwd_noalloc", load().laga_attn_bwd_noalloc(
        ctypes.byref(dims), _ptr(q), _ptr(latent), _ptr(gamma), _ptr(rstd), _ptr(k_nope), _ptr(k_pe),
        _ptr(v), _ptr(w_kv_b), _ptr(o), _ptr(lse), _ptr(d_o), _ptr(dq), _ptr(d_latent), _ptr(d_k_pe),
        _ptr(d_w_kv_b), _ptr(d_gamma), _stream(stream)))


def attn_bwd_traced(dims, q, latent, gamma, rstd, k_nope, k_pe, v, w_kv_b, o, lse, d_o, dq, d_latent,
                    d_k_pe, d_w_kv_b, d_gamma, workspace, events, stream=None):
    """laga_attn_bwd recording `events` (LAGA_BWD_STAGES + 1 torch.cuda.Event with timing) around its stages."""
    if len(events) != LAGA_BWD_STAGES + 1:
        raise ValueError(f"need {LAGA_BWD_STAGES + 1} events")
    for e in events:
        if e.cuda_event == 0:  # torch creates the HIP event lazily
            e.record()
    arr = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    _check("laga_attn_bwd_traced", load().laga_attn_bwd_traced(
        ctypes.byref(dims), _ptr(q), _ptr(latent), _ptr(gamma), _ptr(rstd), _ptr(k_nope), _ptr(k_pe),
        _ptr(v), _ptr(w_kv_b), _ptr(o), _ptr(lse), _ptr(d_o), _ptr(dq), _ptr(d_latent), _ptr(d_k_pe),
        _ptr(d_w_kv_b), _ptr(d_gamma), _ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
        arr, len(events), _stream(stream)))
