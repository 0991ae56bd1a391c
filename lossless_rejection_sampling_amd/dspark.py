"""Python binding of libdspark.so: the C entry points under the same names.

Argument marshalling only.  Each function checks that the tensors it is given
are contiguous, of the expected dtype and on the GPU, turns them into device
pointers and calls the library on the caller's current HIP stream.  Every step
of the round runs in the library's kernels; when the library is missing or
fails to load the calls raise instead of doing anything else.
"""

from __future__ import annotations

import ctypes
import os
import re
from typing import Optional

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "_lib", "libdspark.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "dspark.h")

DSPARK_BF16, DSPARK_F32 = 0, 1
DSPARK_OK, DSPARK_EINVAL, DSPARK_EHIP, DSPARK_EDATA = 0, -1, -2, -3
DSPARK_W_VOCAB_MAJOR, DSPARK_W_RANK_MAJOR = 0, 1
SCHED_RULES = {"early_stop": 0, "argmax": 1, "fixed": 2, "threshold": 3}
KERNEL_CLASSES = {"draft_gemm": 0, "draft_select": 1, "row_stats": 2, "accept": 3,
                  "residual_gemm": 4, "residual_select": 5, "schedule": 6, "acceptance": 7,
                  "draft_round": 8}
DSPARK_DRAFT_PER_POSITION, DSPARK_DRAFT_RESIDENT = 0, 1


class DsparkError(RuntimeError):
    def __init__(self, fn: str, code: int):
        detail = error_string(code)
        self.hip_error = 0
        if code == DSPARK_EHIP:
            self.hip_error, name = last_hip_error()
            detail += f": {name} ({self.hip_error})"
        super().__init__(f"{fn} failed: {code} ({detail})")
        self.code = code


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_SIG = {
    "dspark_abi_version": (_I, []),
    "dspark_error_string": (ctypes.c_char_p, [_I]),
    "dspark_last_hip_error": (_I, [ctypes.POINTER(ctypes.c_char_p)]),
    "dspark_workspace_bytes": (ctypes.c_size_t, [_I, _I, _I, _I]),
    "dspark_schedule_workspace_bytes": (ctypes.c_size_t, [_I, _I]),
    "dspark_pack_w2": (_I, [_P, _I, _I, _I, _P, _P]),
    "dspark_set_draft_path": (_I, [_I]),
    "dspark_set_resident_wait_bound": (_I, [ctypes.c_double, ctypes.POINTER(ctypes.c_double)]),
    "dspark_draft_round": (_I, [_P, _I, _P, _P, _I, _I, _P, _P, ctypes.c_uint64, _P,
                                _I, _I, _I, _I, _P, _P, _P, _P, _P]),
    "dspark_draft_schedule": (_I, [_P, _I, _P, _P, _I, _I, _P, _P, ctypes.c_uint64, _P, _I, _I, _I, _I, _P, _P,
                                   _P, _P, _P, _P, _P, _I, _I, ctypes.c_double, _P, _P, _P]),
    "dspark_schedule": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _P]),
    "dspark_schedule_static": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _P]),
    "dspark_schedule_ex": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_double, _P, _P, _P]),
    "dspark_verify": (_I, [_P, _P, _I, _P, _P, _I, _I, _P, _P, _P, _P, _P, _P, ctypes.c_uint64, _P,
                           _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _P]),
    "dspark_acceptance": (_I, [_P, _P, _I, _P, _P, _I, _I, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "dspark_status": (_I, [_P, _P]),
    "dspark_profile_enable": (_I, [_I, _I]),
    "dspark_profile_read": (_I, [_I, ctypes.POINTER(_I), ctypes.POINTER(ctypes.c_double)]),
    "dspark_peak_stream_read": (_I, [_P, ctypes.c_size_t, _P, _P]),
    "dspark_peak_mfma_bf16": (_I, [_I, _I, _P, _P]),
}


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() first")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def declared_functions(header: str = HEADER, with_arity: bool = False):
    """Names of the functions include/dspark.h declares (with their parameter
    counts when `with_arity`)."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    decls = re.findall(r"\b(dspark_[a-z0-9_]+)\s*\(([^()]*)\)\s*;", text)
    if with_arity:
        return {n: 0 if p.strip() in ("", "void") else p.count(",") + 1 for n, p in decls}
    return sorted(set(n for n, _ in decls))


def last_hip_error():
    """(code, name) of the HIP error behind this thread's last DSPARK_EHIP."""
    try:
        name = ctypes.c_char_p()
        code = lib().dspark_last_hip_error(ctypes.byref(name))
        return code, (name.value or b"").decode()
    except Exception:
        return -1, "unknown"


def error_string(code: int) -> str:
    try:
        return lib().dspark_error_string(code).decode()
    except Exception:
        return "unknown"


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DSPARK_BF16
    if t.dtype == torch.float32:
        return DSPARK_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t: Optional[torch.Tensor], name: str, dtype=None, optional=False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, rc: int):
    if rc != DSPARK_OK:
        raise DsparkError(fn, rc)


def dspark_abi_version() -> int:
    return lib().dspark_abi_version()


def dspark_workspace_bytes(B: int, gamma: int, V: int, r: int) -> int:
    return int(lib().dspark_workspace_bytes(B, gamma, V, r))


def dspark_schedule_workspace_bytes(B: int, gamma: int) -> int:
    return int(lib().dspark_schedule_workspace_bytes(B, gamma))


def _w_layout(U, W, V, w_layout):
    """The layout code of W2: given, or read from its shape ([V, r]: vocabulary-major,
    [r, V]: rank-major, which the round calls reject)."""
    r = U.shape[1]
    if tuple(U.shape) != (V, r) or U.dtype != W.dtype:
        raise ValueError("U must be [V, r] with the dtype of W")
    if w_layout is None:
        if tuple(W.shape) == (V, r):
            return DSPARK_W_VOCAB_MAJOR
        if tuple(W.shape) == (r, V):
            return DSPARK_W_RANK_MAJOR
        raise ValueError("W must be [V, r] (vocabulary-major) or [r, V]")
    return int(w_layout)


def dspark_pack_w2(W, W_packed, stream=None):
    """W [r, V] -> W_packed [V, r] (the vocabulary-major layout the round reads)."""
    r, V = W.shape
    if tuple(W_packed.shape) != (V, r) or W_packed.dtype != W.dtype:
        raise ValueError("W_packed must be [V, r] with the dtype of W")
    _check("dspark_pack_w2", lib().dspark_pack_w2(_dev(W, "W"), _dtype_code(W), V, r,
                                                  _dev(W_packed, "W_packed"), _stream(stream)))


def dspark_set_draft_path(path):
    """Selects the draft-round implementation (DSPARK_DRAFT_PER_POSITION, the
    default, or DSPARK_DRAFT_RESIDENT) process-wide; returns the previous one."""
    res = lib().dspark_set_draft_path(int(path))
    if res < 0:
        _check("dspark_set_draft_path", res)
    return res


def dspark_set_resident_wait_bound(seconds: float) -> float:
    """Bound (seconds) of the resident draft round's device-wide waits for later
    launches, process-wide; returns the previous bound."""
    prev = ctypes.c_double()
    _check("dspark_set_resident_wait_bound", lib().dspark_set_resident_wait_bound(float(seconds), ctypes.byref(prev)))
    return prev.value


def dspark_draft_round(base_logits, U, W, prev0, temperature, seed, pos_offset,
                       draft_tokens, draft_logq, draft_lse, workspace, stream=None, w_layout=None):
    """base_logits [B, gamma, V]; U [V, r]; W = second factor, [V, r] vocabulary-major."""
    B, gamma, V = base_logits.shape
    r = U.shape[1]
    lay = _w_layout(U, W, V, w_layout)
    rc = lib().dspark_draft_round(
        _dev(base_logits, "base_logits"), _dtype_code(base_logits), _dev(U, "U"), _dev(W, "W"),
        _dtype_code(U), lay, _dev(prev0, "prev0", torch.int32), _dev(temperature, "temperature", torch.float32),
        int(seed) & (2 ** 64 - 1), _dev(pos_offset, "pos_offset", torch.int32, optional=True),
        B, gamma, V, r, _dev(draft_tokens, "draft_tokens", torch.int32),
        _dev(draft_logq, "draft_logq", torch.float32), _dev(draft_lse, "draft_lse", torch.float64),
        _dev(workspace, "workspace", torch.uint8), _stream(stream))
    _check("dspark_draft_round", rc)


def dspark_draft_schedule(base_logits, U, W, prev0, temperature, seed, pos_offset, draft_tokens, draft_logq,
                          draft_lse, conf, tau, sps_B, sps_val, rule, param, budget, workspace, stream=None,
                          w_layout=None):
    """dspark_draft_round then dspark_schedule_ex in one call (the scheduler runs
    in the launch of the last draw)."""
    B, gamma, V = base_logits.shape
    r = U.shape[1]
    lay = _w_layout(U, W, V, w_layout)
    if tuple(conf.shape) != (B, gamma):
        raise ValueError("conf must be [B, gamma]")
    code = SCHED_RULES[rule] if isinstance(rule, str) else int(rule)
    n = int(sps_B.numel()) if sps_B is not None else 0
    rc = lib().dspark_draft_schedule(
        _dev(base_logits, "base_logits"), _dtype_code(base_logits), _dev(U, "U"), _dev(W, "W"),
        _dtype_code(U), lay, _dev(prev0, "prev0", torch.int32), _dev(temperature, "temperature", torch.float32),
        int(seed) & (2 ** 64 - 1), _dev(pos_offset, "pos_offset", torch.int32, optional=True),
        B, gamma, V, r, _dev(draft_tokens, "draft_tokens", torch.int32),
        _dev(draft_logq, "draft_logq", torch.float32), _dev(draft_lse, "draft_lse", torch.float64),
        _dev(conf, "conf", torch.float32), _dev(tau, "tau", torch.float32, optional=True),
        _dev(sps_B, "sps_B", torch.float64, optional=True), _dev(sps_val, "sps_val", torch.float64, optional=True),
        n, code, float(param), _dev(budget, "budget", torch.int32),
        _dev(workspace, "workspace", torch.uint8), _stream(stream))
    _check("dspark_draft_schedule", rc)


def dspark_schedule(conf, sps_B, sps_val, budget, workspace, stream=None):
    B, gamma = conf.shape
    rc = lib().dspark_schedule(
        _dev(conf, "conf", torch.float32), _dev(sps_B, "sps_B", torch.float64),
        _dev(sps_val, "sps_val", torch.float64), int(sps_B.numel()), B, gamma,
        _dev(budget, "budget", torch.int32), _dev(workspace, "workspace", torch.uint8), _stream(stream))
    _check("dspark_schedule", rc)


def dspark_schedule_static(conf, sps_B, sps_val, budget, status=None, stream=None):
    """dspark_schedule on the library's own scratch (no workspace, no allocation);
    status: optional device uint32 [1] that receives the data-error bits."""
    B, gamma = conf.shape
    rc = lib().dspark_schedule_static(
        _dev(conf, "conf", torch.float32), _dev(sps_B, "sps_B", torch.float64),
        _dev(sps_val, "sps_val", torch.float64), int(sps_B.numel()), B, gamma,
        _dev(budget, "budget", torch.int32), _dev(status, "status", optional=True), _stream(stream))
    _check("dspark_schedule_static", rc)


def dspark_schedule_ex(conf, tau, sps_B, sps_val, rule, param, budget, workspace, stream=None):
    """rule: a key of SCHED_RULES (or its code); tau: [gamma] float32 or None;
    sps_B / sps_val may be None for the fixed and threshold rules."""
    B, gamma = conf.shape
    code = SCHED_RULES[rule] if isinstance(rule, str) else int(rule)
    n = int(sps_B.numel()) if sps_B is not None else 0
    rc = lib().dspark_schedule_ex(
        _dev(conf, "conf", torch.float32), _dev(tau, "tau", torch.float32, optional=True),
        _dev(sps_B, "sps_B", torch.float64, optional=True), _dev(sps_val, "sps_val", torch.float64, optional=True),
        n, B, gamma, code, float(param), _dev(budget, "budget", torch.int32),
        _dev(workspace, "workspace", torch.uint8), _stream(stream))
    _check("dspark_schedule_ex", rc)


def dspark_verify(target_logits, base_logits, U, W, prev0, draft_tokens, draft_logq, draft_lse,
                  budget, temperature, seed, pos_offset, out_tokens, num_accepted, num_emitted,
                  workspace, debug_logp_logq=None, debug_residual=None, stream=None, w_layout=None):
    B, gamma, V = base_logits.shape
    r = U.shape[1]
    if tuple(target_logits.shape) != (B, gamma + 1, V) or target_logits.dtype != base_logits.dtype:
        raise ValueError("target_logits must be [B, gamma+1, V] with the dtype of base_logits")
    lay = _w_layout(U, W, V, w_layout)
    rc = lib().dspark_verify(
        _dev(target_logits, "target_logits"), _dev(base_logits, "base_logits"), _dtype_code(base_logits),
        _dev(U, "U"), _dev(W, "W"), _dtype_code(U), lay, _dev(prev0, "prev0", torch.int32),
        _dev(draft_tokens, "draft_tokens", torch.int32), _dev(draft_logq, "draft_logq", torch.float32),
        _dev(draft_lse, "draft_lse", torch.float64), _dev(budget, "budget", torch.int32, optional=True),
        _dev(temperature, "temperature", torch.float32), int(seed) & (2 ** 64 - 1),
        _dev(pos_offset, "pos_offset", torch.int32, optional=True), B, gamma, V, r,
        _dev(out_tokens, "out_tokens", torch.int32), _dev(num_accepted, "num_accepted", torch.int32),
        _dev(num_emitted, "num_emitted", torch.int32),
        _dev(debug_logp_logq, "debug_logp_logq", torch.float32, optional=True),
        _dev(debug_residual, "debug_residual", torch.float32, optional=True),
        _dev(workspace, "workspace", torch.uint8), _stream(stream))
    _check("dspark_verify", rc)


def dspark_acceptance(target_logits, base_logits, U, W, prev0, draft_tokens, draft_lse, temperature,
                      c_star, workspace, stream=None, w_layout=None):
    """c_star [B, gamma] float64 out: sum_v min(p_k, q_k) of every drafted position."""
    B, gamma, V = base_logits.shape
    r = U.shape[1]
    if tuple(target_logits.shape) != (B, gamma + 1, V) or target_logits.dtype != base_logits.dtype:
        raise ValueError("target_logits must be [B, gamma+1, V] with the dtype of base_logits")
    lay = _w_layout(U, W, V, w_layout)
    rc = lib().dspark_acceptance(
        _dev(target_logits, "target_logits"), _dev(base_logits, "base_logits"), _dtype_code(base_logits),
        _dev(U, "U"), _dev(W, "W"), _dtype_code(U), lay, _dev(prev0, "prev0", torch.int32),
        _dev(draft_tokens, "draft_tokens", torch.int32), _dev(draft_lse, "draft_lse", torch.float64),
        _dev(temperature, "temperature", torch.float32), B, gamma, V, r,
        _dev(c_star, "c_star", torch.float64), _dev(workspace, "workspace", torch.uint8), _stream(stream))
    _check("dspark_acceptance", rc)


def dspark_status(workspace, stream=None) -> int:
    return int(lib().dspark_status(_dev(workspace, "workspace", torch.uint8), _stream(stream)))


def dspark_profile_enable(kernel_class: int, enabled=True):
    """enabled: False/0 off, True/1 every launch, k > 1 every k-th launch."""
    _check("dspark_profile_enable", lib().dspark_profile_enable(int(kernel_class), int(enabled)))


def dspark_profile_read(kernel_class: int):
    n = ctypes.c_int(0)
    ms = ctypes.c_double(0.0)
    _check("dspark_profile_read", lib().dspark_profile_read(int(kernel_class), ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


def dspark_peak_stream_read(buf, sink, stream=None):
    """One streaming read of the whole uint8 device tensor `buf` (size a multiple of 16)."""
    _check("dspark_peak_stream_read", lib().dspark_peak_stream_read(
        _dev(buf, "buf", torch.uint8), buf.numel(), _dev(sink, "sink", torch.int32), _stream(stream)))


def dspark_peak_mfma_bf16(blocks, iters, sink, stream=None):
    """blocks * 4 * iters * 4 * 32768 flops of dense bf16 MFMA."""
    _check("dspark_peak_mfma_bf16", lib().dspark_peak_mfma_bf16(
        int(blocks), int(iters), _dev(sink, "sink", torch.int32), _stream(stream)))
