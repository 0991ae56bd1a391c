"""ctypes binding of the C oracle (oracle/dspark_ref.c): the ref_ entry points
on host arrays, returning the numpy oracle's result types.

Test infrastructure only (see the package docstring).  Inputs are the round's
values as float32 arrays (bf16 and fp32 data are exact in fp32); W is W2 as the
pages print it, [r, V].
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from .dspark import DraftResult, ScheduleResult, VerifyResult

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libdspark_ref.so")
_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(f"{LIB} is not built (oracle/build.py)")
        _lib = ctypes.CDLL(LIB)
        _lib.ref_threads.argtypes, _lib.ref_threads.restype = [_I], _I
        _lib.ref_draft_round.argtypes = [_P, _I, _P, _P, _I, _P, _P, ctypes.c_uint64, _P, _P, _I, _I, _I, _I,
                                         _P, _P, _P, _P]
        _lib.ref_draft_round.restype = _I
        _lib.ref_verify.argtypes = [_P, _P, _I, _P, _P, _I, _P, _P, _P, ctypes.c_uint64, _P, _P, _P, _I, _I, _I,
                                    _I, _P, _P, _P, _P, _P, _P, _P, _P]
        _lib.ref_verify.restype = _I
        _lib.ref_schedule.argtypes = [_P, _P, _P, _I, _I, _I, _P, _P]
        _lib.ref_schedule.restype = _I
    return _lib


def threads(n: int = 0) -> int:
    """Sets the OpenMP thread count when n > 0; returns the count in use."""
    return int(lib().ref_threads(int(n)))


def _f32(a):
    x = np.ascontiguousarray(np.asarray(a), dtype=np.float32)
    if np.asarray(a).dtype == np.float64 and not np.array_equal(x.astype(np.float64), np.asarray(a)):
        raise ValueError("the C oracle takes bf16 / fp32 inputs: the values must be exact in fp32")
    return x


def _i32(a):
    return None if a is None else np.ascontiguousarray(np.asarray(a), dtype=np.int32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_P)


def draft_round(base, U, W, prev0, temperature, seed: int, pos_offset=None, req_ids=None) -> DraftResult:
    base, U, W = _f32(base), _f32(U), _f32(W)
    B, gamma, V = base.shape
    r = U.shape[1]
    if U.shape != (V, r) or W.shape != (r, V):
        raise ValueError("U must be [V, r] and W [r, V]")
    prev0, off, ids = _i32(prev0), _i32(pos_offset), _i32(req_ids)
    T = np.ascontiguousarray(temperature, dtype=np.float32)
    tokens = np.zeros((B, gamma), dtype=np.int32)
    logq, lse, margin = (np.zeros((B, gamma)) for _ in range(3))
    rc = lib().ref_draft_round(_ptr(base), 1, _ptr(U), _ptr(W), 1, _ptr(prev0), _ptr(T), int(seed) & (2**64 - 1),
                               _ptr(off), _ptr(ids), B, gamma, V, r, _ptr(tokens), _ptr(logq), _ptr(lse), _ptr(margin))
    if rc != 0:
        raise ValueError("ref_draft_round rejected its inputs")
    return DraftResult(tokens, logq, lse, margin)


def verify(target, base, U, W, prev0, draft_tokens, temperature, seed: int, budget=None, pos_offset=None,
           req_ids=None, keep_residual=False) -> VerifyResult:
    target, base, U, W = _f32(target), _f32(base), _f32(U), _f32(W)
    B, gamma, V = base.shape
    r = U.shape[1]
    if target.shape != (B, gamma + 1, V) or U.shape != (V, r) or W.shape != (r, V):
        raise ValueError("shapes: target [B, gamma+1, V], U [V, r], W [r, V]")
    prev0, drafts, L, off, ids = _i32(prev0), _i32(draft_tokens), _i32(budget), _i32(pos_offset), _i32(req_ids)
    T = np.ascontiguousarray(temperature, dtype=np.float32)
    out = np.zeros((B, gamma + 1), dtype=np.int32)
    n_acc, n_emit, rows_flagged = (np.zeros(B, dtype=np.int32) for _ in range(3))
    logp, logq = np.zeros((B, gamma)), np.zeros((B, gamma))
    margin = np.zeros(B)
    res = np.empty((B, V)) if keep_residual else None
    rc = lib().ref_verify(_ptr(target), _ptr(base), 1, _ptr(U), _ptr(W), 1, _ptr(prev0), _ptr(drafts), _ptr(T),
                          int(seed) & (2**64 - 1), _ptr(L), _ptr(off), _ptr(ids), B, gamma, V, r, _ptr(out),
                          _ptr(n_acc), _ptr(n_emit), _ptr(logp), _ptr(logq), _ptr(margin), _ptr(rows_flagged),
                          _ptr(res))
    if rc != 0:
        raise ValueError("ref_verify rejected its inputs")
    residual = {} if res is None else {b: res[b] for b in range(B) if not np.isnan(res[b, 0])}
    return VerifyResult(out, n_acc, n_emit, logp, logq, residual, margin, rows_flagged)


def schedule(conf, sps_B, sps_val) -> ScheduleResult:
    c = np.ascontiguousarray(conf, dtype=np.float32)
    B, gamma = c.shape
    sB = np.ascontiguousarray(sps_B, dtype=np.float64)
    sv = np.ascontiguousarray(sps_val, dtype=np.float64)
    budget = np.zeros(B, dtype=np.int32)
    gap = ctypes.c_double(0.0)
    rc = lib().ref_schedule(_ptr(c), _ptr(sB), _ptr(sv), len(sB), B, gamma, _ptr(budget), ctypes.byref(gap))
    if rc != 0:
        raise ValueError("ref_schedule rejected its inputs")
    return ScheduleResult(budget, int(budget.sum()), gap.value)
