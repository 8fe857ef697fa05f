"""fp64 CPU oracle for chunkwise causal linear attention — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this
package.  It shares no code with the HIP library: the recurrence itself is plain C
(``linattn_oracle.c``, built with gcc), and ``forms.py`` holds two independent fp64
restatements used to pin it (brute-force masked attention and the parallel form).

Pins (see tests/test_oracle_pins.py): brute force on tiny inputs, the parallel form,
gamma = 1 reducing to plain (Katharopoulos) linear attention, closed forms, a hand-worked
fixture under tests/golden/, split/resume, chained single steps and linearity.
The backward (``bwd``, back-propagation through the same recurrence in C) is pinned in
tests/test_oracle_bwd_pins.py by central finite differences of the pinned forward and by
the closed-form matrix gradients of plain causal linear attention.
The gated delta rule (``gdn_fwd``, C) is pinned in tests/test_oracle_gdn_pins.py by exact
recall, the reduction to decayed linear attention for orthogonal keys, the beta = 0
closed form and an independent chunked (UT-transform) form.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "linattn_oracle.c")
_LIB = os.path.join(_HERE, "liblinattn_oracle.so")

DECAY_CODES = {"none": 0, "gamma": 1, "gate": 2, "token": 3}
PHI_ELU1, NORMALIZE = 1, 2
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (fp64, OpenMP, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                        "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", _SRC, "-o", tmp,
                        "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        p, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_fwd.argtypes = [p, p, p, c_int, p, c_int, p, p, p, i64, p,
                                   i64, i64, i64, i64, i64, c_int, c_int]
        lib.oracle_fwd.restype = c_int
        lib.oracle_step.argtypes = [p, p, p, c_int, p, c_int, p, p, i64, i64, i64, i64,
                                    c_int, c_int]
        lib.oracle_step.restype = c_int
        lib.oracle_bwd.argtypes = [p, p, p, c_int, p, c_int, p, p, p, p, p, p, p, p,
                                   i64, i64, i64, i64, i64, c_int, c_int]
        lib.oracle_bwd.restype = c_int
        lib.oracle_gdn_fwd.argtypes = [p, p, p, c_int, p, p, p, p, p, i64, i64, i64, i64, i64,
                                       c_int]
        lib.oracle_gdn_fwd.restype = c_int
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(x: np.ndarray) -> int:
    if x.dtype == np.uint16:
        return 1
    if x.dtype == np.float32:
        return 0
    if x.dtype == np.float64:
        return 2     # values the oracle derived itself (fwd_proj's projections)
    raise TypeError("oracle inputs are fp32 / fp64 arrays or bf16 bit patterns (uint16)")


def fwd(q, k, v, decay=None, decay_kind="none", init=None, *, phi_elu1=False,
        normalize=False, rows: Optional[Sequence[int]] = None, want_out=True,
        want_final=True, nthreads=0):
    """Run the recurrence.  q, k: [B,H,T,dk]; v: [B,H,T,dv] (fp32 or uint16 bf16 bits).

    decay: gamma [H], gate [B,H,T,dk] or per-token [B,H,T] fp32 (per decay_kind).
    init: [B,H,dk,dv+n] (fp32 or fp64) or None.  rows: token indices to record.
    Returns (out fp64 [B,H,len(rows) or T,dv] or None, final fp64 [B,H,dk,dv+n] or None).
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k, v must share one dtype")
    B, H, T, dk = q.shape
    dv = v.shape[3]
    if k.shape != q.shape or v.shape[:3] != (B, H, T):
        raise ValueError("shape mismatch")
    kind = DECAY_CODES[decay_kind]
    dec = None if decay is None else np.ascontiguousarray(decay, dtype=np.float32)
    if kind and dec is None:
        raise ValueError("decay values missing")
    ncol = dv + (1 if normalize else 0)
    ini = None
    if init is not None:
        ini = np.ascontiguousarray(init, dtype=np.float64)
        if ini.shape != (B, H, dk, ncol):
            raise ValueError(f"init must be {(B, H, dk, ncol)}")
    rows_arr = None
    nrows = T
    if rows is not None:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        if np.any(np.diff(rows_arr) <= 0) or (rows_arr.size and (rows_arr[0] < 0 or rows_arr[-1] >= T)):
            raise ValueError("rows must be ascending token indices")
        nrows = rows_arr.size
    out = np.empty((B, H, nrows, dv), dtype=np.float64) if want_out else None
    fin = np.empty((B, H, dk, ncol), dtype=np.float64) if want_final else None
    flags = (PHI_ELU1 if phi_elu1 else 0) | (NORMALIZE if normalize else 0)
    rc = _load().oracle_fwd(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(dec), kind, _ptr(ini),
                            _ptr(out), _ptr(rows_arr), nrows, _ptr(fin), B, H, T, dk, dv,
                            flags, int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_fwd failed")
    return out, fin


def step(q, k, v, state, decay=None, decay_kind="none", *, phi_elu1=False, normalize=False,
         nthreads=0):
    """One decoding step.  q, k: [B,H,dk]; v: [B,H,dv]; decay: gamma [H], gate [B,H,dk],
    per-token [B,H]; state fp64 [B,H,dk,dv+n] (updated in place).  Returns out [B,H,dv]."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dt = _dtype_code(q)
    B, H, dk = q.shape
    dv = v.shape[2]
    if state.dtype != np.float64 or not state.flags.c_contiguous:
        raise TypeError("state must be a contiguous fp64 array")
    dec = None if decay is None else np.ascontiguousarray(decay, dtype=np.float32)
    out = np.empty((B, H, dv), dtype=np.float64)
    flags = (PHI_ELU1 if phi_elu1 else 0) | (NORMALIZE if normalize else 0)
    rc = _load().oracle_step(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(dec),
                             DECAY_CODES[decay_kind], _ptr(state), _ptr(out), B, H, dk, dv,
                             flags, int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_step failed")
    return out


def bwd(q, k, v, dout, decay=None, decay_kind="none", init=None, dfinal=None, *,
        phi_elu1=False, want_dgate=True, nthreads=0):
    """Gradients of L = sum(dout * o) + sum(dfinal * h_T) (no normaliser) by back-
    propagation through the recurrence.  q, k, v, dout as in ``fwd`` (dout shares q's
    dtype); init, dfinal: [B,H,dk,dv] or None.

    Returns a dict of fp64 arrays: dq, dk [B,H,T,dk]; dv [B,H,T,dv]; dgate shaped like the
    decay (None without one, or when want_dgate is false); dinit [B,H,dk,dv].
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dout = np.ascontiguousarray(dout)
    dt = _dtype_code(q)
    if any(_dtype_code(x) != dt for x in (k, v, dout)):
        raise TypeError("q, k, v, dout must share one dtype")
    B, H, T, dk = q.shape
    dv = v.shape[3]
    if k.shape != q.shape or v.shape[:3] != (B, H, T) or dout.shape != v.shape:
        raise ValueError("shape mismatch")
    kind = DECAY_CODES[decay_kind]
    dec = None if decay is None else np.ascontiguousarray(decay, dtype=np.float32)
    if kind and dec is None:
        raise ValueError("decay values missing")

    def state(x):
        if x is None:
            return None
        x = np.ascontiguousarray(x, dtype=np.float64)
        if x.shape != (B, H, dk, dv):
            raise ValueError(f"state must be {(B, H, dk, dv)}")
        return x

    ini, dfin = state(init), state(dfinal)
    dq = np.empty((B, H, T, dk))
    dkk = np.empty((B, H, T, dk))
    dvv = np.empty((B, H, T, dv))
    dg = None
    if kind and want_dgate:
        dg = np.empty(dec.shape, dtype=np.float64)
    dini = np.empty((B, H, dk, dv))
    rc = _load().oracle_bwd(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(dec), kind, _ptr(ini),
                            _ptr(dout), _ptr(dfin), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dg),
                            _ptr(dini), B, H, T, dk, dv, PHI_ELU1 if phi_elu1 else 0,
                            int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_bwd failed")
    return {"dq": dq, "dk": dkk, "dv": dvv, "dgate": dg, "dinit": dini}


def gdn_fwd(q, k, v, alpha, beta, init=None, *, want_out=True, want_final=True, nthreads=0):
    """Gated delta rule, token by token.  q, k [B,H,T,dk]; v [B,H,T,dv] (fp32 or bf16 bits);
    alpha, beta fp32 [B,H,T]; init [B,H,dk,dv] or None.  Returns (out fp64 [B,H,T,dv],
    final fp64 [B,H,dk,dv])."""
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k, v must share one dtype")
    B, H, T, dk = q.shape
    dv = v.shape[3]
    al = np.ascontiguousarray(alpha, dtype=np.float32)
    be = np.ascontiguousarray(beta, dtype=np.float32)
    if al.shape != (B, H, T) or be.shape != (B, H, T):
        raise ValueError("alpha and beta must be [B,H,T]")
    ini = None if init is None else np.ascontiguousarray(init, dtype=np.float64)
    if ini is not None and ini.shape != (B, H, dk, dv):
        raise ValueError(f"init must be {(B, H, dk, dv)}")
    out = np.empty((B, H, T, dv)) if want_out else None
    fin = np.empty((B, H, dk, dv)) if want_final else None
    rc = _load().oracle_gdn_fwd(_ptr(q), _ptr(k), _ptr(v), dt, _ptr(al), _ptr(be), _ptr(ini),
                                _ptr(out), _ptr(fin), B, H, T, dk, dv, int(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_gdn_fwd failed")
    return out, fin


def _widen(x: np.ndarray) -> np.ndarray:
    """Stored inputs (bf16 bit patterns or fp32) widened exactly to fp64."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def fwd_proj(x, w_q, w_k, w_v, H, decay=None, decay_kind="none", init=None, *,
             phi_elu1=False, normalize=False, nthreads=0):
    """The layer's input side followed by the recurrence, in fp64: per token the
    projections q = x W_q, k = x W_k, v = x W_v (x [B,T,hidden], W [hidden, H*d], head h
    taking columns h*d .. h*d+d-1, as the FLA guide's layers map [B,T,hidden] to heads),
    then fwd() with phi applied to the projected q and k.  decay: gamma [H], or the gate /
    per-token decay token-major ([B,T,H,dk] / [B,T,H]).  Returns (out [B,T,H,dv] fp64,
    final [B,H,dk,dv(+1)] fp64)."""
    X = _widen(x)
    B, T, _ = X.shape
    dk = np.asarray(w_q).shape[1] // H
    dv = np.asarray(w_v).shape[1] // H

    def heads(w, d):
        y = X @ _widen(w)                                  # [B, T, H*d], fp64
        return np.ascontiguousarray(y.reshape(B, T, H, d).transpose(0, 2, 1, 3))

    q, k, v = heads(w_q, dk), heads(w_k, dk), heads(w_v, dv)
    dec = decay
    if decay is not None and decay_kind in ("gate", "token"):
        dec = np.ascontiguousarray(np.swapaxes(np.asarray(decay), 1, 2))
    out, fin = fwd(q, k, v, dec, decay_kind, init, phi_elu1=phi_elu1, normalize=normalize,
                   nthreads=nthreads)
    return np.ascontiguousarray(out.transpose(0, 2, 1, 3)), fin
