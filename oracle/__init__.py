"""CPU float64 oracle for the OSDN forward and decode step.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg
may import this package; the product path (the HIP library and its Python binding) never
does, and shares no code with it.

``chunk_fwd`` runs the plain token-by-token float64 recurrence of ``osdn_oracle.c``
(OSDN: Improving Delta Rule with Provable Online Preconditioning in Linear Attention,
technical summary, sections 1 and 2.1; gated form from Erase-then-Delta Attention,
section 2.2, eq. 4; channel-wise gate from the same section, eq. 5).  ``step`` is the same loop body for one token.  State is stored as
M = S^T, [B, H, dk, dv].

``precond`` (numpy, float64) is the Phase-1 preconditioner scan that produces the d_t sequence
(same summary, sections 2.2 and 2.3); ``chunkwise`` holds float64 models of the chunk forms
of both recurrences, checked against the token loops; ``backward`` (numpy, float64) is
reverse-mode differentiation of the token recurrence (the gradients of every input).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "osdn_oracle.c")
_LIB = os.path.join(_HERE, "_build", "libosdn_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (IEEE float64: no fast-math, no FMA contraction)."""
    os.makedirs(os.path.dirname(_LIB), exist_ok=True)
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC",
                               "-shared", "-pthread", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.osdn_oracle_fwd.restype = ctypes.c_int
        lib.osdn_oracle_fwd.argtypes = [dp] * 9 + [i64] * 5 + [ctypes.c_int]
        lib.osdn_oracle_fwd2.restype = ctypes.c_int
        lib.osdn_oracle_fwd2.argtypes = [dp] * 10 + [i64] * 5 + [ctypes.c_int]
        _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    if x is None:
        return ctypes.POINTER(ctypes.c_double)()
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def chunk_fwd(q, k, v, beta, d, alpha=None, S0=None, nthreads: Optional[int] = None,
              want_o: bool = True, alpha_ch=None) -> Tuple[Optional[np.ndarray], np.ndarray]:
    """Token-by-token float64 recurrence.

    q, k, d: [B,H,T,dk]; v: [B,H,T,dv]; beta, alpha: [B,H,T]; S0: [B,H,dk,dv] (M = S^T);
    alpha_ch: [B,H,T,dk], the channel-wise (per key feature) gate, or None.
    Returns (o [B,H,T,dv] float64 or None, S_T [B,H,dk,dv] float64).
    """
    q, k, v, beta, d, alpha, S0, alpha_ch = map(_f64, (q, k, v, beta, d, alpha, S0, alpha_ch))
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == (B, H, T, dk) and d.shape == (B, H, T, dk)
    assert v.shape == (B, H, T, dv) and beta.shape == (B, H, T)
    assert alpha is None or alpha.shape == (B, H, T)
    assert S0 is None or S0.shape == (B, H, dk, dv)
    assert alpha_ch is None or alpha_ch.shape == (B, H, T, dk)
    o = np.empty((B, H, T, dv), dtype=np.float64) if want_o else None
    S_T = np.empty((B, H, dk, dv), dtype=np.float64)
    nt = default_threads() if nthreads is None else nthreads
    rc = _load().osdn_oracle_fwd2(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(d), _ptr(alpha),
                                  _ptr(alpha_ch), _ptr(S0), _ptr(o), _ptr(S_T), B, H, T, dk,
                                  dv, nt)
    if rc != 0:
        raise RuntimeError("osdn_oracle_fwd failed")
    return o, S_T


def step(q, k, v, beta, d, alpha, S, nthreads: Optional[int] = None, alpha_ch=None
         ) -> Tuple[np.ndarray, np.ndarray]:
    """One token for every (b,h): q, k, d [B,H,dk]; v [B,H,dv]; beta, alpha [B,H] (alpha may
    be None); alpha_ch [B,H,dk] or None; S [B,H,dk,dv].  Returns (o [B,H,dv],
    S_new [B,H,dk,dv])."""
    add_t = lambda x: None if x is None else np.asarray(x)[:, :, None]
    o, S_new = chunk_fwd(add_t(q), add_t(k), add_t(v), add_t(beta), add_t(d), add_t(alpha), S,
                         nthreads=nthreads, alpha_ch=add_t(alpha_ch))
    return o[:, :, 0], S_new
