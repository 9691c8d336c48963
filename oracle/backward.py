"""Float64 CPU oracle for the gradients of the OSDN forward (reverse mode through the token
recurrence).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module; the product path (the HIP library and its Python binding) never does.

The forward is the token step of the OSDN technical summary, section 2.1 (the delta write with
the write-side key scaled, k~_t = d_t (.) k_t), with the gated-delta decay of Erase-then-Delta
Attention, section 2.2, eq. 4, in the storage convention M = S^T (dk x dv):

    Mh_t = alpha_t M_{t-1}                   decayed old state
    y_t  = Mh_t^T k_t                        what the old state recalls for k_t
    u_t  = beta_t (v_t - y_t)                the write's residual
    M_t  = Mh_t + k~_t u_t^T                 the write
    o_t  = M_t^T q_t                         read-out after the write

The pages give no backward pass; this module is reverse-mode differentiation of those five
lines, taken in reverse order for t = T..1, for a scalar loss L whose gradients with respect to
the outputs are given: do_t = dL/do_t and dS_T = dL/dM_T (zero when absent).  Every line below
is the chain rule applied to one of the lines above:

    dM_t  += q_t do_t^T ;           dq_t  = M_t do_t                       (read-out)
    dk~_t  = dM_t u_t ;             du_t  = dM_t^T k~_t ;  dMh = dM_t      (write)
    dbeta_t = <du_t, v_t - y_t> ;   dv_t  = beta_t du_t ;  dy = -beta_t du_t   (residual)
    dMh   += k_t dy^T ;             dk_t  = Mh_t dy                        (recall)
    dd_t   = dk~_t (.) k_t ;        dk_t += dk~_t (.) d_t                  (write key)
    dalpha_t = <dMh, M_{t-1}>_F ;   dM_{t-1} = alpha_t dMh                 (decay)

and dS0 = dM_0.  With the channel-wise gate of Erase-then-Delta Attention, section 2.2, eq. 5
(a_t in [0,1]^dk scaling the rows of M, the key features), the decay line is
Mh_t = alpha_t Diag(a_t) M_{t-1}, and its reverse is

    da_t[f] = alpha_t <dMh[f,:], M_{t-1}[f,:]> ;  dalpha_t = <dMh, Diag(a_t) M_{t-1}>_F ;
    dM_{t-1} = alpha_t Diag(a_t) dMh .

Everything is float64 and vectorised over (batch, head) only.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def _decay(alpha, alpha_ch, t):
    """The factor the state before token t is multiplied by, broadcast over [B,H,dk,dv]."""
    a = 1.0 if alpha is None else alpha[:, :, t, None, None]
    if alpha_ch is not None:
        a = a * alpha_ch[:, :, t, :, None]
    return a


def forward_states(q, k, v, beta, d, alpha=None, S0=None, alpha_ch=None):
    """The token recurrence above, keeping what the reverse pass needs.

    Returns dict with o [B,H,T,dv], S_T [B,H,dk,dv], and per token the state before the step
    (Mprev [B,H,T,dk,dv]), y and u [B,H,T,dv]; the decayed state is
    alpha_t Diag(a_t) Mprev_t."""
    q, k, v, beta, d, alpha, S0, alpha_ch = map(_f64, (q, k, v, beta, d, alpha, S0, alpha_ch))
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    M = np.zeros((B, H, dk, dv)) if S0 is None else S0.copy()
    o = np.empty((B, H, T, dv))
    Mprev = np.empty((B, H, T, dk, dv))
    ys = np.empty((B, H, T, dv))
    us = np.empty((B, H, T, dv))
    for t in range(T):
        Mprev[:, :, t] = M
        Mh = _decay(alpha, alpha_ch, t) * M
        kt = k[:, :, t]
        y = np.einsum("bhkv,bhk->bhv", Mh, kt)
        u = beta[:, :, t, None] * (v[:, :, t] - y)
        kw = d[:, :, t] * kt
        M = Mh + kw[..., :, None] * u[..., None, :]
        o[:, :, t] = np.einsum("bhkv,bhk->bhv", M, q[:, :, t])
        ys[:, :, t] = y
        us[:, :, t] = u
    return dict(o=o, S_T=M, Mprev=Mprev, y=ys, u=us)


def chunk_bwd(q, k, v, beta, d, alpha=None, S0=None, do=None, dS_T=None,
              alpha_ch=None) -> Dict[str, np.ndarray]:
    """Gradients of L with respect to every input of the forward.

    q, k, d [B,H,T,dk]; v [B,H,T,dv]; beta [B,H,T]; alpha [B,H,T] or None (no decay); S0
    [B,H,dk,dv] or None (zero state); do [B,H,T,dv] (dL/do; zero if None); dS_T [B,H,dk,dv]
    (dL/dS_T; zero if None); alpha_ch [B,H,T,dk] or None (no channel-wise gate).  Returns dq,
    dk, dv, dbeta, dd, dalpha (None without decay), dalpha_ch (None without the channel-wise
    gate) and dS0 (the gradient with respect to the initial state, whether or not S0 was
    given)."""
    q, k, v, beta, d, alpha, S0, do, dS_T, alpha_ch = map(
        _f64, (q, k, v, beta, d, alpha, S0, do, dS_T, alpha_ch))
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    f = forward_states(q, k, v, beta, d, alpha, S0, alpha_ch)
    if do is None:
        do = np.zeros((B, H, T, dv))
    dM = np.zeros((B, H, dk, dv)) if dS_T is None else dS_T.copy()
    g = {name: np.zeros_like(x) for name, x in (("dq", q), ("dk", k), ("dv", v),
                                                 ("dbeta", beta), ("dd", d))}
    g["dalpha"] = None if alpha is None else np.zeros_like(alpha)
    g["dalpha_ch"] = None if alpha_ch is None else np.zeros_like(alpha_ch)
    for t in range(T - 1, -1, -1):
        kt, qt, dot = k[:, :, t], q[:, :, t], do[:, :, t]
        kw = d[:, :, t] * kt
        u, y = f["u"][:, :, t], f["y"][:, :, t]
        Mh = f["Mprev"][:, :, t] * _decay(alpha, alpha_ch, t)
        Mt = Mh + kw[..., :, None] * u[..., None, :]
        # read-out o_t = M_t^T q_t
        dM = dM + qt[..., :, None] * dot[..., None, :]
        g["dq"][:, :, t] = np.einsum("bhkv,bhv->bhk", Mt, dot)
        # write M_t = Mh_t + k~_t u_t^T
        dkw = np.einsum("bhkv,bhv->bhk", dM, u)
        du = np.einsum("bhkv,bhk->bhv", dM, kw)
        dMh = dM
        # residual u_t = beta_t (v_t - y_t)
        g["dbeta"][:, :, t] = np.sum(du * (v[:, :, t] - y), axis=-1)
        g["dv"][:, :, t] = beta[:, :, t, None] * du
        dy = -beta[:, :, t, None] * du
        # recall y_t = Mh_t^T k_t
        dMh = dMh + kt[..., :, None] * dy[..., None, :]
        dkt = np.einsum("bhkv,bhv->bhk", Mh, dy)
        # write key k~_t = d_t (.) k_t
        g["dd"][:, :, t] = dkw * kt
        g["dk"][:, :, t] = dkt + dkw * d[:, :, t]
        # decay Mh_t = alpha_t Diag(a_t) M_{t-1}
        Mp = f["Mprev"][:, :, t]
        if alpha is not None:
            ch = 1.0 if alpha_ch is None else alpha_ch[:, :, t, :, None]
            g["dalpha"][:, :, t] = np.einsum("bhkv,bhkv->bh", dMh, ch * Mp)
        if alpha_ch is not None:
            sc = 1.0 if alpha is None else alpha[:, :, t, None]
            g["dalpha_ch"][:, :, t] = sc * np.einsum("bhkv,bhkv->bhk", dMh, Mp)
        dM = _decay(alpha, alpha_ch, t) * dMh
    g["dS0"] = dM
    g["o"] = f["o"]
    g["S_T"] = f["S_T"]
    return g


def loss(o, S_T, do, dS_T) -> float:
    """The linear loss whose output gradients are (do, dS_T): sum(o * do) + sum(S_T * dS_T)."""
    val = float(np.sum(np.asarray(o, np.float64) * np.asarray(do, np.float64)))
    if dS_T is not None:
        val += float(np.sum(np.asarray(S_T, np.float64) * np.asarray(dS_T, np.float64)))
    return val
