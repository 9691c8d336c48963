"""Pins for a CPU implementation of the OSDN recurrence with the channel-wise gate.

Each pin takes ``impl(q, k, v, beta, d, alpha_ch, S0) -> (o, S_T)`` (float64 numpy arrays in
the [B,H,T,.] layout, alpha_ch [B,H,T,dk], state stored as M = S^T [B,H,dk,dv]) and returns the
worst error it sees.  From the pages and the mathematics, not from the implementation:

* eq5_d1       -- with d = 1 the recurrence is the channel-wise gated delta rule
                  S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T, o_t = S_t^T q_t
                  (Erase-then-Delta Attention, section 2.2, eq. 5; section 3.2, eq. 7),
                  written here as dense matrices in that page's dk x dv convention;
* eq5_scaled   -- with a general d the same matrix form with the write key scaled to
                  k~ = d (.) k (OSDN summary, section 2.1): S_t = (I - b k~ k^T) Diag(a) S + b k~ v^T;
* uniform      -- equal factors on every channel give the scalar gate of eq. 4;
* newton       -- when b_t <d_t, k_t^2> = 1 the write recovers S_t^T k_t = v_t whatever the
                  channel decay (OSDN summary, section 3);
* one_channel  -- a gate that zeroes one key channel at token t removes exactly that row of
                  the state before the write.
"""
from __future__ import annotations

import numpy as np

from tests.pins import _rand_inputs, _rel


def rand_kda(rng, B, H, T, dk, dv, s0=True):
    q, k, v, beta, d, _, S0 = _rand_inputs(rng, B, H, T, dk, dv, alpha=False, s0=s0)
    a = np.exp(-0.2 * np.logaddexp(0, rng.standard_normal((B, H, T, dk))))
    return q, k, v, beta, d, a, S0


def _dense(q, k, v, beta, d, a, S0, b, h):
    T, dk = k.shape[2], k.shape[3]
    dv = v.shape[3]
    S = np.zeros((dk, dv)) if S0 is None else S0[b, h].copy()
    o = np.zeros((T, dv))
    for t in range(T):
        kt, kw = k[b, h, t], d[b, h, t] * k[b, h, t]
        S = (np.eye(dk) - beta[b, h, t] * np.outer(kw, kt)) @ np.diag(a[b, h, t]) @ S \
            + beta[b, h, t] * np.outer(kw, v[b, h, t])
        o[t] = S.T @ q[b, h, t]
    return o, S


def eq5_d1(impl, seed=41) -> float:
    rng = np.random.default_rng(seed)
    q, k, v, beta, _, a, S0 = rand_kda(rng, 1, 2, 30, 5, 4)
    d = np.ones_like(k)
    o, S_T = impl(q, k, v, beta, d, a, S0)
    worst = 0.0
    for h in range(2):
        o_ref, S_ref = _dense(q, k, v, beta, d, a, S0, 0, h)
        worst = max(worst, _rel(o[0, h], o_ref), _rel(S_T[0, h], S_ref))
    return worst


def eq5_scaled(impl, seed=42) -> float:
    rng = np.random.default_rng(seed)
    q, k, v, beta, d, a, S0 = rand_kda(rng, 2, 1, 25, 6, 3)
    o, S_T = impl(q, k, v, beta, d, a, S0)
    worst = 0.0
    for b in range(2):
        o_ref, S_ref = _dense(q, k, v, beta, d, a, S0, b, 0)
        worst = max(worst, _rel(o[b, 0], o_ref), _rel(S_T[b, 0], S_ref))
    return worst


def uniform(impl, seed=43) -> float:
    """Equal channel factors: the scalar-gate recurrence of eq. 4 with the scaled write key,
    written out here token by token in the page's dk x dv convention."""
    rng = np.random.default_rng(seed)
    q, k, v, beta, d, a, S0 = rand_kda(rng, 1, 2, 20, 4, 5)
    a = np.repeat(a[..., :1], 4, axis=-1)
    o, S_T = impl(q, k, v, beta, d, a, S0)
    worst = 0.0
    for h in range(2):
        S = S0[0, h].copy()
        for t in range(20):
            at, kt, kw = a[0, h, t, 0], k[0, h, t], d[0, h, t] * k[0, h, t]
            S = at * S + beta[0, h, t] * np.outer(kw, v[0, h, t] - at * S.T @ kt)
            worst = max(worst, _rel(o[0, h, t], S.T @ q[0, h, t]))
        worst = max(worst, _rel(S_T[0, h], S))
    return worst


def newton(impl, seed=44) -> float:
    rng = np.random.default_rng(seed)
    q, k, v, beta, u, a, S0 = rand_kda(rng, 1, 2, 10, 6, 4)
    d = (1.0 / (beta * np.sum(u * k * k, axis=-1)))[..., None] * u
    worst = 0.0
    S = S0
    for t in range(10):
        sl = slice(t, t + 1)
        _, S = impl(q[:, :, sl], k[:, :, sl], v[:, :, sl], beta[:, :, sl], d[:, :, sl],
                    a[:, :, sl], S)
        recalled = np.einsum("bhij,bhi->bhj", S, k[:, :, t])
        worst = max(worst, _rel(recalled, v[:, :, t]))
    return worst


def one_channel(impl, seed=45) -> float:
    rng = np.random.default_rng(seed)
    q, k, v, beta, d, a, S0 = rand_kda(rng, 1, 1, 1, 5, 3)
    a[:] = 1.0
    a[0, 0, 0, 2] = 0.0
    k[0, 0, 0, 2] = 0.0  # the write then leaves row 2 alone too
    _, S_T = impl(q, k, v, beta, d, a, S0)
    return float(np.max(np.abs(S_T[0, 0, 2])))


KDA_PINS = {
    "eq5_d1": (eq5_d1, 1e-12),
    "eq5_scaled": (eq5_scaled, 1e-12),
    "uniform": (uniform, 1e-12),
    "newton": (newton, 1e-12),
    "one_channel": (one_channel, 0.0),
}
