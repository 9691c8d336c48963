"""Pins for a CPU implementation of the gradients of the OSDN forward.

Each pin takes ``impl(q, k, v, beta, d, alpha, S0, do, dS_T) -> dict`` returning float64 arrays
dq, dk, dv, dbeta, dd, dalpha (None without decay), dS0 and the forward's o, S_T, and returns the
worst relative error it sees.  None of them restates the reverse pass:

* finite_diff   -- central differences of the loss L = <o, do> + <S_T, dS_T>, with the forward
                   evaluated by the C oracle (a separate implementation of the token step), for
                   every element of every input on a tiny problem;
* autograd      -- torch float64 autograd through an independent forward written as dense
                   matrices, S_t = alpha_t (I - b_t k~_t k_t^T) S_{t-1} + b_t k~_t v_t^T in the
                   dk x dv convention of Erase-then-Delta Attention, section 2.2, eq. 4, with the
                   write key scaled as in the OSDN summary, section 2.1;
* homog_q       -- o is linear in q, so sum <dq, q> = <do, o>;
* homog_vs      -- o and S_T are linear in (V, S0) jointly, so sum <dv, v> + <dS0, S0> = L;
* scale_inv     -- the forward depends on beta_t and d_t only through beta_t d_t (OSDN summary,
                   section 2.1), so for every token beta_t dbeta_t = <d_t, dd_t>.
"""
from __future__ import annotations

import numpy as np

import oracle
from oracle import backward
from tests.pins import _rand_inputs


def rand_bwd(rng, B, H, T, dk, dv, alpha=True, s0=True):
    q, k, v, beta, d, a, S0 = _rand_inputs(rng, B, H, T, dk, dv, alpha=alpha, s0=s0)
    do = rng.standard_normal((B, H, T, dv))
    dS_T = rng.standard_normal((B, H, dk, dv))
    return q, k, v, beta, d, a, S0, do, dS_T


def _rel(x, ref):
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    return float(np.max(np.abs(x - ref)) / max(float(np.max(np.abs(ref))), 1e-300))


def _c_loss(q, k, v, beta, d, a, S0, do, dS_T):
    o, S_T = oracle.chunk_fwd(q, k, v, beta, d, a, S0, nthreads=1)
    return backward.loss(o, S_T, do, dS_T)


def finite_diff(impl, seed=51, h=1e-6) -> float:
    rng = np.random.default_rng(seed)
    q, k, v, beta, d, a, S0, do, dS_T = rand_bwd(rng, 1, 2, 6, 3, 2)
    g = impl(q, k, v, beta, d, a, S0, do, dS_T)
    args = dict(q=q, k=k, v=v, beta=beta, d=d, a=a, S0=S0)
    names = dict(q="dq", k="dk", v="dv", beta="dbeta", d="dd", a="dalpha", S0="dS0")
    worst = 0.0
    for name, x in args.items():
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _c_loss(**args, do=do, dS_T=dS_T)
            x[idx] = old - h
            lm = _c_loss(**args, do=do, dS_T=dS_T)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        worst = max(worst, _rel(g[names[name]], fd))
    return worst


def _torch_forward(torch, q, k, v, beta, d, a, S0):
    """Dense-matrix forward in the dk x dv convention: S <- a (I - b k~ k^T) S + b k~ v^T."""
    B, H, T, dk = k.shape
    outs = []
    S = S0
    eye = torch.eye(dk, dtype=torch.float64)
    for t in range(T):
        kt, kw = k[:, :, t], d[:, :, t] * k[:, :, t]
        bt = beta[:, :, t, None, None]
        trans = eye - bt * kw[..., :, None] * kt[..., None, :]
        S = a[:, :, t, None, None] * (trans @ S) + bt * kw[..., :, None] * v[:, :, t, None, :]
        outs.append((S.transpose(-1, -2) @ q[:, :, t, :, None])[..., 0])
    return torch.stack(outs, dim=2), S


def autograd(impl, seed=52) -> float:
    import torch
    rng = np.random.default_rng(seed)
    q, k, v, beta, d, a, S0, do, dS_T = rand_bwd(rng, 2, 2, 30, 8, 5)
    g = impl(q, k, v, beta, d, a, S0, do, dS_T)
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, beta, d, a, S0)]
    o, S_T = _torch_forward(torch, *ts)
    L = (o * torch.tensor(do)).sum() + (S_T * torch.tensor(dS_T)).sum()
    grads = torch.autograd.grad(L, ts)
    worst = 0.0
    for name, tg in zip(("dq", "dk", "dv", "dbeta", "dd", "dalpha", "dS0"), grads):
        worst = max(worst, _rel(g[name], tg.numpy()))
    return worst


def homog_q(impl, seed=53) -> float:
    rng = np.random.default_rng(seed)
    q, k, v, beta, d, a, S0, do, dS_T = rand_bwd(rng, 2, 3, 40, 6, 4)
    g = impl(q, k, v, beta, d, a, S0, do, dS_T)
    lhs = np.sum(g["dq"] * q)
    rhs = np.sum(g["o"] * do)
    return abs(lhs - rhs) / max(abs(rhs), 1e-300)


def homog_vs(impl, seed=54) -> float:
    rng = np.random.default_rng(seed)
    q, k, v, beta, d, a, S0, do, dS_T = rand_bwd(rng, 2, 3, 40, 6, 4)
    g = impl(q, k, v, beta, d, a, S0, do, dS_T)
    lhs = np.sum(g["dv"] * v) + np.sum(g["dS0"] * S0)
    rhs = backward.loss(g["o"], g["S_T"], do, dS_T)
    return abs(lhs - rhs) / max(abs(rhs), 1e-300)


def scale_inv(impl, seed=55) -> float:
    rng = np.random.default_rng(seed)
    q, k, v, beta, d, a, S0, do, dS_T = rand_bwd(rng, 2, 2, 40, 6, 4)
    g = impl(q, k, v, beta, d, a, S0, do, dS_T)
    lhs = beta * g["dbeta"]
    rhs = np.sum(d * g["dd"], axis=-1)
    return float(np.max(np.abs(lhs - rhs)) / max(float(np.max(np.abs(rhs))), 1e-300))


# name -> (pin, tolerance); the tolerances sit far above float64 rounding and far below what
# a wrong term gives
BWD_PINS = {
    "finite_diff": (finite_diff, 1e-6),
    "autograd": (autograd, 1e-10),
    "homog_q": (homog_q, 1e-10),
    "homog_vs": (homog_vs, 1e-10),
    "scale_inv": (scale_inv, 1e-10),
}


# ---- the channel-wise gate ---------------------------------------------------------------------
# Pins for ``impl(q, k, v, beta, d, a, S0, do, dS_T) -> dict`` where ``a`` is the channel-wise gate
# [B,H,T,dk] (no scalar decay); the dict holds dalpha_ch in place of dalpha.  As above, none of
# them restates a reverse pass: finite differences of the C oracle's forward, torch autograd
# through the dense form of Erase-then-Delta Attention, section 2.2, eq. 5 (with the write key
# scaled), the same linear identities, and the reduction of equal channel factors to the scalar
# gate (the gradient of a common factor is the sum of the per-channel gradients).

def rand_bwd_kda(rng, B, H, T, dk, dv, lo=None):
    q, k, v, beta, d, _, S0 = _rand_inputs(rng, B, H, T, dk, dv, alpha=False, s0=True)
    if lo is None:
        a = np.exp(-0.2 * np.logaddexp(0, rng.standard_normal((B, H, T, dk))))
    else:
        a = rng.uniform(lo, 1.0, (B, H, T, dk))
    do = rng.standard_normal((B, H, T, dv))
    dS_T = rng.standard_normal((B, H, dk, dv))
    return q, k, v, beta, d, a, S0, do, dS_T


def _c_loss_kda(q, k, v, beta, d, a, S0, do, dS_T):
    o, S_T = oracle.chunk_fwd(q, k, v, beta, d, None, S0, nthreads=1, alpha_ch=a)
    return backward.loss(o, S_T, do, dS_T)


def kda_finite_diff(impl, seed=61, h=1e-6) -> float:
    rng = np.random.default_rng(seed)
    q, k, v, beta, d, a, S0, do, dS_T = rand_bwd_kda(rng, 1, 2, 6, 3, 2, lo=0.05)
    g = impl(q, k, v, beta, d, a, S0, do, dS_T)
    args = dict(q=q, k=k, v=v, beta=beta, d=d, a=a, S0=S0)
    names = dict(q="dq", k="dk", v="dv", beta="dbeta", d="dd", a="dalpha_ch", S0="dS0")
    worst = 0.0
    for name, x in args.items():
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _c_loss_kda(**args, do=do, dS_T=dS_T)
            x[idx] = old - h
            lm = _c_loss_kda(**args, do=do, dS_T=dS_T)
            x[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        worst = max(worst, _rel(g[names[name]], fd))
    return worst


def _torch_forward_kda(torch, q, k, v, beta, d, a, S0):
    """Dense-matrix forward in the dk x dv convention: S <- (I - b k~ k^T) Diag(a) S + b k~ v^T."""
    B, H, T, dk = k.shape
    outs = []
    S = S0
    eye = torch.eye(dk, dtype=torch.float64)
    for t in range(T):
        kt, kw = k[:, :, t], d[:, :, t] * k[:, :, t]
        bt = beta[:, :, t, None, None]
        trans = eye - bt * kw[..., :, None] * kt[..., None, :]
        S = trans @ (a[:, :, t, :, None] * S) + bt * kw[..., :, None] * v[:, :, t, None, :]
        outs.append((S.transpose(-1, -2) @ q[:, :, t, :, None])[..., 0])
    return torch.stack(outs, dim=2), S


def kda_autograd(impl, seed=62) -> float:
    import torch
    rng = np.random.default_rng(seed)
    q, k, v, beta, d, a, S0, do, dS_T = rand_bwd_kda(rng, 2, 2, 30, 8, 5, lo=0.02)
    g = impl(q, k, v, beta, d, a, S0, do, dS_T)
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, beta, d, a, S0)]
    o, S_T = _torch_forward_kda(torch, *ts)
    L = (o * torch.tensor(do)).sum() + (S_T * torch.tensor(dS_T)).sum()
    grads = torch.autograd.grad(L, ts)
    worst = 0.0
    for name, tg in zip(("dq", "dk", "dv", "dbeta", "dd", "dalpha_ch", "dS0"), grads):
        worst = max(worst, _rel(g[name], tg.numpy()))
    return worst


def kda_identities(impl, seed=63) -> float:
    """sum <dq, q> = <do, o>;  sum <dv, v> + <dS0, S0> = L;  beta_t dbeta_t = <d_t, dd_t>."""
    rng = np.random.default_rng(seed)
    q, k, v, beta, d, a, S0, do, dS_T = rand_bwd_kda(rng, 2, 3, 40, 6, 4)
    g = impl(q, k, v, beta, d, a, S0, do, dS_T)
    L = backward.loss(g["o"], g["S_T"], do, dS_T)
    e1 = abs(np.sum(g["dq"] * q) - np.sum(g["o"] * do)) / abs(np.sum(g["o"] * do))
    e2 = abs(np.sum(g["dv"] * v) + np.sum(g["dS0"] * S0) - L) / abs(L)
    rhs = np.sum(d * g["dd"], axis=-1)
    e3 = float(np.max(np.abs(beta * g["dbeta"] - rhs)) / np.max(np.abs(rhs)))
    return max(e1, e2, e3)


def kda_uniform(impl, seed=64) -> float:
    """Equal factors a_t = alpha_t on every channel: the forward is the scalar-gate one, and the
    scalar gate's gradient (from the finite differences of the C oracle with the scalar gate)
    is the sum over channels of the per-channel gradients."""
    rng = np.random.default_rng(seed)
    q, k, v, beta, d, a, S0, do, dS_T = rand_bwd_kda(rng, 1, 2, 5, 3, 2)
    al = a[..., 0].copy()
    a = np.repeat(al[..., None], k.shape[-1], axis=-1)
    g = impl(q, k, v, beta, d, a, S0, do, dS_T)
    h = 1e-6
    fd = np.zeros_like(al)
    for idx in np.ndindex(*al.shape):
        old = al[idx]
        al[idx] = old + h
        lp = _c_loss(q, k, v, beta, d, al, S0, do, dS_T)
        al[idx] = old - h
        lm = _c_loss(q, k, v, beta, d, al, S0, do, dS_T)
        al[idx] = old
        fd[idx] = (lp - lm) / (2 * h)
    return _rel(np.sum(g["dalpha_ch"], axis=-1), fd)


KDA_BWD_PINS = {
    "kda_finite_diff": (kda_finite_diff, 1e-6),
    "kda_autograd": (kda_autograd, 1e-10),
    "kda_identities": (kda_identities, 1e-10),
    "kda_uniform": (kda_uniform, 1e-6),
}
