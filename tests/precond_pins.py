"""Pins for a CPU implementation of the Phase-1 preconditioner scan.

Each pin takes ``impl(k, beta, eta, r, d1) -> (d, d_next)`` (float64 numpy arrays: k
[B,H,T,dk], beta and r [B,H,T], d1 [B,H,dk]; d [B,H,T,dk] holds the d_t each token writes
with, d_next [B,H,dk] the preconditioner after the last token) and returns the worst error it
sees.  The pins come from the pages and the mathematics, not from the implementation:

* hand_example   -- the two-token scan worked by hand (tests/golden);
* descent        -- the step equals -eta times a finite-difference gradient of h_t taken from
                    its *definition* (f_t(S_t) - f_t(S_{t-1})) / ||grad f_t(S_{t-1})||_F^2, with
                    f_t(S) = 1/2 ||S k_t - v_t||^2 and S_t the preconditioned write, on random
                    S_{t-1} and v_t (OSDN summary, sections 1, 2.1, 2.2, 2.3);
* newton         -- a token that already meets b_t <d_t, k_t^2> = 1 (the gated Newton
                    condition, OSDN summary, section 3) leaves d unchanged apart from r_t;
* contraction    -- with one key repeated, constant b and r = 1, the residual factor
                    e_t = 1 - b <d_t, k^2> shrinks by exactly 1 - eta b^2 ||k^2||^2 / ||k||^2 a token;
* eta_zero       -- with eta = 0 only the retention gate acts: d_t = (prod_{s<t} r_s) d_1;
* zero_key       -- a zero key takes no gradient step (h_t is 0/0 there): d_{t+1} = r_t d_t;
* split          -- running T1 tokens then T2 from d_next equals running T1 + T2;
* affine_form    -- brute force with dense per-token affine maps on tiny inputs.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rand_inputs(rng, B, H, T, dk, apf=True, d1=True, unit=True):
    """Keys L2-normalised per token (unit=True) or with a random norm around 1."""
    k = rng.standard_normal((B, H, T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    if not unit:
        k *= np.exp(0.5 * rng.standard_normal((B, H, T, 1)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T))))
    r = np.exp(-0.05 * np.logaddexp(0, rng.standard_normal((B, H, T)))) if apf else None
    d = np.exp(0.25 * rng.standard_normal((B, H, dk))) if d1 else None
    return k, beta, r, d


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def hand_example(impl) -> float:
    with open(os.path.join(GOLDEN, "precond_hand_2tok.json")) as f:
        g = json.load(f)
    arr = lambda x: np.asarray(x, dtype=np.float64)[None, None]
    k, beta = arr(g["tokens"]["k"]), arr(g["tokens"]["beta"])
    d1 = arr(g["d1"])
    worst = 0.0
    for case in g["cases"]:
        r = None if case["r"] is None else arr(case["r"])
        d, d_next = impl(k, beta, g["eta"], r, d1)
        worst = max(worst, float(np.max(np.abs(d[0, 0] - np.asarray(case["d"])))),
                    float(np.max(np.abs(d_next[0, 0] - np.asarray(case["d_next"])))))
    return worst


def _h_by_definition(d, k, v, beta, S_prev):
    """(f(S_t) - f(S_{t-1})) / ||grad f(S_{t-1})||_F^2 with S dv x dk as on the OSDN page."""
    f = lambda S: 0.5 * np.sum((S @ k - v) ** 2)
    S_t = S_prev + beta * np.outer(v - S_prev @ k, d * k)
    grad = np.outer(S_prev @ k - v, k)          # d f / d S at S_{t-1}
    return (f(S_t) - f(S_prev)) / np.sum(grad * grad)


def descent(impl, seed=21) -> float:
    rng = np.random.default_rng(seed)
    dk, dv, T, eta = 5, 3, 12, 0.7
    k, beta, r, d1 = rand_inputs(rng, 1, 2, T, dk, unit=False)
    d, d_next = impl(k, beta, eta, r, d1)
    seq = np.concatenate([d, d_next[:, :, None]], axis=2)
    worst = 0.0
    step = 1e-5
    for h in range(2):
        for t in range(T):
            S_prev = rng.standard_normal((dv, dk))
            v = rng.standard_normal(dv)
            dt, kt, bt = seq[0, h, t], k[0, h, t], beta[0, h, t]
            g = np.zeros(dk)
            for i in range(dk):
                e = np.zeros(dk)
                e[i] = step
                g[i] = (_h_by_definition(dt + e, kt, v, bt, S_prev)
                        - _h_by_definition(dt - e, kt, v, bt, S_prev)) / (2 * step)
            expect = r[0, h, t] * dt - eta * g
            worst = max(worst, _rel(seq[0, h, t + 1], expect))
    return worst


def newton(impl, seed=22) -> float:
    rng = np.random.default_rng(seed)
    k, beta, r, u = rand_inputs(rng, 2, 3, 1, 6)
    scale = 1.0 / (beta[:, :, 0] * np.sum(u * k[:, :, 0] ** 2, axis=-1))
    d1 = scale[..., None] * u
    d, d_next = impl(k, beta, 1.3, r, d1)
    return max(_rel(d[:, :, 0], d1), _rel(d_next, r[:, :, 0, None] * d1))


def contraction(impl, seed=23) -> float:
    rng = np.random.default_rng(seed)
    dk, T, eta, b = 7, 20, 0.9, 0.8
    kk = rng.standard_normal(dk)
    k = np.broadcast_to(kk, (1, 1, T, dk)).copy()
    beta = np.full((1, 1, T), b)
    d1 = np.exp(0.3 * rng.standard_normal((1, 1, dk)))
    d, d_next = impl(k, beta, eta, None, d1)
    x = kk * kk
    q = 1.0 - eta * b * b * np.sum(x * x) / np.sum(x)
    seq = np.concatenate([d[0, 0], d_next[0, 0][None]], axis=0)
    e = 1.0 - b * seq @ x
    expect = e[0] * q ** np.arange(T + 1)
    return _rel(e, expect)


def eta_zero(impl, seed=24) -> float:
    rng = np.random.default_rng(seed)
    k, beta, r, d1 = rand_inputs(rng, 2, 2, 9, 4)
    d, d_next = impl(k, beta, 0.0, r, d1)
    keep = np.concatenate([np.ones((2, 2, 1)), np.cumprod(r, axis=2)], axis=2)
    expect = keep[..., None] * d1[:, :, None, :]
    return max(_rel(d, expect[:, :, :-1]), _rel(d_next, expect[:, :, -1]))


def zero_key(impl, seed=25) -> float:
    rng = np.random.default_rng(seed)
    k, beta, r, d1 = rand_inputs(rng, 1, 2, 3, 4)
    k[:, :, 1] = 0.0
    d, d_next = impl(k, beta, 0.8, r, d1)
    return _rel(d[:, :, 2], r[:, :, 1, None] * d[:, :, 1])


def split(impl, seed=26) -> float:
    rng = np.random.default_rng(seed)
    k, beta, r, d1 = rand_inputs(rng, 1, 2, 23, 5)
    d, d_next = impl(k, beta, 0.6, r, d1)
    cut = 9
    da, na = impl(k[:, :, :cut], beta[:, :, :cut], 0.6, r[:, :, :cut], d1)
    db, nb = impl(k[:, :, cut:], beta[:, :, cut:], 0.6, r[:, :, cut:], na)
    return max(float(np.max(np.abs(np.concatenate([da, db], axis=2) - d))),
               float(np.max(np.abs(nb - d_next))))


def affine_form(impl, seed=27) -> float:
    """d_{t+1} = A_t d_t + c_t with A_t = r_t I - eta b_t^2 x_t x_t^T / n_t, c_t = eta b_t x_t / n_t
    (x = k^2, n = ||k||^2), composed as dense matrices."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (dk, T) in [(1, 3), (2, 5), (3, 6), (4, 8)]:
        k, beta, r, d1 = rand_inputs(rng, 1, 1, T, dk, unit=False)
        eta = 1.1
        d, d_next = impl(k, beta, eta, r, d1)
        x = k[0, 0] ** 2
        n = np.sum(x, axis=-1)
        A = [r[0, 0, t] * np.eye(dk) - eta * beta[0, 0, t] ** 2 * np.outer(x[t], x[t]) / n[t]
             for t in range(T)]
        c = [eta * beta[0, 0, t] * x[t] / n[t] for t in range(T)]
        for tt in range(T + 1):
            P = np.eye(dk)
            acc = np.zeros(dk)
            for t in range(tt):
                P = A[t] @ P
            for t in range(tt):
                prod = np.eye(dk)
                for s in range(t + 1, tt):
                    prod = A[s] @ prod
                acc = acc + prod @ c[t]
            dt = P @ d1[0, 0] + acc
            got = d[0, 0, tt] if tt < T else d_next[0, 0]
            worst = max(worst, _rel(got, dt))
    return worst


# pin name -> (function, tolerance)
PINS = {
    "hand_example": (hand_example, 1e-12),
    "descent": (descent, 1e-7),
    "newton": (newton, 1e-12),
    "contraction": (contraction, 1e-10),
    "eta_zero": (eta_zero, 1e-14),
    "zero_key": (zero_key, 1e-14),
    "split": (split, 0.0),
    "affine_form": (affine_form, 1e-12),
}
