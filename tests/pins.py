"""Pins for a CPU implementation of the OSDN recurrence.

Each pin takes an implementation ``impl(q, k, v, beta, d, alpha, S0) -> (o, S_T)`` (float64
numpy arrays in the [B,H,T,.] layout, state stored as M = S^T [B,H,dk,dv]) and returns the
worst error it sees.  The pins come from what the pages and the mathematics fix, never from
the implementation under test:

* hand_example     -- the two-token example worked by hand (tests/golden);
* deltanet_d1      -- with d = 1 and no decay the write is DeltaNet's (OSDN summary, section 1),
                      written here in the page's own dv x dk convention;
* gdn_d1           -- with d = 1 and a decay, the gated-delta matrix form
                      S_t = a_t (I - b_t k_t k_t^T) S_{t-1} + b_t k_t v_t^T, o_t = S_t^T q_t
                      (Erase-then-Delta Attention, section 2.2, eq. 4);
* newton           -- when b_t <d_t, k_t^2> = 1 the write recovers S_t k_t = v_t exactly
                      (OSDN summary, section 3, gated Newton condition);
* residual_ratio   -- per token, v - S_t k = (1 - b<d,k^2>)(v - a S_{t-1} k), which at a = 1 is
                      the closed-form hypergradient surrogate of the OSDN summary, section 2.2;
* scale_invariance -- only the product b_t d_t enters the write (OSDN summary, section 2.1);
* linearity        -- o and S_T are linear in (V, S0) and separable over value columns;
* split            -- running T1 then T2 from S_T(T1) equals running T1 + T2;
* product_form     -- brute force with dense transition matrices on tiny inputs.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand_inputs(rng, B, H, T, dk, dv, alpha=True, s0=True):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T))))
    d = np.exp(0.5 * rng.standard_normal((B, H, T, dk)))
    a = np.exp(-0.2 * np.logaddexp(0, rng.standard_normal((B, H, T)))) if alpha else None
    S0 = 0.3 * rng.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, beta, d, a, S0


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def hand_example(impl) -> float:
    with open(os.path.join(GOLDEN, "hand_example_2tok.json")) as f:
        g = json.load(f)
    tok = g["tokens"]
    arr = lambda x: np.asarray(x, dtype=np.float64)[None, None]
    q, k, v, d = (arr(tok[n]) for n in ("q", "k", "v", "d"))
    beta = arr(tok["beta"])
    worst = 0.0
    for case in g["cases"]:
        alpha = arr(case["alpha"])
        o, S_T = impl(q, k, v, beta, d, alpha, None)
        worst = max(worst, float(np.max(np.abs(o[0, 0] - np.asarray(case["o"])))),
                    float(np.max(np.abs(S_T[0, 0] - np.asarray(case["M_T"])))))
    return worst


def deltanet_d1(impl, seed=1) -> float:
    rng = np.random.default_rng(seed)
    q, k, v, beta, _, _, _ = _rand_inputs(rng, 1, 2, 40, 5, 3, alpha=False, s0=False)
    d = np.ones_like(k)
    o, S_T = impl(q, k, v, beta, d, None, None)
    worst = 0.0
    for h in range(2):
        S = np.zeros((3, 5))  # dv x dk, as on the OSDN page
        o_ref = np.zeros((40, 3))
        for t in range(40):
            S = S + beta[0, h, t] * np.outer(v[0, h, t] - S @ k[0, h, t], k[0, h, t])
            o_ref[t] = S @ q[0, h, t]
        worst = max(worst, _rel(o[0, h], o_ref), _rel(S_T[0, h], S.T))
    return worst


def gdn_d1(impl, seed=2) -> float:
    rng = np.random.default_rng(seed)
    q, k, v, beta, _, a, S0 = _rand_inputs(rng, 1, 2, 40, 4, 6)
    d = np.ones_like(k)
    o, S_T = impl(q, k, v, beta, d, a, S0)
    worst = 0.0
    for h in range(2):
        S = S0[0, h].copy()  # dk x dv, as in the gated-delta equation
        o_ref = np.zeros((40, 6))
        I = np.eye(4)
        for t in range(40):
            kt = k[0, h, t]
            S = a[0, h, t] * (I - beta[0, h, t] * np.outer(kt, kt)) @ S \
                + beta[0, h, t] * np.outer(kt, v[0, h, t])
            o_ref[t] = S.T @ q[0, h, t]
        worst = max(worst, _rel(o[0, h], o_ref), _rel(S_T[0, h], S))
    return worst


def _stepwise_states(impl, q, k, v, beta, d, a, S0):
    """States after every token, obtained by chaining one-token calls."""
    B, H, T, dk = q.shape
    S = S0
    states = []
    for t in range(T):
        sl = slice(t, t + 1)
        _, S = impl(q[:, :, sl], k[:, :, sl], v[:, :, sl], beta[:, :, sl], d[:, :, sl],
                    None if a is None else a[:, :, sl], S)
        states.append(S)
    return states


def newton(impl, seed=3) -> float:
    rng = np.random.default_rng(seed)
    q, k, v, beta, u, a, S0 = _rand_inputs(rng, 1, 2, 12, 6, 4)
    c = 1.0 / (beta * np.sum(u * k * k, axis=-1))
    d = c[..., None] * u
    states = _stepwise_states(impl, q, k, v, beta, d, a, S0)
    worst = 0.0
    for t, S in enumerate(states):
        recalled = np.einsum("bhij,bhi->bhj", S, k[:, :, t])
        worst = max(worst, _rel(recalled, v[:, :, t]))
    return worst


def residual_ratio(impl, seed=4) -> float:
    rng = np.random.default_rng(seed)
    q, k, v, beta, d, a, S0 = _rand_inputs(rng, 1, 2, 12, 6, 4)
    states = _stepwise_states(impl, q, k, v, beta, d, a, S0)
    worst = 0.0
    prev = S0
    for t, S in enumerate(states):
        kt, vt = k[:, :, t], v[:, :, t]
        after = vt - np.einsum("bhij,bhi->bhj", S, kt)
        before = vt - a[:, :, t, None] * np.einsum("bhij,bhi->bhj", prev, kt)
        lam = 1.0 - beta[:, :, t] * np.sum(d[:, :, t] * kt * kt, axis=-1)
        worst = max(worst, _rel(after, lam[..., None] * before))
        prev = S
    # the closed-form surrogate at a = 1: (f(S_t) - f(S_{t-1})) / ||grad f(S_{t-1})||_F^2
    ones = np.ones_like(a)
    states = _stepwise_states(impl, q, k, v, beta, d, ones, S0)
    prev = S0
    for t, S in enumerate(states):
        kt, vt = k[:, :, t], v[:, :, t]
        r_prev = np.einsum("bhij,bhi->bhj", prev, kt) - vt
        r_new = np.einsum("bhij,bhi->bhj", S, kt) - vt
        f_prev = 0.5 * np.sum(r_prev ** 2, axis=-1)
        f_new = 0.5 * np.sum(r_new ** 2, axis=-1)
        grad2 = np.sum(r_prev ** 2, axis=-1) * np.sum(kt ** 2, axis=-1)
        h_obs = (f_new - f_prev) / grad2
        lam = 1.0 - beta[:, :, t] * np.sum(d[:, :, t] * kt * kt, axis=-1)
        h_closed = (lam ** 2 - 1.0) / (2.0 * np.sum(kt ** 2, axis=-1))
        worst = max(worst, _rel(h_obs, h_closed))
        prev = S
    return worst


def scale_invariance(impl, seed=5) -> float:
    rng = np.random.default_rng(seed)
    q, k, v, beta, d, a, S0 = _rand_inputs(rng, 2, 2, 30, 5, 4)
    c = np.exp(rng.standard_normal(beta.shape))
    o1, S1 = impl(q, k, v, beta, d, a, S0)
    o2, S2 = impl(q, k, v, beta * c, d / c[..., None], a, S0)
    return max(_rel(o2, o1), _rel(S2, S1))


def linearity(impl, seed=6) -> float:
    rng = np.random.default_rng(seed)
    q, k, v1, beta, d, a, S01 = _rand_inputs(rng, 1, 2, 30, 5, 4)
    v2 = rng.standard_normal(v1.shape)
    S02 = rng.standard_normal(S01.shape)
    x, y = 0.7, -1.3
    o1, s1 = impl(q, k, v1, beta, d, a, S01)
    o2, s2 = impl(q, k, v2, beta, d, a, S02)
    o3, s3 = impl(q, k, x * v1 + y * v2, beta, d, a, x * S01 + y * S02)
    worst = max(_rel(o3, x * o1 + y * o2), _rel(s3, x * s1 + y * s2))
    perm = np.array([2, 0, 3, 1])
    o4, s4 = impl(q, k, v1[..., perm], beta, d, a, S01[..., perm])
    return max(worst, _rel(o4, o1[..., perm]), _rel(s4, s1[..., perm]))


def split(impl, seed=7) -> float:
    rng = np.random.default_rng(seed)
    q, k, v, beta, d, a, S0 = _rand_inputs(rng, 1, 2, 37, 5, 4)
    o, S = impl(q, k, v, beta, d, a, S0)
    cut = 16
    first = lambda x: x[:, :, :cut]
    last = lambda x: x[:, :, cut:]
    oa, Sa = impl(*(first(x) for x in (q, k, v, beta, d, a)), S0)
    ob, Sb = impl(*(last(x) for x in (q, k, v, beta, d, a)), Sa)
    return max(float(np.max(np.abs(np.concatenate([oa, ob], axis=2) - o))),
               float(np.max(np.abs(Sb - S))))


def product_form(impl, seed=8) -> float:
    """Dense transitions: M_T = P_T..P_1 M0 + sum_t P_T..P_{t+1} b_t k~_t v_t^T,
    P_t = a_t (I - b_t k~_t k_t^T); o_t read from M_t."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (dk, dv, T) in [(1, 1, 3), (2, 3, 5), (4, 2, 8), (3, 4, 7)]:
        q, k, v, beta, d, a, S0 = _rand_inputs(rng, 1, 1, T, dk, dv)
        o, S_T = impl(q, k, v, beta, d, a, S0)
        kt = d[0, 0] * k[0, 0]
        P = [a[0, 0, t] * (np.eye(dk) - beta[0, 0, t] * np.outer(kt[t], k[0, 0, t]))
             for t in range(T)]
        for tt in range(1, T + 1):
            Mt = S0[0, 0].copy()
            for t in range(tt):
                Mt = P[t] @ Mt
            for t in range(tt):
                prod = np.eye(dk)
                for s in range(t + 1, tt):
                    prod = P[s] @ prod
                Mt = Mt + prod @ (beta[0, 0, t] * np.outer(kt[t], v[0, 0, t]))
            worst = max(worst, _rel(o[0, 0, tt - 1], Mt.T @ q[0, 0, tt - 1]))
            if tt == T:
                worst = max(worst, _rel(S_T[0, 0], Mt))
    return worst


# pin name -> (function, tolerance)
PINS = {
    "hand_example": (hand_example, 1e-12),
    "deltanet_d1": (deltanet_d1, 1e-12),
    "gdn_d1": (gdn_d1, 1e-12),
    "newton": (newton, 1e-12),
    "residual_ratio": (residual_ratio, 1e-10),
    "scale_invariance": (scale_invariance, 1e-12),
    "linearity": (linearity, 1e-12),
    "split": (split, 0.0),
    "product_form": (product_form, 1e-12),
}
