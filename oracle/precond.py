"""Float64 CPU oracle for the Phase-1 preconditioner scan of OSDN.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module; the product path (the HIP library and its Python binding) never does.

What it computes (OSDN: Improving Delta Rule with Provable Online Preconditioning in Linear
Attention, technical summary):

* section 1 -- the per-token regression loss f_t(S) = 1/2 ||S k_t - v_t||^2;
* section 2.2 -- the diagonal preconditioner d_t is moved by online gradient descent on the
  hypergradient surrogate h_t(d) = (f_t(S_t) - f_t(S_{t-1})) / ||grad f_t(S_{t-1})||_F^2, whose
  closed form ((1 - b_t <d, k_t^2>)^2 - 1) / (2 ||k_t||^2) depends on k_t and b_t only.  Its
  gradient is  grad_d h_t(d) = -b_t (1 - b_t <d, k_t^2>) k_t^2 / ||k_t||^2 ;
  Phase 1 walks the keys in order, carrying only the dk-vector d, and emits every d_t;
* section 2.3 (APF) -- a per-token, per-head retention gate r_t multiplies the preconditioner
  state (and nothing else) before the gradient step.

So, per (batch, head) sequence, token by token:

    token t writes with d_t  (the value before its own update);
    d_{t+1} = r_t d_t - eta grad_d h_t(d_t)
            = r_t d_t + eta b_t (1 - b_t <d_t, k_t^2>) k_t^2 / ||k_t||^2 .

Readings where the pages leave a step open:

* sign -- the APF line prints "+ eta grad h"; section 2.2 calls the update gradient *descent*
  on h_t, so the step is taken against the gradient (with r_t = 1 it is plain OGD);
* the bar on d_{t+1} in the APF line names no projection set; none is applied;
* order -- h_t is evaluated at the d_t used in token t's own write (it measures that write),
  so the write of token t uses d_t and the update that consumes k_t produces d_{t+1};
* ||k_t|| = 0 leaves h_t undefined (0/0); that token takes no gradient step: d_{t+1} = r_t d_t;
* d_1 (the first token's preconditioner) and eta are inputs; d_1 = 1 (plain DeltaNet's
  write) when not given, and r = 1 (no APF) when not given.
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def surrogate(d, k, beta):
    """Closed-form hypergradient surrogate h_t(d) (technical summary, section 2.2)."""
    d, k = _f64(d), _f64(k)
    x = k * k
    n = np.sum(x, axis=-1)
    e = 1.0 - np.asarray(beta, dtype=np.float64) * np.sum(d * x, axis=-1)
    return (e * e - 1.0) / (2.0 * n)


def surrogate_grad(d, k, beta):
    """grad_d h_t(d) for a batch of tokens: d, k [..., dk]; beta [...]; 0 where ||k|| = 0."""
    d, k = _f64(d), _f64(k)
    beta = np.asarray(beta, dtype=np.float64)
    x = k * k
    n = np.sum(x, axis=-1)
    e = 1.0 - beta * np.sum(d * x, axis=-1)
    scale = np.divide(-beta * e, n, out=np.zeros_like(n), where=n > 0)
    return scale[..., None] * x


def precond_scan(k, beta, eta: float, r=None, d1=None) -> Tuple[np.ndarray, np.ndarray]:
    """Phase-1 scan over whole sequences.

    k [B,H,T,dk]; beta [B,H,T]; r [B,H,T] or None (no retention gate); d1 [B,H,dk] or None
    (ones).  Returns (d [B,H,T,dk] -- the d_t each token writes with, d_next [B,H,dk] -- the
    preconditioner after the last token), both float64.
    """
    k, beta, r, d1 = map(_f64, (k, beta, r, d1))
    B, H, T, dk = k.shape
    assert beta.shape == (B, H, T)
    assert r is None or r.shape == (B, H, T)
    assert d1 is None or d1.shape == (B, H, dk)
    d = np.ones((B, H, dk)) if d1 is None else d1.copy()
    out = np.empty((B, H, T, dk))
    for t in range(T):
        out[:, :, t] = d
        g = surrogate_grad(d, k[:, :, t], beta[:, :, t])
        keep = 1.0 if r is None else r[:, :, t, None]
        d = keep * d - eta * g
    return out, d


def precond_step(k, beta, eta: float, r, d) -> Tuple[np.ndarray, np.ndarray]:
    """One token for every (b,h): k [B,H,dk]; beta, r [B,H] (r may be None); d [B,H,dk].
    Returns (d_used [B,H,dk], d_next [B,H,dk])."""
    add_t = lambda x: None if x is None else np.asarray(x)[:, :, None]
    out, d_next = precond_scan(add_t(k), add_t(beta), eta, add_t(r), d)
    return out[:, :, 0], d_next
