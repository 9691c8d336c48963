"""The oracle's channel-wise gate against what the pages and the mathematics fix (CPU)."""
import numpy as np
import pytest

import oracle
from tests import kda_pins as pins


def oracle_impl(q, k, v, beta, d, a, S0):
    return oracle.chunk_fwd(q, k, v, beta, d, None, S0, nthreads=2, alpha_ch=a)


@pytest.mark.parametrize("name", sorted(pins.KDA_PINS))
def test_oracle_meets_pin(name):
    fn, tol = pins.KDA_PINS[name]
    err = fn(oracle_impl)
    assert err <= tol, f"{name}: {err:.3e} > {tol:.1e}"


def _mutant(kind):
    def impl(q, k, v, beta, d, a, S0):
        B, H, T, dk = q.shape
        dv = v.shape[-1]
        o = np.zeros((B, H, T, dv))
        S_T = np.zeros((B, H, dk, dv))
        for b in range(B):
            for h in range(H):
                M = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=float)
                for t in range(T):
                    at, kt, vt = a[b, h, t], k[b, h, t], v[b, h, t]
                    kw = d[b, h, t] * kt
                    old = M
                    if kind == "decay_on_values":
                        M = M * np.resize(at, dv)[None, :]
                    elif kind != "decay_after_write":
                        M = at[:, None] * M
                    r = vt - (old if kind == "residual_undecayed" else M).T @ kt
                    M = M + beta[b, h, t] * np.outer(kw, r)
                    if kind == "decay_after_write":
                        M = at[:, None] * M
                    o[b, h, t] = M.T @ q[b, h, t]
                S_T[b, h] = M
        return o, S_T
    return impl


MUTANTS = ["decay_on_values", "decay_after_write", "residual_undecayed"]


def test_mutant_harness_is_faithful():
    impl = _mutant("none")
    for name, (fn, tol) in pins.KDA_PINS.items():
        assert fn(impl) <= max(tol, 1e-12), name


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_reject_mutant(kind):
    impl = _mutant(kind)
    failed = [n for n, (fn, tol) in pins.KDA_PINS.items() if not fn(impl) <= max(tol, 1e-9)]
    assert failed, f"mutant {kind} passed every pin"


@pytest.mark.parametrize("gates", ["generator", "strong", "tiny", "mixed"])
def test_chunk_model_equals_recurrence(gates):
    """The chunk algebra with the gate folded into the operands by anchored products (every
    factor a product of gates, no reciprocal; the form the matrix-core path uses) against the
    recurrence, for gates from mild to 1e-30 (eq. 5 sets no lower bound on a_t)."""
    from oracle import chunkwise
    rng = np.random.default_rng(46)
    q, k, v, beta, d, a, S0 = pins.rand_kda(rng, 1, 2, 150, 8, 5)
    if gates == "strong":
        a = rng.uniform(0.05, 0.6, a.shape)
    elif gates == "tiny":
        a = rng.uniform(1e-30, 1e-20, a.shape)
    elif gates == "mixed":
        a = rng.uniform(0.5, 1.0, a.shape)
        a[rng.random(a.shape) < 0.1] = 1e-35
    o_ref, S_ref = oracle.chunk_fwd(q, k, v, beta, d, None, S0, alpha_ch=a)
    for chunk in (1, 16, 64, 150):
        o, S = chunkwise.chunk_fwd_channel(q, k, v, beta, d, a, S0, chunk=chunk)
        assert np.max(np.abs(o - o_ref)) <= 1e-10 * np.max(np.abs(o_ref))
        assert np.max(np.abs(S - S_ref)) <= 1e-10 * np.max(np.abs(S_ref))
