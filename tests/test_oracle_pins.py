"""The float64 oracle against what the pages and the mathematics fix (CPU only)."""
import numpy as np
import pytest

import oracle
from oracle import chunkwise
from tests import pins


def oracle_impl(q, k, v, beta, d, alpha, S0):
    return oracle.chunk_fwd(q, k, v, beta, d, alpha, S0, nthreads=2)


@pytest.mark.parametrize("name", sorted(pins.PINS))
def test_oracle_meets_pin(name):
    fn, tol = pins.PINS[name]
    err = fn(oracle_impl)
    assert err <= tol, f"{name}: {err:.3e} > {tol:.1e}"


# ---- the pins reject plausible mistakes ---------------------------------------------------
# Each mutant is the recurrence with one plausible slip (a wrong reading of the pages, a
# dropped term, a sign, a transposed operand).  Every one must fail at least one pin, which
# shows the pins constrain the oracle beyond its own say-so.

def _mutant(kind):
    def impl(q, k, v, beta, d, alpha, S0):
        B, H, T, dk = q.shape
        dv = v.shape[-1]
        o = np.zeros((B, H, T, dv))
        S_T = np.zeros((B, H, dk, dv))
        for b in range(B):
            for h in range(H):
                M = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=float)
                for t in range(T):
                    a = 1.0 if alpha is None else alpha[b, h, t]
                    kt, vt, qt, dt = k[b, h, t], v[b, h, t], q[b, h, t], d[b, h, t]
                    bt = beta[b, h, t]
                    if kind == "readout_before_write":
                        o[b, h, t] = (a * M).T @ qt
                    if kind == "residual_undecayed":
                        r = vt - M.T @ kt
                        M = a * M
                    elif kind == "decay_after_write":
                        r = vt - M.T @ kt
                    else:
                        M = a * M
                        r = vt - M.T @ kt
                    if kind == "d_on_read_side":
                        r = vt - M.T @ (dt * kt)
                        M = M + bt * np.outer(kt, r)
                    elif kind == "residual_sign":
                        M = M - bt * np.outer(dt * kt, r)
                    elif kind == "no_beta":
                        M = M + np.outer(dt * kt, r)
                    elif kind == "d_squared":
                        M = M + bt * np.outer(dt * dt * kt, r)
                    else:
                        M = M + bt * np.outer(dt * kt, r)
                    if kind == "decay_after_write":
                        M = a * M
                    if kind == "transposed_readout":
                        # the stored [dk][dv] buffer read as if it held S ([dv][dk])
                        o[b, h, t] = M.reshape(dv, dk) @ qt
                    elif kind != "readout_before_write":
                        o[b, h, t] = M.T @ qt
                S_T[b, h] = M
        return o, S_T
    return impl


MUTANTS = ["readout_before_write", "residual_undecayed", "decay_after_write",
           "d_on_read_side", "residual_sign", "no_beta", "d_squared", "transposed_readout"]


def test_reference_mutant_harness_is_faithful():
    """The unmutated numpy loop meets every pin (so mutant failures are due to the slip)."""
    impl = _mutant("none")
    for name, (fn, tol) in pins.PINS.items():
        assert fn(impl) <= max(tol, 1e-12), name


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_reject_mutant(kind):
    impl = _mutant(kind)
    failed = []
    for name, (fn, tol) in pins.PINS.items():
        try:
            err = fn(impl)
        except Exception:  # a mutant that cannot even run fails the pin
            err = np.inf
        if not err <= max(tol, 1e-9):
            failed.append(name)
    assert failed, f"mutant {kind} passed every pin"


# ---- chunk algebra against the recurrence -------------------------------------------------

def _inputs(seed, B=1, H=2, T=200, dk=16, dv=8, alpha=True, s0=True):
    rng = np.random.default_rng(seed)
    return pins._rand_inputs(rng, B, H, T, dk, dv, alpha=alpha, s0=s0)


@pytest.mark.parametrize("chunk", [1, 2, 16, 64, 200])
def test_chunkwise_model_equals_recurrence(chunk):
    q, k, v, beta, d, a, S0 = _inputs(11)
    o_ref, S_ref = oracle.chunk_fwd(q, k, v, beta, d, a, S0)
    o, S = chunkwise.chunk_fwd(q, k, v, beta, d, a, S0, chunk=chunk)
    assert pins._rel(o, o_ref) <= 1e-12
    assert pins._rel(S, S_ref) <= 1e-12


def test_chunkwise_model_rejects_transposed_gram():
    """The Gram matrix K K~^T (not K~ K^T) is the one that matches the recurrence when d != 1."""
    q, k, v, beta, d, a, S0 = _inputs(12, T=64)
    o_ref, _ = oracle.chunk_fwd(q, k, v, beta, d, a, S0)
    o_ok, _ = chunkwise.chunk_fwd(q, k, v, beta, d, a, S0, chunk=64)
    assert pins._rel(o_ok, o_ref) <= 1e-12
    # swap the roles of k and k~ in the Gram matrix only: A' = b e^{g_r-g_s} <k~_r, k_s>
    B, H, T, dk = q.shape
    g = np.cumsum(np.log(a), axis=-1)
    kt = d * k
    worst = 0.0
    for h in range(H):
        G = np.exp(g[0, h][:, None] - g[0, h][None, :])
        A_bad = np.tril(beta[0, h][:, None] * G * (kt[0, h] @ k[0, h].T), -1)
        rhs = beta[0, h][:, None] * (v[0, h] - np.exp(g[0, h])[:, None] * (k[0, h] @ S0[0, h]))
        U = np.linalg.solve(np.eye(T) + A_bad, rhs)
        P = np.tril((q[0, h] @ kt[0, h].T) * G)
        o_h = np.exp(g[0, h])[:, None] * (q[0, h] @ S0[0, h]) + P @ U
        worst = max(worst, pins._rel(o_h, o_ref[0, h]))
    assert worst > 1e-3


def test_whole_sequence_is_one_triangular_solve():
    """With one chunk covering the sequence, the pseudo-values solve one dense unit-lower
    system (numpy.linalg.solve), and the outputs follow from them."""
    q, k, v, beta, d, a, S0 = _inputs(13, T=48)
    o_ref, S_ref = oracle.chunk_fwd(q, k, v, beta, d, a, S0)
    for h in range(2):
        K, Kt, Q, V = k[0, h], d[0, h] * k[0, h], q[0, h], v[0, h]
        g = np.cumsum(np.log(a[0, h]))
        G = np.exp(g[:, None] - g[None, :])
        lhs = np.eye(48) + np.tril(beta[0, h][:, None] * G * (K @ Kt.T), -1)
        rhs = beta[0, h][:, None] * (V - np.exp(g)[:, None] * (K @ S0[0, h]))
        U = np.linalg.solve(lhs, rhs)
        o = np.exp(g)[:, None] * (Q @ S0[0, h]) + np.tril((Q @ Kt.T) * G) @ U
        M = np.exp(g[-1]) * S0[0, h] + (np.exp(g[-1] - g)[:, None] * Kt).T @ U
        assert pins._rel(o, o_ref[0, h]) <= 1e-12
        assert pins._rel(M, S_ref[0, h]) <= 1e-12


# ---- contract details of the oracle ---------------------------------------------------------

def test_alpha_none_equals_alpha_one():
    q, k, v, beta, d, a, S0 = _inputs(14, T=33)
    o1, s1 = oracle.chunk_fwd(q, k, v, beta, d, None, S0)
    o2, s2 = oracle.chunk_fwd(q, k, v, beta, d, np.ones_like(a), S0)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_zero_length_returns_initial_state():
    q, k, v, beta, d, a, S0 = _inputs(15, T=0)
    o, s = oracle.chunk_fwd(q, k, v, beta, d, a, S0)
    assert o.shape[2] == 0 and np.array_equal(s, S0)
    _, s = oracle.chunk_fwd(q, k, v, beta, d, a, None)
    assert not np.any(s)


def test_thread_count_does_not_change_results():
    q, k, v, beta, d, a, S0 = _inputs(16, B=3, H=3, T=40)
    o1, s1 = oracle.chunk_fwd(q, k, v, beta, d, a, S0, nthreads=1)
    o2, s2 = oracle.chunk_fwd(q, k, v, beta, d, a, S0, nthreads=5)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_step_is_one_token_of_the_recurrence():
    q, k, v, beta, d, a, S0 = _inputs(17, T=5)
    o, s = oracle.chunk_fwd(q, k, v, beta, d, a, S0)
    S = S0
    for t in range(5):
        ot, S = oracle.step(q[:, :, t], k[:, :, t], v[:, :, t], beta[:, :, t], d[:, :, t],
                            a[:, :, t], S)
        assert np.array_equal(ot, o[:, :, t])
    assert np.array_equal(S, s)
