"""The Phase-1 preconditioner oracle against what the pages and the mathematics fix (CPU)."""
import numpy as np
import pytest

from oracle import precond
from tests import precond_pins as pins


def oracle_impl(k, beta, eta, r, d1):
    return precond.precond_scan(k, beta, eta, r, d1)


@pytest.mark.parametrize("name", sorted(pins.PINS))
def test_oracle_meets_pin(name):
    fn, tol = pins.PINS[name]
    err = fn(oracle_impl)
    assert err <= tol, f"{name}: {err:.3e} > {tol:.1e}"


def test_closed_form_surrogate_matches_its_definition():
    """The closed form the summary prints for h_t (section 2.2) equals the definition built
    from f_t and the preconditioned write, on random states and values."""
    rng = np.random.default_rng(31)
    for _ in range(20):
        dk, dv = 6, 4
        k = rng.standard_normal(dk)
        d = np.exp(0.4 * rng.standard_normal(dk))
        beta = float(rng.uniform(0.05, 1.0))
        S_prev = rng.standard_normal((dv, dk))
        v = rng.standard_normal(dv)
        h_def = pins._h_by_definition(d, k, v, beta, S_prev)
        assert abs(precond.surrogate(d, k, beta) - h_def) <= 1e-12 * max(1.0, abs(h_def))


def test_step_is_one_token_of_the_scan():
    rng = np.random.default_rng(32)
    k, beta, r, d1 = pins.rand_inputs(rng, 2, 3, 5, 8)
    d, d_next = precond.precond_scan(k, beta, 0.9, r, d1)
    state = d1
    for t in range(5):
        used, state = precond.precond_step(k[:, :, t], beta[:, :, t], 0.9, r[:, :, t], state)
        assert np.array_equal(used, d[:, :, t])
    assert np.array_equal(state, d_next)


def test_defaults_are_ones_and_no_retention():
    rng = np.random.default_rng(33)
    k, beta, r, _ = pins.rand_inputs(rng, 1, 2, 6, 4)
    a = precond.precond_scan(k, beta, 0.5, None, None)
    b = precond.precond_scan(k, beta, 0.5, np.ones_like(r), np.ones((1, 2, 4)))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_zero_length_returns_initial_state():
    d1 = np.arange(8.0).reshape(1, 2, 4)
    d, d_next = precond.precond_scan(np.zeros((1, 2, 0, 4)), np.zeros((1, 2, 0)), 0.5, None, d1)
    assert d.shape == (1, 2, 0, 4) and np.array_equal(d_next, d1)


# ---- the pins reject plausible mistakes ---------------------------------------------------

def _mutant(kind):
    def impl(k, beta, eta, r, d1):
        B, H, T, dk = k.shape
        d = np.ones((B, H, dk)) if d1 is None else np.array(d1, dtype=float)
        out = np.empty((B, H, T, dk))
        for t in range(T):
            x = k[:, :, t] ** 2
            n = np.sum(x, axis=-1)
            if kind == "norm_not_squared":
                n = np.sqrt(n)
            elif kind == "no_normalisation":
                n = np.ones_like(n)
            bt = beta[:, :, t]
            e = 1.0 - (1.0 if kind == "beta_missing_in_residual" else bt) * np.sum(d * x, -1)
            xg = k[:, :, t] if kind == "key_not_squared" else x
            coef = np.divide(bt * e, n, out=np.zeros_like(n), where=n > 0)
            if kind == "beta_squared_in_step":
                coef = coef * bt
            g = coef[..., None] * xg                     # = -grad h
            rt = 1.0 if r is None else r[:, :, t, None]
            new = {"ascent": rt * d - eta * g,
                   "retention_on_step": rt * (d + eta * g)}.get(kind, rt * d + eta * g)
            out[:, :, t] = new if kind == "writes_with_updated_d" else d
            d = new
        return out, d
    return impl


MUTANTS = ["ascent", "retention_on_step", "norm_not_squared", "no_normalisation",
           "beta_missing_in_residual", "key_not_squared", "beta_squared_in_step",
           "writes_with_updated_d"]


def test_mutant_harness_is_faithful():
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
        except Exception:
            err = np.inf
        if not err <= max(tol, 1e-9):
            failed.append(name)
    assert failed, f"mutant {kind} passed every pin"


# ---- chunk algebra against the token scan -------------------------------------------------

@pytest.mark.parametrize("chunk", [1, 3, 16, 64, 100])
def test_chunk_model_equals_scan(chunk):
    from oracle import chunkwise
    rng = np.random.default_rng(34)
    k, beta, r, d1 = pins.rand_inputs(rng, 1, 2, 100, 12, unit=False)
    k[0, 1, 5] = 0.0                                  # a zero key inside a chunk
    d_ref, n_ref = precond.precond_scan(k, beta, 1.7, r, d1)
    d, n = chunkwise.precond_scan(k, beta, 1.7, r, d1, chunk=chunk)
    assert pins._rel(d, d_ref) <= 1e-12 and pins._rel(n, n_ref) <= 1e-12


def test_chunk_model_without_gate_or_start():
    from oracle import chunkwise
    rng = np.random.default_rng(35)
    k, beta, _, _ = pins.rand_inputs(rng, 2, 1, 70, 8)
    d_ref, n_ref = precond.precond_scan(k, beta, 0.8)
    d, n = chunkwise.precond_scan(k, beta, 0.8, chunk=32)
    assert pins._rel(d, d_ref) <= 1e-12 and pins._rel(n, n_ref) <= 1e-12
