"""The backward oracle against what the mathematics fixes (CPU): finite differences of the C
oracle's forward, torch autograd through an independent dense forward, and exact identities."""
import numpy as np
import pytest

import oracle
from oracle import backward
from tests import bwd_pins as pins


def oracle_impl(q, k, v, beta, d, a, S0, do, dS_T):
    return backward.chunk_bwd(q, k, v, beta, d, a, S0, do, dS_T)


@pytest.mark.parametrize("name", sorted(pins.BWD_PINS))
def test_oracle_meets_pin(name):
    fn, tol = pins.BWD_PINS[name]
    err = fn(oracle_impl)
    assert err <= tol, f"{name}: {err:.3e} > {tol:.1e}"


def test_forward_states_match_c_oracle():
    rng = np.random.default_rng(56)
    q, k, v, beta, d, a, S0, do, dS_T = pins.rand_bwd(rng, 2, 2, 33, 7, 5)
    g = backward.chunk_bwd(q, k, v, beta, d, a, S0, do, dS_T)
    o, S_T = oracle.chunk_fwd(q, k, v, beta, d, a, S0, nthreads=2)
    assert pins._rel(g["o"], o) < 1e-13 and pins._rel(g["S_T"], S_T) < 1e-13


def test_no_decay_equals_unit_decay():
    rng = np.random.default_rng(57)
    q, k, v, beta, d, a, S0, do, dS_T = pins.rand_bwd(rng, 1, 2, 20, 5, 4)
    g0 = backward.chunk_bwd(q, k, v, beta, d, None, S0, do, dS_T)
    g1 = backward.chunk_bwd(q, k, v, beta, d, np.ones_like(a), S0, do, dS_T)
    assert g0["dalpha"] is None
    for n in ("dq", "dk", "dv", "dbeta", "dd", "dS0"):
        assert np.array_equal(g0[n], g1[n]), n


def _mutant(kind):
    """The reverse pass with one planted mistake (kind == "none": faithful)."""
    def impl(q, k, v, beta, d, a, S0, do, dS_T):
        f = backward.forward_states(q, k, v, beta, d, a, S0)
        B, H, T, dk = k.shape
        dM = np.array(dS_T, dtype=np.float64)
        g = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dbeta", beta),
                                              ("dd", d), ("dalpha", a))}
        for t in range(T - 1, -1, -1):
            kt, qt, dot = k[:, :, t], q[:, :, t], do[:, :, t]
            kw = d[:, :, t] * kt
            u, y = f["u"][:, :, t], f["y"][:, :, t]
            Mh = a[:, :, t, None, None] * f["Mprev"][:, :, t]
            Mt = Mh + kw[..., :, None] * u[..., None, :]
            dM = dM + qt[..., :, None] * dot[..., None, :]
            Mread = f["Mprev"][:, :, t] if kind == "readout_before_write" else Mt
            g["dq"][:, :, t] = np.einsum("bhkv,bhv->bhk", Mread, dot)
            dkw = np.einsum("bhkv,bhv->bhk", dM, u)
            du = np.einsum("bhkv,bhk->bhv", dM, kt if kind == "du_plain_key" else kw)
            res = v[:, :, t] if kind == "dbeta_no_recall" else v[:, :, t] - y
            g["dbeta"][:, :, t] = np.sum(du * res, axis=-1)
            g["dv"][:, :, t] = beta[:, :, t, None] * du
            dy = (1.0 if kind == "dy_sign" else -1.0) * beta[:, :, t, None] * du
            dMh = dM + kt[..., :, None] * dy[..., None, :]
            dkt = np.einsum("bhkv,bhv->bhk", Mh, dy)
            g["dd"][:, :, t] = dkw * kt
            g["dk"][:, :, t] = dkt if kind == "dk_no_write_key" else dkt + dkw * d[:, :, t]
            g["dalpha"][:, :, t] = np.einsum("bhkv,bhkv->bh", dMh, f["Mprev"][:, :, t])
            dM = dMh if kind == "carry_undecayed" else a[:, :, t, None, None] * dMh
        g["dS0"] = dM
        g["o"], g["S_T"] = f["o"], f["S_T"]
        return g
    return impl


MUTANTS = ["readout_before_write", "du_plain_key", "dbeta_no_recall", "dy_sign",
           "dk_no_write_key", "carry_undecayed"]


def test_mutant_harness_is_faithful():
    impl = _mutant("none")
    for name, (fn, tol) in pins.BWD_PINS.items():
        assert fn(impl) <= tol, name


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_reject_mutant(kind):
    impl = _mutant(kind)
    failed = [n for n, (fn, tol) in pins.BWD_PINS.items() if not fn(impl) <= tol]
    assert len(failed) >= 2, f"mutant {kind} fails only {failed}"


@pytest.mark.parametrize("chunk", [1, 3, 16, 64, 150])
def test_chunk_model_equals_reverse_pass(chunk):
    """The chunk form of the backward (what the GPU kernels compute) against the token
    reverse pass, with and without decay and initial state."""
    from oracle import chunkwise
    rng = np.random.default_rng(58 + chunk)
    q, k, v, beta, d, a, S0, do, dS_T = pins.rand_bwd(rng, 2, 2, 130, 8, 5)
    for aa, ss, dst in ((a, S0, dS_T), (None, None, None)):
        ref = backward.chunk_bwd(q, k, v, beta, d, aa, ss, do, dst)
        got = chunkwise.chunk_bwd(q, k, v, beta, d, aa, ss, do, dst, chunk=chunk)
        for n in ("dq", "dk", "dv", "dbeta", "dd", "dS0") + (("dalpha",) if aa is not None else ()):
            assert pins._rel(got[n], ref[n]) < 1e-12, (n, chunk)


# ---- the channel-wise gate ---------------------------------------------------------------------

def oracle_impl_kda(q, k, v, beta, d, a, S0, do, dS_T):
    return backward.chunk_bwd(q, k, v, beta, d, None, S0, do, dS_T, alpha_ch=a)


@pytest.mark.parametrize("name", sorted(pins.KDA_BWD_PINS))
def test_oracle_meets_kda_pin(name):
    fn, tol = pins.KDA_BWD_PINS[name]
    err = fn(oracle_impl_kda)
    assert err <= tol, f"{name}: {err:.3e} > {tol:.1e}"


def test_kda_forward_states_match_c_oracle():
    rng = np.random.default_rng(65)
    q, k, v, beta, d, a, S0, do, dS_T = pins.rand_bwd_kda(rng, 2, 2, 33, 7, 5)
    g = backward.chunk_bwd(q, k, v, beta, d, None, S0, do, dS_T, alpha_ch=a)
    o, S_T = oracle.chunk_fwd(q, k, v, beta, d, None, S0, nthreads=2, alpha_ch=a)
    assert pins._rel(g["o"], o) < 1e-13 and pins._rel(g["S_T"], S_T) < 1e-13


def _kda_mutant(kind):
    """The reverse pass with the channel-wise gate and one planted mistake in its decay line."""
    def impl(q, k, v, beta, d, a, S0, do, dS_T):
        f = backward.forward_states(q, k, v, beta, d, None, S0, alpha_ch=a)
        B, H, T, dk = k.shape
        dM = np.array(dS_T, dtype=np.float64)
        g = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dbeta", beta),
                                              ("dd", d), ("dalpha_ch", a))}
        for t in range(T - 1, -1, -1):
            kt, qt, dot = k[:, :, t], q[:, :, t], do[:, :, t]
            kw = d[:, :, t] * kt
            u, y = f["u"][:, :, t], f["y"][:, :, t]
            Mp = f["Mprev"][:, :, t]
            Mh = a[:, :, t, :, None] * Mp
            Mt = Mh + kw[..., :, None] * u[..., None, :]
            dM = dM + qt[..., :, None] * dot[..., None, :]
            g["dq"][:, :, t] = np.einsum("bhkv,bhv->bhk", Mt, dot)
            dkw = np.einsum("bhkv,bhv->bhk", dM, u)
            du = np.einsum("bhkv,bhk->bhv", dM, kw)
            g["dbeta"][:, :, t] = np.sum(du * (v[:, :, t] - y), axis=-1)
            g["dv"][:, :, t] = beta[:, :, t, None] * du
            dy = -beta[:, :, t, None] * du
            dMh = dM + kt[..., :, None] * dy[..., None, :]
            g["dd"][:, :, t] = dkw * kt
            g["dk"][:, :, t] = np.einsum("bhkv,bhv->bhk", Mh, dy) + dkw * d[:, :, t]
            src = Mh if kind == "da_from_decayed" else Mp
            g["dalpha_ch"][:, :, t] = np.einsum("bhkv,bhkv->bhk", dMh, src)
            if kind == "da_before_recall":
                g["dalpha_ch"][:, :, t] = np.einsum("bhkv,bhkv->bhk", dM, Mp)
            dM = dMh if kind == "carry_undecayed" else a[:, :, t, :, None] * dMh
        g["dS0"] = dM
        g["o"], g["S_T"] = f["o"], f["S_T"]
        return g
    return impl


KDA_MUTANTS = ["da_from_decayed", "da_before_recall", "carry_undecayed"]


def test_kda_mutant_harness_is_faithful():
    impl = _kda_mutant("none")
    for name in ("kda_autograd", "kda_identities"):
        fn, tol = pins.KDA_BWD_PINS[name]
        assert fn(impl) <= tol, name


@pytest.mark.parametrize("kind", KDA_MUTANTS)
def test_kda_pins_catch_mutant(kind):
    impl = _kda_mutant(kind)
    failed = [n for n in ("kda_autograd", "kda_identities", "kda_uniform")
              if pins.KDA_BWD_PINS[n][0](impl) > pins.KDA_BWD_PINS[n][1]]
    assert failed, f"mutant {kind} passes every pin"


@pytest.mark.parametrize("lo", [None, 0.05, 1e-3])
@pytest.mark.parametrize("chunk", [1, 3, 16, 32, 75])
def test_kda_chunk_form_equals_token_reverse_pass(lo, chunk):
    """The chunk algebra the GPU backward implements (oracle.chunkwise.chunk_bwd_channel)
    against the token reverse pass, at chunk sizes from 1 to T and gates down to 1e-3."""
    from oracle import chunkwise
    rng = np.random.default_rng(66)
    q, k, v, beta, d, a, S0, do, dS_T = pins.rand_bwd_kda(rng, 2, 2, 75, 6, 5, lo=lo)
    ref = backward.chunk_bwd(q, k, v, beta, d, None, S0, do, dS_T, alpha_ch=a)
    g = chunkwise.chunk_bwd_channel(q, k, v, beta, d, a, S0, do, dS_T, chunk=chunk)
    for n in ("dq", "dk", "dv", "dbeta", "dd", "dalpha_ch", "dS0"):
        assert pins._rel(g[n], ref[n]) < 1e-12, n
