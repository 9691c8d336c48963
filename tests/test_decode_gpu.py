"""GPU tests of the recurrent decode step: parity with the oracle's token step, the gated
Newton condition, and agreement between the chunkwise and the step-by-step paths."""
import numpy as np
import pytest

import oracle
from delta_rule_sequence_chunkwise_amd import osdn, synth
from tests.gpu_util import TOL, rel_err, say, to_dev, to_np, torch_dev

pytestmark = pytest.mark.gpu


def run_steps(x, qkv, steps, S0=None):
    """Run `steps` calls of osdn_step from S0 (default: the generator's); returns (o, S)."""
    torch, dev = torch_dev()
    S = to_dev(x["S0"] if S0 is None else S0, "f32").clone()
    outs = []
    for t in range(steps):
        o = osdn.osdn_step(to_dev(x["q"][t], qkv), to_dev(x["k"][t], qkv),
                           to_dev(x["v"][t], qkv), to_dev(x["beta"][t], "f32"),
                           to_dev(x["d"][t], "f32"),
                           None if x["alpha"] is None else to_dev(x["alpha"][t], "f32"), S)
        outs.append(o)
    torch.cuda.synchronize()
    return np.stack([to_np(o) for o in outs]), to_np(S)


def oracle_steps(x, steps):
    S = x["S0"].astype(np.float64)
    outs = []
    for t in range(steps):
        o, S = oracle.step(x["q"][t], x["k"][t], x["v"][t], x["beta"][t], x["d"][t],
                           None if x["alpha"] is None else x["alpha"][t], S)
        outs.append(o)
    return np.stack(outs), S


@pytest.mark.parametrize("qkv,dk,dv", [("f32", 64, 64), ("f32", 128, 64), ("bf16", 64, 128),
                                       ("bf16", 128, 128)])
def test_step_parity(qkv, dk, dv):
    w = synth.Workload("dec", B=3, H=5, T=1, dk=dk, dv=dv, qkv=qkv, s0=True, steps=6,
                       seed_index=40)
    x = synth.make_decode_inputs(w)
    say("step parity", qkv, dk, dv)
    o, S = run_steps(x, qkv, 6)
    o_ref, S_ref = oracle_steps(x, 6)
    eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
    say(f"  e_o={eo:.3e} e_S={es:.3e}")
    assert eo <= TOL[qkv] and es <= TOL[qkv]
    if qkv == "f32":  # pure fp32 arithmetic: far inside the bound
        assert eo <= 1e-5 and es <= 1e-5


def test_decode_workload_first_steps():
    """The full decode shape (B=128, H=16, dk=dv=128, bf16) for a few steps."""
    w = synth.WORKLOADS["decode"]
    x = synth.make_decode_inputs(w, steps=4)
    say("decode workload, 4 steps")
    o, S = run_steps(x, "bf16", 4)
    o_ref, S_ref = oracle_steps(x, 4)
    eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
    say(f"  e_o={eo:.3e} e_S={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_step_newton_condition():
    """With beta <d, k^2> = 1 the step stores the association exactly: S_t^T k = v."""
    torch, dev = torch_dev()
    rng = np.random.default_rng(0)
    B, H, dk, dv = 2, 3, 128, 64
    k = rng.standard_normal((B, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    u = np.exp(0.3 * rng.standard_normal((B, H, dk)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H))))
    d = u / (beta * np.sum(u * k * k, axis=-1))[..., None]
    f = lambda a: np.asarray(a, dtype=np.float32)
    q, v = f(rng.standard_normal((B, H, dk))), f(rng.standard_normal((B, H, dv)))
    alpha = f(np.full((B, H), 0.9))
    S = to_dev(f(0.1 * rng.standard_normal((B, H, dk, dv))), "f32")
    say("newton step")
    osdn.osdn_step(to_dev(q, "f32"), to_dev(f(k), "f32"), to_dev(v, "f32"),
                   to_dev(f(beta), "f32"), to_dev(f(d), "f32"), to_dev(alpha, "f32"), S)
    torch.cuda.synchronize()
    recalled = np.einsum("bhij,bhi->bhj", to_np(S), f(k).astype(np.float64))
    assert rel_err(recalled, v) <= 1e-5


@pytest.mark.parametrize("qkv", ["f32", "bf16"])
def test_chunk_and_step_paths_agree(qkv):
    w = synth.Workload("dec", B=2, H=3, T=1, dk=128, dv=128, qkv=qkv, s0=True, steps=150,
                       seed_index=41)
    x = synth.make_decode_inputs(w)
    say("chunk vs step", qkv)
    o_step, S_step = run_steps(x, qkv, 150)
    seq = lambda a: np.ascontiguousarray(np.moveaxis(a, 0, 2))  # [steps,B,H,.] -> [B,H,T,.]
    xc = {n: seq(x[n]) for n in ("q", "k", "v", "beta", "d", "alpha")}
    xc["S0"] = x["S0"]
    from tests.gpu_util import gpu_chunk
    o_chunk, S_chunk = gpu_chunk(xc, qkv=qkv)
    o_step = np.moveaxis(o_step, 0, 2)
    eo, es = rel_err(o_chunk, o_step), rel_err(S_chunk, S_step)
    say(f"  chunk vs step: e_o={eo:.3e} e_S={es:.3e}")
    assert eo <= TOL[qkv] and es <= TOL[qkv]


@pytest.mark.slow
def test_decode_workload_chunk_vs_step_1024():
    """The decode workload run both ways for all 1024 tokens from the same initial state,
    each checked against the oracle."""
    w = synth.WORKLOADS["decode"]
    x = synth.make_decode_inputs(w)
    say("decode workload: 1024 steps")
    o_step, S_step = run_steps(x, "bf16", w.steps)
    seq = lambda a: np.ascontiguousarray(np.moveaxis(a, 0, 2))
    xc = {n: seq(x[n]) for n in ("q", "k", "v", "beta", "d", "alpha")}
    xc["S0"] = x["S0"]
    from tests.gpu_util import gpu_chunk
    say("decode workload: one 1024-token chunk_fwd")
    o_chunk, S_chunk = gpu_chunk(xc, qkv="bf16")
    o_ref, S_ref = oracle.chunk_fwd(xc["q"], xc["k"], xc["v"], xc["beta"], xc["d"],
                                    xc["alpha"], xc["S0"])
    o_step = np.moveaxis(o_step, 0, 2)
    for name, o, S in (("step", o_step, S_step), ("chunk", o_chunk, S_chunk)):
        eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
        say(f"  {name}: e_o={eo:.3e} e_S={es:.3e}")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    assert rel_err(o_chunk, o_step) <= TOL["bf16"]
