"""GPU parity of the backward with the channel-wise gate (osdn_chunk_bwd_kda) against the
float64 reverse pass of the oracle (oracle.backward.chunk_bwd with alpha_ch) on the same seeded
inputs and output gradients.

Error measure per gradient: max |g - g_ref| / max |g_ref| over the whole tensor.  Bounds: 1e-4
for fp32 inputs; 2e-2 for bf16 inputs (fp32 arithmetic throughout, the gradients stored in
bf16)."""
import numpy as np
import pytest

from delta_rule_sequence_chunkwise_amd import osdn, synth
from oracle import backward
from tests.gpu_util import TOL, oracle_inputs, rel_err, say, to_dev, to_np, torch_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dbeta", "dd", "dalpha_ch", "dS0")
GPU_NAME = dict(dq="grad_q", dk="grad_k", dv="grad_v", dbeta="grad_beta", dd="grad_d",
                dalpha_ch="grad_alpha_ch", dS0="grad_S0")


def inputs(B, H, T, dk, dv, qkv, seed, gates=None, s0=True, dst=True):
    x = synth.make_shape(B, H, T, dk, dv, qkv=qkv, alpha=False, s0=s0, seed=seed)
    if gates is None:
        x["alpha_ch"] = synth.make_channel_gate(B, H, T, dk, seed=seed)
    else:
        x["alpha_ch"] = synth.make_channel_gate_uniform(B, H, T, dk, *gates, seed=seed)
    g = synth.make_output_grads(B, H, T, dk, dv, qkv=qkv, seed=seed, state=dst)
    return x, g


def run_gpu(x, g, qkv, d_dtype="f32", grads=None):
    torch, _ = torch_dev()
    out = osdn.osdn_chunk_bwd_kda(
        to_dev(x["q"], qkv), to_dev(x["k"], qkv), to_dev(x["v"], qkv), to_dev(x["beta"], "f32"),
        to_dev(x["d"], d_dtype), to_dev(x["alpha_ch"], "f32"), to_dev(x.get("S0"), "f32"),
        to_dev(g["do"], qkv), to_dev(g.get("dS_T"), "f32"), grads=grads)
    torch.cuda.synchronize()
    return {n: to_np(out[GPU_NAME[n]]) for n in NAMES}


def run_oracle(x, g, d_dtype="f32"):
    q, k, v, beta, d, _, S0 = oracle_inputs(x, d_dtype)
    return backward.chunk_bwd(q, k, v, beta, d, None, S0, g["do"], g.get("dS_T"),
                              alpha_ch=x["alpha_ch"])


def check(x, g, qkv, d_dtype="f32", label=""):
    say("chunk_bwd_kda", label, qkv, d_dtype, x["q"].shape)
    got = run_gpu(x, g, qkv, d_dtype)
    ref = run_oracle(x, g, d_dtype)
    errs = {}
    for n in NAMES:
        assert np.all(np.isfinite(got[n])), n
        errs[n] = rel_err(got[n], ref[n])
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= TOL[qkv]}
    assert not bad, bad


CASES = [
    # qkv, B, H, T, dk, dv, gates, S0, dS_T, d dtype
    ("f32", 1, 2, 100, 64, 64, None, True, True, "f32"),
    ("f32", 2, 1, 67, 128, 64, None, True, False, "f32"),
    ("f32", 1, 1, 33, 64, 128, (0.05, 0.6), False, True, "f32"),
    ("f32", 1, 2, 130, 128, 128, (0.3, 1.0), True, True, "f32"),
    ("f32", 1, 1, 1, 64, 64, None, True, True, "f32"),
    ("f32", 1, 2, 90, 64, 64, (1e-3, 1.0), True, True, "f32"),
    ("bf16", 2, 2, 257, 128, 128, None, True, True, "f32"),
    ("bf16", 1, 2, 96, 64, 128, (0.05, 0.6), True, True, "bf16"),
    ("bf16", 2, 1, 150, 128, 64, (1e-3, 1.0), True, True, "f32"),
    ("bf16", 1, 1, 31, 128, 128, (0.5, 0.7), False, False, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_bwd_kda(case):
    qkv, B, H, T, dk, dv, gates, s0, dst, dd = case
    x, g = inputs(B, H, T, dk, dv, qkv, seed=T + dk + 3, gates=gates, s0=s0, dst=dst)
    check(x, g, qkv, dd, label=str(case))


@pytest.mark.parametrize("T", [31, 32, 33, 64, 65])
def test_bwd_kda_chunk_boundaries(T):
    x, g = inputs(1, 1, T, 64, 64, "f32", seed=T + 1)
    check(x, g, "f32", label=f"T={T}")


def test_bwd_kda_uniform_channels_match_scalar_gate():
    """Equal factors on every channel: the gradients of q, k, v, beta, d and S0 equal those of
    the scalar-gate backward, and the per-channel gate gradients sum to the scalar one."""
    torch, _ = torch_dev()
    say("chunk_bwd_kda uniform channels")
    B, H, T, dk, dv = 1, 2, 100, 64, 64
    x, g = inputs(B, H, T, dk, dv, "f32", seed=21)
    a = synth.make_channel_gate_uniform(B, H, T, 1, 0.8, 1.0, seed=21)[..., 0]
    x["alpha"] = a
    x["alpha_ch"] = np.ascontiguousarray(np.repeat(a[..., None], dk, axis=-1))
    got = run_gpu(x, g, "f32")
    sc = osdn.osdn_chunk_bwd(
        to_dev(x["q"], "f32"), to_dev(x["k"], "f32"), to_dev(x["v"], "f32"),
        to_dev(x["beta"], "f32"), to_dev(x["d"], "f32"), to_dev(x["alpha"], "f32"),
        to_dev(x["S0"], "f32"), to_dev(g["do"], "f32"), to_dev(g["dS_T"], "f32"))
    torch.cuda.synchronize()
    for n, gn in (("dq", "grad_q"), ("dk", "grad_k"), ("dv", "grad_v"), ("dbeta", "grad_beta"),
                  ("dd", "grad_d"), ("dS0", "grad_S0")):
        assert rel_err(got[n], to_np(sc[gn])) <= 1e-4, n
    assert rel_err(got["dalpha_ch"].sum(-1), to_np(sc["grad_alpha"])) <= 1e-4


def test_bwd_kda_empty_sequence_passes_state_gradient():
    say("chunk_bwd_kda T=0")
    x, g = inputs(2, 3, 0, 64, 64, "f32", seed=5)
    out = run_gpu(x, g, "f32")
    assert np.array_equal(out["dS0"], np.asarray(g["dS_T"], np.float32).astype(np.float64))


def test_bwd_kda_is_deterministic_and_writes_in_bounds():
    torch, dev = torch_dev()
    say("chunk_bwd_kda repeat + sentinel")
    B, H, T, dk, dv = 2, 2, 150, 128, 128
    x, g = inputs(B, H, T, dk, dv, "bf16", seed=9)
    n = B * H * T * dk
    buf = torch.full((n + 4096,), 7.0, dtype=torch.float32, device=dev)
    grads = {"grad_alpha_ch": buf[:n].view(B, H, T, dk)}
    args = (to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"),
            to_dev(x["beta"], "f32"), to_dev(x["d"], "f32"), to_dev(x["alpha_ch"], "f32"),
            to_dev(x["S0"], "f32"), to_dev(g["do"], "bf16"), to_dev(g["dS_T"], "f32"))
    a = osdn.osdn_chunk_bwd_kda(*args, grads=grads)
    first = {k: v.clone() for k, v in a.items() if v is not None}
    b = osdn.osdn_chunk_bwd_kda(*args, grads=grads)
    torch.cuda.synchronize()
    assert torch.all(buf[n:] == 7.0)
    for k, v in first.items():
        assert torch.equal(v, b[k]), k


def test_bwd_kda_many_chunks():
    """2 x 8 sequences of 1100 tokens: 560 chunks of 32 rows, the last of each ragged."""
    x, g = inputs(2, 8, 1100, 128, 128, "bf16", seed=31, gates=(0.3, 1.0))
    check(x, g, "bf16", label="560 chunks")


def test_bwd_kda_full_1p3b_sampled():
    """The 1.3B-shape workload (B=4, H=16, T=4096, bf16) with the generator's channel gate
    through the GPU backward in one call; two sampled (b, h) sequences compared element by
    element with the oracle run on them alone (sequences are independent)."""
    w = synth.WORKLOADS["1.3b"]
    say("chunk_bwd_kda full 1.3b")
    x = synth.make_inputs(w)
    x.pop("alpha", None)
    x["alpha_ch"] = synth.make_channel_gate(w.B, w.H, w.T, w.dk, seed=w.seed)
    g = synth.make_output_grads(w.B, w.H, w.T, w.dk, w.dv, qkv=w.qkv, seed=w.seed, state=True)
    got = run_gpu(x, g, "bf16")
    for b, h in ((0, 0), (w.B - 1, w.H - 1)):
        sl = lambda a: None if a is None else np.ascontiguousarray(a[b:b + 1, h:h + 1])
        xs = {k: sl(v) for k, v in x.items()}
        gs = {k: sl(v) for k, v in g.items()}
        ref = run_oracle(xs, gs)
        errs = {n: rel_err(got[n][b:b + 1, h:h + 1], ref[n]) for n in NAMES}
        say(f"  seq ({b},{h}): " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
        assert all(e <= TOL["bf16"] for e in errs.values()), errs
