"""GPU parity of the channel-wise (KDA) gate: osdn_chunk_fwd_kda and osdn_step_kda against the
float64 oracle on the same seeded inputs.

Error measure and bounds as for the scalar gate: max |x - x_ref| / max |x_ref| for o and the
final state, 1e-4 for fp32 inputs and 2e-2 for bf16 inputs (fp32 accumulation).  On the bf16
path the gate-scaled operands (products of gates, each at most 1, times q, k or k~) are rounded
to bf16 once, as the forward rounds its operands anyway.  Gates from the generator's mild
recipe, strong decay U(0.05, 0.6), tiny gates down to 1e-30, and gates of exactly 0 are
covered (Erase-then-Delta Attention, section 2.2, eq. 5 bounds a_t only by (0, 1))."""
import numpy as np
import pytest

import oracle
from delta_rule_sequence_chunkwise_amd import osdn, synth
from tests.gpu_util import TOL, oracle_inputs, rel_err, say, to_dev, to_np, torch_dev

pytestmark = pytest.mark.gpu


def kda_inputs(B, H, T, dk, dv, qkv, seed, s0=True, gates=None):
    x = synth.make_shape(B, H, T, dk, dv, qkv=qkv, alpha=False, s0=s0, seed=seed)
    if gates is None:
        x["alpha_ch"] = synth.make_channel_gate(B, H, T, dk, seed=seed)
    elif gates == "zeros":  # mild gates with about 2% exact zeros
        a = synth.make_channel_gate_uniform(B, H, T, dk, 0.5, 1.0, seed=seed)
        z = synth.make_channel_gate_uniform(B, H, T, dk, 0.0, 1.0, seed=seed + 1)
        a[z < 0.02] = 0.0
        x["alpha_ch"] = a
    else:
        lo, hi = gates
        x["alpha_ch"] = synth.make_channel_gate_uniform(B, H, T, dk, lo, hi, seed=seed)
    return x


def run_kda(x, qkv, d_dtype="f32", chunk=64):
    torch, _ = torch_dev()
    o, S = osdn.osdn_chunk_fwd_kda(
        to_dev(x["q"], qkv), to_dev(x["k"], qkv), to_dev(x["v"], qkv), to_dev(x["beta"], "f32"),
        to_dev(x["d"], d_dtype), to_dev(x["alpha_ch"], "f32"), to_dev(x.get("S0"), "f32"),
        chunk=chunk)
    torch.cuda.synchronize()
    return to_np(o), to_np(S)


def check(x, qkv, d_dtype="f32", chunk=64, label=""):
    say("chunk_fwd_kda", label, qkv, d_dtype, chunk, x["q"].shape)
    o, S = run_kda(x, qkv, d_dtype, chunk)
    q, k, v, beta, d, _, S0 = oracle_inputs(x, d_dtype)
    o_ref, S_ref = oracle.chunk_fwd(q, k, v, beta, d, None, S0, alpha_ch=x["alpha_ch"])
    eo, es = rel_err(o, o_ref), rel_err(S, S_ref)
    say(f"  e_o={eo:.3e} e_S={es:.3e}")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    assert eo <= TOL[qkv] and es <= TOL[qkv], (eo, es)


BF16_CASES = [
    # B, H, T, dk, dv, d dtype, S0
    (1, 2, 64, 128, 128, "f32", True),
    (2, 1, 130, 128, 64, "f32", False),
    (1, 1, 1, 64, 64, "f32", True),
    (1, 2, 333, 64, 128, "bf16", True),
    (2, 2, 257, 128, 128, "bf16", False),
]


@pytest.mark.parametrize("case", BF16_CASES, ids=lambda c: "x".join(map(str, c)))
def test_kda_bf16(case):
    B, H, T, dk, dv, dd, s0 = case
    check(kda_inputs(B, H, T, dk, dv, "bf16", seed=T + dk, s0=s0), "bf16", dd, label=str(case))


F32_CASES = [
    # B, H, T, dk, dv, chunk
    (1, 2, 200, 64, 64, 16),
    (2, 1, 67, 128, 64, 32),
    (1, 1, 130, 128, 128, 64),
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: "x".join(map(str, c)))
def test_kda_f32(case):
    B, H, T, dk, dv, chunk = case
    check(kda_inputs(B, H, T, dk, dv, "f32", seed=T + 7), "f32", chunk=chunk, label=str(case))


STRONG = [
    # qkv, B, H, T, dk, dv, gates, chunk (fp32)
    ("bf16", 1, 2, 256, 128, 128, (0.05, 0.6), 64),
    ("bf16", 2, 1, 200, 64, 128, (0.05, 0.6), 64),
    ("bf16", 1, 2, 192, 128, 64, (0.2, 0.6), 64),
    ("bf16", 1, 1, 130, 128, 128, (1e-30, 1e-20), 64),
    ("bf16", 2, 1, 150, 64, 64, (1e-6, 1.0), 64),
    ("bf16", 1, 2, 160, 128, 128, "zeros", 64),
    ("f32", 1, 2, 192, 128, 128, (0.05, 0.6), 64),
    ("f32", 1, 1, 100, 64, 64, (0.05, 0.6), 16),
    ("f32", 1, 1, 96, 128, 64, (1e-30, 1e-20), 32),
    ("f32", 1, 2, 130, 64, 128, "zeros", 64),
]


@pytest.mark.parametrize("case", STRONG, ids=lambda c: "x".join(map(str, c)))
def test_kda_strong_decay(case):
    qkv, B, H, T, dk, dv, gates, chunk = case
    x = kda_inputs(B, H, T, dk, dv, qkv, seed=T + dk + 5, gates=gates)
    check(x, qkv, chunk=chunk, label=str(case))


def test_kda_more_chunks_than_compute_units():
    """2 x 8 sequences of 1100 tokens: 288 chunks (the last of each ragged), more than the
    planes kernel's persistent workgroups, so each takes several in turn."""
    x = kda_inputs(2, 8, 1100, 128, 128, "bf16", seed=31, gates=(0.3, 1.0))
    check(x, "bf16", label="288 chunks")


def test_uniform_channels_match_scalar_gate():
    """Equal channel factors on the GPU's KDA path against the scalar-gate path on the GPU."""
    torch, _ = torch_dev()
    say("kda uniform vs scalar")
    x = synth.make_shape(2, 2, 190, 128, 128, qkv="bf16", alpha=True, s0=True, seed=21)
    x["alpha_ch"] = np.repeat(x["alpha"][..., None], 128, axis=-1)
    o_k, S_k = run_kda(x, "bf16")
    o_s, S_s = osdn.osdn_chunk_fwd(to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"),
                                   to_dev(x["v"], "bf16"), to_dev(x["beta"], "f32"),
                                   to_dev(x["d"], "f32"), to_dev(x["alpha"], "f32"),
                                   to_dev(x["S0"], "f32"))
    torch.cuda.synchronize()
    assert rel_err(o_k, to_np(o_s)) <= 2e-2 and rel_err(S_k, to_np(S_s)) <= 2e-2


def test_kda_step_chain_matches_oracle_and_chunk():
    torch, dev = torch_dev()
    say("step_kda chain")
    B, H, T, dk, dv = 2, 3, 24, 128, 128
    x = kda_inputs(B, H, T, dk, dv, "bf16", seed=22)
    S = to_dev(x["S0"], "f32")
    outs = []
    for t in range(T):
        sl = lambda a: np.ascontiguousarray(a[:, :, t])
        outs.append(to_np(osdn.osdn_step_kda(
            to_dev(sl(x["q"]), "bf16"), to_dev(sl(x["k"]), "bf16"), to_dev(sl(x["v"]), "bf16"),
            to_dev(sl(x["beta"]), "f32"), to_dev(sl(x["d"]), "f32"),
            to_dev(sl(x["alpha_ch"]), "f32"), S)))
    torch.cuda.synchronize()
    o_step = np.stack(outs, axis=2)
    q, k, v, beta, d, _, S0 = oracle_inputs(x)
    o_ref, S_ref = oracle.chunk_fwd(q, k, v, beta, d, None, S0, alpha_ch=x["alpha_ch"])
    assert rel_err(o_step, o_ref) <= 2e-2 and rel_err(to_np(S), S_ref) <= 1e-4
    o_c, S_c = run_kda(x, "bf16")
    assert rel_err(o_c, o_step) <= 2e-2 and rel_err(S_c, to_np(S)) <= 2e-2


def test_kda_output_stays_in_bounds_and_workspace_reuse():
    torch, dev = torch_dev()
    say("kda bounds")
    B, H, T, dk, dv = 2, 3, 70, 128, 128
    x = kda_inputs(B, H, T, dk, dv, "bf16", seed=23)
    n = B * H * T * dv
    buf = torch.full((n + 4096,), 7.0, dtype=torch.bfloat16, device=dev)
    o = buf[:n].view(B, H, T, dv)
    ws = torch.empty(osdn.kda_workspace_bytes(B, H, T, dk, 64, osdn.OSDN_BF16) + 4096,
                     dtype=torch.uint8, device=dev)
    args = (to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"),
            to_dev(x["beta"], "f32"), to_dev(x["d"], "f32"), to_dev(x["alpha_ch"], "f32"),
            to_dev(x["S0"], "f32"))
    _, S1 = osdn.osdn_chunk_fwd_kda(*args, o=o, workspace=ws)
    o1 = to_np(o).copy()
    _, S2 = osdn.osdn_chunk_fwd_kda(*args, o=o, workspace=ws)  # stale workspace contents
    torch.cuda.synchronize()
    assert torch.all(buf[n:] == 7.0)
    assert np.array_equal(o1, to_np(o)) and torch.equal(S1, S2)


def test_kda_full_size_1p3b():
    """The 1.3B-shape workload with a channel-wise gate, the whole output compared."""
    w = synth.WORKLOADS["1.3b"]
    say("chunk_fwd_kda full 1.3b")
    x = synth.make_inputs(w)
    x["alpha_ch"] = synth.make_channel_gate(w.B, w.H, w.T, w.dk, seed=w.seed)
    check(x, "bf16", label="1.3b")
