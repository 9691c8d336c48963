"""GPU: the channel-wise forward through the entry point that allocates nothing
(osdn_chunk_fwd_kda_noalloc, called through the C ABI) against the entry point that takes a
caller's workspace (osdn_chunk_fwd_kda), on two calls in a row, the second smaller, so the second
runs over the first's stale scratch contents.  Same kernels, so the outputs must be bitwise
equal; both are also held to the oracle's bounds (2e-2 for bf16 inputs, 1e-4 for fp32)."""
import numpy as np
import pytest

import oracle
from delta_rule_sequence_chunkwise_amd import osdn, synth
from tests.gpu_util import TOL, oracle_inputs, rel_err, say, to_dev, to_np, torch_dev

pytestmark = pytest.mark.gpu


def inputs(B, H, T, dk, dv, qkv, seed):
    x = synth.make_shape(B, H, T, dk, dv, qkv=qkv, alpha=False, s0=True, seed=seed)
    x["alpha_ch"] = synth.make_channel_gate_uniform(B, H, T, dk, 0.05, 1.0, seed=seed)
    return x


def run_both(x, qkv, chunk):
    torch, dev = torch_dev()
    args = (to_dev(x["q"], qkv), to_dev(x["k"], qkv), to_dev(x["v"], qkv),
            to_dev(x["beta"], "f32"), to_dev(x["d"], "f32"), to_dev(x["alpha_ch"], "f32"),
            to_dev(x["S0"], "f32"))
    B, H, T, dk = x["q"].shape
    dv = x["v"].shape[-1]
    dt = args[0].dtype
    o_n = torch.empty((B, H, T, dv), dtype=dt, device=dev)
    S_n = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    osdn.osdn_chunk_fwd_kda_noalloc(*args, o_n, S_n, chunk=chunk)
    o_w, S_w = osdn.osdn_chunk_fwd_kda(*args, chunk=chunk)
    torch.cuda.synchronize()
    return to_np(o_n), to_np(S_n), to_np(o_w), to_np(S_w)


@pytest.mark.parametrize("qkv,chunk", [("bf16", 64), ("f32", 32)])
def test_noalloc_matches_workspace_entry_point(qkv, chunk):
    # the first call fills more of the scratch than the second overwrites
    for B, H, T, dk, dv, seed in ((2, 4, 700, 128, 128, 1), (1, 2, 130, 64, 128, 2)):
        say("kda noalloc", qkv, B, H, T, dk, dv)
        x = inputs(B, H, T, dk, dv, qkv, seed)
        o_n, S_n, o_w, S_w = run_both(x, qkv, chunk)
        assert np.array_equal(o_n, o_w) and np.array_equal(S_n, S_w)
        q, k, v, beta, d, _, S0 = oracle_inputs(x)
        o_ref, S_ref = oracle.chunk_fwd(q, k, v, beta, d, None, S0, alpha_ch=x["alpha_ch"])
        eo, es = rel_err(o_n, o_ref), rel_err(S_n, S_ref)
        say(f"  e_o={eo:.3e} e_S={es:.3e}")
        assert eo <= TOL[qkv] and es <= TOL[qkv]


def test_noalloc_rejects_a_problem_larger_than_its_scratch():
    torch, dev = torch_dev()
    B, H, T, dk, dv = 1, 16, 8192, 128, 128
    assert osdn.kda_workspace_bytes(B, H, T, dk, 64, osdn.OSDN_BF16) > osdn.NOALLOC_SCRATCH_BYTES
    z = lambda *shape, dt=torch.bfloat16: torch.zeros(shape, dtype=dt, device=dev)
    with pytest.raises(osdn.OSDNError) as e:
        osdn.osdn_chunk_fwd_kda_noalloc(z(B, H, T, dk), z(B, H, T, dk), z(B, H, T, dv),
                                        z(B, H, T, dt=torch.float32),
                                        z(B, H, T, dk, dt=torch.float32),
                                        z(B, H, T, dk, dt=torch.float32), None,
                                        z(B, H, T, dv), None)
    assert e.value.status == -7
