"""GPU parity of the backward (osdn_chunk_bwd) against the float64 reverse pass of the oracle
on the same seeded inputs and output gradients.

Error measure per gradient: max |g - g_ref| / max |g_ref| over the whole tensor.  Bounds: 1e-4
for fp32 inputs; 2e-2 for bf16 inputs, whose state checkpoints and products are fp32 but whose
output gradients are stored in bf16 (one rounding, 2^-9) and whose d may be stored in bf16."""
import numpy as np
import pytest

from delta_rule_sequence_chunkwise_amd import osdn, synth
from oracle import backward
from tests.gpu_util import TOL, oracle_inputs, rel_err, say, to_dev, to_np, torch_dev

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dbeta", "dd", "dalpha", "dS0")
GPU_NAME = dict(dq="grad_q", dk="grad_k", dv="grad_v", dbeta="grad_beta", dd="grad_d",
                dalpha="grad_alpha", dS0="grad_S0")


def bwd_inputs(B, H, T, dk, dv, qkv, seed, alpha=True, s0=True, dst=True):
    x = synth.make_shape(B, H, T, dk, dv, qkv=qkv, alpha=alpha, s0=s0, seed=seed)
    g = synth.make_output_grads(B, H, T, dk, dv, qkv=qkv, seed=seed, state=dst)
    return x, g


def run_gpu(x, g, qkv, d_dtype="f32", workspace=None):
    torch, _ = torch_dev()
    out = osdn.osdn_chunk_bwd(
        to_dev(x["q"], qkv), to_dev(x["k"], qkv), to_dev(x["v"], qkv), to_dev(x["beta"], "f32"),
        to_dev(x["d"], d_dtype), to_dev(x.get("alpha"), "f32"), to_dev(x.get("S0"), "f32"),
        to_dev(g["do"], qkv), to_dev(g.get("dS_T"), "f32"), workspace=workspace)
    torch.cuda.synchronize()
    return {n: to_np(out[GPU_NAME[n]]) for n in NAMES}


def run_oracle(x, g, d_dtype="f32"):
    q, k, v, beta, d, a, S0 = oracle_inputs(x, d_dtype)
    return backward.chunk_bwd(q, k, v, beta, d, a, S0, g["do"], g.get("dS_T"))


def check(x, g, qkv, d_dtype="f32", label=""):
    say("chunk_bwd", label, qkv, d_dtype, x["q"].shape)
    got = run_gpu(x, g, qkv, d_dtype)
    ref = run_oracle(x, g, d_dtype)
    errs = {}
    for n in NAMES:
        if ref[n] is None:
            assert got[n] is None, n
            continue
        assert np.all(np.isfinite(got[n])), n
        errs[n] = rel_err(got[n], ref[n])
    say("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= TOL[qkv]}
    assert not bad, bad


F32_CASES = [
    # B, H, T, dk, dv, alpha, S0, dS_T
    (1, 2, 256, 64, 64, False, False, False),   # the Tiny workload's shape
    (1, 2, 100, 64, 64, True, True, True),
    (2, 1, 67, 128, 64, True, True, True),
    (1, 1, 33, 64, 128, True, False, True),
    (1, 1, 1, 64, 64, True, True, True),
    (1, 1, 32, 128, 128, True, True, False),
]


@pytest.mark.parametrize("case", F32_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bwd_f32(case):
    B, H, T, dk, dv, al, s0, dst = case
    x, g = bwd_inputs(B, H, T, dk, dv, "f32", seed=T + dk + dv, alpha=al, s0=s0, dst=dst)
    check(x, g, "f32", label=str(case))


BF16_CASES = [
    # B, H, T, dk, dv, d dtype, alpha, S0, dS_T
    (1, 2, 130, 128, 128, "f32", True, True, True),
    (2, 1, 64, 128, 128, "f32", True, False, True),
    (1, 1, 65, 64, 128, "bf16", True, True, True),
    (1, 2, 200, 128, 64, "f32", False, True, False),
    (1, 1, 1, 128, 128, "f32", True, True, True),
    (2, 2, 257, 64, 64, "bf16", True, True, True),
    # sequence counts that are multiples of 8 take the reverse pass's XCD-grouped mapping
    (2, 4, 130, 128, 128, "f32", True, True, True),
    (1, 8, 100, 64, 128, "bf16", True, False, True),
]


@pytest.mark.parametrize("case", BF16_CASES, ids=lambda c: "x".join(map(str, c)))
def test_bwd_bf16(case):
    B, H, T, dk, dv, dd, al, s0, dst = case
    x, g = bwd_inputs(B, H, T, dk, dv, "bf16", seed=T + 3 * dk, alpha=al, s0=s0, dst=dst)
    check(x, g, "bf16", dd, label=str(case))


@pytest.mark.parametrize("case", [(1, 8, 2100, 64, 64, "bf16"), (1, 4, 4200, 128, 64, "f32")],
                         ids=lambda c: "x".join(map(str, c)))
def test_bwd_bf16_several_chunks_per_workgroup(case):
    """More chunks than compute units (264 > 256), so the persistent per-chunk pass takes
    several chunks in one workgroup, one of them ragged."""
    B, H, T, dk, dv, dd = case
    x, g = bwd_inputs(B, H, T, dk, dv, "bf16", seed=T + dk)
    check(x, g, "bf16", dd, label=str(case))


def test_bwd_empty_sequence_passes_state_gradient():
    torch, dev = torch_dev()
    say("chunk_bwd T=0")
    x, g = bwd_inputs(2, 3, 0, 64, 64, "f32", seed=5)
    out = run_gpu(x, g, "f32")
    assert np.array_equal(out["dS0"], np.asarray(g["dS_T"], np.float32).astype(np.float64))


def test_bwd_is_deterministic_and_writes_in_bounds():
    torch, dev = torch_dev()
    say("chunk_bwd repeat + sentinel")
    B, H, T, dk, dv = 2, 2, 150, 128, 128
    x, g = bwd_inputs(B, H, T, dk, dv, "bf16", seed=9)
    n = B * H * T * dk
    buf = torch.full((n + 4096,), 7.0, dtype=torch.bfloat16, device=dev)
    grads = {"grad_q": buf[:n].view(B, H, T, dk)}
    args = (to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"), to_dev(x["v"], "bf16"),
            to_dev(x["beta"], "f32"), to_dev(x["d"], "f32"), to_dev(x["alpha"], "f32"),
            to_dev(x["S0"], "f32"), to_dev(g["do"], "bf16"), to_dev(g["dS_T"], "f32"))
    a = osdn.osdn_chunk_bwd(*args, grads=grads)
    first = {k: v.clone() for k, v in a.items() if v is not None}
    b = osdn.osdn_chunk_bwd(*args, grads=grads)
    torch.cuda.synchronize()
    assert torch.all(buf[n:] == 7.0)
    for k, v in first.items():
        assert torch.equal(v, b[k]), k


@pytest.mark.parametrize("T", [63, 64, 65, 128])
def test_bwd_chunk_boundaries_bf16(T):
    x, g = bwd_inputs(1, 1, T, 128, 128, "bf16", seed=T)
    check(x, g, "bf16", label=f"T={T}")


@pytest.mark.parametrize("T", [31, 32, 33])
def test_bwd_chunk_boundaries_f32(T):
    x, g = bwd_inputs(1, 1, T, 64, 64, "f32", seed=T)
    check(x, g, "f32", label=f"T={T}")


def test_bwd_full_1p3b_sampled():
    """The 1.3B-shape workload (B=4, H=16, T=4096) through the GPU backward in one call; two
    sampled (b, h) sequences compared element by element with the oracle run on them alone
    (sequences are independent)."""
    torch, dev = torch_dev()
    w = synth.WORKLOADS["1.3b"]
    say("chunk_bwd full 1.3b")
    x = synth.make_inputs(w)
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


def _workspace_states(ws, B, H, T, dk, dv, qkv):
    """The backward's own recomputed states and (bf16) U: the workspace's first region, and its
    region after the two checkpoints and the per-chunk planes."""
    torch, _ = torch_dev()
    C = 64 if qkv == "bf16" else 32
    nch = (T + C - 1) // C
    n = B * H * nch * dk * dv
    r256 = lambda x: (x + 255) // 256 * 256
    dt = torch.bfloat16 if qkv == "bf16" else torch.float32
    if qkv != "bf16":
        return ws[: n * 4].view(dt).view(B, H, nch, dk, dv), None
    ck = ws[: n * 2].view(dt).view(B, H, nch, dv // 16, dk, 16)  # column tiles
    off = 2 * r256(n * 2) + r256(B * H * nch * (3 * C * C + C * dk) * 2)
    return ck, ws[off:off + B * H * nch * C * dv * 2].view(dt).view(B, H, nch, dv // 16, C, 16)


@pytest.mark.parametrize("case", [(1, 2, 130, 128, 128, "bf16"), (2, 1, 64, 64, 128, "bf16"),
                                  (2, 4, 100, 128, 64, "bf16"),
                                  (1, 1, 67, 64, 64, "f32"), (1, 2, 33, 128, 64, "f32")],
                         ids=lambda c: "x".join(map(str, c)))
def test_training_pair_matches_recompute_bitwise(case):
    """osdn_chunk_fwd_states gives osdn_chunk_fwd's o and S_T (at the backward's chunk size)
    and the backward's own checkpoints (and, for bf16, U); osdn_chunk_bwd with those states
    gives the gradients of the recomputing backward, bitwise."""
    torch, dev = torch_dev()
    B, H, T, dk, dv, qkv = case
    say("training pair", case)
    x, g = bwd_inputs(B, H, T, dk, dv, qkv, seed=T + dk)
    args = (to_dev(x["q"], qkv), to_dev(x["k"], qkv), to_dev(x["v"], qkv), to_dev(x["beta"], "f32"),
            to_dev(x["d"], "f32"), to_dev(x["alpha"], "f32"), to_dev(x["S0"], "f32"))
    C = 64 if qkv == "bf16" else 32
    o_ref, s_ref = osdn.osdn_chunk_fwd(*args, chunk=C)
    o, s_t, states = osdn.osdn_chunk_fwd_states(*args)
    go, gst = to_dev(g["do"], qkv), to_dev(g["dS_T"], "f32")
    ws = torch.empty(osdn.bwd_workspace_bytes(B, H, T, dk, dv, osdn._dtype_code(args[0])),
                     dtype=torch.uint8, device=dev)
    ref = osdn.osdn_chunk_bwd(*args, go, gst, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(s_t, s_ref)
    ck, u = osdn.states_parts(states, B, H, T, dk, dv, args[0].dtype)
    ck_ref, u_ref = _workspace_states(ws, B, H, T, dk, dv, qkv)
    assert torch.equal(ck, ck_ref)
    # the documented layout: slot c holds the state after the first c chunks, per the oracle
    import oracle
    q_, k_, v_, b_, d_, a_, s0_ = oracle_inputs(x, "f32")
    mats = to_np(osdn.checkpoint_matrix(ck))
    for c in range(ck.shape[2]):
        if c == 0:
            ref_c = s0_
        else:
            t_ = c * C
            _, ref_c = oracle.chunk_fwd(q_[:, :, :t_], k_[:, :, :t_], v_[:, :, :t_], b_[:, :, :t_],
                                        d_[:, :, :t_], a_[:, :, :t_], s0_)
        assert rel_err(mats[:, :, c], ref_c) <= TOL[qkv], f"checkpoint {c}"
    assert (u is None) == (u_ref is None) and (u is None or torch.equal(u, u_ref))
    got = osdn.osdn_chunk_bwd(*args, go, gst, states=states)
    torch.cuda.synchronize()
    for name, t in ref.items():
        if t is not None:
            assert torch.equal(got[name], t), name
