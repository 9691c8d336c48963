"""GPU parity of the Phase-1 preconditioner scan (osdn_precond_scan, osdn_precond_step) against
the float64 oracle on the same seeded inputs.

Error measure: max |d_gpu - d_ref| / max |d_ref| over the whole output.  Bounds:
* token-serial form (fp32 arithmetic): 1e-4 for fp32 outputs;
* chunkwise form (bf16 matrix-core products with fp32 accumulation): 3e-3 for the emitted d_t,
  whose in-chunk correction W X is a bf16 product, and 1e-3 for the carried state, which
  takes bf16 rounding only inside L (the Gram matrix of k^2);
* a bf16 output adds its own rounding, at most half an ulp = 2^-8 of the value (bf16 keeps 8
  significant bits): 5e-3 (serial) and 7e-3 (chunkwise: 2^-8 + 3e-3).
"""
import numpy as np
import pytest

from delta_rule_sequence_chunkwise_amd import osdn, synth
from oracle import precond
from tests.gpu_util import rel_err, say, to_dev, to_np, torch_dev

pytestmark = pytest.mark.gpu

TOL_SERIAL = {"f32": 1e-4, "bf16": 5e-3}
TOL_CHUNK = {"f32": 3e-3, "bf16": 7e-3}
TOL_CHUNK_STATE = 1e-3


def inputs(B, H, T, dk, kdt, seed, apf=True, d1=True, zero_rows=()):
    x = synth.make_shape(B, H, T, dk, dk, qkv=kdt, alpha=False, seed=seed)
    g = synth.make_precond_gates(B, H, T, dk, seed=seed)
    k = x["k"].copy()
    for (b, h, t) in zero_rows:
        if t < T:
            k[b, h, t] = 0.0
    return k, x["beta"], (g["r"] if apf else None), (g["d1"] if d1 else None)


def run_gpu(k, beta, r, d1, eta, kdt, ddt, chunk, state=True):
    torch, _ = torch_dev()
    d, dn = osdn.osdn_precond_scan(
        to_dev(k, kdt), to_dev(beta, "f32"), to_dev(r, "f32"), to_dev(d1, "f32"), eta=eta,
        chunk=chunk, d_dtype={"f32": torch.float32, "bf16": torch.bfloat16}[ddt],
        want_state=state)
    torch.cuda.synchronize()
    return to_np(d), to_np(dn)


def check(case, chunk):
    B, H, T, dk, kdt, ddt, apf, d1, eta = case
    say("precond_scan", "chunk", chunk, case)
    k, beta, r, dd1 = inputs(B, H, T, dk, kdt, seed=T + dk + 3 * B, apf=apf, d1=d1,
                             zero_rows=((0, 0, 5), (B - 1, H - 1, T // 2)))
    d, dn = run_gpu(k, beta, r, dd1, eta, kdt, ddt, chunk)
    d_ref, dn_ref = precond.precond_scan(k, beta, eta, r, dd1)
    e_d, e_n = rel_err(d, d_ref), rel_err(dn, dn_ref)
    say(f"  e_d={e_d:.3e} e_next={e_n:.3e}")
    assert np.all(np.isfinite(d)) and np.all(np.isfinite(dn))
    if chunk == 1:
        assert e_d <= TOL_SERIAL[ddt] and e_n <= TOL_SERIAL["f32"], (e_d, e_n)
    else:
        assert e_d <= TOL_CHUNK[ddt] and e_n <= TOL_CHUNK_STATE, (e_d, e_n)


SERIAL_CASES = [
    # B, H, T, dk, key dtype, d dtype, APF gate, d1 given, eta
    (1, 2, 256, 64, "f32", "f32", True, True, 2.0),
    (2, 1, 67, 128, "f32", "f32", False, False, 0.7),
    (1, 3, 1, 64, "bf16", "f32", True, False, 1.0),
    (1, 1, 130, 128, "bf16", "bf16", True, True, 2.0),
    (3, 2, 200, 128, "f32", "bf16", True, True, 4.0),
]


@pytest.mark.parametrize("case", SERIAL_CASES, ids=lambda c: "x".join(map(str, c)))
def test_serial_scan(case):
    check(case, chunk=1)


CHUNK_CASES = [
    (1, 2, 64, 128, "bf16", "f32", True, True, 2.0),
    (2, 1, 1, 128, "bf16", "f32", True, True, 2.0),
    (1, 1, 63, 64, "bf16", "f32", False, False, 1.0),
    (1, 2, 65, 128, "bf16", "f32", True, False, 2.0),
    (2, 2, 333, 128, "bf16", "bf16", True, True, 4.0),
    (1, 3, 1000, 64, "bf16", "bf16", True, True, 2.0),
    (3, 1, 130, 64, "bf16", "f32", False, True, 0.5),
    (1, 1, 1024, 128, "bf16", "f32", False, True, 8.0),
]


@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: "x".join(map(str, c)))
def test_chunk_scan(case):
    check(case, chunk=64)


def test_chunk_and_serial_agree():
    """The two GPU forms of the scan on the same bf16 keys."""
    say("precond_scan chunk vs serial")
    k, beta, r, d1 = inputs(2, 2, 517, 128, "bf16", seed=11)
    dc, nc = run_gpu(k, beta, r, d1, 2.0, "bf16", "f32", 64)
    ds, ns = run_gpu(k, beta, r, d1, 2.0, "bf16", "f32", 1)
    assert rel_err(dc, ds) <= TOL_CHUNK["f32"] and rel_err(nc, ns) <= TOL_CHUNK_STATE


def test_zero_length_copies_start_state():
    torch, dev = torch_dev()
    say("precond_scan T=0")
    d1 = torch.arange(2 * 128, dtype=torch.float32, device=dev).reshape(1, 2, 128)
    k = torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device=dev)
    beta = torch.zeros((1, 2, 0), dtype=torch.float32, device=dev)
    for chunk in (1, 64):
        d, dn = osdn.osdn_precond_scan(k, beta, None, d1, eta=1.0, chunk=chunk)
        torch.cuda.synchronize()
        assert d.shape == (1, 2, 0, 128) and torch.equal(dn, d1)


@pytest.mark.parametrize("chunk", [1, 64])
def test_in_place_carry_and_split(chunk):
    """Running T1 then T2 tokens, carrying d_next in place over d1, equals one run of T1 + T2
    (to rounding for the chunkwise form: the chunk boundaries move)."""
    torch, dev = torch_dev()
    say("precond_scan split", chunk)
    k, beta, r, d1 = inputs(1, 2, 300, 128, "bf16", seed=12)
    d_all, n_all = run_gpu(k, beta, r, d1, 2.0, "bf16", "f32", chunk)
    state = to_dev(d1, "f32")
    outs = []
    for lo, hi in ((0, 100), (100, 300)):
        d, _ = osdn.osdn_precond_scan(to_dev(k[:, :, lo:hi], "bf16"),
                                      to_dev(beta[:, :, lo:hi], "f32"),
                                      to_dev(r[:, :, lo:hi], "f32"), state, eta=2.0,
                                      chunk=chunk, d_next=state)
        outs.append(to_np(d))
    torch.cuda.synchronize()
    d_split, n_split = np.concatenate(outs, axis=2), to_np(state)
    if chunk == 1:
        assert np.array_equal(d_split, d_all) and np.array_equal(n_split, n_all)
    else:
        assert rel_err(d_split, d_all) <= TOL_CHUNK["f32"]
        assert rel_err(n_split, n_all) <= TOL_CHUNK_STATE


@pytest.mark.parametrize("chunk", [1, 64])
def test_output_stays_in_bounds(chunk):
    """d is the head of a larger buffer whose tail holds a sentinel; T is ragged."""
    torch, dev = torch_dev()
    say("precond_scan bounds", chunk)
    B, H, T, dk = 2, 3, 70, 128
    k, beta, r, d1 = inputs(B, H, T, dk, "bf16", seed=13)
    n = B * H * T * dk
    buf = torch.full((n + 4096,), 7.0, dtype=torch.float32, device=dev)
    d = buf[:n].view(B, H, T, dk)
    osdn.osdn_precond_scan(to_dev(k, "bf16"), to_dev(beta, "f32"), to_dev(r, "f32"),
                           to_dev(d1, "f32"), eta=2.0, chunk=chunk, d=d)
    torch.cuda.synchronize()
    assert torch.all(buf[n:] == 7.0)
    d_ref, _ = precond.precond_scan(k, beta, 2.0, r, d1)
    assert rel_err(to_np(d), d_ref) <= TOL_CHUNK["f32"]


@pytest.mark.parametrize("kdt,ddt", [("bf16", "f32"), ("f32", "bf16")])
def test_decode_step_chain_equals_scan(kdt, ddt):
    """osdn_precond_step, one token at a time with the state in place, gives the serial scan
    bit for bit and the oracle to its bound."""
    torch, dev = torch_dev()
    say("precond_step chain", kdt, ddt)
    B, H, T, dk = 4, 2, 40, 128
    k, beta, r, d1 = inputs(B, H, T, dk, kdt, seed=14)
    d_scan, n_scan = run_gpu(k, beta, r, d1, 2.0, kdt, ddt, 1)
    state = to_dev(d1, "f32")
    kd, bd, rd = to_dev(k, kdt), to_dev(beta, "f32"), to_dev(r, "f32")
    outs = []
    for t in range(T):
        outs.append(to_np(osdn.osdn_precond_step(
            kd[:, :, t].contiguous(), bd[:, :, t].contiguous(), rd[:, :, t].contiguous(),
            state, eta=2.0, d_dtype={"f32": torch.float32, "bf16": torch.bfloat16}[ddt])))
    torch.cuda.synchronize()
    d_step = np.stack(outs, axis=2)
    assert np.array_equal(d_step, d_scan) and np.array_equal(to_np(state), n_scan)
    d_ref, n_ref = precond.precond_scan(k, beta, 2.0, r, d1)
    assert rel_err(d_step, d_ref) <= TOL_SERIAL[ddt]
    assert rel_err(to_np(state), n_ref) <= TOL_SERIAL["f32"]


def test_phase1_then_phase2_end_to_end():
    """Phase 1 on the GPU feeds Phase 2 on the GPU; the oracle runs both phases in float64."""
    import oracle
    torch, dev = torch_dev()
    say("precond_scan -> chunk_fwd")
    B, H, T, dk, dv = 1, 2, 260, 128, 128
    x = synth.make_shape(B, H, T, dk, dv, qkv="bf16", alpha=True, s0=True, seed=15)
    g = synth.make_precond_gates(B, H, T, dk, seed=15)
    d, _ = osdn.osdn_precond_scan(to_dev(x["k"], "bf16"), to_dev(x["beta"], "f32"),
                                  to_dev(g["r"], "f32"), to_dev(g["d1"], "f32"),
                                  eta=synth.PRECOND_ETA, chunk=64)
    o, S = osdn.osdn_chunk_fwd(to_dev(x["q"], "bf16"), to_dev(x["k"], "bf16"),
                               to_dev(x["v"], "bf16"), to_dev(x["beta"], "f32"), d,
                               to_dev(x["alpha"], "f32"), to_dev(x["S0"], "f32"))
    torch.cuda.synchronize()
    d_ref, _ = precond.precond_scan(x["k"], x["beta"], synth.PRECOND_ETA, g["r"], g["d1"])
    o_ref, S_ref = oracle.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], d_ref, x["alpha"],
                                    x["S0"])
    eo, es = rel_err(to_np(o), o_ref), rel_err(to_np(S), S_ref)
    say(f"  e_o={eo:.3e} e_S={es:.3e}")
    assert eo <= 2e-2 and es <= 2e-2


@pytest.mark.parametrize("name", ["1.3b", "long"])
def test_full_size_workload(name):
    """The scan at the full size of the model-shaped and long-context workloads (keys and gates
    of the workload), in the launch configuration the benchmark times, whole output compared."""
    w = synth.WORKLOADS[name]
    say("precond_scan full", name)
    x = synth.make_inputs(w)
    g = synth.make_precond_gates(w.B, w.H, w.T, w.dk, seed=w.seed)
    d, dn = run_gpu(x["k"], x["beta"], g["r"], g["d1"], synth.PRECOND_ETA, "bf16", "f32", 64)
    d_ref, dn_ref = precond.precond_scan(x["k"], x["beta"], synth.PRECOND_ETA, g["r"], g["d1"])
    e_d, e_n = rel_err(d, d_ref), rel_err(dn, dn_ref)
    say(f"  e_d={e_d:.3e} e_next={e_n:.3e}")
    assert e_d <= TOL_CHUNK["f32"] and e_n <= TOL_CHUNK_STATE
