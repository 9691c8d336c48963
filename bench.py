#!/usr/bin/env python3
"""Benchmark of libosdn on one MI355X.

One step = one osdn_chunk_fwd call over the 1.3B-shape workload (B=4, H=16, T=4096,
dk=dv=128, chunk 64, bf16 q/k/v/o, fp32 beta/d/alpha, fp32 final state emitted), i.e. one
pass of the whole chunkwise hot path over one batch of synthetic input already resident in
HBM.  Prints ONE JSON line.  Besides the contract fields it carries:

  roofline      the chunk kernel against HBM: algorithmic bytes per launch / average
                launch time from HIP events on the launch stream (peak 8 TB/s); `traffic` is
                the rocprofv3 FETCH_SIZE/WRITE_SIZE figure stored under profiles/ for the same
                kernel source (null once the source has changed);
  mfma          algorithmic FLOPs per launch / launch time against the bf16 dense peak;
  cpu_baseline  the float64 oracle on the host cores, same workload, with the parity error
                of the GPU output against it (whole tensor and worst single sequence), and
                the oracle's single-core rate on one sequence;
  configs       the same figures (time per step, tokens/s, TFLOP/s, both roofline
                fractions, parity, oracle timing) for the other forward workloads: tiny
                (fp32), 340m and long;
  decode        osdn_step over the decode workload (B=128, H=16, dk=dv=128), timed over
                `--decode-steps` consecutive calls (state updated in place), and a control
                that rotates the calls over four distinct 128 MiB states (512 MiB, more
                than the 256 MB Infinity Cache holds);
  precond_scan  the Phase-1 preconditioner scan (osdn_precond_scan, chunkwise form) over the
                same workload's keys and gates, with its own HBM roofline, its oracle timed on
                the host, and the forward with the scan in front (scan + chunkwise forward);
  kda           the forward with the channel-wise gate (osdn_chunk_fwd_kda: the chunk planes
                kernel, then the chunkwise forward) on the same workload with a per-feature
                gate, with its HBM roofline and the parity of its output;
  bwd           the backward (osdn_chunk_bwd: forward state checkpoints, the chunk inverses, the
                reverse pass over chunks, the per-chunk gradients) on the same workload with
                seeded output gradients, with its HBM roofline, its matrix-core FLOP count, and
                the float64 reverse pass on one sampled sequence (parity and CPU baseline);
  kda_bwd       the backward with the channel-wise gate (osdn_chunk_bwd_kda: the score tiles and
                their inverse, the fp32 forward recording chunk-start states, the reverse pass,
                the per-chunk gradients) on the
                same workload with the channel gate of `kda`, its HBM roofline, and the float64
                reverse pass on one sampled sequence (parity and CPU baseline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "tokens/s + TFLOP/s (fraction of bf16 MFMA peak), OSDN chunkwise fwd"
PEAK_HBM = 8.0e12      # bytes/s, MI355X HBM3E
PEAK_BF16 = 2.5e15     # FLOP/s, MI355X dense bf16 matrix peak
_CSRC = "delta_rule_sequence_chunkwise_amd/csrc/"
CHUNK_KERNEL_SRC = [_CSRC + f for f in ("osdn_chunk_mfma.hip", "osdn_mfma.h", "osdn_internal.h")]
STEP_KERNEL_SRC = [_CSRC + f for f in ("osdn_step.hip", "osdn_internal.h")]
KDA_KERNEL_SRC = [_CSRC + f for f in ("osdn_kda.hip", "osdn_chunk_mfma.hip", "osdn_mfma.h",
                                      "osdn_internal.h")]
PRECOND_KERNEL_SRC = [_CSRC + f for f in ("osdn_precond.hip", "osdn_mfma.h", "osdn_internal.h")]


def flops_per_head_token(dk, dv, C):
    """Chunkwise FLOPs per head-token counting only the useful triangular halves: the three
    state products (W M or K M, Q M, K~^T U) 6 dk dv; the Gram, P and the dk-side of the WY
    factors C (3 dk + 2 dv); the triangular inverse C^2 / 3."""
    return 6 * dk * dv + C * (3 * dk + 2 * dv) + C * C / 3.0


def bytes_per_head_token(dk, dv, eq, ed, alpha=True):
    """Compulsory HBM bytes per head-token: q, k, v in; d in; beta (and alpha) in; o out."""
    return (2 * dk + dv) * eq + dk * ed + 4 + (4 if alpha else 0) + dv * eq


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(name, paths):
    """Counter-measured HBM bytes per launch from profiles/<name>.json, if the kernel source
    has not changed since the counters were taken."""
    fn = os.path.join(ROOT, "profiles", f"{name}.json")
    if not os.path.exists(fn):
        return None
    with open(fn) as f:
        rec = json.load(f)
    if rec.get("source_hash") != source_hash(paths):
        return None
    return rec.get("traffic_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # Long enough for the board's clocks to settle: timed launch by launch at the 1.3B shape,
    # the forward takes ~150 us for its first ~10 launches, ~190 us around launch 20, and
    # settles at ~152 us after ~60 launches; the timed steps follow that transient.
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--precond-steps", type=int, default=20)
    ap.add_argument("--kda-steps", type=int, default=10)
    ap.add_argument("--bwd-steps", type=int, default=20)
    # untimed backward calls before each timed backward loop, past the clock transient that a
    # few calls leave the board in (five calls timed right after the other legs read ~20 %
    # slower than the settled figure)
    ap.add_argument("--bwd-warmup", type=int, default=20)
    ap.add_argument("--kda-bwd-steps", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="1.3b")
    ap.add_argument("--configs", default="tiny,340m,long",
                    help="other forward workloads measured beside the main one ('' for none)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (3 times): the "
                         "reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: libosdn has no multi-GPU path (the (b,h) "
              "sequences would shard across GPUs with no communication). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4, "copies": 3}), flush=True)
        return

    from delta_rule_sequence_chunkwise_amd import osdn, synth

    if not os.path.exists(osdn.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    cpu = not args.no_cpu_baseline
    main_rec, ctx = bench_forward(synth.WORKLOADS[args.workload], args.steps, args.warmup,
                                  torch, dev, cpu, keep=True)
    w, x = ctx["w"], ctx["x"]
    q, k, v, beta, d, alpha, S0, o, S_T = ctx["dev"]
    B, H, T = w.B, w.H, w.T

    line = {
        "metric": METRIC,
        "value": main_rec["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.qkv,
        "data": "synthetic (seeded generator; q,k unit-norm, v normal, beta sigmoid, "
                "d log-normal, alpha in (0.86, 0.995))",
        "config": main_rec["config"],
    }
    for key in ("head_tokens_per_s", "tflops", "mfma", "roofline", "cpu_baseline", "parity"):
        if key in main_rec:
            line[key] = main_rec[key]
    line["roofline"]["traffic"] = load_traffic("chunk_fwd_1.3b_traffic", CHUNK_KERNEL_SRC) \
        if w.name == "1.3b" else None
    line["roofline"]["traffic_source"] = (
        "profiles/chunk_fwd_1.3b_traffic.json: rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 "
        "per launch (factors from a plain copy), taken on the same kernel source; null when "
        "the source has changed since")

    if args.configs:
        line["configs"] = {}
        for name in args.configs.split(","):
            if name and name != w.name:
                steps = max(3, args.steps // 4) if name == "long" else args.steps
                rec, _ = bench_forward(synth.WORKLOADS[name], steps, args.warmup, torch, dev, cpu)
                line["configs"][name] = rec

    if args.decode_steps > 0:
        line["decode"] = bench_decode(args.decode_steps, torch, dev, synth)

    if args.precond_steps > 0:
        line["precond_scan"] = bench_precond(args.precond_steps, torch, dev, synth, w, x,
                                             (q, k, v, beta, alpha, S0, o, S_T),
                                             not args.no_cpu_baseline)

    if args.kda_steps > 0:
        line["kda"] = bench_kda(args.kda_steps, torch, dev, synth, w, x, (q, k, v, beta, d, S0),
                                not args.no_cpu_baseline)

    if args.bwd_steps > 0:
        line["bwd"] = bench_bwd(args.bwd_steps, args.bwd_warmup, torch, dev, synth, w, x,
                                (q, k, v, beta, d, alpha, S0), not args.no_cpu_baseline)

    if args.kda_bwd_steps > 0:
        line["kda_bwd"] = bench_kda_bwd(args.kda_bwd_steps, torch, dev, synth, w, x,
                                        (q, k, v, beta, d, S0), not args.no_cpu_baseline)

    print(json.dumps(line), flush=True)


def bench_forward(w, n_steps, warmup, torch, dev, cpu, keep=False):
    """Times osdn_chunk_fwd on workload `w`: `warmup` untimed calls, then `n_steps` calls
    bracketed by HIP events on the launch stream (and the host clock).  With `cpu`, the float64
    oracle runs on the same inputs on all host cores (parity of the GPU output, whole tensor and
    worst single sequence) and on one core over one sequence."""
    import numpy as np
    import oracle
    from delta_rule_sequence_chunkwise_amd import osdn, synth

    x = synth.make_inputs(w)
    qdt = torch.bfloat16 if w.qkv == "bf16" else torch.float32
    to = lambda a, dt: None if a is None else torch.from_numpy(a).to(dev).to(dt)
    q, k, v = (to(x[n], qdt) for n in ("q", "k", "v"))
    beta, d, alpha, S0 = (to(x[n], torch.float32) for n in ("beta", "d", "alpha", "S0"))
    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    o = torch.empty((B, H, T, dv), dtype=qdt, device=dev)
    S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)

    def step():
        osdn.osdn_chunk_fwd(q, k, v, beta, d, alpha, S0, chunk=w.chunk, o=o, S_T=S_T)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(n_steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_s = (t1 - t0) / n_steps
    launch_s = ev0.elapsed_time(ev1) / 1e3 / n_steps

    head_tokens = B * H * T
    eq = 2 if w.qkv == "bf16" else 4
    alg_bytes = head_tokens * bytes_per_head_token(dk, dv, eq, 4, alpha is not None) \
        + B * H * dk * dv * 4 * (2 if S0 is not None else 1)
    alg_flops = head_tokens * flops_per_head_token(dk, dv, w.chunk)
    t_floor = max(alg_bytes / PEAK_HBM, alg_flops / PEAK_BF16)
    rec = {
        "config": {"workload": f"{w.name}-shape OSDN chunkwise forward: B={B} H={H} T={T} "
                               f"dk={dk} dv={dv} chunk={w.chunk}, {w.qkv} q/k/v/o, fp32 "
                               f"beta/d{'/alpha' if alpha is not None else ''}, fp32 final "
                               "state",
                   "B": B, "H": H, "T": T, "dk": dk, "dv": dv, "chunk": w.chunk},
        "ms_per_step": round(wall_s * 1e3, 4),
        "launch_ms": round(launch_s * 1e3, 4),
        "tokens_per_s": round(B * T / wall_s, 1),
        "head_tokens_per_s": round(head_tokens / wall_s, 1),
        "tflops": round(alg_flops / launch_s / 1e12, 3),
        "mfma": {"achieved": round(alg_flops / launch_s / 1e12, 3), "peak": PEAK_BF16 / 1e12,
                 "unit": "TFLOP/s", "frac": round(alg_flops / launch_s / PEAK_BF16, 5),
                 "flops_per_launch": alg_flops},
        "roofline": {"bound": "hbm", "achieved": round(alg_bytes / launch_s / 1e9, 2),
                     "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": round(alg_bytes / launch_s / PEAK_HBM, 5),
                     "alg_bytes_per_launch": alg_bytes, "launch_ms": round(launch_s * 1e3, 4),
                     "frac_of_binding_floor": round(t_floor / launch_s, 5)},
    }
    if cpu:
        nt = oracle.default_threads()
        c0 = time.perf_counter()
        o_ref, S_ref = oracle.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["d"],
                                        x["alpha"], x["S0"], nthreads=nt)
        cpu_s = time.perf_counter() - c0
        one = lambda a: None if a is None else np.ascontiguousarray(a[:1, :1])
        c1 = time.perf_counter()
        oracle.chunk_fwd(one(x["q"]), one(x["k"]), one(x["v"]), one(x["beta"]), one(x["d"]),
                         one(x["alpha"]), one(x["S0"]), nthreads=1)
        one_s = time.perf_counter() - c1
        o_gpu = o.float().cpu().numpy()
        S_gpu = S_T.cpu().numpy()
        rel = lambda a, b: float(np.max(np.abs(a - b)) / np.max(np.abs(b)))
        worst = lambda a, b: max(rel(a[i, j], b[i, j]) for i in range(B) for j in range(H))
        rec["cpu_baseline"] = {"value": round(B * T / cpu_s, 1), "unit": "tokens/s",
                               "cores": nt, "kind": "oracle",
                               "sample": f"the whole {w.name} workload ({B * H} sequences x "
                                         f"{T} tokens), float64 C recurrence, {cpu_s:.2f} s "
                                         "wall",
                               "single_core": {"value": round(T / one_s, 1),
                                               "unit": "head-tokens/s", "cores": 1,
                                               "sample": f"one sequence ({T} tokens), "
                                                         f"{one_s:.2f} s wall"}}
        rec["parity"] = {"e_o": rel(o_gpu, o_ref), "e_S": rel(S_gpu, S_ref),
                         "worst_sequence_e_o": worst(o_gpu, o_ref),
                         "worst_sequence_e_S": worst(S_gpu, S_ref),
                         "tol": 2e-2 if w.qkv == "bf16" else 1e-4}
        del o_ref, S_ref
    ctx = {"w": w, "x": x, "dev": (q, k, v, beta, d, alpha, S0, o, S_T)} if keep else None
    return rec, ctx


def bwd_flops_per_head_token(dk, dv, C):
    """FLOPs per head-token of the backward launches, counting useful triangular halves: the
    forward recompute (the forward's count), the reverse pass with the chunk inverses (K~ dM,
    Q^T dO, K^T dR: 3 dk dv MACs; P^T dO and T^T dU: C dv; the Gram and P: C dk) and the
    per-chunk pass (K M0, Q M0, K~ dMC and the three dk x dv gradient products: 6 dk dv; T R,
    T^T dU, P^T dO, dP and dA: 2.5 C dv; the Gram, P and the four C-contractions: 3 C dk).
    Split-precision products count once."""
    fwd = flops_per_head_token(dk, dv, C)
    rev = 2 * (3 * dk * dv + C * dv + C * dk)
    per_chunk = 2 * (6 * dk * dv + 2.5 * C * dv + 3 * C * dk)
    return fwd + rev + per_chunk


def bench_bwd(n_steps, n_warm, torch, dev, synth, w, x, fwd, cpu):
    """Times `n_steps` osdn_chunk_bwd calls on the workload (output gradients seeded), after
    `n_warm` untimed ones."""
    import numpy as np
    from delta_rule_sequence_chunkwise_amd import osdn

    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    q, k, v, beta, d, alpha, S0 = fwd
    gr = synth.make_output_grads(B, H, T, dk, dv, qkv=w.qkv, seed=w.seed, state=True)
    do = torch.from_numpy(gr["do"]).to(dev).to(q.dtype)
    dS_T = torch.from_numpy(gr["dS_T"]).to(dev)
    ws = torch.empty(osdn.bwd_workspace_bytes(B, H, T, dk, dv, osdn.OSDN_BF16),
                     dtype=torch.uint8, device=dev)
    grads = osdn.osdn_chunk_bwd(q, k, v, beta, d, alpha, S0, do, dS_T, workspace=ws)
    for _ in range(n_warm):
        osdn.osdn_chunk_bwd(q, k, v, beta, d, alpha, S0, do, dS_T, grads=grads, workspace=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n_steps):
        osdn.osdn_chunk_bwd(q, k, v, beta, d, alpha, S0, do, dS_T, grads=grads, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    per = e0.elapsed_time(e1) / 1e3 / n_steps
    # the training pair: the forward that keeps the chunk-start states, and the backward that
    # takes them (no forward recompute inside)
    o_buf, st_buf, states = osdn.osdn_chunk_fwd_states(q, k, v, beta, d, alpha, S0)
    for _ in range(max(1, n_warm)):
        osdn.osdn_chunk_fwd_states(q, k, v, beta, d, alpha, S0, o=o_buf, S_T=st_buf, states=states)
        osdn.osdn_chunk_bwd(q, k, v, beta, d, alpha, S0, do, dS_T, grads=grads, workspace=ws,
                            states=states)
    torch.cuda.synchronize()
    e2 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n_steps):
        osdn.osdn_chunk_fwd_states(q, k, v, beta, d, alpha, S0, o=o_buf, S_T=st_buf, states=states)
    e1.record(stream)
    for _ in range(n_steps):
        osdn.osdn_chunk_bwd(q, k, v, beta, d, alpha, S0, do, dS_T, grads=grads, workspace=ws,
                            states=states)
    e2.record(stream)
    torch.cuda.synchronize()
    fwd_states_ms = e0.elapsed_time(e1) / n_steps
    bwd_states_ms = e1.elapsed_time(e2) / n_steps
    head_tokens = B * H * T
    eq = 2 if w.qkv == "bf16" else 4
    # in: q, k, v, do (qkv type), d (fp32), beta, alpha; out: grad q, k, v (qkv type), grad d
    # (fp32), grad beta, alpha; per sequence: S0 and dS_T in, grad S0 out (fp32)
    alg = head_tokens * ((2 * dk + 2 * dv) * eq + dk * 4 + 8 + (2 * dk + dv) * eq + dk * 4 + 8) \
        + B * H * dk * dv * 4 * 3
    flops = head_tokens * bwd_flops_per_head_token(dk, dv, 64)
    rec = {"workload": f"{w.name}-shape backward: B={B} H={H} T={T} dk={dk} dv={dv}, bf16 "
                       "q/k/v/do and gradients of q/k/v, fp32 beta/d/alpha and their gradients, "
                       "fp32 S0, dS_T and grad S0",
           "ms_per_step": round(per * 1e3, 4),
           "tokens_per_s": round(B * T / per, 1),
           "training_pair": {"fwd_states_ms": round(fwd_states_ms, 4),
                             "bwd_from_states_ms": round(bwd_states_ms, 4),
                             "step_ms": round(fwd_states_ms + bwd_states_ms, 4),
                             "note": "osdn_chunk_fwd_states (o, S_T and the chunk-start states) "
                                     "then osdn_chunk_bwd_states (no forward recompute)"},
           "roofline": {"bound": "hbm", "achieved": round(alg / per / 1e9, 2),
                        "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                        "frac": round(alg / per / PEAK_HBM, 5), "alg_bytes_per_step": alg,
                        "note": "four launches; the state checkpoints (bf16, 2 x 134 MB written "
                                "and read), the chunk planes (168 MB) and U and dR (67 MB "
                                "each) are beyond alg"},
           "mfma": {"achieved": round(flops / per / 1e12, 3), "peak": PEAK_BF16 / 1e12,
                    "unit": "TFLOP/s", "frac": round(flops / per / PEAK_BF16, 5),
                    "flops_per_step": flops,
                    "note": "useful FLOPs; the products run on bf16 matrix cores"}}
    if cpu:
        from oracle import backward
        b, h = 0, 0
        sl = lambda a: None if a is None else np.ascontiguousarray(a[b:b + 1, h:h + 1])
        c0 = time.perf_counter()
        ref = backward.chunk_bwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["beta"]), sl(x["d"]),
                                 sl(x["alpha"]), sl(x["S0"]), sl(gr["do"]), sl(gr["dS_T"]))
        cpu_s = time.perf_counter() - c0
        rel = lambda p, r: float(np.max(np.abs(p - r)) / np.max(np.abs(r)))
        par = {}
        for n, gn in (("dq", "grad_q"), ("dk", "grad_k"), ("dv", "grad_v"), ("dbeta", "grad_beta"),
                      ("dd", "grad_d"), ("dalpha", "grad_alpha"), ("dS0", "grad_S0")):
            par[n] = rel(grads[gn][b:b + 1, h:h + 1].float().cpu().numpy(), ref[n])
        par["tol"] = 2e-2
        rec["parity"] = par
        rec["cpu_baseline"] = {"value": round(T / cpu_s, 1), "unit": "head-tokens/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"one (b,h) sequence of the workload ({T} tokens), "
                                         f"float64 numpy reverse pass, {cpu_s:.2f} s wall"}
    return rec


def bench_kda_bwd(n_steps, torch, dev, synth, w, x, fwd, cpu):
    """Times `n_steps` osdn_chunk_bwd_kda calls on the workload with the channel-wise gate of
    bench_kda (output gradients seeded as in bench_bwd)."""
    import numpy as np
    from delta_rule_sequence_chunkwise_amd import osdn

    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    q, k, v, beta, d, S0 = fwd
    a_np = synth.make_channel_gate(B, H, T, dk, seed=w.seed)
    a = torch.from_numpy(a_np).to(dev)
    gr = synth.make_output_grads(B, H, T, dk, dv, qkv=w.qkv, seed=w.seed, state=True)
    do = torch.from_numpy(gr["do"]).to(dev).to(q.dtype)
    dS_T = torch.from_numpy(gr["dS_T"]).to(dev)
    ws = torch.empty(osdn.bwd_kda_workspace_bytes(B, H, T, dk, dv, osdn.OSDN_BF16),
                     dtype=torch.uint8, device=dev)
    grads = osdn.osdn_chunk_bwd_kda(q, k, v, beta, d, a, S0, do, dS_T, workspace=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n_steps):
        osdn.osdn_chunk_bwd_kda(q, k, v, beta, d, a, S0, do, dS_T, grads=grads, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    per = e0.elapsed_time(e1) / 1e3 / n_steps
    head_tokens = B * H * T
    eq = 2 if w.qkv == "bf16" else 4
    # in: q, k, v, do (qkv type), d and the gate (fp32), beta; out: grads of q, k, v (qkv type),
    # of d and the gate (fp32), of beta; per sequence: S0 and dS_T in, grad S0 out (fp32)
    alg = head_tokens * ((2 * dk + 2 * dv) * eq + 2 * dk * 4 + 4 + (2 * dk + dv) * eq
                         + 2 * dk * 4 + 4) + B * H * dk * dv * 4 * 3
    rec = {"workload": f"{w.name}-shape backward with a channel-wise gate a[B,H,T,dk]: B={B} "
                       f"H={H} T={T} dk={dk} dv={dv}, bf16 q/k/v/do and gradients of q/k/v, "
                       "fp32 beta/d/gate and their gradients, fp32 S0, dS_T and grad S0",
           "ms_per_step": round(per * 1e3, 4),
           "tokens_per_s": round(B * T / per, 1),
           "roofline": {"bound": "hbm", "achieved": round(alg / per / 1e9, 2),
                        "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                        "frac": round(alg / per / PEAK_HBM, 5), "alg_bytes_per_step": alg,
                        "note": "four launches in fp32 (32-row chunks; the products of the "
                                "reverse and per-chunk passes on the fp32 matrix cores, the "
                                "per-feature decay of every score term formed in the product); "
                                "the fp32 state checkpoints (2 x 268 MB written and read) and "
                                "the chunk score tiles and inverse (101 MB) are beyond alg"}}
    if cpu:
        from oracle import backward
        b, h = 0, 0
        sl = lambda t: None if t is None else np.ascontiguousarray(t[b:b + 1, h:h + 1])
        c0 = time.perf_counter()
        ref = backward.chunk_bwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["beta"]), sl(x["d"]),
                                 None, sl(x["S0"]), sl(gr["do"]), sl(gr["dS_T"]),
                                 alpha_ch=sl(a_np))
        cpu_s = time.perf_counter() - c0
        rel = lambda p, r: float(np.max(np.abs(p - r)) / np.max(np.abs(r)))
        par = {}
        for n, gn in (("dq", "grad_q"), ("dk", "grad_k"), ("dv", "grad_v"), ("dbeta", "grad_beta"),
                      ("dd", "grad_d"), ("dalpha_ch", "grad_alpha_ch"), ("dS0", "grad_S0")):
            par[n] = rel(grads[gn][b:b + 1, h:h + 1].float().cpu().numpy(), ref[n])
        par["tol"] = 2e-2
        rec["parity"] = par
        rec["cpu_baseline"] = {"value": round(T / cpu_s, 1), "unit": "head-tokens/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"one (b,h) sequence of the workload ({T} tokens), "
                                         f"float64 numpy reverse pass, {cpu_s:.2f} s wall"}
    return rec


def bench_kda(n_steps, torch, dev, synth, w, x, fwd, cpu):
    """Times `n_steps` osdn_chunk_fwd_kda calls (gate scaling + forward) on the workload with a
    channel-wise gate in place of the scalar one."""
    import numpy as np
    from delta_rule_sequence_chunkwise_amd import osdn

    B, H, T, dk, dv = w.B, w.H, w.T, w.dk, w.dv
    q, k, v, beta, d, S0 = fwd
    a_np = synth.make_channel_gate(B, H, T, dk, seed=w.seed)
    a = torch.from_numpy(a_np).to(dev)
    o = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
    S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    ws = torch.empty(osdn.kda_workspace_bytes(B, H, T, dk, w.chunk, osdn.OSDN_BF16),
                     dtype=torch.uint8, device=dev)

    def step():
        osdn.osdn_chunk_fwd_kda(q, k, v, beta, d, a, S0, chunk=w.chunk, o=o, S_T=S_T,
                                workspace=ws)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(n_steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    per = e0.elapsed_time(e1) / 1e3 / n_steps
    head_tokens = B * H * T
    # q, k, v, o in bf16; d and the channel gate in fp32; beta; the final state
    alg = head_tokens * ((2 * dk + 2 * dv) * 2 + dk * 4 + dk * 4 + 4) \
        + B * H * dk * dv * 4 * (2 if S0 is not None else 1)
    rec = {"workload": f"{w.name}-shape forward with a channel-wise gate a[B,H,T,dk] in place "
                       f"of the scalar one: B={B} H={H} T={T} dk={dk} dv={dv}, bf16 q/k/v/o, fp32 "
                       "beta/d/gate, fp32 final state",
           "ms_per_step": round(per * 1e3, 4),
           "tokens_per_s": round(B * T / per, 1),
           "roofline": {"bound": "hbm", "achieved": round(alg / per / 1e9, 2),
                        "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                        "frac": round(alg / per / PEAK_HBM, 5), "alg_bytes_per_step": alg,
                        "traffic": load_traffic("kda_1.3b_traffic", KDA_KERNEL_SRC),
                        "note": "two launches: the planes kernel writes and the forward "
                                "reads the gate-scaled q, k, k~ and the chunk planes "
                                "(workspace traffic beyond alg); traffic is both launches' "
                                "rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0 from "
                                "profiles/kda_1.3b_traffic.json"}}
    if cpu:
        import oracle
        o_ref, S_ref = oracle.chunk_fwd(x["q"], x["k"], x["v"], x["beta"], x["d"], None,
                                        x["S0"], alpha_ch=a_np)
        rel = lambda p, r: float(np.max(np.abs(p - r)) / np.max(np.abs(r)))
        rec["parity"] = {"e_o": rel(o.float().cpu().numpy(), o_ref),
                         "e_S": rel(S_T.cpu().numpy(), S_ref), "tol": 2e-2}
    return rec


def bench_decode(n_steps, torch, dev, synth, distinct=64):
    """Times `n_steps` consecutive osdn_step calls on the decode workload.  The generator
    draws `distinct` per-step input tuples, used round-robin (the values do not change the
    kernel's cost); the state is carried in place from call to call."""
    from delta_rule_sequence_chunkwise_amd import osdn

    w = synth.WORKLOADS["decode"]
    n_in = min(distinct, n_steps)
    y = synth.make_decode_inputs(w, steps=n_in)
    to = lambda a, dt: torch.from_numpy(a).to(dev).to(dt)
    q, k, v = (to(y[n], torch.bfloat16) for n in ("q", "k", "v"))
    beta, d, alpha = (to(y[n], torch.float32) for n in ("beta", "d", "alpha"))
    S = to(y["S0"], torch.float32)
    BH = w.B * w.H
    o = torch.empty((n_in, w.B, w.H, w.dv), dtype=torch.bfloat16, device=dev)
    Sw = S.clone()
    for t in range(min(3, n_in)):  # warm-up on a scratch copy of the state
        osdn.osdn_step(q[t], k[t], v[t], beta[t], d[t], alpha[t], Sw, o=o[t])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for t in range(n_steps):
        i = t % n_in
        osdn.osdn_step(q[i], k[i], v[i], beta[i], d[i], alpha[i], S, o=o[i])
    ev1.record(stream)
    torch.cuda.synchronize()
    per = ev0.elapsed_time(ev1) / 1e3 / n_steps
    # control: the calls rotate over `nrot` distinct states, so each state is touched again
    # only after nrot - 1 others (nrot x 128 MiB, more than the 256 MB Infinity Cache holds)
    nrot = 4
    states = [S.clone() for _ in range(nrot)]
    for t in range(nrot):
        osdn.osdn_step(q[t], k[t], v[t], beta[t], d[t], alpha[t], states[t], o=o[t])
    torch.cuda.synchronize()
    ev0.record(stream)
    for t in range(n_steps):
        i = t % n_in
        osdn.osdn_step(q[i], k[i], v[i], beta[i], d[i], alpha[i], states[t % nrot], o=o[i])
    ev1.record(stream)
    torch.cuda.synchronize()
    per_rot = ev0.elapsed_time(ev1) / 1e3 / n_steps
    del states
    state_bytes = 2 * BH * w.dk * w.dv * 4
    io_bytes = BH * ((2 * w.dk + 2 * w.dv) * 2 + w.dk * 4 + 8)
    alg = state_bytes + io_bytes
    return {"workload": f"osdn_step B={w.B} H={w.H} dk={w.dk} dv={w.dv}, bf16 q/k/v/o, fp32 "
                        f"beta/d/alpha/state, {n_steps} consecutive steps over {n_in} "
                        "distinct input tuples",
            "us_per_step": round(per * 1e6, 3), "alg_bytes_per_step": alg,
            "achieved_GBps": round(alg / per / 1e9, 1),
            "frac_of_hbm_peak": round(alg / per / PEAK_HBM, 4),
            "traffic": load_traffic("step_decode_traffic", STEP_KERNEL_SRC),
            "traffic_source": "profiles/step_decode_traffic.json: rocprofv3 FETCH_SIZE x 2.0 + "
                              "WRITE_SIZE x 1.0 per launch (L2-to-fabric requests; Infinity "
                              "Cache hits are behind the fabric and count too)",
            "state_rotation": {"states": nrot, "footprint_MiB": nrot * state_bytes // 2 // (1 << 20),
                               "us_per_step": round(per_rot * 1e6, 3),
                               "achieved_GBps": round(alg / per_rot / 1e9, 1),
                               "frac_of_hbm_peak": round(alg / per_rot / PEAK_HBM, 4),
                               "note": "each call updates a different state, so a state is "
                                       "read again only after three others (384 MiB) were "
                                       "streamed: it cannot be served from the Infinity Cache"},
            "note": "in place, the 128 MiB state could stay in the 256 MB Infinity Cache, but the "
                    "kernel's state accesses are non-temporal; the state_rotation figure (four "
                    "states, 512 MiB) is free of the cache by construction"}


def bench_precond(n_steps, torch, dev, synth, w, x, fwd, cpu):
    """Times `n_steps` launches of the chunkwise Phase-1 scan over the workload's keys and
    gates (fp32 d out, final state out), then `n_steps` forwards with the scan in front."""
    import numpy as np
    from delta_rule_sequence_chunkwise_amd import osdn

    B, H, T, dk = w.B, w.H, w.T, w.dk
    g = synth.make_precond_gates(B, H, T, dk, seed=w.seed)
    eta = synth.PRECOND_ETA
    q, k, v, beta, alpha, S0, o, S_T = fwd
    r = torch.from_numpy(g["r"]).to(dev)
    d1 = torch.from_numpy(g["d1"]).to(dev)
    d = torch.empty((B, H, T, dk), dtype=torch.float32, device=dev)
    dn = torch.empty((B, H, dk), dtype=torch.float32, device=dev)

    def scan():
        osdn.osdn_precond_scan(k, beta, r, d1, eta=eta, chunk=w.chunk, d=d, d_next=dn)

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n_steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3 / n_steps

    per = timed(scan)
    head_tokens = B * H * T
    alg = head_tokens * (2 * dk + 8 + 4 * dk) + 2 * B * H * dk * 4
    d_gpu = d.cpu().numpy()

    def fwd_with_scan():
        scan()
        osdn.osdn_chunk_fwd(q, k, v, beta, d, alpha, S0, chunk=w.chunk, o=o, S_T=S_T)

    per_fwd = timed(fwd_with_scan)
    rec = {"workload": f"{w.name}-shape keys and gates: B={B} H={H} T={T} dk={dk}, chunk "
                       f"{w.chunk}, bf16 k, fp32 beta/r/d1, eta={eta}, fp32 d and final d out",
           "launch_ms": round(per * 1e3, 4),
           "head_tokens_per_s": round(head_tokens / per, 1),
           "roofline": {"bound": "hbm", "achieved": round(alg / per / 1e9, 2),
                        "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                        "frac": round(alg / per / PEAK_HBM, 5),
                        "traffic": load_traffic("precond_scan_1.3b_traffic",
                                                PRECOND_KERNEL_SRC),
                        "alg_bytes_per_launch": alg},
           "fwd_with_scan": {"ms_per_step": round(per_fwd * 1e3, 4),
                             "tokens_per_s": round(B * T / per_fwd, 1)}}
    if cpu:
        from oracle import precond
        c0 = time.perf_counter()
        d_ref, _ = precond.precond_scan(x["k"], x["beta"], eta, g["r"], g["d1"])
        cpu_s = time.perf_counter() - c0
        rec["cpu_baseline"] = {"value": round(head_tokens / cpu_s, 1), "unit": "head-tokens/s",
                               "cores": 1, "kind": "oracle",
                               "sample": f"the whole workload ({B * H} sequences x {T} tokens),"
                                         f" float64 numpy token loop, {cpu_s:.2f} s wall"}
        rec["parity"] = {"e_d": float(np.max(np.abs(d_gpu - d_ref)) / np.max(np.abs(d_ref))),
                         "tol": 3e-3}
    return rec


if __name__ == "__main__":
    main()
