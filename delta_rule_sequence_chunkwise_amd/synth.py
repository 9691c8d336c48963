"""Seeded synthetic inputs for the OSDN chunkwise forward and the recurrent decode step.

This module only draws random tensors and rounds them to the storage precision.  It holds
none of the method's arithmetic, so both the CPU oracle and the GPU path take their inputs
from here.

Recipe (the pages print no workload data; the model-level benchmarks they quote need trained
weights and datasets, so these synthetic tensors stand in for them):

* generator: ``numpy.random.Generator(PCG64(seed))``, float64 draws;
* draw order, each in the head-major layout ``[B, H, T, .]``: q, k, v, beta logits,
  log-d normals, alpha normals (alpha normals are drawn only when the decay is on);
* q, k ~ N(0, 1), then divided by their L2 norm over the feature axis (per b, h, t);
* v ~ N(0, 1);  beta = sigmoid(N(0, 1));  d = exp(sigma_d * N(0, 1));
* alpha = exp(-0.05 * softplus(N(0, 1)))  (per token and head, in (0.86, 0.995));
* every tensor is rounded to float32 (RNE); q/k/v of a bf16 workload are rounded again to
  bfloat16 (RNE) and kept as float32 arrays holding exactly bf16-representable values, so
  that the GPU copy (bf16) and the oracle copy (float64) hold the same numbers.

The Phase-1 preconditioner scan takes the workload's k and beta and, from a stream of its
own (seed + 7919, so the draws above are unchanged), its retention gate and start value:
r = exp(-0.01 * softplus(N(0, 1))) per token and head (in (0.97, 1)), d_1 = exp(0.25 N(0, 1))
per head and feature, both rounded to float32.  The meta step eta = 2 is a workload constant.

The channel-wise (KDA) gate a_t [B,H,T,dk] of the KDA variant comes from a stream of its own
(seed + 104729): a = exp(-0.05 * softplus(N(0, 1))) per token, head and key feature, i.e. the
scalar gate's recipe drawn per feature, rounded to float32.

The backward's output gradients come from a stream of their own (seed + 15485863): do ~ N(0, 1)
[B,H,T,dv] (rounded to the qkv type) and dS_T ~ N(0, 1) [B,H,dk,dv] (float32).

The decode workload draws its initial state first (S0 ~ N(0, 0.02^2), float32, stored as
M = S^T, i.e. ``[B, H, dk, dv]``), then the per-step tuples in the order above.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

BASE_SEED = 20260513


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload shape.  ``qkv`` is "f32" or "bf16"; beta, d, alpha are float32."""

    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    chunk: int = 64
    qkv: str = "bf16"
    alpha: bool = True
    s0: bool = False
    sigma_d: float = 0.25
    sigma_d_late: Optional[float] = None  # regime shift: used for t >= T // 2
    steps: int = 0  # >0 only for the decode workload
    seed_index: int = 0

    @property
    def seed(self) -> int:
        return BASE_SEED + self.seed_index


# The five workloads: the small case, the two model-shaped cases, long context and decode.
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", B=1, H=2, T=256, dk=64, dv=64, qkv="f32", alpha=False,
                     seed_index=0),
    "340m": Workload("340m", B=8, H=8, T=2048, dk=128, dv=128, seed_index=1),
    "1.3b": Workload("1.3b", B=4, H=16, T=4096, dk=128, dv=128, seed_index=2),
    "long": Workload("long", B=1, H=16, T=65536, dk=128, dv=128, sigma_d_late=0.75,
                     seed_index=3),
    "decode": Workload("decode", B=128, H=16, T=1, dk=128, dv=128, s0=True, steps=1024,
                       seed_index=4),
}


def round_f32(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 with round-to-nearest-even (numpy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_bf16(x32: np.ndarray) -> np.ndarray:
    """float32 -> nearest-even bfloat16, returned as float32 holding the bf16 value."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    bits = x32.view(np.uint32)
    bias = ((bits >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((bits + bias) & np.uint32(0xFFFF0000)).astype(np.uint32)
    return out.view(np.float32)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _draw_token_block(rng: np.random.Generator, lead: tuple, dk: int, dv: int, qkv: str,
                      alpha: bool, sigma_d) -> Dict[str, np.ndarray]:
    """Draw q, k, v, beta, d, alpha for a block of tokens with leading shape ``lead``."""
    q = _unit_rows(rng.standard_normal(lead + (dk,)))
    k = _unit_rows(rng.standard_normal(lead + (dk,)))
    v = rng.standard_normal(lead + (dv,))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(lead)))
    logd = rng.standard_normal(lead + (dk,))
    if callable(sigma_d):
        logd = logd * sigma_d(logd.shape)
    else:
        logd = logd * sigma_d
    d = np.exp(logd)
    out = {"q": round_f32(q), "k": round_f32(k), "v": round_f32(v),
           "beta": round_f32(beta), "d": round_f32(d), "alpha": None}
    if alpha:
        a = np.exp(-0.05 * np.logaddexp(0.0, rng.standard_normal(lead)))
        out["alpha"] = round_f32(a)
    if qkv == "bf16":
        for name in ("q", "k", "v"):
            out[name] = round_bf16(out[name])
    elif qkv != "f32":
        raise ValueError(f"unknown qkv dtype {qkv!r}")
    return out


def make_inputs(w: Workload, seed: Optional[int] = None, T: Optional[int] = None
                ) -> Dict[str, np.ndarray]:
    """Inputs of a chunkwise-forward workload.

    Returns float32 arrays q, k [B,H,T,dk], v [B,H,T,dv], beta [B,H,T], d [B,H,T,dk],
    alpha [B,H,T] or None, S0 [B,H,dk,dv] or None.  ``T`` overrides the workload length.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    T = w.T if T is None else T
    sigma = w.sigma_d
    if w.sigma_d_late is not None:
        half = T // 2
        late = w.sigma_d_late

        def sigma(shape, _half=half, _early=w.sigma_d, _late=late):
            s = np.full(shape, _early)
            s[:, :, _half:, :] = _late
            return s
    out = _draw_token_block(rng, (w.B, w.H, T), w.dk, w.dv, w.qkv, w.alpha, sigma)
    out["S0"] = None
    if w.s0:
        out["S0"] = round_f32(0.02 * rng.standard_normal((w.B, w.H, w.dk, w.dv)))
    return out


def make_decode_inputs(w: Workload, steps: Optional[int] = None, seed: Optional[int] = None,
                       B: Optional[int] = None, H: Optional[int] = None
                       ) -> Dict[str, np.ndarray]:
    """Inputs of the recurrent decode workload.

    Returns S0 [B,H,dk,dv] and per-step stacks q, k [steps,B,H,dk], v [steps,B,H,dv],
    beta, alpha [steps,B,H], d [steps,B,H,dk].
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    steps = w.steps if steps is None else steps
    B = w.B if B is None else B
    H = w.H if H is None else H
    S0 = round_f32(0.02 * rng.standard_normal((B, H, w.dk, w.dv)))
    per = [_draw_token_block(rng, (B, H), w.dk, w.dv, w.qkv, w.alpha, w.sigma_d)
           for _ in range(steps)]
    out = {"S0": S0}
    for name in ("q", "k", "v", "beta", "d", "alpha"):
        if per and per[0][name] is not None:
            out[name] = np.stack([p[name] for p in per])
        else:
            out[name] = None
    return out


def make_shape(B: int, H: int, T: int, dk: int, dv: int, *, qkv: str = "f32",
               alpha: bool = True, s0: bool = False, sigma_d: float = 0.25,
               seed: int = 0) -> Dict[str, np.ndarray]:
    """Inputs of an arbitrary shape, drawn by the same recipe (used by small parity cases)."""
    w = Workload("custom", B=B, H=H, T=T, dk=dk, dv=dv, qkv=qkv, alpha=alpha, s0=s0,
                 sigma_d=sigma_d, seed_index=0)
    return make_inputs(w, seed=BASE_SEED + 1000 + seed)


PRECOND_ETA = 2.0


def make_precond_gates(B: int, H: int, T: int, dk: int, seed: int) -> Dict[str, np.ndarray]:
    """Retention gate r [B,H,T] and start value d1 [B,H,dk] of the Phase-1 scan."""
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    r = np.exp(-0.01 * np.logaddexp(0.0, rng.standard_normal((B, H, T))))
    d1 = np.exp(0.25 * rng.standard_normal((B, H, dk)))
    return {"r": round_f32(r), "d1": round_f32(d1)}


def make_channel_gate(B: int, H: int, T: int, dk: int, seed: int) -> np.ndarray:
    """Channel-wise gate a [B,H,T,dk] (the scalar gate's recipe, one draw per key feature)."""
    rng = np.random.Generator(np.random.PCG64(seed + 104729))
    return round_f32(np.exp(-0.05 * np.logaddexp(0.0, rng.standard_normal((B, H, T, dk)))))


def make_channel_gate_uniform(B: int, H: int, T: int, dk: int, lo: float, hi: float,
                              seed: int) -> np.ndarray:
    """Channel-wise gate a [B,H,T,dk] ~ U(lo, hi), rounded to float32: the strong-decay and
    tiny-gate regimes (stream seed + 104723, apart from the other draws)."""
    rng = np.random.Generator(np.random.PCG64(seed + 104723))
    return round_f32(rng.uniform(lo, hi, (B, H, T, dk)))


def make_output_grads(B: int, H: int, T: int, dk: int, dv: int, *, qkv: str, seed: int,
                      state: bool = True) -> Dict[str, Optional[np.ndarray]]:
    """Output gradients for the backward: do [B,H,T,dv] ~ N(0,1) (rounded to the qkv type) and,
    when ``state``, dS_T [B,H,dk,dv] ~ N(0,1) (fp32), from a stream of their own (seed + 15485863)."""
    rng = np.random.Generator(np.random.PCG64(seed + 15485863))
    do = round_f32(rng.standard_normal((B, H, T, dv)))
    if qkv == "bf16":
        do = round_bf16(do)
    dS_T = round_f32(rng.standard_normal((B, H, dk, dv))) if state else None
    return {"do": do, "dS_T": dS_T}
