"""Python binding of libosdn: argument marshalling over the C ABI of include/osdn.h.

Every step of the computation runs in the library's HIP kernels; this module only checks
tensor types, allocates outputs with torch (device memory is torch's), and passes raw device
pointers and the current HIP stream.  If libosdn.so has not been built, importing the
library raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libosdn.so")

OSDN_F32 = 0
OSDN_BF16 = 1
ABI_VERSION = 6

STATUS = {0: "OSDN_OK", -1: "OSDN_ERR_NULL", -2: "OSDN_ERR_SHAPE", -3: "OSDN_ERR_UNSUPPORTED",
          -4: "OSDN_ERR_ALIGN", -5: "OSDN_ERR_ALIAS", -6: "OSDN_ERR_LAUNCH",
          -7: "OSDN_ERR_SCRATCH"}
EXPORTS = ("osdn_chunk_fwd", "osdn_step", "osdn_precond_scan", "osdn_precond_step",
           "osdn_chunk_fwd_kda", "osdn_chunk_fwd_kda_workspace", "osdn_chunk_fwd_kda_noalloc",
           "osdn_step_kda",
           "osdn_chunk_bwd", "osdn_chunk_bwd_workspace", "osdn_chunk_bwd_states_workspace",
           "osdn_chunk_states_bytes",
           "osdn_chunk_fwd_states", "osdn_chunk_bwd_states",
           "osdn_chunk_bwd_kda", "osdn_chunk_bwd_kda_workspace", "osdn_status_string",
           "osdn_abi_version")


class OSDNError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status_string(status)})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libosdn.so (raises if it is missing or has another ABI version)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libosdn.so is not built ({LIB_PATH}); run "
                          "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.osdn_chunk_fwd.restype = ctypes.c_int
    L.osdn_chunk_fwd.argtypes = [vp] * 9 + [i64, i64, i64, i32, i32, i32, ctypes.c_int,
                                             ctypes.c_int, vp]
    L.osdn_step.restype = ctypes.c_int
    L.osdn_step.argtypes = [vp] * 8 + [i64, i64, i32, i32, ctypes.c_int, ctypes.c_int, vp]
    L.osdn_precond_scan.restype = ctypes.c_int
    L.osdn_precond_scan.argtypes = [vp] * 4 + [ctypes.c_float, vp, vp, i64, i64, i64, i32, i32,
                                               ctypes.c_int, ctypes.c_int, vp]
    L.osdn_precond_step.restype = ctypes.c_int
    L.osdn_precond_step.argtypes = [vp] * 5 + [ctypes.c_float, i64, i64, i32, ctypes.c_int,
                                               ctypes.c_int, vp]
    L.osdn_chunk_fwd_kda_workspace.restype = i64
    L.osdn_chunk_fwd_kda_workspace.argtypes = [i64, i64, i64, i32, i32, ctypes.c_int]
    L.osdn_chunk_fwd_kda.restype = ctypes.c_int
    L.osdn_chunk_fwd_kda.argtypes = [vp] * 10 + [i64, i64, i64, i64, i32, i32, i32, ctypes.c_int,
                                                 ctypes.c_int, vp]
    L.osdn_chunk_fwd_kda_noalloc.restype = ctypes.c_int
    L.osdn_chunk_fwd_kda_noalloc.argtypes = [vp] * 9 + [i64, i64, i64, i32, i32, i32,
                                                          ctypes.c_int, ctypes.c_int, vp]
    L.osdn_step_kda.restype = ctypes.c_int
    L.osdn_step_kda.argtypes = [vp] * 8 + [i64, i64, i32, i32, ctypes.c_int, ctypes.c_int, vp]
    L.osdn_chunk_bwd_workspace.restype = i64
    L.osdn_chunk_bwd_workspace.argtypes = [i64, i64, i64, i32, i32, ctypes.c_int]
    L.osdn_chunk_bwd_states_workspace.restype = i64
    L.osdn_chunk_bwd_states_workspace.argtypes = [i64, i64, i64, i32, i32, ctypes.c_int]
    L.osdn_chunk_bwd.restype = ctypes.c_int
    L.osdn_chunk_bwd.argtypes = [vp] * 17 + [i64, i64, i64, i64, i32, i32, ctypes.c_int,
                                             ctypes.c_int, vp]
    L.osdn_chunk_states_bytes.restype = i64
    L.osdn_chunk_states_bytes.argtypes = [i64, i64, i64, i32, i32, ctypes.c_int]
    L.osdn_chunk_fwd_states.restype = ctypes.c_int
    L.osdn_chunk_fwd_states.argtypes = [vp] * 10 + [i64, i64, i64, i32, i32, ctypes.c_int,
                                                    ctypes.c_int, vp]
    L.osdn_chunk_bwd_states.restype = ctypes.c_int
    L.osdn_chunk_bwd_states.argtypes = [vp] * 18 + [i64, i64, i64, i64, i32, i32, ctypes.c_int,
                                                    ctypes.c_int, vp]
    L.osdn_chunk_bwd_kda_workspace.restype = i64
    L.osdn_chunk_bwd_kda_workspace.argtypes = [i64, i64, i64, i32, i32, ctypes.c_int]
    L.osdn_chunk_bwd_kda.restype = ctypes.c_int
    L.osdn_chunk_bwd_kda.argtypes = [vp] * 17 + [i64, i64, i64, i64, i32, i32, ctypes.c_int,
                                                 ctypes.c_int, vp]
    L.osdn_status_string.restype = ctypes.c_char_p
    L.osdn_status_string.argtypes = [ctypes.c_int]
    L.osdn_abi_version.restype = ctypes.c_int32
    L.osdn_abi_version.argtypes = []
    if L.osdn_abi_version() != ABI_VERSION:
        raise ImportError(f"libosdn ABI {L.osdn_abi_version()} != {ABI_VERSION}")
    _lib = L
    return L


def status_string(status: int) -> str:
    try:
        return lib().osdn_status_string(status).decode()
    except ImportError:
        return "?"


# ---- torch marshalling ------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return OSDN_F32
    if t.dtype == torch.bfloat16:
        return OSDN_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream, device) -> int:
    torch = _torch()
    s = torch.cuda.current_stream(device) if stream is None else stream
    return s.cuda_stream


def osdn_chunk_fwd(q, k, v, beta, d, alpha=None, S0=None, *, chunk: int = 64, o=None,
                   S_T=None, want_state: bool = True, stream=None):
    """Chunkwise OSDN forward.  q, k, d [B,H,T,dk]; v [B,H,T,dv]; beta, alpha [B,H,T] fp32;
    S0 [B,H,dk,dv] fp32 (M = S^T).  Returns (o, S_T) (S_T is None unless ``want_state`` or
    an ``S_T`` buffer is given).  ``S_T`` may be ``S0`` for an in-place carry."""
    torch = _torch()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    for name, t, shape in (("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                           ("beta", beta, (B, H, T)), ("d", d, (B, H, T, dk)),
                           ("o", o, (B, H, T, dv))):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    if alpha is not None and tuple(alpha.shape) != (B, H, T):
        raise ValueError("alpha must be [B,H,T]")
    for name, t in (("S0", S0), ("S_T", S_T)):
        if t is not None and (tuple(t.shape) != (B, H, dk, dv) or t.dtype != torch.float32):
            raise ValueError(f"{name} must be float32 [B,H,dk,dv]")
    for name, t in (("beta", beta), ("alpha", alpha)):
        if t is not None and t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if k.dtype != q.dtype or v.dtype != q.dtype or o.dtype != q.dtype:
        raise TypeError("q, k, v and o must share one dtype")
    st = lib().osdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(d), _ptr(alpha),
                              _ptr(S0), _ptr(o), _ptr(S_T), B, H, T, dk, dv, chunk,
                              _dtype_code(q), _dtype_code(d), _stream(stream, q.device))
    if st != 0:
        raise OSDNError(st, "osdn_chunk_fwd")
    return o, S_T


def states_bytes(B: int, H: int, T: int, dk: int, dv: int, dtype_code: int) -> int:
    n = lib().osdn_chunk_states_bytes(B, H, T, dk, dv, dtype_code)
    if n < 0:
        raise ValueError("invalid sizes for osdn_chunk_fwd_states")
    return n


def checkpoint_matrix(ck):
    """The [B,H,nchunks,dk,dv] values of a bf16 checkpoint view [B,H,nchunks,dv/16,dk,16]
    (a copy; fp32 views pass through)."""
    if ck.dim() == 5:
        return ck
    B, H, nch, nt, dk, w = ck.shape
    return ck.permute(0, 1, 2, 4, 3, 5).reshape(B, H, nch, dk, nt * w)


def rows_matrix(u, T: int):
    """The [B,H,T,dv] values of a per-row buffer view [B,H,nchunks,dv/16,64,16] (a copy)."""
    B, H, nch, nt, c, w = u.shape
    return u.permute(0, 1, 2, 4, 3, 5).reshape(B, H, nch * c, nt * w)[:, :, :T]


def states_parts(states, B: int, H: int, T: int, dk: int, dv: int, dtype):
    """Views of the training pair's states buffer: (checkpoints, U or None); dtype is the
    inputs' (torch.bfloat16 or torch.float32).  The checkpoints are [B,H,nchunks,dk,dv] for fp32
    inputs and, for bf16 inputs, dv/16 contiguous column tiles [B,H,nchunks,dv/16,dk,16]
    (checkpoint_matrix gives the [..., dk, dv] values); U (bf16 inputs) is per 64-row chunk
    dv/16 contiguous 64 x 16 tiles, [B,H,nchunks,dv/16,64,16] (rows_matrix gives [B,H,T,dv])."""
    torch = _torch()
    bf = dtype == torch.bfloat16
    chunk = 64 if bf else 32
    nch = (T + chunk - 1) // chunk
    n = B * H * nch * dk * dv * (2 if bf else 4)
    if not bf:
        return states[:n].view(torch.float32).view(B, H, nch, dk, dv), None
    ck = states[:n].view(torch.bfloat16).view(B, H, nch, dv // 16, dk, 16)
    uoff = (n + 255) // 256 * 256
    u = states[uoff:uoff + B * H * nch * chunk * dv * 2].view(torch.bfloat16)
    return ck, u.view(B, H, nch, dv // 16, chunk, 16)


def osdn_chunk_fwd_states(q, k, v, beta, d, alpha=None, S0=None, *, o=None, S_T=None,
                          states=None, want_state: bool = True, stream=None):
    """osdn_chunk_fwd with the backward's chunk size (64 rows for bf16, 32 for fp32) that also
    keeps what the backward would recompute, for osdn_chunk_bwd(..., states=...).  Returns
    (o, S_T, states): states is a uint8 buffer of osdn_chunk_states_bytes bytes holding the
    state at every chunk start ([B,H,nchunks,dk,dv], bf16 for bf16 inputs, fp32 for fp32) and,
    for bf16 inputs, the pseudo-values U of every row after them (states_parts splits it)."""
    torch = _torch()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    nbytes = states_bytes(B, H, T, dk, dv, _dtype_code(q))
    if states is None:
        states = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if states.dtype != torch.uint8 or not states.is_contiguous() or states.numel() < nbytes:
        raise ValueError(f"states must be a contiguous uint8 buffer of at least {nbytes} bytes")
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    for name, t, shape in (("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                           ("beta", beta, (B, H, T)), ("d", d, (B, H, T, dk)),
                           ("o", o, (B, H, T, dv))):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    if alpha is not None and (tuple(alpha.shape) != (B, H, T) or alpha.dtype != torch.float32):
        raise ValueError("alpha must be float32 [B,H,T]")
    for name, t in (("S0", S0), ("S_T", S_T)):
        if t is not None and (tuple(t.shape) != (B, H, dk, dv) or t.dtype != torch.float32):
            raise ValueError(f"{name} must be float32 [B,H,dk,dv]")
    if k.dtype != q.dtype or v.dtype != q.dtype or o.dtype != q.dtype:
        raise TypeError("q, k, v and o must share one dtype")
    st = lib().osdn_chunk_fwd_states(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(d),
                                     _ptr(alpha), _ptr(S0), _ptr(o), _ptr(S_T), _ptr(states),
                                     B, H, T, dk, dv, _dtype_code(q), _dtype_code(d),
                                     _stream(stream, q.device))
    if st != 0:
        raise OSDNError(st, "osdn_chunk_fwd_states")
    return o, S_T, states


def osdn_step(q, k, v, beta, d, alpha, S, *, o=None, stream=None):
    """One decode step, S [B,H,dk,dv] fp32 updated in place.  q, k, d [B,H,dk]; v [B,H,dv];
    beta, alpha [B,H] fp32 (alpha may be None).  Returns o [B,H,dv]."""
    torch = _torch()
    B, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    if tuple(S.shape) != (B, H, dk, dv) or S.dtype != torch.float32:
        raise ValueError("S must be float32 [B,H,dk,dv]")
    if k.dtype != q.dtype or v.dtype != q.dtype or o.dtype != q.dtype:
        raise TypeError("q, k, v and o must share one dtype")
    st = lib().osdn_step(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(d), _ptr(alpha), _ptr(S),
                         _ptr(o), B, H, dk, dv, _dtype_code(q), _dtype_code(d),
                         _stream(stream, q.device))
    if st != 0:
        raise OSDNError(st, "osdn_step")
    return o


def osdn_precond_scan(k, beta, r=None, d1=None, *, eta: float, chunk: Optional[int] = None,
                      d_dtype=None, d=None, d_next=None, want_state: bool = True, stream=None):
    """Phase-1 preconditioner scan.  k [B,H,T,dk]; beta, r [B,H,T] fp32 (r may be None);
    d1 [B,H,dk] fp32 (None: ones).  Returns (d [B,H,T,dk] in ``d_dtype`` (default float32),
    d_next [B,H,dk] fp32 or None).  ``chunk`` defaults to 64 for bf16 keys and 1 otherwise;
    ``d_next`` may be ``d1`` for an in-place carry."""
    torch = _torch()
    B, H, T, dk = k.shape
    if chunk is None:
        chunk = 64 if k.dtype == torch.bfloat16 else 1
    if d is None:
        d = torch.empty((B, H, T, dk), dtype=d_dtype or torch.float32, device=k.device)
    if d_next is None and want_state:
        d_next = torch.empty((B, H, dk), dtype=torch.float32, device=k.device)
    if tuple(d.shape) != (B, H, T, dk):
        raise ValueError(f"d has shape {tuple(d.shape)}, expected {(B, H, T, dk)}")
    for name, t, shape in (("beta", beta, (B, H, T)), ("r", r, (B, H, T)),
                           ("d1", d1, (B, H, dk)), ("d_next", d_next, (B, H, dk))):
        if t is not None and (tuple(t.shape) != shape or t.dtype != torch.float32):
            raise ValueError(f"{name} must be float32 {shape}")
    st = lib().osdn_precond_scan(_ptr(k), _ptr(beta), _ptr(r), _ptr(d1), float(eta), _ptr(d),
                                 _ptr(d_next), B, H, T, dk, chunk, _dtype_code(k),
                                 _dtype_code(d), _stream(stream, k.device))
    if st != 0:
        raise OSDNError(st, "osdn_precond_scan")
    return d, d_next


def osdn_precond_step(k, beta, r, dstate, *, eta: float, d_out=None, d_dtype=None,
                      stream=None):
    """One decode token of the scan: k [B,H,dk]; beta, r [B,H] fp32 (r may be None); dstate
    [B,H,dk] fp32 updated in place.  Returns d_out [B,H,dk] (the d this token writes with)."""
    torch = _torch()
    B, H, dk = k.shape
    if d_out is None:
        d_out = torch.empty((B, H, dk), dtype=d_dtype or torch.float32, device=k.device)
    if tuple(dstate.shape) != (B, H, dk) or dstate.dtype != torch.float32:
        raise ValueError("dstate must be float32 [B,H,dk]")
    for name, t in (("beta", beta), ("r", r)):
        if t is not None and (tuple(t.shape) != (B, H) or t.dtype != torch.float32):
            raise ValueError(f"{name} must be float32 [B,H]")
    st = lib().osdn_precond_step(_ptr(k), _ptr(beta), _ptr(r), _ptr(dstate), _ptr(d_out),
                                 float(eta), B, H, dk, _dtype_code(k), _dtype_code(d_out),
                                 _stream(stream, k.device))
    if st != 0:
        raise OSDNError(st, "osdn_precond_step")
    return d_out


def kda_workspace_bytes(B: int, H: int, T: int, dk: int, chunk: int, dtype_code: int) -> int:
    n = lib().osdn_chunk_fwd_kda_workspace(B, H, T, dk, chunk, dtype_code)
    if n < 0:
        raise ValueError("invalid shape for the channel-wise gate's workspace")
    return n


def osdn_chunk_fwd_kda(q, k, v, beta, d, alpha_ch, S0=None, *, chunk: int = 64, o=None,
                       S_T=None, want_state: bool = True, workspace=None, stream=None):
    """Chunkwise forward with the channel-wise gate alpha_ch [B,H,T,dk] fp32 (no scalar alpha).
    Other arguments as osdn_chunk_fwd.  ``workspace`` (a uint8 device tensor of at least
    kda_workspace_bytes(...) bytes) is allocated with torch when not given."""
    torch = _torch()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=q.dtype, device=q.device)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    for name, t, shape in (("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                           ("beta", beta, (B, H, T)), ("d", d, (B, H, T, dk)),
                           ("alpha_ch", alpha_ch, (B, H, T, dk)), ("o", o, (B, H, T, dv))):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    for name, t in (("S0", S0), ("S_T", S_T)):
        if t is not None and (tuple(t.shape) != (B, H, dk, dv) or t.dtype != torch.float32):
            raise ValueError(f"{name} must be float32 [B,H,dk,dv]")
    for name, t in (("beta", beta), ("alpha_ch", alpha_ch)):
        if t.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    if k.dtype != q.dtype or v.dtype != q.dtype or o.dtype != q.dtype:
        raise TypeError("q, k, v and o must share one dtype")
    need = kda_workspace_bytes(B, H, T, dk, chunk, _dtype_code(q))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    st = lib().osdn_chunk_fwd_kda(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(d),
                                  _ptr(alpha_ch), _ptr(S0), _ptr(o), _ptr(S_T),
                                  _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  B, H, T, dk, dv, chunk, _dtype_code(q), _dtype_code(d),
                                  _stream(stream, q.device))
    if st != 0:
        raise OSDNError(st, "osdn_chunk_fwd_kda")
    return o, S_T


NOALLOC_SCRATCH_BYTES = 64 << 20


def osdn_chunk_fwd_kda_noalloc(q, k, v, beta, d, alpha_ch, S0, o, S_T, *, chunk: int = 64,
                               stream=None):
    """osdn_chunk_fwd_kda through the entry point that allocates nothing: the caller passes the
    outputs o [B,H,T,dv] and S_T [B,H,dk,dv] (or None); the library's own scratch array holds the
    workspace.  Raises OSDNError (status -7) when the problem needs more scratch than it has."""
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    st = lib().osdn_chunk_fwd_kda_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(d),
                                          _ptr(alpha_ch), _ptr(S0), _ptr(o), _ptr(S_T),
                                          B, H, T, dk, dv, chunk, _dtype_code(q),
                                          _dtype_code(d), _stream(stream, q.device))
    if st != 0:
        raise OSDNError(st, "osdn_chunk_fwd_kda_noalloc")
    return o, S_T


def osdn_step_kda(q, k, v, beta, d, alpha_ch, S, *, o=None, stream=None):
    """One decode step with the channel-wise gate alpha_ch [B,H,dk] fp32; S [B,H,dk,dv] fp32
    updated in place.  Returns o [B,H,dv]."""
    torch = _torch()
    B, H, dk = q.shape
    dv = v.shape[-1]
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=q.device)
    if tuple(S.shape) != (B, H, dk, dv) or S.dtype != torch.float32:
        raise ValueError("S must be float32 [B,H,dk,dv]")
    if tuple(alpha_ch.shape) != (B, H, dk) or alpha_ch.dtype != torch.float32:
        raise ValueError("alpha_ch must be float32 [B,H,dk]")
    if k.dtype != q.dtype or v.dtype != q.dtype or o.dtype != q.dtype:
        raise TypeError("q, k, v and o must share one dtype")
    st = lib().osdn_step_kda(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(d), _ptr(alpha_ch),
                             _ptr(S), _ptr(o), B, H, dk, dv, _dtype_code(q), _dtype_code(d),
                             _stream(stream, q.device))
    if st != 0:
        raise OSDNError(st, "osdn_step_kda")
    return o


def bwd_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, dtype_code: int) -> int:
    n = lib().osdn_chunk_bwd_workspace(B, H, T, dk, dv, dtype_code)
    if n < 0:
        raise ValueError("invalid sizes for osdn_chunk_bwd")
    return n


def bwd_states_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, dtype_code: int) -> int:
    n = lib().osdn_chunk_bwd_states_workspace(B, H, T, dk, dv, dtype_code)
    if n < 0:
        raise ValueError("invalid shape for the backward's workspace")
    return n


def osdn_chunk_bwd(q, k, v, beta, d, alpha, S0, grad_o, grad_S_T=None, *, grads=None,
                   want_grad_S0: bool = True, workspace=None, states=None, stream=None):
    """Gradients of osdn_chunk_fwd(q, k, v, beta, d, alpha, S0) for output gradients grad_o
    [B,H,T,dv] (dtype of q) and grad_S_T [B,H,dk,dv] fp32 (None: zero).  Returns a dict with
    grad_q, grad_k, grad_v (dtype of q), grad_beta (fp32), grad_d (dtype of d), grad_alpha
    (fp32, None without alpha) and grad_S0 (fp32, None unless want_grad_S0).  ``grads`` may
    supply some of those output tensors; the rest and the workspace are allocated with torch.
    ``states`` (from osdn_chunk_fwd_states on the same inputs) spares the forward recompute."""
    torch = _torch()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    for name, t, shape in (("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                           ("beta", beta, (B, H, T)), ("d", d, (B, H, T, dk)),
                           ("grad_o", grad_o, (B, H, T, dv))):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    for name, t in (("S0", S0), ("grad_S_T", grad_S_T)):
        if t is not None and (tuple(t.shape) != (B, H, dk, dv) or t.dtype != torch.float32):
            raise ValueError(f"{name} must be float32 [B,H,dk,dv]")
    if alpha is not None and (tuple(alpha.shape) != (B, H, T) or alpha.dtype != torch.float32):
        raise ValueError("alpha must be float32 [B,H,T]")
    if k.dtype != q.dtype or v.dtype != q.dtype or grad_o.dtype != q.dtype:
        raise TypeError("q, k, v and grad_o must share one dtype")
    g = dict(grads or {})
    new = lambda shape, dt: torch.empty(shape, dtype=dt, device=q.device)
    g.setdefault("grad_q", new((B, H, T, dk), q.dtype))
    g.setdefault("grad_k", new((B, H, T, dk), q.dtype))
    g.setdefault("grad_v", new((B, H, T, dv), q.dtype))
    g.setdefault("grad_beta", new((B, H, T), torch.float32))
    g.setdefault("grad_d", new((B, H, T, dk), d.dtype))
    if alpha is not None:
        g.setdefault("grad_alpha", new((B, H, T), torch.float32))
    else:
        g["grad_alpha"] = None
    if want_grad_S0:
        g.setdefault("grad_S0", new((B, H, dk, dv), torch.float32))
    else:
        g["grad_S0"] = None
    need = (bwd_workspace_bytes if states is None else bwd_states_workspace_bytes)(
        B, H, T, dk, dv, _dtype_code(q))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    wsb = workspace.numel() * workspace.element_size()
    tail = (B, H, T, dk, dv, _dtype_code(q), _dtype_code(d), _stream(stream, q.device))
    grad_ptrs = (_ptr(g["grad_q"]), _ptr(g["grad_k"]), _ptr(g["grad_v"]), _ptr(g["grad_beta"]),
                 _ptr(g["grad_d"]), _ptr(g["grad_alpha"]), _ptr(g["grad_S0"]))
    ins = (_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(d), _ptr(alpha), _ptr(S0))
    if states is None:
        st = lib().osdn_chunk_bwd(*ins, _ptr(grad_o), _ptr(grad_S_T), *grad_ptrs,
                                  _ptr(workspace), wsb, *tail)
        name = "osdn_chunk_bwd"
    else:
        if states.numel() * states.element_size() < states_bytes(B, H, T, dk, dv, _dtype_code(q)):
            raise ValueError("states is smaller than osdn_chunk_states_bytes")
        st = lib().osdn_chunk_bwd_states(*ins, _ptr(states), _ptr(grad_o), _ptr(grad_S_T),
                                         *grad_ptrs, _ptr(workspace), wsb, *tail)
        name = "osdn_chunk_bwd_states"
    if st != 0:
        raise OSDNError(st, name)
    return g


def bwd_kda_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, dtype_code: int) -> int:
    n = lib().osdn_chunk_bwd_kda_workspace(B, H, T, dk, dv, dtype_code)
    if n < 0:
        raise ValueError("invalid sizes for osdn_chunk_bwd_kda")
    return n


def osdn_chunk_bwd_kda(q, k, v, beta, d, alpha_ch, S0, grad_o, grad_S_T=None, *, grads=None,
                       want_grad_S0: bool = True, workspace=None, stream=None):
    """Gradients of osdn_chunk_fwd_kda(q, k, v, beta, d, alpha_ch, S0) for output gradients
    grad_o [B,H,T,dv] (dtype of q) and grad_S_T [B,H,dk,dv] fp32 (None: zero).  Returns a dict
    with grad_q, grad_k, grad_v (dtype of q), grad_beta (fp32), grad_d (dtype of d),
    grad_alpha_ch (fp32 [B,H,T,dk]) and grad_S0 (fp32, None unless want_grad_S0).  ``grads``
    may supply some of those output tensors; the rest and the workspace are allocated with
    torch."""
    torch = _torch()
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    for name, t, shape in (("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                           ("beta", beta, (B, H, T)), ("d", d, (B, H, T, dk)),
                           ("grad_o", grad_o, (B, H, T, dv))):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    for name, t in (("S0", S0), ("grad_S_T", grad_S_T)):
        if t is not None and (tuple(t.shape) != (B, H, dk, dv) or t.dtype != torch.float32):
            raise ValueError(f"{name} must be float32 [B,H,dk,dv]")
    if tuple(alpha_ch.shape) != (B, H, T, dk) or alpha_ch.dtype != torch.float32:
        raise ValueError("alpha_ch must be float32 [B,H,T,dk]")
    if k.dtype != q.dtype or v.dtype != q.dtype or grad_o.dtype != q.dtype:
        raise TypeError("q, k, v and grad_o must share one dtype")
    g = dict(grads or {})
    new = lambda shape, dt: torch.empty(shape, dtype=dt, device=q.device)
    g.setdefault("grad_q", new((B, H, T, dk), q.dtype))
    g.setdefault("grad_k", new((B, H, T, dk), q.dtype))
    g.setdefault("grad_v", new((B, H, T, dv), q.dtype))
    g.setdefault("grad_beta", new((B, H, T), torch.float32))
    g.setdefault("grad_d", new((B, H, T, dk), d.dtype))
    g.setdefault("grad_alpha_ch", new((B, H, T, dk), torch.float32))
    if want_grad_S0:
        g.setdefault("grad_S0", new((B, H, dk, dv), torch.float32))
    else:
        g["grad_S0"] = None
    need = bwd_kda_workspace_bytes(B, H, T, dk, dv, _dtype_code(q))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    wsb = workspace.numel() * workspace.element_size()
    st = lib().osdn_chunk_bwd_kda(
        _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(d), _ptr(alpha_ch), _ptr(S0), _ptr(grad_o),
        _ptr(grad_S_T), _ptr(g["grad_q"]), _ptr(g["grad_k"]), _ptr(g["grad_v"]),
        _ptr(g["grad_beta"]), _ptr(g["grad_d"]), _ptr(g["grad_alpha_ch"]), _ptr(g["grad_S0"]),
        _ptr(workspace), wsb, B, H, T, dk, dv, _dtype_code(q), _dtype_code(d),
        _stream(stream, q.device))
    if st != 0:
        raise OSDNError(st, "osdn_chunk_bwd_kda")
    return g
