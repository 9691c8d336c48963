"""libosdn's C ABI on the host: it loads, exports what include/osdn.h declares, and every
validation path returns its status before anything is enqueued (no GPU needed: these calls
never reach a launch)."""
import ctypes
import os
import re

import pytest

from delta_rule_sequence_chunkwise_amd import osdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(osdn.LIB_PATH):
        from delta_rule_sequence_chunkwise_amd import build
        build.build()
    return osdn.lib()


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"\b(osdn_\w+)\s*\(", text)
    return sorted(set(names))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(osdn.EXPORTS) <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    assert L.osdn_abi_version() == osdn.ABI_VERSION
    for code in osdn.STATUS:
        s = L.osdn_status_string(code)
        assert s and s.decode()
    assert L.osdn_status_string(12345) == b"unknown status"


# fake, 256-byte aligned device addresses: validation compares them, never dereferences
BASE = 1 << 40
SPAN = 1 << 32


def addr(i):
    return BASE + i * SPAN


def chunk_args(**over):
    a = dict(q=addr(1), k=addr(2), v=addr(3), beta=addr(4), d=addr(5), alpha=addr(6),
             S0=addr(7), o=addr(8), S_T=addr(9), B=2, H=3, T=100, dk=128, dv=64, chunk=64,
             qkv=osdn.OSDN_BF16, d_dtype=osdn.OSDN_F32, stream=None)
    a.update(over)
    return a


def call_chunk(L, **over):
    a = chunk_args(**over)
    return L.osdn_chunk_fwd(a["q"], a["k"], a["v"], a["beta"], a["d"], a["alpha"], a["S0"],
                            a["o"], a["S_T"], a["B"], a["H"], a["T"], a["dk"], a["dv"],
                            a["chunk"], a["qkv"], a["d_dtype"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(beta=None), -1),
    (dict(d=None), -1), (dict(o=None), -1),
    (dict(B=-1), -2), (dict(H=-2), -2), (dict(T=-5), -2),
    (dict(B=1 << 40, H=1 << 20), -2), (dict(T=1 << 45), -2),
    (dict(dk=96), -3), (dict(dv=32), -3), (dict(dk=256), -3),
    (dict(chunk=32), -3), (dict(qkv=osdn.OSDN_F32, chunk=48), -3), (dict(qkv=7), -3),
    (dict(d_dtype=3), -3),
    (dict(q=addr(1) + 8), -4), (dict(o=addr(8) + 4), -4), (dict(S0=addr(7) + 4), -4),
    (dict(beta=addr(4) + 2), -4), (dict(alpha=addr(6) + 1), -4),
    (dict(o=addr(1)), -5), (dict(o=addr(3) + 256), -5), (dict(S_T=addr(8)), -5),
    (dict(S_T=addr(2)), -5), (dict(S_T=addr(7) + 4096), -5), (dict(o=addr(9)), -5),
])
def test_chunk_fwd_rejects(L, over, status):
    assert call_chunk(L, **over) == status


def test_chunk_fwd_empty_work_is_ok_without_touching_memory(L):
    assert call_chunk(L, B=0) == 0
    assert call_chunk(L, H=0, q=None) == 0
    # T == 0 with no final state requested: nothing to do, inputs may be NULL
    assert call_chunk(L, T=0, q=None, k=None, v=None, beta=None, d=None, o=None,
                      S_T=None) == 0


def step_args(**over):
    a = dict(q=addr(1), k=addr(2), v=addr(3), beta=addr(4), d=addr(5), alpha=addr(6),
             S=addr(7), o=addr(8), B=4, H=2, dk=128, dv=128, qkv=osdn.OSDN_BF16,
             d_dtype=osdn.OSDN_F32, stream=None)
    a.update(over)
    return a


def call_step(L, **over):
    a = step_args(**over)
    return L.osdn_step(a["q"], a["k"], a["v"], a["beta"], a["d"], a["alpha"], a["S"], a["o"],
                       a["B"], a["H"], a["dk"], a["dv"], a["qkv"], a["d_dtype"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(q=None), -1), (dict(S=None), -1), (dict(o=None), -1), (dict(d=None), -1),
    (dict(B=-1), -2), (dict(B=1 << 40, H=1 << 30), -2),
    (dict(dk=32), -3), (dict(dv=100), -3), (dict(qkv=2), -3),
    (dict(S=addr(7) + 4), -4), (dict(q=addr(1) + 2), -4),
    (dict(o=addr(7)), -5), (dict(S=addr(1)), -5), (dict(o=addr(2) + 64), -5),
])
def test_step_rejects(L, over, status):
    assert call_step(L, **over) == status


def test_step_empty_is_ok(L):
    assert call_step(L, B=0, q=None) == 0


def test_python_binding_refuses_host_tensors(L):
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        osdn.osdn_chunk_fwd(x, x, x, torch.zeros(1, 1, 4), x, want_state=False,
                            o=torch.zeros(1, 1, 4, 64))


def precond_args(**over):
    a = dict(k=addr(1), beta=addr(2), r=addr(3), d1=addr(4), eta=0.5, d=addr(5),
             d_next=addr(6), B=2, H=3, T=100, dk=128, chunk=64, k_dtype=osdn.OSDN_BF16,
             d_dtype=osdn.OSDN_F32, stream=None)
    a.update(over)
    return a


def call_precond(L, **over):
    a = precond_args(**over)
    return L.osdn_precond_scan(a["k"], a["beta"], a["r"], a["d1"], a["eta"], a["d"],
                               a["d_next"], a["B"], a["H"], a["T"], a["dk"], a["chunk"],
                               a["k_dtype"], a["d_dtype"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(k=None), -1), (dict(beta=None), -1), (dict(d=None), -1),
    (dict(B=-1), -2), (dict(T=-1), -2), (dict(B=1 << 40, H=1 << 20), -2),
    (dict(dk=96), -3), (dict(chunk=32), -3), (dict(chunk=0), -3),
    (dict(chunk=64, k_dtype=osdn.OSDN_F32), -3), (dict(k_dtype=5), -3), (dict(d_dtype=2), -3),
    (dict(k=addr(1) + 8), -4), (dict(d=addr(5) + 4), -4), (dict(beta=addr(2) + 2), -4),
    (dict(d1=addr(4) + 4), -4), (dict(d_next=addr(6) + 8), -4), (dict(r=addr(3) + 1), -4),
    (dict(d=addr(1)), -5), (dict(d=addr(2) - 256), -5), (dict(d_next=addr(5) + 1024), -5),
    (dict(d_next=addr(1)), -5), (dict(d_next=addr(4) + 16), -5), (dict(d=addr(6)), -5),
])
def test_precond_scan_rejects(L, over, status):
    assert call_precond(L, **over) == status


def test_precond_scan_empty_work_is_ok(L):
    assert call_precond(L, B=0) == 0
    assert call_precond(L, T=0, k=None, beta=None, d=None, d_next=None) == 0
    # the serial form takes either key type
    assert call_precond(L, B=0, chunk=1, k_dtype=osdn.OSDN_F32) == 0


def call_precond_step(L, **over):
    a = dict(k=addr(1), beta=addr(2), r=addr(3), dstate=addr(4), d_out=addr(5), eta=0.5, B=4,
             H=2, dk=64, k_dtype=osdn.OSDN_BF16, d_dtype=osdn.OSDN_BF16, stream=None)
    a.update(over)
    return L.osdn_precond_step(a["k"], a["beta"], a["r"], a["dstate"], a["d_out"], a["eta"],
                               a["B"], a["H"], a["dk"], a["k_dtype"], a["d_dtype"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(k=None), -1), (dict(dstate=None), -1), (dict(beta=None), -1),
    (dict(B=-3), -2), (dict(dk=100), -3), (dict(k_dtype=9), -3),
    (dict(dstate=addr(4) + 4), -4), (dict(d_out=addr(5) + 8), -4),
    (dict(d_out=addr(4)), -5), (dict(dstate=addr(1)), -5), (dict(d_out=addr(2)), -5),
])
def test_precond_step_rejects(L, over, status):
    assert call_precond_step(L, **over) == status


def test_precond_step_empty_is_ok(L):
    assert call_precond_step(L, H=0, k=None) == 0


def call_kda(L, **over):
    a = dict(q=addr(1), k=addr(2), v=addr(3), beta=addr(4), d=addr(5), alpha_ch=addr(6),
             S0=addr(7), o=addr(8), S_T=addr(9), ws=addr(10), wsb=1 << 31, B=2, H=3, T=100,
             dk=128, dv=64, chunk=64, qkv=osdn.OSDN_BF16, d_dtype=osdn.OSDN_F32, stream=None)
    a.update(over)
    return L.osdn_chunk_fwd_kda(a["q"], a["k"], a["v"], a["beta"], a["d"], a["alpha_ch"],
                                a["S0"], a["o"], a["S_T"], a["ws"], a["wsb"], a["B"], a["H"],
                                a["T"], a["dk"], a["dv"], a["chunk"], a["qkv"], a["d_dtype"],
                                a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(alpha_ch=None), -1), (dict(ws=None), -1), (dict(q=None), -1),
    (dict(T=-1), -2), (dict(wsb=1000), -2), (dict(dk=32), -3), (dict(chunk=16), -3),
    (dict(ws=addr(10) + 128), -4), (dict(alpha_ch=addr(6) + 2), -4),
    (dict(alpha_ch=addr(6) + 4), -4),
    (dict(ws=addr(1)), -5), (dict(o=addr(10)), -5), (dict(S_T=addr(10) + 512), -5),
])
def test_chunk_fwd_kda_rejects(L, over, status):
    assert call_kda(L, **over) == status


def test_kda_workspace_size(L):
    n = L.osdn_chunk_fwd_kda_workspace(2, 3, 100, 128, 64, osdn.OSDN_BF16)
    # gate-scaled q, k, k~ (bf16), the chunk planes (P 64 x 72, four 16 x 16 inverses, six
    # 16 x 16 off-diagonal blocks, bf16, two chunks), G_C (fp32, two chunks), each rounded up
    # to 256 bytes
    planes = 2 * 3 * 2 * (64 * 72 + 4 * 256 + 6 * 256) * 2
    assert n == 3 * (2 * 3 * 100 * 128 * 2) + planes + 2 * 3 * 2 * 128 * 4
    assert L.osdn_chunk_fwd_kda_workspace(2, 3, 100, 96, 64, osdn.OSDN_BF16) == -1
    # fp32 inputs need no workspace
    assert L.osdn_chunk_fwd_kda_workspace(1, 1, 10, 64, 16, osdn.OSDN_F32) == 0
    assert call_kda(L, B=0) == 0 and call_kda(L, T=0, q=None, S_T=None, ws=None) == 0


def test_kda_noalloc_rejects_before_touching_the_gpu(L):
    """The no-allocation entry point checks the problem against its scratch array (64 MiB)
    before any HIP call: too large a problem returns OSDN_ERR_SCRATCH, an unsupported one the
    usual status.  (Fake addresses: nothing is dereferenced.)"""
    ptrs = [addr(i) for i in range(1, 10)]
    call = lambda B, H, T, dk, dv, chunk, qkv: L.osdn_chunk_fwd_kda_noalloc(
        *ptrs, B, H, T, dk, dv, chunk, qkv, osdn.OSDN_F32, None)
    need = L.osdn_chunk_fwd_kda_workspace(4, 16, 4096, 128, 64, osdn.OSDN_BF16)
    assert need > osdn.NOALLOC_SCRATCH_BYTES
    assert call(4, 16, 4096, 128, 128, 64, osdn.OSDN_BF16) == -7
    assert call(4, 16, 4096, 96, 128, 64, osdn.OSDN_BF16) == -3
    assert call(1, 1, 10, 128, 128, 32, osdn.OSDN_BF16) == -3
    assert call(0, 16, 4096, 128, 128, 64, osdn.OSDN_BF16) == 0
    assert L.osdn_status_string(-7).decode().startswith("problem needs more scratch")


def test_step_kda_rejects(L):
    args = [addr(1), addr(2), addr(3), addr(4), addr(5), addr(6), addr(7), addr(8), 4, 2, 128,
            128, osdn.OSDN_BF16, osdn.OSDN_F32, None]
    assert L.osdn_step_kda(*args[:5], None, *args[6:]) == -1
    bad = list(args)
    bad[5] = addr(6) + 2
    assert L.osdn_step_kda(*bad) == -4
    bad = list(args)
    bad[7] = addr(6)
    assert L.osdn_step_kda(*bad) == -5
    bad = list(args)
    bad[8] = 0
    assert L.osdn_step_kda(*bad) == 0


def call_bwd(L, **over):
    a = dict(q=addr(1), k=addr(2), v=addr(3), beta=addr(4), d=addr(5), alpha=addr(6),
             S0=addr(7), go=addr(8), gST=addr(9), gq=addr(10), gk=addr(11), gv=addr(12),
             gb=addr(13), gd=addr(14), ga=addr(15), gS0=addr(16), ws=addr(17), wsb=1 << 31,
             B=2, H=3, T=100, dk=128, dv=64, qkv=osdn.OSDN_BF16, d_dtype=osdn.OSDN_F32,
             stream=None)
    a.update(over)
    return L.osdn_chunk_bwd(a["q"], a["k"], a["v"], a["beta"], a["d"], a["alpha"], a["S0"],
                            a["go"], a["gST"], a["gq"], a["gk"], a["gv"], a["gb"], a["gd"],
                            a["ga"], a["gS0"], a["ws"], a["wsb"], a["B"], a["H"], a["T"],
                            a["dk"], a["dv"], a["qkv"], a["d_dtype"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(q=None), -1), (dict(go=None), -1), (dict(gd=None), -1), (dict(ws=None), -1),
    (dict(T=-1), -2), (dict(wsb=1000), -2), (dict(dk=96), -3), (dict(qkv=7), -3),
    (dict(q=addr(1) + 8), -4), (dict(ws=addr(17) + 128), -4), (dict(gb=addr(13) + 2), -4),
    (dict(gq=addr(1)), -5), (dict(ws=addr(8)), -5), (dict(gk=addr(10) + 256), -5),
    (dict(gS0=addr(17) + 4096), -5),
])
def test_chunk_bwd_rejects(L, over, status):
    assert call_bwd(L, **over) == status


def test_bwd_workspace_size(L):
    # bf16 inputs: two bf16 checkpoints [B,H,nchunks,dk,dv] (64-row chunks), per chunk three
    # bf16 64 x 64 planes (the inverse's hi and lo, the scores) and K~ (64 x dk bf16), and two
    # bf16 per-row buffers U and dR in whole 64-row chunks (the last padded), each rounded up to
    # 256 bytes
    nch = (100 + 63) // 64
    ck = 2 * 3 * nch * 128 * 64 * 2
    ti = 2 * 3 * nch * (3 * 64 * 64 + 64 * 128) * 2
    ub = (2 * 3 * nch * 64 * 64 * 2 + 255) // 256 * 256
    assert L.osdn_chunk_bwd_workspace(2, 3, 100, 128, 64, osdn.OSDN_BF16) == 2 * ck + ti + 2 * ub
    # fp32 inputs: two fp32 checkpoints (32-row chunks), no inverses
    nch = (100 + 31) // 32
    assert L.osdn_chunk_bwd_workspace(2, 3, 100, 128, 64, osdn.OSDN_F32) == 2 * (2 * 3 * nch * 128 * 64 * 4)
    assert L.osdn_chunk_bwd_workspace(2, 3, 100, 96, 64, osdn.OSDN_BF16) == -1
    assert L.osdn_chunk_bwd_workspace(2, 3, -1, 128, 64, osdn.OSDN_BF16) == -1
    need = L.osdn_chunk_bwd_workspace(2, 3, 100, 128, 64, osdn.OSDN_BF16)
    assert call_bwd(L, wsb=need - 1) == -2
    assert call_bwd(L, B=0) == 0


def call_fwd_states(L, **over):
    a = dict(q=addr(1), k=addr(2), v=addr(3), beta=addr(4), d=addr(5), alpha=addr(6),
             S0=addr(7), o=addr(8), S_T=addr(9), states=addr(10), B=2, H=3, T=100, dk=128,
             dv=64, qkv=osdn.OSDN_BF16, d_dtype=osdn.OSDN_F32, stream=None)
    a.update(over)
    return L.osdn_chunk_fwd_states(a["q"], a["k"], a["v"], a["beta"], a["d"], a["alpha"],
                                   a["S0"], a["o"], a["S_T"], a["states"], a["B"], a["H"],
                                   a["T"], a["dk"], a["dv"], a["qkv"], a["d_dtype"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(states=None), -1), (dict(q=None), -1), (dict(T=-1), -2), (dict(dk=96), -3),
    (dict(qkv=7), -3), (dict(states=addr(10) + 8), -4), (dict(states=addr(8) + 256), -5),
    (dict(states=addr(1)), -5), (dict(o=addr(10) + 4096), -5),
])
def test_chunk_fwd_states_rejects(L, over, status):
    assert call_fwd_states(L, **over) == status


def test_states_size_and_empty_work(L):
    # the state at every chunk start, [B,H,nchunks,dk,dv]: bf16 with 64-row chunks for bf16
    # inputs, then U from a 256-byte boundary on, bf16, whole 64-row chunks (the last padded);
    # fp32 with 32-row chunks for fp32 inputs
    ub = (2 * 3 * 128 * 64 * 2 + 255) // 256 * 256
    assert L.osdn_chunk_states_bytes(2, 3, 100, 128, 64, osdn.OSDN_BF16) == 2 * 3 * 2 * 128 * 64 * 2 + ub
    assert L.osdn_chunk_states_bytes(2, 3, 100, 128, 64, osdn.OSDN_F32) == 2 * 3 * 4 * 128 * 64 * 4
    assert L.osdn_chunk_states_bytes(2, 3, 0, 128, 64, osdn.OSDN_BF16) == 0
    assert L.osdn_chunk_states_bytes(2, 3, 100, 96, 64, osdn.OSDN_BF16) == -1
    assert call_fwd_states(L, B=0) == 0
    assert call_fwd_states(L, T=0, q=None, states=None, S_T=None) == 0


@pytest.mark.parametrize("B,H,T,dk,dv,bf", [(2, 3, 100, 128, 64, True), (1, 1, 1, 64, 64, True),
                                             (2, 1, 67, 64, 128, False)])
def test_states_parts_layout(L, B, H, T, dk, dv, bf):
    """The training pair's states buffer: checkpoints first, then (bf16 inputs) U from the next
    256-byte boundary, ending inside osdn_chunk_states_bytes."""
    import torch
    dt = torch.bfloat16 if bf else torch.float32
    nbytes = osdn.states_bytes(B, H, T, dk, dv, osdn.OSDN_BF16 if bf else osdn.OSDN_F32)
    buf = torch.zeros(nbytes, dtype=torch.uint8)
    ck, u = osdn.states_parts(buf, B, H, T, dk, dv, dt)
    nch = (T + (64 if bf else 32) - 1) // (64 if bf else 32)
    # bf16 checkpoints are dv/16 contiguous dk x 16 column tiles
    assert ck.shape == ((B, H, nch, dv // 16, dk, 16) if bf else (B, H, nch, dk, dv))
    assert ck.dtype == dt
    assert osdn.checkpoint_matrix(ck).shape == (B, H, nch, dk, dv)
    assert ck.data_ptr() == buf.data_ptr()
    if not bf:
        assert u is None
        return
    off = u.data_ptr() - buf.data_ptr()
    assert u.shape == (B, H, nch, dv // 16, 64, 16) and u.dtype == torch.bfloat16
    assert osdn.rows_matrix(u, T).shape == (B, H, T, dv)
    assert off % 256 == 0 and off >= ck.numel() * 2
    assert off + u.numel() * 2 <= nbytes


def call_bwd_states(L, **over):
    a = dict(q=addr(1), k=addr(2), v=addr(3), beta=addr(4), d=addr(5), alpha=addr(6),
             S0=addr(7), states=addr(18), go=addr(8), gST=addr(9), gq=addr(10), gk=addr(11),
             gv=addr(12), gb=addr(13), gd=addr(14), ga=addr(15), gS0=addr(16), ws=addr(17),
             wsb=1 << 31, B=2, H=3, T=100, dk=128, dv=64, qkv=osdn.OSDN_BF16,
             d_dtype=osdn.OSDN_F32, stream=None)
    a.update(over)
    return L.osdn_chunk_bwd_states(a["q"], a["k"], a["v"], a["beta"], a["d"], a["alpha"],
                                   a["S0"], a["states"], a["go"], a["gST"], a["gq"], a["gk"],
                                   a["gv"], a["gb"], a["gd"], a["ga"], a["gS0"], a["ws"],
                                   a["wsb"], a["B"], a["H"], a["T"], a["dk"], a["dv"], a["qkv"],
                                   a["d_dtype"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(states=None), -1), (dict(gq=None), -1), (dict(wsb=1000), -2),
    (dict(states=addr(18) + 8), -4), (dict(states=addr(10) + 512), -5),
    (dict(states=addr(17)), -5), (dict(gS0=addr(18) + 4096), -5),
])
def test_chunk_bwd_states_rejects(L, over, status):
    assert call_bwd_states(L, **over) == status


def test_bwd_states_workspace_is_smaller(L):
    """With the forward's states given, the backward's workspace drops the M0 checkpoints and U
    (the caller's states hold them): exactly that size is accepted, one byte less rejected."""
    full = L.osdn_chunk_bwd_workspace(2, 3, 100, 128, 64, osdn.OSDN_BF16)
    sw = L.osdn_chunk_bwd_states_workspace(2, 3, 100, 128, 64, osdn.OSDN_BF16)
    states = L.osdn_chunk_states_bytes(2, 3, 100, 128, 64, osdn.OSDN_BF16)
    assert sw + states == full
    # sizes are checked before any launch (fake addresses: only the rejection can be observed
    # without a device)
    assert call_bwd_states(L, wsb=sw - 1) == -2
    f32 = L.osdn_chunk_bwd_states_workspace(2, 3, 100, 128, 64, osdn.OSDN_F32)
    assert f32 + L.osdn_chunk_states_bytes(2, 3, 100, 128, 64, osdn.OSDN_F32) == \
        L.osdn_chunk_bwd_workspace(2, 3, 100, 128, 64, osdn.OSDN_F32)
    assert L.osdn_chunk_bwd_states_workspace(2, 3, 100, 96, 64, osdn.OSDN_BF16) == -1


def test_chunk_bwd_states_empty_work_is_ok(L):
    assert call_bwd_states(L, B=0) == 0


def call_bwd_kda(L, **over):
    a = dict(q=addr(1), k=addr(2), v=addr(3), beta=addr(4), d=addr(5), a=addr(6),
             S0=addr(7), go=addr(8), gST=addr(9), gq=addr(10), gk=addr(11), gv=addr(12),
             gb=addr(13), gd=addr(14), ga=addr(15), gS0=addr(16), ws=addr(17), wsb=1 << 31,
             B=2, H=3, T=100, dk=128, dv=64, qkv=osdn.OSDN_BF16, d_dtype=osdn.OSDN_F32,
             stream=None)
    a.update(over)
    return L.osdn_chunk_bwd_kda(a["q"], a["k"], a["v"], a["beta"], a["d"], a["a"], a["S0"],
                                a["go"], a["gST"], a["gq"], a["gk"], a["gv"], a["gb"], a["gd"],
                                a["ga"], a["gS0"], a["ws"], a["wsb"], a["B"], a["H"], a["T"],
                                a["dk"], a["dv"], a["qkv"], a["d_dtype"], a["stream"])


@pytest.mark.parametrize("over,status", [
    (dict(a=None), -1), (dict(q=None), -1), (dict(gd=None), -1), (dict(ws=None), -1),
    (dict(T=-1), -2), (dict(wsb=1000), -2), (dict(dk=96), -3), (dict(d_dtype=7), -3),
    (dict(a=addr(6) + 4), -4), (dict(ws=addr(17) + 128), -4), (dict(ga=addr(15) + 2), -4),
    (dict(ga=addr(6)), -5), (dict(gq=addr(15)), -5), (dict(ws=addr(6)), -5),
])
def test_chunk_bwd_kda_rejects(L, over, status):
    assert call_bwd_kda(L, **over) == status


def test_bwd_kda_workspace_size(L):
    # two fp32 checkpoints [B,H,nchunks,dk,dv] with 32-row chunks, for either input type, then
    # the score tiles and their inverse [B,H,nchunks,3,32,32] fp32 (each region rounded up to
    # 256 bytes)
    nch = (100 + 31) // 32
    r256 = lambda n: (n + 255) // 256 * 256
    for qkv in (osdn.OSDN_BF16, osdn.OSDN_F32):
        assert L.osdn_chunk_bwd_kda_workspace(2, 3, 100, 128, 64, qkv) == \
            2 * r256(2 * 3 * nch * 128 * 64 * 4) + r256(2 * 3 * nch * 3 * 32 * 32 * 4)
    assert L.osdn_chunk_bwd_kda_workspace(2, 3, 100, 96, 64, osdn.OSDN_BF16) == -1
    assert L.osdn_chunk_bwd_kda_workspace(2, 3, -1, 128, 64, osdn.OSDN_BF16) == -1
    need = L.osdn_chunk_bwd_kda_workspace(2, 3, 100, 128, 64, osdn.OSDN_BF16)
    assert call_bwd_kda(L, wsb=need - 1) == -2
    assert call_bwd_kda(L, B=0) == 0
    assert call_bwd_kda(L, T=0, gS0=None) == 0  # nothing to write


def test_header_compiles_as_c_and_links(L, tmp_path):
    """include/osdn.h is plain C (C99, no C++ types in the signatures): a C program that
    includes it compiles warning-free, links against the library and sees the same ABI
    version as the library."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "abi.c"
    src.write_text('#include "osdn.h"\n'
                   "int main(void) { return osdn_abi_version() == OSDN_ABI_VERSION ? 0 : 1; }\n")
    exe = tmp_path / "abi"
    lib_dir = os.path.dirname(osdn.LIB_PATH)
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    "-L", lib_dir, "-losdn", f"-Wl,-rpath,{lib_dir}"], check=True)
    subprocess.run([str(exe)], check=True)
