"""The C ABI: the library loads, exports every entry point include/kda.h declares,
and its host-only functions behave as documented.  No GPU work is launched here:
the argument-error cases fail validation before any HIP call.  They pass fake
device addresses, so they are skipped wherever a GPU is visible: a validation
mistake must never turn into a launch on fake pointers.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def _lib():
    from gated_delta_rule_47_amd import _lib as L
    return L.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    from gated_delta_rule_47_amd import _lib as L
    assert _declared() == sorted(L.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared():
        assert hasattr(lib, name), name


def test_read_scale():
    lib = _lib()
    for K in (1, 8, 64, 128):
        assert lib.kda_read_scale(K) == pytest.approx(K ** -0.5, rel=1e-7)
    assert lib.kda_read_scale(8) == pytest.approx(1 / 2.8284271247461903, rel=1e-7)
    assert lib.kda_read_scale(0) == 0.0


def test_status_strings_and_counters():
    lib = _lib()
    assert lib.kda_status_string(0) == b"ok"
    names = {lib.kda_status_string(s) for s in range(-10, 1)}
    assert len(names) == 11 and b"unknown status" not in names
    assert lib.kda_status_string(-99) == b"unknown status"
    n = lib.kda_get_counters(None, 0)
    arr = (ctypes.c_ulonglong * n)()
    assert lib.kda_get_counters(arr, n) == n == 6


def test_workspace_bytes():
    lib = _lib()
    assert lib.kda_chunk_bwd_workspace_bytes(2, 16, 8192, 128, 128, 64) > 2 * 16 * 8192 * 128 * 4
    assert lib.kda_chunk_bwd_workspace_bytes(1, 1, 32, 7, 8, 16) == 0
    assert lib.kda_chunk_bwd_workspace_bytes(1, 1, 32, 8, 8, 48) == 0
    assert lib.kda_chunk_bwd_workspace_bytes(0, 1, 32, 8, 8, 16) == 0
    # gate adjoint: one (dz, dg*g) pair of per-channel sums per (b, h, 256-token tile)
    assert lib.kda_gate_bwd_workspace_bytes(2, 3, 300, 8) == 2 * 3 * 2 * 2 * 8 * 4
    assert lib.kda_gate_bwd_workspace_bytes(1, 1, 0, 8) == 0
    assert lib.kda_gate_bwd_workspace_bytes(1, 1, 16, 0) == 0
    # paired forward: bf16 with V = 128 and chunk 32/64 only; one ring per head up to 128
    fw = lib.kda_chunk_fwd_workspace_bytes
    one = fw(1, 1, 64, 128, 128, 64, 1)
    assert one > 6 * 35 * 1024 and fw(4, 32, 16384, 128, 128, 64, 1) == 256 + 128 * (one - 256)
    assert fw(8, 32, 64, 128, 128, 64, 1) == fw(4, 32, 64, 128, 128, 64, 1)
    assert fw(1, 1, 64, 128, 128, 32, 1) == one
    assert fw(1, 1, 64, 64, 128, 64, 1) < one and fw(1, 1, 64, 8, 128, 64, 1) == fw(1, 1, 64, 32, 128, 64, 1) > 0
    for args in ((1, 1, 64, 128, 128, 16, 1), (1, 1, 64, 128, 64, 64, 1), (1, 1, 64, 128, 128, 64, 0),
                 (1, 1, 0, 128, 128, 64, 1), (0, 1, 64, 128, 128, 64, 1), (1, 1, 64, 128, 96, 64, 1)):
        assert fw(*args) == 0, args


def _gpu_visible():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="fake device pointers: CPU-only check")
def test_argument_errors_before_launch():
    lib = _lib()
    P = ctypes.c_void_p
    fake = [P(0x10000 * (i + 1)) for i in range(12)]
    q, k, v, z, A, dt, b, s_in, o, s_out = fake[:10]
    rej0 = (ctypes.c_ulonglong * 6)()
    lib.kda_get_counters(rej0, 6)
    # null input
    assert lib.kda_chunk_fwd(None, k, v, z, A, dt, b, s_in, 0.1, 64, o, s_out, None, 0, 1, 1, 16, 8, 8, 0, None) == -1
    # bad dtype
    assert lib.kda_chunk_fwd(q, k, v, z, A, dt, b, s_in, 0.1, 64, o, s_out, None, 0, 1, 1, 16, 8, 8, 7, None) == -3
    # bad shapes
    assert lib.kda_chunk_fwd(q, k, v, z, A, dt, b, s_in, 0.1, 64, o, s_out, None, 0, 1, 1, 16, 12, 8, 0, None) == -2
    assert lib.kda_chunk_fwd(q, k, v, z, A, dt, b, s_in, 0.1, 64, o, s_out, None, 0, 0, 1, 16, 8, 8, 0, None) == -2
    assert lib.kda_chunk_fwd(q, k, v, z, A, dt, b, s_in, 0.1, 64, o, s_out, None, 0, 1, 1, -1, 8, 8, 0, None) == -2
    # one head's sequence too long for 32-bit offsets (2^31 / (128 * 2) tokens, bf16)
    assert lib.kda_chunk_fwd(q, k, v, z, A, dt, b, s_in, 0.1, 64, o, s_out, None, 0, 1, 1, 1 << 23, 128, 128, 1,
                             None) == -2
    # bad chunk
    assert lib.kda_chunk_fwd(q, k, v, z, A, dt, b, s_in, 0.1, 48, o, s_out, None, 0, 1, 1, 16, 8, 8, 0, None) == -4
    # activation pointer not aligned to two elements
    assert lib.kda_chunk_fwd(q, P(0x20002), v, z, A, dt, b, s_in, 0.1, 64, o, s_out, None, 0, 1, 1, 16, 8, 8, 1,
                             None) == -8
    assert lib.kda_chunk_fwd(q, k, v, P(0x40004), A, dt, b, s_in, 0.1, 64, o, s_out, None, 0, 1, 1, 16, 8, 8, 0,
                             None) == -8
    # output aliasing an input
    assert lib.kda_chunk_fwd(q, k, v, z, A, dt, b, s_in, 0.1, 64, q, s_out, None, 0, 1, 1, 16, 8, 8, 0, None) == -5
    assert lib.kda_chunk_fwd(q, k, v, z, A, dt, b, s_in, 0.1, 64, o, k, None, 0, 1, 1, 16, 8, 8, 0, None) == -5
    # decode step
    assert lib.kda_recurrent_step(q, k, v, z, A, dt, b, None, 0.1, o, 1, 1, 8, 8, 0, None) == -1
    assert lib.kda_recurrent_step(q, k, v, z, A, dt, b, s_in, 0.1, o, 1, 1, 8, 24, 0, None) == -2
    assert lib.kda_recurrent_step(q, k, v, z, A, dt, b, s_in, 0.1, q, 1, 1, 8, 8, 0, None) == -5
    # the state overlapping beta, A_log or dt_bias; o overlapping A_log (decode step), and
    # the forward's outputs overlapping A_log or dt_bias: each written while still read
    assert lib.kda_recurrent_step(q, k, v, z, A, dt, b, b, 0.1, o, 1, 1, 8, 8, 0, None) == -5
    assert lib.kda_recurrent_step(q, k, v, z, A, dt, b, A, 0.1, o, 1, 1, 8, 8, 0, None) == -5
    assert lib.kda_recurrent_step(q, k, v, z, A, dt, b, s_in, 0.1, dt, 1, 1, 8, 8, 0, None) == -5
    assert lib.kda_chunk_fwd(q, k, v, z, A, dt, b, s_in, 0.1, 64, A, s_out, None, 0, 1, 1, 16, 8, 8, 0, None) == -5
    assert lib.kda_chunk_fwd(q, k, v, z, A, dt, b, s_in, 0.1, 64, o, dt, None, 0, 1, 1, 16, 8, 8, 0, None) == -5
    # gate
    assert lib.kda_gate(None, A, dt, o, None, 1, 1, 4, 8, 0, None) == -1
    assert lib.kda_gate(z, A, dt, z, None, 1, 1, 4, 8, 0, None) == -5
    # adjoint: bf16 not taken yet; workspace missing / too small
    g = fake[10:12]
    args = [q, k, v, z, A, dt, b, s_in, 0.1, 64, o, None, *fake[:6]]
    assert lib.kda_chunk_bwd(*args, g[0], 1 << 40, 1, 1, 16, 8, 8, 1, None) == -3
    assert lib.kda_chunk_bwd(*args, None, 0, 1, 1, 16, 8, 8, 0, None) == -7
    assert lib.kda_chunk_bwd(*args, g[0], 16, 1, 1, 16, 8, 8, 0, None) == -7
    assert lib.kda_chunk_bwd(*args, P(g[0].value + 4), 1 << 40, 1, 1, 16, 8, 8, 0, None) == -8
    argv = [q, k, P(v.value + 8)] + args[3:]                   # v 8-byte but not 16-byte aligned
    assert lib.kda_chunk_bwd(*argv, g[0], 1 << 40, 1, 1, 16, 8, 8, 0, None) == -8
    argq = [P(q.value + 8)] + args[1:]                          # q likewise
    assert lib.kda_chunk_bwd(*argq, g[0], 1 << 40, 1, 1, 16, 8, 8, 0, None) == -8
    # gate adjoint: no output / null input, bad dtype, bad shape, workspace, aliasing
    ws = fake[11]
    assert lib.kda_gate_bwd(z, A, dt, g[0], None, None, None, ws, 1 << 20, 1, 1, 16, 8, 0, None) == -1
    assert lib.kda_gate_bwd(None, A, dt, g[0], o, None, None, ws, 1 << 20, 1, 1, 16, 8, 0, None) == -1
    assert lib.kda_gate_bwd(z, A, dt, g[0], o, None, None, ws, 1 << 20, 1, 1, 16, 8, 5, None) == -3
    assert lib.kda_gate_bwd(z, A, dt, g[0], o, None, None, ws, 1 << 20, 1, 1, 16, 0, 0, None) == -2
    assert lib.kda_gate_bwd(z, A, dt, g[0], o, None, None, None, 0, 1, 1, 16, 8, 0, None) == -7
    assert lib.kda_gate_bwd(z, A, dt, g[0], o, None, None, ws, 4, 1, 1, 16, 8, 0, None) == -7
    assert lib.kda_gate_bwd(z, A, dt, g[0], z, None, None, ws, 1 << 20, 1, 1, 16, 8, 0, None) == -5
    assert lib.kda_gate_bwd(z, A, dt, g[0], o, dt, None, ws, 1 << 20, 1, 1, 16, 8, 0, None) == -5
    assert lib.kda_gate_bwd(z, A, dt, g[0], P(g[0].value + 4), None, None, ws, 1 << 20, 1, 1, 16, 8, 0,
                            None) == -5
    # the allocation-free gate adjoint: the same checks, and sizes beyond its built-in
    # scratch (16 MiB of partial sums: 256 heads x 64 tiles x 2 x 128 channels x 4 B fit,
    # 257 heads do not) rejected before anything runs
    assert lib.kda_gate_bwd_noalloc(None, A, dt, g[0], o, None, None, 1, 1, 16, 8, 0, None) == -1
    assert lib.kda_gate_bwd_noalloc(z, A, dt, g[0], o, None, None, 1, 1, 16, 8, 5, None) == -3
    assert lib.kda_gate_bwd_noalloc(z, A, dt, g[0], o, None, None, 1, 1, 16, 0, 0, None) == -2
    assert lib.kda_gate_bwd_noalloc(z, A, dt, g[0], z, None, None, 1, 1, 16, 8, 0, None) == -5
    assert lib.kda_gate_bwd_workspace_bytes(1, 256, 16384, 128) == 16 << 20
    assert lib.kda_gate_bwd_noalloc(z, A, dt, g[0], o, None, None, 1, 257, 16384, 128, 0, None) == -10
    assert lib.kda_gate_bwd_noalloc(z, A, dt, g[0], o, None, None, 2, 1, 16384 * 128 + 1, 128, 0, None) == -10
    rej1 = (ctypes.c_ulonglong * 6)()
    lib.kda_get_counters(rej1, 6)
    assert rej1[4] - rej0[4] == 42 and list(rej1[:4]) == list(rej0[:4]) and rej1[5] == rej0[5]


@pytest.mark.skipif(_gpu_visible(), reason="fake device pointers: CPU-only check")
def test_scalar_decay_argument_errors_before_launch():
    lib = _lib()
    P = ctypes.c_void_p
    q, k, v, a, A, dt, b, s_in, o, s_out = [P(0x10000 * (i + 1)) for i in range(10)]
    rej0 = (ctypes.c_ulonglong * 6)()
    lib.kda_get_counters(rej0, 6)
    f = lib.kda_chunk_fwd_scalar
    assert f(q, k, v, None, A, dt, b, s_in, 0.1, 64, o, s_out, None, 0, 1, 1, 16, 8, 8, 1, None) == -1
    assert f(q, k, v, a, A, dt, b, s_in, 0.1, 64, o, s_out, None, 0, 1, 1, 16, 8, 8, 9, None) == -3
    assert f(q, k, v, a, A, dt, b, s_in, 0.1, 64, o, s_out, None, 0, 1, 1, 16, 8, 24, 1, None) == -2
    assert f(q, k, v, a, A, dt, b, s_in, 0.1, 8, o, s_out, None, 0, 1, 1, 16, 8, 8, 1, None) == -4
    # the gate input needs one-element alignment only; q, k, v keep the two-element rule
    assert f(q, k, v, P(0x40001), A, dt, b, s_in, 0.1, 64, o, s_out, None, 0, 1, 1, 16, 8, 8, 1, None) == -8
    assert f(q, P(0x20002), v, a, A, dt, b, s_in, 0.1, 64, o, s_out, None, 0, 1, 1, 16, 8, 8, 1, None) == -8
    # o or state_out over the gate input (B*H*T elements)
    assert f(q, k, v, a, A, dt, b, s_in, 0.1, 64, P(a.value + 2), s_out, None, 0, 1, 1, 16, 8, 8, 1, None) == -5
    assert f(q, k, v, a, A, dt, b, s_in, 0.1, 64, o, P(a.value - 4), None, 0, 1, 1, 16, 8, 8, 0, None) == -5
    g = lib.kda_recurrent_step_scalar
    assert g(q, k, v, None, A, dt, b, s_in, 0.1, o, 1, 1, 8, 8, 0, None) == -1
    assert g(q, k, v, a, A, dt, b, s_in, 0.1, o, 1, 1, 8, 12, 0, None) == -2
    assert g(q, k, v, a, A, dt, b, s_in, 0.1, a, 1, 1, 8, 8, 0, None) == -5
    rej1 = (ctypes.c_ulonglong * 6)()
    lib.kda_get_counters(rej1, 6)
    assert rej1[4] - rej0[4] == 11 and list(rej1[:4]) == list(rej0[:4])


@pytest.mark.skipif(_gpu_visible(), reason="fake device pointers: CPU-only check")
def test_paired_forward_workspace_errors_before_launch():
    lib = _lib()
    P = ctypes.c_void_p
    q, k, v, z, A, dt, b, s_in, o, s_out = [P(0x1000000 * (i + 1)) for i in range(10)]
    need = lib.kda_chunk_fwd_workspace_bytes(1, 2, 64, 128, 128, 64, 1)
    ws = P(0x40000000)
    rej0 = (ctypes.c_ulonglong * 6)()
    lib.kda_get_counters(rej0, 6)
    f = lib.kda_chunk_fwd
    # too small, misaligned, overlapping an input or an output
    assert f(q, k, v, z, A, dt, b, s_in, 0.1, 64, o, s_out, ws, need - 1, 1, 2, 64, 128, 128, 1, None) == -7
    assert f(q, k, v, z, A, dt, b, s_in, 0.1, 64, o, s_out, P(ws.value + 16), need, 1, 2, 64, 128, 128, 1,
             None) == -8
    assert f(q, k, v, z, A, dt, b, s_in, 0.1, 64, o, s_out, P(v.value - 256), need, 1, 2, 64, 128, 128, 1,
             None) == -5
    assert f(q, k, v, z, A, dt, b, s_in, 0.1, 64, o, s_out, P(s_out.value - 256), need, 1, 2, 64, 128, 128, 1,
             None) == -5
    assert f(q, k, v, z, A, dt, b, s_in, 0.1, 64, o, s_out, P(A.value), need, 1, 2, 64, 128, 128, 1,
             None) == -5
    g = lib.kda_chunk_fwd_scalar
    assert g(q, k, v, z, A, dt, b, s_in, 0.1, 32, o, s_out, ws, 100, 1, 2, 64, 128, 128, 1, None) == -7
    assert lib.kda_chunk_fwd_status(None, None) == -1
    rej1 = (ctypes.c_ulonglong * 6)()
    lib.kda_get_counters(rej1, 6)
    assert rej1[4] - rej0[4] == 7 and list(rej1[:4]) == list(rej0[:4])


def test_exchange_timeout_setting():
    lib = _lib()
    assert lib.kda_set_exchange_timeout_us(0) == 0
    assert lib.kda_set_exchange_timeout_us(1000000) == 0
