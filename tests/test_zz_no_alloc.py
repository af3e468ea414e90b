"""The allocation-free gate adjoint (kda_gate_bwd_noalloc) against the entry point that
takes a caller workspace (kda_gate_bwd), through the C ABI: two calls in a row, the
second smaller than the first (the built-in scratch keeps the first call's partial sums,
which the second must not pick up), then T = 0.  The two entry points run the same
kernels in the same order, so the results must be bit-identical; the small call is also
checked against the oracle's gate adjoint."""
import numpy as np
import pytest
import torch

import gated_delta_rule_47_amd as kda
from oracle import kda_ref as R

from gpu_helpers import DEV, host, say, to_dev

pytestmark = pytest.mark.gpu


def _inputs_dev(B, H, T, K, dtype, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    z = (torch.randn((B, H, T, K), generator=g, device=DEV) * 4).to(dtype)
    A_log = torch.linspace(-3.0, 2.0, H, device=DEV)
    dt = 0.5 * torch.randn((H, K), generator=g, device=DEV)
    dg = torch.randn((B, H, T, K), generator=g, device=DEV)
    return z, A_log, dt, dg


def _same(a, b):
    for x, y, name in zip(a, b, ("dz", "dA_log", "d_dt_bias")):
        assert torch.equal(x, y), name


def test_noalloc_gate_bwd_matches_workspace_call_twice_then_smaller():
    # 1: the long workload's gate shape (4 x 32 heads x 16384 tokens, K = 128, bf16):
    #    8 MiB of partial sums, half the scratch
    B, H, T, K = 4, 32, 16384, 128
    assert kda.gate_bwd_workspace_bytes(B, H, T, K) == 8 << 20
    z, A_log, dt, dg = _inputs_dev(B, H, T, K, torch.bfloat16, seed=5)
    say("noalloc call 1", B, H, T, K)
    got = kda.gate_bwd_noalloc(z, A_log, dt, dg)
    ref = kda.gate_bwd(z, A_log, dt, dg)
    torch.cuda.synchronize()
    _same(got, ref)
    del z, dg, got, ref
    # 2: smaller (fewer heads, ragged token tile, K = 64): bit-identical and against the oracle
    rng = np.random.default_rng(7)
    B, H, T, K = 2, 3, 300, 64
    z = (rng.standard_normal((B, H, T, K)) * 4).astype(np.float32)
    A_log = np.array([-3.0, 25.0, 0.0], dtype=np.float32)
    dt = (0.5 * rng.standard_normal((H, K))).astype(np.float32)
    dg = rng.standard_normal((B, H, T, K)).astype(np.float32)
    zd, Ad, dtd, dgd = (to_dev(x, torch.float32) for x in (z, A_log, dt, dg))
    say("noalloc call 2", B, H, T, K)
    got = kda.gate_bwd_noalloc(zd, Ad, dtd, dgd)
    ref = kda.gate_bwd(zd, Ad, dtd, dgd)
    torch.cuda.synchronize()
    _same(got, ref)
    dzr, dAr, ddbr = R.gate_adjoint(z, A_log, dt, dg)
    for name, a, b, tol in (("dz", got[0], dzr, 2e-6), ("dA_log", got[1], dAr, 1e-4), ("d_dt_bias", got[2], ddbr, 1e-4)):
        e = R.rel_err(host(a), b)
        say("  %-10s rel_err %.3e (bar %.0e)" % (name, e, tol))
        assert e <= tol, (name, e)
    # 3: T = 0 (no partial sums at all): zero parameter gradients
    z0 = torch.empty((1, 2, 0, 8), device=DEV)
    dg0 = torch.empty((1, 2, 0, 8), device=DEV)
    _, dA0, ddb0 = kda.gate_bwd_noalloc(z0, Ad[:2].contiguous(), dtd[:2, :8].contiguous(), dg0, want_dz=False)
    torch.cuda.synchronize()
    assert torch.all(dA0 == 0) and torch.all(ddb0 == 0)


def test_noalloc_gate_bwd_rejects_sizes_beyond_its_scratch():
    z = torch.empty((1, 257, 16384, 128), dtype=torch.bfloat16, device=DEV)
    dg = torch.empty((1, 257, 16384, 128), dtype=torch.float32, device=DEV)
    A_log = torch.zeros(257, device=DEV)
    dt = torch.zeros((257, 128), device=DEV)
    with pytest.raises(kda.KdaError) as ei:
        kda.gate_bwd_noalloc(z, A_log, dt, dg, want_dz=False)
    assert ei.value.status == -10
