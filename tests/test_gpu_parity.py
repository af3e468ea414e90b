"""GPU parity: every entry point of libkda against the f64 oracle, through the C ABI.

Bars (max|x - ref| / max|ref| per tensor): 1e-4 for fp32 activations, 2e-2 for
bf16 activations (the stated parity tolerances of the KDA forward), on o and the
final state; the adjoint's gradients at 1e-4 (fp32).  Full-size workloads are
checked on sampled heads, which the oracle evaluates one by one.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_47_amd as kda
import kda_synth as ks
from oracle import kda_ref as R

from gpu_helpers import check, DEV, TOL, act_dtype, host, oracle_heads, oracle_heads_from_slices, say, to_dev, upload

pytestmark = pytest.mark.gpu


def _fwd(d, chunk, scale=None, state_in=True):
    return kda.chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["A_log"], d["dt_bias"], d["beta"],
                         d["state_in"] if state_in else None, scale=scale, chunk=chunk)


_check = check


# ----------------------------------------------------------------------------- gate
# K % 4 == 0 with aligned buffers takes the four-channel kernel: at K = 64 each thread
# keeps one channel group, at K = 12 and K = 2056 (more groups than threads) the group
# advances every pass; a bf16 z 8 bytes off a 16-byte boundary still qualifies.  An fp32
# z 8 bytes off, or a bf16 z 4 bytes off, takes the one-channel kernel.  T = 37 leaves a
# ragged last tile.
@pytest.mark.parametrize("dtype,K,off", [("f32", 64, 0), ("bf16", 64, 0), ("f32", 12, 0), ("bf16", 2056, 0),
                                         ("bf16", 64, 4), ("f32", 64, 2), ("bf16", 64, 2)])
def test_gate(dtype, K, off):
    rng = np.random.default_rng(11)
    B, H, T = 2, 3, 37
    z = rng.standard_normal((B, H, T, K)).astype(np.float32) * 4
    z[0, 0, 0, :8] = [-50, -20, -5, 0, 5, 20, 50, 1]
    if dtype == "bf16":
        z = ks.round_bf16(z)
    A_log = np.array([-3.0, 0.0, 25.0], dtype=np.float32)
    dt = (0.5 * rng.standard_normal((H, K))).astype(np.float32)
    zt = torch.bfloat16 if dtype == "bf16" else torch.float32
    zd = to_dev(z, zt)
    if off:
        buf = torch.empty(zd.numel() + off, dtype=zt, device=zd.device)
        zd = buf[off:].view(zd.shape).copy_(zd)
    g, a = kda.gate(zd, to_dev(A_log, torch.float32), to_dev(dt, torch.float32))
    gr, ar = R.gate(z, A_log, dt)
    _check("g", host(g), gr, 2e-6)
    _check("alpha", host(a), ar, 2e-6)
    assert torch.all(g <= 0)


# ----------------------------------------------------------------------------- decode step
@pytest.mark.parametrize("wl_name,T", [("tiny", 32), ("layer", 64), ("nano", 48)])
def test_recurrent_step_matches_token_recurrence(wl_name, T):
    wl = ks.WORKLOADS[wl_name]
    if wl_name == "nano":
        wl = wl.with_(B=2, H=3)
    x = ks.generate(wl, T=T)
    d = upload(wl, x)
    S = d["state_in"].clone()
    os_ = []
    for t in range(T):
        os_.append(kda.recurrent_step(d["q"][:, :, t].contiguous(), d["k"][:, :, t].contiguous(),
                                      d["v"][:, :, t].contiguous(), d["z"][:, :, t].contiguous(),
                                      d["A_log"], d["dt_bias"], d["beta"][:, :, t].contiguous(), S))
    o = torch.stack(os_, dim=2)
    o_ref, S_ref = oracle_heads(wl, x, [(b, h) for b in range(wl.B) for h in range(wl.H)])
    say(wl_name)
    _check("o", host(o).reshape(1, -1, T, wl.V), o_ref, TOL[wl.dtype])
    _check("state", host(S).reshape(1, -1, wl.K, wl.V), S_ref, 1e-4)


def _decode(d, T0, T1):
    """Tokens T0 .. T1-1 through the decode step, from the state in d["S"] (updated)."""
    os_ = []
    for t in range(T0, T1):
        os_.append(kda.recurrent_step(d["q"][:, :, t].contiguous(), d["k"][:, :, t].contiguous(),
                                      d["v"][:, :, t].contiguous(), d["z"][:, :, t].contiguous(),
                                      d["A_log"], d["dt_bias"], d["beta"][:, :, t].contiguous(), d["S"]))
    return torch.stack(os_, dim=2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_recurrent_step_k128(dtype):
    """The decode step at K = V = 128 (two 64-column value tiles per head), fp32 and bf16
    activations, 40 tokens against the token recurrence."""
    base = ks.WORKLOADS["layer"] if dtype == "f32" else ks.WORKLOADS["nano"]
    wl = base.with_(B=2, H=3, K=128, V=128, state="normal:0.1")
    T = 40
    x = ks.generate(wl, T=T)
    d = upload(wl, x)
    d["S"] = d["state_in"].clone()
    o = _decode(d, 0, T)
    o_ref, S_ref = oracle_heads(wl, x, [(b, h) for b in range(2) for h in range(3)])
    say("decode K=V=128", dtype)
    _check("o", host(o).reshape(1, 6, T, 128), o_ref, TOL[wl.dtype])
    _check("state", host(d["S"]).reshape(1, 6, 128, 128), S_ref, 1e-4)


def test_prefill_decode_handoff_long_workload():
    """The long workload's shape (B=4, H=32, K=V=128, bf16): the chunked forward over the
    first 16380 tokens, then the decode step for the last 4 from its final state, on the
    whole batch; eight heads (one per XCD) against the oracle over all 16384 tokens."""
    wl = ks.WORKLOADS["long"]
    T, Tp = wl.T, wl.T - 4
    say("generating long")
    x = ks.generate(wl)
    d = upload(wl, x)
    del x
    o_p, S_p = kda.chunk_fwd(*(d[n][:, :, :Tp].contiguous() for n in ("q", "k", "v", "z")), d["A_log"],
                             d["dt_bias"], d["beta"][:, :, :Tp].contiguous(), d["state_in"], chunk=wl.chunk)
    d["S"] = S_p
    o_d = _decode(d, Tp, T)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_heads_from_slices(wl, LONG_HEADS)
    _check("o prefill", np.stack([host(o_p[b, h]) for b, h in LONG_HEADS])[None], o_ref[:, :, :Tp], TOL["bf16"])
    _check("o decode", np.stack([host(o_d[b, h]) for b, h in LONG_HEADS])[None], o_ref[:, :, Tp:], TOL["bf16"])
    _check("state", np.stack([host(d["S"][b, h]) for b, h in LONG_HEADS])[None], S_ref, TOL["bf16"])


# ----------------------------------------------------------------------------- chunked forward
@pytest.mark.parametrize("wl_name", ["tiny", "layer"])
def test_chunk_fwd_fp32_workloads(wl_name):
    wl = ks.WORKLOADS[wl_name]
    x = ks.generate(wl)
    d = upload(wl, x)
    o, S = _fwd(d, wl.chunk)
    heads = [(b, h) for b in range(wl.B) for h in range(wl.H)]
    o_ref, S_ref = oracle_heads(wl, x, heads)
    say(wl_name)
    _check("o", host(o).reshape(1, -1, wl.T, wl.V), o_ref, TOL["f32"])
    _check("state", host(S).reshape(1, -1, wl.K, wl.V), S_ref, TOL["f32"])


def test_chunk_fwd_nano_short_all_heads():
    wl = ks.WORKLOADS["nano"]
    x = ks.generate(wl, T=384)
    d = upload(wl, x)
    o, S = _fwd(d, wl.chunk)
    o_ref, S_ref = oracle_heads(wl, x, [(b, h) for b in range(wl.B) for h in range(wl.H)])
    _check("o", host(o).reshape(1, -1, 384, wl.V), o_ref, TOL["bf16"])
    _check("state", host(S).reshape(1, -1, wl.K, wl.V), S_ref, TOL["bf16"])


# Sampled heads, one per XCD: the forward runs workgroup x on XCD x % 8 and maps the
# value tiles of head bh to XCD bh // (heads / 8) (both tiles of a head on one XCD).
NANO_HEADS = [(0, 0), (1, 3), (2, 6), (3, 1), (4, 4), (5, 7), (6, 2), (7, 5)]        # bh // 8 = 0..7
LONG_HEADS = [(0, 0), (0, 21), (1, 10), (1, 31), (2, 4), (2, 25), (3, 14), (3, 19)]  # bh // 16 = 0..7


@pytest.mark.parametrize("wl_name,heads", [("nano", NANO_HEADS), ("long", LONG_HEADS)])
def test_chunk_fwd_full_size_sampled_heads(wl_name, heads):
    """The full workload, launched exactly as the benchmark launches it; the oracle
    recomputes a few heads from their regenerated slices."""
    wl = ks.WORKLOADS[wl_name]
    say("generating", wl_name)
    x = ks.generate(wl)
    d = upload(wl, x)
    del x
    o, S = _fwd(d, wl.chunk)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    o_ref, S_ref = oracle_heads_from_slices(wl, heads)
    og = np.stack([host(o[b, h]) for b, h in heads])[None]
    Sg = np.stack([host(S[b, h]) for b, h in heads])[None]
    _check("o", og, o_ref, TOL["bf16"])
    _check("state", Sg, S_ref, TOL["bf16"])


@pytest.mark.parametrize("T", [1024, 4096])
def test_chunk_fwd_long_error_growth_with_T(T):
    """bf16 error against the sequence length at the long workload's shape (B=4, H=32,
    K=V=128): T = 1k and 4k here, 16k in the full-size test, on the same eight heads (one
    per XCD).  The fp32 state carries the whole sequence, so a drift of the carried
    state would show as growth with T."""
    wl = ks.WORKLOADS["long"]
    x = ks.generate(wl, T=T)
    d = upload(wl, x)
    o, S = _fwd(d, wl.chunk)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_heads(wl, x, LONG_HEADS)
    say("long, T =", T)
    _check("o", np.stack([host(o[b, h]) for b, h in LONG_HEADS])[None], o_ref, TOL["bf16"])
    _check("state", np.stack([host(S[b, h]) for b, h in LONG_HEADS])[None], S_ref, TOL["bf16"])


CASES = [  # (dtype, K, V, chunk, T)
    ("f32", 8, 8, 16, 1), ("f32", 8, 8, 16, 45), ("f32", 16, 32, 32, 70), ("f32", 32, 64, 64, 130),
    ("f32", 64, 16, 32, 77), ("f32", 128, 128, 64, 100), ("f32", 128, 32, 16, 40), ("f32", 64, 128, 64, 129),
    ("bf16", 32, 32, 32, 97), ("bf16", 64, 64, 64, 200), ("bf16", 128, 128, 64, 150), ("bf16", 128, 64, 32, 65),
    ("bf16", 16, 8, 16, 33), ("bf16", 8, 128, 64, 64), ("bf16", 64, 128, 16, 50),
    # the gate/decay stage runs whole blocks through a loop without the identity-token test and the
    # rest (a ragged last block, the steps past the end) through the general one: 7 whole blocks and
    # a ragged eighth, and 9 whole blocks (three iterations of the first loop, then the final steps)
    ("bf16", 128, 128, 64, 229), ("bf16", 64, 64, 32, 288),
]


@pytest.mark.parametrize("dtype,K,V,chunk,T", CASES)
def test_chunk_fwd_shapes_chunks_ragged(dtype, K, V, chunk, T):
    base = ks.WORKLOADS["nano"] if dtype == "bf16" else ks.WORKLOADS["layer"].with_(a_log="uniform:-3,1")
    wl = base.with_(B=2, H=2, K=K, V=V, chunk=chunk, state="normal:0.1")
    x = ks.generate(wl, T=T)
    d = upload(wl, x)
    o, S = _fwd(d, chunk)
    o_ref, S_ref = oracle_heads(wl, x, [(b, h) for b in range(2) for h in range(2)])
    say(dtype, K, V, chunk, T)
    _check("o", host(o).reshape(1, 4, T, V), o_ref, TOL[dtype])
    _check("state", host(S).reshape(1, 4, K, V), S_ref, TOL[dtype] if dtype == "bf16" else 1e-4)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_saturated_gates_take_the_token_path(dtype):
    """A_log = 20 and large z: alpha underflows to 0 within a token, so the block
    factors would overflow; those chunks run token by token.  Mixed with mild heads."""
    base = ks.WORKLOADS["nano"] if dtype == "bf16" else ks.WORKLOADS["layer"]
    wl = base.with_(B=1, H=4, K=64, V=64, chunk=64, a_log="list:20,-3,8,0", state="normal:0.1")
    x = ks.generate(wl, T=150)
    x["z"][0, 2, 40:70] += 6.0
    if dtype == "bf16":
        x["z"] = ks.round_bf16(x["z"])
    d = upload(wl, x)
    o, S = _fwd(d, 64)
    o_ref, S_ref = oracle_heads(wl, x, [(0, h) for h in range(4)])
    _check("o", host(o).reshape(1, 4, 150, 64), o_ref, TOL[dtype])
    _check("state", host(S).reshape(1, 4, 64, 64), S_ref, TOL[dtype])


def test_T0_state_none_alias_and_scale():
    wl = ks.WORKLOADS["layer"].with_(B=1, H=2, state="normal:0.1")
    x = ks.generate(wl, T=70)
    d = upload(wl, x)
    # T = 0: state_out = state_in, no output rows
    o0, S0 = kda.chunk_fwd(d["q"][:, :, :0], d["k"][:, :, :0], d["v"][:, :, :0], d["z"][:, :, :0], d["A_log"],
                           d["dt_bias"], d["beta"][:, :, :0], d["state_in"], chunk=64)
    assert o0.numel() == 0 and torch.equal(S0, d["state_in"])
    # no initial state == zero initial state
    o1, S1 = _fwd(d, 64, state_in=False)
    o2, S2 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["A_log"], d["dt_bias"], d["beta"],
                           torch.zeros_like(d["state_in"]), chunk=64)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    # in place: state_out == state_in
    ref_o, ref_S = _fwd(d, 64)
    st = d["state_in"].clone()
    o3, S3 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["A_log"], d["dt_bias"], d["beta"], st, chunk=64,
                           state_out=st)
    assert S3.data_ptr() == st.data_ptr() and torch.equal(S3, ref_S) and torch.equal(o3, ref_o)
    # scale: o linear in it, state independent of it; scale = 0 gives o = 0
    oa, Sa = _fwd(d, 64, scale=1.0)
    ob, Sb = _fwd(d, 64, scale=0.25)
    oz, Sz = _fwd(d, 64, scale=0.0)
    assert torch.equal(Sa, Sb) and torch.equal(Sa, Sz) and torch.all(oz == 0)
    assert R.rel_err(host(ob), 0.25 * host(oa)) < 1e-6


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_resume_split_and_prefill_decode_handoff(dtype):
    base = ks.WORKLOADS["nano"] if dtype == "bf16" else ks.WORKLOADS["layer"].with_(a_log="uniform:-3,1")
    wl = base.with_(B=1, H=2, state="normal:0.1")
    x = ks.generate(wl, T=200)
    d = upload(wl, x)
    o, S = _fwd(d, 64)
    cut = 77
    sl = lambda t, a, b_: t[:, :, a:b_].contiguous()
    oa, Sa = kda.chunk_fwd(*(sl(d[n], 0, cut) for n in ("q", "k", "v", "z")), d["A_log"], d["dt_bias"],
                           sl(d["beta"], 0, cut), d["state_in"], chunk=64)
    ob, Sb = kda.chunk_fwd(*(sl(d[n], cut, 199) for n in ("q", "k", "v", "z")), d["A_log"], d["dt_bias"],
                           sl(d["beta"], cut, 199), Sa, chunk=32)
    ot = kda.recurrent_step(*(d[n][:, :, 199].contiguous() for n in ("q", "k", "v", "z")), d["A_log"],
                            d["dt_bias"], d["beta"][:, :, 199].contiguous(), Sb)
    got = torch.cat([oa, ob, ot[:, :, None]], dim=2)
    tol = TOL[dtype]
    assert R.rel_err(host(got), host(o)) < tol and R.rel_err(host(Sb), host(S)) < tol


def test_determinism_and_poisoned_outputs():
    wl = ks.WORKLOADS["nano"].with_(B=2, H=4, K=128, V=128)
    x = ks.generate(wl, T=300)
    d = upload(wl, x)
    o1 = torch.full((2, 4, 300, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    S1 = torch.full((2, 4, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
    kda.chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["A_log"], d["dt_bias"], d["beta"], d["state_in"], chunk=64,
                  out=o1, state_out=S1)
    o2, S2 = _fwd(d, 64)
    assert torch.isfinite(o1.float()).all() and torch.isfinite(S1).all()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


# ----------------------------------------------------------------------------- adjoint
def _bwd(d, chunk, d_state_out=None):
    return kda.chunk_bwd(d["q"], d["k"], d["v"], d["z"], d["A_log"], d["dt_bias"], d["beta"], d["state_in"],
                         d["d_out"], d_state_out, chunk=chunk)


def _oracle_bwd(wl, x, heads, d_state_out=None):
    sel = lambda a: np.stack([a[b, h] for b, h in heads])[None]
    g, _ = R.gate(sel(x["z"]), np.array([x["A_log"][h] for _, h in heads]),
                  np.stack([x["dt_bias"][h] for _, h in heads]))
    dso = None if d_state_out is None else sel(d_state_out)
    return R.adjoint(sel(x["q"]), sel(x["k"]), sel(x["v"]), g, sel(x["beta"]), sel(x["state_in"]),
                     sel(x["d_out"]), dso)


GRADS = ("dq", "dk", "dv", "dg", "dbeta", "dstate_in")


@pytest.mark.parametrize("K,V,chunk,T,with_ds", [(8, 8, 16, 32, False), (8, 8, 16, 45, True), (32, 64, 32, 100, True),
                                                 (64, 16, 64, 130, False), (128, 128, 64, 70, True)])
def test_chunk_bwd_small(K, V, chunk, T, with_ds):
    wl = ks.WORKLOADS["adjoint"].with_(B=2, H=2, K=K, V=V, chunk=chunk)
    x = ks.generate(wl, T=T)
    d = upload(wl, x)
    dso = np.random.default_rng(5).standard_normal((2, 2, K, V)).astype(np.float32) if with_ds else None
    gr = _bwd(d, chunk, to_dev(dso, torch.float32) if with_ds else None)
    heads = [(b, h) for b in range(2) for h in range(2)]
    ref = _oracle_bwd(wl, x, heads, dso)
    say(K, V, chunk, T, with_ds)
    for n in GRADS:
        got = host(gr[n]).reshape(ref[n].shape)
        _check(n, got, ref[n], 1e-4)


@pytest.mark.parametrize("T", [1, 150])
def test_chunk_bwd_saturated_gates_take_the_token_path(T):
    """Heads whose decay inside a 32-token chunk leaves the factorised form's range
    (A_log = 20 and 8, and a run of large z on a third head) are evaluated token by token
    in the reverse and gradient passes; the heads next to them keep the MFMA path."""
    wl = ks.WORKLOADS["adjoint"].with_(B=1, H=4, a_log="list:20,-3,8,0")
    x = ks.generate(wl, T=T)
    if T > 70:
        x["z"][0, 2, 40:70] += 6.0
    d = upload(wl, x)
    dso = np.random.default_rng(8).standard_normal((1, 4, wl.K, wl.V)).astype(np.float32)
    gr = _bwd(d, wl.chunk, to_dev(dso, torch.float32))
    heads = [(0, h) for h in range(4)]
    ref = _oracle_bwd(wl, x, heads, dso)
    say("saturated adjoint, T =", T)
    for n in GRADS:
        got = host(gr[n]).reshape(ref[n].shape)
        _check(n, got, ref[n], 1e-4)


def test_chunk_bwd_adjoint_workload_sampled_heads():
    wl = ks.WORKLOADS["adjoint"]
    x = ks.generate(wl)
    d = upload(wl, x)
    gr = _bwd(d, wl.chunk)
    torch.cuda.synchronize()
    heads = [(0, 0), (0, 7), (1, 8), (1, 15)]
    ref = _oracle_bwd(wl, x, heads)
    for n in GRADS:
        got = np.stack([host(gr[n][b, h]) for b, h in heads])[None]
        _check(n, got, ref[n], 1e-4)


# ----------------------------------------------------------------------------- gate adjoint
# K = 64 and 256 take the four-channel first pass (K = 256: two column passes in the
# reduction); K = 24 and 320 (K / 4 does not divide the workgroup) the one-channel pass
GATE_BWD_CASES = [("f32", 2, 3, 300, 64), ("bf16", 2, 3, 300, 64), ("f32", 1, 2, 17, 24), ("f32", 1, 2, 0, 8),
                  ("bf16", 1, 2, 513, 320), ("f32", 1, 2, 70, 256)]


def _gate_bwd_inputs(B, H, T, K, dtype, seed=23):
    rng = np.random.default_rng(seed)
    z = (rng.standard_normal((B, H, T, K)) * 4).astype(np.float32)
    if T:
        z[0, 0, 0, :8] = [-50, -20, -5, 0, 5, 20, 50, 1]
    if dtype == "bf16":
        z = ks.round_bf16(z)
    A_log = np.array([-3.0, 25.0, 0.0][:H], dtype=np.float32)     # head 1 clamped: no dA_log
    dt = (0.5 * rng.standard_normal((H, K))).astype(np.float32)
    dg = rng.standard_normal((B, H, T, K)).astype(np.float32)
    return z, A_log, dt, dg


@pytest.mark.parametrize("dtype,B,H,T,K", GATE_BWD_CASES)
def test_gate_bwd(dtype, B, H, T, K):
    """dz, dA_log and d dt_bias against the oracle's gate adjoint: ragged token tiles,
    K above one pass of 256 lanes, T = 0, a clamped multiplier, dz computed in place
    over dg, and bitwise-repeatable parameter gradients."""
    z, A_log, dt, dg = _gate_bwd_inputs(B, H, T, K, dtype)
    zd = to_dev(z, torch.bfloat16 if dtype == "bf16" else torch.float32)
    Ad, dtd, dgd = (to_dev(x, torch.float32) for x in (A_log, dt, dg))
    dz, dA, ddb = kda.gate_bwd(zd, Ad, dtd, dgd)
    dzr, dAr, ddbr = R.gate_adjoint(z, A_log, dt, dg)
    say(dtype, B, H, T, K)
    if T:
        _check("dz", host(dz), dzr, 2e-6)
        _check("dA_log", host(dA), dAr, 1e-4)
        _check("d_dt_bias", host(ddb), ddbr, 1e-4)
        if H > 1:
            assert host(dA)[1] == 0.0
    else:
        assert np.all(host(dA) == 0.0) and np.all(host(ddb) == 0.0)
    _, dA2, ddb2 = kda.gate_bwd(zd, Ad, dtd, dgd, want_dz=False)
    assert torch.equal(dA, dA2) and torch.equal(ddb, ddb2)
    if T:
        dg_inplace = dgd.clone()
        dzi, _, _ = kda.gate_bwd(zd, Ad, dtd, dg_inplace, dz_out=dg_inplace)
        assert dzi.data_ptr() == dg_inplace.data_ptr()
        assert torch.equal(dzi, dz)


@pytest.mark.parametrize("K", [64, 10])
def test_gate_and_gate_bwd_without_bias_or_alpha(K):
    """No dt_bias (a null pointer: zero bias) and no alpha output, through both gate
    kernels (K = 64: four channels per thread; K = 10: one channel) and both first
    passes of the gate adjoint; the same against the oracle with a zero bias."""
    rng = np.random.default_rng(41)
    B, H, T = 2, 3, 45
    z = (rng.standard_normal((B, H, T, K)) * 4).astype(np.float32)
    A_log = np.array([-3.0, 0.5, 25.0], dtype=np.float32)
    dg = rng.standard_normal((B, H, T, K)).astype(np.float32)
    zero = np.zeros((H, K), dtype=np.float32)
    zd, Ad, dgd = to_dev(z, torch.float32), to_dev(A_log, torch.float32), to_dev(dg, torch.float32)
    g, a = kda.gate(zd, Ad, None, want_alpha=False)
    assert a is None
    gr, _ = R.gate(z, A_log, zero)
    _check("g", host(g), gr, 2e-6)
    dz, dA, ddb = kda.gate_bwd(zd, Ad, None, dgd)
    dzr, dAr, ddbr = R.gate_adjoint(z, A_log, zero, dg)
    _check("dz", host(dz), dzr, 2e-6)
    _check("dA_log", host(dA), dAr, 1e-4)
    _check("d_dt_bias", host(ddb), ddbr, 1e-4)


def test_gate_bwd_after_chunk_bwd_end_to_end():
    """The training chain: the adjoint's dg fed to the gate adjoint gives dz, dA_log and
    d dt_bias of sum(o * d_o); the oracle runs the same chain in f64."""
    K, V, chunk, T = 8, 8, 16, 45
    wl = ks.WORKLOADS["adjoint"].with_(B=2, H=2, K=K, V=V, chunk=chunk)
    x = ks.generate(wl, T=T)
    d = upload(wl, x)
    gr = _bwd(d, chunk, None)
    dz, dA, ddb = kda.gate_bwd(d["z"], d["A_log"], d["dt_bias"], gr["dg"])
    heads = [(b, h) for b in range(2) for h in range(2)]
    ref = _oracle_bwd(wl, x, heads, None)
    dg_ref = ref["dg"].reshape(2, 2, T, K)
    dzr, dAr, ddbr = R.gate_adjoint(x["z"], x["A_log"], x["dt_bias"], dg_ref)
    _check("dz", host(dz), dzr, 1e-4)
    _check("dA_log", host(dA), dAr, 1e-4)
    _check("d_dt_bias", host(ddb), ddbr, 1e-4)


def test_gate_bwd_adjoint_workload_full_size():
    """The gate adjoint at the adjoint workload's full size (2 x 16 heads x 8192 tokens,
    K = 128, fp32): dz on sampled heads, the parameter gradients (sums over every token)
    in full, against the oracle."""
    wl = ks.WORKLOADS["adjoint"]
    x = ks.generate(wl)
    dg = np.random.default_rng(31).standard_normal((wl.B, wl.H, wl.T, wl.K)).astype(np.float32)
    d = upload(wl, x)
    dz, dA, ddb = kda.gate_bwd(d["z"], d["A_log"], d["dt_bias"], to_dev(dg, torch.float32))
    torch.cuda.synchronize()
    dzr, dAr, ddbr = R.gate_adjoint(x["z"], x["A_log"], x["dt_bias"], dg)
    for b, h in [(0, 0), (1, 9)]:
        _check("dz[%d,%d]" % (b, h), host(dz[b, h]), dzr[b, h], 2e-6)
    _check("dA_log", host(dA), dAr, 1e-4)
    _check("d_dt_bias", host(ddb), ddbr, 1e-4)


# ----------------------------------------------------------------------------- K = V = 128, bf16, many heads
def test_k128_saturated_gates_and_many_heads():
    """K = V = 128 bf16 (two value-tile workgroups per head): token-path blocks mixed
    with mild heads, more heads than the device has compute units, a ragged tail,
    checked on heads spread over the whole grid."""
    wl = ks.WORKLOADS["nano"].with_(B=2, H=80, K=128, V=128, chunk=64, a_log="uniform:-3,1", state="normal:0.1")
    x = ks.generate(wl, T=45)
    x["A_log"][3] = 20.0
    x["z"][1, 3, 10:30] += 6.0
    x["z"] = ks.round_bf16(x["z"])
    d = upload(wl, x)
    o, S = _fwd(d, 64)
    heads = [(0, 0), (0, 3), (1, 3), (1, 47), (1, 48), (1, 79)]
    o_ref, S_ref = oracle_heads(wl, x, heads)
    og = np.stack([host(o[b, h]) for b, h in heads])[None]
    Sg = np.stack([host(S[b, h]) for b, h in heads])[None]
    _check("o", og, o_ref, TOL["bf16"])
    _check("state", Sg, S_ref, TOL["bf16"])


def test_k128_gate_inputs_beyond_the_direct_softplus_range():
    """The fused kernel takes softplus as log2(1 + 2^x) directly, which is +inf from
    x = z log2(e) >= 128 (z >= ~89): such a block must take the exact token path and still
    match, even where the true decay is mild (A_log = -10, so -g stays tiny), while z = 80
    (2^115, finite) stays on the factorised path."""
    wl = ks.WORKLOADS["nano"].with_(B=1, H=3, K=128, V=128, chunk=64, a_log="list:-10,0,-3", state="normal:0.1")
    x = ks.generate(wl, T=100)
    x["z"][0, 0, 5] = 120.0                     # mild head: only the +inf sends this block to the token path
    x["z"][0, 0, 40:44] = 80.0
    x["z"][0, 1, 70, :64] = 100.0               # half of the channels of one token
    x["z"][0, 2, 33] = 80.0
    x["z"] = ks.round_bf16(x["z"])
    d = upload(wl, x)
    o, S = _fwd(d, 64)
    heads = [(0, 0), (0, 1), (0, 2)]
    o_ref, S_ref = oracle_heads(wl, x, heads)
    og = np.stack([host(o[b, h]) for b, h in heads])[None]
    Sg = np.stack([host(S[b, h]) for b, h in heads])[None]
    assert np.isfinite(og).all() and np.isfinite(Sg).all()
    _check("o", og, o_ref, TOL["bf16"])
    _check("state", Sg, S_ref, TOL["bf16"])


def test_k128_state_none_and_in_place_state():
    wl = ks.WORKLOADS["nano"].with_(B=1, H=4, K=128, V=128, chunk=64, state="normal:0.1")
    x = ks.generate(wl, T=97)
    d = upload(wl, x)
    o0, S0 = _fwd(d, 64, state_in=False)
    x0 = dict(x)
    x0["state_in"] = np.zeros_like(x["state_in"])
    o_ref, S_ref = oracle_heads(wl, x0, [(0, h) for h in range(4)])
    _check("o", host(o0).reshape(1, 4, 97, 128), o_ref, TOL["bf16"])
    _check("state", host(S0).reshape(1, 4, 128, 128), S_ref, TOL["bf16"])
    S_io = d["state_in"].clone()
    o1 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["A_log"], d["dt_bias"], d["beta"], S_io, chunk=64,
                       state_out=S_io)[0]
    o_ref1, S_ref1 = oracle_heads(wl, x, [(0, h) for h in range(4)])
    _check("o", host(o1).reshape(1, 4, 97, 128), o_ref1, TOL["bf16"])
    _check("state", host(S_io).reshape(1, 4, 128, 128), S_ref1, TOL["bf16"])
