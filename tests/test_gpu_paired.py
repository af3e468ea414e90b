"""GPU parity of the paired forward: bf16 activations with V = 128 and blocks of 32 tokens,
where the two value-tile workgroups of a head compute the gate and WY stages of alternate
blocks once and hand them to each other through the caller's workspace.

Checks, all through the C ABI: the f64 oracle on o and the final state (bar 2e-2, as for
every bf16 forward) over key dims, chunk sizes, one to eleven blocks, ragged tails ending
in either workgroup's block, more heads than one launch holds, the scalar-decay variant
and the token-by-token blocks of saturated gates; the call without a workspace (each
value tile computing every block itself) against the same oracle; bitwise repeatability;
a HIP graph replaying the call (each replay must advance the workspace's epoch); and the
failure path, forced from the host with a zero wait bound, which must report
KDA_ERR_EXCHANGE and leave the next call correct.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_47_amd as kda
import kda_synth as ks
from oracle import kda_ref as R

from gpu_helpers import check, DEV, TOL, host, oracle_heads, say, upload

pytestmark = pytest.mark.gpu

KDA_ERR_EXCHANGE = -9


_check = check


def _workspace(B, H, T, K, chunk):
    n = kda.chunk_fwd_workspace_bytes(B, H, T, K, 128, chunk)
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device=DEV)


def _fwd(d, chunk, ws, state=True, **kw):
    return kda.chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["A_log"], d["dt_bias"], d["beta"],
                         d["state_in"] if state else None, chunk=chunk, workspace=ws, **kw)


def _wl(B, H, K, chunk, **kw):
    return ks.WORKLOADS["nano"].with_(B=B, H=H, K=K, V=128, chunk=chunk, state="normal:0.1", **kw)


CASES = [  # (K, chunk, T): blocks 1 .. 11, last block owned by either workgroup, ragged tails
    (128, 64, 1), (128, 64, 31), (128, 32, 32), (128, 64, 33), (128, 64, 64), (128, 32, 95), (128, 64, 97),
    (128, 64, 160), (128, 32, 352), (64, 64, 129), (64, 32, 96), (32, 64, 200), (16, 64, 45), (8, 32, 70),
]


@pytest.mark.parametrize("K,chunk,T", CASES)
def test_paired_forward_matches_oracle(K, chunk, T):
    wl = _wl(2, 3, K, chunk)
    x = ks.generate(wl, T=T)
    d = upload(wl, x)
    ws = _workspace(2, 3, T, K, chunk)
    say("paired", K, chunk, T)
    o, S = _fwd(d, chunk, ws)
    assert kda.chunk_fwd_status(ws) == 0
    heads = [(b, h) for b in range(2) for h in range(3)]
    o_ref, S_ref = oracle_heads(wl, x, heads)
    _check("o", host(o).reshape(1, 6, T, 128), o_ref, TOL["bf16"])
    _check("state", host(S).reshape(1, 6, K, 128), S_ref, TOL["bf16"])
    # without a workspace each value tile computes every block itself: the same function
    o2, S2 = _fwd(d, chunk, None)
    _check("o solo", host(o2).reshape(1, 6, T, 128), o_ref, TOL["bf16"])
    _check("state solo", host(S2).reshape(1, 6, K, 128), S_ref, TOL["bf16"])


def test_paired_state_none_in_place_scale_and_repeatability():
    wl = _wl(1, 4, 128, 64)
    T = 230
    x = ks.generate(wl, T=T)
    d = upload(wl, x)
    ws = _workspace(1, 4, T, 128, 64)
    ref_o, ref_S = _fwd(d, 64, ws)
    o_b, S_b = _fwd(d, 64, ws)                 # the same workspace again (next epoch)
    assert torch.equal(ref_o, o_b) and torch.equal(ref_S, S_b)
    o1, S1 = _fwd(d, 64, ws, state=False)
    o2, S2 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["A_log"], d["dt_bias"], d["beta"],
                           torch.zeros_like(d["state_in"]), chunk=64, workspace=ws)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    st = d["state_in"].clone()
    o3, S3 = kda.chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["A_log"], d["dt_bias"], d["beta"], st, chunk=64,
                           state_out=st, workspace=ws)
    assert S3.data_ptr() == st.data_ptr() and torch.equal(S3, ref_S) and torch.equal(o3, ref_o)
    oa, Sa = _fwd(d, 64, ws, scale=1.0)
    oz, Sz = _fwd(d, 64, ws, scale=0.0)
    assert torch.equal(Sa, Sz) and torch.all(oz == 0)
    assert kda.chunk_fwd_status(ws) == 0
    o_ref, S_ref = oracle_heads(wl, x, [(0, h) for h in range(4)])
    _check("o", host(ref_o).reshape(1, 4, T, 128), o_ref, TOL["bf16"])


def test_paired_more_heads_than_one_launch():
    """144 heads: two launches (128 + 16 heads) that reuse the same rings in stream order."""
    wl = _wl(3, 48, 128, 64)
    T = 70
    x = ks.generate(wl, T=T)
    d = upload(wl, x)
    ws = _workspace(3, 48, T, 128, 64)
    o, S = _fwd(d, 64, ws)
    assert kda.chunk_fwd_status(ws) == 0
    heads = [(0, 0), (1, 17), (2, 31), (2, 32), (2, 39), (2, 40), (2, 47)]   # head 127 and 128 straddle the launches
    o_ref, S_ref = oracle_heads(wl, x, heads)
    _check("o", np.stack([host(o[b, h]) for b, h in heads])[None], o_ref, TOL["bf16"])
    _check("state", np.stack([host(S[b, h]) for b, h in heads])[None], S_ref, TOL["bf16"])


def test_paired_saturated_gates_take_the_token_path():
    wl = _wl(1, 4, 128, 64, a_log="list:20,-3,8,0")
    T = 150
    x = ks.generate(wl, T=T)
    x["z"][0, 2, 40:70] += 6.0
    x["z"] = ks.round_bf16(x["z"])
    d = upload(wl, x)
    ws = _workspace(1, 4, T, 128, 64)
    o, S = _fwd(d, 64, ws)
    assert kda.chunk_fwd_status(ws) == 0
    o_ref, S_ref = oracle_heads(wl, x, [(0, h) for h in range(4)])
    _check("o", host(o).reshape(1, 4, T, 128), o_ref, TOL["bf16"])
    _check("state", host(S).reshape(1, 4, 128, 128), S_ref, TOL["bf16"])


@pytest.mark.parametrize("T", [33, 200])
def test_paired_scalar_decay(T):
    wl = _wl(2, 2, 128, 64)
    x = ks.generate(wl, T=T)
    d = upload(wl, x)
    a = d["z"][..., 0].contiguous()
    dtb = d["dt_bias"][:, 0].contiguous()
    ws = _workspace(2, 2, T, 128, 64)
    o, S = kda.chunk_fwd_scalar(d["q"], d["k"], d["v"], a, d["A_log"], dtb, d["beta"], d["state_in"], chunk=64,
                                workspace=ws)
    assert kda.chunk_fwd_status(ws) == 0
    heads = [(b, h) for b in range(2) for h in range(2)]
    sel = lambda arr: np.stack([arr[b, h] for b, h in heads])[None]
    g, _ = R.gate_scalar(sel(x["z"][..., 0]), np.array([x["A_log"][h] for _, h in heads]),
                         np.array([x["dt_bias"][h, 0] for _, h in heads]))
    o_ref, S_ref = R.recurrent_scalar(sel(x["q"]), sel(x["k"]), sel(x["v"]), g, sel(x["beta"]), sel(x["state_in"]))
    _check("o", host(o).reshape(1, 4, T, 128), o_ref, TOL["bf16"])
    _check("state", host(S).reshape(1, 4, 128, 128), S_ref, TOL["bf16"])


def test_paired_forward_replays_in_a_graph():
    wl = _wl(2, 4, 128, 64)
    T = 190
    x = ks.generate(wl, T=T)
    d = upload(wl, x)
    ws = _workspace(2, 4, T, 128, 64)
    o = torch.empty((2, 4, T, 128), dtype=torch.bfloat16, device=DEV)
    S = torch.empty_like(d["state_in"])

    def work():
        _fwd(d, 64, ws, out=o, state_out=S)

    work()
    torch.cuda.synchronize()
    ref = (o.clone(), S.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(3):
        o.fill_(float("nan"))
        S.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("replay", rep)
        assert torch.equal(o, ref[0]) and torch.equal(S, ref[1])
        _ = (d["q"].float() * 2).sum().item()
    assert kda.chunk_fwd_status(ws) == 0


def test_paired_gives_up_when_the_wait_bound_is_zero():
    """The failure path, forced from the host: with a zero bound every wait for the other
    workgroup gives up at once; the kernels still finish, the call reports
    KDA_ERR_EXCHANGE, and the next call with the normal bound is correct."""
    wl = _wl(1, 2, 128, 64)
    T = 130
    x = ks.generate(wl, T=T)
    d = upload(wl, x)
    ws = _workspace(1, 2, T, 128, 64)
    try:
        kda.set_exchange_timeout_us(0)
        _fwd(d, 64, ws)
        assert kda.chunk_fwd_status(ws) == KDA_ERR_EXCHANGE
    finally:
        kda.set_exchange_timeout_us(1000000)
    assert kda.chunk_fwd_status(ws) == 0       # read-and-clear
    o, S = _fwd(d, 64, ws)
    assert kda.chunk_fwd_status(ws) == 0
    o_ref, S_ref = oracle_heads(wl, x, [(0, 0), (0, 1)])
    _check("o", host(o).reshape(1, 2, T, 128), o_ref, TOL["bf16"])
    _check("state", host(S).reshape(1, 2, 128, 128), S_ref, TOL["bf16"])
