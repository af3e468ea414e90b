"""GPU parity of the forward with the fused output RMSNorm (kda_chunk_fwd_norm), bf16.

o = r / sqrt(mean_v r^2 + eps) * w_h for the read r, compared with the f64 oracle's
recurrence followed by its rmsnorm (bar 2e-2 on o and on the final state, as for every
bf16 forward): one and two value tiles per head (V = 128: the tiles exchange per-token
sums of squares through the workspace), key dims 16..128, one to eleven blocks with
ragged tails, blocks on the token-by-token path, more heads than one launch holds, and
the two full-size workloads on sampled heads (the long one on eight heads, one per XCD).
Also: no weight equals a weight of ones, the read scale is absorbed up to eps, bitwise
repeatability, graph replays (each must advance the workspace's epoch), and the
failure path forced from the host with a zero wait bound.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_47_amd as kda
import kda_synth as ks
from oracle import kda_ref as R

from gpu_helpers import check, DEV, TOL, host, oracle_heads, oracle_heads_from_slices, say, to_dev, upload

pytestmark = pytest.mark.gpu

KDA_ERR_EXCHANGE = -9
EPS = 1e-5


_check = check


def _weight(H, V, seed=9):
    return (1.0 + 0.5 * np.random.default_rng(seed).standard_normal((H, V))).astype(np.float32)


def _norm(d, w, **kw):
    return kda.chunk_fwd_norm(d["q"], d["k"], d["v"], d["z"], d["A_log"], d["dt_bias"], d["beta"], d["state_in"],
                              norm_weight=w, eps=kw.pop("eps", EPS), **kw)


def _ref(wl, x, heads, w, eps=EPS, T=None, slices=False):
    o_ref, S_ref = oracle_heads_from_slices(wl, heads, T) if slices else oracle_heads(wl, x, heads)
    wsel = None if w is None else np.stack([w[h] for _, h in heads])
    return R.rmsnorm(o_ref, wsel, eps), S_ref


CASES = [  # (K, V, T): two tiles (V = 128) and one; blocks 1 .. 11 with ragged tails
    (128, 128, 1), (128, 128, 31), (128, 128, 33), (128, 128, 97), (128, 128, 200), (128, 128, 352),
    (64, 128, 129), (32, 128, 70), (16, 128, 45), (128, 64, 95), (64, 64, 200), (64, 32, 77), (32, 16, 40),
]


@pytest.mark.parametrize("K,V,T", CASES)
def test_norm_forward_matches_oracle(K, V, T):
    wl = ks.WORKLOADS["nano"].with_(B=2, H=3, K=K, V=V, state="normal:0.1")
    x = ks.generate(wl, T=T)
    d = upload(wl, x)
    w = _weight(3, V)
    ws_bytes = kda.chunk_fwd_norm_workspace_bytes(2, 3, T, K, V)
    assert (ws_bytes > 0) == (V > 64)
    say("norm", K, V, T)
    o, S = _norm(d, to_dev(w, torch.float32))
    heads = [(b, h) for b in range(2) for h in range(3)]
    y_ref, S_ref = _ref(wl, x, heads, w)
    _check("o", host(o).reshape(1, 6, T, V), y_ref, TOL["bf16"])
    _check("state", host(S).reshape(1, 6, K, V), S_ref, TOL["bf16"])


def test_norm_workspace_status_repeatability_and_weightless():
    wl = ks.WORKLOADS["nano"].with_(B=1, H=4, K=128, V=128, state="normal:0.1")
    T = 230
    x = ks.generate(wl, T=T)
    d = upload(wl, x)
    ws = torch.zeros(kda.chunk_fwd_norm_workspace_bytes(1, 4, T, 128, 128), dtype=torch.uint8, device=DEV)
    ones = torch.ones((4, 128), device=DEV)
    o1, S1 = _norm(d, ones, workspace=ws)
    assert kda.chunk_fwd_status(ws) == 0
    o2, S2 = _norm(d, None, workspace=ws)                # the same workspace again (next epoch)
    assert kda.chunk_fwd_status(ws) == 0
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    # the state is the plain forward's
    _, Sp = kda.chunk_fwd(d["q"], d["k"], d["v"], d["z"], d["A_log"], d["dt_bias"], d["beta"], d["state_in"])
    assert torch.equal(S1, Sp)
    # the read scale is absorbed by the norm up to O(eps / mean(o^2)): with these inputs
    # mean(o^2) is ~1e-4, so eps = 1e-9 puts eps / mean(o^2) at the page's ~1e-5, and the
    # two outputs then differ by their bf16 rounding only
    oa, _ = _norm(d, ones, workspace=ws, eps=1e-9)
    ob, _ = _norm(d, ones, workspace=ws, eps=1e-9, scale=1.0)
    e = R.rel_err(host(ob), host(oa))
    say("  scale 1 vs K^-0.5 at eps 1e-9: rel diff %.2e" % e)
    assert e < 1e-2
    y_ref, _ = _ref(wl, x, [(0, h) for h in range(4)], None)
    _check("o", host(o1).reshape(1, 4, T, 128), y_ref, TOL["bf16"])


def test_norm_saturated_gates_take_the_token_path():
    wl = ks.WORKLOADS["nano"].with_(B=1, H=4, K=128, V=128, state="normal:0.1", a_log="list:20,-3,8,0")
    T = 150
    x = ks.generate(wl, T=T)
    x["z"][0, 2, 40:70] += 6.0
    x["z"] = ks.round_bf16(x["z"])
    d = upload(wl, x)
    w = _weight(4, 128, seed=2)
    o, S = _norm(d, to_dev(w, torch.float32))
    y_ref, S_ref = _ref(wl, x, [(0, h) for h in range(4)], w)
    _check("o", host(o).reshape(1, 4, T, 128), y_ref, TOL["bf16"])
    _check("state", host(S).reshape(1, 4, 128, 128), S_ref, TOL["bf16"])


def test_norm_more_heads_than_one_launch():
    """144 heads with two tiles each: two launches (128 + 16 heads)."""
    wl = ks.WORKLOADS["nano"].with_(B=3, H=48, K=128, V=128, state="normal:0.1")
    T = 70
    x = ks.generate(wl, T=T)
    d = upload(wl, x)
    w = _weight(48, 128, seed=4)
    o, S = _norm(d, to_dev(w, torch.float32))
    heads = [(0, 0), (1, 17), (2, 31), (2, 32), (2, 39), (2, 40), (2, 47)]
    y_ref, S_ref = _ref(wl, x, heads, w)
    _check("o", np.stack([host(o[b, h]) for b, h in heads])[None], y_ref, TOL["bf16"])
    _check("state", np.stack([host(S[b, h]) for b, h in heads])[None], S_ref, TOL["bf16"])


def test_norm_replays_in_a_graph():
    wl = ks.WORKLOADS["nano"].with_(B=2, H=4, K=128, V=128, state="normal:0.1")
    T = 190
    x = ks.generate(wl, T=T)
    d = upload(wl, x)
    w = to_dev(_weight(4, 128), torch.float32)
    ws = torch.zeros(kda.chunk_fwd_norm_workspace_bytes(2, 4, T, 128, 128), dtype=torch.uint8, device=DEV)
    o = torch.empty((2, 4, T, 128), dtype=torch.bfloat16, device=DEV)
    S = torch.empty_like(d["state_in"])

    def work():
        _norm(d, w, workspace=ws, out=o, state_out=S)

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


def test_norm_gives_up_when_the_wait_bound_is_zero():
    wl = ks.WORKLOADS["nano"].with_(B=1, H=2, K=128, V=128, state="normal:0.1")
    T = 130
    x = ks.generate(wl, T=T)
    d = upload(wl, x)
    ws = torch.zeros(kda.chunk_fwd_norm_workspace_bytes(1, 2, T, 128, 128), dtype=torch.uint8, device=DEV)
    try:
        kda.set_exchange_timeout_us(0)
        _norm(d, None, workspace=ws)
        assert kda.chunk_fwd_status(ws) == KDA_ERR_EXCHANGE
    finally:
        kda.set_exchange_timeout_us(1000000)
    assert kda.chunk_fwd_status(ws) == 0
    o, S = _norm(d, None, workspace=ws)
    assert kda.chunk_fwd_status(ws) == 0
    y_ref, S_ref = _ref(wl, x, [(0, 0), (0, 1)], None)
    _check("o", host(o).reshape(1, 2, T, 128), y_ref, TOL["bf16"])


@pytest.mark.parametrize("wl_name,heads", [
    ("nano", [(0, 0), (3, 5), (7, 7)]),
    # one head per XCD: head b*32 + h of the launch runs on XCD (b*32 + h) % 8
    ("long", [(0, 0), (0, 9), (1, 2), (1, 11), (2, 4), (2, 13), (3, 6), (3, 31)]),
])
def test_norm_full_size_sampled_heads(wl_name, heads):
    wl = ks.WORKLOADS[wl_name]
    say("generating", wl_name)
    x = ks.generate(wl)
    d = upload(wl, x)
    del x
    w = _weight(wl.H, wl.V, seed=12)
    o, S = _norm(d, to_dev(w, torch.float32))
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    y_ref, S_ref = _ref(wl, None, heads, w, slices=True)
    _check("o", np.stack([host(o[b, h]) for b, h in heads])[None], y_ref, TOL["bf16"])
    _check("state", np.stack([host(S[b, h]) for b, h in heads])[None], S_ref, TOL["bf16"])
