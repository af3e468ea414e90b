"""GPU parity of the scalar-decay entry points (kda_chunk_fwd_scalar, kda_recurrent_step_scalar)
through the C ABI.

The scalar gate input of each workload is channel 0 of its z and the bias channel 0 of its
dt_bias, so the inputs keep the workload's distributions.  Checks: the f64 oracle's scalar
recurrence (bars 1e-4 fp32, 2e-2 bf16 on o and the final state, as for the per-channel
forward), and bit-for-bit equality with the per-channel entry point fed the same gate on
every channel (the scalar path evaluates the same expressions once per token).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_47_amd as kda
import kda_synth as ks
from oracle import kda_ref as R

from gpu_helpers import check, TOL, act_dtype, host, say, to_dev, upload

pytestmark = pytest.mark.gpu


_check = check


def _scalar_inputs(wl, x):
    """Device tensors of a workload with the gate reduced to one value per token and head."""
    d = upload(wl, x)
    d["a"] = d["z"][..., 0].contiguous()
    d["dtb"] = d["dt_bias"][:, 0].contiguous()
    return d


def _oracle(x, heads, scale=None, T=None):
    sel = lambda arr: np.stack([arr[b, h] for b, h in heads])[None]
    g, _ = R.gate_scalar(sel(x["z"][..., 0]), np.array([x["A_log"][h] for _, h in heads]),
                         np.array([x["dt_bias"][h, 0] for _, h in heads]))
    return R.recurrent_scalar(sel(x["q"]), sel(x["k"]), sel(x["v"]), g, sel(x["beta"]), sel(x["state_in"]), scale)


CASES = [  # (dtype, K, V, chunk, T)
    ("f32", 8, 8, 16, 33), ("f32", 64, 64, 64, 130), ("f32", 128, 32, 32, 70), ("f32", 32, 16, 16, 1),
    ("bf16", 128, 128, 64, 200), ("bf16", 64, 64, 32, 77), ("bf16", 8, 16, 16, 45), ("bf16", 128, 64, 16, 50),
]


def _base(dtype):
    return ks.WORKLOADS["nano"] if dtype == "bf16" else ks.WORKLOADS["layer"].with_(a_log="uniform:-3,1")


@pytest.mark.parametrize("dtype,K,V,chunk,T", CASES)
def test_scalar_forward_against_oracle_and_broadcast(dtype, K, V, chunk, T):
    wl = _base(dtype).with_(B=2, H=2, K=K, V=V, chunk=chunk, state="normal:0.1")
    x = ks.generate(wl, T=T)
    d = _scalar_inputs(wl, x)
    say("scalar forward", dtype, K, V, chunk, T)
    o, S = kda.chunk_fwd_scalar(d["q"], d["k"], d["v"], d["a"], d["A_log"], d["dtb"], d["beta"], d["state_in"],
                                chunk=chunk)
    o_ref, S_ref = _oracle(x, [(b, h) for b in range(2) for h in range(2)])
    _check("o", host(o).reshape(1, 4, T, V), o_ref, TOL[dtype])
    _check("state", host(S).reshape(1, 4, K, V), S_ref, TOL[dtype])
    # the per-channel entry point with the same gate on every channel: the same bits
    zb = d["a"][..., None].expand(-1, -1, -1, K).contiguous()
    db = d["dtb"][:, None].expand(-1, K).contiguous()
    o2, S2 = kda.chunk_fwd(d["q"], d["k"], d["v"], zb, d["A_log"], db, d["beta"], d["state_in"], chunk=chunk)
    assert torch.equal(o, o2) and torch.equal(S, S2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scalar_saturated_gate_token_path_and_no_bias(dtype):
    """Strong decays (A_log up to 6, past the factorised path's range) force the token-by-token
    blocks; dt_bias absent means a zero bias."""
    wl = _base(dtype).with_(B=1, H=4, K=128, V=64, chunk=64, a_log="list:6,-2,3,0", state="normal:0.1")
    x = ks.generate(wl, T=150)
    d = _scalar_inputs(wl, x)
    o, S = kda.chunk_fwd_scalar(d["q"], d["k"], d["v"], d["a"], d["A_log"], None, d["beta"], d["state_in"], chunk=64)
    x0 = dict(x, dt_bias=np.zeros_like(x["dt_bias"]))
    o_ref, S_ref = _oracle(x0, [(0, h) for h in range(4)])
    _check("o", host(o).reshape(1, 4, 150, 64), o_ref, TOL[dtype])
    _check("state", host(S).reshape(1, 4, 128, 64), S_ref, TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scalar_decode_steps_and_prefill_handoff(dtype):
    """Prefill T-1 tokens with the chunked entry point, then one decode step: equals the
    scalar recurrence over all T tokens."""
    wl = _base(dtype).with_(B=2, H=3, K=64, V=32, chunk=32, state="normal:0.1")
    T = 41
    x = ks.generate(wl, T=T)
    d = _scalar_inputs(wl, x)
    sl = lambda t: t[:, :, :T - 1].contiguous()
    _, S = kda.chunk_fwd_scalar(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["a"]), d["A_log"], d["dtb"], sl(d["beta"]),
                                d["state_in"], chunk=32)
    last = lambda t: t[:, :, T - 1].contiguous()
    ot = kda.recurrent_step_scalar(last(d["q"]), last(d["k"]), last(d["v"]), last(d["a"]), d["A_log"], d["dtb"],
                                   last(d["beta"]), S)
    o_ref, S_ref = _oracle(x, [(b, h) for b in range(2) for h in range(3)])
    _check("o_last", host(ot).reshape(1, 6, 32), o_ref[:, :, -1], TOL[dtype])
    _check("state", host(S).reshape(1, 6, 64, 32), S_ref, TOL[dtype])


def test_scalar_long_workload_sampled_heads():
    """The long workload's shape (B=4, H=32, T=16384, K=V=128, bf16) with the scalar gate,
    launched as the benchmark's scalar line launches it; sampled heads against the oracle."""
    wl = ks.WORKLOADS["long"]
    say("generating long")
    x = ks.generate(wl)
    d = _scalar_inputs(wl, x)
    heads = [(0, 3), (3, 30)]
    sub = {n: np.stack([x[n][b, h] for b, h in heads])[None] for n in ("q", "k", "v", "z", "beta", "state_in")}
    sub["A_log"] = np.array([x["A_log"][h] for _, h in heads])
    sub["dt_bias"] = np.stack([x["dt_bias"][h] for _, h in heads])
    del x
    for n in ("z", "dt_bias"):
        d.pop(n)
    o, S = kda.chunk_fwd_scalar(d["q"], d["k"], d["v"], d["a"], d["A_log"], d["dtb"], d["beta"], d["state_in"],
                                chunk=wl.chunk)
    torch.cuda.synchronize()
    g, _ = R.gate_scalar(sub["z"][..., 0], sub["A_log"], sub["dt_bias"][:, 0])
    o_ref, S_ref = R.recurrent_scalar(sub["q"], sub["k"], sub["v"], g, sub["beta"], sub["state_in"])
    _check("o", np.stack([host(o[b, h]) for b, h in heads])[None], o_ref, TOL["bf16"])
    _check("state", np.stack([host(S[b, h]) for b, h in heads])[None], S_ref, TOL["bf16"])


def test_scalar_T0_state_none_and_in_place():
    """T = 0 copies state_in to state_out; no initial state equals a zero one; state_out may
    be state_in (bf16, the pipelined kernel)."""
    wl = ks.WORKLOADS["nano"].with_(B=1, H=3, K=128, V=128, state="normal:0.1")
    x = ks.generate(wl, T=90)
    d = _scalar_inputs(wl, x)
    e = lambda t: t[:, :, :0]
    o0, S0 = kda.chunk_fwd_scalar(e(d["q"]), e(d["k"]), e(d["v"]), e(d["a"]), d["A_log"], d["dtb"], e(d["beta"]),
                                  d["state_in"], chunk=64)
    assert o0.numel() == 0 and torch.equal(S0, d["state_in"])
    args = (d["q"], d["k"], d["v"], d["a"], d["A_log"], d["dtb"], d["beta"])
    o1, S1 = kda.chunk_fwd_scalar(*args, None, chunk=64)
    o2, S2 = kda.chunk_fwd_scalar(*args, torch.zeros_like(d["state_in"]), chunk=64)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    ref_o, ref_S = kda.chunk_fwd_scalar(*args, d["state_in"], chunk=64)
    st = d["state_in"].clone()
    o3, S3 = kda.chunk_fwd_scalar(*args, st, chunk=64, state_out=st)
    assert S3.data_ptr() == st.data_ptr() and torch.equal(S3, ref_S) and torch.equal(o3, ref_o)
