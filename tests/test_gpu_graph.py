"""The forward and decode entry points under HIP graph capture (torch.cuda.CUDAGraph):
they launch only kernels on the caller's stream and allocate nothing when the outputs are
given, so a captured call replays.  Each replay, with eager work and synchronisations in
between, must reproduce the eager result bit for bit."""
import pytest
import torch

import gated_delta_rule_47_amd as kda
import kda_synth as ks

from gpu_helpers import say, upload

pytestmark = pytest.mark.gpu


def test_chunk_fwd_and_decode_step_replay_in_a_graph():
    wl = ks.WORKLOADS["nano"].with_(B=2, H=4, state="normal:0.1")
    T = 300
    x = ks.generate(wl, T=T + 1)
    d = upload(wl, x)
    sl = lambda t: t[:, :, :T].contiguous()
    last = lambda t: t[:, :, T].contiguous()
    q, k, v, z, beta = (sl(d[n]) for n in ("q", "k", "v", "z", "beta"))
    qt, kt, vt, zt, bt = (last(d[n]) for n in ("q", "k", "v", "z", "beta"))
    o = torch.empty((2, 4, T, wl.V), dtype=q.dtype, device=q.device)
    S = torch.empty_like(d["state_in"])
    ot = torch.empty((2, 4, wl.V), dtype=q.dtype, device=q.device)

    def work():
        kda.chunk_fwd(q, k, v, z, d["A_log"], d["dt_bias"], beta, d["state_in"], chunk=64, out=o, state_out=S)
        kda.recurrent_step(qt, kt, vt, zt, d["A_log"], d["dt_bias"], bt, S, out=ot)

    work()
    torch.cuda.synchronize()
    ref = (o.clone(), S.clone(), ot.clone())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):               # warm-up on the capture stream
        work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(3):
        o.fill_(float("nan"))
        S.fill_(float("nan"))
        ot.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say("replay", rep)
        assert torch.equal(o, ref[0]) and torch.equal(S, ref[1]) and torch.equal(ot, ref[2])
        _ = (q.float() * 2).sum().item()        # eager work between replays
