"""Shared helpers of the GPU parity tests: device upload of the seeded inputs and
per-head oracle evaluation.  Nothing here computes any part of the method: the
expected values always come from oracle/."""
import json
import os
import sys

import numpy as np
import torch

import kda_synth as ks
from oracle import kda_ref as R

DEV = "cuda:0"
TOL = {"f32": 1e-4, "bf16": 2e-2}   # max|x - ref| / max|ref| per tensor


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check(name, got, ref, tol):
    """rel_err of one output tensor against the oracle, asserted against its bar.  When
    the environment variable KDA_MARGINS_OUT names a file, one JSON line per check is
    appended to it (test id, tensor, rel_err, bar): the parity margins summary is built
    from those lines (tests/margins_table.py)."""
    e = R.rel_err(got, ref)
    say("  %-10s rel_err %.3e (bar %.0e)" % (name, e, tol))
    out = os.environ.get("KDA_MARGINS_OUT")
    if out:
        test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
        with open(out, "a") as f:
            f.write(json.dumps({"test": test, "tensor": name, "rel_err": e, "bar": tol,
                                "finite": bool(np.all(np.isfinite(got)))}) + "\n")
    assert np.all(np.isfinite(got)), name
    assert e <= tol, (name, e)


def to_dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(DEV).to(dtype).contiguous()


def act_dtype(wl):
    return torch.bfloat16 if wl.dtype == "bf16" else torch.float32


def upload(wl, x):
    dt = act_dtype(wl)
    d = {n: to_dev(x[n], dt) for n in ("q", "k", "v", "z", "beta")}
    d["A_log"] = to_dev(x["A_log"], torch.float32)
    d["dt_bias"] = to_dev(x["dt_bias"], torch.float32)
    d["state_in"] = to_dev(x["state_in"], torch.float32)
    if "d_out" in x:
        d["d_out"] = to_dev(x["d_out"], dt)
    return d


def oracle_heads(wl, x, heads, scale=None):
    """Oracle forward (token recurrence, f64) of the listed (b, h) heads."""
    sel = lambda a: np.stack([a[b, h] for b, h in heads])[None]
    g, _ = R.gate(sel(x["z"]), np.array([x["A_log"][h] for _, h in heads]),
                  np.stack([x["dt_bias"][h] for _, h in heads]))
    return R.recurrent(sel(x["q"]), sel(x["k"]), sel(x["v"]), g, sel(x["beta"]), sel(x["state_in"]), scale)


def oracle_heads_from_slices(wl, heads, T=None, scale=None):
    """Oracle forward of single heads regenerated slice by slice (for multi-GB workloads)."""
    A_log, dt_bias = ks.head_params(wl)
    sl = [ks.head_slice(wl, b, h, T) for b, h in heads]
    st = lambda n: np.stack([s[n] for s in sl])[None]
    g, _ = R.gate(st("z"), np.array([A_log[h] for _, h in heads]), np.stack([dt_bias[h] for _, h in heads]))
    return R.recurrent(st("q"), st("k"), st("v"), g, st("beta"), st("state_in"), scale)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)
