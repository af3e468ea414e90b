"""Seeded synthetic inputs for the KDA chunked forward, decode step and adjoint.

This module is shared by the f64 oracle tests and by the HIP-path tests and the
benchmark.  It holds no arithmetic of the method itself: it only draws random
tensors with the distributions of the workloads below and rounds activations to
bfloat16 where a workload runs in bfloat16.

Every tensor of every (batch, head) slice is drawn from its own PCG64 stream,
seeded by (workload seed, tensor id, b, h).  Any single head can therefore be
regenerated without generating the rest, which is how the full-size parity
tests and the CPU baseline sample a few heads of a multi-GB workload.

Distributions (per workload, see WORKLOADS):
  q, k      N(0,1), then L2-normalised over the key dimension per token
  v         N(0,1)
  z         N(0,1)                      (gate pre-activation)
  beta      sigmoid(N(0,1))             (one scalar per token and head)
  A_log     per head: fixed list, U(-10,20) or U(-3,1)
  dt_bias   per head and key channel: 0 or N(0, 0.1)
  state_in  N(0, 0.1) or zeros          (fp32, (B,H,K,V))
  d_out     N(0,1)                      (adjoint workload only)
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "z": 4, "beta": 5, "state_in": 6, "d_out": 7,
               "A_log": 8, "dt_bias": 9, "d_state_out": 10}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    K: int
    V: int
    chunk: int
    dtype: str            # "f32" or "bf16": activations (q, k, v, z, beta, o)
    seed: int
    a_log: str            # "list:-3,0" | "uniform:-10,20" | "uniform:-3,1"
    dt_bias: str          # "zero" | "normal:0.1"
    state: str            # "normal:0.1" | "zero"
    adjoint: bool = False
    desc: str = ""

    @property
    def head_tokens(self) -> int:
        return self.B * self.H * self.T

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload(
        "tiny", B=1, H=2, T=32, K=8, V=8, chunk=16, dtype="f32", seed=47000,
        a_log="list:-3,0", dt_bias="zero", state="normal:0.1",
        desc="tiny fp32 forward, two chunks of 16, A_log = -3 and 0 (the A=0 control head)"),
    "layer": Workload(
        "layer", B=1, H=8, T=256, K=64, V=64, chunk=64, dtype="f32", seed=47001,
        a_log="uniform:-10,20", dt_bias="zero", state="zero",
        desc="single-layer fp32 forward, A_log ~ U(-10,20), zero initial state"),
    "nano": Workload(
        "nano", B=8, H=8, T=4096, K=64, V=64, chunk=64, dtype="bf16", seed=47002,
        a_log="uniform:-3,1", dt_bias="normal:0.1", state="normal:0.1",
        desc="nano-model KDA layer (d_model 512 = 8 heads x 64), bf16 activations, fp32 state"),
    "long": Workload(
        "long", B=4, H=32, T=16384, K=128, V=128, chunk=64, dtype="bf16", seed=47003,
        a_log="uniform:-3,1", dt_bias="normal:0.1", state="normal:0.1",
        desc="long-context KDA forward B=4 H=32 T=16384 K=V=128, bf16 activations, fp32 state"),
    "adjoint": Workload(
        "adjoint", B=2, H=16, T=8192, K=128, V=128, chunk=64, dtype="f32", seed=47004,
        a_log="uniform:-3,1", dt_bias="normal:0.1", state="normal:0.1", adjoint=True,
        desc="chunked adjoint, fp32, B=2 H=16 T=8192 K=V=128, d_out ~ N(0,1)"),
}


# ----------------------------------------------------------------------------- bf16 casts
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 value (still stored as float32)."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


# ----------------------------------------------------------------------------- draws
def _rng(wl: Workload, tensor: str, b: int = 0, h: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence([wl.seed, _TENSOR_IDS[tensor], b, h])
    return np.random.Generator(np.random.PCG64(ss))


def _l2norm(x: np.ndarray) -> np.ndarray:
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def head_params(wl: Workload):
    """A_log (H,) and dt_bias (H,K), float32."""
    kind, _, arg = wl.a_log.partition(":")
    if kind == "list":
        vals = [float(s) for s in arg.split(",")]
        a_log = np.array([vals[h % len(vals)] for h in range(wl.H)], dtype=np.float64)
    elif kind == "uniform":
        lo, hi = (float(s) for s in arg.split(","))
        a_log = _rng(wl, "A_log").uniform(lo, hi, size=wl.H)
    else:
        raise ValueError(wl.a_log)
    kind, _, arg = wl.dt_bias.partition(":")
    if kind == "zero":
        dt_bias = np.zeros((wl.H, wl.K))
    elif kind == "normal":
        dt_bias = _rng(wl, "dt_bias").normal(0.0, float(arg), size=(wl.H, wl.K))
    else:
        raise ValueError(wl.dt_bias)
    return a_log.astype(np.float32), dt_bias.astype(np.float32)


def head_slice(wl: Workload, b: int, h: int, T: int | None = None) -> dict:
    """Inputs of one (batch, head) slice as float32 arrays.

    Activations of bf16 workloads are returned already rounded to bfloat16 values,
    so the oracle (upcasting them to f64) sees exactly what the kernel reads.
    """
    T = wl.T if T is None else T
    out = {}
    q = _l2norm(_rng(wl, "q", b, h).standard_normal((T, wl.K)))
    k = _l2norm(_rng(wl, "k", b, h).standard_normal((T, wl.K)))
    v = _rng(wl, "v", b, h).standard_normal((T, wl.V))
    z = _rng(wl, "z", b, h).standard_normal((T, wl.K))
    beta = _sigmoid(_rng(wl, "beta", b, h).standard_normal(T))
    for name, arr in (("q", q), ("k", k), ("v", v), ("z", z), ("beta", beta)):
        a32 = arr.astype(np.float32)
        out[name] = round_bf16(a32) if wl.dtype == "bf16" else a32
    kind, _, arg = wl.state.partition(":")
    if kind == "zero":
        out["state_in"] = np.zeros((wl.K, wl.V), dtype=np.float32)
    else:
        out["state_in"] = _rng(wl, "state_in", b, h).normal(0.0, float(arg), (wl.K, wl.V)).astype(np.float32)
    if wl.adjoint:
        out["d_out"] = _rng(wl, "d_out", b, h).standard_normal((T, wl.V)).astype(np.float32)
    return out


def generate(wl: Workload, T: int | None = None, threads: int | None = None) -> dict:
    """All inputs of a workload, float32 arrays in head-major (B,H,T,D) layout.

    q,k,z: (B,H,T,K)  v: (B,H,T,V)  beta: (B,H,T)  state_in: (B,H,K,V)
    A_log: (H,)  dt_bias: (H,K)  d_out: (B,H,T,V) for the adjoint workload.
    """
    T = wl.T if T is None else T
    B, H, K, V = wl.B, wl.H, wl.K, wl.V
    shapes = {"q": (B, H, T, K), "k": (B, H, T, K), "z": (B, H, T, K), "v": (B, H, T, V),
              "beta": (B, H, T), "state_in": (B, H, K, V)}
    if wl.adjoint:
        shapes["d_out"] = (B, H, T, V)
    out = {n: np.empty(s, dtype=np.float32) for n, s in shapes.items()}

    def fill(bh):
        b, h = bh
        sl = head_slice(wl, b, h, T)
        for n in shapes:
            out[n][b, h] = sl[n]

    n_threads = threads or min(16, len(os.sched_getaffinity(0)))
    pairs = [(b, h) for b in range(B) for h in range(H)]
    if n_threads > 1 and len(pairs) > 1:
        with ThreadPoolExecutor(n_threads) as ex:
            list(ex.map(fill, pairs))
    else:
        for bh in pairs:
            fill(bh)
    out["A_log"], out["dt_bias"] = head_params(wl)
    return out

