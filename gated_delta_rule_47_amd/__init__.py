"""Kimi Delta Attention (KDA) on AMD Instinct MI355X: Python binding of libkda.

Argument marshalling only: every function checks the tensors, passes their device
pointers and the current HIP stream to the C ABI declared in include/kda.h, and
raises KdaError on a non-zero status.  All arithmetic runs in the library's HIP
kernels; there is no Python or CPU implementation behind these functions.

Layouts (head-major, contiguous): q, k, z (B,H,T,K); v, o (B,H,T,V); beta (B,H,T);
state (B,H,K,V) float32; A_log (H,) float32; dt_bias (H,K) float32.  Activations are
float32 or bfloat16 (one dtype for q, k, v, z, beta and o).
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

__all__ = ["KdaError", "read_scale", "gate", "chunk_fwd", "chunk_fwd_scalar", "chunk_fwd_workspace_bytes",
           "chunk_fwd_status", "set_exchange_timeout_us", "chunk_fwd_norm",
           "chunk_fwd_norm_workspace_bytes", "recurrent_step", "recurrent_step_scalar", "chunk_bwd",
           "chunk_bwd_workspace_bytes", "gate_bwd", "gate_bwd_workspace_bytes", "gate_bwd_noalloc",
           "GATE_BWD_SCRATCH_BYTES", "counters", "status_string",
           "library_path"]


class KdaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (fn, status_string(status), status))


def library_path() -> str:
    return _lib.LIB_PATH


def status_string(status: int) -> str:
    return _lib.load().kda_status_string(int(status)).decode()


def read_scale(K: int) -> float:
    """FLA's default read scale K**-0.5, as the library computes it."""
    return float(_lib.load().kda_read_scale(int(K)))


def counters() -> dict:
    lib = _lib.load()
    n = lib.kda_get_counters(None, 0)
    arr = (ctypes.c_ulonglong * n)()
    lib.kda_get_counters(arr, n)
    return {name: int(arr[i]) for i, name in enumerate(_lib.COUNTER_NAMES[:n])}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return _lib.KDA_F32
    if t.dtype == torch.bfloat16:
        return _lib.KDA_BF16
    raise TypeError("activations must be float32 or bfloat16, got %s" % t.dtype)


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _check_f32(name, t, shape):
    if t is None:
        return
    if t.dtype != torch.float32:
        raise TypeError("%s must be float32" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _check_out(name, t, shape, dtype, device):
    """A caller-supplied output must have exactly the shape, dtype and device the kernels
    write: the C ABI sees only a pointer and cannot check its size."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _call(fn_name, *args):
    st = getattr(_lib.load(), fn_name)(*args)
    if st != _lib.KDA_OK:
        raise KdaError(fn_name, st)


def gate(z, A_log, dt_bias=None, want_alpha=True):
    """g = -exp(clamp(A_log)) * softplus(z + dt_bias) and alpha = exp(g), float32."""
    B, H, T, K = z.shape
    _check_f32("A_log", A_log, (H,))
    _check_f32("dt_bias", dt_bias, (H, K))
    g = torch.empty(z.shape, dtype=torch.float32, device=z.device)
    alpha = torch.empty_like(g) if want_alpha else None
    _call("kda_gate", _ptr(z), _ptr(A_log), _ptr(dt_bias), _ptr(g), _ptr(alpha), B, H, T, K,
          _dtype_code(z), _stream(z.device))
    return g, alpha


def _check_acts(q, k, v, z, beta, scalar_gate=False):
    B, H, T, K = q.shape
    V = v.shape[-1]
    zshape = (B, H, T) if scalar_gate else (B, H, T, K)
    for name, t, shape in (("k", k, (B, H, T, K)), ("z", z, zshape), ("v", v, (B, H, T, V)),
                           ("beta", beta, (B, H, T))):
        if tuple(t.shape) != shape:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), shape))
        if t.dtype != q.dtype:
            raise TypeError("%s has dtype %s, q has %s" % (name, t.dtype, q.dtype))
    return B, H, T, K, V


def chunk_fwd_workspace_bytes(B, H, T, K, V, chunk=64, dtype=torch.bfloat16) -> int:
    """Workspace bytes kda_chunk_fwd can use (nonzero for bf16, V = 128, chunk 32/64)."""
    code = _lib.KDA_BF16 if dtype == torch.bfloat16 else _lib.KDA_F32
    return int(_lib.load().kda_chunk_fwd_workspace_bytes(B, H, T, K, V, chunk, code))


def chunk_fwd_status(workspace) -> int:
    """Synchronizes the current stream and returns (and clears) the status of the last
    paired forward that used `workspace`: 0, or KDA_ERR_EXCHANGE (-9)."""
    return int(_lib.load().kda_chunk_fwd_status(_ptr(workspace), _stream(workspace.device)))


def set_exchange_timeout_us(us: int) -> None:
    """Bound of the paired forward's waits in microseconds (0: give up at once)."""
    _call("kda_set_exchange_timeout_us", ctypes.c_ulonglong(int(us)))


def chunk_fwd(q, k, v, z, A_log, dt_bias, beta, state_in=None, scale=None, chunk=64,
              output_state=True, out=None, state_out=None, workspace=None):
    """Chunked KDA forward.  Returns (o, state_out); state_out is None when
    output_state is False.  scale=None means K**-0.5.  workspace: None runs without one
    (each value tile computes every block's gate and WY stages), "auto" allocates the
    buffer chunk_fwd_workspace_bytes() asks for (torch's caching allocator), or a uint8
    CUDA tensor of at least that size (the paired path)."""
    return _chunk_fwd("kda_chunk_fwd", q, k, v, z, A_log, dt_bias, beta, state_in, scale, chunk, output_state,
                      out, state_out, workspace)


def chunk_fwd_scalar(q, k, v, a, A_log, dt_bias, beta, state_in=None, scale=None, chunk=64,
                     output_state=True, out=None, state_out=None, workspace=None):
    """Chunked forward under a scalar decay: a (B,H,T) one gate input per token and
    head, dt_bias (H,) or None.  Otherwise as chunk_fwd."""
    return _chunk_fwd("kda_chunk_fwd_scalar", q, k, v, a, A_log, dt_bias, beta, state_in, scale, chunk,
                      output_state, out, state_out, workspace)


def _chunk_fwd(fn, q, k, v, z, A_log, dt_bias, beta, state_in, scale, chunk, output_state, out, state_out,
               workspace):
    scalar_gate = fn == "kda_chunk_fwd_scalar"
    B, H, T, K, V = _check_acts(q, k, v, z, beta, scalar_gate)
    _check_f32("A_log", A_log, (H,))
    _check_f32("dt_bias", dt_bias, (H,) if scalar_gate else (H, K))
    _check_f32("state_in", state_in, (B, H, K, V))
    _check_out("out", out, (B, H, T, V), q.dtype, q.device)
    _check_out("state_out", state_out, (B, H, K, V), torch.float32, q.device)
    if scale is None:
        scale = read_scale(K)
    o = out if out is not None else torch.empty((B, H, T, V), dtype=q.dtype, device=q.device)
    if output_state and state_out is None:
        state_out = torch.empty((B, H, K, V), dtype=torch.float32, device=q.device)
    if not output_state:
        state_out = None
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a tensor")
        need = chunk_fwd_workspace_bytes(B, H, T, K, V, chunk, q.dtype)
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    wbytes = 0
    if workspace is not None:
        if workspace.device != q.device:
            raise ValueError("workspace is on %s, expected %s" % (workspace.device, q.device))
        wbytes = workspace.numel() * workspace.element_size()
    _call(fn, _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A_log), _ptr(dt_bias), _ptr(beta),
          _ptr(state_in), float(scale), int(chunk), _ptr(o), _ptr(state_out), _ptr(workspace), wbytes,
          B, H, T, K, V, _dtype_code(q), _stream(q.device))
    return o, state_out


def chunk_fwd_norm_workspace_bytes(B, H, T, K, V, dtype=torch.bfloat16) -> int:
    code = _lib.KDA_BF16 if dtype == torch.bfloat16 else _lib.KDA_F32
    return int(_lib.load().kda_chunk_fwd_norm_workspace_bytes(B, H, T, K, V, code))


def chunk_fwd_norm(q, k, v, z, A_log, dt_bias, beta, state_in=None, norm_weight=None, eps=1e-6, scale=None,
                   chunk=64, output_state=True, out=None, state_out=None, workspace="auto"):
    """chunk_fwd with the output RMSNorm fused into its output stage (bf16 only): o holds
    r / sqrt(mean_v r^2 + eps) * norm_weight[h] for the read r.  norm_weight (H, V) float32
    or None (ones).  workspace: "auto" allocates (zero-filled) what
    chunk_fwd_norm_workspace_bytes() asks for (nonzero when V > 64), or a uint8 CUDA tensor
    of at least that size, zero-filled before its first use and used for this call only."""
    B, H, T, K, V = _check_acts(q, k, v, z, beta)
    _check_f32("A_log", A_log, (H,))
    _check_f32("dt_bias", dt_bias, (H, K))
    _check_f32("state_in", state_in, (B, H, K, V))
    _check_f32("norm_weight", norm_weight, (H, V))
    _check_out("out", out, (B, H, T, V), q.dtype, q.device)
    _check_out("state_out", state_out, (B, H, K, V), torch.float32, q.device)
    if scale is None:
        scale = read_scale(K)
    o = out if out is not None else torch.empty((B, H, T, V), dtype=q.dtype, device=q.device)
    if output_state and state_out is None:
        state_out = torch.empty((B, H, K, V), dtype=torch.float32, device=q.device)
    if not output_state:
        state_out = None
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', None or a tensor")
        need = chunk_fwd_norm_workspace_bytes(B, H, T, K, V, q.dtype)
        workspace = torch.zeros(need, dtype=torch.uint8, device=q.device) if need else None
    wbytes = 0
    if workspace is not None:
        if workspace.device != q.device:
            raise ValueError("workspace is on %s, expected %s" % (workspace.device, q.device))
        wbytes = workspace.numel() * workspace.element_size()
    _call("kda_chunk_fwd_norm", _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A_log), _ptr(dt_bias), _ptr(beta),
          _ptr(state_in), float(scale), int(chunk), _ptr(norm_weight), float(eps), _ptr(o), _ptr(state_out),
          _ptr(workspace), wbytes, B, H, T, K, V, _dtype_code(q), _stream(q.device))
    return o, state_out


def recurrent_step(q, k, v, z, A_log, dt_bias, beta, state, scale=None, out=None):
    """One decode token per (b,h): q,k,z (B,H,K), v (B,H,V), beta (B,H).  Updates
    `state` (B,H,K,V) float32 in place and returns o (B,H,V)."""
    return _recurrent_step("kda_recurrent_step", q, k, v, z, A_log, dt_bias, beta, state, scale, out)


def recurrent_step_scalar(q, k, v, a, A_log, dt_bias, beta, state, scale=None, out=None):
    """Decode step under a scalar decay: a (B,H) one gate input per sequence and head,
    dt_bias (H,) or None.  Otherwise as recurrent_step."""
    return _recurrent_step("kda_recurrent_step_scalar", q, k, v, a, A_log, dt_bias, beta, state, scale, out)


def _recurrent_step(fn, q, k, v, z, A_log, dt_bias, beta, state, scale, out):
    scalar_gate = fn == "kda_recurrent_step_scalar"
    B, H, K = q.shape
    V = v.shape[-1]
    zshape = (B, H) if scalar_gate else (B, H, K)
    for name, t, shape in (("k", k, (B, H, K)), ("z", z, zshape), ("v", v, (B, H, V)), ("beta", beta, (B, H))):
        if tuple(t.shape) != shape:
            raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), shape))
        if t.dtype != q.dtype:
            raise TypeError("%s has dtype %s, q has %s" % (name, t.dtype, q.dtype))
    _check_f32("A_log", A_log, (H,))
    _check_f32("dt_bias", dt_bias, (H,) if scalar_gate else (H, K))
    _check_f32("state", state, (B, H, K, V))
    _check_out("out", out, (B, H, V), q.dtype, q.device)
    if scale is None:
        scale = read_scale(K)
    o = out if out is not None else torch.empty((B, H, V), dtype=q.dtype, device=q.device)
    _call(fn, _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A_log), _ptr(dt_bias), _ptr(beta),
          _ptr(state), float(scale), _ptr(o), B, H, K, V, _dtype_code(q), _stream(q.device))
    return o


def chunk_bwd_workspace_bytes(B, H, T, K, V, chunk=64) -> int:
    return int(_lib.load().kda_chunk_bwd_workspace_bytes(B, H, T, K, V, chunk))


def chunk_bwd(q, k, v, z, A_log, dt_bias, beta, state_in, d_o, d_state_out=None, scale=None, chunk=64,
              workspace=None):
    """Gradients of sum(o*d_o) + sum(state_out*d_state_out); float32 activations.
    Returns dict(dq, dk, dv, dg, dbeta, dstate_in), all float32."""
    B, H, T, K, V = _check_acts(q, k, v, z, beta)
    _check_f32("A_log", A_log, (H,))
    _check_f32("dt_bias", dt_bias, (H, K))
    _check_f32("state_in", state_in, (B, H, K, V))
    _check_f32("d_state_out", d_state_out, (B, H, K, V))
    if tuple(d_o.shape) != (B, H, T, V) or d_o.dtype != q.dtype:
        raise ValueError("d_o must match o's shape and dtype")
    if scale is None:
        scale = read_scale(K)
    need = chunk_bwd_workspace_bytes(B, H, T, K, V, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dq=torch.empty((B, H, T, K), **f32), dk=torch.empty((B, H, T, K), **f32),
               dv=torch.empty((B, H, T, V), **f32), dg=torch.empty((B, H, T, K), **f32),
               dbeta=torch.empty((B, H, T), **f32), dstate_in=torch.empty((B, H, K, V), **f32))
    _call("kda_chunk_bwd", _ptr(q), _ptr(k), _ptr(v), _ptr(z), _ptr(A_log), _ptr(dt_bias), _ptr(beta),
          _ptr(state_in), float(scale), int(chunk), _ptr(d_o), _ptr(d_state_out), _ptr(out["dq"]),
          _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dstate_in"]),
          _ptr(workspace), workspace.numel() * workspace.element_size(), B, H, T, K, V, _dtype_code(q),
          _stream(dev))
    return out


def gate_bwd_workspace_bytes(B, H, T, K) -> int:
    return int(_lib.load().kda_gate_bwd_workspace_bytes(B, H, T, K))


def gate_bwd(z, A_log, dt_bias, dg, want_dz=True, workspace=None, dz_out=None):
    """Adjoint of gate() for a cotangent dg on g: returns (dz or None, dA_log (H,),
    d_dt_bias (H, K)), float32.  dz_out may be dg itself (computed in place)."""
    B, H, T, K = z.shape
    _check_f32("A_log", A_log, (H,))
    _check_f32("dt_bias", dt_bias, (H, K))
    _check_f32("dg", dg, (B, H, T, K))
    dev = z.device
    f32 = dict(dtype=torch.float32, device=dev)
    _check_out("dz_out", dz_out, (B, H, T, K), torch.float32, dev)
    dz = (dz_out if dz_out is not None else torch.empty((B, H, T, K), **f32)) if want_dz else None
    dA = torch.empty((H,), **f32)
    ddb = torch.empty((H, K), **f32)
    need = gate_bwd_workspace_bytes(B, H, T, K)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _call("kda_gate_bwd", _ptr(z), _ptr(A_log), _ptr(dt_bias), _ptr(dg), _ptr(dz), _ptr(dA), _ptr(ddb),
          _ptr(workspace), workspace.numel() * workspace.element_size(), B, H, T, K, _dtype_code(z), _stream(dev))
    return dz, dA, ddb


# Bytes of the library's built-in scratch that gate_bwd_noalloc uses (per GPU).
GATE_BWD_SCRATCH_BYTES = 16 << 20


def gate_bwd_noalloc(z, A_log, dt_bias, dg, dz_out=None, dA_out=None, ddb_out=None, want_dz=True):
    """gate_bwd through the entry point that allocates no device memory: the partial sums
    live in the library's per-GPU scratch (sizes needing more than GATE_BWD_SCRATCH_BYTES
    are rejected).  Outputs are allocated here unless given; calls that may overlap on one
    GPU (unordered streams) race on the scratch."""
    B, H, T, K = z.shape
    _check_f32("A_log", A_log, (H,))
    _check_f32("dt_bias", dt_bias, (H, K))
    _check_f32("dg", dg, (B, H, T, K))
    dev = z.device
    f32 = dict(dtype=torch.float32, device=dev)
    _check_out("dz_out", dz_out, (B, H, T, K), torch.float32, dev)
    _check_out("dA_out", dA_out, (H,), torch.float32, dev)
    _check_out("ddb_out", ddb_out, (H, K), torch.float32, dev)
    dz = (dz_out if dz_out is not None else torch.empty((B, H, T, K), **f32)) if want_dz else None
    dA = dA_out if dA_out is not None else torch.empty((H,), **f32)
    ddb = ddb_out if ddb_out is not None else torch.empty((H, K), **f32)
    _call("kda_gate_bwd_noalloc", _ptr(z), _ptr(A_log), _ptr(dt_bias), _ptr(dg), _ptr(dz), _ptr(dA), _ptr(ddb),
          B, H, T, K, _dtype_code(z), _stream(dev))
    return dz, dA, ddb
