"""ctypes loader for libkda.so and the C prototypes of include/kda.h."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

KDA_OK = 0
KDA_F32 = 0
KDA_BF16 = 1
COUNTER_NAMES = ("gate", "chunk_fwd", "recurrent_step", "chunk_bwd", "rejected", "gate_bwd")
EXPORTED = ("kda_read_scale", "kda_gate", "kda_chunk_fwd_workspace_bytes", "kda_chunk_fwd", "kda_chunk_fwd_scalar",
            "kda_chunk_fwd_status", "kda_set_exchange_timeout_us", "kda_recurrent_step",
            "kda_recurrent_step_scalar",
            "kda_chunk_bwd_workspace_bytes", "kda_chunk_bwd", "kda_gate_bwd_workspace_bytes", "kda_gate_bwd", "kda_gate_bwd_noalloc", "kda_chunk_fwd_norm_workspace_bytes", "kda_chunk_fwd_norm",
            "kda_status_string", "kda_get_counters")

_lib = None

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

_PROTOS = {
    "kda_read_scale": (_f, [_i]),
    "kda_gate": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p]),
    "kda_chunk_fwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "kda_chunk_fwd_norm_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "kda_chunk_fwd_norm": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _f, _i, _p, _f, _p, _p, _p, _sz, _i, _i, _i, _i, _i, _i,
                                _p]),
    "kda_chunk_fwd": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _f, _i, _p, _p, _p, _sz, _i, _i, _i, _i, _i, _i, _p]),
    "kda_chunk_fwd_scalar": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _f, _i, _p, _p, _p, _sz, _i, _i, _i, _i, _i, _i,
                                  _p]),
    "kda_chunk_fwd_status": (_i, [_p, _p]),
    "kda_set_exchange_timeout_us": (_i, [ctypes.c_ulonglong]),
    "kda_recurrent_step": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _f, _p, _i, _i, _i, _i, _i, _p]),
    "kda_recurrent_step_scalar": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _f, _p, _i, _i, _i, _i, _i, _p]),
    "kda_chunk_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "kda_chunk_bwd": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _f, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz,
                           _i, _i, _i, _i, _i, _i, _p]),
    "kda_gate_bwd_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "kda_gate_bwd": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _sz, _i, _i, _i, _i, _i, _p]),
    "kda_gate_bwd_noalloc": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _p]),
    "kda_status_string": (ctypes.c_char_p, [_i]),
    "kda_get_counters": (_i, [ctypes.POINTER(ctypes.c_ulonglong), _i]),
}


def load(path: str | None = None):
    """Load (once) and return the library.  Raises if it has not been built: there
    is no other implementation to fall back to."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise ImportError(
            "libkda.so not found at %s: build it first (python -m gated_delta_rule_47_amd._build "
            "or __graft_entry__.build())" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in _PROTOS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
