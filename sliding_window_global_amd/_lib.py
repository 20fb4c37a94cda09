"""ctypes view of ``libplamo_attn.so`` (the C ABI in include/plamo_attn.h)."""

from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

c_int, c_ll, c_size, c_float, c_void_p = (ctypes.c_int, ctypes.c_longlong, ctypes.c_size_t,
                                           ctypes.c_float, ctypes.c_void_p)


class PlamoRope(ctypes.Structure):
    _fields_ = [("theta", ctypes.c_double), ("yarn_factor", ctypes.c_double),
                ("orig_ctx", ctypes.c_double), ("beta_fast", ctypes.c_double),
                ("beta_slow", ctypes.c_double), ("partial", ctypes.c_double)]


# name -> (restype, argtypes), mirroring include/plamo_attn.h
SIGNATURES = {
    "plamo_rope_table_bytes": (c_size, [c_ll, c_int]),
    "plamo_rope_table_init": (c_int, [c_void_p, c_size, c_ll, c_int, ctypes.POINTER(PlamoRope), c_void_p]),
    "plamo_prefill_padded_len": (c_ll, [c_ll]),
    "plamo_kv_append": (c_int, [c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_float, c_float,
                                c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_ll, c_int, c_int, c_int,
                                c_int, c_int, c_int, c_ll, c_void_p, c_size, c_int, c_void_p]),
    "plamo_prefill_pack": (c_int, [c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_ll, c_int, c_int,
                                   c_void_p]),
    "plamo_attn_prefill": (c_int, [c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int,
                                   c_int, c_int, c_ll, c_float, c_void_p]),
    "plamo_attn_prefill_fused_q": (c_int, [c_int, c_void_p, c_void_p, c_float, c_float, c_void_p, c_void_p,
                                           c_void_p, c_int, c_int, c_int, c_int, c_int, c_int, c_ll, c_void_p,
                                           c_size, c_int, c_float, c_void_p]),
    "plamo_attn_prefill_fused_q_ragged": (c_int, [c_int, c_void_p, c_void_p, c_float, c_float, c_void_p,
                                                  c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int, c_int,
                                                  c_void_p, c_void_p, c_ll, c_void_p, c_size, c_int, c_float,
                                                  c_void_p]),
    "plamo_attn_decode_workspace_bytes": (c_size, [c_int, c_int, c_int, c_int, c_int, c_ll]),
    "plamo_attn_decode": (c_int, [c_int, c_void_p, c_void_p, c_void_p, c_ll, c_void_p, c_void_p, c_size, c_int,
                                  c_int, c_int, c_int, c_int, c_int, c_ll, c_void_p, c_size, c_float, c_int,
                                  c_void_p]),
    "plamo_decode_step_workspace_bytes": (c_size, [c_int, c_int, c_int, c_int, c_int, c_ll]),
    "plamo_decode_step": (c_int, [c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_float, c_float,
                                  c_void_p, c_void_p, c_ll, c_void_p, c_void_p, c_size, c_int, c_int, c_int,
                                  c_int, c_int, c_ll, c_void_p, c_size, c_float, c_int, c_void_p]),
    "plamo_attn_decode_noalloc": (c_int, [c_int, c_void_p, c_void_p, c_void_p, c_ll, c_void_p, c_int, c_int,
                                          c_int, c_int, c_int, c_int, c_ll, c_void_p, c_size, c_float, c_int,
                                          c_void_p]),
    "plamo_kv_append_ragged": (c_int, [c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_float, c_float,
                                       c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_ll, c_int, c_int,
                                       c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_ll, c_void_p, c_size,
                                       c_int, c_void_p]),
    "plamo_attn_prefill_ragged": (c_int, [c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int, c_int,
                                          c_int, c_int, c_int, c_void_p, c_void_p, c_ll, c_float, c_void_p]),
    "plamo_attn_decode_ragged_workspace_bytes": (c_size, [c_int, c_int, c_int, c_int, c_int, c_ll]),
    "plamo_attn_decode_ragged": (c_int, [c_int, c_void_p, c_void_p, c_void_p, c_ll, c_void_p, c_void_p, c_size,
                                         c_int, c_int, c_int, c_int, c_int, c_void_p, c_ll, c_void_p, c_size,
                                         c_float, c_int, c_void_p]),
    "plamo_linear": (c_int, [c_void_p, c_void_p, c_void_p, c_ll, c_int, c_int, c_void_p]),
    "plamo_qkv_projection": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_ll, c_int, c_int, c_int,
                                     c_int, c_void_p]),
    "plamo_rms_norm": (c_int, [c_int, c_void_p, c_void_p, c_float, c_float, c_void_p, c_void_p, c_ll, c_int,
                               c_void_p]),
    "plamo_status_str": (ctypes.c_char_p, [c_int]),
    "plamo_last_error": (ctypes.c_char_p, []),
}

_LIB = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the built library (once). Raises if it has not been built: there is no
    fallback path."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = path or os.environ.get("PLAMO_ATTN_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib
