"""ctypes loader for libbsattn.so (the C ABI declared in include/bsattn.h).

The library is built in-tree by ``block_sparse_attention_07_amd.build``.  There
is no fallback: if the shared library is missing, loading raises ImportError.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbsattn.so")

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float

# name -> argument types (every entry point returns int except those in RESTYPES)
SIGNATURES = {
    "bsa_mask_words": [_i, _i],
    "sparse_attn_fwd": [_p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _p],
    "sparse_attn_fwd_noalloc": [_p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _p],
    "sparse_attn_workspace_bytes": [_i, _i, _i],
    "sparse_attn_fwd_ws": [_p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _p, ctypes.c_size_t, _p],
    "sparse_attn_fwd_f32": [_p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _p],
    "sparse_attn_plan": [_p, _i, _i, _i, _p, _p, _p, _p],
    "sparse_attn_fwd_planned": [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _p],
    "sparse_attn_fwd_b128": [_p, _p, _p, _p, _i, _i, _i, _f, _p, _p],
    "mask_b128_to_b64": [_p, _i, _i, _p, _p],
    "mask_from_stripes": [_p, _i, _i, _i, _i, _i, _p, _p],
    "block_scores_meanpool": [_p, _p, _i, _i, _i, _i, _f, _p, _p],
    "mask_from_block_scores_topp": [_p, _i, _i, _i, _f, _i, _p, _p],
    "mask_from_threshold_map": [_p, _p, _i, _i, _i, _p, _p],
    "mask_resize": [_p, _i, _i, _i, _p, _p],
    "threshold_map_resize": [_p, _i, _i, _i, _p, _p],
    "attn_fidelity": [_p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p, _p, _p],
    "permute_tokens": [_p, _p, _i, _i, _i, _i, _i, _p, _p],
    "hilbert3d_order": [_i, _i, _i, _p],
    "bsa_mfma_probe": [_i, _p, ctypes.c_longlong, _p, _p],
}
RESTYPES = {"sparse_attn_workspace_bytes": ctypes.c_size_t}
EXPORTS = ["bsa_last_error", *SIGNATURES]

_lib = None


class BsaError(RuntimeError):
    """A library entry point returned a non-zero status."""


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m block_sparse_attention_07_amd.build` (there is no fallback path)")
        handle = ctypes.CDLL(LIB_PATH)
        handle.bsa_last_error.restype = ctypes.c_char_p
        handle.bsa_last_error.argtypes = []
        for name, args in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = RESTYPES.get(name, ctypes.c_int)
        _lib = handle
    return _lib


def check(rc: int, what: str) -> None:
    if rc != 0:
        msg = lib().bsa_last_error().decode(errors="replace")
        raise BsaError(f"{what} failed with status {rc}: {msg}")
