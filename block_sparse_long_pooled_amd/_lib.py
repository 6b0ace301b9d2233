"""ctypes loader and signatures for libflashprefill.so (include/flashprefill.h).

The library is built in-tree by ``block_sparse_long_pooled_amd.build``; loading
fails loudly when it is missing -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int, c_int64, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
# FLASHPREFILL_LIB selects another build of the same library (e.g. a debug build)
LIB_PATH = os.environ.get("FLASHPREFILL_LIB") or os.path.join(HERE, "libflashprefill.so")

FP_OK, FP_EINVAL, FP_EUNSUPPORTED, FP_EHIP = 0, 1, 2, 3
ABI_VERSION = 4  # the signatures below; the library must report the same version
FP_BF16, FP_FP8_E4M3 = 0, 1


class FlashPrefillError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


STATUS_NAMES = {FP_OK: "FP_OK", FP_EINVAL: "FP_EINVAL", FP_EUNSUPPORTED: "FP_EUNSUPPORTED", FP_EHIP: "FP_EHIP"}

_p = c_void_p
_i64 = c_int64
_SIGNATURES = {
    "fp_status_string": (c_char_p, [c_int]),
    "fp_last_error": (c_char_p, []),
    "fp_abi_version": (c_int, []),
    "fp_num_blocks": (c_int64, [c_int64, c_int]),
    "fp_idx_capacity": (c_int64, [c_int, c_int64]),
    "fp_discover": (c_int, [_p, _p, c_int, _p, _p, c_int, c_int, c_int, c_int, c_int,
                            _i64, _i64, _i64, _i64, _p, _p, _p]),
    "fp_threshold_compact": (c_int, [_p, _p, c_int, c_int, c_int, c_int, c_double, c_double, c_int, c_int,
                                     _p, _p, _p, _p]),
    "fp_sparse_attn": (c_int, [_p, _p, _p, c_int, _p, _p, _p, c_int, c_int, c_int, c_int, c_int,
                               _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _p, _p, c_float, _p, _p, _p]),
    "fp_dense_attn": (c_int, [_p, _p, _p, c_int, _p, _p, _p, c_int, c_int, c_int, c_int, c_int,
                              _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, c_float, _p, _p, _p]),
    "fp_mask_words": (c_int, [c_int64]),
    "fp_threshold_mask": (c_int, [_p, _p, c_int, c_int, c_int, c_int, c_double, c_double, c_int, c_int, _p, _p]),
    "fp_sparse_attn_masked": (c_int, [_p, _p, _p, c_int, _p, _p, _p, c_int, c_int, c_int, c_int, c_int,
                                      _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _p, c_float, _p, _p, _p]),
    "fp_pool": (c_int, [_p, c_int, _p, c_int, c_int, c_int, c_int, _i64, _i64, _p, _p]),
    "fp_mean_correct": (c_int, [_p, c_int, _p, _p, _p, c_int, c_int, c_int, c_int, c_int,
                                _i64, _i64, _i64, _i64, _p, _p, c_float, _p, _p, _p, _i64, _p]),
    "fp_mean_correct_workspace_bytes": (c_int64, [c_int, c_int]),
    "fp_mean_correct_varlen": (c_int, [_p, c_int, _p, _p, _p, _p, c_int, c_int, _i64, _i64, _i64,
                                       c_int, c_int, c_int, c_int, _i64, _i64, _i64, _i64, _p, _p, c_float,
                                       _p, _p, _p, _i64, _p]),
    "fp_mean_correct_varlen_workspace_bytes": (c_int64, [c_int64, c_int, c_int]),
    "fp_pool_varlen": (c_int, [_p, c_int, _p, _p, c_int, c_int, _i64, _i64, _p, c_int, c_int, c_int, c_int, c_int,
                               _i64, _i64, _i64, _p, _p]),
    "fp_mean_correct_noalloc": (c_int, [_p, c_int, _p, _p, _p, c_int, c_int, c_int, c_int, c_int,
                                        _i64, _i64, _i64, _i64, _p, _p, c_float, _p, _p, _p]),
    "fp_union_compact": (c_int, [_p, c_int, c_int, c_int, _p, _p, _p]),
    "fp_sparse_attn_grouped": (c_int, [_p, _p, _p, c_int, _p, _p, _p, c_int, c_int, c_int, c_int, c_int,
                                       _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _p, _p, c_float, _p, _p, _p]),
    "fp_discover_chunked": (c_int, [_p, _p, c_int, _p, _p, _p, _p, c_int, c_int, c_int, _i64, _i64, _i64, _i64,
                                    _p, c_int, c_int, c_int, c_int, c_int, c_int,
                                    _i64, _i64, _i64, _i64, _i64, _p, _p, _p]),
    "fp_threshold_compact_chunked": (c_int, [_p, _p, _p, _p, c_int, c_int, c_int, _i64, _i64, _i64,
                                             c_int, c_int, c_int, c_double, c_double, c_int, c_int, _p, _p, _p]),
    "fp_sparse_attn_chunked": (c_int, [_p, _p, _p, c_int, _p, _p, _p, _p, _p, c_int, c_int, c_int,
                                       _i64, _i64, _i64, _i64, _i64, _p, c_int, c_int,
                                       c_int, c_int, c_int, c_int,
                                       _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                       _p, _p, c_float, _p, _p, _p]),
    "fp_discover_paged": (c_int, [_p, _p, c_int, _p, _p, _p, c_int, c_int, _i64, _i64, _p, c_int, c_int,
                                  c_int, c_int, c_int, c_int, _i64, _i64, _i64, _i64, _i64, _p, _p, _p]),
    "fp_threshold_compact_varlen": (c_int, [_p, _p, _p, c_int, c_int, _i64, _i64, c_int, c_int, c_int,
                                            c_double, c_double, c_int, c_int, _p, _p, _p]),
    "fp_sparse_attn_paged": (c_int, [_p, _p, _p, c_int, _p, _p, _p, _p, c_int, c_int, _i64, _i64, _i64,
                                     _p, c_int, c_int, c_int, c_int, c_int, c_int,
                                     _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                     _p, _p, c_float, _p, _p, _p]),
}

EXPORTED = tuple(_SIGNATURES)

_lib = None


def load():
    """Load the shared library once and attach the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m block_sparse_long_pooled_amd.build` "
            "(there is no CPU fallback for the HIP path)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.fp_abi_version.restype = c_int
    if lib.fp_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {lib.fp_abi_version()}, the binding expects {ABI_VERSION}: "
                          "rebuild it with `python -m block_sparse_long_pooled_amd.build`")
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def call(name: str, *args) -> None:
    """Call an entry point and raise FlashPrefillError on a non-zero status."""
    lib = load()
    rc = getattr(lib, name)(*args)
    if rc != FP_OK:
        raise FlashPrefillError(rc, name, lib.fp_last_error().decode())


def status_of(name: str, *args) -> int:
    """Call an entry point and return its raw status (used by the ABI tests)."""
    return getattr(load(), name)(*args)
