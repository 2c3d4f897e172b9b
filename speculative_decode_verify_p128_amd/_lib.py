"""ctypes declarations of libsdv.so (the C ABI in include/sdv.h) and of the cross-check
build libsdv_xcheck.so (the same library plus sdv_xcheck_* entry points that take the
kernel family as an argument; the tests use it to run every kernel implementation).

Loading fails loudly when a library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsdv.so")
XCHECK_LIB_PATH = os.path.join(_HERE, "libsdv_xcheck.so")

SDV_OK = 0
SDV_ERR_NULL_POINTER = 1
SDV_ERR_DTYPE = 2
SDV_ERR_GEOMETRY = 3
SDV_ERR_SHAPE = 4
SDV_ERR_WORKSPACE = 5
SDV_ERR_HIP = 6

SDV_F32 = 0
SDV_BF16 = 1
SDV_FP8_E4M3 = 2

NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024   # SDV_NOALLOC_SCRATCH_BYTES

SDV_OP_VERIFY_DENSE = 1
SDV_OP_VERIFY_SPARSE = 2
SDV_OP_VERIFY_PAGED = 3

# Kernel families of the cross-check entry points: 0 = the default kernel for the
# arguments; 1 = vector-ALU kernels; 3 = one LDS block stream per wave; 4 = the
# workgroup-shared LDS block ring; 5 = the persistent equal-range partition with the
# per-wave body (dense and paged, num_splits >= 2); 6 = the same partition over one ring
# per workgroup.  A family that does not serve a call runs the default kernel.
FAMILY_AUTO, FAMILY_VALU, FAMILY_WAVES, FAMILY_RING, FAMILY_PERSIST, FAMILY_FLAT = 0, 1, 3, 4, 5, 6

DEVERR_QO_LEN = 1
DEVERR_KV_CAPACITY = 2
DEVERR_PAGE_RANGE = 4
DEVERR_TOPK_INDEX = 8
DEVERR_COPY_RANGE = 16


class SubpageGeom(C.Structure):
    _fields_ = [
        ("phys_page", C.c_int32), ("sub_page", C.c_int32), ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32), ("slot_stride", C.c_int32), ("kv_offset", C.c_int32),
        ("num_layers", C.c_int32), ("num_slots", C.c_int32), ("pool_index_scale", C.c_int32),
        ("kv_dtype", C.c_int32), ("k_scale", C.c_float), ("v_scale", C.c_float),
        ("k_root", C.c_void_p),
    ]


class SubpageView(C.Structure):
    _fields_ = [
        ("k_root", C.c_void_p), ("kv_dtype", C.c_int32), ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32), ("index_scale", C.c_int32), ("num_slots", C.c_int32),
        ("k_scale", C.c_float), ("v_scale", C.c_float), ("num_sub_pages", C.c_int64),
    ]


class PagedKV(C.Structure):
    _fields_ = [
        ("k", C.c_void_p), ("v", C.c_void_p), ("page_stride", C.c_int64),
        ("num_pages", C.c_int32), ("page_size", C.c_int32), ("num_kv_heads", C.c_int32),
        ("head_dim", C.c_int32), ("kv_dtype", C.c_int32), ("k_scale", C.c_float),
        ("v_scale", C.c_float),
    ]


_P = C.c_void_p
_I = C.c_int32
_F = C.c_float
_S = C.c_size_t

# name -> (restype, argtypes)
SIGNATURES = {
    "kv_subpage_view_init": (_I, [C.POINTER(SubpageGeom), _P, _I, _I, _I, _P,
                                  C.POINTER(SubpageView), _P, _P]),
    "verify_attention_dense": (_I, [_P, _I, _P, _P, _I, _I, _I, C.POINTER(SubpageView), _P, _I,
                                    _F, _I, _P, _S, _P, _I, _P, _P]),
    "verify_attention_dense_view": (_I, [_P, _I, _P, _P, _I, _I, _I, C.POINTER(SubpageView), _P,
                                         _I, _I, _F, _I, _P, _S, _P, _I, _P, _P]),
    "verify_attention_dense_view_noalloc": (_I, [_P, _I, _P, _P, _I, _I, _I,
                                                 C.POINTER(SubpageView), _P, _I, _I, _F, _I, _P,
                                                 _I, _P, _P]),
    "proxy_page_scores": (_I, [_P, _I, _P, _P, _I, _I, _I, C.POINTER(PagedKV), _P, _I, _I, _P,
                               _P, _P]),
    "ladder_topk_pages": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "verify_attention_sparse": (_I, [_P, _I, _P, _P, _I, _I, _I, C.POINTER(PagedKV), _P, _I, _I,
                                     _P, _I, _F, _I, _P, _S, _P, _I, _P, _P]),
    "verify_attention_sparse_select": (_I, [_P, _I, _P, _P, _I, _I, _I, C.POINTER(PagedKV), _P,
                                            _I, _I, _P, _I, _P, _P, _F, _I, _P, _S, _P, _I, _P,
                                            _P]),
    "verify_attention_paged": (_I, [_P, _I, _P, _P, _I, _I, _I, C.POINTER(PagedKV), _P, _I, _I,
                                    _F, _I, _P, _S, _P, _I, _P, _P]),
    "stage_verify_kv_paged": (_I, [_P, _P, _I, _P, _P, _I, _I, C.POINTER(PagedKV), _P, _I, _I,
                                   _P, _P]),
    "stage_verify_kv_view": (_I, [_P, _P, _I, _P, _P, _I, _I, C.POINTER(SubpageView), _P, _I,
                                  _P, _P]),
    "hnd_head_slice_descriptors": (_I, [_I, _I, _I, _I, _I, _I, _I, _I, _I, _P, _P, _I, _P, _I,
                                        _P]),
    "copy_descriptors": (_I, [_P, _S, _P, _S, _P, _I, _P, _P]),
    "greedy_accept": (_I, [_P, _I, _I, _P, _P, _P, _I, _I, _P, _S, _P, _P, _P, _P, _P, _P]),
    "sdv_greedy_accept_workspace_bytes": (_S, [_I, _I, _I, _I]),
    "lse_combine": (_I, [_P, _P, _I, _I, _I, _I, _P, _I, _P, _P]),
    "sdv_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "sdv_status_string": (C.c_char_p, [_I]),
    "sdv_last_error": (C.c_char_p, []),
    "sdv_fill_u32": (_I, [_P, _S, C.c_uint32, _P]),
    "sdv_read_probe": (_I, [_P, _S, _P, _I, _P]),
    "sdv_read_units_probe": (_I, [_P, _S, _P, C.c_int64, _I, _P, _I, _P]),
}

# The cross-check build's extra entry points: the attention calls with a leading family.
XCHECK_SIGNATURES = {
    f"sdv_xcheck_{name}": (SIGNATURES[name][0], [_I, *SIGNATURES[name][1]])
    for name in ("verify_attention_dense", "verify_attention_dense_view",
                 "verify_attention_sparse", "verify_attention_sparse_select",
                 "verify_attention_paged")
}

_lib = None
_xlib = None


def _open(path: str, signatures) -> C.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(hipcc, gfx950); there is no fallback implementation")
    lib = C.CDLL(path)
    for name, (res, args) in signatures.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


def load() -> C.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _open(LIB_PATH, SIGNATURES)
    return _lib


def load_xcheck() -> C.CDLL:
    """The cross-check build (raises if it has not been built)."""
    global _xlib
    if _xlib is None:
        _xlib = _open(XCHECK_LIB_PATH, {**SIGNATURES, **XCHECK_SIGNATURES})
    return _xlib


class SdvError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"sdv status {status}: {message}")
        self.status = status
        self.message = message


def check(status: int, lib: C.CDLL = None) -> None:
    if status != SDV_OK:
        lib = lib or load()
        raise SdvError(status, lib.sdv_last_error().decode() or lib.sdv_status_string(status).decode())
