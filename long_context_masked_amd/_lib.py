"""ctypes view of the C interface declared in include/attn.h.

Argument marshalling only: every step of the computation runs in libattn.so.
Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_NOMEM, ATTN_ERR_DEVICE = range(5)
STATUS_NAMES = {0: "ATTN_OK", 1: "ATTN_ERR_INVALID", 2: "ATTN_ERR_UNSUPPORTED",
                3: "ATTN_ERR_NOMEM", 4: "ATTN_ERR_DEVICE"}

MASK_FULL, MASK_CAUSAL, MASK_SLIDING, MASK_DOCUMENT, MASK_PREFIX_LM, MASK_COLUMN_BOUNDS = range(6)

P32 = C.POINTER(C.c_int32)
PU8 = C.POINTER(C.c_uint8)


class Shape(C.Structure):
    _fields_ = [("B", C.c_int64), ("S", C.c_int64), ("Hq", C.c_int64), ("Hkv", C.c_int64),
                ("d", C.c_int64), ("scale", C.c_float)]


class MaskDesc(C.Structure):
    _fields_ = [("kind", C.c_int32), ("causal", C.c_int32), ("window_left", C.c_int32),
                ("window_right", C.c_int32), ("num_docs", C.c_int32),
                ("cu_seqlens", P32), ("prefix_lens", P32), ("col_bounds", P32),
                ("block_bitmap", PU8), ("bitmap_heads", C.c_int32), ("n_qblk", C.c_int32),
                ("n_kblk", C.c_int32), ("q_blk_offsets", P32), ("k_blk_offsets", P32),
                ("dynamic", C.c_int32), ("bwd_key_tile", C.c_int32)]


class Stats(C.Structure):
    _fields_ = [("nnz_per_batch", C.c_int64), ("nnz_total", C.c_int64),
                ("flops_fwd", C.c_double), ("flops_bwd", C.c_double),
                ("fwd_items", C.c_int64), ("fwd_tiles_full", C.c_int64),
                ("fwd_tiles_partial", C.c_int64), ("bwd_items", C.c_int64),
                ("bwd_tiles_full", C.c_int64), ("bwd_tiles_partial", C.c_int64),
                ("fwd_tile_rows", C.c_int64), ("fwd_tile_cols", C.c_int64),
                ("bwd_tile_rows", C.c_int64), ("bwd_tile_cols", C.c_int64),
                ("heads_per_item", C.c_int64), ("device_bytes", C.c_int64),
                ("bwd_head_entries", C.c_int64)]


class Layout(C.Structure):
    _fields_ = [("blob", C.c_void_p), ("blob_bytes", C.c_int64),
                ("off_rowb", C.c_int64), ("off_colb", C.c_int64),
                ("off_fwd_items", C.c_int64), ("n_fwd_items", C.c_int64),
                ("off_fwd_list", C.c_int64), ("n_fwd_list", C.c_int64),
                ("off_bwd_items", C.c_int64), ("n_bwd_items", C.c_int64),
                ("off_bwd_list", C.c_int64), ("n_bwd_list", C.c_int64),
                ("off_bits", C.c_int64), ("off_qblk", C.c_int64), ("off_kblk", C.c_int64),
                ("off_qoffs", C.c_int64), ("off_koffs", C.c_int64),
                ("off_bwd_slot", C.c_int64), ("off_bwd_reduce", C.c_int64),
                ("n_bwd_reduce", C.c_int64), ("n_slots", C.c_int64),
                ("off_kwords", C.c_int64), ("off_rwords", C.c_int64)]


# Every symbol include/attn.h declares, with its ctypes signature.
SIGNATURES = {
    "attn_plan_create": (C.c_int, [C.POINTER(Shape), C.POINTER(MaskDesc), C.POINTER(C.c_void_p)]),
    "attn_plan_device_bytes": (C.c_size_t, [C.c_void_p]),
    "attn_plan_bind": (C.c_int, [C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]),
    "attn_plan_set_bitmap": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p]),
    "attn_plan_stats": (C.c_int, [C.c_void_p, C.POINTER(Stats)]),
    "attn_plan_get_layout": (C.c_int, [C.c_void_p, C.POINTER(Layout)]),
    "attn_bwd_workspace_bytes": (C.c_size_t, [C.c_void_p]),
    "attn_fwd": (C.c_int, [C.c_void_p] * 5 + [C.c_void_p, C.c_void_p]),
    "attn_bwd": (C.c_int, [C.c_void_p] * 11 + [C.c_size_t, C.c_void_p]),
    "attn_bwd_preprocess": (C.c_int, [C.c_void_p] * 5 + [C.c_size_t, C.c_void_p]),
    "attn_bwd_dkdv": (C.c_int, [C.c_void_p] * 9 + [C.c_size_t, C.c_void_p]),
    "attn_bwd_dq": (C.c_int, [C.c_void_p] * 8 + [C.c_size_t, C.c_void_p]),
    "attn_bwd_atomic_dq": (C.c_int, [C.c_void_p] * 11 + [C.c_size_t, C.c_void_p]),
    "attn_bwd_noalloc": (C.c_int, [C.c_void_p] * 11),
    "attn_bwd_noalloc_max_workspace_bytes": (C.c_size_t, []),
    "attn_bwd_atomic_workspace_bytes": (C.c_size_t, [C.c_void_p]),
    "attn_fwd_partial": (C.c_int, [C.c_void_p] * 7),
    "attn_merge": (C.c_int, [C.c_void_p] * 5 + [C.c_int, C.c_void_p] + [C.c_int64] * 4 + [C.c_void_p]),
    "attn_desc_plan_bytes": (C.c_int, [C.POINTER(Shape), C.POINTER(MaskDesc), C.POINTER(C.c_size_t),
                                       C.POINTER(C.c_size_t), C.POINTER(C.c_uint64)]),
    "attn_fwd_desc": (C.c_int, [C.POINTER(Shape), C.POINTER(MaskDesc)] + [C.c_void_p] * 6
                      + [C.c_size_t, C.c_void_p]),
    "attn_bwd_desc": (C.c_int, [C.POINTER(Shape), C.POINTER(MaskDesc)] + [C.c_void_p] * 10
                      + [C.c_size_t, C.c_void_p, C.c_size_t, C.c_void_p]),
    "attn_desc_release": (None, [C.c_void_p]),
    "attn_desc_cache_clear": (None, []),
    "attn_plan_destroy": (None, [C.c_void_p]),
    "attn_last_error": (C.c_char_p, []),
    "attn_version": (C.c_char_p, []),
}

_lib = None


def lib():
    """The loaded libattn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
                " (there is no fallback path)")
        # torch ships its own HIP runtime under the same soname as the
        # system one that libattn.so names.  Loading torch first makes the
        # library bind to that copy; loaded the other way round, the process
        # would hold two HIP runtimes and the second to start sees no device.
        import torch  # noqa: F401
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class AttnError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


def check(status):
    if status != ATTN_OK:
        msg = lib().attn_last_error()
        raise AttnError(status, msg.decode() if msg else "")
