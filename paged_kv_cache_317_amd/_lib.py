"""ctypes loader for libpkv.so and its C declarations (argument marshalling only)."""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("PKV_LIB", os.path.join(HERE, "libpkv.so"))

PKV_F32, PKV_BF16 = 0, 1

STATUS_NAMES = {
    0: "PKV_OK", 1: "PKV_ERR_NULL", 2: "PKV_ERR_SHAPE", 3: "PKV_ERR_DTYPE",
    4: "PKV_ERR_UNSUPPORTED", 5: "PKV_ERR_WORKSPACE", 6: "PKV_ERR_HIP", 7: "PKV_ERR_ALIGN",
    8: "PKV_ERR_NO_BLOCKS", 9: "PKV_ERR_KEY",
}


class CacheDesc(ctypes.Structure):
    """Mirror of ``pkv_cache_desc``."""
    _fields_ = [
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class BmStats(ctypes.Structure):
    """Mirror of ``pkv_bm_stats``."""
    _fields_ = [(name, ctypes.c_int64) for name in (
        "allocated_blocks", "allocated_slots", "used_slots", "free_blocks", "sequences",
        "logical_tokens", "copies", "preemptions", "cached_blocks", "reused_blocks",
        "host_blocks_used", "swapped_sequences", "swap_outs", "unused_slots")] + [
        ("waste_fraction", ctypes.c_double)]


class PkvError(RuntimeError):
    """A non-OK ``pkv_status``, with the library's message."""

    def __init__(self, status, message):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


_vp, _i32, _i64, _f32, _sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                              ctypes.c_float, ctypes.c_size_t)
_desc = ctypes.POINTER(CacheDesc)
_p = ctypes.POINTER

SIGNATURES = {
    "pkv_paged_kv_write": (_i32, [_vp, _vp, _vp, _i64, _vp, _vp, _desc, _vp]),
    "pkv_paged_attn_decode": (_i32, [_vp, _vp, _vp, _desc, _vp, _i32, _vp, _i32, _i32, _i32,
                                     _f32, _vp, _i32, _vp, _sz, _vp]),
    "pkv_paged_attn_decode_noalloc": (_i32, [_vp, _vp, _vp, _desc, _vp, _i32, _vp, _i32, _i32,
                                             _i32, _f32, _vp, _i32, _vp]),
    "pkv_decode_noalloc_max_workspace": (_sz, []),
    "pkv_paged_attn_extend": (_i32, [_vp, _vp, _vp, _desc, _vp, _i32, _vp, _vp, _i32, _i32,
                                     _i32, _i32, _i32, _f32, _vp, _i32, _vp, _sz, _vp]),
    "pkv_extend_partition_tokens": (_i32, [_desc, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_extend_workspace_size": (_sz, [_desc, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_decode_partition_tokens": (_i32, [_desc, _i32, _i32, _i32, _i32]),
    "pkv_decode_workspace_size": (_sz, [_desc, _i32, _i32, _i32, _i32]),
    "pkv_decode_runs": (_i32, [_desc, _i32, _i32, _i32, _i32]),
    "pkv_paged_block_copy": (_i32, [_vp, _i32, _vp, _vp, _desc, _vp]),
    "pkv_paged_block_move": (_i32, [_vp, _i32, _vp, _vp, _desc, _vp, _vp, _desc, _vp]),
    "pkv_bm_create": (_i32, [_i32, _i32, _vp, _p(_vp)]),
    "pkv_bm_destroy": (None, [_vp]),
    "pkv_bm_add": (_i32, [_vp, _i64]),
    "pkv_bm_fork": (_i32, [_vp, _i64, _i64]),
    "pkv_bm_append": (_i32, [_vp, _i64, _i32, _vp, _vp, _i32, _p(_i32)]),
    "pkv_bm_blocks_needed": (_i32, [_vp, _i64, _i32, _p(_i32)]),
    "pkv_bm_add_cached": (_i32, [_vp, _i64, _vp, _i32, _p(_i32)]),
    "pkv_bm_append_tokens": (_i32, [_vp, _i64, _vp, _i32, _vp, _vp, _i32, _p(_i32)]),
    "pkv_bm_free": (_i32, [_vp, _i64]),
    "pkv_bm_set_swap_space": (_i32, [_vp, _i32]),
    "pkv_bm_swap_out": (_i32, [_vp, _i64, _vp, _i32, _p(_i32)]),
    "pkv_bm_swap_in": (_i32, [_vp, _i64, _vp, _i32, _p(_i32)]),
    "pkv_bm_preempt": (_i32, [_vp, _i64]),
    "pkv_bm_length": (_i32, [_vp, _i64, _p(_i32)]),
    "pkv_bm_table": (_i32, [_vp, _vp, _i32, _i32, _vp]),
    "pkv_bm_get_stats": (_i32, [_vp, _p(BmStats)]),
    "pkv_capacity": (_i32, [_i64, _i32, _vp, _i32, _i32, _p(_i32), _p(_i32)]),
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (ctypes.c_char_p, []),
}

_LIB = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"libpkv.so not found at {LIB_PATH}; build it with "
                "`python -m paged_kv_cache_317_amd.build` (there is no fallback path)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def check(status):
    if status != 0:
        raise PkvError(status, lib().pkv_last_error().decode())
    return status


def last_error():
    return lib().pkv_last_error().decode()
