"""ctypes loader for libpa.so and the declarations of its C ABI (include/pa.h).

The library is built in-tree by ``paged_kv_cache_454_amd.build``; loading
fails loudly when it is missing. There is no fallback of any kind.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpa.so")

PA_OK, PA_EINVAL, PA_EUNSUPPORTED, PA_ENOMEM, PA_EHIP, PA_ENOTFOUND = range(6)
PA_F32, PA_BF16, PA_FP8_E4M3 = 0, 1, 2
STATUS_NAMES = {0: "PA_OK", 1: "PA_EINVAL", 2: "PA_EUNSUPPORTED", 3: "PA_ENOMEM",
                4: "PA_EHIP", 5: "PA_ENOTFOUND"}

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_u32 = ctypes.c_uint32
_f32 = ctypes.c_float
_st = ctypes.c_int

# name -> (restype, argtypes); mirrors include/pa.h
SIGNATURES = {
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_version": (ctypes.c_char_p, []),
    "pa_reshape_and_cache": (_st, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _st, _p]),
    "pa_copy_blocks": (_st, [_p, _p, _p, _i32, _i32, _i32, _i32, _i32, _st, _p]),
    "pa_reshape_and_cache_fp8": (_st, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _st,
                                       _f32, _f32, _p]),
    "pa_decode_fp8": (_st, [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                            _f32, _f32, _f32, _st, _p]),
    "pa_decode_partitioned_fp8": (_st, [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32,
                                        _i32, _i32, _i32, _f32, _f32, _f32, _i32, _i32, _p]),
    "pa_decode_partitioned_fp8_planned": (_st, [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32,
                                                _i32, _i32, _i32, _i32, _i32, _f32, _f32, _f32,
                                                _i32, _i32, _p, _u32, _p]),
    "pa_decode": (_st, [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
                        _st, _st, _p]),
    "pa_partition_workspace_bytes": (ctypes.c_size_t, [_i32, _i32, _i32, _i32]),
    "pa_decode_partitioned": (_st, [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32,
                                    _i32, _i32, _f32, _i32, _i32, _st, _p]),
    "pa_reduce": (_st, [_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _st, _p]),
    "pa_decode_step": (_st, [_p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32,
                             _i32, _i32, _i32, _f32, _i32, _i32, _st, _st, _p, _u32, _p]),
    "pa_decode_plan_bytes": (ctypes.c_size_t, []),
    "pa_decode_partitioned_planned": (_st, [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32,
                                            _i32, _i32, _i32, _i32, _f32, _i32, _i32, _st, _p,
                                            _u32, _p]),
    "pa_decode_scratch_bytes": (ctypes.c_size_t, []),
    "pa_decode_balanced": (_st, [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                 _i32, _f32, _st, _st, _p, ctypes.c_size_t, _p]),
    "pa_decode_balanced_static": (_st, [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32,
                                        _i32, _i32, _f32, _st, _st, _p]),
    "pa_decode_partitioned_balanced": (_st, [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32,
                                             _i32, _i32, _i32, _i32, _f32, _i32, _i32, _st, _p,
                                             ctypes.c_size_t, _p]),
    "pa_prefill_chunk": (_st, [_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                               _i32, _i32, _i32, _f32, _st, _st, _p]),
    "pa_alloc_create": (_st, [_i32, _i32, _p, ctypes.POINTER(_p)]),
    "pa_alloc_destroy": (None, [_p]),
    "pa_alloc_append": (_st, [_p, _i64, _i32, _p]),
    "pa_alloc_free": (_st, [_p, _i64]),
    "pa_alloc_num_free": (_i32, [_p]),
    "pa_alloc_seq_len": (_i32, [_p, _i64]),
    "pa_alloc_block_table": (_st, [_p, _p, _i32, _i32, _p, _p]),
    "pa_alloc_fork": (_st, [_p, _i64, _i64]),
    "pa_alloc_take_copies": (_i32, [_p, _p, _i32]),
    "pa_alloc_block_refs": (_i32, [_p, _i32]),
    "pa_alloc_step": (_st, [_p, _p, _p, _i32, _p, _i32, _p, _p]),
    "pa_swap_blocks": (_st, [_p, _p, _i32, _p, _p, _i32, _p, _i32, _i32, _i32, _i32, _st, _p]),
    "pa_alloc_set_host_pool": (_st, [_p, _i32, _p]),
    "pa_alloc_num_free_host": (_i32, [_p]),
    "pa_alloc_is_swapped": (_i32, [_p, _i64]),
    "pa_alloc_swap_out": (_st, [_p, _i64, _i32, _p, _p]),
    "pa_alloc_swap_in": (_st, [_p, _i64, _i32, _p, _p]),
    "pa_read_probe_sink_words": (_i64, []),
    "pa_read_probe": (_st, [_p, _i64, _p, _i32, _p, _i64, _p]),
}

_LIB = None


class PAError(RuntimeError):
    """A non-OK status from libpa; ``status`` holds the code."""

    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def lib():
    """The loaded library (loaded once). Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_454_amd.build` "
                "(or __graft_entry__.build()); there is no fallback path")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def check(status):
    if status != PA_OK:
        raise PAError(status, lib().pa_last_error().decode())
