"""ctypes declarations of libpkv.so's C ABI (include/pkv.h) and a checked-call helper."""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIBRARY overrides the in-tree build (for comparing builds); there is no other fallback
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(_HERE, "libpkv.so")

PKV_F32, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2
PKV_NO_SPLIT_PHASE = 1 << 30
PKV_DECODE_STATIC_SCRATCH_BYTES = 64 << 20
ERRORS = {-1: "PKV_ERR_INVAL", -2: "PKV_ERR_OOM", -3: "PKV_ERR_LOCK", -4: "PKV_ERR_SLOT", -5: "PKV_ERR_NODE",
          -6: "PKV_ERR_HIP", -7: "PKV_ERR_UNSUPPORTED", -8: "PKV_ERR_INTERNAL"}


class PkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


_p = C.c_void_p
_i32, _i64, _f32, _sz = C.c_int32, C.c_int64, C.c_float, C.c_size_t
_pi32, _pi64 = C.POINTER(C.c_int32), C.POINTER(C.c_int64)

# name: (restype, argtypes)
SIGNATURES = {
    "pkv_last_error": (C.c_char_p, []),
    "pkv_version": (C.c_int, []),
    "pkv_source_hash": (C.c_char_p, []),
    "rt_create": (C.c_int, [_i64, _p, _i64, C.POINTER(_p)]),
    "rt_create_policy": (C.c_int, [_i64, _p, _i64, _i32, C.POINTER(_p)]),
    "rt_destroy": (None, [_p]),
    "rt_match_prefix": (_i64, [_p, _p, _i64, _p, _pi64]),
    "rt_insert": (_i64, [_p, _p, _p, _i64, _pi64]),
    "rt_insert_priority": (_i64, [_p, _p, _p, _i64, _i32, _pi64]),
    "rt_peek_prefix": (_i64, [_p, _p, _i64]),
    "rt_schedule_longest_prefix": (C.c_int, [_p, _i32, _p, _p, _p, _p]),
    "rt_dump_stats": (_i64, [_p, _p, _i64]),
    "rt_inc_lock_ref": (C.c_int, [_p, _i64]),
    "rt_dec_lock_ref": (C.c_int, [_p, _i64]),
    "rt_evict": (_i64, [_p, _i64]),
    "rt_alloc": (_i64, [_p, _i64, _p]),
    "rt_free": (C.c_int, [_p, _p, _i64]),
    "rt_eviction_log_size": (C.c_int, [_p, _pi64, _pi64]),
    "rt_set_eviction_log": (C.c_int, [_p, C.c_int32]),
    "rt_take_eviction_log": (C.c_int, [_p, _p, _p, _i64, _p, _i64]),
    "rt_evictable_size": (_i64, [_p]),
    "rt_protected_size": (_i64, [_p]),
    "rt_free_size": (_i64, [_p]),
    "rt_clock": (_i64, [_p]),
    "rt_copy_free_list": (_i64, [_p, _p, _i64]),
    "rt_dump": (_i64, [_p, _p, _i64]),
    "rt_prepare_extend": (_i64, [_p, _i32, _p, _p, _p, _i64, _p, _p, _p, _p, _i64, _p]),
    "rt_prepare_extend_prio": (_i64, [_p, _i32, _p, _p, _p, _p, _i64, _p, _p, _p, _p, _i64, _p]),
    "rt_release": (C.c_int, [_p, _p, _i32]),
    "rt_decode_step": (_i64, [_p, _i32, _p, _i64, _p, _p]),
    "rt_finish": (C.c_int, [_p, _i32, _p, _p, _p, _i64, _p, _p, _p]),
    "rt_chunk_launch": (_i32, [_p, _i32, _p, _p, _p, _i32, _i64, _p, _p]),
    "rt_serve_round": (_i32, [_p, _i32, _p, _p, _p, _p, _i32, _i32, _i32, _p]),
    "rt_chunk_prepare": (_i32, [_p, _i32, _p, _p, _p, _p, _i32, _i64, _p, _i64, _p, _p, _p, _p, _i64, _p, _p, _p]),
    "rt_chunk_finish": (_i32, [_p, _i32, _p, _p, _i32, _p, _p, _i32]),
    "pkv_kv_scatter": (C.c_int, [_p, _p, _i32, _p, _i64, _p, _p, _i32, _i64, _i32, _i32, _p, _p, _p]),
    "pkv_append_slots": (C.c_int, [_p, _i64, _p, _p, _i32, _p]),
    "pkv_extend_plan_size": (_i64, [_p, _i32, _i32]),
    "pkv_extend_plan": (_i64, [_p, _p, _i32, _i32, _p, _i64]),
    "pkv_extend_tile": (_i32, [_i32, _i32, _i32, _i32, _i32]),
    "pkv_extend_attention": (C.c_int, [_p, _p, _i32, _p, _p, _i32, _i64, _p, _p, _p, _i64, _p, _p, _p, _i32, _p,
                                       _i64, _i32, _i32, _i32, _f32, _p]),
    "pkv_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pkv_decode_chunk": (_i32, [_i32, _i32, _i32]),
    "pkv_decode_attention": (C.c_int, [_p, _p, _i32, _p, _p, _i32, _i64, _p, _p, _p, _i64, _p, _i32, _i32, _i32,
                                       _i32, _i32, _f32, _i32, _p, _sz, _p]),
    "pkv_decode_shared_plan": (_i64, [_p, _i64, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _i64]),
    "pkv_decode_shared_rows": (_i32, [_i32, _i32, _i32, _i32, _i32]),
    "pkv_decode_first_split": (_i32, [_p, _p, _i32, _i32]),
    "pkv_stream_read_words": (_i32, []),
    "pkv_stream_read": (C.c_int, [_p, _i64, _p, _p]),
    "pkv_decode_plan_items_cap": (_i64, [_p, _i32, _i64, _i32, _i32]),
    "pkv_decode_plan": (_i64, [_p, _i64, _p, _i32, _i32, _i32, _i32, _i32, _i32, _p, _p, _p, _i64, _pi32]),
    "pkv_decode_attention_shared": (C.c_int, [_p, _p, _i32, _p, _p, _i32, _i64, _p, _p, _p, _i64, _p, _i32, _i32,
                                              _i32, _i32, _i32, _f32, _i32, _p, _p, _p, _i64, _i32, _p, _sz, _p]),
    "pkv_decode_attention_static": (C.c_int, [_p, _p, _i32, _p, _p, _i32, _i64, _p, _p, _p, _i64, _p, _i32, _i32,
                                              _i32, _i32, _i32, _f32, _i32, _p, _p, _p, _i64, _i32, _p]),
}

_lib = None


def lib() -> C.CDLL:
    """The loaded libpkv.so; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m prefix_shared_kv_match_amd.build`")
        h = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        if LIB_PATH == os.path.join(_HERE, "libpkv.so"):
            from .build import source_hash
            built = h.pkv_source_hash().decode()
            if built != source_hash():
                raise ImportError(f"{LIB_PATH} was built from other sources (build {built}, sources "
                                  f"{source_hash()}): rebuild with `python -m prefix_shared_kv_match_amd.build`")
        _lib = h
    return _lib


def check(rc: int) -> int:
    if rc < 0:
        msg = lib().pkv_last_error()
        raise PkvError(int(rc), msg.decode() if msg else "")
    return rc
