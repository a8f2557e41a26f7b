"""ctypes declarations of libpagedkv.so (the C ABI in include/pagedkv.h).

Loading fails loudly: there is no fallback path when the library is missing.
"""

import ctypes
import os

# PKV_LIBRARY names another build of the library to load instead of the
# in-tree one (the host-sanitizer build of the CPU tests).
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                          "libpagedkv.so")

# pkv_status
PKV_OK = 0
PKV_ERR_NULL = -1
PKV_ERR_SHAPE = -2
PKV_ERR_DTYPE = -3
PKV_ERR_UNSUPPORTED = -4
PKV_ERR_WORKSPACE = -5
PKV_ERR_HIP = -6

# pkv_decode_plan_make flags
PKV_PLAN_BLOCKS_NOT_SHARED = 1
PKV_PLAN_BLOCKS_SHARED = 2

PKV_STATIC_SCRATCH_BYTES = 64 << 20

# pkv_dtype
PKV_F32 = 0
PKV_BF16 = 1
PKV_FP8_E4M3 = 2
PKV_INT4 = 3


class PkvCache(ctypes.Structure):
    _fields_ = [
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("block_stride", ctypes.c_int64),
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


class PkvDecodePlan(ctypes.Structure):
    _fields_ = [
        ("split_blocks", ctypes.c_int32),
        ("max_splits", ctypes.c_int32),
        ("heads_per_item", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
        ("scheme", ctypes.c_int32),
        ("num_workers", ctypes.c_int32),
        ("lead_workers", ctypes.c_int32),
        ("trail_share_pct", ctypes.c_int32),
    ]


_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_int = ctypes.c_int

# name -> (restype, argtypes); the names match include/pagedkv.h one for one.
SIGNATURES = {
    "pkv_status_string": (ctypes.c_char_p, [_int]),
    "pkv_kv_bytes_per_token": (_i64, [_i32, _i32, _i32, _i32]),
    "pkv_num_blocks_for_budget": (_i64, [_i64, ctypes.c_double, _i64, _i32, _i32, _i32, _i32, _i32]),
    "pkv_slot_mapping": (_int, [_vp, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "pkv_cache_write": (_int, [_vp, _vp, _i32, _i64, _i64, _vp, _i32, ctypes.POINTER(PkvCache), _vp]),
    "pkv_slot_mapping_cache_write": (_int, [_vp, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _i64,
                                            _i64, ctypes.POINTER(PkvCache), _vp]),
    "pkv_decode_plan_make": (_int, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                    ctypes.POINTER(PkvDecodePlan)]),
    "pkv_decode_plan_resize": (_int, [_i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(PkvDecodePlan)]),
    "pkv_paged_attention_decode": (_int, [_vp, _vp, _i32, _i32, _i32, ctypes.POINTER(PkvCache), _vp, _i32,
                                          _vp, _i32, _f32, _i32, _vp, _sz, _vp]),
    "pkv_paged_attention_decode_static": (_int, [_vp, _vp, _i32, _i32, _i32, ctypes.POINTER(PkvCache), _vp,
                                                 _i32, _vp, _i32, _f32, _i32, _vp]),
    "pkv_paged_attention_decode_partials": (_int, [_vp, _vp, _i32, _i32, _i32, ctypes.POINTER(PkvCache), _vp,
                                                   _i32, _vp, _i32, _f32, _i32, ctypes.POINTER(PkvDecodePlan),
                                                   _vp, _sz, _vp]),
    "pkv_paged_attention_decode_step": (_int, [_vp, _vp, _i32, _vp, _vp, _i32, _i32, ctypes.POINTER(PkvCache), _vp,
                                               _i32, _vp, _i32, _f32, _i32, ctypes.POINTER(PkvDecodePlan), _vp,
                                               _sz, _vp, _vp]),
    "pkv_paged_attention_decode_combine": (_int, [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _i32,
                                                  ctypes.POINTER(PkvDecodePlan), _vp, _sz, _vp]),
    "pkv_chunked_workspace_size": (_int, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                          ctypes.POINTER(_sz)]),
    "pkv_paged_attention_chunked": (_int, [_vp, _vp, _i32, _i32, _i32, _vp, _vp, _i32, _i32,
                                           ctypes.POINTER(PkvCache), _vp, _i32, _i32, _f32, _i32, _i32,
                                           _i32, _vp, _sz, _vp]),
    "pkv_copy_blocks": (_int, [ctypes.POINTER(PkvCache), _vp, _vp, _i32, _vp, _vp]),
    "pkv_fp8_e4m3_quantize": (_int, [_vp, _i32, _i64, _f32, _vp, _vp]),
    "pkv_fp8_e4m3_dequantize": (_int, [_vp, _i64, _f32, _i32, _vp, _vp]),
    "pkv_int4_quantize": (_int, [_vp, _i32, _i64, _f32, _vp, _vp]),
    "pkv_int4_dequantize": (_int, [_vp, _i64, _f32, _i32, _vp, _vp]),
}

_lib = None


def load():
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libpagedkv.so is not built (expected at %s); run "
            "`python -c 'import __graft_entry__ as g; g.build()'` first" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class PkvError(RuntimeError):
    def __init__(self, fn, status):
        msg = load().pkv_status_string(status)
        super().__init__("%s failed: %s (%d)" % (fn, msg.decode() if msg else "?", status))
        self.status = status


def check(fn, status):
    if status != PKV_OK:
        raise PkvError(fn, status)
