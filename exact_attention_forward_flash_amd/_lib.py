"""ctypes loader for libwf.so and its C ABI (include/wf.h). No fallback: if the library is
missing, loading raises."""
from __future__ import annotations

import ctypes
import os

# WF_LIBRARY names another build of the same sources (the host-sanitizer build, for one)
LIB_PATH = os.environ.get("WF_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                        "libwf.so")

WF_F32, WF_F16, WF_BF16, WF_BOOL, WF_I32 = 0, 1, 2, 3, 4

STATUS = {0: "WF_OK", 1: "WF_ERR_NULL", 2: "WF_ERR_SHAPE", 3: "WF_ERR_DTYPE",
          4: "WF_ERR_LAYOUT", 5: "WF_ERR_UNSUPPORTED", 6: "WF_ERR_CHUNK_ORDER",
          7: "WF_ERR_CACHE_CONFIG", 8: "WF_ERR_WORKSPACE", 9: "WF_ERR_HIP"}
ERR_SHAPE = 2
ERR_CHUNK_ORDER = 6
ERR_CACHE_CONFIG = 7


class WfTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("ndim", ctypes.c_int32),
                ("shape", ctypes.c_int64 * 4), ("stride", ctypes.c_int64 * 4)]


class WfBlockKvState(ctypes.Structure):
    _fields_ = [("cache_len", ctypes.c_int64), ("sink", ctypes.c_int64),
                ("window", ctypes.c_int64), ("chunk", ctypes.c_int64),
                ("last_chunk", ctypes.c_int64)]


class WfRope(ctypes.Structure):
    _fields_ = [("cos", ctypes.c_void_p), ("sin", ctypes.c_void_p), ("max_pos", ctypes.c_int64),
                ("rot_dim", ctypes.c_int), ("style", ctypes.c_int), ("q_pos0", ctypes.c_int64),
                ("k_pos0", ctypes.c_int64)]


_T = ctypes.POINTER(WfTensor)
_S = ctypes.POINTER(WfBlockKvState)
_vp, _i32, _i64, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

# name -> (restype, argtypes); the full exported surface of include/wf.h
SIGNATURES = {
    "wf_sdpa_fwd": (_i32, [_T, _T, _T, _T, _i32, _f, _f, _T, ctypes.POINTER(ctypes.c_float), _vp]),
    "wf_sdpa_rope_workspace_size": (_sz, [_T, _T]),
    "wf_sdpa_rope_fwd": (_i32, [_T, _T, _T, _T, _i32, _f, ctypes.POINTER(WfRope), _T,
                                ctypes.POINTER(ctypes.c_float), _vp, _sz, _vp]),
    "wf_sdpa_decode_workspace_size": (_sz, [_T, _T, _T, _i32]),
    "wf_sdpa_decode": (_i32, [_T, _T, _T, _i32, _f, _T, ctypes.POINTER(ctypes.c_float), _vp, _sz,
                              _vp]),
    "wf_varlen_mla_prefill_workspace_size": (_sz, [_i32, _i64, _i32]),
    "wf_varlen_mla_prefill": (_i32, [_T, _T, _T, _T, _T, _vp, _vp, _i32, _i32, _i32, _f, _i32,
                                     _T, _vp, _sz, _vp]),
    "wf_varlen_mla_prefill_noalloc": (_i32, [_T, _T, _T, _T, _T, _vp, _vp, _i32, _i32, _i32, _f,
                                             _i32, _T, _vp]),
    "wf_block_kv_init": (_i32, [_S, _i64, _i64, _i64, _i64]),
    "wf_block_kv_cache_update": (_i32, [_S, _i64, _T, _T, _T, _T, _vp]),
    "wf_block_kv_visible": (_i32, [_S, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "wf_block_kv_gather": (_i32, [_S, _T, _T, _vp]),
    "wf_block_kv_attend_workspace_size": (_sz, [_S, _i32, _i32, _i32, _i32]),
    "wf_block_kv_attend": (_i32, [_S, _T, _T, _T, _i32, _f, _T, _vp, _sz, _vp]),
    "wf_block_kv_update_attend": (_i32, [_S, _i64, _T, _T, _T, _T, _T, _i32, _f, _T, _vp, _sz, _vp]),
    "wf_status_string": (ctypes.c_char_p, [_i32]),
    "wf_last_error": (ctypes.c_char_p, []),
    "wf_tune_set": (_i32, [ctypes.c_char_p, _i32]),
    "wf_tune_get": (_i32, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_int)]),
    "wf_build_id": (ctypes.c_char_p, []),
}

_lib = None


def check_build_id(lib_id, expected=None):
    """Raises unless the library was built from the sources in this tree."""
    from .build import source_hash
    expected = expected or source_hash()
    if lib_id != expected:
        raise RuntimeError(f"{LIB_PATH} was built from other sources (build id {lib_id[:12]}, the "
                           f"sources hash to {expected[:12]}); rebuild it with "
                           "`python -m exact_attention_forward_flash_amd.build`")


def load():
    """Loads libwf.so once; raises if it has not been built or is older than the sources."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m exact_attention_forward_flash_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        if not hasattr(lib, "wf_build_id"):
            raise RuntimeError(f"{LIB_PATH} has no build id; rebuild it")
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        check_build_id(lib.wf_build_id().decode())
        _lib = lib
    return _lib


class WfError(RuntimeError):
    def __init__(self, status, detail):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


class ChunkOrderError(WfError, ValueError):
    pass


class CacheConfigError(WfError, ValueError):
    pass


def check(rc):
    if rc != 0:
        detail = load().wf_last_error().decode()
        cls = {ERR_CHUNK_ORDER: ChunkOrderError, ERR_CACHE_CONFIG: CacheConfigError}.get(rc, WfError)
        raise cls(rc, detail)
