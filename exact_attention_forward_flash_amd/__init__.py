"""Exact attention forward on AMD Instinct MI355X (gfx950).

The computation lives in libwf.so (hand-written HIP kernels behind the C ABI declared in
include/wf.h); this package only loads it and marshals torch tensors to it.
"""
from ._lib import ChunkOrderError, CacheConfigError, WfError, load
from .api import (BlockKVCache, describe, flattened_sdpa, sdpa, sdpa_decode, sdpa_decode_workspace_size,
                  sdpa_rope, tune, varlen_mla_prefill, varlen_mla_prefill_noalloc,
                  varlen_mla_prefill_workspace_size)

__all__ = ["sdpa", "flattened_sdpa", "sdpa_decode", "sdpa_decode_workspace_size", "sdpa_rope", "varlen_mla_prefill",
           "varlen_mla_prefill_noalloc",
           "varlen_mla_prefill_workspace_size", "BlockKVCache", "WfError", "ChunkOrderError",
           "CacheConfigError", "load", "describe", "tune"]
