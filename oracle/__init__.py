"""CPU fp64 oracle for exact attention forward.

TEST INFRASTRUCTURE ONLY. This package is the slow, obviously-correct definition the
GPU library is checked against. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it; the product path (the HIP library and its Python
binding) never does, and shares no code with it.

Sources (the pages this project implements):
  * WorldFoundry API reference, page "Core 注意力" (core attention): sections
    "选择最窄的入口" (choose the narrowest entry point: PyTorch SDPA contract, GQA
    expansion, exact matmul fallback), the CPU/GPU example, the mask sentence after it
    (bool = kept scores, float = added to scores) and "Block KV cache 的调用顺序"
    (block KV cache call order, sink/window rule).
  * Huawei Ascend CANN ATB page "MLA Prefill": the definition of
    AtbMLAPreFillGetWorkspaceSize and its parameter table (Q/QRope/K/kRope/V layouts,
    qSeqLen/kvSeqLen, headNum, kvHeadNum, qkScale, maskType).
  * "Core 注意力", the responsibility list at its top (the core applies RoPE): oracle.rotary.

Parity status of every function is stated in its module header.
"""
from .attention import sdpa, varlen_mla_prefill, cu_seqlens
from .block_kv_cache import BlockKVCacheOracle, CacheOrderError, CacheConfigError
from .rotary import rope, sdpa_rope

__all__ = ["sdpa", "varlen_mla_prefill", "cu_seqlens", "BlockKVCacheOracle",
           "CacheOrderError", "CacheConfigError", "rope", "sdpa_rope"]
