"""Seeded input recipes, one per workload.

Every draw is on the CPU with torch's generator in fp32, then rounded (RNE) to the
workload's dtype; consumers receive the rounded tensors. Draw orders are fixed per
workload so a seed names the exact inputs.

Workloads (sizes as used for measurement; every function also takes smaller sizes for
parity cases):
  page_example   fp32 q[2,8,32,64] k[2,8,48,64] v[2,8,48,96], global seed 7, draw order
                 q, k, v (the "Core 注意力" page's CPU/GPU example).
  causal_gqa     bf16 B=4, Hq=32, Hkv=8, L=4096, d=128, N(0,1); draw order q, k, v.
  varlen_mla     bf16, 16 sequences with lengths uniform in [128, 8192]; q_len = kv_len;
                 16 q heads = 16 kv heads; nope/V width 128, rope width 64; draw order
                 lengths, q, q_rope, k, k_rope, v.
  masked_bool    fp16 B=2, H=16, L=2048, d=64; keep-mask [2,1,L,L] Bernoulli(0.9) with
                 the diagonal forced true; draw order q, k, v, mask.
  masked_float   as masked_bool with an additive fp16 mask [2,1,L,L] N(0,1), 10% of
                 entries set to -inf, the diagonal kept finite; draw order q, k, v,
                 mask values, mask drop pattern.
  cache_stream   fp16 B=1, 24 heads, d=128, chunk 256, sink 256, window 3840, 64 chunks;
                 per chunk the draw order is q_c, k_c, v_c.
"""
from __future__ import annotations

import math

import torch

_DT = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}


def _gen(seed):
    return torch.Generator().manual_seed(int(seed))


def _randn(shape, dtype, g):
    return torch.randn(*shape, generator=g, dtype=torch.float32).to(_DT.get(dtype, dtype))


def page_example_fp32():
    """The page's example, drawn exactly as printed: global seed 7, then q, k, v."""
    torch.manual_seed(7)
    q = torch.randn(2, 8, 32, 64)
    k = torch.randn(2, 8, 48, 64)
    v = torch.randn(2, 8, 48, 96)
    return {"q": q, "k": k, "v": v, "scale": 1.0 / math.sqrt(64), "is_causal": False}


def random_sdpa_inputs(B, Hq, Hkv, Lq, Lk, Dqk, Dv, dtype="bf16", seed=0, scale=None):
    g = _gen(seed)
    q = _randn((B, Hq, Lq, Dqk), dtype, g)
    k = _randn((B, Hkv, Lk, Dqk), dtype, g)
    v = _randn((B, Hkv, Lk, Dv), dtype, g)
    return {"q": q, "k": k, "v": v,
            "scale": (1.0 / math.sqrt(Dqk)) if scale is None else scale}


def causal_gqa_prefill(B=4, Hq=32, Hkv=8, L=4096, D=128, dtype="bf16", seed=7):
    w = random_sdpa_inputs(B, Hq, Hkv, L, L, D, D, dtype, seed)
    w["is_causal"] = True
    return w


def varlen_mla_prefill_inputs(batch=16, heads=16, kv_heads=16, lo=128, hi=8192, dv=128,
                              drope=64, dtype="bf16", seed=7, lengths=None):
    g = _gen(seed)
    if lengths is None:
        lengths = torch.randint(lo, hi + 1, (batch,), generator=g, dtype=torch.int64)
    lengths = torch.as_tensor(lengths, dtype=torch.int32)
    n = int(lengths.sum())
    q = _randn((n, heads, dv), dtype, g)
    q_rope = _randn((n, heads, drope), dtype, g)
    k = _randn((n, kv_heads, dv), dtype, g)
    k_rope = _randn((n, kv_heads, drope), dtype, g)
    v = _randn((n, kv_heads, dv), dtype, g)
    return {"q": q, "q_rope": q_rope, "k": k, "k_rope": k_rope, "v": v,
            "q_seqlen": lengths.clone(), "kv_seqlen": lengths.clone(),
            "head_num": heads, "kv_head_num": kv_heads,
            "qk_scale": 1.0 / math.sqrt(dv + drope), "mask_type": 1}


def masked_sdpa_inputs(kind="bool", B=2, H=16, L=2048, D=64, dtype="fp16", seed=7,
                       keep_p=0.9, drop_p=0.1):
    g = _gen(seed)
    q = _randn((B, H, L, D), dtype, g)
    k = _randn((B, H, L, D), dtype, g)
    v = _randn((B, H, L, D), dtype, g)
    eye = torch.eye(L, dtype=torch.bool).expand(B, 1, L, L)
    if kind == "bool":
        mask = torch.rand(B, 1, L, L, generator=g) < keep_p
        mask = mask | eye
    elif kind == "float":
        vals = torch.randn(B, 1, L, L, generator=g)
        drop = (torch.rand(B, 1, L, L, generator=g) < drop_p) & ~eye
        mask = vals.masked_fill(drop, float("-inf")).to(_DT[dtype])
    else:
        raise ValueError(kind)
    return {"q": q, "k": k, "v": v, "mask": mask, "scale": 1.0 / math.sqrt(D),
            "is_causal": False}


def cache_stream_chunks(B=1, H=24, D=128, chunk=256, sink=256, window=3840, chunks=64,
                        dtype="fp16", seed=7):
    """Yields (chunk_idx, q_c, k_c, v_c) for the rolling-cache stream, each [B,H,chunk,D]."""
    g = _gen(seed)
    for c in range(chunks):
        q = _randn((B, H, chunk, D), dtype, g)
        k = _randn((B, H, chunk, D), dtype, g)
        v = _randn((B, H, chunk, D), dtype, g)
        yield c, q, k, v


WORKLOADS = {
    "page_example": dict(desc="page example SDPA, fp32, q[2,8,32,64] k[2,8,48,64] v[2,8,48,96]"),
    "causal_gqa": dict(desc="causal GQA prefill, bf16, B=4 Hq=32 Hkv=8 L=4096 d=128"),
    "varlen_mla": dict(desc="varlen packed MLA causal prefill, bf16, 16 seqs L~U[128,8192], "
                            "16 heads, d=128+64"),
    "masked_bool": dict(desc="masked SDPA, fp16, B=2 H=16 L=2048 d=64, bool keep-mask"),
    "masked_float": dict(desc="masked SDPA, fp16, B=2 H=16 L=2048 d=64, additive mask"),
    "cache_stream": dict(desc="rolling block KV cache, fp16, 24 heads d=128, chunk 256, "
                              "sink 256 + window 3840, 64 chunks"),
    "rope_gqa": dict(desc="causal GQA prefill with rotate-half RoPE over all 128 dims (cos/sin "
                          "tables of base 10000), bf16, B=4 Hq=32 Hkv=8 L=4096 (beyond the five "
                          "configurations)"),
    "decode": dict(desc="GQA decode, bf16, B=8 Hq=32 Hkv=8, 1 query over 16384 keys, d=128 "
                        "(split-KV; beyond the five configurations)"),
}
