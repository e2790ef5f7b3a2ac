"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and casts them; it holds none of the attention
arithmetic, so both the GPU path's tests and the CPU oracle can consume its output
without sharing any computation.
"""
from .workloads import (page_example_fp32, causal_gqa_prefill, varlen_mla_prefill_inputs,
                        masked_sdpa_inputs, cache_stream_chunks, random_sdpa_inputs,
                        WORKLOADS)

__all__ = ["page_example_fp32", "causal_gqa_prefill", "varlen_mla_prefill_inputs",
           "masked_sdpa_inputs", "cache_stream_chunks", "random_sdpa_inputs", "WORKLOADS"]
