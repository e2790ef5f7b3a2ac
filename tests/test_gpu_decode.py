"""GPU parity of wf_sdpa_decode (split-KV attention for few queries over a long K/V) against
the fp64 oracle, with the queries placed at the end of the keys when causal."""
import zlib

import numpy as np
import pytest
import torch

import oracle
from exact_attention_forward_flash_amd import WfError, sdpa, sdpa_decode, sdpa_decode_workspace_size, tune
from synth import random_sdpa_inputs
from tests.parity import assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

CASES = [  # dtype, B, Hq, Hkv, Lq, Lk, D, causal
    ("bf16", 2, 8, 2, 1, 4096, 128, False),     # GQA 4: one work group per KV head and split
    ("bf16", 1, 32, 8, 1, 32768 + 17, 128, False),
    ("fp16", 3, 6, 3, 4, 1000, 64, True),       # speculative: 4 new tokens, causal among them
    ("bf16", 2, 4, 4, 7, 5, 128, True),         # Lk < Lq: the first rows keep no key
    ("fp16", 1, 2, 1, 1, 1, 64, False),         # single key -> that V row
    ("bf16", 1, 16, 16, 33, 2048, 128, True),   # two query tiles
    ("fp16", 2, 12, 4, 2, 777, 64, False),      # GQA 3 (one head per work group)
    ("bf16", 1, 64, 8, 1, 130, 128, False),     # GQA 8, few tiles: one split
    # more than 4 heads per KV head: (head, position) rows packed into the tiles
    ("bf16", 1, 64, 1, 1, 8192, 128, False),    # multi-query: 64 heads on one KV head
    ("fp16", 2, 16, 2, 3, 2000, 64, True),      # GQA 8, 3 new tokens each, causal
    ("bf16", 1, 48, 1, 5, 700, 128, True),      # 240 packed rows: two row blocks
]


def _run(w, causal, lse=False):
    q, k, v = (w[n].to(DEV) for n in ("q", "k", "v"))
    return sdpa_decode(q, k, v, is_causal=causal, scale=w["scale"], return_lse=lse)


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_decode_shapes(case):
    dt, B, Hq, Hkv, Lq, Lk, D, causal = case
    w = random_sdpa_inputs(B, Hq, Hkv, Lq, Lk, D, D, dt, seed=zlib.crc32(str(case).encode()) % 1000)
    ref, ref_lse = oracle.sdpa(w["q"], w["k"], w["v"], is_causal=causal,
                               scale=np.float32(w["scale"]), causal_align="bottom_right")
    out, lse = _run(w, causal, lse=True)
    assert_close(out, ref, w["q"].dtype, str(case))
    live = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(to64(lse)), live)
    if live.any():
        assert np.abs(to64(lse)[live] - ref_lse[live]).max() < 1e-3
    assert_close(_run(w, causal), ref, w["q"].dtype, str(case) + " (no lse)")


def test_decode_matches_sdpa_without_mask():
    w = random_sdpa_inputs(2, 8, 4, 1, 5000, 128, 128, "bf16", seed=3)
    q, k, v = (w[n].to(DEV) for n in ("q", "k", "v"))
    a = sdpa_decode(q, k, v, scale=w["scale"])
    b = sdpa(q, k, v, scale=w["scale"])
    assert (a.float() - b.float()).abs().max().item() < 2e-2


def test_decode_empty_keys_and_deterministic():
    w = random_sdpa_inputs(1, 4, 4, 1, 0, 128, 128, "bf16", seed=4)
    out, lse = _run(w, False, lse=True)
    assert torch.count_nonzero(out).item() == 0 and torch.isinf(lse).all()
    w = random_sdpa_inputs(2, 8, 2, 3, 3000, 64, 64, "fp16", seed=5)
    assert torch.equal(_run(w, True), _run(w, True))


def test_decode_workspace_checks():
    w = random_sdpa_inputs(1, 8, 2, 1, 4096, 128, 128, "bf16", seed=6)
    q, k, v = (w[n].to(DEV) for n in ("q", "k", "v"))
    need = sdpa_decode_workspace_size(q, k, v)
    assert need > 256
    with pytest.raises(WfError):
        sdpa_decode(q, k, v, workspace=torch.empty(need - 1, dtype=torch.uint8, device=DEV))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    ref, _ = oracle.sdpa(w["q"], w["k"], w["v"], scale=np.float32(w["scale"]))
    assert_close(sdpa_decode(q, k, v, scale=w["scale"], workspace=ws), ref, torch.bfloat16, "ws")


def test_decode_bench_shape_sampled():
    # the decode bench shape (B=8, Hq=32, Hkv=8, one query, 16k keys) on two batch entries
    w = random_sdpa_inputs(8, 32, 8, 1, 16384, 128, 128, "bf16", seed=7)
    out = _run(w, False)
    for b in (0, 7):
        ref, _ = oracle.sdpa(w["q"][b:b + 1], w["k"][b:b + 1], w["v"][b:b + 1],
                             scale=np.float32(w["scale"]))
        assert_close(out[b:b + 1], ref, torch.bfloat16, f"batch {b}")


def test_packed_rows_match_unpacked():
    # the same call with (head, position) packing turned off agrees within rounding
    w = random_sdpa_inputs(2, 32, 2, 2, 3000, 128, 128, "bf16", seed=8)
    packed = _run(w, True)
    with tune(decode_pack=0):
        plain = _run(w, True)
    assert (packed.float() - plain.float()).abs().max().item() < 2e-2
