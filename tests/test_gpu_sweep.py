"""Seeded random sweep of wf_sdpa_fwd against the fp64 oracle across the dispatch matrix:
dtype, batch, GQA factor, ragged lengths (including 1 and 0 keys), head dim, causal or not,
bool / 16-bit / fp32 masks, with and without the lse, contiguous or [B, S, H, D]-strided
inputs. Which kernel runs (persistent, 64-query or 32-query, masked or not) follows from these,
so the sweep covers every routing decision of the dense entry point."""
import numpy as np
import pytest
import torch

import oracle
from exact_attention_forward_flash_amd import sdpa
from tests.parity import assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_CASES = 40


def _case(i):
    r = np.random.default_rng(1000 + i)
    dt = r.choice(["bf16", "fp16"])
    B = int(r.integers(1, 4))
    Hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 2, 3, 4, 8]))
    D = int(r.choice([64, 128]))
    Lq = int(r.choice([1, 2, 31, 64, 65, 200, 257, 640]))
    Lk = int(r.choice([0, 1, 17, 64, 100, 255, 512, 700])) if i % 5 else Lq
    while B * Hkv * G * Lq * max(Lk, 1) * D > 6e7:   # keep the oracle to a fraction of a second
        Lq = max(1, Lq // 2)
    causal = bool(r.random() < 0.4)
    mask = None if causal or r.random() < 0.4 else str(r.choice(["bool", "half", "f32"]))
    lse = bool(r.random() < 0.5)
    strided = bool(r.random() < 0.3)
    return dict(dt=dt, B=B, Hkv=Hkv, G=G, D=D, Lq=Lq, Lk=Lk, causal=causal, mask=mask, lse=lse,
                strided=strided, seed=i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    c = _case(i)
    g = torch.Generator().manual_seed(c["seed"])
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[c["dt"]]
    B, Hkv, G, D, Lq, Lk = c["B"], c["Hkv"], c["G"], c["D"], c["Lq"], c["Lk"]
    Hq = Hkv * G
    q = torch.randn(B, Hq, Lq, D, generator=g).to(dt)
    k = torch.randn(B, Hkv, Lk, D, generator=g).to(dt)
    v = torch.randn(B, Hkv, Lk, D, generator=g).to(dt)
    m = None
    if c["mask"] == "bool":
        m = torch.rand(B, 1, Lq, Lk, generator=g) < 0.85
    elif c["mask"] in ("half", "f32"):
        m = torch.randn(B, Hq, Lq, Lk, generator=g)
        m[torch.rand(m.shape, generator=g) < 0.1] = -float("inf")
        m = m.to(dt if c["mask"] == "half" else torch.float32)
    scale = 1.0 / np.sqrt(D)
    ref, ref_lse = oracle.sdpa(q, k, v, mask=m, is_causal=c["causal"], scale=np.float32(scale))

    def dev(t):  # optionally a [B, S, H, D]-strided view of the same values
        t = t.to(DEV)
        return t.transpose(1, 2).contiguous().transpose(1, 2) if c["strided"] else t
    args = (dev(q), dev(k), dev(v))
    md = None if m is None else m.to(DEV)
    if c["lse"]:
        out, lse = sdpa(*args, attn_mask=md, is_causal=c["causal"], scale=scale, return_lse=True)
        live = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(to64(lse)), live), str(c)
        if live.any():
            assert np.abs(to64(lse)[live] - ref_lse[live]).max() < 1e-3, str(c)
    else:
        out = sdpa(*args, attn_mask=md, is_causal=c["causal"], scale=scale)
    assert_close(out, ref, dt, str(c))
