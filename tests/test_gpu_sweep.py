"""Seeded random sweep of wf_sdpa_fwd against the fp64 oracle across the dispatch matrix:
dtype, batch, GQA factor, ragged lengths (including 1 and 0 keys), head dims (value width equal
to or different from the key width), causal or not,
bool / 16-bit / fp32 masks, with and without the lse, contiguous or [B, S, H, D]-strided
inputs. Which kernel runs (persistent, 64-query or 32-query, masked or not) follows from these,
so the sweep covers every routing decision of the dense entry point."""
import numpy as np
import pytest
import torch

import oracle
from exact_attention_forward_flash_amd import sdpa, sdpa_decode, sdpa_rope, varlen_mla_prefill
from tests.parity import assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
N_CASES = 300


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
    # value width: the key width, or (64 -> 96, 128 -> 64); drawn last, so the other fields of
    # every case are as they were before this draw existed
    Dv = D if r.random() < 0.7 else {64: 96, 128: 64}[D]
    return dict(dt=dt, B=B, Hkv=Hkv, G=G, D=D, Dv=Dv, Lq=Lq, Lk=Lk, causal=causal, mask=mask,
                lse=lse, strided=strided, seed=i)


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    c = _case(i)
    g = torch.Generator().manual_seed(c["seed"])
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[c["dt"]]
    B, Hkv, G, D, Lq, Lk = c["B"], c["Hkv"], c["G"], c["D"], c["Lq"], c["Lk"]
    Hq = Hkv * G
    q = torch.randn(B, Hq, Lq, D, generator=g).to(dt)
    k = torch.randn(B, Hkv, Lk, D, generator=g).to(dt)
    v = torch.randn(B, Hkv, Lk, c["Dv"], generator=g).to(dt)
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



# ---------------------------------------------------------------- decode --------------------

@pytest.mark.parametrize("i", range(80))
def test_random_decode(i):
    r = np.random.default_rng(5000 + i)
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[str(r.choice(["bf16", "fp16"]))]
    B, Hkv = int(r.integers(1, 4)), int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 2, 3, 4, 6, 8, 16]))
    D = int(r.choice([64, 128]))
    Lq = int(r.choice([1, 1, 2, 3, 5, 8]))
    Lk = int(r.choice([0, 1, 63, 64, 65, 500, 1999, 4096]))
    causal = bool(r.random() < 0.5)
    g = torch.Generator().manual_seed(i)
    q = torch.randn(B, Hkv * G, Lq, D, generator=g).to(dt)
    k = torch.randn(B, Hkv, Lk, D, generator=g).to(dt)
    v = torch.randn(B, Hkv, Lk, D, generator=g).to(dt)
    ref, ref_lse = oracle.sdpa(q, k, v, is_causal=causal, scale=np.float32(1 / np.sqrt(D)),
                               causal_align="bottom_right")
    out, lse = sdpa_decode(q.to(DEV), k.to(DEV), v.to(DEV), is_causal=causal,
                           scale=1 / np.sqrt(D), return_lse=True)
    what = f"decode case {i}: B={B} Hkv={Hkv} G={G} D={D} Lq={Lq} Lk={Lk} causal={causal}"
    assert_close(out, ref, dt, what)
    live = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(to64(lse)), live), what
    if live.any():
        assert np.abs(to64(lse)[live] - ref_lse[live]).max() < 1e-3, what


# ---------------------------------------------------------------- MLA prefill ---------------

@pytest.mark.parametrize("i", range(40))
def test_random_mla(i):
    r = np.random.default_rng(7000 + i)
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[str(r.choice(["bf16", "fp16"]))]
    batch = int(r.integers(1, 6))
    H = int(r.choice([1, 2, 4, 8, 16]))
    Hkv = int(r.choice([h for h in (1, 2, 4, 8, 16) if H % h == 0]))
    qlens = [int(x) for x in r.choice([0, 1, 2, 63, 64, 65, 255, 256, 257, 700], batch)]
    kvlens = [q if r.random() < 0.5 else int(r.choice([0, 1, 70, 300, 800])) for q in qlens]
    mt = int(r.integers(0, 2))
    padded = bool(r.random() < 0.3)
    dv = 128 if r.random() < 0.7 else 64   # drawn last: the other fields are as before
    g = torch.Generator().manual_seed(100 + i)
    nq, nk = sum(qlens), sum(kvlens)
    q, qr = torch.randn(nq, H, dv, generator=g).to(dt), torch.randn(nq, H, 64, generator=g).to(dt)
    k, kr = torch.randn(nk, Hkv, dv, generator=g).to(dt), torch.randn(nk, Hkv, 64, generator=g).to(dt)
    v = torch.randn(nk, Hkv, dv, generator=g).to(dt)
    ql, kl = torch.tensor(qlens, dtype=torch.int32), torch.tensor(kvlens, dtype=torch.int32)
    scale = 1 / np.sqrt(dv + 64.0)
    ref = oracle.varlen_mla_prefill(q, qr, k, kr, v, ql, kl, H, Hkv, np.float32(scale), mt)
    if padded:   # the same tokens, [batch, max_seq, Hkv, d] with zero padding rows
        ms = max(max(kvlens), 1)
        cu = np.concatenate([[0], np.cumsum(kvlens)])
        pads = []
        for t in (k, kr, v):
            p = torch.zeros((batch, ms) + tuple(t.shape[1:]), dtype=dt)
            for b in range(batch):
                p[b, :kvlens[b]] = t[cu[b]:cu[b + 1]]
            pads.append(p.to(DEV))
        kd, krd, vd = pads
    else:
        kd, krd, vd = k.to(DEV), kr.to(DEV), v.to(DEV)
    out = varlen_mla_prefill(q.to(DEV), qr.to(DEV), kd, krd, vd, ql.to(DEV), kl.to(DEV), H, Hkv,
                             scale, mt, kv_layout="padded" if padded else "packed")
    assert_close(out, ref, dt, f"MLA case {i}: q {qlens} kv {kvlens} H={H}/{Hkv} dv={dv} mask={mt} "
                               f"padded={padded}")


# ---------------------------------------------------------------- RoPE ----------------------

@pytest.mark.parametrize("i", range(40))
def test_random_rope(i):
    r = np.random.default_rng(9000 + i)
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[str(r.choice(["bf16", "fp16"]))]
    B, Hkv, G = int(r.integers(1, 3)), int(r.choice([1, 2, 4])), int(r.choice([1, 2, 4]))
    D = int(r.choice([64, 128]))
    rot = int(r.choice([d for d in (16, 32, 48, 64, 96, 128) if d <= D]))
    style = int(r.integers(0, 2))
    Lq, Lk = int(r.choice([1, 33, 128, 300])), int(r.choice([1, 64, 200, 400]))
    qp, kp = int(r.integers(0, 50)), int(r.integers(0, 50))
    causal = bool(r.random() < 0.4)
    g = torch.Generator().manual_seed(300 + i)
    q = torch.randn(B, Hkv * G, Lq, D, generator=g).to(dt)
    k = torch.randn(B, Hkv, Lk, D, generator=g).to(dt)
    v = torch.randn(B, Hkv, Lk, D, generator=g).to(dt)
    npos = max(qp + Lq, kp + Lk)
    theta = 10000.0 ** (-np.arange(rot // 2) * 2.0 / rot)
    ang = np.arange(npos)[:, None] * theta[None, :]
    c, s_ = torch.from_numpy(np.cos(ang)).float(), torch.from_numpy(np.sin(ang)).float()
    ref, _ = oracle.sdpa_rope(q, k, v, c.double(), s_.double(), rot, style, qp, kp,
                              is_causal=causal, scale=np.float32(1 / np.sqrt(D)))
    out = sdpa_rope(q.to(DEV), k.to(DEV), v.to(DEV), c.to(DEV), s_.to(DEV), rot, style, qp, kp,
                    is_causal=causal, scale=1 / np.sqrt(D))
    assert_close(out, ref, dt, f"rope case {i}: B={B} Hkv={Hkv} G={G} D={D} rot={rot} style={style} "
                               f"Lq={Lq} Lk={Lk} pos={qp},{kp} causal={causal}")


# ---------------------------------------------------------------- block KV cache attend -----

@pytest.mark.parametrize("i", range(16))
def test_random_cache_attend(i):
    from exact_attention_forward_flash_amd import BlockKVCache
    r = np.random.default_rng(11000 + i)
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[str(r.choice(["bf16", "fp16"]))]
    chunk = int(r.choice([16, 64, 128]))
    window = chunk * int(r.integers(1, 6))
    sink = chunk * int(r.integers(0, 3))
    Hkv, G, D = int(r.choice([1, 2, 4])), int(r.choice([1, 2, 4, 8])), int(r.choice([64, 128]))
    B = int(r.integers(1, 3))
    shape = (B, Hkv, sink + window, D)
    c = BlockKVCache(shape, shape, 2, chunk, window, sink, device=DEV, dtype=dt)
    o = oracle.BlockKVCacheOracle(shape, shape, 2, chunk, window, sink)
    g = torch.Generator().manual_seed(400 + i)
    steps = int(r.integers(1, 14))
    Lq = int(r.choice([1, 3, chunk]))
    # drawn after the case's other fields: causal attend, and the last chunk through the
    # fused update + attend
    causal = bool(r.random() < 0.4)
    fused = bool(r.random() < 0.5)
    for idx in range(steps):
        k = torch.randn(B, Hkv, chunk, D, generator=g).to(dt)
        v = torch.randn(B, Hkv, chunk, D, generator=g).to(dt)
        o.update(idx, k.float().numpy(), v.float().numpy())
        c.before_update(idx)
        if idx + 1 < steps or not fused:
            c.update(k.to(DEV), v.to(DEV))
            c.after_update(idx)
    q = torch.randn(B, Hkv * G, Lq, D, generator=g).to(dt)
    kv = torch.from_numpy(o.cached_k()).to(dt)
    vv = torch.from_numpy(o.cached_v()).to(dt)
    if fused:
        out = c.update_attend(k.to(DEV), v.to(DEV), q.to(DEV), is_causal=causal)
        c.after_update(steps - 1)
    else:
        out = c.attend(q.to(DEV), is_causal=causal)
    assert torch.equal(c.cached_k().cpu(), kv)
    ref, _ = oracle.sdpa(q, kv, vv, is_causal=causal, scale=np.float32(1 / np.sqrt(D)),
                         causal_align="bottom_right")
    assert_close(out, ref, dt, f"cache case {i}: sink={sink} window={window} chunk={chunk} "
                               f"B={B} Hkv={Hkv} G={G} D={D} steps={steps} Lq={Lq} "
                               f"causal={causal} fused={fused}")
