"""Pins for the CPU fp64 oracle, against facts other than the oracle itself.

* library routine: torch's CPU fp64 scaled_dot_product_attention (the PyTorch SDPA
  contract the "Core 注意力" page adopts, with its GQA expansion and masks);
* closed forms: a single key returns its V row; all-zero keys return the mean of V with
  lse = log(Lk);
* invariants: kept-all bool mask = no mask, zero float mask = no mask, bool M = float
  where(M, 0, -inf), causal = additive triangle, per-row constant shift, scale folding,
  key permutation, GQA = explicitly repeated KV heads, bottom-right causal = suffix of the
  square top-left case;
* the pages' worked examples (tests/golden): the SDPA example's shape and the block KV
  cache example's visible counts and values.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import (BlockKVCacheOracle, CacheConfigError, CacheOrderError, cu_seqlens, sdpa,
                    varlen_mla_prefill)
from synth import page_example_fp32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TIGHT = dict(rtol=1e-11, atol=1e-12)


def _t(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(*shape, generator=g, dtype=torch.float64)


def _torch_sdpa(q, k, v, **kw):
    return F.scaled_dot_product_attention(q, k, v, enable_gqa=True, **kw).numpy()


CASES = [  # B, Hq, Hkv, Lq, Lk, Dqk, Dv
    (1, 1, 1, 1, 1, 8, 8),
    (2, 4, 4, 5, 7, 16, 24),
    (2, 8, 2, 33, 17, 32, 16),
    (1, 6, 3, 40, 40, 64, 64),
    (3, 2, 1, 9, 50, 8, 3),
]


@pytest.mark.parametrize("case", CASES)
def test_sdpa_matches_torch_no_mask(case):
    B, Hq, Hkv, Lq, Lk, Dqk, Dv = case
    q, k, v = _t((B, Hq, Lq, Dqk), 1), _t((B, Hkv, Lk, Dqk), 2), _t((B, Hkv, Lk, Dv), 3)
    out, _ = sdpa(q, k, v)
    np.testing.assert_allclose(out, _torch_sdpa(q, k, v), **TIGHT)
    out, _ = sdpa(q, k, v, scale=0.37)
    np.testing.assert_allclose(out, _torch_sdpa(q, k, v, scale=0.37), **TIGHT)


@pytest.mark.parametrize("case", CASES)
def test_sdpa_matches_torch_causal_top_left(case):
    B, Hq, Hkv, Lq, Lk, Dqk, Dv = case
    q, k, v = _t((B, Hq, Lq, Dqk), 4), _t((B, Hkv, Lk, Dqk), 5), _t((B, Hkv, Lk, Dv), 6)
    out, _ = sdpa(q, k, v, is_causal=True)
    np.testing.assert_allclose(out, _torch_sdpa(q, k, v, is_causal=True), **TIGHT)


@pytest.mark.parametrize("case", CASES[1:])
def test_sdpa_matches_torch_bool_mask(case):
    B, Hq, Hkv, Lq, Lk, Dqk, Dv = case
    q, k, v = _t((B, Hq, Lq, Dqk), 7), _t((B, Hkv, Lk, Dqk), 8), _t((B, Hkv, Lk, Dv), 9)
    g = torch.Generator().manual_seed(10)
    m = torch.rand(B, 1, Lq, Lk, generator=g) < 0.7
    m[..., 0] = True  # torch's math path gives NaN on fully masked rows; keep one key
    out, _ = sdpa(q, k, v, mask=m)
    np.testing.assert_allclose(out, _torch_sdpa(q, k, v, attn_mask=m), **TIGHT)
    mh = torch.rand(B, Hq, Lq, Lk, generator=g) < 0.5  # per-head mask
    mh[..., -1] = True
    out, _ = sdpa(q, k, v, mask=mh)
    np.testing.assert_allclose(out, _torch_sdpa(q, k, v, attn_mask=mh), **TIGHT)


@pytest.mark.parametrize("case", CASES[1:])
def test_sdpa_matches_torch_float_mask(case):
    B, Hq, Hkv, Lq, Lk, Dqk, Dv = case
    q, k, v = _t((B, Hq, Lq, Dqk), 11), _t((B, Hkv, Lk, Dqk), 12), _t((B, Hkv, Lk, Dv), 13)
    fm = _t((1, Hq, Lq, Lk), 14)
    g = torch.Generator().manual_seed(15)
    fm[torch.rand(fm.shape, generator=g) < 0.2] = float("-inf")
    fm[..., 0] = 0.5
    out, _ = sdpa(q, k, v, mask=fm, scale=0.21)
    np.testing.assert_allclose(out, _torch_sdpa(q, k, v, attn_mask=fm, scale=0.21), **TIGHT)


def test_single_key_returns_its_value_row():
    q, k, v = _t((2, 4, 6, 16), 20), _t((2, 2, 1, 16), 21), _t((2, 2, 1, 5), 22)
    out, lse = sdpa(q, k, v, scale=0.3)
    for h in range(4):
        np.testing.assert_array_equal(out[:, h], np.broadcast_to(v[:, h // 2].numpy(), (2, 6, 5)))
    s = 0.3 * np.einsum("bhid,bhjd->bhij", q.numpy(), np.repeat(k.numpy(), 2, axis=1))[..., 0]
    np.testing.assert_allclose(lse, s, **TIGHT)


def test_uniform_scores_return_mean_of_values():
    q, v = _t((1, 3, 7, 8), 23), _t((1, 3, 11, 4), 24)
    k = torch.zeros(1, 3, 11, 8, dtype=torch.float64)
    out, lse = sdpa(q, k, v)
    np.testing.assert_allclose(out, np.broadcast_to(v.numpy().mean(axis=2, keepdims=True), out.shape), **TIGHT)
    np.testing.assert_allclose(lse, np.full(lse.shape, math.log(11)), **TIGHT)
    # under a bool mask the mean is over the kept keys only
    m = torch.zeros(1, 1, 7, 11, dtype=torch.bool)
    m[..., 2:5] = True
    out, lse = sdpa(q, k, v, mask=m)
    np.testing.assert_allclose(out, np.broadcast_to(v.numpy()[:, :, 2:5].mean(axis=2, keepdims=True), out.shape), **TIGHT)
    np.testing.assert_allclose(lse, np.full(lse.shape, math.log(3)), **TIGHT)


def test_mask_invariants():
    q, k, v = _t((2, 4, 13, 16), 30), _t((2, 2, 19, 16), 31), _t((2, 2, 19, 8), 32)
    ref, ref_lse = sdpa(q, k, v)
    out, _ = sdpa(q, k, v, mask=torch.ones(1, 1, 13, 19, dtype=torch.bool))
    np.testing.assert_array_equal(out, ref)
    out, _ = sdpa(q, k, v, mask=torch.zeros(2, 4, 13, 19, dtype=torch.float64))
    np.testing.assert_array_equal(out, ref)
    g = torch.Generator().manual_seed(33)
    bm = torch.rand(2, 1, 13, 19, generator=g) < 0.6
    bm[..., 3] = True
    fm = torch.where(bm, 0.0, float("-inf")).double()
    np.testing.assert_array_equal(sdpa(q, k, v, mask=bm)[0], sdpa(q, k, v, mask=fm)[0])
    # a per-row constant added to a float mask changes nothing (softmax shift invariance)
    fr = _t((2, 4, 13, 19), 34)
    shift = _t((2, 4, 13, 1), 35) * 10
    np.testing.assert_allclose(sdpa(q, k, v, mask=fr)[0], sdpa(q, k, v, mask=fr + shift)[0], **TIGHT)
    # causal == additive lower triangle
    tri = torch.tril(torch.ones(13, 19, dtype=torch.bool))
    np.testing.assert_array_equal(sdpa(q, k, v, is_causal=True)[0],
                                  sdpa(q, k, v, mask=torch.where(tri, 0.0, float("-inf")).double())[0])


def test_scale_folding_and_key_permutation():
    q, k, v = _t((1, 2, 9, 16), 40), _t((1, 2, 14, 16), 41), _t((1, 2, 14, 6), 42)
    a, _ = sdpa(q, k, v, scale=0.5)
    b, _ = sdpa(q * 0.5, k, v, scale=1.0)
    np.testing.assert_allclose(a, b, **TIGHT)
    perm = torch.randperm(14, generator=torch.Generator().manual_seed(43))
    c, _ = sdpa(q, k[:, :, perm], v[:, :, perm], scale=0.5)
    np.testing.assert_allclose(a, c, **TIGHT)


def test_gqa_equals_repeated_heads():
    q, k, v = _t((2, 8, 10, 16), 50), _t((2, 2, 12, 16), 51), _t((2, 2, 12, 8), 52)
    a, la = sdpa(q, k, v, is_causal=True)
    b, lb = sdpa(q, k.repeat_interleave(4, dim=1), v.repeat_interleave(4, dim=1), is_causal=True)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)
    # and a different head grouping (h % Hkv) would not agree
    c, _ = sdpa(q, k.repeat(1, 4, 1, 1), v.repeat(1, 4, 1, 1), is_causal=True)
    assert np.abs(a - c).max() > 1e-3


def test_bottom_right_causal_is_suffix_of_square_case():
    Lk, Lq = 21, 8
    q_full, k, v = _t((1, 2, Lk, 16), 60), _t((1, 2, Lk, 16), 61), _t((1, 2, Lk, 4), 62)
    sq = _torch_sdpa(q_full, k, v, is_causal=True)
    br, _ = sdpa(q_full[:, :, -Lq:], k, v, is_causal=True, causal_align="bottom_right")
    np.testing.assert_allclose(br, sq[:, :, -Lq:], **TIGHT)


def test_fully_masked_row_is_zero_with_minus_inf_lse():
    q, k, v = _t((1, 1, 4, 8), 70), _t((1, 1, 6, 8), 71), _t((1, 1, 6, 3), 72)
    m = torch.ones(1, 1, 4, 6, dtype=torch.bool)
    m[0, 0, 2] = False
    out, lse = sdpa(q, k, v, mask=m)
    assert np.all(out[0, 0, 2] == 0) and lse[0, 0, 2] == -np.inf
    assert np.all(np.isfinite(out))
    # top-left causal with Lq > Lk still keeps key 0 for every row; with Lk = 0 nothing is kept
    out, lse = sdpa(q, k[:, :, :0], v[:, :, :0])
    assert out.shape == (1, 1, 4, 3) and np.all(out == 0) and np.all(lse == -np.inf)


def test_page_worked_example_shape_and_values():
    gold = json.load(open(os.path.join(GOLDEN, "sdpa_worked_example.json")))
    w = page_example_fp32()
    assert list(w["q"].shape) == gold["q_shape"] and list(w["v"].shape) == gold["v_shape"]
    out, _ = sdpa(w["q"], w["k"], w["v"], scale=w["scale"])
    assert list(out.shape) == gold["expected_out_shape"]
    ref = _torch_sdpa(w["q"].double(), w["k"].double(), w["v"].double())
    np.testing.assert_allclose(out, ref, **TIGHT)


# ---------------------------------------------------------------- MLA prefill ----------

def _mla_inputs(lengths, kv_lengths, H, Hkv, dv=16, dr=8, seed=80):
    nq, nk = int(sum(lengths)), int(sum(kv_lengths))
    return (_t((nq, H, dv), seed), _t((nq, H, dr), seed + 1), _t((nk, Hkv, dv), seed + 2),
            _t((nk, Hkv, dr), seed + 3), _t((nk, Hkv, dv), seed + 4))


@pytest.mark.parametrize("mask_type", [0, 1])
def test_mla_equals_sdpa_on_concatenated_dims(mask_type):
    lengths = [5, 1, 12, 7]
    H, Hkv, scale = 4, 2, 0.19
    q, qr, k, kr, v = _mla_inputs(lengths, lengths, H, Hkv)
    out = varlen_mla_prefill(q, qr, k, kr, v, lengths, lengths, H, Hkv, scale, mask_type)
    cu = cu_seqlens(lengths)
    for i in range(len(lengths)):
        a, b = cu[i], cu[i + 1]
        qc = torch.cat([q[a:b], qr[a:b]], dim=-1).permute(1, 0, 2)[None]
        kc = torch.cat([k[a:b], kr[a:b]], dim=-1).permute(1, 0, 2)[None]
        vc = v[a:b].permute(1, 0, 2)[None]
        ref = _torch_sdpa(qc, kc, vc, scale=scale, is_causal=bool(mask_type))[0]
        np.testing.assert_allclose(out[a:b], ref.transpose(1, 0, 2), **TIGHT)


@pytest.mark.parametrize("mask_type", [0, 1])
def test_mla_padded_kv_equals_sdpa_per_sequence(mask_type):
    # The table's padded form [batch, max_seq, kv_head*d]: sequence i reads rows
    # [0, kv_len[i]) of entry i; the padding rows (filled with large values here) are unused.
    qlens, kvlens, max_seq = [5, 1, 7], [6, 3, 7], 9
    H, Hkv, scale, dv, dr = 4, 2, 0.21, 16, 8
    q, qr, _, _, _ = _mla_inputs(qlens, kvlens, H, Hkv, dv, dr)
    kp = _t((3, max_seq, Hkv, dv), 90) + 0.0
    krp = _t((3, max_seq, Hkv, dr), 91) + 0.0
    vp = _t((3, max_seq, Hkv, dv), 92) + 0.0
    for i, lk in enumerate(kvlens):
        kp[i, lk:] = 50.0
        krp[i, lk:] = -40.0
        vp[i, lk:] = 1e3
    out = varlen_mla_prefill(q, qr, kp.reshape(3, max_seq, -1), krp, vp, qlens, kvlens, H, Hkv,
                             scale, mask_type, kv_layout="padded")
    cq = cu_seqlens(qlens)
    G = H // Hkv
    for i, (lq, lk) in enumerate(zip(qlens, kvlens)):
        a, b = cq[i], cq[i + 1]
        qc = torch.cat([q[a:b], qr[a:b]], dim=-1).permute(1, 0, 2)[None]
        kc = torch.cat([kp[i, :lk], krp[i, :lk]], dim=-1).permute(1, 0, 2)[None]
        vc = vp[i, :lk].permute(1, 0, 2)[None]
        kc = kc.repeat_interleave(G, dim=1)
        vc = vc.repeat_interleave(G, dim=1)
        if mask_type:  # bottom-right: query r keeps key j <= r + lk - lq
            keep = torch.arange(lk)[None, :] <= torch.arange(lq)[:, None] + (lk - lq)
            ref = _torch_sdpa(qc, kc, vc, scale=scale, attn_mask=keep)[0]
        else:
            ref = _torch_sdpa(qc, kc, vc, scale=scale)[0]
        np.testing.assert_allclose(out[a:b], ref.transpose(1, 0, 2), **TIGHT)


def test_mla_padded_kv_rejects_long_sequence():
    q, qr, _, _, _ = _mla_inputs([2], [2], 2, 2)
    kp, vp = _t((1, 3, 2, 16), 1), _t((1, 3, 2, 16), 2)
    with pytest.raises(ValueError):
        varlen_mla_prefill(q, qr, kp, _t((1, 3, 2, 8), 3), vp, [2], [4], 2, 2, 0.3, 0,
                           kv_layout="padded")


@pytest.mark.parametrize("layout", ["packed", "padded"])
def test_mla_without_tokens_and_without_keys(layout):
    # no query tokens at all: an empty [0, Hq, Dv] result, flat or 3-D inputs alike; a
    # sequence without keys: its rows are 0 (fully masked rows give 0)
    q, qr, k, kr, v = _mla_inputs([0, 0], [3, 0], 2, 1)
    if layout == "padded":
        k, kr, v = (torch.stack([t, torch.zeros_like(t)]) for t in (k, kr, v))
    for qq, qqr in ((q, qr), (q.reshape(0, 2 * 16), qr.reshape(0, 2 * 8))):
        out = varlen_mla_prefill(qq, qqr, k, kr, v, [0, 0], [3, 0], 2, 1, 0.3, 1, kv_layout=layout)
        assert out.shape == (0, 2, v.shape[-1])
    q, qr, k, kr, v = _mla_inputs([2, 3], [2, 0], 2, 1)
    if layout == "padded":
        k, kr, v = (torch.stack([t, torch.zeros_like(t)]) for t in (k, kr, v))
    out = varlen_mla_prefill(q, qr, k, kr, v, [2, 3], [2, 0], 2, 1, 0.3, 0, kv_layout=layout)
    assert np.all(out[2:] == 0) and np.all(np.isfinite(out[:2])) and np.any(out[:2] != 0)


def test_mla_flat_layout_equals_3d_layout():
    lengths = [3, 9]
    q, qr, k, kr, v = _mla_inputs(lengths, lengths, 2, 2)
    a = varlen_mla_prefill(q, qr, k, kr, v, lengths, lengths, 2, 2, 0.3, 1)
    b = varlen_mla_prefill(q.reshape(12, -1), qr.reshape(12, -1), k, kr, v, lengths, lengths, 2, 2, 0.3, 1)
    np.testing.assert_array_equal(a, b)


def test_mla_bottom_right_with_longer_kv():
    qlens, kvlens = [4, 3], [9, 3]
    q, qr, k, kr, v = _mla_inputs(qlens, kvlens, 2, 1)
    out = varlen_mla_prefill(q, qr, k, kr, v, qlens, kvlens, 2, 1, 0.25, 1)
    # the first sequence's 4 queries are the last 4 rows of a square 9-token causal case
    qpad = torch.cat([_t((5, 2, 16), 99), q[:4]], dim=0)
    qrpad = torch.cat([_t((5, 2, 8), 98), qr[:4]], dim=0)
    full = varlen_mla_prefill(qpad, qrpad, k[:9], kr[:9], v[:9], [9], [9], 2, 1, 0.25, 1)
    np.testing.assert_allclose(out[:4], full[5:], **TIGHT)


def test_mla_no_cross_sequence_leakage():
    lengths = [6, 4, 8]
    q, qr, k, kr, v = _mla_inputs(lengths, lengths, 2, 2)
    a = varlen_mla_prefill(q, qr, k, kr, v, lengths, lengths, 2, 2, 0.3, 1)
    k2, v2 = k.clone(), v.clone()
    k2[6:10] += 5.0
    v2[6:10] -= 3.0
    b = varlen_mla_prefill(q, qr, k2, kr, v2, lengths, lengths, 2, 2, 0.3, 1)
    np.testing.assert_array_equal(a[:6], b[:6])
    np.testing.assert_array_equal(a[10:], b[10:])
    assert np.abs(a[6:10] - b[6:10]).max() > 1e-3


def test_mla_packing_invariance():
    lengths = [7, 2, 5]
    q, qr, k, kr, v = _mla_inputs(lengths, lengths, 2, 1)
    packed = varlen_mla_prefill(q, qr, k, kr, v, lengths, lengths, 2, 1, 0.4, 1)
    cu = cu_seqlens(lengths)
    for i in range(3):
        a, b = cu[i], cu[i + 1]
        single = varlen_mla_prefill(q[a:b], qr[a:b], k[a:b], kr[a:b], v[a:b], [b - a], [b - a], 2, 1, 0.4, 1)
        np.testing.assert_array_equal(packed[a:b], single)


# ---------------------------------------------------------------- block KV cache -------

def test_cache_page_example():
    gold = json.load(open(os.path.join(GOLDEN, "block_kv_cache_example.json")))
    c = BlockKVCacheOracle(gold["k_shape"], gold["v_shape"], gold["seq_dim"], gold["chunk_size"],
                           gold["window_size"], gold["sink_size"])
    for idx in range(gold["chunks"]):
        k = np.full((1, 1, 2, 2), float(idx), dtype=np.float32)
        v = np.full((1, 1, 2, 3), float(idx), dtype=np.float32)
        c.update(idx, k, v)
        vk, vv = c.cached_k(), c.cached_v()
        assert vk.shape[2] == gold["expected_visible_counts"][idx]
        assert vk[0, 0, :, 0].tolist() == gold["expected_visible_values"][idx]
        assert np.all(vk == vk[..., :1]) and np.all(vv[0, 0, :, 0] == vk[0, 0, :, 0])
        assert vv.shape == (1, 1, gold["expected_visible_counts"][idx], 3)


def test_cache_order_rules():
    c = BlockKVCacheOracle((1, 2, 8, 4), (1, 2, 8, 4), 2, 2, 6, 2)
    z = np.zeros((1, 2, 2, 4))
    with pytest.raises(CacheOrderError):
        c.update(1, z, z)  # the first chunk must be 0
    c.update(0, z, z)
    c.update(0, z + 1, z + 1)  # repeat overwrites the same logical chunk
    assert c.visible_tokens() == [0, 1] and np.all(c.cached_k() == 1)
    c.update(1, z + 2, z + 2)
    with pytest.raises(CacheOrderError):
        c.update(3, z, z)  # skipping raises
    with pytest.raises(CacheOrderError):
        c.update(0, z, z)  # going back raises
    assert c.last_chunk == 1
    with pytest.raises(ValueError):
        c.update(2, np.zeros((1, 2, 3, 4)), np.zeros((1, 2, 3, 4)))


@pytest.mark.parametrize("bad", [
    dict(chunk_size=2, window_size=5, sink_size=2),   # sink + window != length
    dict(chunk_size=3, window_size=6, sink_size=2),   # length 8 not divisible by 3
    dict(chunk_size=4, window_size=2, sink_size=6),   # window smaller than a chunk
])
def test_cache_config_rules(bad):
    with pytest.raises(CacheConfigError):
        BlockKVCacheOracle((1, 1, 8, 2), (1, 1, 8, 2), 2, **bad)


def _expected_cache_walk(sink, window, chunk, steps, seed):
    """Drive the oracle with a random legal index walk, tracking writes on the side."""
    rng = np.random.default_rng(seed)
    L = sink + window
    c = BlockKVCacheOracle((1, 1, L, 1), (1, 1, L, 2), 2, chunk, window, sink)
    last_write = {}
    idx, n = 0, 0
    for _ in range(steps):
        val = float(n)
        n += 1
        k = np.full((1, 1, chunk, 1), val) + np.arange(chunk)[None, None, :, None] * 1000
        v = np.repeat(k, 2, axis=3) * -1
        c.update(idx, k, v)
        for r in range(chunk):
            last_write[idx * chunk + r] = val + r * 1000
        T = (idx + 1) * chunk
        vis = c.visible_tokens()
        assert len(vis) == min(T, L)
        assert vis == sorted(vis) and len(set(vis)) == len(vis)
        assert all(t in vis for t in range(min(T, sink)))
        assert all(t in vis for t in range(idx * chunk, T))  # newest chunk always visible
        assert all(t >= T - window or t < sink for t in vis)
        ck = c.cached_k()[0, 0, :, 0]
        assert ck.tolist() == [last_write[t] for t in vis]
        assert np.array_equal(c.cached_v()[0, 0, :, 1], -ck)
        idx = idx + 1 if rng.random() < 0.7 else idx
    return c


@pytest.mark.parametrize("sink,window,chunk", [
    (s, w, ch) for ch in (1, 2, 3, 4) for s in range(0, 9) for w in range(1, 13)
    if (s + w) % ch == 0 and w >= ch and s + w <= 16])
def test_cache_walk_invariants(sink, window, chunk):
    _expected_cache_walk(sink, window, chunk, steps=14, seed=sink * 100 + window * 10 + chunk)


# ---------------------------------------------------------------- rotary embedding ----

from oracle.rotary import rope, sdpa_rope, INTERLEAVED, ROTATE_HALF


def _tables(max_pos, rot_dim, base=10000.0):
    theta = base ** (-np.arange(rot_dim // 2) * 2.0 / rot_dim)
    ang = np.arange(max_pos)[:, None] * theta[None, :]
    return np.cos(ang), np.sin(ang)


def test_rope_single_pair_is_a_plane_rotation():
    # one pair at one position: the 2-d rotation matrix by that angle
    for style in (ROTATE_HALF, INTERLEAVED):
        x = np.array([[[0.3, -1.2]]])
        phi = 0.7
        out = rope(x, np.array([[np.cos(phi)]] * 2), np.array([[np.sin(phi)]] * 2), 2, style, pos0=1)
        rot = np.array([[np.cos(phi), -np.sin(phi)], [np.sin(phi), np.cos(phi)]])
        np.testing.assert_allclose(out[0, 0], rot @ x[0, 0], rtol=0, atol=1e-15)


@pytest.mark.parametrize("style", [ROTATE_HALF, INTERLEAVED])
def test_rope_preserves_norms_and_the_tail(style):
    x = _t((2, 3, 17, 24), 5).numpy().astype(np.float64)
    c, s = _tables(40, 16)
    out = rope(x, c, s, 16, style, pos0=7)
    np.testing.assert_allclose(np.linalg.norm(out, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-12)
    np.testing.assert_array_equal(out[..., 16:], x[..., 16:])     # dims past rot_dim unchanged
    assert np.abs(out[..., :16] - x[..., :16]).max() > 1e-2       # and the rest did move
    np.testing.assert_array_equal(rope(x, c, s, 0, style), x)     # rot_dim 0: identity


@pytest.mark.parametrize("style", [ROTATE_HALF, INTERLEAVED])
def test_rope_scores_depend_on_distance_only(style):
    # with tables cos(p*theta), sin(p*theta) the rotated q_m . k_n is a function of m - n
    q = _t((1, 2, 5, 32), 6).numpy().astype(np.float64)
    k = _t((1, 2, 5, 32), 7).numpy().astype(np.float64)
    c, s = _tables(64, 32)
    a = rope(q, c, s, 32, style, 3) @ rope(k, c, s, 32, style, 0).swapaxes(-1, -2)
    b = rope(q, c, s, 32, style, 40) @ rope(k, c, s, 32, style, 37).swapaxes(-1, -2)
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-10)
    # and not an invariant of everything: a different distance changes the scores
    d = rope(q, c, s, 32, style, 41) @ rope(k, c, s, 32, style, 37).swapaxes(-1, -2)
    assert np.abs(a - d).max() > 1e-3


def test_rope_styles_differ_by_a_permutation_of_dims():
    x = _t((1, 1, 6, 8), 8).numpy().astype(np.float64)
    c, s = _tables(10, 8)
    perm = np.array([0, 4, 1, 5, 2, 6, 3, 7])          # interleaved position -> half position
    half = rope(x[..., perm], c, s, 8, INTERLEAVED, 2)  # dims 2i, 2i+1 hold i, i+4
    np.testing.assert_allclose(half[..., np.argsort(perm)], rope(x, c, s, 8, ROTATE_HALF, 2),
                               rtol=0, atol=1e-14)


def test_sdpa_rope_equals_sdpa_of_rotated_inputs():
    q, k, v = _t((2, 4, 9, 16), 9), _t((2, 2, 11, 16), 10), _t((2, 2, 11, 8), 11)
    c, s = _tables(32, 12)
    out, lse = sdpa_rope(q, k, v, c, s, 12, ROTATE_HALF, q_pos0=2, k_pos0=0, is_causal=True)
    qr = torch.from_numpy(rope(q, c, s, 12, ROTATE_HALF, 2))
    kr = torch.from_numpy(rope(k, c, s, 12, ROTATE_HALF, 0))
    ref = _torch_sdpa(qr, kr, v.double(), is_causal=True)
    np.testing.assert_allclose(out, ref, **TIGHT)
    with pytest.raises(ValueError):
        rope(q, c, s, 12, ROTATE_HALF, pos0=30)        # positions past the tables
