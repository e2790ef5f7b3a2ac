"""GPU checks of the rolling block KV cache: contents and indices bit-exact against the
oracle's token list, and the attend within tolerance of the oracle's SDPA on that view."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from exact_attention_forward_flash_amd import BlockKVCache, ChunkOrderError, tune
from synth import cache_stream_chunks
from tests.parity import assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_page_example_on_gpu():
    gold = json.load(open(os.path.join(GOLDEN, "block_kv_cache_example.json")))
    c = BlockKVCache(gold["k_shape"], gold["v_shape"], gold["seq_dim"], gold["chunk_size"],
                     gold["window_size"], gold["sink_size"], device=DEV, dtype=torch.float32)
    for idx in range(gold["chunks"]):
        k = torch.full((1, 1, 2, 2), float(idx), device=DEV)
        v = torch.full((1, 1, 2, 3), float(idx), device=DEV)
        c.before_update(idx)
        c.update(k, v)
        vk, vv = c.cached_k().cpu(), c.cached_v().cpu()
        c.after_update(idx)
        assert vk.shape[2] == gold["expected_visible_counts"][idx]
        assert vk[0, 0, :, 0].tolist() == gold["expected_visible_values"][idx]
        assert torch.equal(vv[0, 0, :, :], vk[0, 0, :, :1].expand(-1, 3))


@pytest.mark.parametrize("sink,window,chunk,dtype,seq_dim", [
    (2, 6, 2, torch.float16, 2), (0, 8, 4, torch.bfloat16, 2), (5, 3, 2, torch.float16, 2),
    (4, 12, 4, torch.float32, 1), (3, 9, 3, torch.bfloat16, 1)])
def test_random_walk_bit_exact(sink, window, chunk, dtype, seq_dim):
    L, H, D = sink + window, 2, 64
    shape = (1, H, L, D) if seq_dim == 2 else (1, L, H, D)
    c = BlockKVCache(shape, shape, seq_dim, chunk, window, sink, device=DEV, dtype=dtype)
    o = oracle.BlockKVCacheOracle(shape, shape, seq_dim, chunk, window, sink)
    g = torch.Generator().manual_seed(L * 10 + chunk)
    rng = np.random.default_rng(L)
    idx = 0
    cshape = (1, H, chunk, D) if seq_dim == 2 else (1, chunk, H, D)
    for step in range(14):
        k = torch.randn(cshape, generator=g).to(dtype)
        v = torch.randn(cshape, generator=g).to(dtype)
        o.update(idx, k.numpy() if dtype != torch.bfloat16 else k.float().numpy(),
                 v.numpy() if dtype != torch.bfloat16 else v.float().numpy())
        c.before_update(idx)
        c.update(k.to(DEV), v.to(DEV))
        assert np.array_equal(c.cached_k().cpu().float().numpy(), o.cached_k().astype(np.float32))
        assert np.array_equal(c.cached_v().cpu().float().numpy(), o.cached_v().astype(np.float32))
        c.after_update(idx)
        idx = idx + 1 if rng.random() < 0.7 else idx
    with pytest.raises(ChunkOrderError):
        c.before_update(idx + 2)
        c.update(torch.zeros(cshape, dtype=dtype, device=DEV), torch.zeros(cshape, dtype=dtype, device=DEV))


def _attend_check(c, o, q, what):
    out = c.attend(q.to(DEV))
    kv, vv = o.cached_k(), o.cached_v()
    ref, _ = oracle.sdpa(q, torch.from_numpy(kv), torch.from_numpy(vv),
                         scale=np.float32(1.0 / np.sqrt(q.shape[-1])))
    assert_close(out, ref, q.dtype, what)


@pytest.mark.parametrize("heads,check_chunks", [(4, {0, 1, 14, 15, 16, 17, 40, 63}), (24, {16, 63})])
def test_cache_stream(heads, check_chunks):
    """fp16, d=128, chunk 256, sink 256 + window 3840, 64 chunks; per chunk: update, then the
    chunk's 256 queries attend (non-causally) to every visible token including themselves."""
    shape = (1, heads, 4096, 128)
    c = BlockKVCache(shape, shape, 2, 256, 3840, 256, device=DEV, dtype=torch.float16)
    o = oracle.BlockKVCacheOracle(shape, shape, 2, 256, 3840, 256)
    for idx, q, k, v in cache_stream_chunks(H=24):
        q, k, v = q[:, :heads], k[:, :heads], v[:, :heads]
        c.before_update(idx)
        c.update(k.to(DEV), v.to(DEV))
        o.update(idx, k.numpy(), v.numpy())
        if idx in check_chunks:
            n, slots = c.visible()
            assert n == min((idx + 1) * 256, 4096) == c.n_visible() == len(slots)
            assert np.array_equal(c.cached_k().cpu().numpy(), o.cached_k())
            _attend_check(c, o, q, f"chunk {idx}")
        else:
            c.attend(q.to(DEV))
        c.after_update(idx)


def test_attend_small_split_and_dense_paths():
    """Few visible tokens take the single-split path; many take split-KV plus the combine."""
    for sink, window, chunk, steps in ((0, 64, 64, 1), (64, 448, 64, 12)):
        shape = (1, 2, sink + window, 64)
        c = BlockKVCache(shape, shape, 2, chunk, window, sink, device=DEV, dtype=torch.bfloat16)
        o = oracle.BlockKVCacheOracle(shape, shape, 2, chunk, window, sink)
        g = torch.Generator().manual_seed(steps)
        for idx in range(steps):
            k = torch.randn(1, 2, chunk, 64, generator=g).to(torch.bfloat16)
            v = torch.randn(1, 2, chunk, 64, generator=g).to(torch.bfloat16)
            q = torch.randn(1, 4, 100, 64, generator=g).to(torch.bfloat16)  # GQA: 4 q heads
            c.before_update(idx)
            c.update(k.to(DEV), v.to(DEV))
            o.update(idx, k.float().numpy(), v.float().numpy())
            kv = torch.from_numpy(o.cached_k()).to(torch.bfloat16)
            vv = torch.from_numpy(o.cached_v()).to(torch.bfloat16)
            out = c.attend(q.to(DEV))
            ref, _ = oracle.sdpa(q, kv, vv, scale=np.float32(1.0 / 8.0))
            assert_close(out, ref, torch.bfloat16, f"step {idx}")
            c.after_update(idx)


def test_decode_over_the_cache_gqa():
    """One new query per head over a GQA cache (4 query heads per cached KV head), as in
    decoding: the attend shares each K/V tile among the query heads of its KV head."""
    sink, window, chunk = 64, 960, 64
    shape = (2, 2, sink + window, 128)
    c = BlockKVCache(shape, shape, 2, chunk, window, sink, device=DEV, dtype=torch.float16)
    o = oracle.BlockKVCacheOracle(shape, shape, 2, chunk, window, sink)
    g = torch.Generator().manual_seed(21)
    for idx in range(20):
        k = torch.randn(2, 2, chunk, 128, generator=g).to(torch.float16)
        v = torch.randn(2, 2, chunk, 128, generator=g).to(torch.float16)
        c.before_update(idx)
        c.update(k.to(DEV), v.to(DEV))
        o.update(idx, k.float().numpy(), v.float().numpy())
        if idx in (0, 5, 16, 19):
            q = torch.randn(2, 8, 1, 128, generator=g).to(torch.float16)
            kv = torch.from_numpy(o.cached_k()).to(torch.float16)
            vv = torch.from_numpy(o.cached_v()).to(torch.float16)
            out = c.attend(q.to(DEV))
            ref, _ = oracle.sdpa(q, kv, vv, scale=np.float32(1.0 / np.sqrt(128.0)))
            assert_close(out, ref, torch.float16, f"chunk {idx}")
        c.after_update(idx)


def test_snapshot_restore_continues_bit_identically():
    """A snapshot taken mid-stream (state plus both tensors) restored into a second cache: both
    copies then take the same chunks, with a repeated chunk and the roll past the window, and
    agree bit for bit in contents, visible slots and attend outputs; restoring the original
    cache to the snapshot replays the same trajectory again."""
    sink, window, chunk, H, D = 64, 448, 64, 2, 128
    shape = (1, H, sink + window, D)
    g = torch.Generator().manual_seed(21)
    chunks = [(i, torch.randn(1, H, chunk, D, generator=g).half(),
               torch.randn(1, H, chunk, D, generator=g).half(),
               torch.randn(1, 2 * H, 96, D, generator=g).half()) for i in range(16)]
    chunks.insert(12, (11,) + chunks[11][1:])          # repeat chunk 11 (overwrite)
    a = BlockKVCache(shape, shape, 2, chunk, window, sink, device=DEV, dtype=torch.float16)

    def step(c, item):
        idx, k, v, q = item
        c.before_update(idx)
        c.update(k.to(DEV), v.to(DEV))
        out = c.attend(q.to(DEV))
        c.after_update(idx)
        return out

    for item in chunks[:6]:
        step(a, item)
    snap = a.snapshot()
    b = BlockKVCache(shape, shape, 2, chunk, window, sink, device=DEV, dtype=torch.float16)
    b.restore(snap)
    assert b.visible() == a.visible() and b.last_chunk == a.last_chunk == 5
    outs_a = [step(a, item) for item in chunks[6:]]
    outs_b = [step(b, item) for item in chunks[6:]]
    assert all(torch.equal(x, y) for x, y in zip(outs_a, outs_b))
    assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    assert a.visible() == b.visible() and a.last_chunk == b.last_chunk == 15
    a.restore(snap)
    outs_r = [step(a, item) for item in chunks[6:]]
    assert all(torch.equal(x, y) for x, y in zip(outs_r, outs_b))
    assert torch.equal(a.k, b.k) and a.visible() == b.visible()
    assert torch.isfinite(outs_b[-1].float()).all()


@pytest.mark.parametrize("sink,window,chunk,H,Hkv,dt,nw", [
    (64, 448, 64, 2, 2, torch.float16, -1), (0, 256, 64, 4, 1, torch.bfloat16, -1),
    (32, 96, 32, 8, 2, torch.float16, -1), (256, 3840, 256, 4, 4, torch.float16, -1),
    (128, 896, 256, 2, 2, torch.bfloat16, -1),
    (256, 3840, 256, 4, 4, torch.float16, 8), (128, 896, 256, 2, 2, torch.bfloat16, 8)])
def test_causal_attend_reads_keys_in_chronological_order(sink, window, chunk, H, Hkv, dt, nw):
    """Causal attend (the chunk's queries are the newest visible tokens) across the roll of
    the window: only a kernel that reads the ring in chronological order matches the oracle's
    causal attention over its token list once the ring has wrapped; the non-causal attend
    of the same chunk is checked too, and a single new query as in decoding. nw=8 forces the
    8-wave split groups (one query head per KV head, more than 128 queries; automatic only
    for many heads over long caches)."""
    with tune(attend_nw=nw):
        _causal_attend_case(sink, window, chunk, H, Hkv, dt)


def _causal_attend_case(sink, window, chunk, H, Hkv, dt):
    D = 64 if chunk < 256 else 128
    shape = (1, Hkv, sink + window, D)
    c = BlockKVCache(shape, shape, 2, chunk, window, sink, device=DEV, dtype=dt)
    o = oracle.BlockKVCacheOracle(shape, shape, 2, chunk, window, sink)
    g = torch.Generator().manual_seed(sink + window + chunk + H)
    steps = (sink + window) // chunk + 5 if chunk < 256 else 18
    for idx in range(steps):
        k = torch.randn(1, Hkv, chunk, D, generator=g).to(dt)
        v = torch.randn(1, Hkv, chunk, D, generator=g).to(dt)
        q = torch.randn(1, H, chunk, D, generator=g).to(dt)
        c.before_update(idx)
        c.update(k.to(DEV), v.to(DEV))
        o.update(idx, k.float().numpy(), v.float().numpy())
        if idx % 3 == 2 or idx == steps - 1:
            kv = torch.from_numpy(o.cached_k()).to(dt)
            vv = torch.from_numpy(o.cached_v()).to(dt)
            sc = np.float32(1.0 / np.sqrt(D))
            ref, _ = oracle.sdpa(q, kv, vv, is_causal=True, scale=sc, causal_align="bottom_right")
            assert_close(c.attend(q.to(DEV), is_causal=True), ref, dt, f"causal, chunk {idx}")
            ref, _ = oracle.sdpa(q, kv, vv, scale=sc)
            assert_close(c.attend(q.to(DEV)), ref, dt, f"non-causal, chunk {idx}")
            q1 = q[:, :, -1:].contiguous()
            ref, _ = oracle.sdpa(q1, kv, vv, is_causal=True, scale=sc, causal_align="bottom_right")
            assert_close(c.attend(q1.to(DEV), is_causal=True), ref, dt, f"one query, chunk {idx}")
        c.after_update(idx)


@pytest.mark.parametrize("sink,window,chunk,H,Hkv,causal,nw", [
    (64, 448, 64, 2, 2, False, -1), (0, 256, 64, 4, 1, True, -1), (256, 3840, 256, 24, 24, False, -1),
    (32, 96, 32, 8, 2, True, -1), (256, 768, 256, 4, 4, True, -1),
    (256, 3840, 256, 24, 24, False, 8), (256, 768, 256, 4, 4, True, 8)])
def test_fused_update_attend_matches_the_two_calls(sink, window, chunk, H, Hkv, causal, nw):
    """update_attend gives the output of update then attend (bit for bit when the attend takes
    the split kernel too; a non-causal attend over a single key split may take a dense kernel
    instead, which rounds differently) and leaves the same cache contents, across the roll of
    the window and a repeated chunk; nw=8 forces the 8-wave split groups."""
    with tune(attend_nw=nw):
        _fused_case(sink, window, chunk, H, Hkv, causal)


def _fused_case(sink, window, chunk, H, Hkv, causal):
    D = 128
    shape = (1, Hkv, sink + window, D)
    a = BlockKVCache(shape, shape, 2, chunk, window, sink, device=DEV, dtype=torch.float16)
    b = BlockKVCache(shape, shape, 2, chunk, window, sink, device=DEV, dtype=torch.float16)
    g = torch.Generator().manual_seed(sink + window + H)
    steps = min((sink + window) // chunk + 4, 20)
    order = list(range(steps))
    order.insert(5, 4)                      # chunk 4 again: overwrite
    for idx in order:
        k = torch.randn(1, Hkv, chunk, D, generator=g).half().to(DEV)
        v = torch.randn(1, Hkv, chunk, D, generator=g).half().to(DEV)
        q = torch.randn(1, H, chunk, D, generator=g).half().to(DEV)
        a.before_update(idx)
        a.update(k, v)
        ref = a.attend(q, is_causal=causal)
        a.after_update(idx)
        b.before_update(idx)
        got = b.update_attend(k, v, q, is_causal=causal)
        b.after_update(idx)
        if causal:
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"chunk {idx}"
        else:
            d = (got.float() - ref.float()).abs()
            assert d.max().item() < 4e-3 and d.mean().item() < 2e-4, f"chunk {idx}: {d.max().item()}"
        assert torch.equal(a.k, b.k) and torch.equal(a.v, b.v), f"cache after chunk {idx}"
        assert a.last_chunk == b.last_chunk == idx
