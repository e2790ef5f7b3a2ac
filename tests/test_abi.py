"""Host-side checks of the C ABI: the library loads, exports every function include/wf.h
declares, rejects bad arguments before enqueuing anything, and runs the block KV cache state
machine. No GPU needed: calls either fail validation or carry empty tensors (no launch)."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

from exact_attention_forward_flash_amd import _lib
from exact_attention_forward_flash_amd._lib import WfBlockKvState, WfTensor
from oracle import BlockKVCacheOracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wf.h")

OK, NULL, SHAPE, DTYPE, LAYOUT, UNSUP, ORDER, CONFIG, WS = 0, 1, 2, 3, 4, 5, 6, 7, 8


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from exact_attention_forward_flash_amd.build import build
        build(verbose=False)
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wf_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


FAKE = 1 << 20  # an aligned non-null address; never dereferenced on these paths


def T(shape, dtype=_lib.WF_BF16, stride=None, data=FAKE):
    t = WfTensor()
    t.data = data
    t.dtype = dtype
    t.ndim = len(shape)
    if stride is None:
        stride, acc = [], 1
        for s in reversed(shape):
            stride.insert(0, acc)
            acc *= s
    for i, (s, st) in enumerate(zip(shape, stride)):
        t.shape[i], t.stride[i] = s, st
    return t


def sdpa(lib, q, k, v, mask=None, causal=0, dropout=0.0, scale=float("nan"), out=None):
    out = out or T([q.shape[0], q.shape[1], q.shape[2], v.shape[3]], q.dtype)
    return lib.wf_sdpa_fwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                           ctypes.byref(mask) if mask else None, causal, dropout, scale,
                           ctypes.byref(out), None, None)


def test_sdpa_validation_errors(lib):
    q, k, v = T([2, 8, 16, 128]), T([2, 2, 24, 128]), T([2, 2, 24, 128])
    assert lib.wf_sdpa_fwd(None, ctypes.byref(k), ctypes.byref(v), None, 0, 0.0, 1.0,
                           ctypes.byref(T([2, 8, 16, 128])), None, None) == NULL
    assert sdpa(lib, q, k, v, dropout=0.1) == UNSUP
    assert sdpa(lib, q, T([2, 3, 24, 128]), T([2, 3, 24, 128])) == SHAPE  # 8 % 3 != 0
    assert sdpa(lib, q, T([2, 2, 24, 128], _lib.WF_F16), v) == DTYPE
    assert sdpa(lib, q, k, T([2, 2, 25, 128])) == SHAPE
    assert sdpa(lib, q, k, v, scale=-1.0) == UNSUP
    assert sdpa(lib, q, k, v, scale=float("inf")) == UNSUP
    assert sdpa(lib, T([2, 8, 16, 96]), T([2, 2, 24, 96]), T([2, 2, 24, 96])) == UNSUP
    assert sdpa(lib, T([2, 8, 16, 128], stride=[1, 1, 1, 2]), k, v) == LAYOUT
    assert sdpa(lib, T([2, 8, 16, 128], data=FAKE + 2), k, v) == LAYOUT
    m = T([2, 1, 16, 24], _lib.WF_BOOL)
    assert sdpa(lib, q, k, v, mask=m, causal=1) == UNSUP
    assert sdpa(lib, q, k, v, mask=T([2, 1, 16, 23], _lib.WF_BOOL)) == SHAPE
    assert sdpa(lib, q, k, v, mask=T([2, 1, 16, 24], _lib.WF_F16)) == DTYPE
    assert sdpa(lib, q, k, v, mask=T([2, 1, 16, 24], _lib.WF_BOOL, stride=[384, 384, 24, 2])) == LAYOUT
    # empty problems validate and return without launching
    assert sdpa(lib, T([0, 8, 16, 128]), T([0, 2, 24, 128]), T([0, 2, 24, 128])) == OK


def test_decode_validation_errors(lib):
    q, k, v = T([2, 8, 1, 128]), T([2, 2, 4096, 128]), T([2, 2, 4096, 128])
    need = lib.wf_sdpa_decode_workspace_size(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 0)
    assert need > 256
    # a shape-only size: the causal variant and a longer K/V give sizes of their own
    assert lib.wf_sdpa_decode_workspace_size(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 1) > 256
    assert lib.wf_sdpa_decode_workspace_size(ctypes.byref(T([2, 8, 1, 96])), ctypes.byref(T([2, 2, 64, 96])),
                                             ctypes.byref(T([2, 2, 64, 96])), 0) == 0

    def call(q=q, k=k, v=v, out=None, causal=0, scale=0.1, ws=FAKE, wsb=need):
        out = out or T([q.shape[0], q.shape[1], q.shape[2], v.shape[3]], q.dtype)
        return lib.wf_sdpa_decode(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), causal, scale,
                                  ctypes.byref(out), None, ws, wsb, None)
    assert call(ws=None) == WS
    assert call(wsb=need - 1) == WS
    assert call(ws=FAKE + 64) == WS                               # 256-byte alignment
    assert call(q=T([2, 8, 1, 128], _lib.WF_F32), k=T([2, 2, 4096, 128], _lib.WF_F32),
                v=T([2, 2, 4096, 128], _lib.WF_F32)) == DTYPE
    assert call(k=T([2, 3, 4096, 128]), v=T([2, 3, 4096, 128])) == SHAPE   # 8 % 3 != 0
    assert call(q=T([2, 8, 1, 96]), k=T([2, 2, 64, 96]), v=T([2, 2, 64, 96])) == UNSUP
    # a value width other than the key width: wf_sdpa_fwd takes it, the split kernels do not
    q64, k64, v96 = T([2, 8, 1, 64]), T([2, 2, 64, 64]), T([2, 2, 64, 96])
    assert lib.wf_sdpa_decode_workspace_size(ctypes.byref(q64), ctypes.byref(k64), ctypes.byref(v96), 0) == 0
    assert call(q=q64, k=k64, v=v96, out=T([2, 8, 1, 96])) == UNSUP
    assert call(out=T([2, 8, 2, 128])) == SHAPE
    assert call(scale=0.0) == UNSUP
    assert call(q=T([0, 8, 1, 128]), k=T([0, 2, 4096, 128]), v=T([0, 2, 4096, 128])) == OK


def test_rope_validation_errors(lib):
    q, k, v = T([1, 4, 16, 128]), T([1, 2, 24, 128]), T([1, 2, 24, 128])
    out = T([1, 4, 16, 128])
    need = lib.wf_sdpa_rope_workspace_size(ctypes.byref(q), ctypes.byref(k))
    assert need >= (4 * 16 + 2 * 24) * 128 * 2   # rotated copies of q and k

    def call(rot=64, style=0, qp=0, kp=0, max_pos=64, cos=FAKE, ws=FAKE, wsb=need, rope=True, q=q, k=k, v=v,
             out=out):
        r = _lib.WfRope(cos, FAKE, max_pos, rot, style, qp, kp)
        return lib.wf_sdpa_rope_fwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), None, 0, 0.1,
                                    ctypes.byref(r) if rope else None, ctypes.byref(out), None,
                                    ws, wsb, None)
    assert call(rope=False) == NULL
    assert call(rot=40) == UNSUP                      # not a multiple of 16
    assert call(rot=144) == UNSUP                     # past the head dim
    assert call(style=2) == UNSUP
    assert call(cos=None) == NULL
    assert call(cos=FAKE + 4) == LAYOUT               # 16-byte aligned tables
    assert call(qp=50) == SHAPE                       # q positions 50..65 past 64 rows
    assert call(kp=-1) == SHAPE
    assert call(ws=None) == WS
    assert call(wsb=need - 1) == WS
    assert call(k=T([1, 3, 24, 128]), v=T([1, 3, 24, 128])) == SHAPE   # SDPA checks come first
    assert call(q=T([0, 4, 16, 128]), k=T([0, 2, 24, 128]), v=T([0, 2, 24, 128]),
                out=T([0, 4, 16, 128])) == OK   # empty: validated, nothing launched


def test_status_strings(lib):
    assert lib.wf_status_string(0) == b"WF_OK"
    assert lib.wf_status_string(6) == b"WF_ERR_CHUNK_ORDER"
    sdpa(lib, T([2, 8, 16, 128]), T([2, 2, 24, 128]), T([2, 2, 24, 128]), dropout=0.5)
    assert b"dropout" in lib.wf_last_error()


def test_mla_validation_errors(lib):
    n, H = 100, 4
    q, qr = T([n, H, 128]), T([n, H, 64])
    k, kr, v = T([n, H, 128]), T([n, H, 64]), T([n, H, 128])
    out = T([n, H, 128])
    need = lib.wf_varlen_mla_prefill_workspace_size(3, n, H)
    assert need > 0

    def call(q=q, qr=qr, k=k, kr=kr, v=v, out=out, batch=3, hn=H, kvh=H, scale=0.1, mt=1,
             ws=FAKE, wsb=need, lens=FAKE):
        return lib.wf_varlen_mla_prefill(ctypes.byref(q), ctypes.byref(qr), ctypes.byref(k),
                                         ctypes.byref(kr), ctypes.byref(v), lens, lens, batch,
                                         hn, kvh, scale, mt, ctypes.byref(out), ws, wsb, None)
    assert call(qr=T([n, H, 32])) == SHAPE          # rope part must be 64 wide
    assert call(hn=3, kvh=2) == SHAPE                 # head counts
    assert call(mt=2) == UNSUP                        # SPEC / MASK_FREE are not built
    assert call(wsb=need - 1) == WS
    assert call(ws=None) == WS
    assert call(ws=FAKE + 16) == WS                   # 256-byte alignment
    assert call(lens=None) == NULL
    assert call(q=T([n, H, 128], _lib.WF_F32), qr=T([n, H, 64], _lib.WF_F32)) == DTYPE
    assert call(scale=0.0) == UNSUP
    # the flat [nTokens, H*d] form is accepted (and empty batch launches nothing)
    assert call(q=T([n, H * 128]), out=T([n, H * 128]), batch=0) == OK
    # padded K/V [batch, max_seq, Hkv, d]: all three padded, one batch entry per sequence
    pk, pkr, pv = T([3, 40, H, 128]), T([3, 40, H, 64]), T([3, 40, H, 128])
    assert call(k=pk, kr=pkr, v=pv, batch=3, ws=None) == WS      # layout accepted up to the workspace
    assert call(k=pk, kr=kr, v=pv) == LAYOUT                      # mixed packed / padded
    assert call(k=pk, kr=pkr, v=T([3, 40, H, 64])) == SHAPE       # value width
    assert call(k=T([2, 40, H, 128]), kr=T([2, 40, H, 64]), v=T([2, 40, H, 128])) == SHAPE  # batch
    assert call(k=T([0, 40, H, 128]), kr=T([0, 40, H, 64]), v=T([0, 40, H, 128]), batch=0) == OK


def _state(lib, L, sink, window, chunk):
    s = WfBlockKvState()
    rc = lib.wf_block_kv_init(ctypes.byref(s), L, sink, window, chunk)
    return s, rc


def test_cache_config_rules(lib):
    assert _state(lib, 8, 2, 6, 2)[1] == OK
    assert _state(lib, 8, 2, 5, 2)[1] == CONFIG   # sink + window != length
    assert _state(lib, 8, 2, 6, 3)[1] == CONFIG   # 8 % 3 != 0
    assert _state(lib, 8, 6, 2, 4)[1] == CONFIG   # window < chunk
    assert _state(lib, 8, -1, 9, 4)[1] == CONFIG
    assert lib.wf_block_kv_init(None, 8, 2, 6, 2) == NULL


def _empty_update(lib, s, idx, chunk, L, D=8):
    z = T([0, 1, chunk, D], _lib.WF_F16)
    c = T([0, 1, L, D], _lib.WF_F16)
    return lib.wf_block_kv_cache_update(ctypes.byref(s), idx, ctypes.byref(z), ctypes.byref(z),
                                        ctypes.byref(c), ctypes.byref(c), None)


def test_cache_chunk_order_state_machine(lib):
    s, _ = _state(lib, 8, 2, 6, 2)
    assert _empty_update(lib, s, 1, 2, 8) == ORDER and s.last_chunk == -1  # first must be 0
    assert _empty_update(lib, s, 0, 2, 8) == OK and s.last_chunk == 0
    assert _empty_update(lib, s, 0, 2, 8) == OK and s.last_chunk == 0      # repeat overwrites
    assert _empty_update(lib, s, 1, 2, 8) == OK and s.last_chunk == 1
    assert _empty_update(lib, s, 3, 2, 8) == ORDER and s.last_chunk == 1   # skip
    assert _empty_update(lib, s, 0, 2, 8) == ORDER and s.last_chunk == 1   # backwards
    z = T([0, 1, 3, 8], _lib.WF_F16)
    c = T([0, 1, 8, 8], _lib.WF_F16)
    assert lib.wf_block_kv_cache_update(ctypes.byref(s), 2, ctypes.byref(z), ctypes.byref(z),
                                        ctypes.byref(c), ctypes.byref(c), None) == SHAPE
    assert s.last_chunk == 1


def _visible(lib, s):
    n = ctypes.c_int64()
    assert lib.wf_block_kv_visible(ctypes.byref(s), ctypes.byref(n), None) == OK
    idx = (ctypes.c_int64 * max(1, n.value))()
    assert lib.wf_block_kv_visible(ctypes.byref(s), ctypes.byref(n), idx) == OK
    return list(idx)[:n.value]


@pytest.mark.parametrize("sink,window,chunk", [
    (s, w, c) for c in (1, 2, 3) for s in range(0, 7) for w in range(1, 10)
    if (s + w) % c == 0 and w >= c])
def test_cache_slots_hold_the_oracles_visible_tokens(lib, sink, window, chunk):
    """Replays a token stream through the library's slot map and the oracle's token list:
    writing token t into slot(t) for every update must leave, at the library's visible slots,
    exactly the oracle's visible tokens in the oracle's order."""
    L = sink + window
    s, rc = _state(lib, L, sink, window, chunk)
    assert rc == OK
    o = BlockKVCacheOracle((1, 1, L, 1), (1, 1, L, 1), 2, chunk, window, sink)
    slots = [None] * L
    rng = np.random.default_rng(L * 100 + chunk)
    idx, stamp = 0, 0
    for _ in range(12):
        rows = np.arange(stamp, stamp + chunk, dtype=np.float64).reshape(1, 1, chunk, 1)
        stamp += chunk
        o.update(idx, rows, rows)
        assert _empty_update(lib, s, idx, chunk, L) == OK
        for r in range(chunk):  # what the copy kernel writes, by the slot rule in wf.h
            t = idx * chunk + r
            slot = t if t < sink else sink + (t - sink) % window
            slots[slot] = rows[0, 0, r, 0]
        vis = _visible(lib, s)
        assert [slots[p] for p in vis] == o.cached_k()[0, 0, :, 0].tolist()
        idx = idx + 1 if rng.random() < 0.75 else idx


def test_noalloc_prefill_rejects_before_touching_the_device(lib):
    n, H = 100, 4
    q, qr = T([n, H, 128]), T([n, H, 64])
    k, kr, v, out = T([n, H, 128]), T([n, H, 64]), T([n, H, 128]), T([n, H, 128])

    def call(q=q, batch=3):
        return lib.wf_varlen_mla_prefill_noalloc(q if q is None else ctypes.byref(q),
                                                 ctypes.byref(qr), ctypes.byref(k),
                                                 ctypes.byref(kr), ctypes.byref(v), FAKE, FAKE,
                                                 batch, H, H, 0.1, 1, ctypes.byref(out), None)
    assert call(q=None) == NULL
    many = 200_000                                   # 8 bytes of schedule per sequence: > 1 MiB
    assert lib.wf_varlen_mla_prefill_workspace_size(many, n, H) > (1 << 20)
    assert call(batch=many) == WS
    assert "1048576" in lib.wf_last_error().decode()


def test_library_build_id_matches_the_sources(lib):
    from exact_attention_forward_flash_amd.build import source_hash
    assert lib.wf_build_id().decode() == source_hash()
    with pytest.raises(RuntimeError, match="rebuild"):
        _lib.check_build_id("0" * 64)


def test_source_hash_follows_every_source_and_header(tmp_path, monkeypatch):
    import shutil
    from exact_attention_forward_flash_amd import build as b
    root = tmp_path / "tree"
    shutil.copytree(b.CSRC, root / "pkg" / "csrc")
    shutil.copytree(os.path.join(b.ROOT, "include"), root / "include")
    monkeypatch.setattr(b, "ROOT", str(root))
    monkeypatch.setattr(b, "CSRC", str(root / "pkg" / "csrc"))
    base = b.source_hash()
    for rel in ("pkg/csrc/attn_fwd_p.hpp", "pkg/csrc/wf_api.cpp", "include/wf.h"):
        p = root / rel
        text = p.read_bytes()
        p.write_bytes(text + b"\n")
        assert b.source_hash() != base, rel
        p.write_bytes(text)
        assert b.source_hash() == base


def test_fused_update_attend_checks_both_calls_before_anything(lib):
    """The fused update + attend runs every check of the update and of the attend first: a
    bad chunk index, bad update shapes or bad attend arguments leave the state unchanged.
    Empty tensors (B = 0) pass the checks without a launch and commit the chunk."""
    s, _ = _state(lib, 8, 2, 6, 2)

    def call(idx, q=None, out=None, z=None, ws=FAKE, wsb=1 << 20):
        z = z or T([0, 1, 2, 64], _lib.WF_F16)
        c = T([0, 1, 8, 64], _lib.WF_F16)
        q = q or T([0, 1, 2, 64], _lib.WF_F16)
        out = out or T([0, 1, 2, 64], _lib.WF_F16)
        return lib.wf_block_kv_update_attend(ctypes.byref(s), idx, ctypes.byref(z), ctypes.byref(z),
                                             ctypes.byref(c), ctypes.byref(c), ctypes.byref(q), 0,
                                             0.125, ctypes.byref(out), ws, wsb, None)
    assert call(1) == ORDER and s.last_chunk == -1
    assert call(0, z=T([0, 1, 3, 64], _lib.WF_F16)) == SHAPE and s.last_chunk == -1
    assert call(0, q=T([0, 1, 2, 32], _lib.WF_F16)) == SHAPE and s.last_chunk == -1   # q width
    assert call(0, out=T([0, 1, 3, 64], _lib.WF_F16)) == SHAPE and s.last_chunk == -1
    assert call(0, ws=None) == WS and s.last_chunk == -1
    assert call(0, q=T([0, 1, 2, 64], _lib.WF_F32)) == DTYPE and s.last_chunk == -1
    assert call(0) == OK and s.last_chunk == 0
    assert call(0) == OK and s.last_chunk == 0      # repeat
    assert call(2) == ORDER and s.last_chunk == 0
