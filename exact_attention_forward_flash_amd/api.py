"""Python surface over libwf.so: torch tensors in, torch tensors out.

Argument marshalling only: shapes and strides are described to the C ABI, outputs and
workspaces are allocated with torch on the inputs' device, and every computation runs in
the library's HIP kernels on torch's current stream.
"""
from __future__ import annotations

import contextlib
import ctypes
import math

import torch

from . import _lib
from ._lib import WfBlockKvState, WfTensor, check

_DTYPES = {torch.float32: _lib.WF_F32, torch.float16: _lib.WF_F16, torch.bfloat16: _lib.WF_BF16,
           torch.bool: _lib.WF_BOOL, torch.int32: _lib.WF_I32}


def describe(t: torch.Tensor | None):
    """A wf_tensor view of a torch tensor (no copy), or None."""
    if t is None:
        return None
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    if t.dim() > 4:
        raise ValueError("at most 4 dimensions")
    d = WfTensor()
    d.data = t.data_ptr() if t.numel() > 0 else None
    d.dtype = _DTYPES[t.dtype]
    d.ndim = t.dim()
    for i in range(t.dim()):
        d.shape[i] = t.shape[i]
        d.stride[i] = t.stride(i)
    return d


def _ref(d):
    return ctypes.byref(d) if d is not None else None


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _scale(scale):
    return float("nan") if scale is None else float(scale)


@contextlib.contextmanager
def tune(**settings):
    """Overrides the library's kernel choice for the calls inside the block (names and values
    as wf_tune_set in include/wf.h; -1 = automatic), restoring the previous values after."""
    lib = _lib.load()
    old = {}
    for name, value in settings.items():
        cur = ctypes.c_int()
        check(lib.wf_tune_get(name.encode(), ctypes.byref(cur)))
        old[name] = cur.value
        check(lib.wf_tune_set(name.encode(), int(value)))
    try:
        yield
    finally:
        for name, value in old.items():
            lib.wf_tune_set(name.encode(), value)


def sdpa(q, k, v, attn_mask=None, dropout_p=0.0, is_causal=False, scale=None,
         return_lse=False):
    """Exact scaled-dot-product attention forward on the GPU (PyTorch SDPA contract with GQA:
    q [B,Hq,Lq,Dqk], k [B,Hkv,Lk,Dqk], v [B,Hkv,Lk,Dv]; bool mask = keep, float mask = added
    to the scaled scores; is_causal is top-left aligned)."""
    lib = _lib.load()
    out = torch.empty(q.shape[:3] + (v.shape[3],), dtype=q.dtype, device=q.device)
    lse = None
    if return_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    dq, dk, dv, dm, do = describe(q), describe(k), describe(v), describe(attn_mask), describe(out)
    lse_ptr = ctypes.cast(lse.data_ptr(), ctypes.POINTER(ctypes.c_float)) if lse is not None and lse.numel() else None
    check(lib.wf_sdpa_fwd(_ref(dq), _ref(dk), _ref(dv), _ref(dm), int(bool(is_causal)),
                          float(dropout_p), _scale(scale), _ref(do), lse_ptr, _stream(q)))
    return (out, lse) if return_lse else out


def flattened_sdpa(q, k, v, num_heads, num_kv_heads=None, attn_mask=None, is_causal=False,
                   scale=None):
    """Attention on (batch, sequence, hidden) activations that only lack the head split
    (WorldFoundry "Core 注意力", section "选择最窄的入口": the flattened multi-head entry):
    q [B, Sq, Hq*D], k [B, Sk, Hkv*D], v [B, Sk, Hkv*Dv] -> out [B, Sq, Hq*Dv]. The heads are
    split out by strides and the kernels write the output in place in the flattened layout
    (no copies); semantics as sdpa()."""
    kvh = num_heads if num_kv_heads is None else int(num_kv_heads)
    B, Sq, Sk = q.shape[0], q.shape[1], k.shape[1]
    qv = q.view(B, Sq, num_heads, -1).transpose(1, 2)
    kv = k.view(B, Sk, kvh, -1).transpose(1, 2)
    vv = v.view(B, Sk, kvh, -1).transpose(1, 2)
    out = torch.empty((B, Sq, num_heads, vv.shape[3]), dtype=q.dtype, device=q.device)
    lib = _lib.load()
    dq, dk, dv, dm = describe(qv), describe(kv), describe(vv), describe(attn_mask)
    do = describe(out.transpose(1, 2))
    check(lib.wf_sdpa_fwd(_ref(dq), _ref(dk), _ref(dv), _ref(dm), int(bool(is_causal)), 0.0,
                          _scale(scale), _ref(do), None, _stream(q)))
    return out.view(B, Sq, -1)


def sdpa_rope(q, k, v, cos, sin, rot_dim=None, style=0, q_pos0=0, k_pos0=0, attn_mask=None,
              is_causal=False, scale=None, return_lse=False, workspace=None):
    """sdpa() with rotary position embedding on q and k: cos/sin fp32 [max_pos, rot_dim/2]
    device tables (pair i of a row at position p turns by cos[p, i], sin[p, i]); style 0 pairs
    (i, i + rot_dim/2), style 1 pairs (2i, 2i + 1); query row r sits at q_pos0 + r, key row j at
    k_pos0 + j. rot_dim defaults to 2 * cos.shape[1]."""
    lib = _lib.load()
    cos, sin = cos.contiguous(), sin.contiguous()
    rot = 2 * cos.shape[1] if rot_dim is None else int(rot_dim)
    out = torch.empty(q.shape[:3] + (v.shape[3],), dtype=q.dtype, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    dq, dk, dv, dm, do = describe(q), describe(k), describe(v), describe(attn_mask), describe(out)
    need = int(lib.wf_sdpa_rope_workspace_size(_ref(dq), _ref(dk)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    r = _lib.WfRope(cos.data_ptr(), sin.data_ptr(), cos.shape[0], rot, int(style), int(q_pos0),
                    int(k_pos0))
    lse_ptr = ctypes.cast(lse.data_ptr(), ctypes.POINTER(ctypes.c_float)) if lse is not None and lse.numel() else None
    check(lib.wf_sdpa_rope_fwd(_ref(dq), _ref(dk), _ref(dv), _ref(dm), int(bool(is_causal)),
                               _scale(scale), ctypes.byref(r), _ref(do), lse_ptr,
                               ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(q)))
    return (out, lse) if return_lse else out


def sdpa_decode_workspace_size(q, k, v, is_causal=False):
    return int(_lib.load().wf_sdpa_decode_workspace_size(_ref(describe(q)), _ref(describe(k)),
                                                         _ref(describe(v)), int(bool(is_causal))))


def sdpa_decode(q, k, v, is_causal=False, scale=None, return_lse=False, workspace=None):
    """Attention of few queries over a long K/V, split over the keys (decode; speculative
    decoding when Lq > 1): q [B,Hq,Lq,D], k/v [B,Hkv,Lk,D], D in {64, 128}, 16-bit. is_causal
    puts the queries at the end of the key sequence (bottom-right). No mask."""
    lib = _lib.load()
    out = torch.empty(q.shape[:3] + (v.shape[3],), dtype=q.dtype, device=q.device)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if return_lse else None
    need = sdpa_decode_workspace_size(q, k, v, is_causal)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    dq, dk, dv, do = describe(q), describe(k), describe(v), describe(out)
    lse_ptr = ctypes.cast(lse.data_ptr(), ctypes.POINTER(ctypes.c_float)) if lse is not None and lse.numel() else None
    check(lib.wf_sdpa_decode(_ref(dq), _ref(dk), _ref(dv), int(bool(is_causal)), _scale(scale),
                             _ref(do), lse_ptr, ctypes.c_void_p(workspace.data_ptr()),
                             workspace.numel(), _stream(q)))
    return (out, lse) if return_lse else out


def varlen_mla_prefill_workspace_size(batch, total_q_tokens, head_num):
    return int(_lib.load().wf_varlen_mla_prefill_workspace_size(int(batch), int(total_q_tokens),
                                                                int(head_num)))


def _mla_kv(k, k_rope, v, kv_head_num, kv_layout):
    if kv_layout == "padded":
        return tuple(t if t.dim() == 4 else t.view(t.shape[0], t.shape[1], int(kv_head_num), -1)
                     for t in (k, k_rope, v))
    if kv_layout != "packed":
        raise ValueError("kv_layout must be 'packed' or 'padded'")
    return k, k_rope, v


def varlen_mla_prefill(q, q_rope, k, k_rope, v, q_seqlen, kv_seqlen, head_num, kv_head_num,
                       qk_scale, mask_type=1, workspace=None, kv_layout="packed", check_lengths=None):
    """Varlen MLA prefill: q [nTq,Hq,128], q_rope [nTq,Hq,64], device int32 lengths [batch];
    mask_type 0 = none, 1 = causal (bottom-right). K/V come packed (kv_layout "packed":
    k/v [nTk,Hkv,128], k_rope [nTk,Hkv,64]) or padded per sequence (kv_layout "padded":
    k/v [batch,max_seq,Hkv*128] or [batch,max_seq,Hkv,128], k_rope likewise with 64).
    Returns out [nTq, Hq, 128].

    The lengths live on the device, so the library checks them there: bad lengths (negative,
    summing past nTq or nTk, longer than max_seq) compute nothing and set int32 word 2 of the
    workspace to 1. With check_lengths (the default when no workspace is passed, since the
    word would otherwise be lost with the temporary workspace) the call waits for the stream
    and raises WfError on that word; with a caller's workspace and check_lengths False the
    call stays asynchronous and the caller reads the word."""
    lib = _lib.load()
    batch = int(q_seqlen.numel())
    k, k_rope, v = _mla_kv(k, k_rope, v, kv_head_num, kv_layout)
    n_q = q.shape[0]
    out = torch.empty((n_q, head_num, v.shape[-1]), dtype=q.dtype, device=q.device)
    need = varlen_mla_prefill_workspace_size(batch, n_q, head_num)
    if check_lengths is None:
        check_lengths = workspace is None
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    ds = [describe(t) for t in (q, q_rope, k, k_rope, v, out)]
    check(lib.wf_varlen_mla_prefill(_ref(ds[0]), _ref(ds[1]), _ref(ds[2]), _ref(ds[3]), _ref(ds[4]),
                                    ctypes.c_void_p(q_seqlen.data_ptr()),
                                    ctypes.c_void_p(kv_seqlen.data_ptr()), batch, int(head_num),
                                    int(kv_head_num), _scale(qk_scale), int(mask_type),
                                    _ref(ds[5]), ctypes.c_void_p(workspace.data_ptr()),
                                    workspace.numel(), _stream(q)))
    if check_lengths and batch > 0 and n_q > 0:
        if int(workspace[8:12].view(torch.int32).item()) != 0:     # .item() waits for the stream
            raise _lib.WfError(_lib.ERR_SHAPE, "varlen_mla_prefill: device sequence lengths are "
                               "negative, sum past the token counts or exceed max_seq; nothing "
                               "was computed")
    return out


def varlen_mla_prefill_noalloc(q, q_rope, k, k_rope, v, q_seqlen, kv_seqlen, head_num, kv_head_num,
                               qk_scale, out, mask_type=1, kv_layout="packed"):
    """varlen_mla_prefill into a caller's `out` [nTq, Hq, 128] with the library's fixed 1 MiB
    device workspace: nothing is allocated, so the call can sit in a HIP graph capture or a
    serving loop that must not allocate. Calls on one device share that workspace and must
    not overlap. Bad device lengths compute nothing and are not reported. Returns out."""
    lib = _lib.load()
    batch = int(q_seqlen.numel())
    k, k_rope, v = _mla_kv(k, k_rope, v, kv_head_num, kv_layout)
    ds = [describe(t) for t in (q, q_rope, k, k_rope, v, out)]
    check(lib.wf_varlen_mla_prefill_noalloc(_ref(ds[0]), _ref(ds[1]), _ref(ds[2]), _ref(ds[3]),
                                            _ref(ds[4]), ctypes.c_void_p(q_seqlen.data_ptr()),
                                            ctypes.c_void_p(kv_seqlen.data_ptr()), batch,
                                            int(head_num), int(kv_head_num), _scale(qk_scale),
                                            int(mask_type), _ref(ds[5]), _stream(q)))
    return out


class BlockKVCache:
    """Rolling sink + window KV cache (WorldFoundry "Core 注意力", "Block KV cache 的调用顺序").

    Each chunk follows before_update(i) -> update(k, v) -> cached_k()/cached_v() ->
    after_update(i); i must repeat the current chunk (overwrite) or be the next one.
    The cache tensors live on `device`; the index bookkeeping is the library's state.
    """

    def __init__(self, k_shape, v_shape, seq_dim, chunk_size, window_size, sink_size=0,
                 device="cuda", dtype=torch.float16):
        self.k_shape, self.v_shape = tuple(k_shape), tuple(v_shape)
        if len(self.k_shape) != 4 or len(self.v_shape) != 4 or seq_dim not in (1, 2):
            raise ValueError("4-d cache shapes with seq_dim 1 or 2 (head dim last)")
        self.seq_dim = seq_dim
        self.k = torch.zeros(self.k_shape, dtype=dtype, device=device)
        self.v = torch.zeros(self.v_shape, dtype=dtype, device=device)
        self.state = WfBlockKvState()
        check(_lib.load().wf_block_kv_init(ctypes.byref(self.state), self.k_shape[seq_dim],
                                           int(sink_size), int(window_size), int(chunk_size)))
        self._pending = None

    def _bhsd(self, t):  # view with the sequence axis third
        return t if self.seq_dim == 2 else t.transpose(1, 2)

    @property
    def last_chunk(self):
        return int(self.state.last_chunk)

    def before_update(self, chunk_idx):
        self._pending = int(chunk_idx)

    def update(self, k, v):
        if self._pending is None:
            raise RuntimeError("update() without before_update()")
        dk, dv = describe(self._bhsd(k)), describe(self._bhsd(v))
        dkc, dvc = describe(self._bhsd(self.k)), describe(self._bhsd(self.v))
        check(_lib.load().wf_block_kv_cache_update(ctypes.byref(self.state), self._pending,
                                                   _ref(dk), _ref(dv), _ref(dkc), _ref(dvc),
                                                   _stream(self.k)))

    def after_update(self, chunk_idx):
        if self._pending != int(chunk_idx):
            raise RuntimeError("after_update() index differs from before_update()")
        self._pending = None

    def snapshot(self):
        """A copy of the cache: the library state and both tensors (queued on k's stream)."""
        if self._pending is not None:
            raise RuntimeError("snapshot() between before_update() and after_update()")
        st = WfBlockKvState()
        ctypes.memmove(ctypes.byref(st), ctypes.byref(self.state), ctypes.sizeof(st))
        return st, self.k.clone(), self.v.clone()

    def restore(self, snap):
        """Return the cache to a snapshot taken from a cache of the same shapes and sizes."""
        st, k, v = snap
        if tuple(k.shape) != self.k_shape or tuple(v.shape) != self.v_shape:
            raise ValueError("snapshot shapes differ from this cache's")
        if (st.cache_len, st.sink, st.window, st.chunk) != (self.state.cache_len, self.state.sink,
                                                             self.state.window, self.state.chunk):
            raise ValueError("snapshot sizes differ from this cache's")
        self.k.copy_(k)
        self.v.copy_(v)
        ctypes.memmove(ctypes.byref(self.state), ctypes.byref(st), ctypes.sizeof(st))
        self._pending = None

    def n_visible(self):
        """Number of visible cached tokens (the library's count, without the slot list)."""
        n = ctypes.c_int64()
        check(_lib.load().wf_block_kv_visible(ctypes.byref(self.state), ctypes.byref(n), None))
        return n.value

    def visible(self):
        """(n_visible, slot of each visible token in chronological order) from the library."""
        lib = _lib.load()
        n = ctypes.c_int64()
        check(lib.wf_block_kv_visible(ctypes.byref(self.state), ctypes.byref(n), None))
        idx = (ctypes.c_int64 * max(1, n.value))()
        check(lib.wf_block_kv_visible(ctypes.byref(self.state), ctypes.byref(n), idx))
        return n.value, list(idx)[:n.value]

    def _gather(self, cache):
        n, _ = self.visible()
        shape = list(self._bhsd(cache).shape)
        shape[2] = n
        out = torch.empty(shape, dtype=cache.dtype, device=cache.device)
        check(_lib.load().wf_block_kv_gather(ctypes.byref(self.state), _ref(describe(self._bhsd(cache))),
                                             _ref(describe(out)), _stream(cache)))
        return out if self.seq_dim == 2 else out.transpose(1, 2)

    def cached_k(self):
        return self._gather(self.k)

    def cached_v(self):
        return self._gather(self.v)

    def update_attend(self, k, v, q, scale=None, workspace=None, is_causal=False):
        """update(k, v) then attend(q) in one attention launch (between before_update and
        after_update, like update); returns the attend's output."""
        if self._pending is None:
            raise RuntimeError("update_attend() without before_update()")
        lib = _lib.load()
        kc, vc = self._bhsd(self.k), self._bhsd(self.v)
        B, Hq, Lq = q.shape[:3]
        out = torch.empty((B, Hq, Lq, vc.shape[3]), dtype=q.dtype, device=q.device)
        need = int(lib.wf_block_kv_attend_workspace_size(ctypes.byref(self.state), B, Hq, Lq,
                                                         vc.shape[3]))
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
        check(lib.wf_block_kv_update_attend(
            ctypes.byref(self.state), self._pending, _ref(describe(self._bhsd(k))),
            _ref(describe(self._bhsd(v))), _ref(describe(kc)), _ref(describe(vc)), _ref(describe(q)),
            1 if is_causal else 0, _scale(scale), _ref(describe(out)),
            ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(q)))
        return out

    def attend(self, q, scale=None, workspace=None, is_causal=False):
        """Attention of q [B,Hq,Lq,D] over every visible cached token, in chronological order;
        is_causal: the queries are the last Lq visible tokens (bottom-right causal)."""
        lib = _lib.load()
        kc, vc = self._bhsd(self.k), self._bhsd(self.v)
        B, Hq, Lq = q.shape[:3]
        Dv = vc.shape[3]
        out = torch.empty((B, Hq, Lq, Dv), dtype=q.dtype, device=q.device)
        need = int(lib.wf_block_kv_attend_workspace_size(ctypes.byref(self.state), B, Hq, Lq, Dv))
        if workspace is None:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
        check(lib.wf_block_kv_attend(ctypes.byref(self.state), _ref(describe(q)), _ref(describe(kc)),
                                     _ref(describe(vc)), 1 if is_causal else 0, _scale(scale),
                                     _ref(describe(out)),
                                     ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                     _stream(q)))
        return out
