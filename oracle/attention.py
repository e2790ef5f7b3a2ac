"""Exact softmax attention, written out as its definition in fp64 (numpy).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the benchmark's CPU
baseline, never by the product path. No blocking, fusion or reordering beyond the plain
definition: a row block of queries only bounds memory; every score row is materialised
whole before its softmax.

Definition followed (WorldFoundry "Core 注意力", section "选择最窄的入口": the PyTorch
SDPA contract with GQA expansion and an exact matmul path; the sentence after the CPU/GPU
example: a bool mask marks the scores that are kept, a float mask is added to the score
matrix; Ascend "MLA Prefill" parameter table: qkScale multiplies Q*K^T, the score of MLA is
the value-width part plus the 64-wide rotary part, packed sequences by qSeqLen/kvSeqLen):

    g       = h // (Hq / Hkv)                                  (GQA head grouping)
    s_ij    = scale * <q_i, k_j>  (+ <qRope_i, kRope_j> for MLA)  (+ fmask_ij)
    keep_ij = bmask_ij  and  causal_ok(i, j)
    s_ij    = -inf where not keep_ij
    out_i   = sum_j exp(s_ij - M_i) v_j / sum_j exp(s_ij - M_i),  M_i = max_j s_ij
    lse_i   = M_i + log(sum_j exp(s_ij - M_i))

Readings where the pages are silent (each is listed in the design notes):
  * scale default 1/sqrt(Dqk); float mask is added after the scale.
  * causal alignment: "top_left" keeps j <= i (PyTorch SDPA contract); "bottom_right"
    keeps j <= i + (Lk - Lq) (prefill: extra keys are earlier context).
  * a row with no kept score gives out = 0 and lse = -inf.
  * mask_type for MLA prefill: 0 = no mask (UNDEFINED, an all-zero mask), 1 = causal.

Parity pins (tests/test_oracle.py): torch's CPU fp64 scaled_dot_product_attention
(library routine), closed forms (single key -> that V row; zero keys -> mean of V),
invariants (kept-all bool mask = no mask, bool = float where(M,0,-inf), causal = float
triangle, per-row constant shift, scale folding, key permutation, GQA = repeated heads),
MLA = SDPA on concatenated [q|qRope],[k|kRope] per sequence, packing invariance,
padded K/V = the same rows packed.
"""
from __future__ import annotations

import math

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1


def _heads(x, H, lead):
    """[*lead axes, H*d] or [*lead axes, H, d] -> [*lead axes, H, d]. The head width is
    computed rather than inferred, so a tensor with no tokens keeps its shape too."""
    if x.ndim == lead + 1:
        return x.reshape(x.shape[:lead] + (H, x.shape[lead] // H))
    return x.reshape(x.shape[:lead] + (H, x.shape[-1]))


def _f64(x):
    """Exact upcast of a torch tensor or array to a float64 numpy array."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor; plain CPU ops only
        x = x.detach().cpu()
        if x.dtype.is_floating_point:
            x = x.double()
        return x.numpy()
    x = np.asarray(x)
    return x.astype(np.float64) if np.issubdtype(x.dtype, np.floating) else x


def _softmax_rows(s, vg):
    """out, lse for one block of fully materialised score rows s [r, Lk] and values vg [Lk, Dv]."""
    out = np.zeros((s.shape[0], vg.shape[1]), dtype=np.float64)
    lse = np.full(s.shape[0], -np.inf, dtype=np.float64)
    if s.shape[1] == 0:  # no keys at all: every row is fully masked
        return out, lse
    m = s.max(axis=1)
    live = np.isfinite(m)
    if live.any():
        sl = s[live]
        p = np.exp(sl - m[live][:, None])
        den = p.sum(axis=1)
        out[live] = (p @ vg) / den[:, None]
        lse[live] = m[live] + np.log(den)
    return out, lse


def sdpa(q, k, v, mask=None, is_causal=False, scale=None, causal_align="top_left",
         row_block=512):
    """Exact attention forward under the PyTorch SDPA contract.

    q [B,Hq,Lq,Dqk], k [B,Hkv,Lk,Dqk], v [B,Hkv,Lk,Dv]; mask None or broadcastable to
    [B,Hq,Lq,Lk], bool (True = keep) or float (added to the scaled score).
    Returns (out [B,Hq,Lq,Dv], lse [B,Hq,Lq]) as float64 arrays.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Lq, Dqk = q.shape
    Bk, Hkv, Lk, Dk = k.shape
    if v.shape[:3] != (Bk, Hkv, Lk) or Bk != B or Dk != Dqk:
        raise ValueError("q/k/v shapes disagree")
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if mask is not None and is_causal:
        raise ValueError("mask and is_causal together are not accepted")
    G = Hq // Hkv
    Dv = v.shape[3]
    scale = 1.0 / math.sqrt(Dqk) if scale is None else float(scale)
    bmask = fmask = None
    if mask is not None:
        m = _f64(mask)
        if m.dtype == np.bool_:
            bmask = np.broadcast_to(m, (B, Hq, Lq, Lk))
        else:
            fmask = np.broadcast_to(m.astype(np.float64), (B, Hq, Lq, Lk))
    shift = 0 if causal_align == "top_left" else Lk - Lq
    out = np.zeros((B, Hq, Lq, Dv), dtype=np.float64)
    lse = np.full((B, Hq, Lq), -np.inf, dtype=np.float64)
    jj = np.arange(Lk)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            kg, vg = k[b, g], v[b, g]
            for r0 in range(0, Lq, row_block):
                r1 = min(Lq, r0 + row_block)
                s = scale * (q[b, h, r0:r1] @ kg.T)
                if fmask is not None:
                    s = s + fmask[b, h, r0:r1]
                keep = np.ones(s.shape, dtype=bool)
                if bmask is not None:
                    keep &= bmask[b, h, r0:r1]
                if is_causal:
                    ii = np.arange(r0, r1)[:, None]
                    keep &= jj[None, :] <= ii + shift
                s = np.where(keep, s, -np.inf)
                out[b, h, r0:r1], lse[b, h, r0:r1] = _softmax_rows(s, vg)
    return out, lse


def cu_seqlens(lengths):
    """Exclusive prefix sums [batch+1] of per-sequence lengths (packed token offsets)."""
    lengths = np.asarray(_f64(lengths), dtype=np.int64).reshape(-1)
    if (lengths < 0).any():
        raise ValueError("negative sequence length")
    return np.concatenate([[0], np.cumsum(lengths)])


def varlen_mla_prefill(q, q_rope, k, k_rope, v, q_seqlen, kv_seqlen, head_num,
                       kv_head_num, qk_scale, mask_type=MASK_NONE, row_block=512,
                       kv_layout="packed"):
    """MLA prefill over a packed batch (Ascend "MLA Prefill" parameter table).

    q [nTq, Hq*Dv] or [nTq, Hq, Dv]; q_rope [nTq, Hq*64] or [nTq, Hq, 64];
    q_seqlen, kv_seqlen int [batch]. The table gives K, kRope and V in two forms:
      kv_layout "packed": k, v [nTk, Hkv*Dv] or [nTk, Hkv, Dv], k_rope [nTk, Hkv*64] or
        [nTk, Hkv, 64]; sequence i owns the kv_seqlen[i] rows after those of sequences < i;
      kv_layout "padded": k, v [batch, max_seq, Hkv*Dv] or [batch, max_seq, Hkv, Dv],
        k_rope [batch, max_seq, Hkv*64] or [..., Hkv, 64]; sequence i owns rows
        [0, kv_seqlen[i]) of batch entry i.
    For sequence i the score is qk_scale * (q . k + qRope . kRope) over that sequence's
    own tokens only; mask_type 1 applies bottom-right causal masking.
    Returns out [nTq, Hq, Dv] as float64.
    """
    Hq, Hkv = int(head_num), int(kv_head_num)
    if Hkv == 0 or Hq % Hkv != 0:
        raise ValueError("headNum must be a multiple of kvHeadNum")
    if mask_type not in (MASK_NONE, MASK_CAUSAL):
        raise ValueError("mask_type must be 0 (none) or 1 (causal)")
    G = Hq // Hkv
    q = _heads(_f64(q), Hq, 1)
    qr = _heads(_f64(q_rope), Hq, 1)
    cq, ck = cu_seqlens(q_seqlen), cu_seqlens(kv_seqlen)
    if len(cq) != len(ck):
        raise ValueError("qSeqLen and kvSeqLen lengths differ")
    if kv_layout == "packed":
        k, kr, v = (_heads(_f64(t), Hkv, 1) for t in (k, k_rope, v))
        if ck[-1] > k.shape[0]:
            raise ValueError("sequence lengths exceed the packed token count")

        def kv_rows(i):  # sequence i's keys, rotary keys and values [lk, Hkv, d]
            return k[ck[i]:ck[i + 1]], kr[ck[i]:ck[i + 1]], v[ck[i]:ck[i + 1]]
    elif kv_layout == "padded":
        k, kr, v = (_heads(_f64(t), Hkv, 2) for t in (k, k_rope, v))
        if k.shape[0] != len(ck) - 1:
            raise ValueError("padded K/V need one batch entry per sequence")
        if len(ck) > 1 and np.diff(ck).max() > k.shape[1]:
            raise ValueError("a kv length exceeds max_seq")

        def kv_rows(i):
            lk_i = ck[i + 1] - ck[i]
            return k[i, :lk_i], kr[i, :lk_i], v[i, :lk_i]
    else:
        raise ValueError("kv_layout must be 'packed' or 'padded'")
    if cq[-1] > q.shape[0]:
        raise ValueError("sequence lengths exceed the packed token count")
    scale = float(qk_scale)
    out = np.zeros((q.shape[0], Hq, v.shape[-1]), dtype=np.float64)
    for i in range(len(cq) - 1):
        lq, lk = cq[i + 1] - cq[i], ck[i + 1] - ck[i]
        if lq == 0:
            continue
        jj = np.arange(lk)
        ki, kri, vi = kv_rows(i)
        for h in range(Hq):
            g = h // G
            kg, krg, vg = ki[:, g], kri[:, g], vi[:, g]
            for r0 in range(0, lq, row_block):
                r1 = min(lq, r0 + row_block)
                rows = slice(cq[i] + r0, cq[i] + r1)
                s = scale * (q[rows, h] @ kg.T + qr[rows, h] @ krg.T)
                if mask_type == MASK_CAUSAL:
                    ii = np.arange(r0, r1)[:, None]
                    s = np.where(jj[None, :] <= ii + (lk - lq), s, -np.inf)
                out[rows, h], _ = _softmax_rows(s, vg)
    return out
