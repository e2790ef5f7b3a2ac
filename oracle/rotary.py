"""Rotary position embedding applied to attention queries and keys, then exact attention.

TEST INFRASTRUCTURE ONLY: imported by tests, never by the product path.

Source: WorldFoundry "Core 注意力" (core attention), the opening responsibility list: the core
applies RoPE before attention. The pages give no convention, so these are readings (listed
in the design notes):
  * the rotation acts on the first rot_dim dimensions of every head (rot_dim even); the rest
    pass through unchanged;
  * style 0, "rotate-half": dimension i pairs with i + rot_dim/2 (i < rot_dim/2);
    style 1, "interleaved": dimension 2i pairs with 2i + 1;
  * pair i at position p turns by the angle whose cosine and sine the caller tabulates as
    cos[p, i] and sin[p, i] (so any frequency schedule can be used):
        (x_a, x_b) -> (x_a cos - x_b sin,  x_b cos + x_a sin);
  * query row r sits at position q_pos0 + r and key row j at k_pos0 + j.

Parity pins (tests/test_oracle.py): a 2-d rotation on a single pair, norm preservation, the
relative-position property (scores depend only on the distance when the tables come from
angles p * theta_i), rot_dim = 0 is the identity, the two styles are one rotation under a
fixed permutation of dimensions, and sdpa_rope = sdpa of the rotated inputs.
"""
from __future__ import annotations

import numpy as np

from .attention import _f64, sdpa

ROTATE_HALF = 0
INTERLEAVED = 1


def rope_pairs(rot_dim, style):
    """Index arrays (a, b) of the rotated pairs: pair i is (a[i], b[i])."""
    h = rot_dim // 2
    if style == ROTATE_HALF:
        return np.arange(h), np.arange(h) + h
    if style == INTERLEAVED:
        return 2 * np.arange(h), 2 * np.arange(h) + 1
    raise ValueError("style must be 0 (rotate-half) or 1 (interleaved)")


def rope(x, cos, sin, rot_dim, style=ROTATE_HALF, pos0=0):
    """x [..., L, D]; cos, sin [max_pos, rot_dim/2]. Returns the rotated x as float64."""
    x = _f64(x).copy()
    cos, sin = _f64(cos), _f64(sin)
    L, D = x.shape[-2], x.shape[-1]
    if rot_dim % 2 or rot_dim > D or rot_dim < 0:
        raise ValueError("rot_dim must be even and at most the head dim")
    if rot_dim == 0:
        return x
    if pos0 < 0 or pos0 + L > cos.shape[0]:
        raise ValueError("positions past the cos/sin tables")
    a, b = rope_pairs(rot_dim, style)
    c = cos[pos0:pos0 + L, :rot_dim // 2]   # [L, rot/2], broadcast over leading dims
    s = sin[pos0:pos0 + L, :rot_dim // 2]
    xa, xb = x[..., a].copy(), x[..., b].copy()
    x[..., a] = xa * c - xb * s
    x[..., b] = xb * c + xa * s
    return x


def sdpa_rope(q, k, v, cos, sin, rot_dim, style=ROTATE_HALF, q_pos0=0, k_pos0=0, mask=None,
              is_causal=False, scale=None):
    """Exact attention of the rotated queries and keys (values unrotated)."""
    return sdpa(rope(q, cos, sin, rot_dim, style, q_pos0), rope(k, cos, sin, rot_dim, style, k_pos0),
                v, mask=mask, is_causal=is_causal, scale=scale)
