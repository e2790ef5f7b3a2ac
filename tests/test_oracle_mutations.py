"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutation edits the oracle's source text (on the CPU, in a private module), swaps
the mutated functions into the pin tests of test_oracle.py and runs them; the mutation
counts as caught when some pin fails. This guards the pins themselves: a pin set that a
plausible slip (dropped term, wrong sign or index, wrong grouping) survives is too weak.
"""
import inspect
import types

import pytest

import oracle.attention as oa
import oracle.block_kv_cache as ob
import oracle.rotary as orope
from tests import test_oracle as pins

MUTATIONS = [
    ("attention", "g = h // G", "g = h % Hkv", "GQA head grouping"),
    ("attention", "s = s + fmask[b, h, r0:r1]", "s = s", "float mask term dropped"),
    ("attention", "keep &= jj[None, :] <= ii + shift", "keep &= jj[None, :] >= ii + shift", "causal sign"),
    ("attention", "s = scale * (q[b, h, r0:r1] @ kg.T)", "s = (q[b, h, r0:r1] @ kg.T)", "scale dropped"),
    ("attention", "shift = 0 if causal_align == \"top_left\" else Lk - Lq", "shift = 0", "bottom-right offset"),
    ("attention", "out[live] = (p @ vg) / den[:, None]", "out[live] = (p @ vg)", "softmax denominator"),
    ("attention", "lse[live] = m[live] + np.log(den)", "lse[live] = np.log(den)", "lse max term"),
    ("attention", "keep &= bmask[b, h, r0:r1]", "keep &= ~bmask[b, h, r0:r1]", "bool mask polarity"),
    ("attention", "+ qr[rows, h] @ krg.T", "", "rope term dropped"),
    ("attention", "ii + (lk - lq)", "ii", "MLA bottom-right offset"),
    ("attention", "v[ck[i]:ck[i + 1]]\n", "v[cq[i]:cq[i + 1]]\n", "value range of the wrong sequence side"),
    ("attention", "kg, krg, vg = ki[:, g], kri[:, g], vi[:, g]", "kg, krg, vg = ki[:, 0], kri[:, g], vi[:, g]", "MLA kv head fixed"),
    ("attention", "return k[i, :lk_i], kr[i, :lk_i], v[i, :lk_i]", "return k[0, :lk_i], kr[i, :lk_i], v[i, :lk_i]", "padded K of the wrong batch entry"),
    ("attention", "return k[i, :lk_i], kr[i, :lk_i], v[i, :lk_i]", "return k[i, :lk_i], kr[i, :lk_i], v[i, 1:lk_i + 1]", "padded V rows shifted"),
    ("rope", "x[..., b] = xb * c + xa * s", "x[..., b] = xb * c - xa * s", "rotation sign"),
    ("rope", "c = cos[pos0:pos0 + L, :rot_dim // 2]", "c = cos[0:L, :rot_dim // 2]", "cos position offset dropped"),
    ("rope", "return np.arange(h), np.arange(h) + h", "return np.arange(h), np.arange(h) + 1", "rotate-half pairing"),
    ("rope", "rope(k, cos, sin, rot_dim, style, k_pos0)", "rope(k, cos, sin, rot_dim, style, q_pos0)", "key positions"),
    ("block_kv_cache", "max(self.sink, T - self.window)", "max(0, T - self.window)", "window start ignores sink"),
    ("block_kv_cache", "(self.last_chunk, self.last_chunk + 1)", "(self.last_chunk, self.last_chunk + 1, self.last_chunk + 2)", "skip allowed"),
    ("block_kv_cache", "min(T, self.sink)", "min(T, self.sink + 1)", "sink length"),
    ("block_kv_cache", "if length % chunk_size != 0:", "if False:", "divisibility rule dropped"),
]


def _mutated_module(which, old, new):
    mod = {"attention": oa, "block_kv_cache": ob, "rope": orope}[which]
    src = inspect.getsource(mod).replace("from .attention import", "from oracle.attention import")
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new)
    m = types.ModuleType(f"mutant_{which}")
    m.__dict__["__name__"] = f"mutant_{which}"
    exec(compile(src, f"<mutant {which}>", "exec"), m.__dict__)
    return m


def _run_all_pins():
    """Run every pin test in test_oracle.py with its parametrizations; return failures."""
    failures = 0
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            calls = [{}]
        else:
            argnames, argvalues = marks[0].args[0], marks[0].args[1]
            names = [a.strip() for a in argnames.split(",")]
            calls = []
            for val in argvalues:
                vals = val if len(names) > 1 else (val,)
                calls.append(dict(zip(names, vals)))
        for kw in calls:
            try:
                fn(**kw)
            except (Exception, pytest.fail.Exception):
                failures += 1
    return failures


@pytest.mark.parametrize("which,old,new,what", MUTATIONS, ids=[m[3] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(monkeypatch, which, old, new, what):
    m = _mutated_module(which, old, new)
    if which == "attention":
        monkeypatch.setattr(pins, "sdpa", m.sdpa)
        monkeypatch.setattr(pins, "varlen_mla_prefill", m.varlen_mla_prefill)
    elif which == "rope":
        monkeypatch.setattr(pins, "rope", m.rope)
        monkeypatch.setattr(pins, "sdpa_rope", m.sdpa_rope)
    else:
        monkeypatch.setattr(pins, "BlockKVCacheOracle", m.BlockKVCacheOracle)
        monkeypatch.setattr(pins, "CacheOrderError", m.CacheOrderError)
        monkeypatch.setattr(pins, "CacheConfigError", m.CacheConfigError)
    assert _run_all_pins() > 0, f"no pin caught the planted mistake: {what}"


def test_unmutated_oracle_passes_every_pin():
    assert _run_all_pins() == 0
