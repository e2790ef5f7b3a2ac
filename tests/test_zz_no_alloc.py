"""wf_varlen_mla_prefill_noalloc (fixed in-library workspace) against wf_varlen_mla_prefill with a
caller's workspace: two calls in a row through the C ABI, the second on a smaller input, so the
second call runs on scratch the first one left behind."""
import ctypes

import pytest
import torch

from exact_attention_forward_flash_amd import _lib, describe
from exact_attention_forward_flash_amd.api import _ref, _scale, _stream
from exact_attention_forward_flash_amd import varlen_mla_prefill_workspace_size

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(qlens, kvlens, H, Hkv, seed):
    g = torch.Generator().manual_seed(seed)
    nq, nk = sum(qlens), sum(kvlens)
    r = lambda *s: torch.randn(*s, generator=g).to(torch.bfloat16).to(DEV)
    return dict(q=r(nq, H, 128), q_rope=r(nq, H, 64), k=r(nk, Hkv, 128), k_rope=r(nk, Hkv, 64),
                v=r(nk, Hkv, 128), ql=torch.tensor(qlens, dtype=torch.int32, device=DEV),
                kl=torch.tensor(kvlens, dtype=torch.int32, device=DEV), H=H, Hkv=Hkv)


def _call(w, noalloc):
    lib = _lib.load()
    out = torch.full((w["q"].shape[0], w["H"], 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    ds = [describe(w[n]) for n in ("q", "q_rope", "k", "k_rope", "v")] + [describe(out)]
    args = [_ref(d) for d in ds[:5]] + [ctypes.c_void_p(w["ql"].data_ptr()),
                                         ctypes.c_void_p(w["kl"].data_ptr()), w["ql"].numel(),
                                         w["H"], w["Hkv"], _scale(192 ** -0.5), 1, _ref(ds[5])]
    if noalloc:
        _lib.check(lib.wf_varlen_mla_prefill_noalloc(*args, _stream(w["q"])))
        return out, None
    need = varlen_mla_prefill_workspace_size(w["ql"].numel(), w["q"].shape[0], w["H"])
    ws = torch.full((need,), 0x7f, dtype=torch.uint8, device=DEV)
    _lib.check(lib.wf_varlen_mla_prefill(*args, ctypes.c_void_p(ws.data_ptr()), need, _stream(w["q"])))
    return out, ws


def test_noalloc_matches_workspace_entry_point_twice():
    big = _inputs([700, 1, 1300, 256, 90], [900, 1, 1300, 300, 90], 4, 2, seed=11)
    small = _inputs([300, 64], [300, 100], 4, 2, seed=12)
    for w in (big, small):
        got, _ = _call(w, noalloc=True)
        ref, ws = _call(w, noalloc=False)
        torch.cuda.synchronize()
        assert int(ws.view(torch.int32)[2]) == 0
        assert torch.isfinite(ref.float()).all()
        # the same kernels on the same schedule: the outputs agree bit for bit
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), \
            f"max |diff| {(got.float() - ref.float()).abs().max().item()}"


def test_noalloc_rejects_a_call_beyond_its_scratch():
    w = _inputs([64], [64], 1, 1, seed=13)
    lib = _lib.load()
    big_q = torch.empty((0, 1, 128), dtype=torch.bfloat16, device=DEV)   # only the shape matters
    many = 200_000                                                        # sequences: > 1 MiB of items
    ql = torch.zeros(many, dtype=torch.int32, device=DEV)
    assert varlen_mla_prefill_workspace_size(many, 0, 1) > (1 << 20)
    out = torch.empty((0, 1, 128), dtype=torch.bfloat16, device=DEV)
    ds = [describe(t) for t in (big_q, w["q_rope"][:0], w["k"], w["k_rope"], w["v"], out)]
    rc = lib.wf_varlen_mla_prefill_noalloc(*[_ref(d) for d in ds[:5]], ctypes.c_void_p(ql.data_ptr()),
                                           ctypes.c_void_p(ql.data_ptr()), many, 1, 1,
                                           _scale(192 ** -0.5), 1, _ref(ds[5]), _stream(w["q"]))
    assert rc == 8, rc                                                    # WF_ERR_WORKSPACE
    assert "1 MiB" in lib.wf_last_error().decode() or "scratch" in lib.wf_last_error().decode()
