"""GPU parity of wf_varlen_mla_prefill (packed varlen, 128 + 64 score split) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from exact_attention_forward_flash_amd import varlen_mla_prefill, varlen_mla_prefill_workspace_size
from synth import varlen_mla_prefill_inputs
from tests.parity import assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _gpu(w, **kw):
    t = {n: w[n].to(DEV) for n in ("q", "q_rope", "k", "k_rope", "v", "q_seqlen", "kv_seqlen")}
    return varlen_mla_prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], t["q_seqlen"],
                              t["kv_seqlen"], w["head_num"], w["kv_head_num"], w["qk_scale"],
                              w["mask_type"], **kw)


def _inputs(qlens, kvlens, H, Hkv, dtype="bf16", seed=1, mask_type=1, dv=128):
    g = torch.Generator().manual_seed(seed)
    nq, nk = sum(qlens), sum(kvlens)
    dt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]
    r = lambda *s: torch.randn(*s, generator=g).to(dt)
    return {"q": r(nq, H, dv), "q_rope": r(nq, H, 64), "k": r(nk, Hkv, dv),
            "k_rope": r(nk, Hkv, 64), "v": r(nk, Hkv, dv),
            "q_seqlen": torch.tensor(qlens, dtype=torch.int32),
            "kv_seqlen": torch.tensor(kvlens, dtype=torch.int32),
            "head_num": H, "kv_head_num": Hkv, "qk_scale": 1.0 / np.sqrt(dv + 64.0),
            "mask_type": mask_type}


def _oracle(w):
    return oracle.varlen_mla_prefill(w["q"], w["q_rope"], w["k"], w["k_rope"], w["v"],
                                     w["q_seqlen"], w["kv_seqlen"], w["head_num"],
                                     w["kv_head_num"], np.float32(w["qk_scale"]), w["mask_type"])


CASES = [  # q lengths, kv lengths, H, Hkv, dtype, mask_type, value width
    ([1, 63, 64, 65, 300, 0, 777], None, 4, 4, "bf16", 1, 128),
    ([1, 63, 64, 65, 300, 0, 777], None, 4, 4, "bf16", 0, 128),
    ([200, 31, 513], [260, 31, 600], 4, 2, "bf16", 1, 128),   # cached prefix: kv_len > q_len
    ([257, 1000], None, 2, 1, "fp16", 1, 128),
    ([90, 5], [40, 5], 2, 2, "fp16", 1, 128),                  # kv_len < q_len: early rows see nothing
    # four / two query heads of a KV head share each K/V tile
    ([1, 63, 64, 65, 300, 0, 777], None, 8, 2, "bf16", 1, 128),
    ([200, 31, 513], [260, 31, 600], 16, 4, "fp16", 1, 128),
    ([129, 700], [129, 900], 6, 3, "bf16", 0, 128),
    ([64, 1, 500], None, 16, 1, "bf16", 1, 128),
    # value width 64 (score width 128)
    ([1, 63, 64, 65, 300, 0, 777], None, 4, 4, "bf16", 1, 64),
    ([200, 31, 513], [260, 31, 600], 8, 2, "fp16", 1, 64),
    ([257, 1000], None, 6, 3, "bf16", 0, 64),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_varlen_small(case):
    qlens, kvlens, H, Hkv, dt, mt, dv = case
    w = _inputs(qlens, kvlens or qlens, H, Hkv, dt, mask_type=mt, dv=dv)
    out = _gpu(w)
    assert tuple(out.shape) == (sum(qlens), H, dv)
    assert_close(out, _oracle(w), w["q"].dtype, str(case))


def test_head_groups_match_one_head_per_group():
    """The kernel sharing K/V tiles among four query heads gives what the one-head-per-group
    kernel gives (both against the oracle, and within a few output ulps of each other)."""
    from exact_attention_forward_flash_amd import tune
    w = _inputs([300, 1000, 77], [300, 1000, 77], 16, 4, "bf16", seed=9)
    ref = _oracle(w)
    shared = _gpu(w)
    with tune(hpw=1):
        single = _gpu(w)
    assert_close(shared, ref, torch.bfloat16, "HPW 4")
    assert_close(single, ref, torch.bfloat16, "HPW 1")
    assert (shared.float() - single.float()).abs().max().item() < 2e-2


def test_flat_layout_and_concatenated_cache():
    w = _inputs([100, 300], [100, 300], 4, 4, "bf16", seed=4)
    ref = _gpu(w)
    t = {n: w[n].to(DEV) for n in ("q", "q_rope", "k", "k_rope", "v", "q_seqlen", "kv_seqlen")}
    kcat = torch.cat([t["k"], t["k_rope"]], dim=-1)          # [nTk, Hkv, 192]: nope then rope
    out = varlen_mla_prefill(t["q"].reshape(400, -1), t["q_rope"].reshape(400, -1), kcat[..., :128],
                             kcat[..., 128:], t["v"], t["q_seqlen"], t["kv_seqlen"], 4, 4,
                             w["qk_scale"], 1)
    assert torch.equal(out, ref)


def _padded(w, max_seq, fill=float("nan")):
    """The packed K/V of w laid out padded per sequence [batch, max_seq, Hkv, d]; rows past a
    sequence's kv length hold `fill` (NaN: any read of them would reach the output)."""
    kvl = w["kv_seqlen"].tolist()
    cu = np.concatenate([[0], np.cumsum(kvl)])
    out = {}
    for n in ("k", "k_rope", "v"):
        t = w[n]
        pad = torch.full((len(kvl), max_seq) + tuple(t.shape[1:]), fill, dtype=t.dtype)
        for i, lk in enumerate(kvl):
            pad[i, :lk] = t[cu[i]:cu[i + 1]]
        out[n] = pad
    return out


PADDED = [  # q lengths, kv lengths, max_seq, H, Hkv, dtype, mask_type
    ([1, 63, 300, 0, 777], [1, 63, 300, 0, 777], 800, 4, 4, "bf16", 1),
    ([200, 31, 513], [260, 31, 600], 640, 4, 2, "bf16", 1),
    ([257, 100], [257, 90], 257, 2, 1, "fp16", 0),
]


@pytest.mark.parametrize("case", PADDED, ids=[str(c) for c in PADDED])
def test_padded_kv_layout(case):
    # [MLA] table: K/kRope/V may also come as [batch, max_seq, kv_head*d].
    qlens, kvlens, max_seq, H, Hkv, dt, mt = case
    w = _inputs(qlens, kvlens, H, Hkv, dt, seed=7, mask_type=mt)
    p = _padded(w, max_seq)
    t = {n: w[n].to(DEV) for n in ("q", "q_rope", "q_seqlen", "kv_seqlen")}
    pd = {n: p[n].to(DEV) for n in p}
    flat = {n: pd[n].reshape(len(kvlens), max_seq, -1) for n in pd}   # the page's 3-d form
    out = varlen_mla_prefill(t["q"], t["q_rope"], flat["k"], flat["k_rope"], flat["v"],
                             t["q_seqlen"], t["kv_seqlen"], H, Hkv, w["qk_scale"], mt,
                             kv_layout="padded")
    ref = oracle.varlen_mla_prefill(w["q"], w["q_rope"], p["k"], p["k_rope"], p["v"],
                                    w["q_seqlen"], w["kv_seqlen"], H, Hkv,
                                    np.float32(w["qk_scale"]), mt, kv_layout="padded")
    assert_close(out, ref, w["q"].dtype, str(case))
    # the same tokens packed give the same bits (same kernel, same order)
    assert torch.equal(out, _gpu(w))


def test_padded_kv_longer_than_max_seq_sets_the_error_word():
    w = _inputs([64, 64], [64, 64], 2, 2, "bf16", seed=8)
    p = _padded(w, 64, fill=0.0)
    t = {n: w[n].to(DEV) for n in ("q", "q_rope")}
    pd = {n: p[n].to(DEV) for n in p}
    long_kv = torch.tensor([64, 65], dtype=torch.int32, device=DEV)
    ql = torch.tensor([64, 64], dtype=torch.int32, device=DEV)
    ws = torch.zeros(varlen_mla_prefill_workspace_size(2, 128, 2), dtype=torch.uint8, device=DEV)
    varlen_mla_prefill(t["q"], t["q_rope"], pd["k"], pd["k_rope"], pd["v"], ql, long_kv, 2, 2,
                       w["qk_scale"], 1, workspace=ws, kv_layout="padded")
    torch.cuda.synchronize()
    assert int(ws.view(torch.int32)[2]) == 1


def test_bad_lengths_set_the_error_word_and_compute_nothing():
    w = _inputs([100, 300], [100, 300], 2, 2, "bf16", seed=5)
    t = {n: w[n].to(DEV) for n in ("q", "q_rope", "k", "k_rope", "v")}
    bad = torch.tensor([100, 301], dtype=torch.int32, device=DEV)    # sums past nTq
    ws = torch.zeros(varlen_mla_prefill_workspace_size(2, 400, 2), dtype=torch.uint8, device=DEV)
    from exact_attention_forward_flash_amd import api
    out = varlen_mla_prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], bad, bad, 2, 2,
                             w["qk_scale"], 1, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws.view(torch.int32)[2]) == 1
    neg = torch.tensor([100, -1], dtype=torch.int32, device=DEV)
    varlen_mla_prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], neg, neg, 2, 2,
                       w["qk_scale"], 1, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws.view(torch.int32)[2]) == 1
    good = t["q"].new_tensor([100, 300], dtype=torch.int32)
    varlen_mla_prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], good, good, 2, 2,
                       w["qk_scale"], 1, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws.view(torch.int32)[2]) == 0


def test_bad_lengths_without_a_workspace_raise():
    """With no workspace passed, the error word would go with the temporary workspace: the
    binding waits and raises instead of returning an output nothing was written to."""
    from exact_attention_forward_flash_amd import WfError
    w = _inputs([100, 300], [100, 300], 2, 2, "bf16", seed=5)
    t = {n: w[n].to(DEV) for n in ("q", "q_rope", "k", "k_rope", "v")}
    bad = torch.tensor([100, 301], dtype=torch.int32, device=DEV)
    with pytest.raises(WfError, match="lengths"):
        varlen_mla_prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], bad, bad, 2, 2,
                           w["qk_scale"], 1)
    good = torch.tensor([100, 300], dtype=torch.int32, device=DEV)
    out = varlen_mla_prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], good, good, 2, 2,
                             w["qk_scale"], 1)
    assert_close(out, _oracle(w), w["q"].dtype, "checked good call")


def test_deterministic():
    w = _inputs([700, 50, 1300], [700, 50, 1300], 4, 4, "bf16", seed=6)
    assert torch.equal(_gpu(w), _gpu(w))


@pytest.fixture(scope="module")
def mla_full_call():
    w = varlen_mla_prefill_inputs()
    return w, _gpu(w).cpu()


@pytest.mark.parametrize("part", range(4))
def test_varlen_mla_full_size_every_row(mla_full_call, part):
    """Every output row of the full-size varlen MLA call (16 sequences, 16 heads) against the
    oracle, sequences split over four parts by length rank so the parts cost about the same;
    rows in blocks of 512, each a bottom-right causal problem over the keys up to its last row."""
    w, out = mla_full_call
    lens = w["q_seqlen"].tolist()
    cu = oracle.cu_seqlens(lens)
    order = [int(i) for i in np.argsort(lens)[::-1]]          # longest first, dealt in a snake
    snake = [i % 4 if (i // 4) % 2 == 0 else 3 - i % 4 for i in range(len(order))]
    mine = [si for si, p in zip(order, snake) if p == part]
    errs = []
    for si in mine:
        L, base = lens[si], int(cu[si])
        for i0 in range(0, L, 512):
            i1 = min(L, i0 + 512)
            rows, keys = slice(base + i0, base + i1), slice(base, base + i1)
            ref = oracle.varlen_mla_prefill(
                w["q"][rows], w["q_rope"][rows], w["k"][keys], w["k_rope"][keys], w["v"][keys],
                [i1 - i0], [i1], 16, 16, np.float32(w["qk_scale"]), 1)
            errs.append((np.abs(to64(out[rows]) - ref), f"seq {si} rows {i0}:{i1}"))
    g = np.concatenate([e.reshape(-1) for e, _ in errs])
    mx, mean = float(g.max()), float(g.mean())
    worst = max(errs, key=lambda e: e[0].max())[1]
    msg = f"sequences {mine}: max abs err {mx:.3g} (at {worst}), mean abs err {mean:.3g}"
    assert np.isfinite(to64(out)).all()
    assert mx <= 2e-2 and mean <= 2e-3, msg
    print(msg)


def test_varlen_mla_full_size_sampled():
    """16 sequences with lengths uniform in [128, 8192] (seed 7), 16 heads, 128 + 64 score
    split, causal; rows sampled from the shortest, longest and a middle sequence."""
    w = varlen_mla_prefill_inputs()
    out = _gpu(w).cpu()
    assert torch.isfinite(out).all()
    lens = w["q_seqlen"].tolist()
    cu = oracle.cu_seqlens(lens)
    order = np.argsort(lens)
    for si in (order[0], order[len(order) // 2], order[-1]):
        L, base = lens[si], cu[si]
        for h in (0, 11):
            for i0, i1 in ((0, 32), (L // 2, L // 2 + 32), (L - 32, L)):
                i1 = min(i1, L)
                rows = slice(base + i0, base + i1)
                keys = slice(base, base + i1)
                ref = oracle.varlen_mla_prefill(
                    w["q"][rows, h:h + 1], w["q_rope"][rows, h:h + 1], w["k"][keys, h:h + 1],
                    w["k_rope"][keys, h:h + 1], w["v"][keys, h:h + 1], [i1 - i0], [i1], 1, 1,
                    np.float32(w["qk_scale"]), 1)
                assert_close(out[rows, h:h + 1], ref, torch.bfloat16, f"seq {si} head {h} rows {i0}:{i1}")
