"""GPU parity of wf_sdpa_fwd against the fp64 oracle (through the C ABI via the binding)."""
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
from exact_attention_forward_flash_amd import sdpa, tune, WfError
from synth import causal_gqa_prefill, masked_sdpa_inputs, page_example_fp32, random_sdpa_inputs
from tests.parity import assert_close, to64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run(w, **kw):
    q, k, v = (w[n].to(DEV) for n in ("q", "k", "v"))
    m = w.get("mask")
    return sdpa(q, k, v, attn_mask=None if m is None else m.to(DEV), scale=w["scale"], **kw)


def test_page_example_fp32():
    w = page_example_fp32()
    out = run(w)
    assert tuple(out.shape) == (2, 8, 32, 96)
    ref, _ = oracle.sdpa(w["q"], w["k"], w["v"], scale=np.float32(w["scale"]))
    assert_close(out, ref, torch.float32, "page example")


CASES = [  # dtype, B, Hq, Hkv, Lq, Lk, D, causal
    ("bf16", 1, 1, 1, 1, 1, 128, False),
    ("bf16", 2, 4, 4, 37, 300, 128, False),
    ("bf16", 2, 8, 2, 256, 256, 128, True),
    ("bf16", 1, 8, 2, 300, 129, 128, False),
    ("bf16", 1, 4, 1, 513, 700, 128, True),
    ("bf16", 2, 4, 2, 700, 513, 64, True),
    ("fp16", 2, 6, 3, 129, 1000, 64, False),
    ("fp16", 1, 8, 8, 1024, 1024, 128, True),
    ("fp16", 3, 2, 1, 77, 77, 64, True),
    ("bf16", 1, 16, 4, 96, 2049, 64, False),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_random_shapes(case):
    dt, B, Hq, Hkv, Lq, Lk, D, causal = case
    w = random_sdpa_inputs(B, Hq, Hkv, Lq, Lk, D, D, dt, seed=zlib.crc32(str(case).encode()) % 1000)
    ref, ref_lse = oracle.sdpa(w["q"], w["k"], w["v"], is_causal=causal, scale=np.float32(w["scale"]))
    out = run(w, is_causal=causal)
    assert_close(out, ref, w["q"].dtype, str(case) + " (no lse)")
    out, lse = run(w, is_causal=causal, return_lse=True)
    assert_close(out, ref, w["q"].dtype, str(case))
    live = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(to64(lse)), live)
    assert np.abs(to64(lse)[live] - ref_lse[live]).max() < 1e-3


@pytest.mark.parametrize("dt", [torch.bfloat16, torch.float16])
def test_page_example_16bit(dt):
    """The page's example (q/k width 64, v width 96) with its inputs rounded to 16 bits."""
    w = page_example_fp32()
    q, k, v = (w[n].to(dt) for n in ("q", "k", "v"))
    ref, ref_lse = oracle.sdpa(q, k, v, scale=np.float32(w["scale"]))
    out, lse = sdpa(q.to(DEV), k.to(DEV), v.to(DEV), scale=w["scale"], return_lse=True)
    assert tuple(out.shape) == (2, 8, 32, 96)
    assert_close(out, ref, dt, "page example, 16-bit")
    assert np.abs(to64(lse) - ref_lse).max() < 1e-3
    assert_close(sdpa(q.to(DEV), k.to(DEV), v.to(DEV), scale=w["scale"]), ref, dt, "no lse")


MIX_CASES = [  # dtype, B, Hq, Hkv, Lq, Lk, Dqk, Dv, causal, mask
    ("bf16", 2, 8, 8, 32, 48, 64, 96, False, None),
    ("fp16", 1, 8, 2, 300, 129, 64, 96, True, None),
    ("bf16", 2, 4, 1, 65, 700, 64, 96, False, "bool"),
    ("fp16", 1, 2, 2, 257, 257, 64, 96, False, "f32"),
    ("bf16", 1, 16, 4, 513, 513, 128, 64, True, None),
    ("fp16", 2, 6, 3, 129, 1000, 128, 64, False, None),
    ("bf16", 1, 2, 1, 1, 300, 128, 64, False, "half"),
    ("fp16", 3, 4, 4, 100, 0, 128, 64, False, None),
]


@pytest.mark.parametrize("case", MIX_CASES, ids=[str(c) for c in MIX_CASES])
def test_value_width_differs_from_key_width(case):
    dt, B, Hq, Hkv, Lq, Lk, Dqk, Dv, causal, mk = case
    w = random_sdpa_inputs(B, Hq, Hkv, Lq, Lk, Dqk, Dv, dt, seed=zlib.crc32(str(case).encode()) % 1000)
    g = torch.Generator().manual_seed(3)
    m = None
    if mk == "bool":
        m = torch.rand(B, 1, Lq, Lk, generator=g) < 0.85
    elif mk is not None:
        m = torch.randn(B, Hq, Lq, Lk, generator=g)
        m[torch.rand(m.shape, generator=g) < 0.1] = -float("inf")
        m = m.to(w["q"].dtype if mk == "half" else torch.float32)
    ref, ref_lse = oracle.sdpa(w["q"], w["k"], w["v"], mask=m, is_causal=causal,
                               scale=np.float32(w["scale"]))
    for lse in (False, True):
        res = sdpa(w["q"].to(DEV), w["k"].to(DEV), w["v"].to(DEV),
                   attn_mask=None if m is None else m.to(DEV), is_causal=causal,
                   scale=w["scale"], return_lse=lse)
        out = res[0] if lse else res
        assert tuple(out.shape) == (B, Hq, Lq, Dv)
        assert_close(out, ref, w["q"].dtype, f"{case} lse={lse}")
        if lse:
            live = np.isfinite(ref_lse)
            assert np.array_equal(np.isfinite(to64(res[1])), live)
            if live.any():
                assert np.abs(to64(res[1])[live] - ref_lse[live]).max() < 1e-3


F32_CASES = [(2, 4, 2, 33, 50, 64, 96, False), (1, 4, 4, 130, 70, 128, 128, True),
             (2, 2, 1, 64, 64, 64, 64, True), (1, 2, 2, 5, 300, 128, 64, False),
             # one 32-query tile per head over several key tiles: the key-split fp32 form
             (2, 4, 2, 32, 48, 64, 96, False), (1, 4, 4, 1, 200, 128, 128, True),
             (1, 2, 1, 17, 129, 64, 64, False), (2, 2, 2, 32, 1000, 128, 96, False),
             (1, 4, 2, 32, 33, 128, 128, True)]


@pytest.mark.parametrize("case", F32_CASES, ids=[str(c) for c in F32_CASES])
def test_fp32_shapes(case):
    B, Hq, Hkv, Lq, Lk, Dqk, Dv, causal = case
    w = random_sdpa_inputs(B, Hq, Hkv, Lq, Lk, Dqk, Dv, "fp32", seed=3)
    out = run(w, is_causal=causal)
    ref, _ = oracle.sdpa(w["q"], w["k"], w["v"], is_causal=causal, scale=np.float32(w["scale"]))
    assert_close(out, ref, torch.float32, str(case))


MASK_CASES = [  # dtype, mask kind, mask broadcast shape, Lq, Lk, D
    ("fp16", "bool", "b1", 200, 320, 64),
    ("bf16", "bool", "11", 64, 301, 128),     # Lk % 4 != 0: element-wise mask loads
    ("fp16", "bool", "bh", 130, 256, 64),
    ("fp16", "half", "b1", 256, 200, 64),
    ("bf16", "half", "bh", 90, 333, 128),
    ("bf16", "f32", "11", 128, 128, 128),
    ("fp32", "bool", "b1", 70, 90, 64),
    ("fp32", "f32", "bh", 33, 130, 128),
    ("fp32", "bool", "bh", 20, 200, 64),      # key-split fp32 form (Lq <= 32, several key tiles)
    ("fp32", "f32", "b1", 32, 97, 128),
]


def _mask(kind, bshape, B, H, Lq, Lk, dtype, g):
    shp = {"b1": (B, 1, Lq, Lk), "11": (1, 1, Lq, Lk), "bh": (B, H, Lq, Lk)}[bshape]
    keep = torch.rand(shp, generator=g) < 0.8
    keep[..., 0] = True
    if kind == "bool":
        return keep
    vals = torch.randn(shp, generator=g).masked_fill(~keep, float("-inf"))
    return vals.to(torch.float32 if kind == "f32" else dtype)


@pytest.mark.parametrize("case", MASK_CASES, ids=[str(c) for c in MASK_CASES])
def test_masks(case):
    dt, kind, bshape, Lq, Lk, D = case
    B, H = 2, 4
    w = random_sdpa_inputs(B, H, H, Lq, Lk, D, D, dt, seed=11)
    g = torch.Generator().manual_seed(12)
    w["mask"] = _mask(kind, bshape, B, H, Lq, Lk, w["q"].dtype, g)
    out = run(w)
    ref, _ = oracle.sdpa(w["q"], w["k"], w["v"], mask=w["mask"], scale=np.float32(w["scale"]))
    assert_close(out, ref, w["q"].dtype, str(case))


def test_fp32_key_split_lse_and_masked_rows():
    """The key-split fp32 form merges the partial (m, l, O) of its four waves: the lse, rows
    whose kept keys all fall in one wave's tiles, and rows with no kept key (output 0, lse
    -inf) against the oracle."""
    B, H, Lq, Lk, D = 2, 3, 24, 260, 64
    w = random_sdpa_inputs(B, H, H, Lq, Lk, D, D, "fp32", seed=21)
    g = torch.Generator().manual_seed(22)
    keep = torch.rand((B, H, Lq, Lk), generator=g) < 0.5
    keep[:, :, 3] = False                  # no kept key
    keep[:, :, 5] = False
    keep[:, :, 5, 40:60] = True            # kept keys only in the tile of the second wave
    keep[:, :, 7] = False
    keep[:, :, 7, 258] = True              # one kept key, in the last (partial) tile
    w["mask"] = keep
    out, lse = run(w, return_lse=True)
    ref, ref_lse = oracle.sdpa(w["q"], w["k"], w["v"], mask=keep, scale=np.float32(w["scale"]))
    assert_close(out, ref, torch.float32, "key-split fp32")
    live = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(to64(lse)), live)
    assert np.abs(to64(lse)[live] - ref_lse[live]).max() < 1e-4
    assert (to64(out)[:, :, 3] == 0).all() and (to64(out)[:, :, 5] != 0).any()


def test_fully_masked_rows_and_empty_keys():
    w = random_sdpa_inputs(1, 2, 2, 40, 70, 64, 64, "bf16", seed=5)
    m = torch.ones(1, 1, 40, 70, dtype=torch.bool)
    m[0, 0, 7] = False
    m[0, 0, 33] = False
    w["mask"] = m
    out, lse = run(w, return_lse=True)
    o = to64(out)
    assert np.all(o[:, :, 7] == 0) and np.all(o[:, :, 33] == 0)
    assert np.all(np.isneginf(to64(lse)[:, :, [7, 33]]))
    ref, _ = oracle.sdpa(w["q"], w["k"], w["v"], mask=m, scale=np.float32(w["scale"]))
    assert_close(out, ref, torch.bfloat16, "fully masked rows")
    out = run(w)  # without lse
    o = to64(out)
    assert np.all(o[:, :, 7] == 0) and np.all(o[:, :, 33] == 0)
    assert_close(out, ref, torch.bfloat16, "fully masked rows (no lse)")
    w0 = random_sdpa_inputs(1, 2, 2, 40, 0, 64, 64, "bf16", seed=6)
    out0 = run(w0)
    assert out0.shape == (1, 2, 40, 64) and torch.all(out0 == 0)


# Every kernel shape on every case, whatever the default choice for it: the persistent
# 64-query-wave kernel (one wave per SIMD, one work group per CU walking a list of work items;
# calls without a mask or lse, head dim 128, causal ones with four query heads per KV head),
# the persistent 32-query kernel (calls without a mask), and the one-item-per-group kernels
# with 64-query waves (one per SIMD, row sums over the 16-bit weights) and 32-query waves (two
# per SIMD). The shape is picked per call through the library's tuning overrides; a call a
# shape does not take falls through to the next one in that order.
SHAPE_CASES = [c + (m,) for c in CASES for m in (None,)] + [
    ("bf16", 2, 4, 4, 130, 301, 128, False, "bool"),
    ("fp16", 2, 4, 4, 97, 200, 64, False, "half"),
    ("bf16", 1, 4, 4, 64, 128, 128, False, "f32"),
]


def _pick_shape(shape):
    if shape == "q64p":
        return tune(q64=1, persist=-1, qpw=-1)
    if shape == "persistent":
        return tune(q64=0, persist=1, qpw=-1)
    return tune(q64=0, persist=0, qpw=int(shape))


@pytest.mark.parametrize("qpw", ["q64p", "persistent", 64, 32])
@pytest.mark.parametrize("case", SHAPE_CASES, ids=[str(c) for c in SHAPE_CASES])
def test_kernel_shapes(case, qpw):
    dt, B, Hq, Hkv, Lq, Lk, D, causal, mkind = case
    w = random_sdpa_inputs(B, Hq, Hkv, Lq, Lk, D, D, dt, seed=zlib.crc32(str(case).encode()) % 997)
    if mkind is not None:
        g = torch.Generator().manual_seed(21)
        w["mask"] = _mask(mkind, "b1", B, Hq, Lq, Lk, w["q"].dtype, g)
    ref, _ = oracle.sdpa(w["q"], w["k"], w["v"], mask=w.get("mask"), is_causal=causal,
                         scale=np.float32(w["scale"]))
    with _pick_shape(qpw):
        out = run(w, is_causal=causal)
    assert_close(out, ref, w["q"].dtype, f"{case} {qpw}")


# Calls with more work items than the GPU has CUs, so that the persistent kernel's work
# groups walk several items each: its K/V copies and Q loads then cross item (and KV-head)
# boundaries. Both work orders are covered: B*Hkv a multiple of 8 (each XCD keeps its KV
# groups) and not.
PERSIST_CASES = [  # dtype, B, Hq, Hkv, Lq, Lk, D, causal
    ("bf16", 2, 32, 8, 1100, 1100, 64, True),     # 18 q-tiles x 16 KV groups, XCD order
    ("fp16", 3, 16, 4, 1500, 1500, 64, True),     # 24 x 12, plain order
    ("bf16", 4, 16, 16, 1100, 300, 128, False),   # HPW 1: 5 q-tiles x 64 groups
    ("fp16", 3, 16, 8, 1300, 777, 128, False),    # HPW 2: 11 x 24
    ("bf16", 2, 32, 8, 777, 2100, 128, True),     # causal with Lq < Lk (top-left)
]


@pytest.mark.parametrize("kernel", ["q64p", "persistent"])
@pytest.mark.parametrize("case", PERSIST_CASES, ids=[str(c) for c in PERSIST_CASES])
def test_persistent_many_items(case, kernel):
    dt, B, Hq, Hkv, Lq, Lk, D, causal = case
    w = random_sdpa_inputs(B, Hq, Hkv, Lq, Lk, D, D, dt, seed=zlib.crc32(str(case).encode()) % 991)
    ref, ref_lse = oracle.sdpa(w["q"], w["k"], w["v"], is_causal=causal, scale=np.float32(w["scale"]))
    with _pick_shape(kernel):
        out, lse = run(w, is_causal=causal, return_lse=True)   # persistent 32-query, fp32 row sums
        assert_close(out, ref, w["q"].dtype, str(case))
        assert np.abs(to64(lse) - ref_lse).max() < 1e-3
        out16 = run(w, is_causal=causal)   # Q pre-scaled; 64-query waves where they apply
    assert_close(out16, ref, w["q"].dtype, f"{case} {kernel} (no lse)")


def test_deterministic():
    w = random_sdpa_inputs(2, 8, 2, 300, 500, 128, 128, "bf16", seed=9)
    a = run(w, is_causal=True)
    b = run(w, is_causal=True)
    assert torch.equal(a, b)


def test_errors_surface_as_exceptions():
    w = random_sdpa_inputs(1, 2, 2, 8, 8, 64, 64, "bf16")
    with pytest.raises(WfError):
        run(w, dropout_p=0.1)


def _sampled_rows_causal(w, out, picks, rows):
    """Rows [i0, i1) of a causal problem: q rows i0..i1-1 against keys 0..i1-1, bottom-right."""
    q, k, v = w["q"], w["k"], w["v"]
    G = q.shape[1] // k.shape[1]
    for b, h in picks:
        for i0, i1 in rows:
            ref, _ = oracle.sdpa(q[b:b + 1, h:h + 1, i0:i1], k[b:b + 1, h // G:h // G + 1, :i1],
                                 v[b:b + 1, h // G:h // G + 1, :i1], is_causal=True,
                                 scale=np.float32(w["scale"]), causal_align="bottom_right")
            assert_close(out[b:b + 1, h:h + 1, i0:i1], ref, q.dtype, f"b{b} h{h} rows {i0}:{i1}")


@pytest.fixture(scope="module")
def gqa_4k_bench_call():
    """The benchmark call (B=4, Hq=32, Hkv=8, L=4096, d=128 bf16 causal, no lse, default
    kernel choice) and its output on the host."""
    w = causal_gqa_prefill()
    with tune():
        out = run(w, is_causal=True)
    return w, out.cpu()


@pytest.mark.parametrize("b", range(4))
def test_causal_gqa_prefill_full_size_every_row(gqa_4k_bench_call, b):
    """Every output row of batch b of the benchmark call against the oracle (all 32 heads, all
    4,096 rows; rows in blocks of 512, each block a bottom-right causal problem over the keys
    up to its last row, which is the same definition restricted to the keys a row can see)."""
    w, out = gqa_4k_bench_call
    assert tuple(out.shape) == (4, 32, 4096, 128)
    q, k, v = w["q"], w["k"], w["v"]
    ref = np.empty((1, 32, 4096, 128))
    for h in range(32):
        for i0 in range(0, 4096, 512):
            i1 = i0 + 512
            ref[:, h:h + 1, i0:i1], _ = oracle.sdpa(
                q[b:b + 1, h:h + 1, i0:i1], k[b:b + 1, h // 4:h // 4 + 1, :i1],
                v[b:b + 1, h // 4:h // 4 + 1, :i1], is_causal=True,
                scale=np.float32(w["scale"]), causal_align="bottom_right")
    mx, mean = assert_close(out[b:b + 1], ref, torch.bfloat16, f"batch {b}, every row")
    print(f"4k causal GQA batch {b}: max abs err {mx:.3g}, mean abs err {mean:.3g}")


@pytest.mark.parametrize("qpw", ["persistent", 64, 32])
def test_causal_gqa_prefill_full_size_sampled(qpw):
    """B=4, Hq=32, Hkv=8, L=4096, d=128 bf16 causal with each kernel the dispatcher can pick
    for it (persistent 32-query waves, one-item-per-group 64- and 32-query waves); sampled rows
    across the sequence checked against the oracle."""
    w = causal_gqa_prefill()
    with _pick_shape(qpw):
        out = run(w, is_causal=True)
    assert tuple(out.shape) == (4, 32, 4096, 128)
    assert torch.isfinite(out).all()
    _sampled_rows_causal(w, out.cpu(), [(0, 0), (1, 5), (2, 17), (3, 31)],
                         [(0, 64), (1000, 1040), (2047, 2113), (4032, 4096)])


@pytest.mark.parametrize("kind", ["bool", "float"])
@pytest.mark.parametrize("pre", [True, False], ids=["prescaled", "exact"])
def test_masked_sdpa_full_size(kind, pre):
    """B=2, H=16, L=2048, d=64 fp16 with a [2,1,L,L] mask broadcast over heads, fully checked,
    through the prescaled-Q kernel (the default without the lse) and the exact one."""
    w = masked_sdpa_inputs(kind)
    with tune(mask_pre=-1 if pre else 0):
        out = run(w)
    ref, _ = oracle.sdpa(w["q"], w["k"], w["v"], mask=w["mask"], scale=np.float32(w["scale"]))
    mx, mean = assert_close(out, ref, torch.float16, f"masked {kind}")
    print(f"masked {kind} {'prescaled' if pre else 'exact'}: max {mx:.3g} mean {mean:.3g}")


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_mask_rows_ending_inside_a_dword(dt):
    # Masks whose rows are 16-byte aligned (one query row, or padded rows viewed narrower)
    # but whose key count is not a multiple of 4 bytes: the last valid keys must count.
    g = torch.Generator().manual_seed(5)
    tdt = {"bf16": torch.bfloat16, "fp16": torch.float16}[dt]
    for Lq, Lk in ((1, 255), (70, 253)):
        q = torch.randn(1, 8, Lq, 64, generator=g).to(tdt)
        k = torch.randn(1, 4, Lk, 64, generator=g).to(tdt)
        v = torch.randn(1, 4, Lk, 64, generator=g).to(tdt)
        wide = torch.rand(1, 1, Lq, 256, generator=g) < 0.85        # rows 256 bytes apart
        m = wide[..., :Lk]
        ref, _ = oracle.sdpa(q, k, v, mask=m.contiguous(), scale=np.float32(0.125))
        out = sdpa(q.to(DEV), k.to(DEV), v.to(DEV), attn_mask=m.to(DEV) if Lq == 1 else
                   wide.to(DEV)[..., :Lk], scale=0.125)
        assert_close(out, ref, tdt, f"Lq={Lq} Lk={Lk}")
