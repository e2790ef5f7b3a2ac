"""GPU checks that the library's calls can be captured into a HIP graph and replayed: the
calls enqueue kernels only (no allocation, memset or synchronisation inside), so a captured
sequence replays the same launches. Every replay is compared bit for bit with the eager run
of the same calls, with the program's own eager work and synchronisations between replays."""
import pytest
import torch

import exact_attention_forward_flash_amd as wf
from synth import cache_stream_chunks, causal_gqa_prefill, varlen_mla_prefill_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _replays_match(run, eager_outs, replays=3):
    """Captures run() into a graph, replays it `replays` times with unrelated eager work and a
    synchronisation between replays, and checks each replay's outputs against eager_outs."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            outs = run()
    torch.cuda.current_stream().wait_stream(side)
    for r in range(replays):
        g.replay()
        junk = torch.randn(1 << 20, device=DEV).cumsum(0)   # the program's own work
        torch.cuda.synchronize()
        assert torch.isfinite(junk).all()
        for i, (got, ref) in enumerate(zip(outs, eager_outs)):
            assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {r}, output {i}"
    return g


def _cache_stream(cache, chunks, ws, fused, causal):
    outs = []
    for idx, q, k, v in chunks:
        cache.before_update(idx)
        if fused:
            outs.append(cache.update_attend(k, v, q, workspace=ws, is_causal=causal))
            cache.after_update(idx)
        else:
            cache.update(k, v)
            cache.after_update(idx)
            outs.append(cache.attend(q, workspace=ws, is_causal=causal))
    return outs


@pytest.mark.parametrize("H,fused,causal", [(4, False, False), (24, False, False), (4, True, True),
                                            (24, True, False)])
def test_cache_stream_graph_replays_match_eager(H, fused, causal):
    """A stream of chunks across the roll of the window (update + attend, or the fused call),
    captured once: each replay rewrites the same slots and gives the eager outputs."""
    sink, window, chunk, n = 256, 768, 256, 8
    chunks = [(c, q.to(DEV), k.to(DEV), v.to(DEV))
              for c, q, k, v in cache_stream_chunks(1, H, 128, chunk, sink, window, n)]
    shape = (1, H, sink + window, 128)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=DEV)
    eager = wf.BlockKVCache(shape, shape, 2, chunk, window, sink, device=DEV)
    eager_outs = [o.clone() for o in _cache_stream(eager, chunks, ws, fused, causal)]
    torch.cuda.synchronize()
    cap = wf.BlockKVCache(shape, shape, 2, chunk, window, sink, device=DEV)
    _replays_match(lambda: _cache_stream(cap, chunks, ws, fused, causal), eager_outs)
    assert torch.equal(cap.k, eager.k) and torch.equal(cap.v, eager.v)


def test_dense_prefill_graph_replays_match_eager():
    """The persistent causal GQA kernel (the benchmark's) inside a graph."""
    w = causal_gqa_prefill(B=1, Hq=8, Hkv=2, L=1024, D=128)
    q, k, v = (w[n].to(DEV) for n in ("q", "k", "v"))
    ref = wf.sdpa(q, k, v, is_causal=True, scale=w["scale"])
    torch.cuda.synchronize()
    _replays_match(lambda: [wf.sdpa(q, k, v, is_causal=True, scale=w["scale"])], [ref])


def test_varlen_mla_graph_replays_match_eager():
    """The varlen MLA prefill (device-built schedule, work counters reset by a kernel each
    call) inside a graph."""
    w = varlen_mla_prefill_inputs(batch=4, seed=3, lengths=torch.tensor([700, 1, 257, 1300]))
    t = {n: w[n].to(DEV) for n in ("q", "q_rope", "k", "k_rope", "v", "q_seqlen", "kv_seqlen")}
    ws = torch.empty(max(256, wf.varlen_mla_prefill_workspace_size(4, t["q"].shape[0], 16)),
                     dtype=torch.uint8, device=DEV)

    def call():
        return wf.varlen_mla_prefill(t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], t["q_seqlen"],
                                     t["kv_seqlen"], w["head_num"], w["kv_head_num"], w["qk_scale"],
                                     1, ws)
    ref = call().clone()
    torch.cuda.synchronize()
    _replays_match(lambda: [call()], [ref])
