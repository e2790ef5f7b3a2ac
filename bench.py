"""Throughput of exact attention forward on one MI355X: causal GQA prefill, bf16,
B=4, Hq=32, Hkv=8, Lq=Lk=4096, head dim 128 (synthetic N(0,1) inputs, seed 7).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms T] [--no-cpu-baseline]

A step is one forward pass over the batch (one launch of the attention kernel) with the
inputs already resident in HBM. Before the W warm-up steps the call runs back to back for T
milliseconds of GPU time (default 300): the GPU's clock governor takes that long to settle
after a fresh start (measured per launch on a fresh box: launches 0-2 0.55 ms, then 0.60-0.72
ms over launches 3-30 while the clock drops, back to 0.55 by launch 35 and a steady 0.52 ms
from about launch 100 on), so a timed region that starts a few launches into the process
measures the governor, not the kernel. The settle phase is reported in the JSON line
("clock_settle": launches and milliseconds). Prints one JSON line with the throughput in TFLOP/s
(4*B*H*L^2*d, halved for causal), the fraction of the bf16 dense MFMA peak, the kernel's
roofline figures (average launch time from HIP events on the launch stream) and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s + % of bf16 MFMA peak (causal GQA prefill, 4k)"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published
CFG = dict(B=4, Hq=32, Hkv=8, L=4096, D=128)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_causal_gqa_4k_traffic.json")
# Sources of the kernel the benchmark launches (the persistent 32-query kernel).
KERNEL_SOURCES = ["exact_attention_forward_flash_amd/csrc/attn_fwd.hpp",
                  "exact_attention_forward_flash_amd/csrc/attn_fwd_p.hpp",
                  "exact_attention_forward_flash_amd/csrc/wf_device.hpp",
                  "exact_attention_forward_flash_amd/csrc/sdpa_bf16_d128_p.hip"]
KERNEL_NAME = "attn_fwd_p_kernel"


def flops_per_step(B, Hq, L, D, causal=True):
    f = 4.0 * B * Hq * L * L * D
    return f / 2 if causal else f


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the kernel as it is now; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline():
    """The fp64 oracle on a bounded sample: batches 0-2 (96 query heads, 24 KV heads), all
    4096 rows, causal. Throughput in the metric's unit over the sample's algorithmic flops."""
    import numpy as np
    import oracle
    from synth import causal_gqa_prefill
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count()
    w = causal_gqa_prefill()
    nb = 3
    q, k, v = w["q"][:nb], w["k"][:nb], w["v"][:nb]
    t0 = time.perf_counter()
    oracle.sdpa(q, k, v, is_causal=True, scale=np.float32(w["scale"]))
    dt = time.perf_counter() - t0
    fl = flops_per_step(nb, CFG["Hq"], CFG["L"], CFG["D"], True)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"batches 0-{nb - 1} of the workload ({nb * CFG['Hq']} query heads), all "
                      f"{CFG['L']} rows, causal, fp64 numpy oracle; {dt:.1f} s wall"}


def write_traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """Turns rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs (KiB per dispatch) of the
    attention kernel and of the plain 256 MiB copy (--copy-calibration) into HBM bytes per
    launch: each counter is scaled by (copy bytes) / (what it reads for the copy)."""
    import csv

    def per_dispatch(path, name_part):
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
                if name_part in r["Kernel_Name"]]
        if not vals:
            raise SystemExit(f"no {name_part} dispatch in {path}")
        vals.sort()
        return vals[len(vals) // 2] * 1024.0  # median, bytes

    copy_bytes = 256 << 20
    f_scale = copy_bytes / per_dispatch(copy_fetch_csv, "copyBuffer")
    w_scale = copy_bytes / per_dispatch(copy_write_csv, "copyBuffer")
    rd = per_dispatch(fetch_csv, KERNEL_NAME) * f_scale
    wr = per_dispatch(write_csv, KERNEL_NAME) * w_scale
    B, Hq, Hkv, L, D = (CFG[x] for x in ("B", "Hq", "Hkv", "L", "D"))
    algo_rd = 2 * (B * Hq * L * D + 2 * B * Hkv * L * D)
    algo_wr = 2 * B * Hq * L * D
    rec = {"kernel_source_hash": kernel_source_hash(), "hbm_bytes_per_launch": int(rd + wr),
           "read_bytes": int(rd), "write_bytes": int(wr),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "algorithmic_read_bytes": algo_rd, "algorithmic_write_bytes": algo_wr}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def clock_settle(step, settle_ms, stream):
    """Runs step() back to back until settle_ms of GPU time have passed (in blocks of 20
    launches timed by HIP events on the launch stream); returns what was run."""
    import torch
    n, spent = 0, 0.0
    while spent < settle_ms:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(20):
            step()
        b.record(stream)
        b.synchronize()
        spent += a.elapsed_time(b)
        n += 20
    return {"launches": n, "ms": round(spent, 1)}


def _time_steps(step, steps, warmup, stream, settle_ms=200.0):
    """Average milliseconds of step() over `steps` runs after settle_ms of back-to-back launches
    and `warmup` more, from HIP events on the launch stream."""
    import torch
    clock_settle(step, settle_ms, stream)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in evs) / len(evs)


def other_workload(name, steps, warmup):
    """Times one of the other configurations (parity cases, not the headline line): one JSON
    line with its kernel throughput. TFLOP/s use 2*Hq*Lq*Lk*(Dqk+Dv) per (batch, sequence),
    halved for causal; the cache stream also reports the cache update's HBM GB/s (bytes the
    update reads plus writes)."""
    import torch
    import exact_attention_forward_flash_amd as wf
    import synth
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    line = {"workload": name, "desc": synth.WORKLOADS[name]["desc"], "steps": steps, "warmup": warmup}
    if name in ("masked_bool", "masked_float"):
        w = synth.masked_sdpa_inputs(name.split("_")[1])
        q, k, v, m = (w[n].to(dev) for n in ("q", "k", "v", "mask"))
        ms = _time_steps(lambda: wf.sdpa(q, k, v, attn_mask=m, scale=w["scale"]), steps, warmup, stream)
        B, H, L, D = q.shape
        fl = 4.0 * B * H * L * L * D
        line.update(ms=round(ms, 4), tflops=round(fl / ms / 1e9, 2))
    elif name == "varlen_mla":
        w = synth.varlen_mla_prefill_inputs()
        t = {n: w[n].to(dev) for n in ("q", "q_rope", "k", "k_rope", "v", "q_seqlen", "kv_seqlen")}
        ws = torch.empty(max(256, wf.varlen_mla_prefill_workspace_size(16, t["q"].shape[0], 16)),
                         dtype=torch.uint8, device=dev)
        ms = _time_steps(lambda: wf.varlen_mla_prefill(
            t["q"], t["q_rope"], t["k"], t["k_rope"], t["v"], t["q_seqlen"], t["kv_seqlen"],
            w["head_num"], w["kv_head_num"], w["qk_scale"], 1, ws), steps, warmup, stream)
        lens = [int(x) for x in w["q_seqlen"]]
        fl = sum(2.0 * w["head_num"] * L * L * (192 + 128) / 2 for L in lens)
        line.update(ms=round(ms, 4), tflops=round(fl / ms / 1e9, 2), tokens=sum(lens))
    elif name == "page_example":
        w = synth.page_example_fp32()
        q, k, v = (w[n].to(dev) for n in ("q", "k", "v"))
        ms = _time_steps(lambda: wf.sdpa(q, k, v, scale=w["scale"]), steps, warmup, stream)
        line.update(ms=round(ms, 4), note="launch-latency bound")
    elif name == "cache_stream":
        B, H, D, C, sink, window, n = 1, 24, 128, 256, 256, 3840, 64
        chunks = [(c, q.to(dev), k.to(dev), v.to(dev)) for c, q, k, v in
                  synth.cache_stream_chunks(B, H, D, C, sink, window, n)]
        ws = torch.empty(64 << 20, dtype=torch.uint8, device=dev)

        # Events are made up front and the loop asks the library only for the visible count,
        # so the host stays ahead of the GPU and the events time the kernels, not Python.
        ev_pool = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in chunks]

        def run_stream(evs, att_fl):
            cache = wf.BlockKVCache((B, H, sink + window, D), (B, H, sink + window, D), 2, C,
                                    window, sink, device=dev)
            for i, (c, q, k, v) in enumerate(chunks):
                e = ev_pool[i]
                cache.before_update(c)
                e[0].record(stream)
                cache.update(k, v)
                e[1].record(stream)
                cache.after_update(c)
                cache.attend(q, workspace=ws)
                e[2].record(stream)
                nv = cache.n_visible()
                evs.append(e)
                att_fl.append(4.0 * B * H * C * nv * D)
            return cache

        for _ in range(max(1, warmup // 10)):
            run_stream([], [])
        torch.cuda.synchronize()
        tot_u = tot_a = 0.0
        fl = 0.0
        reps = max(1, steps // 20)
        for _ in range(reps):
            evs, afl = [], []
            run_stream(evs, afl)
            torch.cuda.synchronize()
            tot_u += sum(e[0].elapsed_time(e[1]) for e in evs)
            tot_a += sum(e[1].elapsed_time(e[2]) for e in evs)
            fl += sum(afl)
        upd_bytes = 2 * (2 * B * H * C * D * 2) * n  # K and V rows read + written, fp16
        line.update(chunks=n, streams=reps, update_ms_per_chunk=round(tot_u / reps / n, 4),
                    update_gbs=round(upd_bytes * reps / (tot_u * 1e-3) / 1e9, 1),
                    attend_ms_per_chunk=round(tot_a / reps / n, 4),
                    attend_tflops=round(fl / (tot_a * 1e-3) / 1e12, 2))

        # the same stream through the fused update + attend (one attention launch per chunk)
        def run_fused(evs):
            cache = wf.BlockKVCache((B, H, sink + window, D), (B, H, sink + window, D), 2, C,
                                    window, sink, device=dev)
            for i, (c, q, k, v) in enumerate(chunks):
                e = ev_pool[i]
                cache.before_update(c)
                e[0].record(stream)
                cache.update_attend(k, v, q, workspace=ws)
                e[1].record(stream)
                cache.after_update(c)
                evs.append(e)

        run_fused([])
        torch.cuda.synchronize()
        tot_f = 0.0
        for _ in range(reps):
            evs = []
            run_fused(evs)
            torch.cuda.synchronize()
            tot_f += sum(e[0].elapsed_time(e[1]) for e in evs)
        line.update(fused_update_attend_ms_per_chunk=round(tot_f / reps / n, 4),
                    separate_update_plus_attend_ms_per_chunk=round((tot_u + tot_a) / reps / n, 4))

        # The same 64-chunk streams captured once into HIP graphs and replayed: the library's
        # calls enqueue kernels only, so a replay is the stream's launches without the host's
        # per-call work between them (the per-call events above include any gap where the GPU
        # waited for the host). tests/test_gpu_graph.py checks replays against eager runs.
        def graph_of(fused):
            cache = wf.BlockKVCache((B, H, sink + window, D), (B, H, sink + window, D), 2, C,
                                    window, sink, device=dev)
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side), torch.cuda.graph(g, stream=side):
                for c, q, k, v in chunks:
                    cache.before_update(c)
                    if fused:
                        cache.update_attend(k, v, q, workspace=ws)
                        cache.after_update(c)
                    else:
                        cache.update(k, v)
                        cache.after_update(c)
                        cache.attend(q, workspace=ws)
            stream.wait_stream(side)
            return g

        g_reps = max(2, steps // 10)
        for fused, key in ((False, "graph_update_plus_attend_ms_per_chunk"),
                           (True, "graph_fused_update_attend_ms_per_chunk")):
            g = graph_of(fused)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(g_reps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            line[key] = round(e0.elapsed_time(e1) / g_reps / n, 4)
            del g
        line["graph_replays"] = g_reps
    elif name == "rope_gqa":
        import numpy as np
        w = synth.causal_gqa_prefill()
        q, k, v = (w[n].to(dev) for n in ("q", "k", "v"))
        theta = 10000.0 ** (-np.arange(64) * 2.0 / 128)
        ang = np.arange(4096)[:, None] * theta[None, :]
        c = torch.from_numpy(np.cos(ang)).float().to(dev)
        sn = torch.from_numpy(np.sin(ang)).float().to(dev)
        ws = torch.empty(2 * (q.numel() + k.numel()) + 1024, dtype=torch.uint8, device=dev)
        ms = _time_steps(lambda: wf.sdpa_rope(q, k, v, c, sn, 128, 0, is_causal=True,
                                               scale=w["scale"], workspace=ws), steps, warmup, stream)
        ms0 = _time_steps(lambda: wf.sdpa(q, k, v, is_causal=True, scale=w["scale"]), steps, warmup,
                          stream)
        fl = flops_per_step(4, 32, 4096, 128, True)
        line.update(ms=round(ms, 4), tflops=round(fl / ms / 1e9, 2), sdpa_ms=round(ms0, 4),
                    rope_pass_ms=round(ms - ms0, 4),
                    rope_pass_gbs=round(2 * (q.numel() + k.numel()) * 2 / ((ms - ms0) * 1e-3) / 1e9, 1))
    elif name == "decode":
        B, Hq, Hkv, Lk, D = 8, 32, 8, 16384, 128
        w = synth.random_sdpa_inputs(B, Hq, Hkv, 1, Lk, D, D, "bf16", seed=7)
        q, k, v = (w[n].to(dev) for n in ("q", "k", "v"))
        ws = torch.empty(max(256, wf.sdpa_decode_workspace_size(q, k, v)), dtype=torch.uint8,
                         device=dev)
        out = torch.empty_like(q)
        ms = _time_steps(lambda: wf.sdpa_decode(q, k, v, scale=w["scale"], workspace=ws),
                         steps, warmup, stream)
        ms_dense = _time_steps(lambda: wf.sdpa(q, k, v, scale=w["scale"]), steps, warmup, stream)
        nbytes = (k.numel() + v.numel() + q.numel() + out.numel()) * 2  # read once + written
        line.update(ms=round(ms, 4), gbs=round(nbytes / (ms * 1e-3) / 1e9, 1),
                    hbm_frac=round(nbytes / (ms * 1e-3) / 8e12, 4),
                    sdpa_fwd_ms=round(ms_dense, 4),
                    sdpa_fwd_gbs=round(nbytes / (ms_dense * 1e-3) / 1e9, 1))
        # multi-query decode (64 query heads on one KV head): packed (head, position) rows
        wm = synth.random_sdpa_inputs(B, 64, 1, 1, Lk, D, D, "bf16", seed=8)
        qm, km, vm = (wm[n].to(dev) for n in ("q", "k", "v"))
        wsm = torch.empty(max(256, wf.sdpa_decode_workspace_size(qm, km, vm)), dtype=torch.uint8,
                          device=dev)
        mbytes = (km.numel() + vm.numel() + 2 * qm.numel()) * 2
        ms_m = _time_steps(lambda: wf.sdpa_decode(qm, km, vm, workspace=wsm), steps, warmup, stream)
        line.update(mqa_desc="B=8 Hq=64 Hkv=1, 1 query over 16384 keys", mqa_ms=round(ms_m, 4),
                    mqa_gbs=round(mbytes / (ms_m * 1e-3) / 1e9, 1))
    else:
        raise SystemExit(f"unknown workload {name}")
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="GPU milliseconds of back-to-back untimed launches before the warm-up "
                         "steps, while the clock governor settles (reported as clock_settle)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default="causal_gqa",
                    choices=["causal_gqa", "varlen_mla", "masked_bool", "masked_float",
                             "cache_stream", "page_example", "decode", "rope_gqa"],
                    help="causal_gqa (default) prints the headline line; the others time one of "
                         "the other configurations and print its kernel throughput")
    ap.add_argument("--write-traffic", nargs=4, metavar="CSV",
                    help="FETCH_SIZE, WRITE_SIZE, copy FETCH_SIZE, copy WRITE_SIZE counter CSVs "
                         "from rocprofv3 --pmc: record HBM bytes per launch and exit")
    ap.add_argument("--tune", action="append", default=[], metavar="NAME=VALUE",
                    help="run --workload under a launch-plan override of the library (wf_tune_set "
                         "names, e.g. attend_nw=4); repeatable; other workloads only")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device-to-device copy 3 times (the reference "
                         "kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the attention path here has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_attention_forward_flash_amd as wf
    from synth import causal_gqa_prefill

    if args.workload != "causal_gqa":
        plan = {}
        for t in args.tune:
            name, _, value = t.partition("=")
            plan[name] = int(value)
        with wf.tune(**plan):
            other_workload(args.workload, args.steps, args.warmup)
        return
    if args.tune:
        print("--tune applies to the other workloads; the headline line runs the default plan",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n}), flush=True)
        return

    if not os.path.exists(wf._lib.LIB_PATH):
        from exact_attention_forward_flash_amd.build import build
        build()
    dev = torch.device("cuda:0")
    w = causal_gqa_prefill(**{k: CFG[k] for k in ("B", "Hq", "Hkv", "L", "D")})
    q, k, v = (w[n].to(dev) for n in ("q", "k", "v"))
    out = torch.empty(q.shape[:3] + (v.shape[3],), dtype=q.dtype, device=dev)
    del w

    # direct C-ABI call with preallocated output: the timed region is exactly the launches
    lib = wf.load()
    import ctypes
    dq, dk, dv, do = (wf.describe(t) for t in (q, k, v, out))
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)

    def step():
        rc = lib.wf_sdpa_fwd(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), None, 1, 0.0,
                             float(w_scale), ctypes.byref(do), None, sp)
        if rc != 0:
            raise RuntimeError(lib.wf_last_error().decode())

    w_scale = 1.0 / (CFG["D"] ** 0.5)
    settle = clock_settle(step, args.settle_ms, stream)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-launch durations from HIP events on the launch stream
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    ms_per_step = wall * 1e3 / args.steps

    fl = flops_per_step(CFG["B"], CFG["Hq"], CFG["L"], CFG["D"], True)
    value = fl / (ms_per_step * 1e-3) / 1e12
    achieved = fl / (kernel_ms * 1e-3) / 1e12
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": "causal GQA prefill, bf16, B=4 Hq=32 Hkv=8 Lq=Lk=4096 d=128, "
                               "scale 1/sqrt(128), N(0,1) seed 7",
                   "global_batch": CFG["B"], "seq_len": CFG["L"], "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(),
                     "kernel_ms": round(kernel_ms, 4)},
    }
    line["clock_settle"] = settle
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
