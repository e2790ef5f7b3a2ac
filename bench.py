"""Throughput of exact attention forward on one MI355X: causal GQA prefill, bf16,
B=4, Hq=32, Hkv=8, Lq=Lk=4096, head dim 128 (synthetic N(0,1) inputs, seed 7).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one forward pass over the batch (one launch of the attention kernel) with the
inputs already resident in HBM. Prints one JSON line with the throughput in TFLOP/s
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # The GPU's clocks settle over the first few dozen launches (a launch takes ~0.6 ms):
    # 100 untimed launches precede the 200 timed ones.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--write-traffic", nargs=4, metavar="CSV",
                    help="FETCH_SIZE, WRITE_SIZE, copy FETCH_SIZE, copy WRITE_SIZE counter CSVs "
                         "from rocprofv3 --pmc: record HBM bytes per launch and exit")
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
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
