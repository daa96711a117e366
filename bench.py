#!/usr/bin/env python3
"""Benchmark of the chunk-sparse decode path on one MI355X.

One step = one sparse_attn_decode call over the whole batch (every query head of one layer
at one decode step) on the Llama-3.1-8B-shaped 128K-token workload: B=16, Hq=32, Hkv=8, d=128,
C=128, g=4 gists per chunk, k=16 chunks + the current chunk, SAS gate on, paged KV.
Inputs are resident in HBM before the timed region; steps rotate over R independent
instances (>= 1 GiB of algorithmic bytes in the rotation) so that the 256 MB last-level
cache cannot serve them.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--instances R] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

METRIC = "decode attn calls/s and effective HBM GB/s (% of peak) at 128K ctx, k=16"
HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, vendor figure


def decode_bytes(cfg, k=None):
    """Algorithmic bytes of one decode call: every byte the method must touch, once.
    Gist rows scored (and attended), the selected chunks' K and V, the current chunk's K and
    V, q, out (fp32), and the page-table entries read."""
    k = cfg.k if k is None else k
    units = cfg.B * cfg.Hkv
    row = cfg.d * 2                               # one bf16 row
    if cfg.levels == 2:
        n_cand = min(cfg.k2, cfg.nG) * cfg.J      # every preset selects full groups
        gist_rows = cfg.nG * cfg.g + n_cand * cfg.g
        k_eff = min(k, n_cand)
    else:
        gist_rows = cfg.H * cfg.g
        k_eff = min(k, cfg.H)
    parts = {
        "gists_kv": units * gist_rows * row * 2,
        "selected_kv": units * k_eff * cfg.C * row * 2,
        "current_kv": units * cfg.cur_len * row * 2,
        "q": cfg.B * cfg.Hq * row,
        "out": cfg.B * cfg.Hq * cfg.d * 4,
        "page_table": units * (k_eff + 1) * 4,
    }
    return sum(parts.values()), parts


def gist_kernel_bytes(cfg):
    """Algorithmic bytes of the gist-scoring kernel (levels = 1): every historical gist row
    (K and V) of every unit, plus q."""
    units = cfg.B * cfg.Hkv
    return units * cfg.H * cfg.g * cfg.d * 2 * 2 + cfg.B * cfg.Hq * cfg.d * 2


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, budget_s):
    """Time the fp64 CPU oracle (as it stands) on this workload's instance 0.  Full calls if
    one fits the budget, else a seeded subset of units scaled to whole calls."""
    import numpy as np
    import oracle
    from top_chunk_sparse_amd.synth import bf16_bits
    c = inp.cfg
    host = dict(q=bf16_bits(inp.q), k_pages=bf16_bits(inp.k_pages), v_pages=bf16_bits(inp.v_pages),
                page_table=inp.page_table.cpu().numpy().astype(np.int32),
                gist_k=bf16_bits(inp.gist_k), gist_v=bf16_bits(inp.gist_v),
                gist2_k=None if inp.gist2_k is None else bf16_bits(inp.gist2_k),
                gist2_v=None if inp.gist2_v is None else bf16_bits(inp.gist2_v))
    args = dict(B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=c.d, N=c.N, C_=c.C, g=c.g, k=c.k, gate=c.gate,
                levels=c.levels, J=c.J, k2=c.k2, **host)
    units = c.B * c.Hkv
    probe = list(range(0, units, max(1, units // 8)))[:8]
    t0 = time.perf_counter()
    oracle.decode(units=probe, **args)
    per_unit = (time.perf_counter() - t0) / len(probe)
    full = per_unit * units
    if full <= budget_s:
        n, t0 = 0, time.perf_counter()
        while True:
            oracle.decode(**args)
            n += 1
            if time.perf_counter() - t0 >= budget_s * 0.5 or n >= 50:
                break
        dt = time.perf_counter() - t0
        value, sample = n / dt, f"{n} full call(s) of instance 0 ({units} units each)"
    else:
        m = max(1, min(units, int(budget_s / max(per_unit, 1e-9))))
        sub = list(range(0, units, max(1, units // m)))[:m]
        t0 = time.perf_counter()
        oracle.decode(units=sub, **args)
        dt = time.perf_counter() - t0
        value = (len(sub) / units) / dt
        sample = f"{len(sub)} of {units} units of one call, scaled to whole calls"
    return {"value": value, "unit": "calls/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": sample, "seconds": round(dt, 3), "cpu": cpu_model()}


def load_traffic(kernel_name, workload):
    """HBM traffic per launch from committed rocprofv3 counter runs, only if the kernel
    sources are unchanged since the counters were taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"traffic_{kernel_name}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(here, "top_chunk_sparse_amd", "csrc", rec.get("source", "decode.hip"))
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if sha != rec.get("source_sha256"):
        return None
    return rec.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--instances", type=int, default=3)
    ap.add_argument("--workload", default="llama31_8b_decode_128k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration under rocprofv3)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    from top_chunk_sparse_amd import configs, ops
    from top_chunk_sparse_amd.synth import make_decode

    cfg = configs.DECODE_CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    R = max(1, args.instances)
    print(f"# generating {R} instance(s) of {cfg.name}", file=sys.stderr, flush=True)
    insts = [make_decode(cfg, configs.seed_for(cfg.name, r), device=dev) for r in range(R)]
    calls = [ops.DecodeCall(inp, with_scores=False) for inp in insts]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    if args.copy_probe:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        calls[i % R]()
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)

    # ---- timed region: K whole calls --------------------------------------------------
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        calls[i % R]()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = e0.elapsed_time(e1)
    ms_per_step = wall * 1e3 / args.steps
    value = args.steps / wall

    # ---- per-kernel durations: the same K calls with events between the kernels ------
    nst = ops.decode_stage_count(calls[0].p)
    import ctypes
    evs = []
    for _ in range(args.steps):
        row = [torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)]
        for e in row:
            e.record(stream)             # creates the underlying hipEvent_t
        evs.append(row)
    torch.cuda.synchronize()
    for i in range(args.steps):
        arr = (ctypes.c_void_p * (nst + 1))(*[e.cuda_event for e in evs[i]])
        calls[i % R](events=arr)
    torch.cuda.synchronize()
    stage_ms = [sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(args.steps)) / args.steps
                for j in range(nst)]
    print("# stage ms:", [round(x, 4) for x in stage_ms], file=sys.stderr, flush=True)

    total_bytes, parts = decode_bytes(cfg)
    eff_gbps = total_bytes / (ms_per_step * 1e-3) / 1e9
    # dominant kernel: gist scoring (stage 1) -- the largest byte stream of the call
    gk_bytes = gist_kernel_bytes(cfg) if cfg.levels == 1 else None
    roof = None
    if gk_bytes:
        gk_ms = stage_ms[0]
        ach = gk_bytes / (gk_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "gist_kernel", "achieved": round(ach, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                "traffic": load_traffic("gist_kernel", cfg.name),
                "algorithmic_bytes": gk_bytes, "avg_ms": round(gk_ms, 5)}

    cpu = None
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(insts[0], args.cpu_seconds)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "calls/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "d": cfg.d,
                   "N": cfg.N, "C": cfg.C, "g": cfg.g, "k": cfg.k, "gate": "sas" if cfg.gate else
                   "none", "levels": cfg.levels, "paged": cfg.paged, "inputs": "bf16",
                   "instances_rotated": R},
        "effective_GBps": round(eff_gbps, 1),
        "pct_of_hbm_peak": round(100 * eff_gbps / HBM_PEAK_GBPS, 2),
        "algorithmic_bytes_per_call": total_bytes,
        "event_ms_per_step": round(ev_ms / args.steps, 5),
        "stage_ms": [round(x, 5) for x in stage_ms],
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
