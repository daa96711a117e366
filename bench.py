#!/usr/bin/env python3
"""Benchmark of the chunk-sparse attention path on one MI355X.

Default workload (decode): one step = one sparse_attn_decode call over the whole batch (every
query head of one layer at one decode step) on the Llama-3.1-8B-shaped 128K-token workload:
B=16, Hq=32, Hkv=8, d=128, C=128, g=4 gists per chunk, k=16 chunks + the current chunk, SAS
gate on, paged KV.  Inputs are resident in HBM before the timed region; steps rotate over R
independent instances (>= 1 GiB of algorithmic bytes in the rotation) so that the 256 MB
last-level cache cannot serve them.  Prints one JSON line.

--workload sas_prefill_16k: one step = one sparse_attn_prefill call (block selection + the
MFMA block-sparse causal forward) on B=1, Hq=32, Hkv=8, d=128, T=16384, 64-token blocks,
top-16 earlier blocks + the diagonal block, SAS gate; reported as algorithmic TFLOP/s.
Add --backward for one sparse_attn_prefill_backward call per step (dq, dk, dv, dS).

--workload ssa_gist_prefill_16k: one step = one sparse_attn_gist_prefill call over 128 chunks
of 128 raw tokens + 4 gists (16,896 positions), same heads; algorithmic TFLOP/s, with the row
launch measured against the HBM roofline.

Every workload: a sustained loop first, then the median of 5 loops of exactly --steps calls
(wall clock between device synchronisations), per-kernel event times, the roofline of the
dominant kernel, and the fp64 CPU oracle timed on the host.

    python bench.py [--steps K] [--warmup W] [--instances R] [--workload NAME] [--backward]
                    [--no-cpu-baseline] [--cpu-seconds S]
"""
import argparse
import json
import os
import sys
import time

METRIC = "decode attn calls/s and effective HBM GB/s (% of peak) at 128K ctx, k=16"
PREFILL_METRIC = "SAS block-sparse causal prefill forward, algorithmic TFLOP/s at 16K tokens, k=16"
GIST_PREFILL_METRIC = ("SSA gist-masked prefill forward, algorithmic TFLOP/s at 16K raw tokens "
                       "(128 chunks of 128 + 4 gists)")
PREFILL_BWD_METRIC = ("SAS block-sparse causal prefill backward (dq, dk, dv, dS), algorithmic "
                      "TFLOP/s at 16K tokens, k=16")
HBM_PEAK_GBPS = 8000.0   # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak, vendor figure


def decode_bytes(cfg, k=None, gist_mode="all", k_eff_mean=None):
    """Algorithmic bytes of one decode call: every byte the method must touch, once.
    Gist rows scored (and attended), the selected chunks' K and V, the current chunk's K and
    V, q, out (fp32), and the page-table entries read.  gist_mode "selected": every gist key is
    read for the scores, but only the selected chunks' gist values (and keys, already read)
    enter the softmax, and at two levels the chosen groups' level-2 gist values."""
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
    if k_eff_mean is not None:   # top-p, per-head union: chunks actually unfolded, unit mean
        k_eff = k_eff_mean
    if gist_mode == "selected":
        sel_v = k_eff * cfg.g + (min(cfg.k2, cfg.nG) * cfg.g if cfg.levels == 2 else 0)
        parts = {"gists_k": units * gist_rows * row, "selected_gists_v": int(units * sel_v * row)}
    else:
        parts = {"gists_kv": units * gist_rows * row * 2}
    parts.update({
        "selected_kv": int(units * k_eff * cfg.C * row * 2),
        "current_kv": units * cfg.cur_len * row * 2,
        "q": cfg.B * cfg.Hq * row,
        "out": cfg.B * cfg.Hq * cfg.d * 4,
        "page_table": int(units * (k_eff + 1) * 4),
    })
    return sum(parts.values()), parts


def gist_kernel_bytes(cfg, gist_mode="all"):
    """Algorithmic bytes of the gist-scoring kernel (levels = 1): every historical gist row
    (K, and V unless only the selected chunks' gists enter the softmax) of every unit, plus q."""
    units = cfg.B * cfg.Hkv
    kv = 1 if gist_mode == "selected" else 2
    return units * cfg.H * cfg.g * cfg.d * 2 * kv + cfg.B * cfg.Hq * cfg.d * 2


def prefill_pairs(cfg):
    """Attended (query, key) pairs of one prefill call: per query head, every row of block i
    sees min(k, i) whole earlier blocks plus the causal part of its own block."""
    nb, blk = cfg.nb, cfg.blk
    per_head = sum(min(cfg.k, i) for i in range(nb)) * blk * blk + nb * blk * (blk + 1) // 2
    return cfg.B * cfg.Hq * per_head


def prefill_flops(cfg):
    """Algorithmic FLOPs: 2 d for q.k and 2 d for p.v per attended pair."""
    return 4 * cfg.d * prefill_pairs(cfg)


def prefill_bwd_flops(cfg, products=5):
    """Algorithmic FLOPs of the gradients: 2 d per attended pair for each product -- q.k and
    dout.v recomputed, and the dq, dk and dv products (5; the gradient kernel's dq part alone
    does 3: q.k, dout.v, dq; its dk / dv part 4: q.k, dout.v, dk, dv)."""
    return 2 * products * cfg.d * prefill_pairs(cfg)


def gist_prefill_pairs(cfg):
    """Attended (query, key) pairs of one SSA gist-masked prefill call, raw rows and gist rows:
    raw row r of chunk c sees c g gists and r + 1 raw keys; gist t of chunk c sees c g + t + 1
    gists and the chunk's L raw keys."""
    M, L, g = cfg.M, cfg.L, cfg.g
    raw = L * g * M * (M - 1) // 2 + M * L * (L + 1) // 2
    gist = g * g * M * (M - 1) // 2 + M * g * (g + 1) // 2 + M * g * L
    return cfg.B * cfg.Hq * raw, cfg.B * cfg.Hq * gist


def gist_prefill_row_bytes(cfg):
    """Algorithmic bytes of the query-row launch of one gist-masked prefill call, each counted
    once: q (bf16, every position), the raw K / V rows (bf16), the gathered gist K / V (bf16,
    the gather kernel's zero-padded output), out and lse (fp32, every position)."""
    Gp = -(-cfg.M * cfg.g // 64) * 64
    units = cfg.B * cfg.Hkv
    return (cfg.B * cfg.Hq * cfg.Tp * cfg.d * 2 + units * cfg.M * cfg.L * cfg.d * 2 * 2
            + units * Gp * cfg.d * 2 * 2 + cfg.B * cfg.Hq * cfg.Tp * (cfg.d + 1) * 4)


def prefill_bytes(cfg):
    """Algorithmic bytes of one prefill call: q, K and V (bf16), S (fp32) read once; out (fp32),
    lse (fp32) and the selection (int32) written once."""
    nb = cfg.nb
    return (cfg.B * cfg.Hq * cfg.T * cfg.d * 2 + 2 * cfg.B * cfg.Hkv * cfg.T * cfg.d * 2
            + cfg.B * cfg.Hkv * nb * nb * 4 + cfg.B * cfg.Hq * cfg.T * (cfg.d + 1) * 4
            + cfg.B * cfg.Hkv * nb * cfg.k * 4)


LOOPS = 5            # timed loops of exactly --steps calls; the median is reported
SUSTAIN_MS = 200.0   # the sustained figure repeats the loop until at least this long


def timed_loops(torch, stream, step, steps, loops=LOOPS):
    """``loops`` timed loops of exactly ``steps`` calls, each bracketed by a device
    synchronisation on both sides.  Returns [(wall_ms, event_ms)] per loop; step(i) enqueues
    call i."""
    out = []
    for _ in range(loops):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)   # instrumentation, outside the wall-clock bracket of the K steps
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        e1.record(stream)   # queued behind the steps while the GPU is still busy with them
        torch.cuda.synchronize()
        out.append(((time.perf_counter() - t0) * 1e3, e0.elapsed_time(e1)))
    return out


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def timing_summary(torch, stream, step, steps):
    """The reported timing: a sustained figure from one loop of at least SUSTAIN_MS (whole
    multiples of ``steps`` calls), then the median over LOOPS loops of exactly ``steps`` calls
    (host wall clock between synchronisations) with the event-timed median beside it.

    The sustained loop runs first because the GPU reaches its steady clock only after some
    tens of milliseconds of continuous work: right after the synthetic inputs are generated
    (or after an idle pause) the first ~20-call loops of the 128K decode measured 88-101 us per
    call against 85-86 us once it had settled, so short loops taken straight after a few
    warmup calls would time that ramp instead of the kernels."""
    (w0, _), = timed_loops(torch, stream, step, steps, loops=1)   # sizes the sustained loop
    reps = max(1, int(SUSTAIN_MS / max(w0, 1e-3)) + 1)
    (sw, se), = timed_loops(torch, stream, step, steps * reps, loops=1)
    loops = timed_loops(torch, stream, step, steps)
    wall = median([w for w, _ in loops])
    ev = median([e for _, e in loops])
    return {"ms_per_step": wall / steps, "event_ms_per_step": ev / steps,
            "loops_ms": [round(w, 4) for w, _ in loops],
            "sustained": {"steps": steps * reps, "ms_per_step": round(sw / (steps * reps), 5),
                          "event_ms_per_step": round(se / (steps * reps), 5),
                          "runs": "before the timed loops"}}


def stream_read_ceiling(torch, ops, dev, gib=2, reps=5):
    """HBM read ceiling on this machine: the library's plain streaming-read kernel over ``gib`` GiB
    (8x the 256 MB last-level cache), median of ``reps`` timed passes, in GB/s."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.empty(ops.STREAM_READ_BLOCKS, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev)
    ops.stream_read(buf, sink)
    torch.cuda.synchronize()
    res = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        ops.stream_read(buf, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        res.append(buf.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf
    torch.cuda.empty_cache()
    g = median(res)
    return {"GBps": round(g, 1), "frac_of_peak": round(g / HBM_PEAK_GBPS, 4),
            "bytes": gib << 30, "passes": reps, "kernel": "stream_read_kernel"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(inp, budget_s, **mode):
    """Time the fp64 CPU oracle (as it stands) on this workload's instance 0, in the same
    token-set and selection mode as the GPU calls (``mode``: the oracle's gists_in_softmax,
    top_p and head_select).  Full calls if one fits the budget, else a seeded subset of units
    scaled to whole calls."""
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
                levels=c.levels, J=c.J, k2=c.k2, **host, **mode)
    units = c.B * c.Hkv
    probe = list(range(0, units, max(1, units // 8)))[:8]
    oracle.decode(units=probe[:1], **args)          # untimed: library load, first touch
    t0 = time.perf_counter()
    oracle.decode(units=probe, **args)
    per_unit = (time.perf_counter() - t0) / len(probe)
    full = per_unit * units
    if full <= budget_s:
        n, t0 = 0, time.perf_counter()
        while True:
            oracle.decode(**args)
            n += 1
            if time.perf_counter() - t0 >= budget_s:
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


def cpu_baseline_prefill(inp, budget_s):
    """Time the fp64 CPU oracle (as it stands) on a seeded sample of query blocks of instance 0,
    scaled to the metric's unit (algorithmic TFLOP/s of whole calls)."""
    import numpy as np
    import oracle
    from top_chunk_sparse_amd.synth import bf16_bits
    c = inp.cfg
    args = dict(B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=c.d, T=c.T, blk=c.blk, k=c.k, gate=c.gate,
                q=bf16_bits(inp.q), k_=bf16_bits(inp.k), v=bf16_bits(inp.v),
                S=inp.S.cpu().numpy().astype(np.float32))
    nblocks = c.B * c.Hkv * c.nb
    rng = np.random.default_rng(12345)
    order = rng.permutation(nblocks).astype(np.int32)
    # pairs attended by the sampled blocks (block i of any unit: G heads x rows)
    def pairs(ids):
        i = ids % c.nb
        return int(sum(c.G * (np.minimum(c.k, i) * c.blk * c.blk + c.blk * (c.blk + 1) // 2)))
    oracle.prefill(blocks=order[:1], **args)       # untimed: library load, first touch
    n, t0 = 8, time.perf_counter()
    oracle.prefill(blocks=order[:n], **args)
    dt = time.perf_counter() - t0
    while dt < budget_s * 0.5 and n < nblocks:    # grow the timed sample to ~budget
        n = min(nblocks, int(n * max(2.0, budget_s / max(dt, 1e-3) * 0.9)))
        t0 = time.perf_counter()
        oracle.prefill(blocks=order[:n], **args)
        dt = time.perf_counter() - t0
    flops = 4 * c.d * pairs(order[:n])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle", "sample": f"{n} of {nblocks} query blocks (all heads of each) of "
            f"instance 0, seeded random choice", "seconds": round(dt, 3), "cpu": cpu_model(),
            "calls_per_s": round(flops / dt / prefill_flops(c), 6)}


def cpu_baseline_prefill_backward(inp, dout, dlse, budget_s):
    """Time the fp64 CPU oracle's backward (as it stands) on instance 0, restricted to the first
    n query blocks of every unit (the oracle's timing sample), grown to about the budget and
    scaled to the metric's unit (algorithmic TFLOP/s)."""
    import numpy as np
    import oracle
    from top_chunk_sparse_amd.synth import bf16_bits
    c = inp.cfg
    args = dict(B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=c.d, T=c.T, blk=c.blk, k=c.k, gate=c.gate,
                q=bf16_bits(inp.q), k_=bf16_bits(inp.k), v=bf16_bits(inp.v),
                S=inp.S.cpu().numpy().astype(np.float32), dout=bf16_bits(dout),
                dlse=dlse.cpu().numpy().astype(np.float32))
    def pairs(n):   # attended pairs of query blocks 0 .. n-1 of every unit
        i = np.arange(n)
        return int(c.B * c.Hkv * c.G * (np.minimum(c.k, i) * c.blk * c.blk
                                         + c.blk * (c.blk + 1) // 2).sum())
    oracle.prefill_backward(n_blocks=1, **args)    # untimed: library load, first touch
    n, t0 = 2, time.perf_counter()
    oracle.prefill_backward(n_blocks=n, **args)
    dt = time.perf_counter() - t0
    while dt < budget_s * 0.5 and n < c.nb:        # grow the timed sample to ~budget
        n = min(c.nb, int(n * max(1.5, (budget_s / max(dt, 1e-3)) ** 0.5)))
        t0 = time.perf_counter()
        oracle.prefill_backward(n_blocks=n, **args)
        dt = time.perf_counter() - t0
    flops = 10 * c.d * pairs(n)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle", "sample": f"query blocks 0..{n - 1} of each of the {c.B * c.Hkv} "
            f"units of instance 0 ({n} of {c.nb} per unit)", "seconds": round(dt, 3),
            "cpu": cpu_model(), "calls_per_s": round(flops / dt / prefill_bwd_flops(c), 6)}


def cpu_baseline_gist_prefill(inp, budget_s):
    """Time the fp64 CPU oracle (as it stands) on a seeded sample of query rows of instance 0,
    scaled to algorithmic TFLOP/s (4 d per attended pair)."""
    import numpy as np
    import oracle
    from top_chunk_sparse_amd.synth import bf16_bits
    c = inp.cfg
    args = dict(B=c.B, Hq=c.Hq, Hkv=c.Hkv, d=c.d, M=c.M, L=c.L, g=c.g, q=bf16_bits(inp.q),
                k_=bf16_bits(inp.k), v=bf16_bits(inp.v))
    total = c.B * c.Hq * c.Tp
    order = np.random.default_rng(12345).permutation(total).astype(np.int32)
    def pairs(rows):
        pos = rows % c.Tp
        ch, off = pos // c.W, pos % c.W
        n = np.where(off < c.L, ch * c.g + off + 1, ch * c.g + (off - c.L) + 1 + c.L)
        return int(n.sum())
    oracle.gist_prefill(rows=order[:8], **args)      # untimed: library load, first touch
    n, t0 = 256, time.perf_counter()
    oracle.gist_prefill(rows=order[:n], **args)
    dt = time.perf_counter() - t0
    while dt < budget_s * 0.5 and n < total:
        n = min(total, int(n * max(2.0, budget_s / max(dt, 1e-3) * 0.9)))
        t0 = time.perf_counter()
        oracle.gist_prefill(rows=order[:n], **args)
        dt = time.perf_counter() - t0
    flops = 4 * c.d * pairs(order[:n])
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle", "sample": f"{n} of {total} query rows of instance 0, seeded random "
            "choice", "seconds": round(dt, 3), "cpu": cpu_model()}


def kernel_times(torch, stream, call, steps, nst):
    """Average duration (ms) of each of a call's nst kernels over `steps` calls: the library
    records a pair of events at each kernel's own start and end (the timed entry points)."""
    import ctypes
    evs = []
    for _ in range(steps):
        row = [torch.cuda.Event(enable_timing=True) for _ in range(2 * nst)]
        for e in row:
            e.record(stream)             # creates the underlying hipEvent_t
        evs.append(row)
    torch.cuda.synchronize()
    for i in range(steps):
        call(i, (ctypes.c_void_p * (2 * nst))(*[e.cuda_event for e in evs[i]]))
    torch.cuda.synchronize()
    return [sum(evs[i][2 * j].elapsed_time(evs[i][2 * j + 1]) for i in range(steps)) / steps
            for j in range(nst)]


def load_traffic(kernel_name, workload):
    """HBM traffic per launch from committed rocprofv3 counter runs, only if the kernel
    sources are unchanged since the counters were taken."""
    import hashlib
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"traffic_{kernel_name}_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in rec.get("sources", []):
        h.update(open(os.path.join(here, f), "rb").read())
    if h.hexdigest() != rec.get("sources_sha256"):
        return None
    return rec.get("bytes_per_launch")


def prefill_cfg(args, configs):
    """The prefill workload, with --tokens (T, a multiple of the block) and --k overrides."""
    cfg = configs.PREFILL_CONFIGS[args.workload]
    if args.tokens > 0:
        cfg = cfg.with_(T=args.tokens)
    if args.k >= 0:
        cfg = cfg.with_(k=args.k)
    return cfg


def run_prefill(args, torch, configs, ops):
    from top_chunk_sparse_amd.synth import make_prefill
    import ctypes
    cfg = prefill_cfg(args, configs)
    dev = torch.device("cuda:0")
    R = max(1, min(args.instances, 2))
    print(f"# generating {R} instance(s) of {cfg.name}", file=sys.stderr, flush=True)
    insts = [make_prefill(cfg, configs.seed_for(cfg.name, r), device=dev) for r in range(R)]
    calls = [ops.PrefillCall(inp) for inp in insts]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        calls[i % R]()
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)
    tm = timing_summary(torch, stream, lambda i: calls[i % R](), args.steps)
    ms_per_step = tm["ms_per_step"]
    stage_ms = kernel_times(torch, stream, lambda i, arr: calls[i % R](events=arr), args.steps, 2)
    print("# stage ms:", [round(x, 4) for x in stage_ms], file=sys.stderr, flush=True)
    flops = prefill_flops(cfg)
    value = flops / (ms_per_step * 1e-3) / 1e12
    fwd_ms = stage_ms[1]
    ach = flops / (fwd_ms * 1e-3) / 1e12
    roof = {"bound": "mfma", "kernel": "prefill_fwd_kernel", "achieved": round(ach, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": load_traffic("prefill_fwd_kernel", cfg.name),
            "algorithmic_flops": flops, "avg_ms": round(fwd_ms, 5)}
    cpu = None
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline_prefill(insts[0], args.cpu_seconds)
    rec = {
        "metric": PREFILL_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name + ("" if args.tokens <= 0 and args.k < 0 else
                                           f"@T={cfg.T},k={cfg.k}"),
                   "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "d": cfg.d,
                   "T": cfg.T, "blk": cfg.blk, "k": cfg.k, "gate": "sas" if cfg.gate else "none",
                   "inputs": "bf16", "accumulation": "fp32", "instances_rotated": R},
        "calls_per_s": round(1e3 / ms_per_step, 2),
        "timing": f"median of {LOOPS} loops of {args.steps} calls, {R} instances rotated, "
                  f"after the sustained loop",
        "loops_ms": tm["loops_ms"],
        "sustained": tm["sustained"],
        "algorithmic_flops_per_call": flops,
        "attended_pairs_per_call": prefill_pairs(cfg),
        "algorithmic_bytes_per_call": prefill_bytes(cfg),
        "event_ms_per_step": round(tm["event_ms_per_step"], 5),
        "stage_ms": [round(x, 5) for x in stage_ms],
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def run_gist_prefill(args, torch, configs, ops):
    from top_chunk_sparse_amd.synth import make_gist_prefill
    import ctypes
    cfg = configs.GIST_PREFILL_CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    R = max(1, min(args.instances, 2))
    print(f"# generating {R} instance(s) of {cfg.name}", file=sys.stderr, flush=True)
    insts = [make_gist_prefill(cfg, configs.seed_for(cfg.name, r), device=dev) for r in range(R)]
    calls = [ops.GistPrefillCall(inp) for inp in insts]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        calls[i % R]()
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)
    tm = timing_summary(torch, stream, lambda i: calls[i % R](), args.steps)
    ms_per_step = tm["ms_per_step"]
    # gist gather, query rows (gist rows and raw rows in one launch)
    stage_ms = kernel_times(torch, stream, lambda i, arr: calls[i % R](events=arr), args.steps, 2)
    print("# stage ms:", [round(x, 4) for x in stage_ms], file=sys.stderr, flush=True)
    raw_pairs, gist_pairs = gist_prefill_pairs(cfg)
    flops = 4 * cfg.d * (raw_pairs + gist_pairs)
    value = flops / (ms_per_step * 1e-3) / 1e12
    # The row launch's arithmetic intensity (FLOPs over its compulsory bytes, about 180 FLOP/B
    # at the 16K workload) is below the ridge of 2.5 PFLOP/s over 8 TB/s (312 FLOP/B): its
    # roofline is the HBM one.  The matrix-core fraction is reported beside it.
    kbytes = gist_prefill_row_bytes(cfg)
    ach = kbytes / (stage_ms[1] * 1e-3) / 1e9
    tflops = flops / (stage_ms[1] * 1e-3) / 1e12
    roof = {"bound": "hbm", "kernel": "gist_prefill_mfma_kernel (gist and raw query rows)",
            "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBPS, 4),
            "traffic": load_traffic("gist_prefill_rows", cfg.name),
            "algorithmic_bytes": kbytes, "algorithmic_flops": flops,
            "intensity_flop_per_byte": round(flops / kbytes, 1),
            "mfma_tflops": round(tflops, 1),
            "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "avg_ms": round(stage_ms[1], 5)}
    cpu = None
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline_gist_prefill(insts[0], args.cpu_seconds)
    rec = {
        "metric": GIST_PREFILL_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "d": cfg.d,
                   "M": cfg.M, "L": cfg.L, "g": cfg.g, "positions": cfg.Tp, "inputs": "bf16",
                   "accumulation": "fp32", "instances_rotated": R},
        "calls_per_s": round(1e3 / ms_per_step, 2),
        "timing": f"median of {LOOPS} loops of {args.steps} calls, {R} instances rotated, "
                  f"after the sustained loop",
        "loops_ms": tm["loops_ms"],
        "sustained": tm["sustained"],
        "algorithmic_flops_per_call": flops,
        "attended_pairs_per_call": raw_pairs + gist_pairs,
        "dense_causal_pairs_per_call": cfg.B * cfg.Hq * cfg.Tp * (cfg.Tp + 1) // 2,
        "event_ms_per_step": round(tm["event_ms_per_step"], 5),
        "stage_ms": [round(x, 5) for x in stage_ms],
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def run_prefill_backward(args, torch, configs, ops):
    from top_chunk_sparse_amd.synth import make_prefill, make_prefill_grads
    import ctypes
    cfg = prefill_cfg(args, configs)
    dev = torch.device("cuda:0")
    R = max(1, min(args.instances, 2))
    print(f"# generating {R} instance(s) of {cfg.name} (+ upstream gradients)", file=sys.stderr,
          flush=True)
    insts = [make_prefill(cfg, configs.seed_for(cfg.name, r), device=dev) for r in range(R)]
    grads = [make_prefill_grads(cfg, configs.seed_for(cfg.name, r), device=dev) for r in range(R)]
    fwds = [ops.PrefillCall(inp)() for inp in insts]   # out and lse for the backward (untimed)
    calls = [ops.PrefillBwdCall(inp, f, g[0], g[1]) for inp, f, g in zip(insts, fwds, grads)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    for i in range(args.warmup):
        calls[i % R]()
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)
    tm = timing_summary(torch, stream, lambda i: calls[i % R](), args.steps)
    ms_per_step = tm["ms_per_step"]
    # per-kernel durations: select, prep (D rows and chosen-by lists), gradients (dq, dk, dv
    # in one grid), dS
    stage_ms = kernel_times(torch, stream, lambda i, arr: calls[i % R](events=arr), args.steps, 4)
    print("# stage ms:", [round(x, 4) for x in stage_ms], file=sys.stderr, flush=True)
    flops = prefill_bwd_flops(cfg)
    value = flops / (ms_per_step * 1e-3) / 1e12
    # dominant kernel: the gradient kernel, credited with the algorithmic five products per
    # pair (it executes seven: q.k and dout.v are formed once for dq and once for dk / dv)
    dom = 2
    name, kflops = "prefill_bwd_grad_kernel", prefill_bwd_flops(cfg, 5)
    ach = kflops / (stage_ms[dom] * 1e-3) / 1e12
    roof = {"bound": "mfma", "kernel": name, "achieved": round(ach, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": load_traffic(name, cfg.name),
            "algorithmic_flops": kflops, "avg_ms": round(stage_ms[dom], 5)}
    cpu = None
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline_prefill_backward(insts[0], grads[0][0], grads[0][1], args.cpu_seconds)
    rec = {
        "metric": PREFILL_BWD_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name + "_backward", "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv,
                   "d": cfg.d, "T": cfg.T, "blk": cfg.blk, "k": cfg.k,
                   "gate": "sas" if cfg.gate else "none", "inputs": "bf16",
                   "accumulation": "fp32", "instances_rotated": R},
        "calls_per_s": round(1e3 / ms_per_step, 2),
        "timing": f"median of {LOOPS} loops of {args.steps} calls, {R} instances rotated, "
                  f"after the sustained loop",
        "loops_ms": tm["loops_ms"],
        "sustained": tm["sustained"],
        "algorithmic_flops_per_call": flops,
        "attended_pairs_per_call": prefill_pairs(cfg),
        "event_ms_per_step": round(tm["event_ms_per_step"], 5),
        "stage_ms": [round(x, 5) for x in stage_ms],
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--instances", type=int, default=3)
    ap.add_argument("--workload", default="llama31_8b_decode_128k")
    ap.add_argument("--gist-mode", choices=["all", "selected"], default="all",
                    help="decode softmax set: every historical gist (default) or only the "
                         "selected chunks' gists")
    ap.add_argument("--tokens", type=int, default=0,
                    help="override the workload's context length (decode N, prefill T)")
    ap.add_argument("--k", type=int, default=-1,
                    help="override k (a value >= the chunk or block count selects all of them)")
    ap.add_argument("--top-p", type=float, default=0.0,
                    help="decode selection: 0 = top-k; in (0, 1] = top-p with a cap of k")
    ap.add_argument("--head-select", action="store_true",
                    help="decode selection: every query head picks its own top-k and the union "
                         "is unfolded (one level; runs the workload with the gate off)")
    ap.add_argument("--adaptive-k", action="store_true",
                    help="decode selection: adaptive top-k, one budget per level (k, k2 caps)")
    ap.add_argument("--backward", action="store_true",
                    help="prefill workloads: time the gradients (dq, dk, dv, dS) instead of "
                         "the forward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
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

    torch.cuda.set_device(0)
    if args.copy_probe:   # a copy of known size, to scale the HBM byte counters
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload in configs.GIST_PREFILL_CONFIGS:
        return run_gist_prefill(args, torch, configs, ops)
    if args.workload in configs.PREFILL_CONFIGS:
        if args.backward:
            return run_prefill_backward(args, torch, configs, ops)
        return run_prefill(args, torch, configs, ops)
    cfg = configs.DECODE_CONFIGS[args.workload]
    if args.tokens > 0:
        cfg = cfg.with_(N=args.tokens)
    if args.k >= 0:
        cfg = cfg.with_(k=args.k)
    if args.head_select:
        cfg = cfg.with_(gate=0)   # per-head selection carries no gate
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    R = max(1, args.instances)
    print(f"# generating {R} instance(s) of {cfg.name}", file=sys.stderr, flush=True)
    insts = [make_decode(cfg, configs.seed_for(cfg.name, r), device=dev) for r in range(R)]
    gmode = ops.GISTS_SELECTED if args.gist_mode == "selected" else ops.GISTS_ALL
    calls = [ops.DecodeCall(inp, with_scores=False, gist_mode=gmode, top_p=args.top_p,
                            head_select=int(args.head_select), adaptive_k=int(args.adaptive_k))
             for inp in insts]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    for i in range(args.warmup):
        calls[i % R]()
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)

    # ---- timed region: LOOPS loops of exactly K calls, rotating over the R instances ----
    tm = timing_summary(torch, stream, lambda i: calls[i % R](), args.steps)
    ms_per_step = tm["ms_per_step"]
    value = 1e3 / ms_per_step
    # warm: the same loops on instance 0 alone (its data partly held by the 256 MB cache)
    warm = timing_summary(torch, stream, lambda i: calls[0](), args.steps)

    # ---- per-kernel durations: the same K calls, each kernel bracketed by its own events ----
    nst = ops.decode_stage_count(calls[0].p)
    stage_ms = kernel_times(torch, stream, lambda i, arr: calls[i % R](events=arr), args.steps, nst)
    print("# stage ms:", [round(x, 4) for x in stage_ms], file=sys.stderr, flush=True)

    k_eff_mean = None
    if args.top_p > 0 or args.head_select or args.adaptive_k:   # chunks each unit kept
        import numpy as np
        k_eff_mean = float(np.mean([(c.sel >= 0).sum(-1).float().mean().item() for c in calls]))
    total_bytes, parts = decode_bytes(cfg, gist_mode=args.gist_mode, k_eff_mean=k_eff_mean)
    eff_gbps = total_bytes / (ms_per_step * 1e-3) / 1e9
    # dominant kernel: gist scoring (stage 1) -- the largest byte stream of the call
    gk_bytes = gist_kernel_bytes(cfg, args.gist_mode) if cfg.levels == 1 else None
    roof = None
    if gk_bytes:
        gk_ms = stage_ms[0]
        ach = gk_bytes / (gk_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "gist_kernel", "achieved": round(ach, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4),
                "traffic": load_traffic("gist_kernel", cfg.name) if args.gist_mode == "all" else None,
                "algorithmic_bytes": gk_bytes, "avg_ms": round(gk_ms, 5)}

    ceiling = stream_read_ceiling(torch, ops, dev)
    cpu = None
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(insts[0], args.cpu_seconds,
                           gists_in_softmax="selected" if args.gist_mode == "selected" else True,
                           top_p=args.top_p, head_select=int(args.head_select),
                           adaptive_k=int(args.adaptive_k))

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
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name + ("" if args.tokens <= 0 and args.k < 0 else
                                           f"@N={cfg.N},k={cfg.k}"),
                   "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "d": cfg.d,
                   "N": cfg.N, "C": cfg.C, "g": cfg.g, "k": cfg.k, "gate": "sas" if cfg.gate else
                   "none", "levels": cfg.levels, "paged": cfg.paged, "gists": args.gist_mode,
                   "top_p": args.top_p or None,
                   "select": "per-head union" if args.head_select else "per KV head",
                   "k_mode": "adaptive" if args.adaptive_k else "fixed",
                   "inputs": "bf16", "accumulation": "fp32",
                   "instances_rotated": R},
        "timing": f"median of {LOOPS} loops of {args.steps} calls after the sustained loop, cold: "
                  f"{R} instances rotated "
                  f"({R * total_bytes / 2 ** 30:.2f} GiB of algorithmic bytes per rotation)",
        "effective_GBps": round(eff_gbps, 1),
        "chunks_selected_mean": k_eff_mean,
        "pct_of_hbm_peak": round(100 * eff_gbps / HBM_PEAK_GBPS, 2),
        "pct_of_stream_read_ceiling": round(100 * eff_gbps / ceiling["GBps"], 2),
        "stream_read_ceiling": ceiling,
        "algorithmic_bytes_per_call": total_bytes,
        "event_ms_per_step": round(tm["event_ms_per_step"], 5),
        "loops_ms": tm["loops_ms"],
        "sustained": tm["sustained"],
        "warm": {"label": "warm: instance 0 only, partly cache-resident",
                 "calls_per_s": round(1e3 / warm["ms_per_step"], 2),
                 "ms_per_step": round(warm["ms_per_step"], 5)},
        "stage_ms": [round(x, 5) for x in stage_ms],
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
