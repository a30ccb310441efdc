#!/usr/bin/env python3
"""Benchmark of the frame-wise Gated DeltaNet forward on one MI355X.

A step is one gdn_fwd over the whole workload (for the streaming workload:
the chain of gdn_chunk_step calls), inputs already resident in HBM.  Prints
ONE JSON line: tokens/s per GDN layer, the path's kernel against the HBM
roofline, and the fp64 CPU oracle timed on this host as a baseline.

    python bench.py [--gpus 1] [--steps 20] [--warmup 50] [--workload clip_241f]

The first tens of calls in a process run slower than the steady state (on the
241-frame layer ~7 % with 5 untimed calls, under 1 % from 50 on, measured in
separate processes), so 50 untimed steps precede the timed ones.

On the MFMA path one gdn_fwd is a short sequence of launches of a single
kernel (scan_kernel: the state pass over one chunk range merged with the
intra-chunk step of the next), and nothing else runs on the stream, so HIP
events on that stream around the timed steps measure that kernel (the gaps
between its launches included).  `roofline.achieved` is the algorithmic bytes
of one step over that time.

`roofline.traffic` is the kernel's measured HBM bytes per step from
profiles/traffic_scan_<workload>.json, reported only while the hash of the
kernel's sources stored there matches the sources of this tree.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published

# The state in and out of one (batch, head): 112 x 112 fp32.
STATE_BYTES = 112 * 112 * 4


def path_algorithmic_bytes(o_bytes: int, row: int = 224) -> int:
    """Bytes per token-head the forward must move by its definition: read the
    q, k, v rows (`row` bytes each: 224 in bf16, 112 in fp8) and g, beta (4 B
    each), write o (448 B fp32, 224 B bf16): 1,128 B for bf16 inputs, fp32 o."""
    return 3 * row + 8 + o_bytes


def flops_per_token_head(C: int = 80, d: int = 112) -> float:
    """Chunked-form flops per token-head: 6 d^2 + 5 C d + C^2 / 3 (triangles once)."""
    return 6 * d * d + 5 * C * d + C * C / 3


def host_cpus():
    """(CPUs this process may run on, the CPU model name)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def _oracle_rate(w, T, threads, min_seconds, bidir):
    from hybrid_linear_attention_gdn_amd.inputs import make_inputs
    from oracle.bidirectional import bidirectional
    from oracle.recurrence import gdn_recurrence
    inp = make_inputs(w, seq_len=T, frame_tokens=w.frame_tokens)
    runs, dt = 0, 0.0
    while runs == 0 or dt < min_seconds:
        t0 = time.perf_counter()
        if bidir:
            bidirectional(inp.q, inp.k, inp.v, inp.g, inp.beta, nthreads=threads)
        else:
            gdn_recurrence(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.state0, nthreads=threads, want_state=True)
        dt += time.perf_counter() - t0
        runs += 1
    return runs * w.batch * T / dt, runs, dt


def cpu_baseline(w, max_tokens: int, min_seconds: float, bidir: bool = False):
    """fp64 oracle on a bounded sample of the same workload: all (batch, head)
    units, the first `max_tokens` tokens, repeated until `min_seconds` of wall
    time have passed, on min(CPUs, B x H) threads (one unit per thread at a
    time); then the same on one thread over a tenth of the tokens."""
    nproc, model = host_cpus()
    threads = max(1, min(nproc, w.batch * w.heads))
    T = min(w.seq_len, max_tokens)
    rate, runs, dt = _oracle_rate(w, T, threads, min_seconds, bidir)
    T1 = max(80, T // 10)
    rate1, runs1, dt1 = _oracle_rate(w, T1, 1, min_seconds / 4, bidir)
    return {"value": round(rate, 1), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{w.name}: all {w.batch}x{w.heads} (batch, head) units, first {T} of {w.seq_len} tokens, "
                      f"{runs} passes ({runs * w.batch * T * w.heads} token-heads, {dt:.1f} s wall, "
                      f"fp64 C recurrence{', forward and reverse scans' if bidir else ''}, one thread per unit)",
            "seconds": round(dt, 3), "nproc": nproc, "cpu_model": model,
            "one_thread": {"value": round(rate1, 1), "unit": "tokens/s", "tokens": T1, "passes": runs1,
                           "seconds": round(dt1, 3)}}


def layer_bench(args):
    """The whole layer around the scan (gdn_layer_fwd): in-projection, scan,
    out-projection on the 241-frame shape (B = 1, 27,280 tokens, 20 heads,
    880-token frames) with seeded synthetic bf16 weights.  The projections are
    dense contractions, so their roofline is the bf16 MFMA peak.  Prints one
    JSON line of its own."""
    import numpy as np
    import torch

    from hybrid_linear_attention_gdn_amd import layer
    from hybrid_linear_attention_gdn_amd.inputs import make_layer_inputs

    B, T, H, ft = 1, 27280, 20, 880
    HD = H * 112
    dev = torch.device("cuda:0")
    li = make_layer_inputs(B, T, H, ft, 900)
    up = lambda b: torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
    x, w_in, w_out = up(li.x_bits), up(li.w_in_bits), up(li.w_out_bits)
    y_dtype = torch.float32 if args.o_dtype == "fp32" else torch.bfloat16
    bidir = args.bidir
    p = layer.problem(B, T, H, ft, y_dtype, bidir)
    ws = torch.empty(layer.workspace_bytes(p), dtype=torch.uint8, device=dev)
    st = None if bidir else torch.zeros((B, H, 112, 112), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        layer.layer_fwd(x, w_in, w_out, ft, st, st, y_dtype=y_dtype, bidirectional=bidir, workspace=ws,
                        stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps

    # each projection alone, on the same stream, timed by its own events
    qkvbg = layer.in_proj(x, w_in, ft, stream=stream)
    o_in = torch.zeros((B, T, HD), dtype=torch.bfloat16, device=dev)

    def timed(fn):
        for _ in range(2):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    t_proj = {"in_proj": timed(lambda: layer.in_proj(x, w_in, ft, stream=stream)),
              "out_proj": timed(lambda: layer.out_proj(o_in, w_out, y_dtype=y_dtype, stream=stream))}
    del qkvbg
    n_in = 3 * HD + 2 * H
    flops = {"in_proj": 2.0 * B * T * HD * n_in, "out_proj": 2.0 * B * T * HD * HD}
    proj = {k: {"ms": round(t_proj[k], 5), "tflops": round(flops[k] / (t_proj[k] * 1e-3) / 1e12, 1)}
            for k in flops}
    dom = "in_proj"
    achieved = proj[dom]["tflops"]
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import layer as LY
        Ts = min(T, 2640)
        t0 = time.perf_counter()
        runs = 0
        while runs == 0 or time.perf_counter() - t0 < args.cpu_seconds:
            LY.layer(li.x[:, :Ts], li.w_in, li.w_out, H, ft, bidirectional_scan=bidir)
            runs += 1
        dt = time.perf_counter() - t0
        cpu = {"value": round(runs * B * Ts / dt, 1), "unit": "tokens/s", "cores": host_cpus()[0],
               "kind": "oracle", "sample": f"layer: first {Ts} of {T} tokens, all {H} heads, {runs} passes, "
                                           f"{dt:.1f} s wall (numpy fp64 projections + C recurrence)"}
    out = {
        "metric": f"GDN layer (projections + {'bidirectional ' if bidir else ''}scan) tokens/s, 20h x 112d, bf16, "
                  "on 1 MI355X",
        "value": round(B * T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) x, N(0, 1/2240) weights in bf16)",
        "config": {"workload": "layer_clip_241f: 27,280 tokens, W_in 6,760 x 2,240, W_out 2,240 x 2,240"
                               + (", bidirectional scan" if bidir else ""),
                   "batch": B, "tokens": T, "heads": H, "head_dim": 112, "y_dtype": args.o_dtype},
        "roofline": {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel_ms": proj[dom]["ms"], "launches_per_step": 1.0},
        "projections": proj,
        "scan_ms_estimate": round(ms - sum(t_proj.values()), 5),
    }
    if cpu:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


def attn_bench(args):
    """The streaming attention block (include/sanawm_attn.h) at the page geometry:
    880-token frames, 3 frames per block, 2 cached blocks, 1 sink frame, 20
    heads x 112.  Blocks 0..3 fill the cache; the timed step re-runs block 3
    (stage + attention: 2,640 queries over 8,800 keys), the steady state of a
    stream.  Prints one JSON line of its own."""
    import numpy as np
    import torch

    from hybrid_linear_attention_gdn_amd import attn
    from hybrid_linear_attention_gdn_amd.inputs import make_attn_stream

    B, H, ft, fpb, C, S = 1, 20, 880, 3, 2, 1
    blocks = 4
    dev = torch.device("cuda:0")
    s = make_attn_stream(B, H, ft, fpb, blocks, 400)
    up = lambda b: torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
    Lb = s.block_tokens
    q, k, v = (up(x) for x in (s.q_bits, s.k_bits, s.v_bits))
    o_dtype = torch.float32 if args.o_dtype == "fp32" else torch.bfloat16
    p = attn.problem(B, H, ft, fpb, C, S, o_dtype)
    cache = attn.new_cache(p)
    parts = [tuple(t[:, n * Lb:(n + 1) * Lb].contiguous() for t in (q, k, v)) for n in range(blocks)]
    o = torch.empty((B, Lb, H, 112), dtype=o_dtype, device=dev)
    stream = torch.cuda.current_stream(dev)
    for n in range(blocks):
        attn.block_fwd(p, n, *parts[n], cache, o, stream)
    step = lambda: attn.block_fwd(p, blocks - 1, *parts[-1], cache, o, stream)  # noqa: E731
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    keys = 10 * ft
    flops = 4.0 * B * H * Lb * keys * 112  # Q K^T and P V, 2 flops per multiply-add
    tflops = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": "streaming attention block TFLOP/s (2,640 queries x 8,800 keys, 20h x 112d, bf16) on 1 MI355X",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded N(0,1) q/k/v)",
        "config": {"workload": "attn_block: block 3 of a stream (sink frame + 2 cached blocks + current block)",
                   "batch": B, "heads": H, "head_dim": 112, "queries": Lb, "keys": keys, "o_dtype": args.o_dtype},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None},
        "tokens_per_s": round(B * Lb / (ms * 1e-3), 1),
    }
    if not args.no_cpu_baseline:
        from oracle import attention as A
        rows = np.concatenate([np.arange(f * ft, (f + 1) * ft) for f in A.context_frames(blocks - 1, fpb, C, S)])
        runs, dt, heads = 0, 0.0, 0
        while runs == 0 or dt < args.cpu_seconds:
            h = runs % H
            t0 = time.perf_counter()
            A.attention(s.q[0, (blocks - 1) * Lb:blocks * Lb, h].astype(np.float64), s.k[0, rows, h], s.v[0, rows, h])
            dt += time.perf_counter() - t0
            runs += 1
            heads += 1
        cpu_flops = 4.0 * heads * Lb * keys * 112
        out["cpu_baseline"] = {"value": round(cpu_flops / dt / 1e12, 5), "unit": "TFLOP/s",
                               "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)),
                               "kind": "oracle", "sample": f"{heads} (head, block) attentions of 2,640 x 8,800 in "
                                                           f"fp64 numpy, {dt:.1f} s wall"}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="clip_241f")
    ap.add_argument("--o-dtype", default="fp32", choices=["fp32", "bf16"])
    ap.add_argument("--fp32-inputs", action="store_true",
                    help="upload q, k, v as fp32 (the vector-ALU kernels) instead of the workload's dtype")
    ap.add_argument("--cpu-tokens", type=int, default=1 << 30, help="tokens of the oracle's CPU sample")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum wall time of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--attn", action="store_true", help="time the streaming attention block instead of the GDN layer")
    ap.add_argument("--layer", action="store_true",
                    help="time the whole layer (projections + scan, gdn_layer_fwd) instead")
    ap.add_argument("--bidir", action="store_true",
                    help="time the bidirectional layer (forward + reverse scan, gdn_bidir_fwd) instead")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the timed steps, one plain device-to-device copy of this many MiB (a kernel of "
                         "known traffic, to calibrate memory counters under a profiler)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU only: the GDN forward's (batch, head) units "
                                   "are independent and would shard without communication; run --gpus 1"}))
        sys.exit(2)
    if args.attn:
        attn_bench(args)
        return
    if args.layer:
        layer_bench(args)
        return

    gdn_bench(args)


def gdn_bench(args):
    import numpy as np
    import torch

    from hybrid_linear_attention_gdn_amd import gdn
    from hybrid_linear_attention_gdn_amd.inputs import WORKLOADS, make_inputs
    from hybrid_linear_attention_gdn_amd.rocprof_summary import kernel_source_hash

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    inp = make_inputs(w)
    if args.fp32_inputs:
        q, k, v = (torch.from_numpy(np.asarray(a, np.float32)).to(dev) for a in (inp.q, inp.k, inp.v))
    elif inp.dtype == "bf16":
        up = lambda b: torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)  # noqa: E731
        q, k, v = up(inp.q_bits), up(inp.k_bits), up(inp.v_bits)
    elif inp.dtype == "fp8":  # E4M3FN codes
        up8 = lambda b: torch.from_numpy(b).to(dev).view(torch.float8_e4m3fn)  # noqa: E731
        q, k, v = up8(inp.q_bits), up8(inp.k_bits), up8(inp.v_bits)
    else:
        q, k, v = (torch.from_numpy(a).to(dev) for a in (inp.q, inp.k, inp.v))
    g, beta = torch.from_numpy(inp.g).to(dev), torch.from_numpy(inp.beta).to(dev)
    s0 = None if inp.state0 is None else torch.from_numpy(inp.state0).to(dev)
    del inp
    o_dtype = torch.float32 if args.o_dtype == "fp32" else torch.bfloat16
    o_bytes = 448 if args.o_dtype == "fp32" else 224
    B, T, H, d = q.shape
    row = d * q.element_size()  # bytes of one q/k/v row
    dtype_name = {torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8_e4m3", torch.float32: "f32"}[q.dtype]
    calls = w.calls
    if args.bidir and calls != 1:
        raise SystemExit("--bidir takes a one-call workload (the bidirectional layer sees the whole clip)")
    Tc = T // calls
    o = torch.empty((B, T, H, d), dtype=o_dtype, device=dev)
    st = torch.empty((B, H, d, d), dtype=torch.float32, device=dev)
    p = gdn.problem(B, Tc, H, d, d, q.dtype, o_dtype)
    lay = gdn.workspace_layout(p)
    mfma = bool(lay.mfma)
    ws = torch.empty(max(gdn.bidir_workspace_bytes(p) if args.bidir else lay.total, 1), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream(dev)
    if calls > 1:
        parts = [tuple(t[:, c * Tc:(c + 1) * Tc].contiguous() for t in (q, k, v, g, beta)) for c in range(calls)]
        o_parts = [torch.empty((B, Tc, H, d), dtype=o_dtype, device=dev) for _ in range(calls)]
    # launches of the MFMA kernel per call: one per chunk range, plus one
    N = -(-Tc // 80)
    ranges = 0
    if mfma and N > 0:
        first = lay.first_range
        ranges = 1 + -(-(N - first) // lay.range_cap) if N > first else 1
    launches_per_call = ranges + 1 if mfma else None

    def step():
        if args.bidir:
            gdn.gdn_bidir_fwd(q, k, v, g, beta, o, workspace=ws, stream=stream)
        elif calls == 1:
            gdn.gdn_fwd(q, k, v, g, beta, s0, st, o, workspace=ws, stream=stream)
        else:
            st.copy_(s0)
            for c in range(calls):
                gdn.gdn_chunk_step(*parts[c], st, st, o_parts[c], workspace=ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] {w.name}: B={B} T={T} H={H} d={d} calls={calls} kernels={'mfma' if mfma else 'portable'} "
          f"launches/call={launches_per_call} warmup done", file=sys.stderr, flush=True)

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    token_heads = B * T * H
    tokens_per_s = B * T / (ms * 1e-3)

    # the path against the HBM roofline: the method's own bytes per step (the
    # bidirectional layer reads its inputs and writes o once, no state in or out;
    # a streaming step copies the initial state once, outside the definition)
    step_bytes = path_algorithmic_bytes(o_bytes, row) * token_heads + (
        0 if args.bidir else 2 * STATE_BYTES * B * H * calls)
    achieved = step_bytes / (ms * 1e-3) / 1e9
    tflops = flops_per_token_head() * token_heads * (2 if args.bidir else 1) / (ms * 1e-3) / 1e12

    # measured HBM bytes per step of the kernel (rocprofv3 FETCH_SIZE and WRITE_SIZE,
    # calibrated on a plain copy), valid only for the sources they were taken on
    traffic = None
    stage = "scan" if mfma else "portable"
    tpath = os.path.join(ROOT, "profiles", f"traffic_{stage}_{w.name}{'_bidir' if args.bidir else ''}.json")
    if os.path.exists(tpath):
        try:
            rec = json.load(open(tpath))
            if rec.get("source_hash") == kernel_source_hash(stage, mfma) and rec.get("o_dtype") == args.o_dtype:
                traffic = rec.get("bytes_per_step")
        except (OSError, ValueError):
            traffic = None

    # cold steps: a 512 MiB buffer is written before each step (outside the timed
    # events) so that the 256 MB last-level cache holds none of the step's data
    cold_steps = min(args.steps, 10)
    flush = torch.empty((512 << 20) // 4, dtype=torch.float32, device=dev)
    cold = []
    for _ in range(cold_steps):
        flush.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        e1.synchronize()
        cold.append(e0.elapsed_time(e1))
    del flush
    cold_ms = float(np.median(cold))

    if args.copy_mib > 0:
        # an elementwise kernel (not a DMA copy, which the counters would not see):
        # reads and writes exactly copy_mib MiB
        src = torch.ones((args.copy_mib << 20) // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    kname = "scan_kernel" if mfma else "prep + portable kernels"
    out = {
        "metric": (f"GDN {'bidirectional ' if args.bidir else ''}fwd tokens/s per layer (20h×112d, {dtype_name}) "
                   "+ % MFMA peak on 1 MI355X"),
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name,
        "data": "synthetic (seeded N(0,1) q/k/v/beta logits, frame-wise log-decay -softplus(N(0,1)+2))",
        "config": {"workload": f"{w.name}: {w.note}" + (", bidirectional (forward + reverse scan)" if args.bidir
                                                           else ""), "batch": B, "tokens": T, "heads": H, "head_dim": d,
                   "calls_per_step": calls, "o_dtype": args.o_dtype, "kernels": "mfma" if mfma else "portable",
                   "chunk": 80},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_step": step_bytes,
                     "bytes_per_token_head": path_algorithmic_bytes(o_bytes, row),
                     "kernel_ms": round(ms, 5), "launches_per_step": (launches_per_call * calls * (2 if args.bidir
                                                                                                  else 1)
                                                                     if mfma else None),
                     "per": "step (all launches of the kernel in one step; HIP events on its stream)"},
        "mfma": {"tflops": round(tflops, 2), "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                 "flops_per_token_head": flops_per_token_head()},
        "cold": {"ms_per_step": round(cold_ms, 5), "tokens_per_s": round(B * T / (cold_ms * 1e-3), 1),
                 "steps": cold_steps, "note": "median over steps each preceded by a 512 MiB write"},
        "gdn_per_dit_forward_ms": {"x20_layers": round(20 * ms, 3), "x15_gdn_layers": round(15 * ms, 3)},
    }
    if calls > 1:  # streaming: latency of one call (state carried in, out) and per chunk of 80 tokens
        per_call_us = 1e3 * ms / calls
        out["streaming"] = {"us_per_call": round(per_call_us, 2),
                            "us_per_chunk": round(per_call_us / -(-(T // calls) // 80), 3),
                            "tokens_per_call": T // calls}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_tokens, args.cpu_seconds, args.bidir)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
