"""Routed-core forward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mid_bf16]

One step = one whole routed-core forward (all D depths: windowing, router,
bucketing, grouped GEMMs, window attention, gated blend) over one batch of
synthetic inputs already resident in HBM.  Prints one JSON line with
tokens/s, the roofline of the dominant kernel (measured with HIP events on
the launch stream), the grouped GEMMs' MFMA utilisation, and the CPU
oracle's rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "routed-core fwd tokens/sec on 1 MI355X; MFMA util % of bf16 peak"
PEAK_BF16_TFLOPS = 2500.0   # dense bf16 MFMA, MI355X
PEAK_HBM_GBS = 8000.0


def gemm_flops(cfg, tokens=None):
    """Algorithmic FLOPs per launch (one depth) of each grouped GEMM kind
    (every token is one grouped row: ``tokens`` of them, default batch n)."""
    T, d, f = (cfg.tokens if tokens is None else tokens), cfg.d, cfg.d_ffn
    up = 2 * f if cfg.mlp == "swiglu" else f
    return {"gemm_qkv": 2.0 * T * 3 * d * d, "gemm_o": 2.0 * T * d * d,
            "gemm_gate_up": 2.0 * T * up * d, "gemm_down": 2.0 * T * d * f}


def hbm_bytes(cfg, tokens=None):
    """Algorithmic HBM bytes per launch (one depth) of the bandwidth-bound
    kernels, and of the down projection's scatter epilogue (read and write of
    the fp32 residual rows)."""
    T, d = (cfg.tokens if tokens is None else tokens), cfg.d
    act = 2 if cfg.dtype == "bf16" else 4
    return {"pool": 4.0 * T * d,                        # read s
            "norm_attn": (4.0 + act) * T * d,           # read s, write u
            "win_attn": act * 4.0 * T * d,              # read q, k, v; write o
            "gemm_down (scatter epilogue)": 8.0 * T * d}


def measure_ceilings(torch, B):
    """What this GPU sustains, measured before the timed region: the bf16
    matrix cores on register-only operands, identical and random (the clock
    follows the power draw, which follows the operands' bit activity), and a
    plain device-to-device copy of 1 GiB (read + written bytes / time)."""
    out = {}
    nbytes = B.load().lol_measure_mfma_bf16_scratch_size()
    scratch = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    # 16x16x32 is the grouped GEMMs' instruction (the random-operand figure
    # is the ceiling their roofline fraction is also quoted against); 32x32x16
    # for comparison
    for shape in (16, 32):
        for name, rnd in (("identical_operands", False), ("random_operands", True)):
            tf, ghz = B.lol_measure_mfma_bf16(shape, rnd, 20000, scratch.data_ptr(), nbytes, st)
            out[f"mfma_bf16_{shape}x{shape}_{name}"] = {"tflops": tf, "clock_ghz": ghz}
    del scratch
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = None
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) / 1e3
        best = t if best is None else min(best, t)
    out["hbm_copy_gbs"] = 2 * src.numel() / best / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return out


def oracle_threads():
    """(threads the oracle's numpy/BLAS calls use, host cores this process
    may run on).  The oracle is numpy float64; its matrix products run on
    the BLAS thread pool, everything else on one thread."""
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    try:
        host = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):  # pragma: no cover
        host = os.cpu_count() or 1
    return int(threads), int(host)


def cpu_baseline(inp, budget_s=12.0, lengths=None):
    """The oracle, unchanged, on whole documents of the workload, one after
    another until about ``budget_s`` seconds of CPU work are done
    (``lengths``: packed documents, document b = the first lengths[b]
    tokens of row b)."""
    import oracle
    threads, host = oracle_threads()
    cfg = inp.cfg
    lens = [cfg.n] * cfg.batch if lengths is None else [int(x) for x in lengths]
    done, tokens, t0 = 0, 0, time.perf_counter()
    while done < cfg.batch:
        oracle.forward(inp, forced_expert=inp.forced_expert, rows=[done], n_tokens=lens[done])
        tokens += lens[done]
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "host_cores": host,
            "kind": "oracle",
            "sample": f"{done} of {cfg.batch} documents of {cfg.name} ({tokens} tokens x "
                      f"{cfg.D} depths), numpy float64 (BLAS on {threads} threads, the rest on "
                      f"one), {dt:.1f} s"}


# source files that define each kernel kind's code and launch shape
KERNEL_SOURCES = {
    "gemm_qkv": ("gemm.hip", "lol_internal.h"), "gemm_o": ("gemm.hip", "lol_internal.h"),
    "gemm_gate_up": ("gemm.hip", "lol_internal.h"), "gemm_down": ("gemm.hip", "lol_internal.h"),
    "win_attn": ("block.hip", "lol_internal.h"), "norm_attn": ("block.hip", "lol_internal.h"),
    "pool": ("route.hip", "lol_internal.h"), "route": ("route.hip", "lol_internal.h"),
}


def kernel_sources_digest(kernel):
    """sha256 over the HIP sources of ``kernel``, to tell whether stored
    counters are stale."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "runtime_routed_transformer_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), "rb") as fh:
            h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()


def stored_traffic(kernel, workload):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 PMC
    summary (FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel's reading), or
    None if there is none or the kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    try:
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(blob)
    except (IndexError, ValueError):
        return None
    if rec.get("sources_sha256") != kernel_sources_digest(kernel):
        return None
    return float(rec["bytes_per_launch"])


FULL_METRIC = ("full-model fwd tokens/sec on 1 MI355X (embedding, causal prelude, routed core, "
               "causal coda, vocabulary readout)")


def bench_full(args):
    """The whole forward of Algorithm 1 (``--workload full_*``): the same
    protocol as the routed core, with the readout GEMM among the candidates
    for the dominant kernel."""
    import torch
    from runtime_routed_transformer_amd import binding as B
    from runtime_routed_transformer_amd.model import DeviceModel
    from runtime_routed_transformer_amd.workloads import FULL_BY_NAME, FullConfig, generate_full

    fcfg = FULL_BY_NAME[args.workload]
    cc = fcfg.core
    model = DeviceModel(generate_full(fcfg), "cuda:0")
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        model.forward(stream)
    torch.cuda.synchronize()

    # breakdown (untimed): events after every step, and the library's
    # per-kernel events inside the three lol_core_forward calls
    B.lol_core_timing_collect()
    B.lol_core_timing_enable(B.LOL_TIMING_ALL)
    step_ms = {k: 0.0 for k in DeviceModel.STEPS}
    for _ in range(args.timing_steps):
        marks = []

        def after(step):
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(stream)
            marks.append((step, ev))

        start = torch.cuda.Event(enable_timing=True)
        start.record(stream)
        model.forward(stream, after=after)
        torch.cuda.synchronize()
        prev = start
        for step, ev in marks:
            step_ms[step] += prev.elapsed_time(ev) / args.timing_steps
            prev = ev
    B.lol_core_timing_enable(0)
    kt = B.lol_core_timing_collect()
    per_kernel = {k: {"ms_avg": v[0] / max(v[1], 1), "launches": v[1]} for k, v in kt.items() if v[1]}
    flops = gemm_flops(cc)
    flops["lm_head"] = 2.0 * cc.tokens * cc.d * fcfg.vocab
    per_fwd = {k: kt[k][0] / args.timing_steps for k in flops if k in kt}
    per_fwd["lm_head"] = step_ms["lm_head"]
    dominant = max(per_fwd, key=per_fwd.get)
    layers = fcfg.prelude + cc.D + fcfg.coda

    # timed region: K whole forwards; the dominant kernel timed with HIP
    # events on the launch stream (library events at one depth per forward,
    # or torch events around the readout)
    head_evs = []
    if dominant != "lm_head":
        B.lol_core_timing_enable(1 << B.kernel_kind(dominant))
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        B.lol_core_timing_depth(i % max(cc.D, fcfg.prelude, fcfg.coda))
        if dominant == "lm_head":
            pair = []

            def after(step, pair=pair):
                if step in ("coda", "lm_head"):
                    ev = torch.cuda.Event(enable_timing=True)
                    ev.record(stream)
                    pair.append(ev)

            model.forward(stream, after=after)
            head_evs.append(pair)
        else:
            model.forward(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    B.lol_core_timing_enable(0)
    B.lol_core_timing_depth(-1)
    ms = ev0.elapsed_time(ev1) / args.steps
    if dominant == "lm_head":
        dom_n = len(head_evs)
        dom_ms = sum(a.elapsed_time(b) for a, b in head_evs) / dom_n
    else:
        dom_total, dom_n = B.lol_core_timing_collect()[dominant]
        dom_ms = dom_total / dom_n
    achieved = flops[dominant] / (dom_ms / 1e3) / 1e12
    gemm_flops_fwd = sum(flops[k] * layers for k in gemm_flops(cc)) + flops["lm_head"]
    gemm_ms_fwd = sum(per_fwd[k] for k in per_fwd)
    result = {
        "metric": FULL_METRIC, "value": cc.tokens / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cc.dtype,
        "data": "synthetic (seeded uniform token ids, N(0,0.02) weights)",
        "config": {"workload": fcfg.name, "batch": cc.batch, "n": cc.n, "d": cc.d,
                   "heads": cc.n_heads, "d_ffn": cc.d_ffn, "mlp": cc.mlp, "vocab": fcfg.vocab,
                   "prelude": fcfg.prelude, "coda": fcfg.coda, "L": cc.L, "D": cc.D, "W": cc.W,
                   "S": cc.S, "film": cc.film, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": dominant, "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "kernel_ms_avg": dom_ms, "kernel_launches_timed": dom_n,
                     "flops_per_launch": flops[dominant]},
        "mfma_util_pct": 100.0 * gemm_flops_fwd / (gemm_ms_fwd / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
        "steps_ms": step_ms,
        "kernels": per_kernel,
    }
    if not args.no_cpu_baseline:
        # the oracle's composition on one 2,048-token document of the same model
        n_s = min(cc.n, 2048)
        sample = FullConfig(f"{fcfg.name}@1x{n_s}", cc.scaled(1, n_s), fcfg.vocab, fcfg.prelude,
                            fcfg.coda, fcfg.seed)
        full = generate_full(sample)
        import oracle
        threads, host = oracle_threads()
        t0 = time.perf_counter()
        oracle.full_forward(full, core_forced_expert=full.core.forced_expert)
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": n_s / dt, "unit": "tokens/s", "cores": threads,
                                  "host_cores": host, "kind": "oracle",
                                  "sample": f"one {n_s}-token document of {fcfg.name}, numpy "
                                            f"float64, {dt:.1f} s"}
    print(json.dumps(result), flush=True)
    return 0


DECODE_METRIC = ("routed-core incremental decode tokens/sec on 1 MI355X (one token per document "
                 "per step through every routed depth)")


def decode_weight_bytes(cfg):
    """Bytes of one expert's matrices read by each projection kind."""
    act = 2 if cfg.dtype == "bf16" else 4
    d, f = cfg.d, cfg.d_ffn
    up = 2 * f if cfg.mlp == "swiglu" else f
    return {"gemm_qkv": 3 * d * d * act, "gemm_o": d * d * act, "gemm_gate_up": up * d * act,
            "gemm_down": f * d * act}


def decode_launch_bytes(cfg, kind, n_experts):
    """Algorithmic HBM bytes of one decode projection launch: the weights of
    the ``n_experts`` distinct experts the documents use at that depth, plus
    each document's input and output rows."""
    act = 2 if cfg.dtype == "bf16" else 4
    d, f, B = cfg.d, cfg.d_ffn, cfg.batch
    io = {"gemm_qkv": B * (d * act + 3 * d * 4), "gemm_o": B * (d * act + 2 * d * 4),
          "gemm_gate_up": B * (d * act + f * act), "gemm_down": B * (f * act + 3 * d * 4)}
    return n_experts * decode_weight_bytes(cfg)[kind] + io[kind]


def bench_decode(args):
    """Incremental decode (``--workload <core>_decode``): documents of the
    core workload are decoded token by token from position 0; one step = one
    token of every document through all D depths.  W untimed steps warm up,
    the state is reset, then K steps (positions 0..K-1) are timed.  The
    dominant projection is timed with HIP events at one depth per step."""
    import numpy as np
    import torch
    from runtime_routed_transformer_amd import binding as B
    from runtime_routed_transformer_amd.core import DeviceCore, DeviceDecoder
    from runtime_routed_transformer_amd.workloads import CONFIG_BY_NAME, generate, load_skewed_bias

    base = args.workload[: -len("_decode")]
    inp = generate(CONFIG_BY_NAME[base])
    cfg = inp.cfg
    load_skewed_bias(inp)   # the stored calibrated bias (skewed workloads only)
    steps = args.steps if args.steps is not None else min(cfg.n, 2 * cfg.W)
    if steps > cfg.n or args.warmup > cfg.n:
        raise SystemExit(f"--steps and --warmup must be at most n = {cfg.n} positions")
    core = DeviceCore(inp, "cuda:0")
    core.set_forcing(inp.forced_expert)
    dec = DeviceDecoder(core)
    stream = torch.cuda.current_stream()
    xs = core.s0.transpose(0, 1).contiguous()    # [n][batch][d]: token p of every document
    core.s0 = core.s_out = None

    def run(n_steps):
        dec.reset(stream)
        for p in range(n_steps):
            dec.step(p, xs[p], stream=stream)

    run(args.warmup)
    torch.cuda.synchronize()
    # per-kernel breakdown over a whole untimed pass of the timed positions
    B.lol_core_timing_collect()
    B.lol_core_timing_enable(B.LOL_TIMING_ALL)
    run(steps)
    torch.cuda.synchronize()
    B.lol_core_timing_enable(0)
    kt = B.lol_core_timing_collect()
    per_kernel = {k: {"ms_avg": v[0] / max(v[1], 1), "launches": v[1]} for k, v in kt.items() if v[1]}
    kinds = ("gemm_qkv", "gemm_o", "gemm_gate_up", "gemm_down")
    dominant = max(kinds, key=lambda k: kt[k][0])

    # timed region
    B.lol_core_timing_enable(1 << B.kernel_kind(dominant))
    dec.reset(stream)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for p in range(steps):
        B.lol_core_timing_depth(p % cfg.D)
        dec.step(p, xs[p], stream=stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    B.lol_core_timing_enable(0)
    B.lol_core_timing_depth(-1)
    assert dec.flags() == 0, "decode state flagged an error"
    ms = ev0.elapsed_time(ev1) / steps
    dom_total, dom_n = B.lol_core_timing_collect()[dominant]
    # distinct experts of every (position, depth) from the path the timed run wrote
    pe = core.path_expert.cpu().numpy()
    n_exp = np.zeros((steps, cfg.D), np.int64)
    for p in range(steps):
        for l in range(cfg.D):
            k = (p + (l * cfg.S) % cfg.W) // cfg.W
            n_exp[p, l] = len(set(pe[l, :, k].tolist()))
    timed_bytes = sum(decode_launch_bytes(cfg, dominant, n_exp[p, p % cfg.D]) for p in range(steps))
    achieved = timed_bytes / (dom_total / 1e3) / 1e9
    step_bytes = sum(decode_launch_bytes(cfg, k, n_exp[p, l]) for k in kinds
                     for p in range(steps) for l in range(cfg.D)) / steps
    proj_ms = sum(kt[k][0] for k in kinds) / steps
    # the same K steps replayed from a HIP graph of one step (each row at its
    # own position, pos = -1), after the timed region: the host issues one
    # graph launch and one 16-byte-row input copy per step
    x_in = torch.empty((cfg.batch, cfg.d), dtype=torch.float32, device=xs.device)
    y_out = torch.empty_like(x_in)
    dec.reset(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dec.step(None, x_in, y=y_out)
    dec.reset(stream)
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for p in range(steps):
        x_in.copy_(xs[p])
        graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    assert dec.flags() == 0, "decode state flagged an error (graph replay)"
    graph_ms = g0.elapsed_time(g1) / steps
    result = {
        "metric": DECODE_METRIC, "value": cfg.batch / (ms / 1e3), "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) states, N(0,0.02) weights)",
        "config": {"workload": args.workload, "batch": cfg.batch, "positions": f"0..{steps - 1}",
                   "d": cfg.d, "heads": cfg.n_heads, "d_ffn": cfg.d_ffn, "mlp": cfg.mlp,
                   "L": cfg.L, "D": cfg.D, "W": cfg.W, "S": cfg.S, "film": cfg.film,
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": None, "kernel_ms_avg": dom_total / dom_n,
                     "kernel_launches_timed": dom_n,
                     "bytes_per_launch_avg": timed_bytes / dom_n},
        "projections_gbs": step_bytes / (proj_ms / 1e3) / 1e9,
        "graph_replay": {"ms_per_step": graph_ms, "tokens_per_s": cfg.batch / (graph_ms / 1e3)},
        "distinct_experts_per_depth_avg": float(n_exp.mean()),
        "kernels": per_kernel,
    }
    if not args.no_cpu_baseline:
        import oracle
        threads, host = oracle_threads()
        # the oracle's decode on document 0, a growing prefix until ~10 s of work
        n_s, dt = 8, 0.0
        while True:
            t0 = time.perf_counter()
            oracle.decode(inp, n_s, forced_expert=inp.forced_expert, rows=[0])
            dt = time.perf_counter() - t0
            if dt >= 5.0 or n_s >= steps:
                break
            n_s = min(steps, n_s * 2)
        result["cpu_baseline"] = {"value": n_s / dt, "unit": "tokens/s", "cores": threads,
                                  "host_cores": host, "kind": "oracle",
                                  "sample": f"oracle.decode of positions 0..{n_s - 1} of document "
                                            f"0 of {base}, numpy float64, {dt:.1f} s"}
    print(json.dumps(result), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 24; decode workloads: 2 W positions)")
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mid_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the matrix-core and copy ceilings measured before the timed region")
    ap.add_argument("--timing-steps", type=int, default=3)
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the routed core shards over documents with no forward communication; "
              "the multi-GPU path is not built)", file=sys.stderr)
        return 2

    from runtime_routed_transformer_amd.workloads import FULL_BY_NAME
    if args.workload.endswith("_decode"):
        return bench_decode(args)
    if args.steps is None:
        args.steps = 24
    if args.workload in FULL_BY_NAME:
        return bench_full(args)

    import torch
    from runtime_routed_transformer_amd import binding as B
    from runtime_routed_transformer_amd.core import DeviceCore
    from runtime_routed_transformer_amd.workloads import (CONFIG_BY_NAME, PACKED_BY_NAME,
                                                          generate, generate_packed,
                                                          load_skewed_bias)

    packed = None
    if args.workload in PACKED_BY_NAME:
        # packed documents: one token stream, a document table
        packed = generate_packed(PACKED_BY_NAME[args.workload])
        inp = packed.core
    else:
        inp = generate(CONFIG_BY_NAME[args.workload])
    cfg = inp.cfg
    load_skewed_bias(inp)   # the stored calibrated bias (skewed workloads only)
    core = DeviceCore(inp, "cuda:0")
    core.set_forcing(inp.forced_expert)
    stream = torch.cuda.current_stream()
    if packed is None:
        tokens = cfg.tokens

        def forward():
            core.forward(stream=stream)
    else:
        tokens = int(packed.length.sum())
        p_in = torch.from_numpy(packed.stream()).to(core.device)
        p_out = torch.empty_like(p_in)
        p_start = torch.from_numpy(packed.start).to(core.device)
        p_len = torch.from_numpy(packed.length).to(core.device)
        core.s0 = core.s_out = None   # the [batch][n] layout is not used

        def forward():
            core.forward_docs(p_in, p_out, p_start, p_len, stream=stream)
    # one plain device-to-device copy of s^(0) (untimed): the reference
    # kernel that the HBM-traffic counters of the profiles are scaled by
    s_ref = core.s0 if packed is None else p_in
    torch.empty_like(s_ref).copy_(s_ref)
    ceilings = None if args.no_ceilings else measure_ceilings(torch, B)

    for _ in range(args.warmup):
        forward()
    torch.cuda.synchronize()

    # per-kernel breakdown: HIP events the library records on the launch
    # stream around every kernel, over a few extra (untimed) steps
    B.lol_core_timing_collect()  # drop anything stale
    B.lol_core_timing_enable(B.LOL_TIMING_ALL)
    for _ in range(args.timing_steps):
        forward()
    torch.cuda.synchronize()
    B.lol_core_timing_enable(0)
    kt = B.lol_core_timing_collect()
    flops = gemm_flops(cfg, tokens)
    per_kernel = {k: {"ms_avg": v[0] / max(v[1], 1), "launches": v[1]} for k, v in kt.items() if v[1]}
    dominant = max(flops, key=lambda k: kt[k][0])
    gemm_ms = sum(kt[k][0] for k in flops) / args.timing_steps
    gemm_tflops = sum(flops.values()) * cfg.D / (gemm_ms / 1e3) / 1e12

    # timed region: K whole forwards.  HIP events on the launch stream time
    # the dominant kernel; each timed launch costs the stream a few
    # microseconds, so every forward times it at one depth, the depth
    # advancing from step to step (all depths are sampled when K >= D)
    B.lol_core_timing_enable(1 << B.kernel_kind(dominant))
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        B.lol_core_timing_depth(i % cfg.D)
        forward()
    ev1.record(stream)
    torch.cuda.synchronize()
    B.lol_core_timing_enable(0)
    B.lol_core_timing_depth(-1)
    ms = ev0.elapsed_time(ev1) / args.steps
    if packed is not None:
        assert core.flags() == 0, "document table rejected by the device"
    tokens_per_s = tokens / (ms / 1e3)
    dom_total, dom_n = B.lol_core_timing_collect()[dominant]
    dom_ms = dom_total / dom_n
    achieved = flops[dominant] / (dom_ms / 1e3) / 1e12
    traffic = stored_traffic(dominant, cfg.name)
    result = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) states, N(0,0.02) weights)",
        "config": {"workload": cfg.name, "batch": cfg.batch, "n": cfg.n, "d": cfg.d,
                   "heads": cfg.n_heads, "d_ffn": cfg.d_ffn, "mlp": cfg.mlp, "L": cfg.L,
                   "D": cfg.D, "W": cfg.W, "S": cfg.S, "film": cfg.film,
                   "router": cfg.router, "film_mode": cfg.film_mode,
                   "parallelism": "single GPU"},
        "packed": None if packed is None else {
            "documents": cfg.batch, "tokens": tokens, "n_tokens": packed.n_tokens,
            "lengths": "log-uniform %d..%d, seed %d" % (packed.cfg.min_len, cfg.n, packed.cfg.seed),
            "min_len": int(packed.length.min()), "max_len": int(packed.length.max())},
        "roofline": {"bound": "mfma", "kernel": dominant, "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                     "kernel_ms_avg": dom_ms, "kernel_launches_timed": dom_n,
                     "flops_per_launch": flops[dominant],
                     # the same kernel against the matrix-core rate this GPU
                     # sustains on random operands (measured below)
                     "frac_of_measured_ceiling": None if ceilings is None else
                     achieved / ceilings["mfma_bf16_16x16_random_operands"]["tflops"]},
        "ceilings": ceilings,
        "mfma_util_pct": 100.0 * gemm_tflops / PEAK_BF16_TFLOPS,
        "grouped_gemm_tflops": gemm_tflops,
        # bandwidth-bound kernels: algorithmic bytes / mean duration (the
        # scatter entry is a lower bound: the down kernel also does its GEMM)
        "hbm_gbs": {k: b / (kt[k.split(" ")[0]][0] / max(kt[k.split(" ")[0]][1], 1) / 1e3) / 1e9
                    for k, b in hbm_bytes(cfg, tokens).items() if kt.get(k.split(" ")[0], (0, 0))[1]},
        "kernels": per_kernel,
    }
    if ceilings is not None:
        result["hbm_frac_of_copy"] = {k: v / ceilings["hbm_copy_gbs"]
                                      for k, v in result["hbm_gbs"].items()}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, lengths=None if packed is None else packed.length)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
