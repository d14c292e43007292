"""Throughput of the NVFP4 W4A4 + residual-compensation MoE hot path on one
MI355X.

    python bench.py [--steps K] [--warmup W] [--config 1..5] [--no-cpu-baseline]
                    [--no-decode] [--no-ceilings]

A step is one forward of the MoE block over one batch, inputs resident in
HBM: route and permute (moe_permute), online activation quantization with
channel scores, channel selection and residual gather, the gate+up grouped
GEMM with the residual correction (SwiGLU fused into its output where the
large-tile kernel takes the shape; --no-fuse-swiglu: into the second
quantizer instead), the second quantizer, selection, the down grouped GEMM
with correction, and the combine.  The weight QDQ of both expert tensors
(nvfp4_qdq_weights) runs once per weight sync, not per forward: it is timed
on its own (weight_qdq_ms_per_sync; ms_per_step_incl_weight_qdq adds it).

Prints ONE JSON line for the large-prefill workload (default --config 5).
`value` = algorithmic GEMM flops of a step (2 * rows * N * (K + k) summed
over both GEMMs) / wall time per step, in TFLOP/s; step_ms_events gives the
p10 / p50 / p90 of per-step HIP-event times.  The step is timed as one HIP
graph replay (captured once; the library allocates nothing and sizes every
grid from shapes, so the whole forward replays without a host launch per
kernel); ms_per_step_eager is the same step launched call by call
(--eager: eager only).  `roofline` covers the grouped
GEMM calls (their small operand-preparation kernels plus the main GEMM
kernel), timed with HIP events on the launch stream over the timed steps:
  * many rows per expert (prefill): algorithmic flops / duration against the
    dense f16/bf16 MFMA peak (the exact NVFP4 product runs on that path);
  * few rows per expert (decode): algorithmic bytes -- weights of experts
    with rows, activation codes, residual rows, output -- / duration against
    HBM bandwidth.
`traffic` is the HBM byte count of the same calls from rocprofv3 counters
(profiles/hbm_traffic.json), or null when the GEMM source has changed since
they were taken.  `decode` is the same report for the decode-sized block
(256 tokens), `rac_overhead` the correction's cost on each GEMM call
(t(k) / t(k = 0) - 1), `ceilings` the MFMA and HBM rates measured on the
chip, `gates` each target against its measurement, and `cpu_baseline` the
CPU oracle on a bounded sample of the same block.

    python bench.py --calibrate-copy     # 1 GiB device copy, for counter scaling
    python bench.py --ceilings           # MFMA and HBM ceilings only
    python bench.py --rac-sweep [--config C]   # compensation strength against cost
    python bench.py --w4a16 [--config C]       # trainer-side W4A16 product, same shapes
    python bench.py --fp8 [--config C]         # FP8 (E4M3) W8A8 baseline, same shapes
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

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense fp4 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=128)
    ap.add_argument("--cpu-experts", type=int, default=4)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device-to-device copy three times")
    ap.add_argument("--rac-sweep", action="store_true",
                    help="only sweep the number of compensated channels k on the first GEMM")
    ap.add_argument("--no-fuse-swiglu", action="store_true",
                    help="time the gate+up GEMM and the SwiGLU pass separately")
    ap.add_argument("--w4a16", action="store_true",
                    help="only time the trainer-side W4A16 product on the block's GEMM shapes")
    ap.add_argument("--fp8", action="store_true",
                    help="only time the FP8 (E4M3) W8A8 baseline on the block's GEMM shapes")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure the MFMA and HBM ceilings of this chip")
    ap.add_argument("--no-decode", action="store_true",
                    help="leave out the decode-sized block's sub-report")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="leave out the ceiling microbenchmarks")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches only (no HIP graph replay of the step)")
    return ap.parse_args()


GEMM_SOURCE = os.path.join(ROOT, "fp4_quantized_gemm_amd", "csrc", "gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def gemm_source_hash():
    with open(GEMM_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def recorded_traffic(workload):
    """HBM bytes per step of the two GEMM calls, from the committed counter
    runs, if they were taken on the current GEMM source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("gemm_source_sha256") != gemm_source_hash():
        return None
    return rec.get("hbm_bytes_per_step")


def calibrate_copy():
    import torch
    n = 1 << 28
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "copies": 3}), flush=True)


def to_dev(bits, dev):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


class Timer:
    """Durations of bracketed regions, from HIP events recorded on the
    current (launch) stream."""

    def __init__(self):
        self.pairs = []

    def start(self):
        import torch
        a = torch.cuda.Event(enable_timing=True)
        a.record()
        return a

    def stop(self, a):
        import torch
        b = torch.cuda.Event(enable_timing=True)
        b.record()
        self.pairs.append((a, b))

    def times(self):
        return [a.elapsed_time(b) for a, b in self.pairs]

    def mean_ms(self):
        t = self.times()
        return sum(t) / len(t) if t else float("nan")


def percentiles(ts):
    import numpy as np
    return {"p10": round(float(np.percentile(ts, 10)), 4),
            "p50": round(float(np.percentile(ts, 50)), 4),
            "p90": round(float(np.percentile(ts, 90)), 4)}


def median_ms(fn, reps):
    """Median of `reps` HIP-event timings of fn() (after two untimed calls)."""
    import numpy as np
    import torch
    ts = []
    for _ in range(reps + 2):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        ts.append((a, b))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ts[2:]]))


def interleaved_ms(fns, reps):
    """Medians of HIP-event timings of several calls, run in turn (so that
    clock drift affects them alike)."""
    import numpy as np
    import torch
    ts = [[] for _ in fns]
    for i in range(reps + 2):
        for j, fn in enumerate(fns):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            if i >= 2:
                ts[j].append((a, b))
    torch.cuda.synchronize()
    return [float(np.median([a.elapsed_time(b) for a, b in t])) for t in ts]


def run_block(cfg, wl, steps, warmup, fuse_swiglu=True, use_graph=True):
    """The block on one GPU.  Weight QDQ runs once per weight sync, so it is
    timed on its own; a step is one forward: route and permute, quantize,
    select, gate+up GEMM (SwiGLU fused where the large-tile kernel forms it),
    quantize h, select, down GEMM, combine."""
    import torch

    import fp4_quantized_gemm_amd as F

    dev = torch.device("cuda:0")
    x = to_dev(wl.x, dev)
    w1 = to_dev(wl.w_first, dev)
    w2 = to_dev(wl.w_down, dev) if wl.w_down is not None else None
    logits = bias = None
    if wl.logits is not None:
        logits = torch.from_numpy(wl.logits).to(dev)
        bias = torch.from_numpy(wl.bias).to(dev) if wl.bias is not None else None
    torch.cuda.synchronize()

    def qdq():
        return (F.nvfp4_qdq_weights(w1, want_qdq=False),
                F.nvfp4_qdq_weights(w2, want_qdq=False) if w2 is not None else None)

    qdq_ms = median_ms(qdq, max(3, steps // 4))
    W1, W2 = qdq()
    del w1, w2
    torch.cuda.empty_cache()

    timers = {n: Timer() for n in ("permute", "quant1", "select1", "gemm1", "quant2",
                                   "select2", "gemm2", "combine")}
    record = [False]
    fuse = fuse_swiglu and W2 is not None

    def timed(name, fn, *a, **kw):
        if not record[0]:
            return fn(*a, **kw)
        t0 = timers[name].start()
        r = fn(*a, **kw)
        timers[name].stop(t0)
        return r

    def gemm1(q, perm, R, S, offs, rows):
        gargs = (q["codes"], q["scales"], q["g"], perm, R, S, W1.packed_codes, W1.packed_scales,
                 W1.g, offs)
        if fuse:
            return F.grouped_w4a4_gemm_rac_swiglu(*gargs, M_total=rows, with_amax=True)
        return F.grouped_w4a4_gemm_rac(*gargs, M_total=rows), None

    def gemm2(q2, R2, S2, offs, rows):
        return F.grouped_w4a4_gemm_rac(q2["codes"], q2["scales"], q2["g"], None, R2, S2,
                                       W2.packed_codes, W2.packed_scales, W2.g, offs, M_total=rows)

    dense_offs = torch.tensor([0, cfg.T], dtype=torch.int32, device=dev)

    def step(keep=False):
        if cfg.kind == "dense":
            offs = dense_offs
            perm, inv, tw = None, None, None
            rows = cfg.T
        else:
            ids, tw, offs, perm, inv = timed("permute", F.moe_permute, logits, cfg.topk, bias)
            rows = perm.numel()
        q = timed("quant1", F.nvfp4_quantize_act, x, False, cfg.k_first > 0)
        S = R = None
        if cfg.k_first:
            S, R = timed("select1", F.select_residual_channels, q["x_used"], q["codes"],
                         q["scales"], q["g"], q["score"], cfg.k_first)
        y1, h_amax = timed("gemm1", gemm1, q, perm, R, S, offs, rows)
        st = dict(q=q, S=S, R=R, perm=perm, offs=offs, rows=rows) if keep else None
        if W2 is None:
            return y1, st
        if fuse:
            q2 = timed("quant2", F.nvfp4_quantize_act_amax, y1, h_amax, cfg.k_down > 0)
        else:
            q2 = timed("quant2", F.nvfp4_quantize_act, y1, True, cfg.k_down > 0)
        S2 = R2 = None
        if cfg.k_down:
            S2, R2 = timed("select2", F.select_residual_channels, q2["x_used"], q2["codes"],
                           q2["scales"], q2["g"], q2["score"], cfg.k_down)
        y2 = timed("gemm2", gemm2, q2, R2, S2, offs, rows)
        if keep:
            st.update(q2=q2, S2=S2, R2=R2)
        return timed("combine", F.moe_unpermute_combine, y2, inv, tw), st

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-step HIP events (their spread), then per-call events (the stage
    # breakdown); both kept out of the wall-clock region
    st_timer = Timer()
    for _ in range(steps):
        a = st_timer.start()
        step()
        st_timer.stop(a)
    torch.cuda.synchronize()
    record[0] = True
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    record[0] = False
    stage_ms = {n: t.mean_ms() for n, t in timers.items() if t.pairs}

    # the same forward step captured once as a HIP graph and replayed: the
    # library allocates nothing, never synchronizes and sizes every grid from
    # shapes alone, so a serving loop can replay the whole step without a
    # host launch per kernel
    graph_ms = graph_pct = None
    if use_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(2):
                step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) / steps * 1e3
        gt = Timer()
        for _ in range(steps):
            a = gt.start()
            g.replay()
            gt.stop(a)
        torch.cuda.synchronize()
        graph_pct = percentiles(gt.times())
        del g

    # residual-compensation overhead of each GEMM call as the step makes it:
    # t(k) / t(k = 0) - 1, the two timed in turn
    _, st = step(keep=True)
    reps = max(steps, 10)
    rac = {}
    if cfg.k_first:
        tk, t0k = interleaved_ms(
            [lambda: gemm1(st["q"], st["perm"], st["R"], st["S"], st["offs"], st["rows"]),
             lambda: gemm1(st["q"], st["perm"], None, None, st["offs"], st["rows"])], reps)
        rac["gemm1"] = {"ms_k": round(tk, 4), "ms_k0": round(t0k, 4),
                        "overhead": round(tk / t0k - 1.0, 4)}
    if W2 is not None and cfg.k_down:
        tk, t0k = interleaved_ms(
            [lambda: gemm2(st["q2"], st["R2"], st["S2"], st["offs"], st["rows"]),
             lambda: gemm2(st["q2"], None, None, st["offs"], st["rows"])], reps)
        rac["gemm2"] = {"ms_k": round(tk, 4), "ms_k0": round(t0k, 4),
                        "overhead": round(tk / t0k - 1.0, 4)}
    if cfg.kind == "dense":
        counts = [cfg.T]
    else:
        o = st["offs"].cpu().numpy()
        counts = list(o[1:] - o[:-1])
    eager_ms = wall / steps * 1e3
    return dict(ms=graph_ms if graph_ms is not None else eager_ms,
                step_ms=graph_pct if graph_pct is not None else percentiles(st_timer.times()),
                eager_ms=eager_ms, eager_step_ms=percentiles(st_timer.times()),
                graph=graph_ms is not None, stage_ms=stage_ms, qdq_ms=qdq_ms, rac=rac,
                counts=counts, fuse=fuse)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, wl, tokens, experts):
    """The oracle, as it stands, on a bounded sample of the same block: the
    first `tokens` tokens routed over the first `experts` experts (top-k
    capped at experts / 2), every stage of the block."""
    from threadpoolctl import threadpool_info

    from oracle import formats as OF
    from oracle import layer

    tk = min(cfg.topk, max(1, experts // 2)) if cfg.kind != "dense" else 1
    T = min(tokens, cfg.T)
    x = OF.bf16_bits_to_f64(wl.x[:T])
    t0 = time.perf_counter()
    if cfg.kind == "dense":
        w = OF.bf16_bits_to_f64(wl.w_first[0])
        layer.dense_forward(x, w, cfg.k_first)
        flops = 2 * T * w.shape[0] * (cfg.H + cfg.k_first)
        desc = f"dense {T}x{w.shape[0]}x{cfg.H}"
    else:
        E = min(experts, cfg.E)
        w1 = OF.bf16_bits_to_f64(wl.w_first[:E])
        w2 = OF.bf16_bits_to_f64(wl.w_down[:E]) if wl.w_down is not None else None
        logits = wl.logits[:T, :E]
        bias = wl.bias[:E] if wl.bias is not None else None
        layer.moe_forward(x, logits, bias, tk, w1, w2, cfg.k_first, cfg.k_down)
        rows = T * tk
        flops = 2 * rows * w1.shape[1] * (cfg.H + cfg.k_first)
        if w2 is not None:
            flops += 2 * rows * cfg.H * (cfg.inter + cfg.k_down)
        desc = (f"{T} tokens x top-{tk} of the first {E} experts of {cfg.name} (hidden "
                f"{cfg.H}, intermediate {cfg.inter}), every stage incl. weight QDQ of those "
                f"experts")
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": desc, "seconds": round(dt, 2), "cpu_model": cpu_model(),
            "cores_available": cores, "blas_threads": threads}


def nvfp4_operands(x_bits, w_bits):
    """MFMA operand values as the large-tile GEMM multiplies them: 64 rows of
    activations and 64 weight rows (bf16 bits, host arrays [64][K]) quantized
    to NVFP4 by the library and decoded to q * s, as [64 lanes][8 A + 8 B
    registers][8] f16 and bf16 bit patterns (device tensors).  Measurement
    only: the decode here is two table lookups."""
    import numpy as np
    import torch

    import fp4_quantized_gemm_amd as F

    dev = torch.device("cuda:0")
    to = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
    q = F.nvfp4_quantize_act(to(x_bits))
    W = F.nvfp4_qdq_weights(to(w_bits)[None], want_qdq=False, want_packed=False)
    grid = torch.tensor([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.0, -0.5, -1, -1.5, -2, -3, -4, -6],
                        dtype=torch.float32, device=dev)

    def values(codes, scales):
        c = codes.reshape(codes.shape[0], -1).to(torch.int64)
        nib = torch.stack([c & 15, c >> 4], dim=-1).reshape(c.shape[0], -1)
        s = scales.reshape(scales.shape[0], -1).view(torch.float8_e4m3fn).to(torch.float32)
        return (grid[nib] * s.repeat_interleave(16, dim=1)).reshape(-1)[:4096]

    a, b = values(q["codes"], q["scales"]), values(W.codes[0], W.scales[0])
    ops = torch.cat([a.reshape(64, 8, 8), b.reshape(64, 8, 8)], dim=1)   # [lane][16][8]
    return ops.to(torch.float16).contiguous(), ops.to(torch.bfloat16).contiguous()


def ceilings(reps=5, operands=None):
    """Sustained rates measured on this chip: each matrix-core instruction
    family the exact NVFP4 product (f16/bf16) and its FP8 baseline can use,
    and HBM streaming read and copy.  With `operands` (nvfp4_operands), also
    the f16 and bf16 rates on exactly decoded NVFP4 values of the workload,
    run long enough for the clock to settle: the matrix cores' rate depends
    on the operand bits."""
    import ctypes

    import torch

    import fp4_quantized_gemm_amd as F

    L = F.lib()
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(4 * cus * 256, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    res = {"cus": cus}
    for kind, name in ((0, "mfma_f16"), (1, "mfma_bf16"), (2, "mfma_fp8"), (3, "mfma_fp4")):
        iters = 4000 if kind < 2 else 2000
        fn = lambda: L.nvfp4_ceiling_mfma(kind, iters, 2 * cus, ctypes.c_void_p(out.data_ptr()),
                                          stream)
        assert fn() == 0
        ms = median_ms(fn, reps)
        flops = 2 * cus * 4 * iters * 4 * L.nvfp4_ceiling_mfma_flops(kind)
        res[name + "_tflops"] = round(flops / ms / 1e9, 1)
    if operands is not None:
        iters = 40000                                  # ~25 ms per call
        for bf, name, ops in ((0, "mfma_f16", operands[0]), (1, "mfma_bf16", operands[1])):
            fn = lambda: L.nvfp4_ceiling_mfma_operands(bf, ctypes.c_void_p(ops.data_ptr()), iters,
                                                       4 * cus, ctypes.c_void_p(out.data_ptr()),
                                                       stream)
            assert fn() == 0
            ms = median_ms(fn, 3)
            flops = 4 * cus * 4 * iters * 8 * 2 * 32 * 32 * 16
            res[name + "_nvfp4_operands_tflops"] = round(flops / ms / 1e9, 1)
    nbytes = 2 << 30                                   # 2 GiB, past the 256 MB cache
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    o32 = torch.empty(1, dtype=torch.int32, device=dev)
    rd = lambda: L.nvfp4_ceiling_read(ctypes.c_void_p(buf.data_ptr()), nbytes,
                                      ctypes.c_void_p(o32.data_ptr()), stream)
    assert rd() == 0
    res["hbm_read_GBps"] = round(nbytes / median_ms(rd, reps) / 1e6, 1)
    half = buf[: nbytes // 2]
    dst = torch.empty_like(half)
    res["hbm_copy_GBps"] = round(2 * half.numel() / median_ms(lambda: dst.copy_(half), reps) / 1e6,
                                 1)
    del buf, dst
    torch.cuda.empty_cache()
    return res


def gemm_kernel_name(cfg, m, n, k, E):
    """The kernel grouped_w4a4_gemm_rac picks for this shape on a 256-CU
    MI355X (the library's own dispatch rule, restated for the report)."""
    if m <= 48 * E and k <= 128:
        return "k_gemm_decode"
    if (k <= 128 or k % 128 == 0) and cfg.H <= 16384 and cfg.inter <= 16384:
        return "k_gemm_big" if k <= 128 else "k_gemm_big, 128-channel W_S tiles after the loop"
    return "k_gemm_generic"


def rac_sweep(cfg, wl, reps, n_experts=8):
    """Compensation strength against cost on the block's first GEMM.  For k
    from 0 to half the hidden size (the pages' "top 50%" of channels): the
    GEMM's duration (HIP events, median of `reps` calls), the duration of the
    second-pass residual QDQ, and the relative Frobenius error of the GEMM
    output against the trainer's W4A16 forward on the same rows (bf16
    activations times the trainer's bf16 fake-quantized weights, float32
    accumulation), over all rows of `n_experts` experts, for the bf16
    residual and for the NVFP4-quantized one; for MoE blocks also the shared
    and per-expert selection calls, the per-expert GEMM and its error."""
    import numpy as np
    import torch

    import fp4_quantized_gemm_amd as F

    dev = torch.device("cuda:0")
    x = to_dev(wl.x, dev)
    w1 = to_dev(wl.w_first, dev)
    Wq = F.nvfp4_qdq_weights(w1, want_qdq=True)
    c1, s1, g1, wq = Wq.packed_codes, Wq.packed_scales, Wq.g, Wq.qdq
    del w1
    if cfg.kind == "dense":
        offs = torch.tensor([0, cfg.T], dtype=torch.int32, device=dev)
        perm, rows = None, cfg.T
    else:
        logits = torch.from_numpy(wl.logits).to(dev)
        bias = torch.from_numpy(wl.bias).to(dev) if wl.bias is not None else None
        _, _, offs, perm, _ = F.moe_permute(logits, cfg.topk, bias)
        rows = perm.numel()
    q = F.nvfp4_quantize_act(x, False, True)
    o = offs.cpu().numpy()
    busy = [e for e in range(len(o) - 1) if o[e + 1] > o[e]][:n_experts]
    xf = x.float()
    refs = []
    for e in busy:
        idx = torch.arange(int(o[e]), int(o[e + 1]), device=dev)
        src = perm[idx].long() if perm is not None else idx
        refs.append((idx, xf[src] @ wq[e].float().t().contiguous()))
    torch.cuda.synchronize()

    def err(y):
        num = den = 0.0
        for idx, ref in refs:
            d = y[idx].float() - ref
            num += float((d * d).sum())
            den += float((ref * ref).sum())
        return (num / den) ** 0.5

    def median_ms(fn):
        ts = []
        for _ in range(reps + 2):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ts.append((a, b))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ts[2:]]))

    def gemm(R, S):
        return F.grouped_w4a4_gemm_rac(q["codes"], q["scales"], q["g"], perm, R, S, c1, s1, g1,
                                       offs, M_total=rows)

    E, N, K = c1.shape[0], c1.shape[2] * 16, c1.shape[3] * 64      # packed codes
    ks = [k for k in (0, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096) if k <= K // 2]
    points = []
    t0 = None
    for k in ks:
        pt = {"k": k, "kernel": gemm_kernel_name(cfg, rows, N, k, E)}
        if k == 0:
            pt["gemm_ms"] = t0 = median_ms(lambda: gemm(None, None))
            pt["err"] = err(gemm(None, None))
        else:
            S, R = F.select_residual_channels(q["x_used"], q["codes"], q["scales"], q["g"],
                                              q["score"], k)
            rq = F.nvfp4_qdq_residual(R)
            pt["gemm_ms"] = median_ms(lambda: gemm(R, S))
            pt["qdq_residual_ms"] = median_ms(lambda: F.nvfp4_qdq_residual(R))
            pt["err_bf16_residual"] = err(gemm(R, S))
            pt["err_nvfp4_residual"] = err(gemm(rq[3], S))
            if cfg.kind != "dense":
                # one channel set per expert, from the rows routed to it
                sel_pe = lambda: F.select_residual_channels_per_expert(
                    q["x_used"], q["codes"], q["scales"], q["g"], None, k, perm, offs,
                    M_total=rows)
                S_e, R_p = sel_pe()
                gemm_pe = lambda: F.grouped_w4a4_gemm_rac_per_expert(
                    q["codes"], q["scales"], q["g"], perm, R_p, S_e, c1, s1, g1, offs,
                    M_total=rows)
                pt["select_ms"] = median_ms(lambda: F.select_residual_channels(
                    q["x_used"], q["codes"], q["scales"], q["g"], q["score"], k))
                pt["per_expert_select_ms"] = median_ms(sel_pe)
                pt["per_expert_gemm_ms"] = median_ms(gemm_pe)
                pt["err_per_expert"] = err(gemm_pe())
        pt["overhead"] = pt["gemm_ms"] / t0 - 1.0
        points.append({kk: (round(v, 6) if isinstance(v, float) else v) for kk, v in pt.items()})
        print(f"# k={k} {points[-1]}", file=sys.stderr, flush=True)
    return {"mode": "rac_sweep", "workload": cfg.name,
            "gemm": f"first {rows}x{N}x{K}", "reference": "trainer W4A16 forward "
            "(bf16 x times bf16 fake-quantized weight, fp32 accumulate)",
            "error": "relative Frobenius norm over all rows of the first "
            f"{len(busy)} experts with rows", "reps": reps, "points": points}


def w4a16_bench(cfg, wl, reps):
    """The trainer-side W4A16 product (grouped_w4a16_gemm) on the block's
    GEMM shapes, beside the W4A4 GEMM without correction on the same shapes:
    HIP-event medians of `reps` calls, flops 2 * rows * N * K against the
    dense bf16 MFMA peak.  The down GEMM's bf16 input is a synthetic N(0,1)
    tensor of the SwiGLU output's shape."""
    import numpy as np
    import torch

    import fp4_quantized_gemm_amd as F

    dev = torch.device("cuda:0")
    x = to_dev(wl.x, dev)
    if cfg.kind == "dense":
        offs = torch.tensor([0, cfg.T], dtype=torch.int32, device=dev)
        perm, rows = None, cfg.T
    else:
        logits = torch.from_numpy(wl.logits).to(dev)
        bias = torch.from_numpy(wl.bias).to(dev) if wl.bias is not None else None
        _, _, offs, perm, _ = F.moe_permute(logits, cfg.topk, bias)
        rows = perm.numel()
    gemms = [("first", x, perm, to_dev(wl.w_first, dev))]
    if wl.w_down is not None:
        g = torch.Generator(device=dev).manual_seed(0)
        h = torch.randn((rows, cfg.inter), generator=g, device=dev).to(torch.bfloat16)
        gemms.append(("down", h, None, to_dev(wl.w_down, dev)))

    def median_ms(fn):
        ts = []
        for _ in range(reps + 2):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ts.append((a, b))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ts[2:]]))

    out = []
    for name, a, a_rows, w in gemms:
        Wq = F.nvfp4_qdq_weights(w, want_qdq=False)
        c, s, gw = Wq.packed_codes, Wq.packed_scales, Wq.g
        del Wq
        del w
        q = F.nvfp4_quantize_act(a, False, False)
        E, N, K = c.shape[0], c.shape[2] * 16, c.shape[3] * 64
        t16 = median_ms(lambda: F.grouped_w4a16_gemm(a, a_rows, c, s, gw, offs, M_total=rows))
        t4 = median_ms(lambda: F.grouped_w4a4_gemm_rac(q["codes"], q["scales"], q["g"], a_rows,
                                                       None, None, c, s, gw, offs, M_total=rows))
        fl = 2.0 * rows * N * K
        out.append({"gemm": f"{name} {rows}x{N}x{K}", "w4a16_ms": round(t16, 4),
                    "w4a16_tflops": round(fl / t16 / 1e9, 1),
                    "w4a16_frac_bf16_peak": round(fl / t16 / 1e9 / PEAK_BF16_TFLOPS, 4),
                    "w4a4_k0_ms": round(t4, 4)})
        print(f"# {out[-1]}", file=sys.stderr, flush=True)
    return {"mode": "w4a16", "workload": cfg.name, "reps": reps, "gemms": out}


def fp8_bench(cfg, wl, reps):
    """The FP8 (E4M3) W8A8 baseline (fp8_quantize + grouped_fp8_gemm) on the
    block's GEMM shapes, beside the NVFP4 path on the same shapes (activation
    quantizer, W4A4 GEMM with the block's k compensated channels, and at
    k = 0): HIP-event medians of `reps` calls.  Flops 2 * rows * N * K against
    the dense fp8 MFMA peak; bytes (E4M3 weights of experts with rows, the
    activation codes of every routed row, bf16 output) against HBM.  The
    down GEMM's input is a synthetic N(0,1) tensor of the SwiGLU output's
    shape."""
    import numpy as np
    import torch

    import fp4_quantized_gemm_amd as F

    dev = torch.device("cuda:0")
    x = to_dev(wl.x, dev)
    if cfg.kind == "dense":
        offs = torch.tensor([0, cfg.T], dtype=torch.int32, device=dev)
        perm, rows = None, cfg.T
    else:
        logits = torch.from_numpy(wl.logits).to(dev)
        bias = torch.from_numpy(wl.bias).to(dev) if wl.bias is not None else None
        _, _, offs, perm, _ = F.moe_permute(logits, cfg.topk, bias)
        rows = perm.numel()
    busy = int((offs[1:] > offs[:-1]).sum().item())
    gemms = [("first", x, perm, to_dev(wl.w_first, dev), cfg.gemm_shapes()[0][4])]
    if wl.w_down is not None:
        g = torch.Generator(device=dev).manual_seed(0)
        h = torch.randn((rows, cfg.inter), generator=g, device=dev).to(torch.bfloat16)
        gemms.append(("down", h, None, to_dev(wl.w_down, dev), cfg.gemm_shapes()[1][4]))

    def median_ms(fn):
        ts = []
        for _ in range(reps + 2):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            ts.append((a, b))
        torch.cuda.synchronize()
        return float(np.median([a.elapsed_time(b) for a, b in ts[2:]]))

    out = []
    for name, a, a_rows, w, k in gemms:
        E, N, K = w.shape
        wc8, gw8 = F.fp8_quantize(w, stacked=True)
        Wq = F.nvfp4_qdq_weights(w, want_qdq=False)
        c, s, gw = Wq.packed_codes, Wq.packed_scales, Wq.g
        del Wq
        del w
        ac8, gx8 = F.fp8_quantize(a)
        q = F.nvfp4_quantize_act(a, False, k > 0)
        S, R = (F.select_residual_channels(q["x_used"], q["codes"], q["scales"], q["g"],
                                           q["score"], k) if k > 0 else (None, None))
        t8 = median_ms(lambda: F.grouped_fp8_gemm(ac8, gx8, a_rows, wc8, gw8, offs, M_total=rows))
        tq8 = median_ms(lambda: F.fp8_quantize(a))
        t4 = median_ms(lambda: F.grouped_w4a4_gemm_rac(q["codes"], q["scales"], q["g"], a_rows,
                                                       R, S, c, s, gw, offs, M_total=rows))
        t40 = median_ms(lambda: F.grouped_w4a4_gemm_rac(q["codes"], q["scales"], q["g"], a_rows,
                                                        None, None, c, s, gw, offs, M_total=rows))
        tq4 = median_ms(lambda: F.nvfp4_quantize_act(a, False, k > 0))
        fl = 2.0 * rows * N * K
        by8 = busy * N * K + rows * K + rows * N * 2
        out.append({"gemm": f"{name} {rows}x{N}x{K}", "fp8_ms": round(t8, 4),
                    "fp8_tflops": round(fl / t8 / 1e9, 1),
                    "fp8_frac_fp8_peak": round(fl / t8 / 1e9 / PEAK_FP8_TFLOPS, 4),
                    "fp8_gbps": round(by8 / t8 / 1e6, 1),
                    "fp8_quantize_act_ms": round(tq8, 4),
                    "nvfp4_k": k, "nvfp4_rac_ms": round(t4, 4), "nvfp4_k0_ms": round(t40, 4),
                    "nvfp4_quantize_act_ms": round(tq4, 4)})
        print(f"# {out[-1]}", file=sys.stderr, flush=True)
    return {"mode": "fp8", "workload": cfg.name, "reps": reps, "gemms": out}


def gemm_algorithmic_bytes(cfg, counts):
    """Bytes one step's GEMM calls must move: NVFP4 weights (codes + E4M3
    scales, 0.5625 B/elem) of experts that have rows, the activation codes of
    every routed row, the residual rows, and the bf16 output."""
    busy = sum(1 for c in counts if c > 0)
    total = 0.0
    for _, m, n, k, kk in cfg.gemm_shapes():
        total += busy * n * k * 0.5625 + m * k * 0.5625 + m * kk * 2 + m * n * 2
    return total


def roofline_of(cfg, res, decode):
    """The grouped GEMM calls of a step against their bound: MFMA (f16/bf16
    dense peak) for prefill, HBM for decode-sized blocks."""
    shapes = cfg.gemm_shapes()
    flops_step = cfg.gemm_flops()
    gemm_ms = res["stage_ms"].get("gemm1", 0.0) + res["stage_ms"].get("gemm2", 0.0)
    alg_bytes = gemm_algorithmic_bytes(cfg, res["counts"])
    if decode:
        achieved = alg_bytes / (gemm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4)}
        kernel = "grouped_w4a4_gemm_rac: k_gemm_decode"
    else:
        achieved = flops_step / (gemm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "frac_of_fp4_peak": round(achieved / PEAK_FP4_TFLOPS, 4)}
        _, m, n, _, kk = shapes[0]
        big = gemm_kernel_name(cfg, m, n, kk, cfg.E).endswith("k_gemm_big")
        name = ("grouped_w4a4_gemm_rac_swiglu + grouped_w4a4_gemm_rac" if res["fuse"]
                else "grouped_w4a4_gemm_rac")
        kernel = (f"{name}: k_decode_a + k_tile_prefix + k_gemm_big" if big
                  else f"{name}: k_tile_prefix + k_gemm_generic")
    roof["traffic"] = recorded_traffic(cfg.name)
    roof["kernel"] = kernel
    roof["algorithmic_bytes"] = round(alg_bytes)
    roof["algorithmic_flops"] = round(flops_step)
    roof["gemm_ms_per_step"] = round(gemm_ms, 4)
    return roof


def quantizer_rates(cfg, res):
    q_bytes = 2.5625 * cfg.T * cfg.H
    out = {"quant1_GBps": round(q_bytes / (res["stage_ms"]["quant1"] * 1e-3) / 1e9, 1)}
    if "quant2" in res["stage_ms"]:
        # h's quantizer: reads h once (amax from the fused GEMM), or reads
        # [gate | up] and forms h
        q2_bytes = (2.5625 if res["fuse"] else 4.5625) * cfg.rows * cfg.inter
        out["quant2_GBps"] = round(q2_bytes / (res["stage_ms"]["quant2"] * 1e-3) / 1e9, 1)
    out["frac_of_hbm"] = {k: round(v / PEAK_HBM_GBPS, 4) for k, v in list(out.items())}
    return out


def block_summary(cfg, res, decode):
    return {
        "workload": cfg.name,
        "ms_per_step": round(res["ms"], 4),
        "step_ms_events": res["step_ms"],
        "step_launch": "one HIP graph replay per step" if res["graph"] else "eager launches",
        "ms_per_step_eager": round(res["eager_ms"], 4),
        "step_ms_events_eager": res["eager_step_ms"],
        "value": round(cfg.gemm_flops() / (res["ms"] * 1e-3) / 1e12, 2),
        "weight_qdq_ms_per_sync": round(res["qdq_ms"], 4),
        "roofline": roofline_of(cfg, res, decode),
        "stages_ms": {k: round(v, 4) for k, v in res["stage_ms"].items()},
        "quantizer": quantizer_rates(cfg, res),
        "rac_overhead": res["rac"],
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the library runs each "
              f"call on one device and has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.ceilings:
        print(json.dumps({"mode": "ceilings", **ceilings()}), flush=True)
        return
    import synth

    cfg = synth.get(args.config)
    wl = synth.make(cfg)
    if args.rac_sweep:
        print(json.dumps(rac_sweep(cfg, wl, max(args.steps // 2, 5))), flush=True)
        return
    if args.w4a16:
        print(json.dumps(w4a16_bench(cfg, wl, max(args.steps // 2, 5))), flush=True)
        return
    if args.fp8:
        print(json.dumps(fp8_bench(cfg, wl, max(args.steps // 2, 5))), flush=True)
        return
    # the SwiGLU is fused where the large-tile kernel forms it in its epilogue;
    # on decode-sized blocks the decode kernel's output goes to the quantizer
    decode = cfg.rows <= 48 * cfg.E and cfg.kind != "dense"
    fuse = not args.no_fuse_swiglu and wl.w_down is not None and not decode
    res = run_block(cfg, wl, args.steps, args.warmup, fuse, not args.eager)
    main_block = block_summary(cfg, res, decode)
    shapes = cfg.gemm_shapes()
    line = {
        "metric": "grouped W4A4+RAC GEMM TFLOP/s and % of MI355X FP4 MFMA peak; quantizer GB/s",
        "value": main_block["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_block["ms_per_step"],
        "step_ms_events": main_block["step_ms_events"],
        "step_launch": main_block["step_launch"],
        "ms_per_step_eager": main_block["ms_per_step_eager"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "storage": "nvfp4 (E2M1 + E4M3/16 + f32) decoded exactly to f16 MFMA operands, bf16 "
                   "residual term, f32 accumulate",
        "data": "synthetic",
        "step": "one forward of the MoE block (route, quantize, select, gate+up GEMM+RAC, "
                "SwiGLU, quantize, select, down GEMM+RAC, combine); the weight QDQ runs once "
                "per weight sync and is reported as weight_qdq_ms_per_sync",
        "weight_qdq_ms_per_sync": main_block["weight_qdq_ms_per_sync"],
        "ms_per_step_incl_weight_qdq": round(res["ms"] + res["qdq_ms"], 4),
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.H, "experts": cfg.E,
                   "topk": cfg.topk, "inter": cfg.inter, "rac_k": [s[4] for s in shapes],
                   "gemms": [f"{n} {m}x{nn}x{k}" for n, m, nn, k, _ in shapes],
                   "swiglu": ("fused into the gate+up GEMM" if fuse else
                              "fused into the second quantizer") if wl.w_down is not None
                   else None},
        "roofline": main_block["roofline"],
        "stages_ms": main_block["stages_ms"],
        "quantizer": main_block["quantizer"],
        "rac_overhead": main_block["rac_overhead"],
    }
    ops = None
    if not args.no_ceilings and wl.w_first is not None:
        ops = nvfp4_operands(wl.x[:64], wl.w_first[0, :64])
    del res, wl
    if not args.no_decode and args.config != 4:
        dcfg = synth.get(4)
        dwl = synth.make(dcfg)
        dres = run_block(dcfg, dwl, args.steps, args.warmup, False, not args.eager)
        line["decode"] = block_summary(dcfg, dres, True)
        del dres
    if not args.no_ceilings:
        line["ceilings"] = ceilings(operands=ops)
        c16 = line["ceilings"].get("mfma_f16_nvfp4_operands_tflops")
        if c16 and line["roofline"]["bound"] == "mfma":
            # the same achieved rate against the f16 matrix-core rate on
            # this workload's own NVFP4 operand values
            line["roofline"]["frac_of_f16_rate_on_these_operands"] = round(
                line["roofline"]["achieved"] / c16, 4)
    gates = {}
    r = line["roofline"]
    if r["bound"] == "mfma":
        gates["prefill_gemm_frac_bf16_peak"] = {"value": r["frac"], "target": 0.5,
                                                "met": r["frac"] >= 0.5}
        gates["prefill_gemm_frac_fp4_peak"] = {"value": r["frac_of_fp4_peak"], "target": 0.5,
                                               "met": r["frac_of_fp4_peak"] >= 0.5,
                                               "ceiling_of_exact_mapping": 0.25}
    dec = line.get("decode", {}).get("roofline") or (r if r["bound"] == "hbm" else None)
    if dec is not None:
        gates["decode_gemm_frac_hbm"] = {"value": dec["frac"], "target": 0.6,
                                         "met": dec["frac"] >= 0.6}
    for blk, tag in ((line, "main"), (line.get("decode"), "decode")):
        if blk:
            for g, v in blk["rac_overhead"].items():
                gates[f"rac_overhead_{tag}_{g}"] = {"value": v["overhead"], "target": 0.10,
                                                    "met": v["overhead"] <= 0.10}
    line["gates"] = gates
    if not args.no_cpu_baseline:
        wl = synth.make(cfg)
        line["cpu_baseline"] = cpu_baseline(cfg, wl, args.cpu_tokens, args.cpu_experts)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
