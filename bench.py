"""Throughput of the quantized attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload large] [--pv 16|fp8|auto]

One step = one sage_attn_fwd call: the quantize pass (K mean, channel balance,
INT8 Q/K codes and scales, V layout) plus the fused attention kernel, over the
workload's whole batch, with the inputs already resident in HBM.  On a frame
cache (--workload window) a step is one streaming step instead: the current
frame's K and V and the queries quantized into the cache once
(sage_attn_quantize_frames, against the frozen mean and exponents of the
cache's first quantization) plus the fused kernel over the sink and window
frames; the whole-cache quantization is timed beside it.  With a block mask
(--workload sparse) the fused kernel skips the dropped tiles and TOPS counts
the kept visible pairs only.  --workload linear times the per-block W8A8
linear layer instead (activation quantization + INT8 GEMM; weights quantized
once beforehand), in TOPS = 2 M N K / time.  Prints ONE
JSON line: TOPS = 4*d*(visible query-key pairs) / time, the roofline of the
dominant kernel (the fused attention, timed with HIP events on its own stream;
its HBM traffic from the committed rocprofv3 counters when they were taken on
the same kernel source, else null), the CPU oracle timed on a bounded sample
of the same workload, and the other P.V mode timed the same way with its own
accuracy on a small sample.  With --graph (default for the frame-cache
streaming workloads) the step is also captured once into a HIP graph
(torch.cuda.CUDAGraph) and replayed, which removes the per-launch overhead of
its short kernels; that timing is reported beside the eager one.
"""

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized-attention TOPS (4·B·H·Nq·Nkv·d) + % of peak MFMA, 75.6k-token 720p shape"
INT8_PEAK_TOPS = 5000.0   # MI355X dense INT8 MFMA, 5.0 POP/s
BF16_PEAK_TOPS = 2500.0   # dense bf16/fp16 MFMA, 2.5 PFLOP/s
FP8_PEAK_TOPS = 5000.0    # dense FP8 MFMA, 5.0 PFLOP/s
HBM_PEAK_GBS = 8000.0


PV_NAMES = {0: "16", 1: "fp8", 2: "auto"}


def mode_peak(pv_mode, f8=None):
    """The MFMA ceiling of one P.V mode: half of the 4 d ops per visible pair
    (Q K^T) run on INT8 matrix cores, the other half (P V) on 16-bit or FP8
    ones, so the time per op at peak is 0.5 / INT8 + 0.5 / (P.V peak).  The
    per-head mode (2) runs a share f8 of the heads' ops in FP8 and the rest
    in 16 bits: the time per op is the share-weighted sum."""
    t16 = 0.5 / INT8_PEAK_TOPS + 0.5 / BF16_PEAK_TOPS
    t8 = 0.5 / INT8_PEAK_TOPS + 0.5 / FP8_PEAK_TOPS
    if pv_mode == 2:
        return 1.0 / (f8 * t8 + (1.0 - f8) * t16)
    return 1.0 / (t8 if pv_mode == 1 else t16)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="large")
    p.add_argument("--pv", default=None, choices=["16", "fp8", "auto"],
                   help="P.V mode (default: the workload's own); auto = FP8 per head unless "
                        "channel balance moved one of its channels")
    p.add_argument("--cpu-heads", type=int, default=None,
                   help="heads in the CPU oracle sample (default 8; 2 with a block mask)")
    p.add_argument("--cpu-rows", type=int, default=None,
                   help="query rows per head in the CPU sample (default 512; 128 with a block mask)")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--profile", action="store_true", help="few steps, no CPU leg (for rocprofv3)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="also run one plain 256 MiB device copy (reference for HBM byte counters)")
    p.add_argument("--single-mode", action="store_true", help="do not time the other P.V mode")
    p.add_argument("--kv-splits", type=int, default=0,
                   help="KV splits per query tile (0: the library's choice)")
    p.add_argument("--graph", dest="graph", action="store_true", default=None,
                   help="also time the step captured in a HIP graph and replayed "
                        "(default: on for the frame-cache workloads)")
    p.add_argument("--no-graph", dest="graph", action="store_false")
    return p.parse_args()


def kernel_traffic(workload, pv):
    """HBM bytes per launch of the workload's dominant kernel from
    profiles/traffic.json (FETCH_SIZE and WRITE_SIZE scaled by the plain-copy
    factors), only if those counters were taken on the current source of that
    kernel (sha256 of the files the record lists); else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))["launches"].get(f"{workload}/{pv}")
    if rec is None:
        return None
    h = hashlib.sha256()
    for f in rec["source_files"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return rec["bytes"] if h.hexdigest() == rec["source_sha256"] else None


def torch_stack(parts):
    import torch
    return torch.stack(parts).contiguous()


def step_parts(sage, w, desc, q, k, v, o, bufs, stream):
    """The two halves of one step as callables: (quantize, attend)."""
    if not w.frame_stride:
        return (lambda: sage.sage_attn_quantize(desc, q, k, v, bufs, stream),
                lambda: sage.sage_attn_fwd_quantized(desc, bufs, o, stream))
    # streaming step: each batch's current frame (its new keys and values, as
    # the model would hand them over) and the queries into the cache
    F = w.frame_len
    fq = [p // F for p in w.q_pos0s()]
    same = all(f == fq[0] for f in fq)
    if same:
        kk, vv = k[:, :, fq[0] * F:(fq[0] + 1) * F], v[:, :, fq[0] * F:(fq[0] + 1) * F]
    else:
        kk = torch_stack([k[b, :, f * F:(f + 1) * F] for b, f in enumerate(fq)])
        vv = torch_stack([v[b, :, f * F:(f + 1) * F] for b, f in enumerate(fq)])
    d2 = sage.Desc.for_tensors(q, kk, vv, nkv=w.Nkv, pv_mode=desc.pv_mode, frame_len=F,
                               frame_stride=w.frame_stride)
    if same:
        def quant():
            sage.sage_attn_quantize_frames(d2, q, kk, vv, fq[0], 1, bufs, stream)
    else:
        def quant():
            sage.sage_attn_quantize_frames_batched(d2, q, kk, vv, fq, 1, bufs, stream)
    return quant, lambda: sage.sage_attn_fwd_quantized(desc, bufs, o, stream)


WARM_SECONDS = 0.3  # 0 under --profile: a profiled run keeps its few dispatches


def warm_up(torch, parts, warm, seconds=None):
    """Untimed steps: at least `warm`, and at least `seconds` of them, so that
    a short step (a frame-cache step takes under a millisecond) is timed at
    the clock the GPU holds under load, not while it ramps up."""
    seconds = WARM_SECONDS if seconds is None else seconds
    import time
    quant, attend = parts
    t0 = time.perf_counter()
    n = 0
    while n < warm or time.perf_counter() - t0 < seconds:
        for _ in range(max(1, warm)):
            quant()
            attend()
        n += max(1, warm)
        torch.cuda.synchronize()


def time_path(torch, parts, stream, steps, warm):
    """Warm up, then time `steps` whole steps (quantize + fused kernel) with
    HIP events on the launch stream around them: ms per step.  Then `steps`
    more with events around each part as well: ms per quantize pass and per
    fused-kernel launch.  (Events between launches add idle time to a short
    step -- 0.07 ms of a 0.74 ms frame-cache step -- so the step time comes
    from the first pass.)  Returns ms per step, per quantize pass and per
    fused-kernel launch (means), and the fused kernel's launch times (ms,
    sorted) of the second pass."""
    quant, attend = parts
    warm_up(torch, parts, warm)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        quant()
        attend()
    end.record(stream)
    end.synchronize()
    ms_step = start.elapsed_time(end) / steps

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record(stream)
        quant()
        e[1].record(stream)
        attend()
        e[2].record(stream)
    torch.cuda.synchronize()
    ms_quant = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    launches = sorted(e[1].elapsed_time(e[2]) for e in ev)
    return ms_step, ms_quant, sum(launches) / steps, launches


def input_digests(torch, tensors):
    """SHA-256 per input tensor, of a digest taken on the GPU: the sum of the
    16-bit patterns (as integers) of every row along the last dimension, so
    that a changed element changes it, without copying the tensors to the
    host."""
    out = {}
    for name, t in tensors.items():
        rows = t.contiguous().view(torch.int16).to(torch.int32).sum(dim=-1, dtype=torch.int64)
        out[name] = hashlib.sha256(rows.cpu().numpy().tobytes()).hexdigest()
    return out


def launch_spread(launches):
    """Median and minimum of the timed launches (ms) beside their mean."""
    n = len(launches)
    med = launches[n // 2] if n % 2 else 0.5 * (launches[n // 2 - 1] + launches[n // 2])
    return {"ms_per_launch_median": round(med, 4), "ms_per_launch_min": round(launches[0], 4)}


def time_graph(torch, parts, steps, warm):
    """Capture one step (quantize + fused kernel) into a HIP graph on a side
    stream and time `steps` replays.  `parts` must launch on the current
    stream (the capture stream while capturing).  Returns ms per replayed
    step."""
    quant, attend = parts
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(max(warm, 1)):
            quant()
            attend()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        quant()
        attend()
    warm_up(torch, (g.replay, lambda: None), warm)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        g.replay()
    end.record()
    end.synchronize()
    return start.elapsed_time(end) / steps


def quantize_bytes(w, pv_mode, f8=None):
    """Bytes of the quantize pass: (the minimum, this design's kernels).

    The minimum reads K twice (the K mean needs every key before any key can
    be smoothed) and Q once, and writes the INT8 codes; FP8 mode adds one
    read of V and its e4m3 codes and E8M0 scales.  The design moves more:
    it reads Q twice, because the channel-balance exponent of a channel
    depends on every query's value in it, so no Q block can be coded before
    all of Q has been read once; and in 16-bit mode it writes V transposed
    per 64-key chunk (the P.V operand layout), reading V once for that.  A
    streaming step over a frame cache moves only the current frame's K and
    V and the queries (the mean and exponents are frozen).  The per-head mode
    (2) prepares V of a share f8 of the heads as in FP8 mode, the rest as in
    16-bit mode."""
    esz = 2
    nq = w.B * w.H * w.Nq * w.d
    if w.frame_stride:
        nk = w.B * w.H * w.frame_len * w.d
        kreads = 1
    else:
        nk = w.B * w.H * w.Nkv * w.d
        kreads = 2
    s8 = {0: 0.0, 1: 1.0}.get(pv_mode, f8)      # share of V prepared as FP8
    vscale = nk // 32
    minimum = nq * esz + kreads * nk * esz + nq + nk + s8 * (nk * esz + nk + vscale)
    design = (1 if w.frame_stride else 2) * nq * esz + kreads * nk * esz + nq + nk + \
        nk * esz + s8 * (nk + vscale) + (1 - s8) * nk * esz
    return int(round(minimum)), int(round(design))


def main():
    global WARM_SECONDS
    args = parse()
    if args.profile:
        WARM_SECONDS = 0.0
    if args.gpus != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} is not supported (the path is "
              "data-parallel over (batch, head): G GPUs would each run the same kernel on H/G heads "
              "with no communication)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_quantized_attention_sage_amd as sage
    import workloads

    sage.load()
    if args.workload == "linear":
        return main_linear(args, torch, sage, workloads)
    w = workloads.get(args.workload)
    # the block-sparse emulation runs tile by tile: a smaller sample keeps it to tens of seconds
    if args.cpu_heads is None:
        args.cpu_heads = 2 if w.block_density else 8
    if args.cpu_rows is None:
        args.cpu_rows = 128 if w.block_density else 512
    if args.pv is not None:
        w.pv_mode = {v: k for k, v in PV_NAMES.items()}[args.pv]
    if w.pv_mode == 2 and w.frame_stride:
        print(f"bench.py: --pv auto needs contiguous keys; the {w.name} workload attends over a frame "
              "cache (use --pv 16 or --pv fp8)", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x = workloads.make(w, dev)
    q, k, v = x["q"], x["k"], x["v"]
    o = torch.empty_like(q)
    mask = workloads.block_mask(w)
    mask_dev = torch.from_numpy(mask).to(dev) if mask is not None else None
    stream = torch.cuda.current_stream()
    steps = 2 if args.profile else args.steps
    warm = 1 if args.profile else args.warmup

    def setup(pv_mode):
        desc = sage.Desc.for_tensors(q, k, v, o, pv_mode=pv_mode, frame_len=w.frame_len,
                                     kv_len=w.kv_len, q_pos0=w.q_pos0, block_mask=mask_dev,
                                     kv_splits=args.kv_splits,
                                     **(dict(nkv=w.Nkv, frame_stride=w.frame_stride,
                                             sink_frames=w.sink_frames, window_frames=w.window_frames)
                                        if w.frame_stride else {}))
        ws = sage.new_workspace(desc, dev)
        bufs = sage.sage_attn_quant_layout(desc, ws)
        if w.frame_stride:
            # the cache as the stream has built it: every frame quantized once,
            # the mean and exponents computed here and frozen from now on
            sage.sage_attn_quantize(desc, q, k, v, bufs, stream)
        return desc, ws, bufs

    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    ops = w.ops()
    others = []
    if not (args.profile or args.single_mode):
        # the other P.V modes first, so that the headline mode's output stays in `o`
        for m2 in ((0, 1) if w.pv_mode == 2 else (1 - w.pv_mode,)):
            desc2, ws2, bufs2 = setup(m2)
            t2 = time_path(torch, step_parts(sage, w, desc2, q, k, v, o, bufs2, stream), stream, steps, warm)
            other = {"pv": PV_NAMES[m2],
                     "value": round(ops / (t2[0] * 1e-3) / 1e12, 2),
                     "attn_tops": round(ops / (t2[2] * 1e-3) / 1e12, 2),
                     "attn_frac_int8_peak": round(ops / (t2[2] * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                     "ms_per_step": round(t2[0], 4)}
            if not args.no_cpu:
                other["accuracy"] = accuracy_sample(w, x, o, desc2, m2, sage,
                                                    rows=64 if w.block_density else 256)
                other["meets_bar"] = bool(other["accuracy"]["cosine_vs_fp64"] >= 0.999 and
                                          other["accuracy"]["max_abs_vs_emulation"] <= 2e-3)
            others.append(other)
            del ws2, bufs2
    desc, ws, bufs = setup(w.pv_mode)
    ms_step, ms_quant, ms_attn, launches = time_path(torch, step_parts(sage, w, desc, q, k, v, o, bufs, stream),
                                                     stream, steps, warm)
    tops = ops / (ms_step * 1e-3) / 1e12
    ms_full_quant = None
    if w.frame_stride:
        # what re-quantizing the whole cache would cost per step
        qfull = (lambda: sage.sage_attn_quantize(desc, q, k, v, bufs, stream), lambda: None)
        ms_full_quant = time_path(torch, qfull, stream, steps, warm)[1]

    ms_graph = None
    if args.graph is None:
        args.graph = bool(w.frame_stride)
    if args.graph and not args.profile:
        ms_graph = time_graph(torch, step_parts(sage, w, desc, q, k, v, o, bufs, None), steps, warm)

    splits = sage.sage_attn_kv_splits(desc)
    attn_tops = ops / (ms_attn * 1e-3) / 1e12
    pvname = PV_NAMES[w.pv_mode]
    traffic = kernel_traffic(w.name, pvname)
    f8 = heads8 = None
    if w.pv_mode == 2:
        # which heads ran FP8 P.V (every channel-balance exponent 0), read
        # back from the quantized operands after the timed steps; their share
        # of the visible pairs weights the mode's ceiling
        shift = sage.quant_views(desc, ws, bufs)["chan_shift"].cpu().numpy()
        is8 = ~(shift != 0).any(axis=-1)                                   # [B,H]
        heads8 = int(is8.sum())
        pairs = np.asarray([1.0 if w.block_density else float(w.row_keys(b).sum()) for b in range(w.B)])
        f8 = float((is8 * pairs[:, None]).sum() / (pairs.sum() * w.H))
    qmin, qdesign = quantize_bytes(w, w.pv_mode, f8)
    mpeak = mode_peak(w.pv_mode, f8)
    record = {
        "metric": METRIC,
        "value": round(tops, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {0: "int8+" + w.dtype, 1: "int8+fp8", 2: "int8+fp8|" + w.dtype}[w.pv_mode],
        "data": "synthetic (seeded Gaussian, video-DiT token grid)",
        "input_digests": input_digests(torch, {"q": q, "k": k, "v": v}),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nkv": w.Nkv, "d": w.d,
                   "in_dtype": w.dtype, "pv": pvname,
                   **({"pv_heads": {"fp8": heads8, "16": w.B * w.H - heads8}} if heads8 is not None else {}),
                   "frame_len": w.frame_len, "kv_splits": splits,
                   **({"block_density": w.block_density, "kept_tiles": round(float(mask.mean()), 4)}
                      if mask is not None else {}),
                   **({"frame_stride": w.frame_stride, "sink_frames": w.sink_frames,
                       "window_frames": w.window_frames, "kv_len": w.kv_lens(), "q_pos0": w.q_pos0s()}
                      if w.frame_stride else {}),
                   "ops_per_step": ops, "pct_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 2)},
        "roofline": {"bound": "mfma",
                     "kernel": "attn_fwd_kernel" + (" (one launch per P.V mode)" if w.pv_mode == 2 else ""),
                     "achieved": round(attn_tops, 2),
                     "peak": INT8_PEAK_TOPS, "unit": "TOPS", "frac": round(attn_tops / INT8_PEAK_TOPS, 4),
                     "mode_peak": round(mpeak, 1), "mode_frac": round(attn_tops / mpeak, 4),
                     "mode_peak_note": (("Q K^T on INT8, P V on " + ("FP8" if w.pv_mode == 1 else "16-bit")
                                         + " matrix cores: 1 / (0.5 / 5000 + 0.5 / "
                                         + ("5000" if w.pv_mode == 1 else "2500") + ") TOPS")
                                        if w.pv_mode != 2 else
                                        f"Q K^T on INT8; P V on FP8 for {f8:.3f} of the ops and on 16-bit "
                                        "matrix cores for the rest: 1 / (f8 (0.5/5000 + 0.5/5000) + "
                                        "(1 - f8) (0.5/5000 + 0.5/2500)) TOPS"),
                     "traffic": traffic, "ms_per_launch": round(ms_attn, 4), **launch_spread(launches)},
        "quantize": {"ms": round(ms_quant, 4), "algorithmic_bytes": qmin,
                     "GB_per_s": round(qmin / (ms_quant * 1e-3) / 1e9, 1),
                     "hbm_frac": round(qmin / (ms_quant * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "design_bytes": qdesign,
                     "design_GB_per_s": round(qdesign / (ms_quant * 1e-3) / 1e9, 1)},
    }
    if ms_graph is not None:
        record["graph_replay"] = {"ms_per_step": round(ms_graph, 4),
                                  "value": round(ops / (ms_graph * 1e-3) / 1e12, 2),
                                  "launches_per_step": "quantize kernels + fused kernel (+ split combine)"}
    if ms_full_quant is not None:
        per_batch = len({p // w.frame_len for p in w.q_pos0s()}) > 1
        record["quantize"]["kind"] = ("append each session's frame + queries (sage_attn_quantize_frames_batched)"
                                      if per_batch else "append one frame + queries (sage_attn_quantize_frames)")
        record["quantize"]["whole_cache_ms"] = round(ms_full_quant, 4)
    if others:
        record["other_pv_modes"] = others
    if not args.profile:
        ex = exact_attention(torch, w, q, k, v, steps, warm, ms_step)
        if ex is not None:
            record["exact_attention"] = ex
    if not args.no_cpu and not args.profile:
        record["cpu_baseline"], record["parity"] = cpu_leg(w, x, o, desc, args, sage, torch, ops)
    print(json.dumps(record), flush=True)


def exact_attention(torch, w, q, k, v, steps, warm, ms_step):
    """torch's fused exact attention (scaled_dot_product_attention with the
    flash or memory-efficient backend only -- never the math path) on the
    same 16-bit inputs: the operation this library stands in for, timed like
    a step.  Full attention over every key only (no mask, cache or block
    mask); else None."""
    if w.frame_len or w.frame_stride or w.block_density or w.kv_len is not None:
        return None
    from torch.nn.attention import sdpa_kernel, SDPBackend
    ops = w.ops()
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
            fn = lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v)  # noqa: E731
            for _ in range(warm):
                fn()
            torch.cuda.synchronize()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            for _ in range(steps):
                fn()
            e.record()
            e.synchronize()
            ms = s.elapsed_time(e) / steps
    except RuntimeError as ex:
        return {"error": str(ex)[:200]}
    return {"kernel": "torch scaled_dot_product_attention (flash / memory-efficient backend)",
            "ms": round(ms, 4), "TFLOPS": round(ops / (ms * 1e-3) / 1e12, 1),
            "step_speedup": round(ms / ms_step, 3)}


def library_gemms(torch, w, x, wt, steps, warm):
    """The ROCm libraries on the same shape, for context (not the metric):
    torch._int_mm (INT8 codes -> int32, no scales, no bias) and the
    unquantized bf16 layer (torch.nn.functional.linear), each timed like a
    step (HIP events around `steps` calls after `warm`)."""
    ops = w.ops()
    out = {}

    def clock(fn):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(steps):
            fn()
        e.record()
        e.synchronize()
        return s.elapsed_time(e) / steps

    g = torch.Generator(device=x.device).manual_seed(w.seed)
    a8 = torch.randint(-127, 128, (w.M, w.K), dtype=torch.int8, device=x.device, generator=g)
    b8 = torch.randint(-127, 128, (w.N, w.K), dtype=torch.int8, device=x.device, generator=g).t()
    ms = clock(lambda: torch._int_mm(a8, b8))
    out["int8_int_mm"] = {"ms": round(ms, 4), "TOPS": round(ops / (ms * 1e-3) / 1e12, 1),
                          "note": "INT8 x INT8 -> int32, no block scales, no bias"}
    del a8, b8
    ms = clock(lambda: torch.nn.functional.linear(x, wt))
    out["bf16_linear"] = {"ms": round(ms, 4), "TFLOPS": round(ops / (ms * 1e-3) / 1e12, 1)}
    return out


def main_linear(args, torch, sage, workloads):
    """The per-block W8A8 linear layer: one step = quantize X + GEMM."""
    w = workloads.get("linear")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t = workloads.make_linear(w, dev)
    x, wt, bias = t["x"], t["w"], t["bias"]
    y = torch.empty((w.M, w.N), dtype=x.dtype, device=dev)
    d = sage.W8A8Desc.for_tensors(x, wt, y)
    xq, xs, wq, ws = sage.w8a8_buffers(d, dev)
    stream = torch.cuda.current_stream()
    sage.sage_w8a8_quantize_weight(d, wt, wq, ws, stream)
    if args.calibrate_copy:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    steps = 2 if args.profile else args.steps
    warm = 1 if args.profile else args.warmup
    parts = (lambda: sage.sage_w8a8_quantize_act(d, x, xq, xs, stream),
             lambda: sage.sage_w8a8_gemm(d, xq, xs, wq, ws, bias, y, stream))
    ms_step, ms_quant, ms_gemm, launches = time_path(torch, parts, stream, steps, warm)
    ops = w.ops()
    qbytes = w.M * w.K * 2 + w.M * w.K + w.M * (w.K // 128) * 4  # read X, write codes and scales
    record = {
        "metric": "per-block W8A8 linear layer TOPS (2·M·N·K), 14B-class video-DiT FFN shape",
        "value": round(ops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warm,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+" + w.dtype,
        "data": "synthetic (seeded Gaussian, 1% activation channels x8)",
        "input_digests": input_digests(torch, {"x": x, "w": wt, "bias": bias.view(1, -1)}),
        "config": {"workload": "linear", "M": w.M, "N": w.N, "K": w.K, "in_dtype": w.dtype, "bias": True,
                   "ops_per_step": ops, "pct_int8_peak": round(100 * ops / (ms_step * 1e-3) / 1e12 / INT8_PEAK_TOPS, 2)},
        "roofline": {"bound": "mfma", "kernel": "w8a8_gemm_kernel", "achieved": round(ops / (ms_gemm * 1e-3) / 1e12, 2),
                     "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                     "frac": round(ops / (ms_gemm * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                     "traffic": kernel_traffic("linear", "16"), "ms_per_launch": round(ms_gemm, 4),
                     **launch_spread(launches)},
        "quantize": {"ms": round(ms_quant, 4), "algorithmic_bytes": qbytes,
                     "GB_per_s": round(qbytes / (ms_quant * 1e-3) / 1e9, 1),
                     "hbm_frac": round(qbytes / (ms_quant * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
    }
    if not args.profile:
        record["library_gemms"] = library_gemms(torch, w, x, wt, steps, warm)
    if not (args.no_cpu or args.profile):
        from threadpoolctl import threadpool_info
        from oracle import w8a8
        rows = workloads.sample_rows(w, 1024)
        X = x[rows].float().cpu().numpy()
        W = wt.float().cpu().numpy()
        B = bias.float().cpu().numpy()
        t0 = time.perf_counter()
        oxq, odx = w8a8.quantize_act(X)
        owq, odw = w8a8.quantize_weight(W)
        y64, _ = w8a8.gemm_exact(oxq, odx, owq, odw, B)
        t_cpu = time.perf_counter() - t0
        ref = w8a8.linear_fp64(X, W, B)
        yg = y[rows].float().cpu().numpy()
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        record["cpu_baseline"] = {"value": round(2 * len(rows) * w.N * w.K / t_cpu / 1e12, 6), "unit": "TOPS",
                                  "cores": threads, "kind": "oracle",
                                  "sample": f"{len(rows)} rows of X against all of W: quantize X and W + exact "
                                            f"quantized product, {t_cpu:.1f} s"}
        cos = float((yg * ref).sum() / np.sqrt((yg ** 2).sum() * (ref ** 2).sum()))
        record["parity"] = {"rows": len(rows), "max_abs_vs_exact_quantized": float(np.abs(yg - y64).max()),
                            "cosine_vs_fp64": round(cos, 6)}
    print(json.dumps(record), flush=True)


def oracle_sample(w, Q, K, V, pv_mode, b, rows, S, heads):
    """The oracle on a sample of batch b (Q, K, V: host arrays of the given heads):
    (emulated output with the kernel's KV splits, float64 attention, seconds
    the emulation -- quantization included -- took, seconds the float64
    attention took)."""
    from oracle import emulate, attention, quant
    import workloads
    kv, qp = [w.kv_lens()[b]], [w.q_pos0s()[b]]
    M = workloads.block_mask(w)
    M = M[b:b + 1, heads] if M is not None else None
    t0 = time.perf_counter()
    if M is not None:
        o64 = emulate.emulate_block_sparse(Q, K, V, pv_mode, w.dtype, M, S, w.frame_len, kv, qp, rows=rows)[0]
    elif w.frame_stride:
        mu = quant.k_mean(K, kv)
        a = quant.channel_shift(Q, K, mu, kv)
        o64 = emulate.emulate_frame_cache(Q, K, V, pv_mode, w.dtype, w.frame_len, w.frame_stride,
                                          w.sink_frames, w.window_frames, kv, qp, mu, a, S, rows=rows)[0]
    else:
        o64, _ = emulate.emulate_from_inputs(Q, K, V, pv_mode, w.dtype, frame_len=w.frame_len, kv_len=kv,
                                             q_pos0=qp, rows=rows, splits=emulate.split_ranges(kv[0], S))
    t_emul = time.perf_counter() - t0
    t0 = time.perf_counter()
    ref = attention.attention_fp64(Q, K, V, frame_len=w.frame_len, kv_len=kv, q_pos0=qp, rows=rows,
                                   sink_frames=w.sink_frames, window_frames=w.window_frames, block_mask=M)
    return o64, ref, t_emul, time.perf_counter() - t0


def accuracy_sample(w, x, o, desc, pv_mode, sage, heads=2, rows=256):
    """Cosine against float64 attention and max-abs against the emulation on a
    small sample (the first `heads` heads of batch 0, `rows` seeded rows)."""
    import workloads
    hs = list(range(min(heads, w.H)))
    r = workloads.sample_rows(w, rows)
    S = sage.sage_attn_kv_splits(desc)
    Q = x["q"][0:1, hs].float().cpu().numpy()
    K = x["k"][0:1, hs].float().cpu().numpy()
    V = x["v"][0:1, hs].float().cpu().numpy()
    o64, ref, _, _ = oracle_sample(w, Q, K, V, pv_mode, 0, r, S, hs)
    og = o[0:1, hs][:, :, r].float().cpu().numpy()
    cos = float((og * ref).sum() / np.sqrt((og ** 2).sum() * (ref ** 2).sum()))
    return {"rows": len(r) * len(hs), "max_abs_vs_emulation": float(np.abs(og - o64).max()),
            "cosine_vs_fp64": round(cos, 6)}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_leg(w, x, o, desc, args, sage, torch, full_ops):
    """Time the oracle (as it stands) on a bounded sample of the same workload,
    and compare the GPU output on the same rows."""
    from threadpoolctl import threadpool_info
    import workloads

    heads = list(range(min(args.cpu_heads, w.H)))
    rows = workloads.sample_rows(w, args.cpu_rows)
    S = sage.sage_attn_kv_splits(desc)
    b = 0
    Q = x["q"][b:b + 1, heads].float().cpu().numpy()
    K = x["k"][b:b + 1, heads].float().cpu().numpy()
    V = x["v"][b:b + 1, heads].float().cpu().numpy()
    o64, ref, t_cpu, t_ref = oracle_sample(w, Q, K, V, w.pv_mode, b, rows, S, heads)
    og = o[b:b + 1, heads][:, :, rows].float().cpu().numpy()
    if w.block_density:
        sample_ops = 4 * w.d * sum(int(w.row_keys(b, rows, h).sum()) for h in heads)
    else:
        sample_ops = 4 * w.d * int(w.row_keys(b, rows).sum()) * len(heads)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    cos = float((og * ref).sum() / np.sqrt((og ** 2).sum() * (ref ** 2).sum()))
    cpu = {"value": round(sample_ops / t_cpu / 1e12, 6), "unit": "TOPS", "cores": threads, "kind": "oracle",
           "sample": f"batch 0, heads {heads[0]}..{heads[-1]}, {len(rows)} query rows each "
                     f"(all their visible keys), quantize + emulated attention, "
                     f"{t_cpu:.1f} s",
           "fp64_reference": {"s": float(f"{t_ref:.4g}"), "TOPS": float(f"{sample_ops / t_ref / 1e12:.4g}")},
           "extrapolated_full_workload_s": round(t_cpu * full_ops / sample_ops, 1),
           "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count()}
    parity = {"rows": len(rows) * len(heads), "max_abs_vs_emulation": float(np.abs(og - o64).max()),
              "cosine_vs_fp64": round(cos, 6)}
    return cpu, parity


if __name__ == "__main__":
    main()
