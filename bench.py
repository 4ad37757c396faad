"""Benchmark: Jensen-bias-corrected INT2 chunk attention on one MI355X.

One step = the whole hot path for one chunk of the c40 workload (B=1, H=40, d=128,
current chunk 4680 tokens, window of 8 cached chunks = 37,440 tokens, per-token INT2
keys and values with Hadamard rotation, Taylor correction):
  1. jb_attn_fwd: corrected attention of the chunk's queries over [window ; chunk],
     with the cached/current masses;
  2. kvq_pack of the chunk's keys and values (what the cache stores for the next chunk).
Inputs are resident in HBM before timing starts. ``value`` is attention TFLOP/s over the
step time, counting the algorithmic FLOP 4 * n_q * (n_c + n_r) * d * B * H (QK^T + PV).

Printed: one JSON line with the driver's fields plus ``roofline`` (the attention kernel,
timed with HIP events on the stream it runs on, against the 2.5 PFLOP/s dense fp16/bf16
MFMA peak) and ``cpu_baseline`` (the float64 oracle on a bounded sample, on host cores).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA_TFLOPS = 2500.0        # MI355X dense fp16/bf16 MFMA
PEAK_FP6_TFLOPS = 10100.0        # MI355X dense fp6/fp4 MFMA
FP6_PASSES = 3                   # query passes of the fp4 x fp6 QK^T


def fp6_qk(w, decode, correction=1):
    """Whether the attention kernel runs QK^T on the scaled fp4/fp6 x fp6 MFMA: per-token
    keys, 2-bit in both kernels, 4-bit in the main kernel (the few-query path keeps int8);
    group-wise keys in two 64-channel groups without the exact correction."""
    if w.k_granularity == "token_group":
        return w.group == 64 and w.d == 128 and correction != 2 and not decode
    return w.k_granularity == "token" and (w.bits == 2 or not decode)


def path_dtype(w, decode, correction=1):
    """The arithmetic of the path: QK^T operands, then the bias / PV MFMAs' fp16."""
    if fp6_qk(w, decode, correction):
        return "fp4xfp6+fp16" if w.bits == 2 else "fp6xfp6+fp16"
    if w.k_granularity == "token_group":
        return "fp16"
    return "int8+fp16"


def mixed_peak():
    """The peak of the fp6 path's instruction mix: half the algorithmic FLOPs (QK^T) run as
    FP6_PASSES fp6 passes at the fp6 peak, the other half (PV) at the fp16 peak."""
    return 1.0 / (0.5 * FP6_PASSES / PEAK_FP6_TFLOPS + 0.5 / PEAK_MFMA_TFLOPS)
PEAK_HBM_GBS = 8000.0
METRIC = "jb_attn TFLOP/s + cache GB/s (% roofline), INT2 corrected, 40H d128 chunk 4680"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "jb_attn_c40_counters.md")
CORR_NAMES = {0: "none", 1: "taylor", 2: "exact"}
KERNEL_SOURCE = os.path.join(ROOT, "bit_kv_cache_kvq_amd", "csrc", "attn.hip")


# Further workloads timed after the headline (attention kernel only, per-launch HIP events):
# name -> (workload, replacements, correction)
OTHERS = {
    "tiny": ("tiny", {}, 1),
    "c24": ("c24", {}, 1),
    "c40_perch": ("c40_perch", {}, 1),
    "c40_perch_span": ("c40_perch_span", {}, 1),
    "long": ("long", {}, 1),
    "c40_int4": ("c40", {"bits": 4}, 1),
    "c40_q16": ("c40", {"n_q": 16}, 1),
    "c40_int4_q16": ("c40", {"n_q": 16, "bits": 4}, 1),
    "long_q16": ("long", {"n_q": 16}, 1),
    "c40_tgroup32": ("c40_tgroup", {"group": 32}, 1),
    "c40_tgroup64": ("c40_tgroup", {"group": 64}, 1),
    "c40_exact": ("c40", {}, 2),
    "c40_perch_exact": ("c40_perch", {}, 2),
}
OTHER_LAUNCHES = 10


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def counters_from_profile():
    """HBM bytes per launch and matrix-core / VALU busy fractions from the committed counter
    summary, if it describes this kernel source (else an empty dict)."""
    try:
        txt = open(TRAFFIC_FILE).read()
    except OSError:
        return {}
    m_hash = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]{16})", txt)
    if not m_hash or m_hash.group(1) != kernel_source_hash():
        return {}
    out = {}
    for key, name in (("hbm_bytes_per_launch", "traffic"), ("mfma_busy", "mfma_busy"), ("valu_busy", "valu_busy")):
        m = re.search(key + r":\s*([0-9.eE+]+)", txt)
        if m:
            out[name] = float(m.group(1))
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def gran_text(w, gran):
    """Words for a quantization granularity of the workload's keys or values."""
    if gran == "token_group":
        return f"per-token groups of {w.group} channels,"
    if gran == "channel":
        return f"per-channel ({w.group}-token groups)"
    return "per-token"


def window_memory(w):
    """Device bytes of this workload's cached window (K and V) in INT2, INT4 and bf16: the
    memory a fixed window takes, or the window a fixed budget holds (§1)."""
    from bit_kv_cache_kvq_amd import kvq, window
    def kv(bits):
        kf = kvq.KvqFormat.make(bits, w.k_granularity, w.group, True, "key")
        vf = kvq.KvqFormat.make(bits, w.v_granularity, w.group, True, "value")
        return sum(window.window_bytes(f, w.B, w.H, w.d, w.chunk_len, w.n_chunks) for f in (kf, vf))
    b2, b4, b16 = kv(2), kv(4), 2 * w.B * w.H * w.n_chunks * w.chunk_len * w.d * 2
    return {"int2_bytes": b2, "int4_bytes": b4, "bf16_bytes": b16, "int2_over_int4": round(b2 / b4, 4),
            "int2_over_bf16": round(b2 / b16, 4)}


def cpu_baseline(w, x, heads, kf_o, vf_o, correction="taylor"):
    """Time the oracle (as it stands) on `heads`: pack of the current chunk + attention."""
    import numpy as np
    import oracle
    from oracle.quant import pack_window

    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"), default=1)
    except Exception:  # pragma: no cover
        blas = affinity
    threads = min(blas, affinity)  # the BLAS threads that do the oracle's matrix products
    xs = {k: np.stack([v[b, h] for (b, h) in heads])[None] for k, v in x.items()}
    cache = oracle.attention.quantize_cache(xs["k_cache"], xs["v_cache"], w.chunk_len, kf_o, vf_o)
    t0 = time.perf_counter()
    pack_window(xs["k_cur"], w.n_r, kf_o)
    pack_window(xs["v_cur"], w.n_r, vf_o)
    O, PS, PR, _ = oracle.reference_call(xs["q"], xs["k_cache"], xs["v_cache"], xs["k_cur"], xs["v_cur"],
                                         chunk_len=w.chunk_len, k_fmt=kf_o, v_fmt=vf_o, correction=correction,
                                         cache=cache)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.n_q * (w.n_c + w.n_r) * w.d * len(heads)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "affinity_cores": affinity,
            "blas_threads": int(blas), "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{len(heads)} of {w.bh} heads, all {w.n_q} query rows: float64 attention over the "
                      f"dequantized window + current chunk, plus float32-contract packing of the current "
                      f"chunk's K and V ({dt:.1f} s)"}, (O, PS, PR)


def measure_other(key, launches=OTHER_LAUNCHES, warmup=3):
    """Time one further workload's attention call (the whole call: split, merge or decode
    kernels included) with per-launch HIP events on its stream; median and min launch."""
    import numpy as np
    import torch

    from bit_kv_cache_kvq_amd import kvq, synth

    name, repl, correction = OTHERS[key]
    w = synth.WORKLOADS[name].replace(**repl)
    x = synth.draw_all(w)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()

    kf = kvq.KvqFormat.make(w.bits, w.k_granularity, w.group, True, "key")
    vf = kvq.KvqFormat.make(w.bits, w.v_granularity, w.group, True, "value")
    q, kr, vr = dev(x["q"]), dev(x["k_cur"]), dev(x["v_cur"])
    kwin = kvq.pack_window(dev(x["k_cache"]), w.chunk_len, kf)
    vwin = kvq.pack_window(dev(x["v_cache"]), w.chunk_len, vf)
    del x
    o = torch.empty((w.B, w.H, w.n_q, w.d), dtype=torch.float32, device="cuda")
    ms = torch.empty((w.B, w.H, w.n_q), dtype=torch.float32, device="cuda")
    mr = torch.empty_like(ms)
    a = kvq.make_args(q, kr, vr, kwin, vwin, w.chunk_len, w.n_chunks, kf, vf, o=o, mass_s=ms, mass_r=mr,
                      correction=correction)
    ws = kvq.attach_workspace(a)
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        kvq.jb_attn_fwd(a, stream)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for e0, e1 in evs:
        e0.record(stream)
        kvq.jb_attn_fwd(a, stream)
        e1.record(stream)
    torch.cuda.synchronize()
    t = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    med = float(np.median(t))
    cache_bytes = sum(v.numel() * v.element_size() for v in (*kwin, *vwin))
    algo_bytes = cache_bytes + 3 * w.bh * w.n_q * w.d * 2 + w.bh * w.n_q * (w.d + 2) * 4
    decode = w.n_q <= 32 and w.k_granularity == "token" and correction != 2 and a.workspace_bytes > 0
    rec = {"workload": f"{w.name} B={w.B} H={w.H} n_q={w.n_q} window {w.n_chunks}x{w.chunk_len} INT{w.bits} "
                       f"K {gran_text(w, w.k_granularity)} correction={CORR_NAMES[correction]}",
           "attn_ms_median": round(med, 5), "attn_ms_min": round(float(t.min()), 5),
           "attn_ms_mean": round(float(t.mean()), 5), "launches": launches,
           "path": "decode" if decode else ("split" if a.workspace_bytes > 0 else "main"),
           "TFLOPs": round(w.flops() / (med * 1e-3) / 1e12, 2)}
    if decode:
        gbs = algo_bytes / (med * 1e-3) / 1e9
        rec.update({"bound": "hbm", "GBps": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)})
    else:
        rec.update({"bound": "mfma", "frac": round(w.flops() / (med * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS, 4)})
        if fp6_qk(w, decode, correction):
            rec["frac_mixed"] = round(w.flops() / (med * 1e-3) / 1e12 / mixed_peak(), 4)
    del ws, q, kr, vr, kwin, vwin, o, ms, mr
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c40")
    ap.add_argument("--bits", type=int, default=None)
    ap.add_argument("--correction", type=int, default=1, choices=sorted(CORR_NAMES),
                    help="0 none, 1 second-order Taylor (the headline), 2 exact")
    ap.add_argument("--cpu-heads", type=int, default=16, help="heads in the oracle timing sample (0: skip)")
    ap.add_argument("--nq", type=int, default=0,
                    help="queries (and current-chunk tokens) per head instead of the workload's; at most 32 "
                         "takes the few-query (decode) path, whose roofline is the HBM stream of the window")
    ap.add_argument("--no-workspace", action="store_true",
                    help="run without a workspace (no split, no decode path): the main kernel alone")
    ap.add_argument("--layers", type=int, default=1,
                    help="independent calls per step (e.g. the layers of one chunk step), run in one batched "
                         "launch (jb_attn_fwd_batch) when above 1")
    ap.add_argument("--group", type=int, default=0,
                    help="replace the workload's group size (channels per group for group-wise keys and values)")
    ap.add_argument("--others", default=",".join(OTHERS),
                    help="comma-separated list of further workloads whose attention kernel is timed after the "
                         "headline (reported under 'workloads'); 'none' skips them")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="only run a device copy of this many MiB (HBM counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by head with no communication; see the design notes)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from bit_kv_cache_kvq_amd import kvq, synth
    from oracle.quant import Format

    torch.cuda.set_device(0)
    if args.calib_copy_mb:
        n = args.calib_copy_mb * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_read": n * 4, "calib_copy_bytes_written": n * 4, "launches": 5}))
        return

    w = synth.WORKLOADS[args.workload]
    if args.bits:
        w = w.replace(bits=args.bits)
    if args.nq:
        w = w.replace(n_q=args.nq)
    if args.group:
        w = w.replace(group=args.group)
    t_gen = time.perf_counter()
    x = synth.draw_all(w)
    print(f"# generated {w.name} inputs in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()

    kf = kvq.KvqFormat.make(w.bits, w.k_granularity, w.group, True, "key")
    vf = kvq.KvqFormat.make(w.bits, w.v_granularity, w.group, True, "value")
    if not 1 <= args.layers <= kvq.KVQ_BATCH_MAX:
        print(f"--layers must be in 1..{kvq.KVQ_BATCH_MAX}", file=sys.stderr)
        sys.exit(2)

    def layer(xl):
        """Device inputs, outputs and call arguments of one layer's attention call."""
        t = {"q": dev(xl["q"]), "kr": dev(xl["k_cur"]), "vr": dev(xl["v_cur"])}
        t["kwin"] = kvq.pack_window(dev(xl["k_cache"]), w.chunk_len, kf)
        t["vwin"] = kvq.pack_window(dev(xl["v_cache"]), w.chunk_len, vf)
        t["o"] = torch.empty((w.B, w.H, w.n_q, w.d), dtype=torch.float32, device="cuda")
        t["ms"] = torch.empty((w.B, w.H, w.n_q), dtype=torch.float32, device="cuda")
        t["mr"] = torch.empty_like(t["ms"])
        t["knext"] = kvq.alloc_window(kf, w.B, w.H, w.d, w.n_r, 1)
        t["vnext"] = kvq.alloc_window(vf, w.B, w.H, w.d, w.n_r, 1)
        t["args"] = kvq.make_args(t["q"], t["kr"], t["vr"], t["kwin"], t["vwin"], w.chunk_len, w.n_chunks, kf, vf,
                                  o=t["o"], mass_s=t["ms"], mass_r=t["mr"], correction=args.correction)
        # split-window partials when the grid is small for the device (one call) and the
        # records of the few-query path
        t["ws"] = None if args.no_workspace else kvq.attach_workspace(t["args"])
        return t

    layers = [layer(x)] + [layer(synth.draw_all(w.replace(seed=w.seed + 1000 + i))) for i in range(1, args.layers)]
    L0 = layers[0]
    q, kr, vr, kwin, vwin, o = L0["q"], L0["kr"], L0["vr"], L0["kwin"], L0["vwin"], L0["o"]
    knext, vnext, a = L0["knext"], L0["vnext"], L0["args"]
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if len(layers) == 1:
            kvq.jb_attn_fwd(a, stream)
        else:
            kvq.jb_attn_fwd_batch([t["args"] for t in layers], stream)
        if ev is not None:
            ev[1].record(stream)
        for t in layers:
            kvq.kvq_pack(t["kr"], kf, 1, 0, *t["knext"], stream)
            kvq.kvq_pack(t["vr"], vf, 1, 0, *t["vnext"], stream)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    attn_all = np.array([e0.elapsed_time(e1) for (e0, e1, _) in evs])
    attn_ms = float(attn_all.mean())
    pack_ms = float(np.mean([e1.elapsed_time(e2) for (_, e1, e2) in evs]))
    # algorithmic bytes of the two packs: the chunk's bf16 keys and values read once, their
    # codes, steps and zero points written once
    nl = len(layers)
    pack_bytes = nl * (2 * w.bh * w.n_r * w.d * 2 + sum(t.numel() * t.element_size() for t in (*knext, *vnext)))

    flops = nl * w.flops()
    cache_bytes = nl * (kwin[0].numel() * 4 + kwin[1].numel() * 2 * 2 + vwin[0].numel() * 4 + vwin[1].numel() * 2 * 2)
    # algorithmic bytes of the step's attention: the cache windows once, Q/K_r/V_r (bf16), O and masses (fp32)
    algo_bytes = cache_bytes + nl * (3 * w.bh * w.n_q * w.d * 2 + w.bh * w.n_q * (w.d + 2) * 4)
    achieved = flops / (attn_ms * 1e-3) / 1e12
    decode = (w.n_q <= 32 and w.k_granularity == "token" and args.correction != 2 and a.workspace_bytes > 0
              and nl == 1)
    value = flops / (ms_step * 1e-3) / 1e12
    # the committed counters describe one c40 launch of this kernel source
    ctr = counters_from_profile() if (w.name == "c40" and nl == 1 and w.bits == 2 and args.correction == 1
                                      and not args.nq and not args.no_workspace) else {}
    traffic = ctr.get("traffic")

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": path_dtype(w, decode, args.correction),
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B={w.B} H={w.H} d={w.d}, current chunk {w.n_q} tokens, window "
                               f"{w.n_chunks}x{w.chunk_len} cached tokens, INT{w.bits} {gran_text(w, w.k_granularity)} K, "
                               f"{gran_text(w, w.v_granularity)} V, Hadamard, correction={CORR_NAMES[args.correction]}",
                   "B": w.B, "H": w.H, "d": w.d, "n_q": w.n_q, "n_c": w.n_c, "bits": w.bits,
                   "parallelism": "none (1 GPU)", "split_workspace_bytes": a.workspace_bytes, "layers": nl,
                   "batched_launch": nl > 1},
        "attn_ms": round(attn_ms, 4),
        "attn_ms_median": round(float(np.median(attn_all)), 4),
        "attn_ms_min": round(float(attn_all.min()), 4),
        "cache_GBps": round(cache_bytes / (attn_ms * 1e-3) / 1e9, 2),
        "window_memory": window_memory(w),
        "cache_frac_hbm": round(cache_bytes / (attn_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 5),
        "pack": {"ms": round(pack_ms, 4), "algorithmic_bytes": pack_bytes,
                 "GBps": round(pack_bytes / (pack_ms * 1e-3) / 1e9, 1),
                 "frac_hbm": round(pack_bytes / (pack_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)},
        "roofline": ({"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_MFMA_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(achieved / PEAK_MFMA_TFLOPS, 4)} if not decode else
                     {"bound": "hbm", "achieved": round(algo_bytes / (attn_ms * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS,
                      "unit": "GB/s", "frac": round(algo_bytes / (attn_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)})
        | ({"peak_mixed": round(mixed_peak(), 1), "frac_mixed": round(achieved / mixed_peak(), 4)}
           if fp6_qk(w, decode, args.correction) and not decode else {})
        | {"traffic": (round(traffic) if traffic is not None else None),
           "algorithmic_bytes": algo_bytes, "kernel_source_sha256_16": kernel_source_hash(),
           "mfma_busy": ctr.get("mfma_busy"), "valu_busy": ctr.get("valu_busy")},
        "path": "decode" if decode else ("batched" if nl > 1 else "main"),
    }
    if args.cpu_heads > 0:
        heads = [(0, h) for h in range(min(args.cpu_heads, w.bh))] if w.B == 1 else \
            [(b, h) for b in range(w.B) for h in range(w.H)][: args.cpu_heads]
        kf_o = Format(w.bits, w.k_granularity, w.group, True, "key")
        vf_o = Format(w.bits, w.v_granularity, w.group, True, "value")
        base, (O, PS, PR) = cpu_baseline(w, x, heads, kf_o, vf_o, CORR_NAMES[args.correction])
        og = np.stack([o[b, h].cpu().numpy() for (b, h) in heads])[None]
        rms = np.sqrt((O ** 2).mean())
        err = np.abs(og - O)
        rec["cpu_baseline"] = base
        rec["parity_on_sample"] = {"max_err_over_rms": float(err.max() / rms), "mean_err_over_rms": float(err.mean() / rms)}
    others = [k for k in args.others.split(",") if k and k != "none"]
    if others:
        del layers, L0, q, kr, vr, kwin, vwin, o, knext, vnext, a, x
        torch.cuda.empty_cache()
        rec["workloads"] = {}
        for k in others:
            if k not in OTHERS:
                print(f"unknown workload {k!r} (known: {', '.join(OTHERS)})", file=sys.stderr)
                sys.exit(2)
            t_o = time.perf_counter()
            rec["workloads"][k] = measure_other(k)
            print(f"# {k}: {rec['workloads'][k]['attn_ms_median']} ms ({time.perf_counter() - t_o:.1f} s)",
                  file=sys.stderr, flush=True)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
