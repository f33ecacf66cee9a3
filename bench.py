"""Throughput of the JEPA ViT encoder forward on one MI355X.

One step = one whole forward of a batch (patchify + patch-embed + every block +
final LayerNorm) plus the pool the workload reports (and, for a workload with
the attentive-pool classifier head, its class scores), with frames already
resident in HBM.  Default workload: the LeVJEPA-style ViT-L/16 video encoder,
16 frames of 224x224, tubelet 1, block-causal, bf16, batch 4 (3137 tokens per
clip), synthetic seeded frames and N(0, 0.02) weights.

Prints one JSON line: tokens/s (whole job), clips/s, MFMA utilisation of the
whole forward against the dense bf16/f16 peak, the roofline of the dominant
kernel, and the CPU oracle timed on a bounded sample.

Two timed regions of K steps each.  The first gives `value`: the encoder as
it runs by default (the batch split into concurrent parts, one HIP stream
each), with no timing events between kernels.  The second gives the
roofline: the same steps with the batch as one part, HIP events around each
launch of the dominant kernel class on its stream, so that a launch's
duration is its own and not shared with another part's kernels; achieved =
algorithmic work per launch / average launch duration.

usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--parts P] [--no-cpu-baseline] [--breakdown]
       python bench.py --gemm-k-sweep    (the large GEMM tile's fixed and per-K-step costs)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from vision_transformer_amd import synth  # noqa: E402

METRIC = "encoder tokens/sec + clips/sec (ViT-L/16, 16 frames), MFMA util % of peak"
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "f32": 157.3}   # dense MFMA, MI355X
PEAK_INT8_TOPS = 5000.0                                          # dense int8 MFMA, MI355X
PEAK_HBM_GBS = 8000.0


# ---------------------------------------------------------------------------
# algorithmic work
# ---------------------------------------------------------------------------

def attention_pairs(dims: dict) -> int:
    """Allowed (query, key) pairs of one item."""
    N = synth.n_tokens(dims)
    if dims["mask"] == "bidir":
        return N * N
    T, h, w = synth.grid(dims)
    per = h * w
    pairs = per * per * T * (T + 1) // 2
    return pairs + (N if dims["has_cls"] else 0)


def class_flops(dims: dict, B: int) -> dict:
    """Algorithmic FLOPs of one launch of each kernel class."""
    D, F = dims["dim"], dims["mlp_dim"]
    M = B * synth.n_tokens(dims)
    return {
        "gemm_patch": 2 * B * synth.n_patches(dims) * synth.patch_dim(dims) * D,
        "gemm_qkv": 2 * M * 3 * D * D,
        "gemm_out": 2 * M * D * D,
        "gemm_fc1": 2 * M * F * D,
        "gemm_fc2": 2 * M * D * F,
        "attention": 4 * B * attention_pairs(dims) * D,
    }


def forward_flops(dims: dict, B: int) -> int:
    f = class_flops(dims, B)
    gemms = f["gemm_qkv"] + f["gemm_out"] + f["gemm_fc1"] + f["gemm_fc2"]
    total = f["gemm_patch"] + dims["depth"] * (gemms + f["attention"])
    if dims.get("head_classes"):
        # the classifier head: its blocks (bidirectional over every token), the
        # keys and values of the tokens, the query row's products and attention
        D, F, C, N = dims["dim"], dims["mlp_dim"], dims["head_classes"], synth.n_tokens(dims)
        M = B * N
        total += dims["head_blocks"] * (gemms + 4 * B * N * N * D)
        total += 2 * (2 * M * D * D) + 2 * B * (2 * D * D + 2 * D * F + D * C) + 4 * B * N * D
    return total


def class_bytes(dims: dict, B: int) -> dict:
    """Algorithmic HBM bytes of one launch of the bandwidth-bound classes."""
    D = dims["dim"]
    M = B * synth.n_tokens(dims)
    es = 4 if dims["act_dtype"] == "f32" else 2
    npad = -(-synth.n_tokens(dims) // 64) * 64
    F = dims["mlp_dim"]
    # the int8 path's input quantiser: per block's four products, three of
    # width D and one of width F, each read in the act dtype and written as
    # int8 codes plus one f32 scale per 32 values (the average launch)
    quant = M * (3 * D + F) * (es + 1 + 4 / 32) / 4
    return {"layernorm": M * D * (4 + es), "final_ln": M * D * 8,
            "transpose_v": M * D * es + B * D * npad * es, "quant_act": int(quant)}


def measured_traffic(workload: str, cls: str):
    """HBM-side bytes per launch of kernel class `cls` from the FETCH_SIZE /
    WRITE_SIZE summaries under profiles/ (copy-calibrated), or None when none
    exists or the kernel's sources changed since the counters were taken."""
    import glob
    import hashlib
    csrc = os.path.join(ROOT, "vision_transformer_amd", "csrc")
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_hbm_traffic.md"))):
        for line in open(path):
            f = line.split()
            if len(f) != 6 or f[0] != "traffic" or f[1] != workload or f[2] != cls:
                continue
            kv = dict(x.split("=", 1) for x in f[3:])
            h = hashlib.sha256()
            try:
                for name in kv["sources"].split(","):
                    h.update(open(os.path.join(csrc, name), "rb").read())
            except OSError:
                return None
            if h.hexdigest() == kv["sha256"]:
                return int(kv["bytes"]), os.path.relpath(path, ROOT)
            return None
    return None


# ---------------------------------------------------------------------------
# CPU oracle on a bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(dims: dict, stored: list, frames: np.ndarray, sample_blocks: int) -> dict:
    from oracle import encoder as E
    try:
        from threadpoolctl import threadpool_info
        cores = max(i.get("num_threads", 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:
        cores = len(os.sched_getaffinity(0))
    ds = dict(dims, depth=sample_blocks)
    names = {n for n, _, _ in synth.tensor_specs(ds)}
    w = E.weights_f64([t for t in stored if t["name"] in names])
    clip = frames[:1]
    load0 = os.getloadavg()[0]
    t0 = time.perf_counter()
    E.encode(ds, w, clip)
    dt = time.perf_counter() - t0
    per_clip = dt * dims["depth"] / sample_blocks
    N = synth.n_tokens(dims)
    return {"value": N / per_clip, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"1 clip of the batch of {len(frames)}, {sample_blocks} of {dims['depth']} blocks "
                       f"(float64 numpy oracle), {dt:.1f} s"
                       + (f", scaled x{dims['depth'] / sample_blocks:g} to a whole clip"
                          if sample_blocks != dims["depth"] else "")),
            "clips_per_s": 1.0 / per_clip, "cpu_model": cpu_model(),
            "cpus_available": len(os.sched_getaffinity(0)), "load_avg_1min_before": load0,
            "load_avg_1min_after": os.getloadavg()[0]}


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

def mfma_probe(_lib, operands: int = 0) -> dict | None:
    """Dense bf16 MFMA TFLOP/s of the calibration kernel: one workgroup per
    CU, about 0.1 s of independent 32x32x16 MFMA chains, timed with events;
    operands 0: constant small values, 1: random values whose bits toggle
    from one MFMA to the next, as a GEMM's do (the rate the chip's power
    allows on real data)."""
    import torch
    try:
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        out = torch.empty(cus * 256, dtype=torch.float32, device="cuda")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

        def run(iters):
            torch.cuda.synchronize()
            e0.record()
            flops = _lib.jepa_op_mfma_probe(cus, iters, out, operands)
            e1.record()
            torch.cuda.synchronize()
            return flops, e0.elapsed_time(e1)

        flops, ms = run(20000)
        iters = max(20000, int(20000 * 100.0 / max(ms, 1e-3)))   # about 100 ms
        flops, ms = run(iters)
        if not torch.isfinite(out).all():
            return None
        return {"tflops": round(flops / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 2), "iters": iters,
                "workgroups": cus}
    except Exception as e:   # a calibration row: report, do not fail the bench
        print(f"[bench] MFMA probe not measured: {e}", file=sys.stderr, flush=True)
        return None


def device_info() -> dict:
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2 ** 30, 1), "hip": torch.version.hip, "torch": torch.__version__}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_probe(mib: int) -> int:
    """A plain device-to-device copy of known size: it reads and writes
    exactly mib MiB per launch, which calibrates FETCH_SIZE / WRITE_SIZE."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    print(json.dumps({"copy_probe_bytes": n, "ms": round(ms, 4), "GB_per_s_read_plus_write": round(2 * n / ms / 1e6, 1)}),
          flush=True)
    return 0


def gemm_k_sweep() -> int:
    """The 256 x 256 tile's time against K at whole rounds of 256 tiles
    (one tile per CU per round): per round, time = fixed + steps * per_step,
    fixed being a tile's prologue (first operand stages in flight, biases)
    plus its epilogue, per_step the steady K loop's 64-deep step.  A
    least-squares line over K >= 512 gives both; per_step is set against the
    same step's MFMA time at the rate jepa_op_mfma_probe measures with random
    operands."""
    import torch
    from vision_transformer_amd import _lib
    os.environ["JEPA_GEMM_VARIANT"] = "big256"
    probe = mfma_probe(_lib, 1)   # random operands: the rate real data allows
    torch.manual_seed(0)
    dev = torch.device("cuda")
    cases = [("store", 12288, 4096), ("gelu", 12288, 4096), ("resid", 16384, 1024)]
    ks = [128, 256, 512, 1024, 2048, 4096]
    res = {"mfma_probe_random_operands_tflops": probe["tflops"] if probe else None, "cases": []}
    for epi, M, N in cases:
        rounds = (M // 256) * (N // 256) / 256
        b = torch.randn(N, device=dev) * 0.02
        out = torch.zeros(M, N, device=dev, dtype=torch.float32 if epi == "resid" else torch.bfloat16)
        pts = []
        for K in ks:
            a = (torch.randn(M, K, device=dev) * 0.5).to(torch.bfloat16)
            w = (torch.randn(N, K, device=dev) * 0.02).to(torch.bfloat16)
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 0.5:   # clocks settle under this load
                _lib.jepa_op_gemm("bf16", a, w, "bf16", N, b, epi, out)
                torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            it = 20
            e0.record()
            for _ in range(it):
                _lib.jepa_op_gemm("bf16", a, w, "bf16", N, b, epi, out)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / it
            pts.append({"K": K, "us": round(us, 2), "us_per_round": round(us / rounds, 3),
                        "tflops": round(2.0 * M * N * K / us / 1e6, 1)})
            print(f"[bench] gemm {epi} M={M} N={N} K={K}: {us:.2f} us", file=sys.stderr, flush=True)
        fit = [(p["K"] / 64, p["us_per_round"]) for p in pts if p["K"] >= 512]
        n = len(fit)
        sx = sum(x for x, _ in fit); sy = sum(y for _, y in fit)
        sxx = sum(x * x for x, _ in fit); sxy = sum(x * y for x, y in fit)
        slope = (n * sxy - sx * sy) / (n * sxx - sx * sx)
        icpt = (sy - slope * sx) / n
        case = {"epilogue": epi, "M": M, "N": N, "rounds": rounds, "points": pts,
                "fixed_us_per_tile": round(icpt, 2), "us_per_k_step": round(slope, 4)}
        if probe:
            # one step: 2 * 256 * 256 * 64 flops on one CU
            ideal = 2.0 * 256 * 256 * 64 / (probe["tflops"] * 1e12 / 256) * 1e6
            case["mfma_us_per_k_step_at_probe_rate"] = round(ideal, 4)
            case["k_loop_fraction_of_probe_rate"] = round(ideal / slope, 3)
        res["cases"].append(case)
    # The same K step with a quarter, half and all of the CUs holding a tile
    # (N 1024, plain store, K 2048 -> 4096): a step slower at full occupancy
    # than on a part of the chip is the clock the chip's power limit allows,
    # not the kernel's schedule.
    occ = []
    N = 1024
    b = torch.randn(N, device=dev) * 0.02
    for M in (4096, 8192, 16384):
        out = torch.zeros(M, N, device=dev, dtype=torch.bfloat16)
        row = {"M": M, "tiles": (M // 256) * (N // 256)}
        for K in (2048, 4096):
            a = (torch.randn(M, K, device=dev) * 0.5).to(torch.bfloat16)
            w = (torch.randn(N, K, device=dev) * 0.02).to(torch.bfloat16)
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 0.5:
                _lib.jepa_op_gemm("bf16", a, w, "bf16", N, b, "store", out)
                torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                _lib.jepa_op_gemm("bf16", a, w, "bf16", N, b, "store", out)
            e1.record()
            torch.cuda.synchronize()
            row[f"us_K{K}"] = round(e0.elapsed_time(e1) * 1e3 / 20, 2)
        row["us_per_k_step"] = round((row["us_K4096"] - row["us_K2048"]) / 32, 4)
        row["tflops_per_cu"] = round(2.0 * 256 * 256 * 64 / (row["us_per_k_step"] * 1e-6) / 1e12, 2)
        occ.append(row)
        print(f"[bench] gemm store M={M} N={N}: {row['us_per_k_step']:.4f} us per K step", file=sys.stderr, flush=True)
    res["occupancy"] = occ
    print(json.dumps({"gemm_k_sweep": res}), flush=True)
    return 0


# The other specified workloads, timed by the default run after the headline
# one (a few steps each, default concurrency): reported beside `value`,
# which stays the headline workload's.
OTHER_WORKLOADS = ["vit_ti14_image_f32", "vit_l16_image_bf16_b32", "vjepa2_vit_l16_16f256_q8_0_b4",
                   "vjepa2_vit_l16_64f256_f16", "vjepa2_vit_l16_64f256_q4_0"]
INT8_WORKLOADS = ["vjepa2_vit_l16_16f256_q8_0_b4", "vjepa2_vit_l16_64f256_q4_0"]


def time_workload(name: str, steps: int, warmup: int, int8: bool = False) -> dict:
    """ms per step, tokens/s, clips/s and MFMA utilisation of one workload's
    forward + its reported pool (+ class scores), the batch in the library's
    default concurrent parts, frames resident.  int8: the block matrices'
    products on the int8 path (jepa_set_int8_matmul)."""
    import torch
    from vision_transformer_amd import _lib
    from vision_transformer_amd.encoder import Encoder
    wl = synth.workload(name)
    dims, B = wl["dims"], wl["batch"]
    N = synth.n_tokens(dims)
    frames = synth.make_frames(dims, B, wl["frame_seed"])
    stored = synth.stored_weights(dims, synth.make_f32_weights(dims, wl["weight_seed"]),
                                  quantize=_lib.jepa_quantize)
    enc = Encoder(dims, stored)
    del stored
    if int8:
        enc.set_int8_matmul(True)
    fr = torch.from_numpy(frames).cuda()
    tokens = torch.empty((B, N, dims["dim"]), dtype=torch.float32, device="cuda")
    pool_mode = "cls" if dims["has_cls"] else "mean"
    pooled = torch.empty((B, dims["dim"]), dtype=torch.float32, device="cuda")

    def step():
        enc.encode(fr, tokens)
        enc.pool(pool_mode, B, pooled)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / steps
    enc.close()
    act = dims["act_dtype"]
    util = forward_flops(dims, B) / (ms * 1e-3) / (PEAK_TFLOPS[act] * 1e12)
    print(f"[bench] {name}{' (int8 products)' if int8 else ''}: {ms:.3f} ms per step", file=sys.stderr, flush=True)
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(B * N / (ms * 1e-3), 1),
            "clips_per_s": round(B / (ms * 1e-3), 2), "mfma_util_pct": round(100 * util, 2),
            "batch": B, "tokens_per_clip": N, "dtype": act, "weights": dims["mat_dtype"],
            "mask": dims["mask"], "steps": steps, "warmup": warmup, "int8_products": int8}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="levjepa_vit_l16_16f_bf16_b4",
                    choices=sorted(synth.WORKLOADS))
    ap.add_argument("--batch", type=int, default=0, help="override the workload's batch")
    ap.add_argument("--parts", type=int, default=0,
                    help="concurrent batch parts of the throughput region (0 = the library default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-blocks", type=int, default=24)
    ap.add_argument("--breakdown", action="store_true", help="print per-kernel-class times to stderr")
    ap.add_argument("--int8", action="store_true",
                    help="run the block matrices' products on the int8 path (q8_0 / q4_0 workloads)")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip timing the other specified workloads after the headline one")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device to device 5 times (the reference kernel of known "
                         "traffic that scales the HBM counters) and exit")
    ap.add_argument("--gemm-k-sweep", action="store_true",
                    help="only time the 256 x 256 GEMM tile against K at whole rounds of tiles "
                         "(fixed cost per tile and per-K-step rate) and exit")
    args = ap.parse_args()
    if args.copy_probe:
        return copy_probe(args.copy_probe)
    if args.gemm_k_sweep:
        return gemm_k_sweep()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the encoder path is built and measured on a single "
              "MI355X (multi-GPU data/sequence parallelism is design-only here). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    import torch
    from vision_transformer_amd import _lib
    from vision_transformer_amd.encoder import Encoder

    wl = synth.workload(args.workload)
    dims = wl["dims"]
    B = args.batch or wl["batch"]
    N = synth.n_tokens(dims)
    act = dims["act_dtype"]
    print(f"[bench] workload {args.workload}: B={B} N={N} D={dims['dim']} L={dims['depth']} "
          f"{dims['mask']} act={act} weights={dims['mat_dtype']}", file=sys.stderr, flush=True)

    frames = synth.make_frames(dims, B, wl["frame_seed"])
    stored = synth.stored_weights(dims, synth.make_f32_weights(dims, wl["weight_seed"]),
                                  quantize=_lib.jepa_quantize)
    enc = Encoder(dims, stored)
    if args.int8:
        enc.set_int8_matmul(True)
    fr = torch.from_numpy(frames).cuda()
    tokens = torch.empty((B, N, dims["dim"]), dtype=torch.float32, device="cuda")
    pool_mode = "cls" if dims["has_cls"] else "mean"
    pooled = torch.empty((B, dims["dim"]), dtype=torch.float32, device="cuda")

    head = bool(dims.get("head_classes"))
    logits = torch.empty((B, dims["head_classes"]), dtype=torch.float32, device="cuda") if head else None

    def step():
        enc.encode(fr, tokens)
        enc.pool(pool_mode, B, pooled)
        if head:
            enc.classify(B, logits)

    def timed(nsteps):
        """Wall seconds and device ms of nsteps back-to-back steps, and each
        step's device ms (events on the caller's stream, which every step
        forks from and joins back onto)."""
        torch.cuda.synchronize()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(nsteps + 1)]
        t0 = time.perf_counter()
        evs[0].record()
        for i in range(nsteps):
            step()
            evs[i + 1].record()
        torch.cuda.synchronize()
        per = [evs[i].elapsed_time(evs[i + 1]) for i in range(nsteps)]
        return time.perf_counter() - t0, evs[0].elapsed_time(evs[-1]), per

    # a short profiled pass (not timed), batch as one part, finds the dominant class
    classes = list(_lib.jepa_kernel_stats(enc.ctx).keys())
    _lib.jepa_set_batch_parts(enc.ctx, 1)
    _lib.jepa_set_profiling(enc.ctx, 0xFFFFFFFF)
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    _lib.jepa_reset_kernel_stats(enc.ctx)
    step()
    torch.cuda.synchronize()
    prof = _lib.jepa_kernel_stats(enc.ctx)
    dominant = max(prof, key=lambda k: prof[k]["total_ms"])
    if args.breakdown:
        tot = sum(v["total_ms"] for v in prof.values())
        for k, v in sorted(prof.items(), key=lambda kv: -kv[1]["total_ms"]):
            if v["launches"]:
                print(f"[bench]   {k:12s} {v['launches']:4d} launches {v['total_ms']:8.3f} ms "
                      f"({100 * v['total_ms'] / tot:5.1f} %)", file=sys.stderr)
    print(f"[bench] dominant kernel class: {dominant}", file=sys.stderr, flush=True)
    _lib.jepa_set_profiling(enc.ctx, 0)

    # timed region 1: throughput, default concurrency, no events between kernels
    _lib.jepa_set_batch_parts(enc.ctx, args.parts)
    for _ in range(args.warmup):
        step()
    wall, dev_ms, per_step = timed(args.steps)
    print(f"[bench] throughput region: {1e3 * wall / args.steps:.3f} ms per step", file=sys.stderr, flush=True)

    # timed region 2: roofline of the dominant class, batch as one part
    _lib.jepa_set_batch_parts(enc.ctx, 1)
    _lib.jepa_set_profiling(enc.ctx, 1 << classes.index(dominant))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    _lib.jepa_reset_kernel_stats(enc.ctx)
    wall1, _, _ = timed(args.steps)
    st = _lib.jepa_kernel_stats(enc.ctx)[dominant]
    _lib.jepa_set_profiling(enc.ctx, 0)
    _lib.jepa_set_batch_parts(enc.ctx, 0)
    print(f"[bench] roofline region (one part): {1e3 * wall1 / args.steps:.3f} ms per step", file=sys.stderr,
          flush=True)

    # one step captured into a HIP graph and replayed (the pages' CUDA-graph
    # replay row), and the API wall time with host frames in and the token
    # map copied back to the host (the pages' wall_ms row; never the value)
    graph_ms = None
    try:
        for _ in range(2):
            step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = 1e3 * (time.perf_counter() - t0) / args.steps
        del graph
    except Exception as e:  # capture is an extra row: report, do not fail the bench
        print(f"[bench] graph replay not measured: {e}", file=sys.stderr, flush=True)
    # the chip's dense bf16 MFMA rate as a single calibration kernel sustains
    # it (one workgroup per CU, independent MFMA chains, about 0.1 s): with
    # constant operands, and with random operands, whose toggling bits draw
    # more power and lower the clock the chip holds (the practical ceiling on
    # real data; the roofline fraction is also quoted against both)
    probe = mfma_probe(_lib)
    probe_rnd = mfma_probe(_lib, 1)
    host_tokens = torch.empty((B, N, dims["dim"]), dtype=torch.float32, pin_memory=True)
    api_steps = max(1, min(args.steps, 5))
    enc.encode(frames, tokens)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(api_steps):
        enc.encode(frames, tokens)          # host frames: staged by the library
        host_tokens.copy_(tokens)
    torch.cuda.synchronize()
    api_ms = 1e3 * (time.perf_counter() - t0) / api_steps
    print(f"[bench] graph replay: {graph_ms if graph_ms is None else round(graph_ms, 3)} ms per step, "
          f"API wall with host frames and host tokens: {api_ms:.3f} ms per step", file=sys.stderr, flush=True)

    ms_per_step = 1e3 * wall / args.steps
    tok_s = B * N * args.steps / wall
    flops = forward_flops(dims, B)
    peak = PEAK_TFLOPS[act]
    util = flops / (ms_per_step * 1e-3) / (peak * 1e12)

    avg_ms = st["total_ms"] / max(1, st["launches"])
    cf, cb = class_flops(dims, B), class_bytes(dims, B)
    if dominant in cf:
        # the int8 path's products run on the int8 MFMA (dense peak 5.0 POP/s)
        i8 = args.int8 and dims["mat_dtype"] in ("q8_0", "q4_0") and dominant.startswith("gemm_") \
            and dominant != "gemm_patch"
        kpeak, kunit = (PEAK_INT8_TOPS, "TOP/s") if i8 else (peak, "TFLOP/s")
        achieved = cf[dominant] / (avg_ms * 1e-3) / 1e12
        roof = {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 2), "peak": kpeak,
                "unit": kunit, "frac": round(achieved / kpeak, 4), "traffic": None,
                "work_per_launch": cf[dominant], "avg_launch_ms": round(avg_ms, 5),
                "launches_timed": st["launches"]}
    else:
        achieved = cb[dominant] / (avg_ms * 1e-3) / 1e9
        roof = {"kernel": dominant, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                "work_per_launch": cb[dominant], "avg_launch_ms": round(avg_ms, 5),
                "launches_timed": st["launches"]}
    parts = min(args.parts or 4, B)
    tr = measured_traffic(args.workload, dominant) if B == wl["batch"] else None
    if tr:
        roof["traffic"], roof["traffic_source"] = tr
    if roof["unit"] == "TFLOP/s" and probe and act != "f32":
        roof["frac_of_measured_mfma"] = round(roof["achieved"] / probe["tflops"], 4)
    if roof["unit"] == "TFLOP/s" and probe_rnd and act != "f32":
        roof["frac_of_measured_mfma_random_operands"] = round(roof["achieved"] / probe_rnd["tflops"], 4)
    roof["batch_parts"] = 1
    roof["region_ms_per_step"] = round(1e3 * wall1 / args.steps, 4)

    out = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": act, "data": "synthetic (seeded uint8 frames, N(0,0.02) weights)",
        "config": {"workload": args.workload, "batch": B, "tokens_per_clip": N,
                   "frames": dims["frames"], "img": [dims["img_h"], dims["img_w"]],
                   "tubelet": dims["tubelet"], "mask": dims["mask"], "weights": dims["mat_dtype"],
                   "parallelism": f"single GPU, batch in {parts} concurrent parts",
                   "int8_products": bool(args.int8)},
        "clips_per_s": round(B * args.steps / wall, 2),
        "mfma_util_pct": round(100 * util, 2),
        "forward_tflop": round(flops / 1e12, 4),
        "device_ms_per_step": round(dev_ms / args.steps, 4),
        "device_ms_per_step_min": round(min(per_step), 4),
        "device_ms_per_step_sd": round(float(np.std(per_step)), 4),
        "graph_replay_ms_per_step": None if graph_ms is None else round(graph_ms, 4),
        "api_wall_ms_per_step_host_io": round(api_ms, 4),
        "roofline": roof,
        "device": device_info(),
        "mfma_probe": probe,
        "mfma_probe_random_operands": probe_rnd,
    }
    enc.close()
    del enc, tokens, pooled, fr, host_tokens
    torch.cuda.empty_cache()
    if not args.no_other_workloads and args.workload == "levjepa_vit_l16_16f_bf16_b4" and not args.batch:
        others = {}
        for name in OTHER_WORKLOADS:
            try:
                others[name] = time_workload(name, max(3, min(args.steps, 10)), 2)
            except Exception as e:   # an extra row: report, do not fail the bench
                print(f"[bench] {name} not measured: {e}", file=sys.stderr, flush=True)
                others[name] = None
            torch.cuda.empty_cache()
        # the block-format workloads again with their products on the int8 path
        for name in INT8_WORKLOADS:
            try:
                others[name + "+int8"] = time_workload(name, max(3, min(args.steps, 10)), 2, int8=True)
            except Exception as e:
                print(f"[bench] {name} (int8) not measured: {e}", file=sys.stderr, flush=True)
                others[name + "+int8"] = None
            torch.cuda.empty_cache()
        out["other_workloads"] = others
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(dims, stored, frames, args.cpu_sample_blocks)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
