#!/usr/bin/env python3
"""Benchmark of the layer-end KV-eviction compressor on one MI355X.

A step is one layer's compression -- pass 1, pass 2, selection and gather --
over one synthetic layer. The default workload is the Llama-3.1-8B layer
geometry at a 64K prompt swept over 32 layers with an independent seed per
layer: every layer's full K/V is resident in HBM before timing starts, and
the retained caches of all layers accumulate in one arena.

Prints one JSON line: throughput in prefix tokens per second per layer (all KV
heads), the roofline of the dominant kernel, and the CPU oracle's rate on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA peak
METRIC = "prefix tokens evicted/sec per layer (all KV heads) + % HBM roofline, S=64K"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
KERNEL_SOURCES = ["score_kernels.hip", "select_kernels.hip", "gather_kernel.hip", "kvc_internal.h"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "compression_kvc_score_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(cfg, rows_total: int) -> dict:
    """Bytes each stage must move at minimum (per launch = one layer)."""
    s, w, hq, hkv, d = cfg.s, cfg.w, cfg.hq, cfg.hkv, cfg.d
    k_bytes = s * hkv * d * 2
    q_bytes = w * hq * d * 2
    mz = 2 * hq * w * 4
    scores = hkv * s * 4
    pool_extra = 2 * scores if cfg.pool > 1 else 0
    return {
        "pass1": k_bytes + q_bytes + mz,
        "pass2": k_bytes + q_bytes + mz + scores,
        "select": scores + pool_extra + rows_total * 4,
        "gather": rows_total * (4 * d * 2 + 4 + 4),
    }


def mfma_flops(cfg) -> float:
    """Q_win.K^T flops of one pass (all KV heads)."""
    return 2.0 * cfg.w * cfg.hq * cfg.s * cfg.d


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(cfg, x, budgets, n_heads: int):
    """The CPU oracle as it stands, on `n_heads` KV heads of one layer (the
    per-head work is identical, so the layer time scales by hkv / n_heads)."""
    import oracle
    G = cfg.group
    t0 = time.perf_counter()
    for g in range(n_heads):
        oracle.compress_layer(x.q[:, g * G:(g + 1) * G, :], x.k[:, g:g + 1, :], x.v[:, g:g + 1, :],
                              [int(budgets[g])], cfg.n_sink, cfg.n_recent, pool=cfg.pool)
    dt = time.perf_counter() - t0
    t_layer = dt * cfg.hkv / n_heads
    return {
        "value": cfg.s / t_layer,
        "unit": "tokens/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": (f"layer 0 of {cfg.name}, KV heads 0..{n_heads - 1} of {cfg.hkv} "
                   f"({dt:.1f} s), scaled to all heads; fp64 numpy, dense W x S softmax"),
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64, help="timed layer compressions")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="llama8b_64k")
    ap.add_argument("--layers", type=int, default=0, help="distinct resident layers (default: the workload's)")
    ap.add_argument("--cpu-heads", type=int, default=3, help="KV heads the CPU baseline runs (0: skip)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the compressor shards by KV head with no "
              "communication, so this build runs and reports a single device (--gpus 1).",
              file=sys.stderr)
        return 2

    import torch
    import compression_kvc_score_amd as kvc
    from synth import get_config, layer_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        return 1
    kvc.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    cfg = get_config(args.workload)
    n_layers = args.layers or cfg.layers
    log(f"workload {cfg.name}: S={cfg.s} W={cfg.w} Hq={cfg.hq} Hkv={cfg.hkv} D={cfg.d} "
        f"b_s={cfg.block} layers={n_layers}")

    # ---- resident inputs for every layer, one retained-cache arena
    layers = []
    x0 = None
    t_gen = time.perf_counter()
    for l in range(n_layers):
        x = layer_inputs(cfg, l)
        if l == 0:
            x0 = x
        if cfg.hetero:
            budgets = kvc.kvc_budgets_inverse_stability(x.s_stable, cfg.total_budget)
        else:
            budgets = np.full(cfg.hkv, cfg.budget, dtype=np.int32)
        q = torch.from_numpy(x.q.view(np.int16)).view(torch.bfloat16).to(dev)
        k = torch.from_numpy(x.k.view(np.int16)).view(torch.bfloat16).to(dev)
        v = torch.from_numpy(x.v.view(np.int16)).view(torch.bfloat16).to(dev)
        layers.append((q, k, v, budgets))
        if l != 0:
            del x
        if l % 4 == 3 or l == n_layers - 1:
            log(f"generated layer {l + 1}/{n_layers} ({time.perf_counter() - t_gen:.0f} s)")

    q0, k0, v0, _ = layers[0]
    desc = kvc.desc_for(q0, k0, v0, block=cfg.block, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                        pool=cfg.pool)
    ws = kvc.alloc_workspace(desc, dev)
    prepared = []
    rows_total = 0
    for (q, k, v, budgets) in layers:
        out = kvc.alloc_outputs(desc, budgets, dev)
        rows_total = max(rows_total, int(out.offsets[-1]))
        prepared.append(kvc.PreparedLayer(desc, q, k, v, budgets, out, ws))
    arena_bytes = sum(p._keep[3].k_hat.nbytes + p._keep[3].v_hat.nbytes for p in prepared)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def staged(p, ev=None):
        if ev is not None:
            ev[0].record(stream)
        p.kvc_score_pass1(sp)
        if ev is not None:
            ev[1].record(stream)
        p.kvc_score_pass2(sp)
        if ev is not None:
            ev[2].record(stream)
        p.kvc_select_topk(sp)
        if ev is not None:
            ev[3].record(stream)
        p.kvc_gather_retained(sp)
        if ev is not None:
            ev[4].record(stream)

    # ---- warmup
    for i in range(args.warmup):
        prepared[i % n_layers].kvc_compress_layer(sp)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # ---- timed region: K layer compressions through the staged entry points,
    # with HIP events on the launch stream between the kernels
    K = args.steps
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        staged(prepared[i % n_layers], events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    stage_names = ["pass1", "pass2", "select", "gather"]
    stage_ms = {n: float(np.mean([events[i][j].elapsed_time(events[i][j + 1]) for i in range(K)]))
                for j, n in enumerate(stage_names)}
    step_gpu_ms = float(np.mean([events[i][0].elapsed_time(events[i][4]) for i in range(K)]))
    log(f"timed {K} steps: {wall * 1e3 / K:.4f} ms/step wall, {step_gpu_ms:.4f} ms/step on GPU; "
        + ", ".join(f"{n} {stage_ms[n] * 1e3:.1f} us" for n in stage_names))

    # ---- the fused entry point over the same steps (reported beside)
    torch.cuda.synchronize()
    f0 = time.perf_counter()
    for i in range(K):
        prepared[i % n_layers].kvc_compress_layer(sp)
    torch.cuda.synchronize()
    fused_ms = (time.perf_counter() - f0) * 1e3 / K
    log(f"fused entry point: {fused_ms:.4f} ms/step wall")

    ms_per_step = wall * 1e3 / K
    value = cfg.s * K / wall

    # ---- roofline of the dominant kernel
    alg = algorithmic_bytes(cfg, rows_total)
    dominant = max(stage_names, key=lambda n: stage_ms[n])
    achieved = alg[dominant] / (stage_ms[dominant] * 1e-3) / 1e9
    traffic = None
    try:
        with open(TRAFFIC_FILE) as f:
            tf = json.load(f)
        if tf.get("kernel_hash") == kernel_source_hash() and tf.get("workload") == cfg.name:
            traffic = tf.get("per_launch_bytes", {}).get(dominant)
    except (OSError, ValueError):
        traffic = None
    roofline = {
        "bound": "hbm",
        "kernel": dominant,
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
    }
    total_alg = sum(alg.values())
    extras = {
        "stage_us": {n: round(stage_ms[n] * 1e3, 2) for n in stage_names},
        "step_gpu_us": round(step_gpu_ms * 1e3, 2),
        "fused_ms_per_step": round(fused_ms, 5),
        "layer_alg_bytes": total_alg,
        "layer_hbm_frac": round(total_alg / (step_gpu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "evicted_tokens_per_s": round((cfg.s - cfg.budget) * K / wall, 1),
        "pass_mfma_tflops": {n: round(mfma_flops(cfg) / (stage_ms[n] * 1e-3) / 1e12, 1)
                             for n in ("pass1", "pass2")},
        "mfma_peak_tflops": MFMA_BF16_PEAK_TFLOPS,
        "retained_arena_bytes": arena_bytes,
        "kernel_hash": kernel_source_hash(),
    }

    cpu = None
    if args.cpu_heads > 0:
        log(f"CPU oracle baseline on {args.cpu_heads} KV heads of layer 0 ...")
        cpu = cpu_baseline(cfg, x0, layers[0][3], min(args.cpu_heads, cfg.hkv))
        log(f"CPU oracle: {cpu['value']:.1f} tokens/s with {cpu['cores']} BLAS threads")

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": cfg.name, "s": cfg.s, "w": cfg.w, "hq": cfg.hq, "hkv": cfg.hkv, "d": cfg.d,
            "block": cfg.block, "budget_per_head": cfg.budget if not cfg.hetero else None,
            "total_budget": int(rows_total), "n_sink": cfg.n_sink, "n_recent": cfg.n_recent,
            "pool": cfg.pool, "layers_resident": n_layers,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "detail": extras,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
