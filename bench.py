#!/usr/bin/env python3
"""Benchmark of the layer-end KV-eviction compressor on one MI355X.

A step is one layer's compression -- pass 1, pass 2, selection and gather --
over one synthetic layer. The default workload is the Llama-3.1-8B layer
geometry at a 64K prompt swept over 32 layers with an independent seed per
layer: every layer's full K/V is resident in HBM before timing starts, and
the retained caches of all layers accumulate in one arena.

Prints one JSON line: throughput in prefix tokens per second per layer (all KV
heads) with one layer in flight (kvc_compress_layer per layer), the roofline
of the dominant kernel, and the CPU oracle's rate on a bounded sample of the
same workload. The detail also reports the same layers through the sweep entry
point kvc_compress_layers, which keeps two layers in flight.
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
KERNEL_SOURCES = ["score_kernels.hip", "stream_kernels.hip", "select_kernels.hip", "gather_kernel.hip", "kvc_internal.h",
                  "scan_select.h", "select_common.h", "wave_ops.h"]


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


def fused_scan_bytes(cfg) -> int:
    """Algorithmic bytes of both scans as one launch: K read twice, Q_win read
    once (it stays in registers), (m, Z) and the scores written once."""
    k_bytes = cfg.s * cfg.hkv * cfg.d * 2
    return 2 * k_bytes + cfg.w * cfg.hq * cfg.d * 2 + 2 * cfg.hq * cfg.w * 4 + cfg.hkv * cfg.s * 4


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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


def cpu_baseline(cfg, host_layers, budgets_of, seconds: float):
    """The CPU oracle as it stands, one KV head at a time over the resident
    layers in order, until about `seconds` of work (every head of a layer is
    the same amount of work, so the rate scales to whole layers)."""
    import oracle
    G = cfg.group
    heads = 0
    t0 = time.perf_counter()
    for li, x in enumerate(host_layers):
        b = budgets_of[li]
        for g in range(cfg.hkv):
            oracle.compress_layer(x.q[:, g * G:(g + 1) * G, :], x.k[:, g:g + 1, :], x.v[:, g:g + 1, :],
                                  [int(b[g])], cfg.n_sink, cfg.n_recent, pool=cfg.pool)
            heads += 1
            if time.perf_counter() - t0 >= seconds:
                break
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    layers_done = heads / cfg.hkv
    return {
        "value": cfg.s * layers_done / dt,
        "unit": "tokens/s",
        "cores": blas_threads(),
        "cpu_model": host_cpu_model(),
        "kind": "oracle",
        "sample": (f"{heads} KV-head compressions ({layers_done:.2f} layers of {cfg.name}, "
                   f"{dt:.1f} s); fp64 numpy oracle, dense W x S softmax per head"),
    }


def cpu_baseline_one_thread(cfg, host_layers, budgets_of, seconds: float):
    """The same oracle sample with the BLAS pool limited to one thread."""
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"):
        r = cpu_baseline(cfg, host_layers, budgets_of, seconds)
    r["cores"] = 1
    return r


def achievable_hbm_gbs(torch, dev) -> float:
    """Read + write bandwidth of a 1 GiB device-to-device copy (the achievable
    streaming rate on this machine, beside the 8 TB/s spec peak)."""
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return gbs


def copy_probe():
    """A device-to-device copy of exactly 256 MiB, five times: the reference a
    profiler's fetch/write byte counters are scaled against."""
    import torch
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 5}))
    return 0


def immediate_eviction(kvc, torch, dev, name, reps, sp, stream):
    """Time one layer's immediate eviction (kvc_compress_chunked: every chunk
    boundary of the prompt) and the layer-end compressor (kvc_compress_layer)
    on the same tensors and budget; HIP events around `reps` back-to-back
    calls of each. Also the per-head overlap of the two retained sets."""
    from synth import chunk_windows, get_config, layer_inputs
    cfg = get_config(name)
    x = layer_inputs(cfg, 0)
    qw = chunk_windows(cfg, cfg.chunk, 0, q_last=x.q)

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v, qwd = dev_bf16(x.q), dev_bf16(x.k), dev_bf16(x.v), dev_bf16(qw)
    del x
    desc = kvc.desc_for(q, k, v, block=cfg.block, n_sink=cfg.n_sink, n_recent=cfg.n_recent, pool=cfg.pool)
    rows = min(cfg.budget, cfg.s)
    k_out = torch.empty((cfg.hkv, rows, cfg.d), dtype=torch.bfloat16, device=dev)
    v_out = torch.empty_like(k_out)
    pos = torch.empty((cfg.hkv, rows), dtype=torch.int32, device=dev)
    ws = torch.empty(kvc.kvc_chunked_workspace_size(desc, cfg.chunk, cfg.budget), dtype=torch.uint8, device=dev)
    imm = kvc.PreparedChunked(desc, cfg.chunk, qwd, k, v, cfg.budget, k_out, v_out, pos, ws)
    budgets = np.full(cfg.hkv, cfg.budget, dtype=np.int32)
    lws = kvc.alloc_workspace(desc, dev)
    lout = kvc.alloc_outputs(desc, budgets, dev, with_intermediates=False)
    delayed = kvc.PreparedLayer(desc, q, k, v, budgets, lout, lws)

    def timed(call):
        for _ in range(2):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps, (time.perf_counter() - t0) * 1e6 / reps

    imm_us, imm_wall = timed(lambda: imm.kvc_compress_chunked(sp))
    del_us, _ = timed(lambda: delayed.kvc_compress_layer(sp))
    # the same boundaries with the fused-selection flag: each evicting
    # boundary is one launch (scans, selection and gather)
    fdesc = kvc.desc_for(q, k, v, block=cfg.block, n_sink=cfg.n_sink, n_recent=cfg.n_recent, pool=cfg.pool,
                         flags=kvc.KVC_FLAG_FUSED_SELECT)
    try:
        fws = torch.empty(kvc.kvc_chunked_workspace_size(fdesc, cfg.chunk, cfg.budget), dtype=torch.uint8, device=dev)
        fimm = kvc.PreparedChunked(fdesc, cfg.chunk, qwd, k, v, cfg.budget, torch.empty_like(k_out),
                                   torch.empty_like(v_out), torch.empty_like(pos), fws)
        fsel_us, _ = timed(lambda: fimm.kvc_compress_chunked(sp))
    except kvc.KvcError as e:
        log(f"immediate eviction {name} with the fused-selection flag: {e}")
        fsel_us = None
    ov = torch.empty(cfg.hkv, dtype=torch.float32, device=dev)
    kvc.kvc_overlap_coefficient(desc, pos.view(-1), lout.idx, budgets, ov)
    torch.cuda.synchronize()
    n_chunks = (cfg.s + cfg.chunk - 1) // cfg.chunk
    # algorithmic bytes of all boundaries: the chunk appended (K, V read and
    # written), the accumulated K read by both scans, the scores written and
    # read once, and the retained K, V rows read and written by the gather
    row = cfg.hkv * cfg.d * 2
    alg, kept = 0, 0
    for b in range(n_chunks):
        c = min(cfg.chunk, cfg.s - b * cfg.chunk)
        s_acc = kept + c
        alg += 4 * c * row
        if s_acc > cfg.budget or b == n_chunks - 1:
            r = min(cfg.budget, s_acc)
            alg += 2 * s_acc * row + 2 * cfg.hkv * s_acc * 4 + 4 * r * row
        kept = min(s_acc, cfg.budget)
    out = {"s": cfg.s, "chunk": cfg.chunk, "budget_per_head": cfg.budget, "boundaries": n_chunks,
           "immediate_us_per_layer": round(imm_us, 2), "immediate_wall_us_per_layer": round(imm_wall, 2),
           "us_per_boundary": round(imm_us / n_chunks, 2), "layer_end_us_per_layer": round(del_us, 2),
           "immediate_over_layer_end": round(imm_us / del_us, 3),
           "retained_overlap_mean": round(float(ov.mean().item()), 4),
           "alg_bytes_per_layer": alg, "hbm_frac": round(alg / (imm_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "fused_select_us_per_layer": round(fsel_us, 2) if fsel_us else None,
           "fused_select_us_per_boundary": round(fsel_us / n_chunks, 2) if fsel_us else None,
           "entry_points": ["kvc_compress_chunked", "kvc_compress_layer"]}
    log(f"immediate eviction {name}: {imm_us:.1f} us/layer over {n_chunks} boundaries "
        f"({imm_us / n_chunks:.2f} us each; wall {imm_wall:.1f} us) vs layer-end {del_us:.1f} us "
        f"({imm_us / del_us:.2f}x); retained-set overlap {out['retained_overlap_mean']:.3f}; with the "
        f"fused-selection flag " + (f"{fsel_us:.1f} us/layer ({fsel_us / n_chunks:.2f} us each)" if fsel_us else "n/a"))
    return out


OTHER_CONFIGS = ["llama8b_16k", "llama8b_128k", "llama8b_128k_pool7"]
SWEEP_CONFIG = "qwen14b_hetero_64k"


def _pct(us):
    us = np.asarray(us, dtype=np.float64)
    return {"median": round(float(np.median(us)), 2), "p10": round(float(np.percentile(us, 10)), 2),
            "p90": round(float(np.percentile(us, 90)), 2)}


def other_configs(kvc, torch, dev, names, reps, sp, stream):
    """kvc_compress_layer on the other single-layer shapes: two resident layers
    of each, two warm calls, then `reps` calls alternating between them, each
    after a 512 MiB read that evicts the memory-side cache, with HIP events
    around each call. Reports median / p10 / p90 per layer, throughput and the
    HBM fraction over the layer's algorithmic bytes (at the median)."""
    from synth import get_config, layer_inputs

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    out = {}
    for name in names:
        cfg = get_config(name)
        preps = []
        rows = 0
        for l in range(2):
            x = layer_inputs(cfg, l)
            budgets = (kvc.kvc_budgets_inverse_stability(x.s_stable, cfg.total_budget) if cfg.hetero
                       else np.full(cfg.hkv, cfg.budget, dtype=np.int32))
            q, k, v = dev_bf16(x.q), dev_bf16(x.k), dev_bf16(x.v)
            del x
            desc = kvc.desc_for(q, k, v, block=cfg.block, n_sink=cfg.n_sink, n_recent=cfg.n_recent, pool=cfg.pool)
            o = kvc.alloc_outputs(desc, budgets, dev, with_intermediates=False)
            rows = max(rows, int(o.offsets[-1]))
            preps.append(kvc.PreparedLayer(desc, q, k, v, budgets, o, kvc.alloc_workspace(desc, dev)))
        for p in preps:
            p.kvc_compress_layer(sp)
        evs = []
        for i in range(reps):
            flush.amax()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            preps[i % 2].kvc_compress_layer(sp)
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        us = [a.elapsed_time(b) * 1e3 for a, b in evs]
        med = float(np.median(us))
        alg = sum(algorithmic_bytes(cfg, rows).values())
        out[name] = {"s": cfg.s, "w": cfg.w, "hq": cfg.hq, "hkv": cfg.hkv, "pool": cfg.pool,
                     "us_per_layer": _pct(us), "reps": reps, "flushed": True,
                     "tokens_per_s": round(cfg.s / (med * 1e-6), 1), "alg_bytes": alg,
                     "hbm_frac": round(alg / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "scans": _scan_label(kvc, preps[0].desc)}
        log(f"{name}: median {med:.1f} us per layer (p10 {out[name]['us_per_layer']['p10']:.1f}, "
            f"p90 {out[name]['us_per_layer']['p90']:.1f}; {reps} calls after a cache flush), "
            f"{out[name]['hbm_frac'] * 100:.1f}% of the HBM peak, {out[name]['scans']} scans")
        del preps
        torch.cuda.empty_cache()
    del flush
    return out


def _scan_label(kvc, desc):
    """How the library runs a layer's scans, from its plan."""
    plan = kvc.kvc_plan_layer(desc)
    if plan.scan != kvc.KVC_SCAN_STREAM:
        return "per-head (K in VGPRs)"
    return "streaming (K staged in LDS)" + (", fused into one launch" if plan.fused_scans else "")


def layer_sweep(kvc, torch, dev, name, sp, stream):
    """A model's layers in order, each resident with its own seed (and, for
    heterogeneous budgets, its own S_stable draw), one kvc_compress_layer call
    per layer into one retained-cache arena, HIP events around each call."""
    from synth import get_config, layer_inputs

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    cfg = get_config(name)
    t0 = time.perf_counter()
    preps, rows = [], []
    ws = None
    for l in range(cfg.layers):
        x = layer_inputs(cfg, l)
        budgets = (kvc.kvc_budgets_inverse_stability(x.s_stable, cfg.total_budget) if cfg.hetero
                   else np.full(cfg.hkv, cfg.budget, dtype=np.int32))
        q, k, v = dev_bf16(x.q), dev_bf16(x.k), dev_bf16(x.v)
        del x
        desc = kvc.desc_for(q, k, v, block=cfg.block, n_sink=cfg.n_sink, n_recent=cfg.n_recent, pool=cfg.pool)
        if ws is None:
            ws = kvc.alloc_workspace(desc, dev)
        o = kvc.alloc_outputs(desc, budgets, dev, with_intermediates=False)
        rows.append(int(o.offsets[-1]))
        preps.append(kvc.PreparedLayer(desc, q, k, v, budgets, o, ws))
    log(f"{name}: generated {cfg.layers} layers ({time.perf_counter() - t0:.0f} s)")
    arena = sum(p._keep[3].k_hat.nbytes + p._keep[3].v_hat.nbytes for p in preps)

    def sweep(ps):
        ps[-1].kvc_compress_layer(sp)  # warm (the last layer; the sweep starts at the first)
        torch.cuda.synchronize()
        evs = []
        for p in ps:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            p.kvc_compress_layer(sp)
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 for a, b in evs]

    us = sweep(preps)
    med = float(np.median(us))
    # the same layers with the fused-selection flag (scans, selection and
    # gather as one launch), into the same retained-cache arena
    fsel = None
    try:
        fpreps, fws = [], None
        for p in preps:
            q, k, v, o, _ = p._keep
            fdesc = kvc.desc_for(q, k, v, block=cfg.block, n_sink=cfg.n_sink, n_recent=cfg.n_recent, pool=cfg.pool,
                                 flags=kvc.KVC_FLAG_FUSED_SELECT)
            if fws is None:
                fws = kvc.alloc_workspace(fdesc, dev)
            fpreps.append(kvc.PreparedLayer(fdesc, q, k, v, p._b, o, fws))
        fsel = _pct(sweep(fpreps))
        del fpreps, fws
    except kvc.KvcError as e:
        log(f"{name} sweep with the fused-selection flag: {e}")
    alg = sum(algorithmic_bytes(cfg, max(rows)).values())
    out = {"s": cfg.s, "w": cfg.w, "hq": cfg.hq, "hkv": cfg.hkv, "layers": cfg.layers,
           "budgets": "inverse stability, total %d per layer" % cfg.total_budget if cfg.hetero else cfg.budget,
           "retained_arena_bytes": arena, "us_per_layer": _pct(us),
           "tokens_per_s": round(cfg.s / (med * 1e-6), 1), "alg_bytes": alg,
           "hbm_frac": round(alg / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "scans": _scan_label(kvc, preps[0].desc), "fused_select_us_per_layer": fsel}
    log(f"{name} sweep over {cfg.layers} layers: median {med:.1f} us per layer (p10 {out['us_per_layer']['p10']:.1f}, "
        f"p90 {out['us_per_layer']['p90']:.1f}), retained arena {arena / 2**20:.0f} MiB, "
        f"{out['hbm_frac'] * 100:.1f}% of the HBM peak; with the fused-selection flag "
        + (f"median {fsel['median']:.1f} us" if fsel else "n/a"))
    del preps, ws
    torch.cuda.empty_cache()
    return out


def fused_select_detail(kvc, torch, dev, sp, stream, reps=6, calls=32):
    """KVC_FLAG_FUSED_SELECT (scans, selection and gather in one launch, the
    scores kept on chip, a workspace that does not grow with S) against the
    default whole-layer call on the same resident layers: four layers per
    shape, `reps` interleaved rounds of `calls` calls each way, HIP events
    around each round; medians."""
    from synth import get_config, layer_inputs

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    out = {}
    for name, over in (("llama8b_16k", {}), ("llama8b_64k", {}), ("llama8b_64k", {"s": 131072})):
        cfg = get_config(name).with_(**over) if over else get_config(name)
        layers = []
        for l in range(4):
            x = layer_inputs(cfg, l)
            layers.append((dev_bf16(x.q), dev_bf16(x.k), dev_bf16(x.v), np.full(cfg.hkv, cfg.budget, dtype=np.int32)))
            del x
        runs = {}
        for flag in (0, kvc.KVC_FLAG_FUSED_SELECT):
            q0, k0, v0, _ = layers[0]
            desc = kvc.desc_for(q0, k0, v0, block=cfg.block, n_sink=cfg.n_sink, n_recent=cfg.n_recent, flags=flag)
            ws = kvc.alloc_workspace(desc, dev)
            runs[flag] = ([kvc.PreparedLayer(desc, q, k, v, b, kvc.alloc_outputs(desc, b, dev, with_intermediates=False), ws)
                           for q, k, v, b in layers], [], int(ws.numel()))
        for r in range(reps):
            for flag in ((0, kvc.KVC_FLAG_FUSED_SELECT) if r % 2 == 0 else (kvc.KVC_FLAG_FUSED_SELECT, 0)):
                preps, ts, _ = runs[flag]
                for i in range(4):
                    preps[i].kvc_compress_layer(sp)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in range(calls):
                    preps[i % 4].kvc_compress_layer(sp)
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3 / calls)
        key = f"{name}_s{cfg.s}"
        out[key] = {"s": cfg.s, "w": cfg.w, "default_us": round(float(np.median(runs[0][1])), 2),
                    "fused_select_us": round(float(np.median(runs[kvc.KVC_FLAG_FUSED_SELECT][1])), 2),
                    "default_workspace_bytes": runs[0][2],
                    "fused_select_workspace_bytes": runs[kvc.KVC_FLAG_FUSED_SELECT][2]}
        log(f"fused select {key}: {out[key]['fused_select_us']:.1f} us per layer (workspace "
            f"{out[key]['fused_select_workspace_bytes']} B) against {out[key]['default_us']:.1f} us "
            f"(workspace {out[key]['default_workspace_bytes']} B)")
        del runs, layers
        torch.cuda.empty_cache()
    return out


def layer_major_prefill(kvc, torch, dev, s=65536, chunk=2048, w=32, budget=4096):
    """The compressor inside the schedule it serves: a random-weight
    Llama-3.1-8B-shaped stack (32 layers) prefilled layer-major in chunks with
    layer-end eviction, against the same prefill without compression and
    against keeping every layer's full K/V until the end (then compressing).
    One warm and one timed run of each; HIP events around the timed run."""
    from compression_kvc_score_amd import prefill as pf
    cfg = pf.ModelConfig()
    model = pf.SyntheticModel(cfg, device=dev, seed=1)
    gen = torch.Generator(device=dev)
    gen.manual_seed(2)
    x0 = torch.randn((s, cfg.hidden), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    budgets = [budget] * cfg.hkv
    out = {"s": s, "chunk": chunk, "w": w, "budget_per_head": budget, "layers": cfg.layers,
           "model": "Llama-3.1-8B geometry, random bf16 weights", "weights_bytes": model.nbytes()}
    for name, kw in [("layer_major_evict", dict(overlap=True)),
                     ("layer_major_no_compression", dict(compress=False)),
                     ("full_kv_then_compress", dict(keep_full_kv=True))]:
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        drv = pf.LayerMajorPrefill(model, s, chunk, w, budgets, 4, 32, device=dev, **kw)
        x = x0.clone()
        drv.run(x)
        x.copy_(x0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        drv.run(x)
        e1.record()
        torch.cuda.synchronize()
        rep = drv.acct.report()
        out[name] = {"ttft_ms": round(e0.elapsed_time(e1), 2),
                     "layer_ms": round(float(np.mean([a.elapsed_time(b) for a, b, _ in drv.layer_events])), 3),
                     "allocator_peak_bytes": int(rep["allocator_peak_bytes"]),
                     "resident_at_peak": {k: int(v) for k, v in rep["peak_parts"].items() if k != "weights"}}
        log(f"layer-major prefill {name}: {out[name]['ttft_ms']:.1f} ms for {cfg.layers} layers of {s} tokens "
            f"({out[name]['layer_ms']:.2f} ms per layer); allocator peak beyond the weights and prompt "
            f"{rep['allocator_peak_bytes'] / 2**30:.3f} GiB")
        if name == "layer_major_evict":
            out["final_cache_bytes"] = int(drv.cache.k.numel() * 2 + drv.cache.v.numel() * 2)
        del drv, x
    # the chunk attention kernel alone against the bf16 MFMA peak: the last
    # 2048-token chunk of the prompt over the whole layer's K/V (random rows)
    pdesc = kvc.PrefillDesc(s=s, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, rope_base=cfg.rope_base, scale=0.0)
    kc = torch.randn((s, cfg.hkv, cfg.d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    vc = torch.randn((s, cfg.hkv, cfg.d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    q = torch.randn((chunk, cfg.hq, cfg.d), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
    o = torch.empty_like(q)
    c0 = s - chunk
    kvc.kvc_chunk_attention(pdesc, q, kc, vc, c0, o)
    torch.cuda.synchronize()
    reps = 10
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        kvc.kvc_chunk_attention(pdesc, q, kc, vc, c0, o)
    e1.record()
    torch.cuda.synchronize()
    att_ms = e0.elapsed_time(e1) / reps
    keys = sum(c0 + t + 1 for t in range(chunk))      # causal (query, key) pairs per head
    flops = 4.0 * cfg.hq * cfg.d * keys                # QK^T and PV
    out["chunk_attention"] = {"c0": c0, "n": chunk, "us": round(att_ms * 1e3, 1), "tflops": round(flops / att_ms / 1e9, 1),
                              "mfma_frac": round(flops / att_ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4)}
    log(f"chunk attention (last {chunk} queries over {s} keys): {att_ms * 1e3:.0f} us, "
        f"{flops / att_ms / 1e9:.0f} TFLOP/s ({out['chunk_attention']['mfma_frac'] * 100:.1f}% of the bf16 MFMA peak)")
    del kc, vc, q, o
    ev, base = out["layer_major_evict"]["ttft_ms"], out["layer_major_no_compression"]["ttft_ms"]
    out["compression_overhead_frac"] = round((ev - base) / base, 5)
    out["transient_reduction_frac"] = round(
        1 - out["layer_major_evict"]["allocator_peak_bytes"] / out["full_kv_then_compress"]["allocator_peak_bytes"], 4)
    del model, x0
    torch.cuda.empty_cache()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64, help="timed layer compressions")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="llama8b_64k")
    ap.add_argument("--layers", type=int, default=0, help="distinct resident layers (default: the workload's)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="CPU-oracle baseline sample length in seconds (0: skip)")
    ap.add_argument("--no-prefill", dest="prefill", action="store_false",
                    help="skip the layer-major prefill run (random-weight model around the compressor)")
    ap.add_argument("--no-configs", dest="configs", action="store_false",
                    help="skip timing the other layer shapes (16K, 128K, 128K with pool 7, Qwen-shaped)")
    ap.add_argument("--roofline-only", action="store_true",
                    help="only the roofline loop (back-to-back kvc_score_layer calls over the resident "
                         "layers), for profiling the dominant kernel")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 256 MiB device copy (to calibrate HBM byte counters)")
    args = ap.parse_args(argv)
    if args.copy_probe:
        return copy_probe()

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
    host_layers = []  # kept on the host for the CPU baseline
    t_gen = time.perf_counter()
    for l in range(n_layers):
        x = layer_inputs(cfg, l)
        if args.cpu_seconds > 0 and l < 16:
            host_layers.append(x)
        if cfg.hetero:
            budgets = kvc.kvc_budgets_inverse_stability(x.s_stable, cfg.total_budget)
        else:
            budgets = np.full(cfg.hkv, cfg.budget, dtype=np.int32)
        q = torch.from_numpy(x.q.view(np.int16)).view(torch.bfloat16).to(dev)
        k = torch.from_numpy(x.k.view(np.int16)).view(torch.bfloat16).to(dev)
        v = torch.from_numpy(x.v.view(np.int16)).view(torch.bfloat16).to(dev)
        layers.append((q, k, v, budgets))
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

    plan = kvc.kvc_plan_layer(desc)

    def roofline_loop(K, W):
        """The dominant kernel alone: K back-to-back kvc_score_layer calls over
        the resident layers after W warm ones, HIP events on the launch stream
        around the K calls. With fused scans each call is one launch."""
        for i in range(W):
            prepared[i % n_layers].kvc_score_layer(sp)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(K):
            prepared[i % n_layers].kvc_score_layer(sp)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    def roofline_object(scan_ms):
        if plan.fused_scans:
            kernel = ("scan_fused_kernel: pass 1, split merge and pass 2 as one launch "
                      "(one kvc_score_layer call)")
            alg_b = fused_scan_bytes(cfg)
        else:
            kernel = "pass 1, split combine and pass 2 (three launches of one kvc_score_layer call)"
            a = algorithmic_bytes(cfg, 0)
            alg_b = a["pass1"] + a["pass2"]
        achieved = alg_b / (scan_ms * 1e-3) / 1e9
        traffic = None
        try:
            with open(TRAFFIC_FILE) as f:
                tf = json.load(f)
            if tf.get("kernel_hash") == kernel_source_hash() and tf.get("workload") == cfg.name:
                traffic = tf.get("per_launch_bytes", {}).get("scan")
        except (OSError, ValueError):
            traffic = None
        return {"bound": "hbm", "kernel": kernel, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "alg_bytes_per_launch": alg_b, "us_per_launch": round(scan_ms * 1e3, 2),
                "launches_timed": args.steps,
                "mfma_tflops": round(2 * mfma_flops(cfg) / (scan_ms * 1e-3) / 1e12, 1),
                "mfma_frac": round(2 * mfma_flops(cfg) / (scan_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}

    if args.roofline_only:
        # at least ~14 ms of warm calls, so that the device has left its idle
        # clocks before the timed calls (the full run's loop follows the
        # whole-layer calls)
        scan_ms = roofline_loop(args.steps, max(args.warmup, 200))
        roof = roofline_object(scan_ms)
        log(f"roofline loop: {scan_ms * 1e3:.2f} us per kvc_score_layer call, {roof['frac'] * 100:.1f}% of the HBM peak")
        print(json.dumps({"metric": METRIC, "mode": "roofline-only", "steps": args.steps, "warmup": max(args.warmup, 200),
                          "config": {"workload": cfg.name, "s": cfg.s, "fused_scans": int(plan.fused_scans)},
                          "roofline": roof, "kernel_hash": kernel_source_hash()}), flush=True)
        return 0

    stage_calls = {
        "pass1": lambda p: p.kvc_score_pass1(sp),
        "pass2": lambda p: p.kvc_score_pass2(sp),
        "select": lambda p: p.kvc_select_topk(sp),
        "gather": lambda p: p.kvc_gather_retained(sp),
    }

    # ---- warmup
    for i in range(args.warmup):
        prepared[i % n_layers].kvc_compress_layer(sp)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # ---- timed region: K layer compressions through the whole-layer entry
    # point, one layer after another (HIP events bracket the region)
    K = args.steps
    ev_start, ev_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev_start.record(stream)
    for i in range(K):
        prepared[i % n_layers].kvc_compress_layer(sp)
    ev_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_gpu_ms = ev_start.elapsed_time(ev_end) / K
    log(f"timed {K} steps: {wall * 1e3 / K:.4f} ms/step wall, {step_gpu_ms:.4f} ms/step on GPU")

    # ---- the dominant kernel alone, for the roofline
    scan_ms = roofline_loop(K, args.warmup)
    log(f"roofline loop: {scan_ms * 1e3:.2f} us per kvc_score_layer call (fused scans: {bool(plan.fused_scans)})")

    # ---- the same calls replayed from a HIP graph: one captured
    # kvc_compress_layer per resident layer (the library enqueues only
    # kernels, so the calls capture as they are), replayed until K layers
    # have run; HIP events around the replays
    graph_ms = None
    try:
        side = torch.cuda.Stream()
        with torch.cuda.stream(side):
            for p in prepared:
                p.kvc_compress_layer()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for p in prepared:
                p.kvc_compress_layer()
        reps = max(1, K // n_layers)
        graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(reps):
            graph.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        graph_ms = g0.elapsed_time(g1) / (reps * n_layers)
        log(f"graph replay of {n_layers} captured layers x {reps}: {graph_ms:.4f} ms/layer on GPU")
        del graph
    except RuntimeError as e:  # capture unavailable: report it, keep the rest
        log(f"graph capture failed: {e}")

    # ---- the same K layer compressions as one layer-major sweep call, which
    # keeps two layers in flight (one layer's selection overlaps the next
    # one's scans); step i compresses resident layer i % n_layers into its
    # own buffers (one set per stream parity, so that no two streams share an
    # output)
    sweep_outs = {}
    for i in range(K):
        key = (i % n_layers, i % kvc.SWEEP_STREAMS)
        if key not in sweep_outs:
            sweep_outs[key] = kvc.alloc_outputs(desc, layers[key[0]][3], dev, with_intermediates=False)
    sweep_ws = kvc.alloc_sweep_workspace(desc, dev)
    sweep = kvc.PreparedSweep(desc, [layers[i % n_layers][:3] for i in range(K)],
                              np.stack([layers[i % n_layers][3] for i in range(K)]),
                              [sweep_outs[(i % n_layers, i % kvc.SWEEP_STREAMS)] for i in range(K)], sweep_ws)
    aux = torch.cuda.Stream()  # the sweep's second lane (default priority)
    sweep.kvc_compress_layers(sp, aux)  # warm
    torch.cuda.synchronize()
    sw_start, sw_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    sw_start.record(stream)
    sweep.kvc_compress_layers(sp, aux)
    sw_end.record(stream)
    torch.cuda.synchronize()
    sweep_wall = time.perf_counter() - t0
    sweep_gpu_ms = sw_start.elapsed_time(sw_end) / K
    log(f"sweep of {K} layers (2 in flight): {sweep_wall * 1e3 / K:.4f} ms/layer wall, "
        f"{sweep_gpu_ms:.4f} ms/layer on GPU")

    # ---- cold layers: before each layer a read of 512 MiB evicts the
    # memory-side cache (256 MB) with clean lines (a write would leave dirty
    # lines that the next kernel pays to write back), then HIP events bracket
    # one kvc_compress_layer call; median and p10 / p90 over the resident layers
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    cold_ev = []
    for i in range(n_layers):
        flush.amax()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        prepared[i].kvc_compress_layer(sp)
        e1.record(stream)
        cold_ev.append((e0, e1))
    torch.cuda.synchronize()
    cold_us = np.array([a.elapsed_time(b) * 1e3 for a, b in cold_ev])
    del flush
    log(f"cold layers (cache flushed before each): median {np.median(cold_us):.1f} us, "
        f"p10 {np.percentile(cold_us, 10):.1f}, p90 {np.percentile(cold_us, 90):.1f} over {n_layers}")

    # ---- per-stage breakdown: each staged entry point called K times back to
    # back over the same layers (same kernels and launch configuration as the
    # whole-layer call; every stage reads what the timed region wrote), HIP
    # events on the launch stream around each batch
    stage_ms = {}
    for name, call in stage_calls.items():
        call(prepared[0])  # warm
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(K):
            call(prepared[i % n_layers])
        e1.record(stream)
        torch.cuda.synchronize()
        stage_ms[name] = e0.elapsed_time(e1) / K
    stage_names = list(stage_calls)
    staged_ms = sum(stage_ms.values())
    log("staged breakdown (back-to-back batches): " + ", ".join(f"{n} {stage_ms[n] * 1e3:.1f} us" for n in stage_names)
        + f" (sum {staged_ms * 1e3:.1f} us)")

    # ---- the two scans in the order the layer runs them: per layer pass 1,
    # pass 2, select, gather, with HIP events between the calls, so each scan
    # sees the cache state it has inside a layer (pass 2 right after pass 1
    # read the same K); the event span also holds the scan's dispatch gap
    ctx_ev = {"pass1": [], "pass2": []}
    for i in range(K + 1):
        p = prepared[i % n_layers]
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        marks[0].record(stream)
        p.kvc_score_pass1(sp)
        marks[1].record(stream)
        p.kvc_score_pass2(sp)
        marks[2].record(stream)
        p.kvc_select_topk(sp)
        p.kvc_gather_retained(sp)
        if i > 0:  # the first layer is a warm-up
            ctx_ev["pass1"].append((marks[0], marks[1]))
            ctx_ev["pass2"].append((marks[1], marks[2]))
    torch.cuda.synchronize()
    ctx_ms = {n: float(np.mean([a.elapsed_time(b) for a, b in evs])) for n, evs in ctx_ev.items()}
    log(f"scans in layer order (events between calls): pass1 {ctx_ms['pass1'] * 1e3:.1f} us, "
        f"pass2 {ctx_ms['pass2'] * 1e3:.1f} us")

    # ---- the raw inner-product score modes on the same layers: the warm
    # whole-layer loop, their one-pass scan (K back-to-back kvc_score_pass2
    # calls) against the HBM peak, and how much their retained sets overlap
    # the softmax ones (per-head overlap coefficient, layer 0)
    mode_detail = {}
    for mode_name, mode in (("logit", kvc.KVC_SCORE_LOGIT), ("int8", kvc.KVC_SCORE_LOGIT_INT8)):
        mdesc = kvc.desc_for(q0, k0, v0, block=cfg.block, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                             pool=cfg.pool, score_mode=mode)
        mprep = [kvc.PreparedLayer(mdesc, q, k, v, budgets, kvc.alloc_outputs(mdesc, budgets, dev), ws)
                 for (q, k, v, budgets) in layers]
        for i in range(args.warmup):
            mprep[i % n_layers].kvc_compress_layer(sp)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            mprep[i % n_layers].kvc_compress_layer(sp)
        torch.cuda.synchronize()
        mwall = time.perf_counter() - t0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(K):
            mprep[i % n_layers].kvc_score_pass2(sp)
        e1.record(stream)
        torch.cuda.synchronize()
        mscan_ms = e0.elapsed_time(e1) / K
        scan_bytes = cfg.s * cfg.hkv * cfg.d * 2 + cfg.w * cfg.hq * cfg.d * 2 + cfg.hkv * cfg.s * 4
        res = torch.empty(cfg.hkv, dtype=torch.float32, device=dev)
        kvc.kvc_overlap_coefficient(desc, prepared[0]._keep[3].idx, mprep[0]._keep[3].idx, layers[0][3], res)
        torch.cuda.synchronize()
        mode_detail[mode_name] = {
            "ms_per_step": round(mwall * 1e3 / K, 5), "value": round(cfg.s * K / mwall, 1),
            "scan_us": round(mscan_ms * 1e3, 2),
            "scan_hbm_frac": round(scan_bytes / (mscan_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "overlap_with_softmax_mean": round(float(res.mean().item()), 4),
        }
        log(f"score mode {mode_name}: {mwall * 1e3 / K:.4f} ms/layer; scan {mscan_ms * 1e3:.1f} us "
            f"({mode_detail[mode_name]['scan_hbm_frac'] * 100:.1f}% of HBM peak); retained-set overlap with "
            f"softmax {mode_detail[mode_name]['overlap_with_softmax_mean']:.3f}")
        del mprep

    # ---- immediate (chunk-boundary) eviction, the schedule layer-end eviction
    # is compared with: the Table-8 setting (16K prompt, 512-token chunks,
    # 1024 keys per head) and the 64K layer with 2048-token chunks and 4096
    # keys, each against the one-shot layer-end compressor on the same tensors
    imm_detail = {name: immediate_eviction(kvc, torch, dev, name, max(4, K // 4), sp, stream)
                  for name in ("llama8b_16k_imm", "llama8b_64k_imm")}
    fsel_detail = fused_select_detail(kvc, torch, dev, sp, stream) if args.configs else None
    configs_detail = other_configs(kvc, torch, dev, OTHER_CONFIGS, 20, sp, stream) if args.configs else None
    if args.configs:
        configs_detail[SWEEP_CONFIG] = layer_sweep(kvc, torch, dev, SWEEP_CONFIG, sp, stream)
    prefill_detail = layer_major_prefill(kvc, torch, dev, s=cfg.s) if args.prefill else None

    copy_gbs = achievable_hbm_gbs(torch, dev)
    log(f"device copy of 1 GiB: {copy_gbs:.0f} GB/s read + write")

    ms_per_step = wall * 1e3 / K
    value = cfg.s * K / wall

    alg = algorithmic_bytes(cfg, rows_total)
    roofline = roofline_object(scan_ms)
    achieved = roofline["achieved"]
    total_alg = sum(alg.values())
    extras = {
        "stage_us": {n: round(stage_ms[n] * 1e3, 2) for n in stage_names},
        "scan_us_in_layer_order": {n: round(ctx_ms[n] * 1e3, 2) for n in ctx_ms},
        "step_gpu_us": round(step_gpu_ms * 1e3, 2),
        "staged_step_us": round(staged_ms * 1e3, 2),
        "layer_alg_bytes": total_alg,
        "layer_hbm_frac": round(total_alg / (step_gpu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "hbm_copy_gbs": round(copy_gbs, 1),
        "layer_frac_of_copy_rate": round(total_alg / (step_gpu_ms * 1e-3) / 1e9 / copy_gbs, 4),
        "roofline_kernel_frac_of_copy_rate": round(achieved / copy_gbs, 4),
        "evicted_tokens_per_s": round((cfg.s - cfg.budget) * K / wall, 1),
        "pass_mfma_tflops": {n: round(mfma_flops(cfg) / (stage_ms[n] * 1e-3) / 1e12, 1)
                             for n in ("pass1", "pass2")},
        "mfma_peak_tflops": MFMA_BF16_PEAK_TFLOPS,
        "retained_arena_bytes": arena_bytes,
        "cold_layer_us": {"median": round(float(np.median(cold_us)), 2),
                          "p10": round(float(np.percentile(cold_us, 10)), 2),
                          "p90": round(float(np.percentile(cold_us, 90)), 2), "layers": n_layers,
                          "note": "a 512 MiB read before each layer evicts the memory-side cache; "
                                  "HIP events around one kvc_compress_layer call"},
        "score_modes": mode_detail,
        "other_configs": configs_detail,
        "immediate_eviction": imm_detail,
        "fused_select": fsel_detail,
        "layer_major_prefill": prefill_detail,
        "sweep": {
            "entry_point": "kvc_compress_layers", "layers_in_flight": kvc.SWEEP_STREAMS,
            "value": round(cfg.s * K / sweep_wall, 1), "unit": "tokens/s",
            "ms_per_step": round(sweep_wall * 1e3 / K, 5),
            "layer_hbm_frac": round(total_alg / (sweep_gpu_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "graph_replay": None if graph_ms is None else {
            "ms_per_layer": round(graph_ms, 5), "value": round(cfg.s / (graph_ms * 1e-3), 1), "unit": "tokens/s",
            "note": "one captured kvc_compress_layer per resident layer, replayed; HIP events around the replays"},
        "kernel_hash": kernel_source_hash(),
    }

    cpu = None
    if args.cpu_seconds > 0:
        log(f"CPU oracle baseline (about {args.cpu_seconds:.0f} s) ...")
        cpu = cpu_baseline(cfg, host_layers, [l[3] for l in layers], args.cpu_seconds)
        log(f"CPU oracle: {cpu['value']:.1f} tokens/s with {cpu['cores']} BLAS threads; {cpu['sample']}")
        cpu1 = cpu_baseline_one_thread(cfg, host_layers, [l[3] for l in layers], max(2.0, args.cpu_seconds / 3))
        extras["cpu_baseline_one_thread"] = cpu1
        log(f"CPU oracle, one thread: {cpu1['value']:.1f} tokens/s; {cpu1['sample']}")

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
            "entry_point": "kvc_compress_layer", "layers_in_flight": 1,
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "detail": extras,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
