"""Deterministic synthetic layer inputs (bf16 bit patterns in uint16 arrays).

Recipe (one layer of one workload):
  * the layer's seed is ``cfg.seed_base + layer``; a numpy ``SeedSequence`` of
    that seed spawns independent child streams for Q, K, V, the planted heavy
    keys and the per-head stabilities, so each tensor is reproducible on its own;
  * K and V are drawn in chunks of ``CHUNK`` tokens, each chunk from its own
    grandchild stream, so the bytes do not depend on how many threads draw them;
  * every value is drawn as float32 N(0, 1) (PCG64) and rounded to bf16 with
    round-to-nearest-even;
  * ``n_heavy`` positions, uniform without replacement in [n_sink, s - w), are
    planted in every KV head g as bf16(3 * sqrt(d) * u_g + eps), where u_g is the
    unit mean of the bf16 window queries of g's query group and eps ~ N(0, I);
  * the first ``n_sink`` keys of every head are multiplied by ``sink_scale``
    (a power of two, so the bf16 product is exact);
  * for the heterogeneous-budget workload, per-KV-head stabilities are drawn
    from U(0.2, 0.9) (float64);
  * for chunked prefill with immediate eviction, chunk b's window (the queries
    at its last w positions) is drawn like Q from child b of the seed
    sequence [layer seed, 1]; the last chunk's window is the layer's Q itself,
    the queries at the prompt's last w positions.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

from .configs import LayerConfig

CHUNK = 4096  # tokens per independently seeded K/V chunk


def layer_seed(cfg: LayerConfig, layer: int) -> int:
    return int(cfg.seed_base) + int(layer)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class LayerInputs:
    cfg: LayerConfig
    layer: int
    q: np.ndarray            # [w, hq, d]  uint16 (bf16 bits)
    k: np.ndarray            # [s, hkv, d] uint16
    v: np.ndarray            # [s, hkv, d] uint16
    heavy_pos: np.ndarray    # [n_heavy] int64, ascending
    s_stable: np.ndarray | None  # [hkv] float64 (heterogeneous budgets only)


def _normal_bf16(seed_seq: np.random.SeedSequence, shape) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed_seq))
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def _chunked_normal_bf16(seed_seq, s, hkv, d, pool) -> np.ndarray:
    n_chunks = (s + CHUNK - 1) // CHUNK
    kids = seed_seq.spawn(n_chunks)
    out = np.empty((s, hkv, d), dtype=np.uint16)

    def fill(c):
        lo = c * CHUNK
        hi = min(s, lo + CHUNK)
        out[lo:hi] = _normal_bf16(kids[c], (hi - lo, hkv, d))

    list(pool.map(fill, range(n_chunks)))
    return out


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def layer_inputs(cfg: LayerConfig, layer: int = 0, threads: int | None = None) -> LayerInputs:
    root = np.random.SeedSequence(layer_seed(cfg, layer))
    ss_q, ss_k, ss_v, ss_heavy, ss_stable = root.spawn(5)
    s, w, hq, hkv, d = cfg.s, cfg.w, cfg.hq, cfg.hkv, cfg.d
    g = cfg.group

    q = _normal_bf16(ss_q, (w, hq, d))
    with ThreadPoolExecutor(max_workers=threads or _threads()) as pool:
        k = _chunked_normal_bf16(ss_k, s, hkv, d, pool)
        v = _chunked_normal_bf16(ss_v, s, hkv, d, pool)

    # Planted heavy keys along each group's mean window-query direction.
    rng_h = np.random.Generator(np.random.PCG64(ss_heavy))
    lo, hi = cfg.n_sink, s - w
    n_heavy = min(cfg.n_heavy, max(0, hi - lo))
    heavy = np.sort(rng_h.choice(hi - lo, size=n_heavy, replace=False).astype(np.int64) + lo) \
        if n_heavy > 0 else np.zeros(0, dtype=np.int64)
    noise = rng_h.standard_normal((n_heavy, hkv, d), dtype=np.float32)
    qf = bf16_bits_to_f32(q).astype(np.float64)
    for kv in range(hkv):
        mean = qf[:, kv * g:(kv + 1) * g, :].reshape(-1, d).mean(axis=0)
        unit = mean / np.linalg.norm(mean)
        planted = (3.0 * np.sqrt(d) * unit)[None, :] + noise[:, kv, :].astype(np.float64)
        k[heavy, kv, :] = f32_to_bf16_bits(planted.astype(np.float32))

    # Sink-like leading keys with a scaled norm.
    if cfg.sink_scale != 1.0 and cfg.n_sink > 0:
        ns = min(cfg.n_sink, s)
        k[:ns] = f32_to_bf16_bits(bf16_bits_to_f32(k[:ns]) * np.float32(cfg.sink_scale))

    s_stable = None
    if cfg.hetero:
        rng_s = np.random.Generator(np.random.PCG64(ss_stable))
        s_stable = rng_s.uniform(0.2, 0.9, size=hkv)

    return LayerInputs(cfg=cfg, layer=layer, q=q, k=k, v=v, heavy_pos=heavy, s_stable=s_stable)


def chunk_windows(cfg: LayerConfig, chunk: int, layer: int = 0, q_last: np.ndarray | None = None) -> np.ndarray:
    """Window queries of every chunk, stacked [n_chunks * w, hq, d] (uint16):
    rows [b * w, (b + 1) * w) are chunk b's window. q_last: the layer's Q
    (drawn here when not given)."""
    n_chunks = (cfg.s + chunk - 1) // chunk
    if q_last is None:
        q_last = layer_inputs(cfg.with_(s=max(cfg.w, 1), n_heavy=0), layer).q
    kids = np.random.SeedSequence([layer_seed(cfg, layer), 1]).spawn(max(n_chunks - 1, 0))
    parts = [_normal_bf16(kids[b], (cfg.w, cfg.hq, cfg.d)) for b in range(n_chunks - 1)]
    parts.append(np.ascontiguousarray(q_last, dtype=np.uint16))
    return np.concatenate(parts, axis=0)


@dataclass
class SynthLayerWeights:
    """bf16 bit patterns of one decoder layer (layouts: w_qkv [(hq + 2 hkv) d,
    hidden], w_o [hidden, hq d], w_gu [2 ffn, hidden], w_down [hidden, ffn],
    norm weights [hidden])."""
    w_attn: np.ndarray
    w_qkv: np.ndarray
    w_o: np.ndarray
    w_mlp: np.ndarray
    w_gu: np.ndarray
    w_down: np.ndarray


def model_weights(hidden: int, hq: int, hkv: int, d: int, ffn: int, layers: int, seed: int):
    """Random decoder weights: projections N(0, 1/fan_in), norm weights
    1 + N(0, 0.01), each drawn as float32 and rounded to bf16; layer l's six
    tensors come from children of the seed sequence [seed, 2, l]."""
    out = []
    for l in range(layers):
        kids = np.random.SeedSequence([seed, 2, l]).spawn(6)

        def draw(k, shape, scale, shift=0.0):
            rng = np.random.Generator(np.random.PCG64(kids[k]))
            return f32_to_bf16_bits((rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
                                     + np.float32(shift)).astype(np.float32))

        out.append(SynthLayerWeights(
            w_attn=draw(0, (hidden,), 0.1, 1.0), w_qkv=draw(1, ((hq + 2 * hkv) * d, hidden), hidden ** -0.5),
            w_o=draw(2, (hidden, hq * d), (hq * d) ** -0.5), w_mlp=draw(3, (hidden,), 0.1, 1.0),
            w_gu=draw(4, (2 * ffn, hidden), hidden ** -0.5), w_down=draw(5, (hidden, ffn), ffn ** -0.5)))
    return out


def prompt_hidden(s: int, hidden: int, seed: int) -> np.ndarray:
    """Synthetic prompt hidden states [s, hidden]: N(0, 1) rounded to bf16."""
    return _normal_bf16(np.random.SeedSequence([seed, 3]), (s, hidden))
