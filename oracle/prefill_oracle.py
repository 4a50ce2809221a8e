"""CPU oracle for the synthetic layer-major chunked prefill (numpy, float64).

TEST INFRASTRUCTURE ONLY, like kvc_oracle: the plain definition the GPU
driver and its kernels are checked against. Only the test suite, the package
smoke check and the benchmark's CPU-baseline leg may import it; it shares no
code with the HIP library.

The schedule (TideKV, Fig. 2 caption: layer-major delayed eviction; Fig. 1
caption, schedule (d)): the prompt is processed layer by layer; within layer
l the chunks j = 0, 1, ... run in order, chunk j's queries attending to the
accumulated uncompressed K/V of chunks 0..j of that layer, and its output
hidden rows replacing its input rows in the hidden-state bridge that feeds
layer l + 1. After the last chunk the layer-end compressor (kvc_oracle's
compress_layer, with the prompt's last W queries as the window) turns the
layer's full K/V into its retained cache, and the full K/V is released.

The model is a decoder layer of the Llama family with random weights (the
pages name Llama-3.1-8B; they give no layer equations, so the standard ones
are written out here):

  xn   = rmsnorm(x) * w_attn            rmsnorm(x) = x / sqrt(mean(x^2) + eps)
  qkv  = xn @ W_qkv^T                   q [Hq, D], k [Hkv, D], v [Hkv, D] per token
  q, k = rope(q, p), rope(k, p)         rotary embedding at absolute position p:
         pairs (i, i + D/2) rotated by p * base^(-2i/D)
  o    = attention(q; k, v over keys at positions <= p), query head h reads
         KV head h // G, scale 1/sqrt(D)
  h    = x + o @ W_o^T
  hn   = rmsnorm(h) * w_mlp
  gu   = hn @ W_gu^T                    gate = first F columns, up = last F
  out  = h + (silu(gate) * up) @ W_down^T,   silu(g) = g / (1 + exp(-g))

The GPU keeps activations in bf16 between operations. `layer_chunk` can
emulate that: each operation is computed exactly (float64) from bf16 inputs
and its output rounded to bf16 (round to nearest even, via float32), at the
same points where the GPU rounds. Without emulation everything stays float64.

Parity pins: closed forms, invariants, library routines and brute force in
the test suite's prefill pin module; none is "parity unpinned".
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .kvc_oracle import bf16_to_f64, compress_layer


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bit patterns: rounded to float32 (nearest even), then
    to bf16 (nearest even). The double rounding differs from one direct
    rounding only when the float32 value lands exactly on a bf16 midpoint."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x [n, H], w [H] (float64): x / sqrt(mean(x^2) + eps) * w per row."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * w


def rope_cos_sin(positions: np.ndarray, d: int, base: float):
    """cos, sin [n, D/2] of the rotation angles p * base^(-2i/D)."""
    i = np.arange(d // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / d)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang), np.sin(ang)


def rope(x: np.ndarray, positions: np.ndarray, base: float) -> np.ndarray:
    """x [n, heads, D]: pairs (i, i + D/2) rotated by the token's angles."""
    n, _, d = x.shape
    c, s = rope_cos_sin(positions, d, base)
    c, s = c[:, None, :], s[:, None, :]
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray, scale: float | None = None):
    """Causal GQA attention. q [n, Hq, D] at positions q_pos; k, v [T, Hkv, D]
    at positions 0..T-1. Row (t, h) attends to keys j <= q_pos[t] of KV head
    h // G with softmax(scale * <q, k_j>)."""
    n, hq, d = q.shape
    t_len, hkv, _ = k.shape
    g = hq // hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.zeros_like(q)
    j = np.arange(t_len)
    for h in range(hq):
        kh, vh = k[:, h // g, :], v[:, h // g, :]
        logits = scale * (q[:, h, :] @ kh.T)                 # [n, T]
        logits = np.where(j[None, :] <= np.asarray(q_pos)[:, None], logits, -np.inf)
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        out[:, h, :] = (p @ vh) / p.sum(axis=1, keepdims=True)
    return out


def silu(x: np.ndarray) -> np.ndarray:
    return x / (1.0 + np.exp(-x))


def swiglu(gu: np.ndarray) -> np.ndarray:
    """gu [n, 2F] -> silu(gate) * up, gate = first F columns."""
    f = gu.shape[-1] // 2
    return silu(gu[..., :f]) * gu[..., f:]


@dataclass
class LayerWeights:
    """bf16 bit patterns. w_qkv [(Hq + 2 Hkv) D, H] (rows: q heads, then k,
    then v), w_o [H, Hq D], w_gu [2F, H] (gate rows, then up rows),
    w_down [H, F], norms [H]."""
    w_attn: np.ndarray
    w_qkv: np.ndarray
    w_o: np.ndarray
    w_mlp: np.ndarray
    w_gu: np.ndarray
    w_down: np.ndarray


@dataclass
class ModelShape:
    hidden: int
    hq: int
    hkv: int
    d: int
    ffn: int
    eps: float = 1e-5
    rope_base: float = 500000.0


def layer_chunk(x, wt: LayerWeights, shp: ModelShape, c0: int, k_cache, v_cache, emulate_bf16=True):
    """One layer on chunk rows [c0, c0 + n) of the bridge.

    x: float64 values [n, H] (bf16 values when emulating). k_cache, v_cache:
    float64 [>= c0 + n, Hkv, D], rows [0, c0) already filled by earlier
    chunks; rows [c0, c0 + n) are written here. Returns (out [n, H], q
    [n, Hq, D] after rope), both float64 values."""
    r = (lambda a: bf16_to_f64(to_bf16_bits(a))) if emulate_bf16 else (lambda a: a)
    f = bf16_to_f64
    n = x.shape[0]
    hq, hkv, d = shp.hq, shp.hkv, shp.d
    pos = np.arange(c0, c0 + n)
    xn = r(rmsnorm(x, f(wt.w_attn), shp.eps))
    qkv = r(xn @ f(wt.w_qkv).T)
    q = r(rope(qkv[:, : hq * d].reshape(n, hq, d), pos, shp.rope_base))
    k = r(rope(qkv[:, hq * d:(hq + hkv) * d].reshape(n, hkv, d), pos, shp.rope_base))
    v = qkv[:, (hq + hkv) * d:].reshape(n, hkv, d)
    k_cache[c0:c0 + n] = k
    v_cache[c0:c0 + n] = v
    o = r(attention(q, k_cache[: c0 + n], v_cache[: c0 + n], pos))
    h = r(x + o.reshape(n, hq * d) @ f(wt.w_o).T)
    hn = r(rmsnorm(h, f(wt.w_mlp), shp.eps))
    gu = r(hn @ f(wt.w_gu).T)
    a = r(swiglu(gu))
    out = r(h + a @ f(wt.w_down).T)
    return out, q


@dataclass
class PrefillResult:
    hidden: np.ndarray          # final bridge [S, H], float64 values
    k: list                     # per layer: full K [S, Hkv, D] (float64 values)
    v: list
    q_win: list                 # per layer: the last W queries after rope [W, Hq, D]
    retained: list              # per layer: kvc_oracle.LayerResult


def prefill_layer_major(x_bits, weights, shp: ModelShape, chunk: int, w: int, budgets, n_sink: int,
                        n_recent: int, emulate_bf16=True, compress=True):
    """The layer-major chunked prefill with layer-end eviction over all
    layers; returns the final bridge, every layer's full K/V and window
    queries, and (compress=True) every layer's retained cache."""
    s = x_bits.shape[0]
    bridge = bf16_to_f64(x_bits)
    res = PrefillResult(hidden=None, k=[], v=[], q_win=[], retained=[])
    for wt in weights:
        k_cache = np.zeros((s, shp.hkv, shp.d))
        v_cache = np.zeros((s, shp.hkv, shp.d))
        q_win = np.zeros((w, shp.hq, shp.d))
        for c0 in range(0, s, chunk):
            c1 = min(c0 + chunk, s)
            out, q = layer_chunk(bridge[c0:c1], wt, shp, c0, k_cache, v_cache, emulate_bf16)
            bridge[c0:c1] = out
            lo = max(c0, s - w)
            if lo < c1:
                q_win[lo - (s - w):c1 - (s - w)] = q[lo - c0:]
        res.k.append(k_cache)
        res.v.append(v_cache)
        res.q_win.append(q_win)
        if compress:
            res.retained.append(compress_layer(to_bf16_bits(q_win), to_bf16_bits(k_cache), to_bf16_bits(v_cache),
                                               budgets, n_sink, n_recent))
    res.hidden = bridge
    return res
