"""CPU oracle for the layer-end KV-eviction compressor (numpy, float64).

TEST INFRASTRUCTURE ONLY. This module is the plain, slow definition that the
GPU path is checked against. Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import it; the product path never does.
It shares no code with the HIP library: it reads bf16 bit patterns and writes
plain numpy arrays.

What it computes (TideKV, Fig. 3 caption: memory-controlled two-pass blockwise
scoring; Fig. 2 caption: layer-end gather of retained KV and absolute
positions). The blockwise two-pass scan on the page is an exact reorganisation
of one dense softmax per window query (the log-sum-exp merge), so the oracle
is that dense definition written out, materialising the W x S
observation-by-prefix tensor that the page's scan avoids:

  rows      r = (h, i): query head h, window query i (prompt position S-W+i)
  logits    l[h,i,j] = scale * <Q_win[i,h], K[j, h // G]>  for j <= S-W+i,
            -inf for later keys (causal); scale defaults to 1/sqrt(D)
  normaliser m[h,i] = max_j l,  Z[h,i] = sum_j exp(l - m)      (natural log units)
  weights   a[h,i,j] = exp(l - m) / Z
  scores    score[g,j] = sum over the G heads of group g and the W window rows
            of a[h,i,j]   (a sum, so sum_j score[g,:] = W * G)
  pooling   optional centred 1-D max-pool of odd width, truncated at the ends
  select    per KV head: mandatory sink [0, n_sink) and recent [S-n_recent, S)
            keys, plus the top K_h - |mandatory| other keys by (score desc,
            index asc); returned ascending
  gather    K_hat = K[idx, g], V_hat = V[idx, g] bit for bit;
            pos = pos_offset + idx

Score modes other than the softmax weights (HillInfer, Algorithmic
Simplification: ranking needs only the order of the keys and the softmax is
monotonic, so the raw inner product Q.K^T is used, without exponentiation or
scaling; Streaming Execution and Asymmetric Precision: those inner products in
INT8 for the ranking only, the streamed keys cast on the fly, the original
rows retrieved afterwards):

  logit     score[g,j] = sum over the visible rows (h, i) of group g of
            <Q_win[i,h], K[j,g]>, with no scale; for one query row this is the
            page's raw inner product. Summed over rows it is one dot product
            of K[j,g] with the pooled query of the rows that see key j.
  int8      the pooled query (summed exactly, rounded once to fp32) and each
            key row quantised symmetrically per vector: s = max |x|,
            x8 = round-half-even(x * fp32(127 / s)), all in fp32; the integer
            dot product is exact and the score is
            fp32(fp32(dot * fp32(s_q / 127)) * fp32(s_k / 127)).
  overlap   the overlap coefficient |A & B| / min(|A|, |B|) of two retained
            index sets (HeteroCache summary, Key Contributions item 1).

Immediate eviction, the schedule TideKV's layer-end eviction is compared
with (TideKV, Fig. 1 caption, schedule (c): chunked prefill that evicts after
every chunk; Table 8: Block-SnapKV): the prompt's keys arrive in chunks of C,
and after chunk b the same scorer and selection run over the keys retained so
far plus chunk b, with chunk b's last W queries as the window and one budget
for every head. Keys keep their prompt positions; the mandatory sink and
recent keys are the first n_sink and last n_recent of the accumulated keys.

Per-KV-head budgets for the heterogeneous workload follow the inverse
stability weighting of the HeteroCache summary (Methodology, Phase 2):
w_h = 1 / S_stable,h and K_h proportional to w_h, rounded to integers that sum
to the total by largest remainder (ties to the lower head index).

Parity pins: every function here is pinned by tests against closed forms,
invariants, library routines or brute force (see the test suite's oracle pin
module); none is "parity unpinned".
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


# ---------------------------------------------------------------------------
# bf16 decoding
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bf16 bit patterns exactly.

    A bf16 value is the upper 16 bits of an IEEE-754 binary32 value (1 sign,
    8 exponent, 7 fraction bits), so widening the pattern to 32 bits and
    reinterpreting gives the exact value, which float64 then holds exactly.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Scoring (TideKV Fig. 3 caption, read as the dense definition)
# ---------------------------------------------------------------------------

def default_scale(d: int) -> float:
    return 1.0 / np.sqrt(float(d))


def group_logits(q: np.ndarray, k: np.ndarray, g: int, scale: float) -> np.ndarray:
    """Causally masked logits of KV head g's query group: [G, W, S] float64.

    q: [W, Hq, D] float64 window queries (prompt positions S-W .. S-1)
    k: [S, Hkv, D] float64 keys
    """
    w, hq, d = q.shape
    s, hkv, _ = k.shape
    grp = hq // hkv
    out = np.empty((grp, w, s), dtype=np.float64)
    kg = k[:, g, :]                                    # [S, D]
    for t in range(grp):
        h = g * grp + t
        out[t] = scale * (q[:, h, :] @ kg.T)           # [W, S]
    qpos = s - w + np.arange(w)                        # absolute position of query i
    future = np.arange(s)[None, :] > qpos[:, None]     # key j after query i
    out[:, future] = -np.inf
    return out


def normalizers(q: np.ndarray, k: np.ndarray, scale: float | None = None):
    """Log-sum-exp normalisers (m, Z), each [Hq, W] float64.

    m is the row maximum of the logits and Z = sum_j exp(l - m), so that the
    softmax weight of key j is exp(l_j - m) / Z.
    """
    w, hq, d = q.shape
    s, hkv, _ = k.shape
    scale = default_scale(d) if scale is None else scale
    grp = hq // hkv
    m = np.empty((hq, w))
    z = np.empty((hq, w))
    for g in range(hkv):
        lg = group_logits(q, k, g, scale)
        mg = lg.max(axis=2)
        zg = np.exp(lg - mg[:, :, None]).sum(axis=2)
        m[g * grp:(g + 1) * grp] = mg
        z[g * grp:(g + 1) * grp] = zg
    return m, z


def scores(q: np.ndarray, k: np.ndarray, scale: float | None = None) -> np.ndarray:
    """Per-key scores [Hkv, S] float64: softmax weights summed over the W window
    rows and the G query heads of each KV head's group."""
    w, hq, d = q.shape
    s, hkv, _ = k.shape
    scale = default_scale(d) if scale is None else scale
    out = np.empty((hkv, s))
    for g in range(hkv):
        lg = group_logits(q, k, g, scale)
        mg = lg.max(axis=2, keepdims=True)
        e = np.exp(lg - mg)
        a = e / e.sum(axis=2, keepdims=True)
        out[g] = a.sum(axis=(0, 1))
    return out


# ---------------------------------------------------------------------------
# Raw inner-product ranking (HillInfer, Algorithmic Simplification) and its
# INT8 form (HillInfer, Streaming Execution and Asymmetric Precision)
# ---------------------------------------------------------------------------

def logit_scores(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """Raw inner-product scores [Hkv, S] float64: for key j of KV head g, the
    unscaled logits <Q_win[i,h], K[j,g]> summed over the rows (h in group g,
    window query i) that see key j under the causal mask."""
    w, hq, d = q.shape
    s, hkv, _ = k.shape
    out = np.empty((hkv, s))
    for g in range(hkv):
        lg = group_logits(q, k, g, 1.0)
        lg[~np.isfinite(lg)] = 0.0        # masked (future) keys contribute nothing
        out[g] = lg.sum(axis=(0, 1))
    return out


def first_visible_row(s: int, w: int) -> np.ndarray:
    """For each key j, the first window row i that sees it: max(0, j - (S-W))."""
    return np.maximum(np.arange(s) - (s - w), 0)


def pooled_query(q_bits: np.ndarray, hkv: int, t: int) -> np.ndarray:
    """fp32 [Hkv, D]: the sum of the bf16 window queries of each group over
    rows i >= t, summed exactly (math.fsum) and rounded once to fp32."""
    import math
    q = bf16_to_f64(q_bits)
    w, hq, d = q.shape
    grp = hq // hkv
    out = np.empty((hkv, d), dtype=np.float32)
    for g in range(hkv):
        blk = q[t:, g * grp:(g + 1) * grp, :].reshape(-1, d)
        for c in range(d):
            out[g, c] = np.float32(math.fsum(blk[:, c]))
    return out


def quantize_int8(x: np.ndarray):
    """Symmetric per-vector INT8 codes of fp32 vectors along the last axis.

    s = max |x|; each element becomes round-half-even(x * fp32(127 / s)),
    computed in fp32 (the decision the kernel takes, in its precision); the
    dequantisation step is fp32(s / 127). An all-zero vector gives zero codes
    and a zero step. Returns (codes int32, step float32).
    """
    x = np.asarray(x, dtype=np.float32)
    s = np.max(np.abs(x), axis=-1).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    r = (np.float32(127.0) / safe).astype(np.float32)
    codes = np.rint((x * r[..., None]).astype(np.float32)).astype(np.int32)
    codes = np.where((s > 0)[..., None], codes, 0)
    step = np.where(s > 0, (s / np.float32(127.0)).astype(np.float32), np.float32(0.0)).astype(np.float32)
    return codes, step


def logit_scores_int8(q_bits: np.ndarray, k_bits: np.ndarray) -> np.ndarray:
    """INT8 raw inner-product scores [Hkv, S] float32: the pooled query of the
    rows that see key j and the key row, each quantised by quantize_int8; the
    score is fp32(fp32(dot * step_q) * step_k) with the exact integer dot."""
    w, hq, d = q_bits.shape
    s, hkv, _ = k_bits.shape
    kf = bf16_to_f64(k_bits).astype(np.float32)        # exact: bf16 fits fp32
    k8, ks = quantize_int8(kf)                          # [S, Hkv, D], [S, Hkv]
    t_of = first_visible_row(s, w)
    out = np.empty((hkv, s), dtype=np.float32)
    for t in np.unique(t_of):
        q8, qs = quantize_int8(pooled_query(q_bits, hkv, int(t)))   # [Hkv, D], [Hkv]
        keys = np.nonzero(t_of == t)[0]
        for g in range(hkv):
            dot = k8[keys, g, :].astype(np.int64) @ q8[g].astype(np.int64)
            out[g, keys] = ((dot.astype(np.float32) * qs[g]).astype(np.float32) * ks[keys, g]).astype(np.float32)
    return out


def overlap_coefficient(a, b) -> float:
    """|A & B| / min(|A|, |B|) of two index sets; 1.0 when either is empty."""
    a, b = np.unique(np.asarray(a)), np.unique(np.asarray(b))
    n = min(a.size, b.size)
    return 1.0 if n == 0 else np.intersect1d(a, b).size / n


# ---------------------------------------------------------------------------
# Optional max-pool over scores
# ---------------------------------------------------------------------------

def maxpool(score: np.ndarray, width: int) -> np.ndarray:
    """Centred 1-D max-pool of odd ``width`` along the last axis, stride 1; the
    window is truncated at both ends (equivalently, padded with -inf)."""
    if width <= 1:
        return np.array(score, dtype=np.float64, copy=True)
    if width % 2 == 0:
        raise ValueError("pool width must be odd")
    r = width // 2
    x = np.asarray(score, dtype=np.float64)
    s = x.shape[-1]
    out = np.array(x, copy=True)
    for t in range(1, r + 1):
        # neighbour t to the right, and t to the left
        out[..., : s - t] = np.maximum(out[..., : s - t], x[..., t:])
        out[..., t:] = np.maximum(out[..., t:], x[..., : s - t])
    return out


# ---------------------------------------------------------------------------
# Selection (TideKV Fig. 3 caption: top K_l - |R_mand| non-mandatory keys
# plus the mandatory sink/recent set)
# ---------------------------------------------------------------------------

def mandatory(s: int, n_sink: int, n_recent: int) -> np.ndarray:
    """Ascending mandatory key indices: [0, n_sink) united with [S - n_recent, S)."""
    sink = np.arange(min(n_sink, s))
    recent = np.arange(max(s - n_recent, 0), s)
    return np.union1d(sink, recent).astype(np.int64)


def select_head(values: np.ndarray, budget: int, n_sink: int, n_recent: int) -> np.ndarray:
    """Retained key indices of one KV head, ascending.

    Keeps every mandatory key, then the ``budget - |mandatory|`` best other keys
    ranked by value descending with the lower index winning ties. A budget of
    at least S keeps every key.
    """
    values = np.asarray(values, dtype=np.float64)
    s = values.shape[0]
    if budget >= s:
        return np.arange(s, dtype=np.int64)
    mand = mandatory(s, n_sink, n_recent)
    if budget < mand.size:
        raise ValueError("budget smaller than the mandatory set")
    is_cand = np.ones(s, dtype=bool)
    is_cand[mand] = False
    cand = np.nonzero(is_cand)[0]
    k_sel = budget - mand.size
    # lexsort sorts by the last key first: value descending, then index ascending
    order = np.lexsort((cand, -values[cand]))
    chosen = cand[order[:k_sel]]
    return np.sort(np.concatenate([mand, chosen])).astype(np.int64)


def select(values: np.ndarray, budgets, n_sink: int, n_recent: int) -> list[np.ndarray]:
    """Per-head retained indices for values [Hkv, S] and budgets [Hkv]."""
    return [select_head(values[g], int(budgets[g]), n_sink, n_recent)
            for g in range(values.shape[0])]


# ---------------------------------------------------------------------------
# Gather (TideKV Fig. 2 caption: retained KV and absolute positions)
# ---------------------------------------------------------------------------

def gather(k_bits: np.ndarray, v_bits: np.ndarray, idx: list[np.ndarray], pos_offset: int = 0):
    """Retained rows, head-major: K_hat, V_hat [sum K_h, D] (bf16 bits, copied
    bit for bit) and positions [sum K_h] int64 = pos_offset + index."""
    k_rows, v_rows, pos = [], [], []
    for g, ix in enumerate(idx):
        k_rows.append(k_bits[ix, g, :])
        v_rows.append(v_bits[ix, g, :])
        pos.append(pos_offset + ix)
    return (np.concatenate(k_rows, axis=0), np.concatenate(v_rows, axis=0),
            np.concatenate(pos).astype(np.int64))


# ---------------------------------------------------------------------------
# Heterogeneous per-head budgets (HeteroCache summary, Methodology, Phase 2)
# ---------------------------------------------------------------------------

def inverse_stability_budgets(s_stable, total: int) -> np.ndarray:
    """Budgets K_h proportional to 1 / S_stable,h summing exactly to ``total``.

    Each head first gets floor(total * w_h / sum w); the remaining slots go,
    one each, to the heads with the largest fractional parts, the lower head
    index first among equal parts. Sums run in head order.
    """
    s_stable = [float(x) for x in s_stable]
    w = [1.0 / x for x in s_stable]
    wsum = 0.0
    for x in w:
        wsum += x
    exact = [total * x / wsum for x in w]
    base = [int(np.floor(e)) for e in exact]
    frac = [e - b for e, b in zip(exact, base)]
    rem = int(total - sum(base))
    order = sorted(range(len(w)), key=lambda h: (-frac[h], h))
    for h in order[:rem]:
        base[h] += 1
    return np.array(base, dtype=np.int64)


# ---------------------------------------------------------------------------
# One layer end to end
# ---------------------------------------------------------------------------

@dataclass
class LayerResult:
    m: np.ndarray          # [Hq, W] (None unless score_mode == "softmax")
    z: np.ndarray          # [Hq, W] (None unless score_mode == "softmax")
    scores: np.ndarray     # [Hkv, S] (not pooled)
    idx: list              # per head, ascending int64
    k_hat: np.ndarray      # [sum K_h, D] uint16
    v_hat: np.ndarray      # [sum K_h, D] uint16
    pos: np.ndarray        # [sum K_h] int64


def compress_layer(q_bits, k_bits, v_bits, budgets, n_sink, n_recent,
                   scale=None, pool=1, pos_offset=0, score_mode="softmax") -> LayerResult:
    """One layer with scores of ``score_mode``: "softmax" (the default),
    "logit" (raw inner products) or "int8" (their INT8 form)."""
    q = bf16_to_f64(q_bits)
    k = bf16_to_f64(k_bits)
    if score_mode == "softmax":
        m, z = normalizers(q, k, scale)
        sc = scores(q, k, scale)
    elif score_mode == "logit":
        m = z = None
        sc = logit_scores(q, k)
    elif score_mode == "int8":
        m = z = None
        sc = logit_scores_int8(q_bits, k_bits).astype(np.float64)
    else:
        raise ValueError(f"unknown score mode {score_mode!r}")
    sel_vals = maxpool(sc, pool) if pool > 1 else sc
    idx = select(sel_vals, budgets, n_sink, n_recent)
    k_hat, v_hat, pos = gather(k_bits, v_bits, idx, pos_offset)
    return LayerResult(m=m, z=z, scores=sc, idx=idx, k_hat=k_hat, v_hat=v_hat, pos=pos)


# ---------------------------------------------------------------------------
# Immediate (chunk-boundary) eviction (TideKV, Fig. 1 caption, schedule (c);
# Table 8, Block-SnapKV)
# ---------------------------------------------------------------------------

def chunk_bounds(s: int, chunk: int) -> list[tuple[int, int]]:
    """Token ranges [c0, c1) of the chunks of an s-token prompt."""
    return [(c0, min(c0 + chunk, s)) for c0 in range(0, s, chunk)]


def compress_chunked(q_windows, k_bits, v_bits, chunk: int, budget: int, n_sink: int,
                     n_recent: int, scale=None, pool=1, pos_offset=0, score_mode="softmax"):
    """Final retained set of immediate eviction: per KV head, ascending prompt
    indices, K_hat / V_hat rows (bf16 bits) and positions, as compress_layer's
    LayerResult (m, z and scores of the last chunk boundary).

    q_windows: bf16 bits [n_chunks, W, Hq, D], window b being the queries at
    the last W positions of chunk b. At each boundary the accumulated keys of
    a head are its retained keys (ascending positions) followed by the
    chunk's keys, so the window's causal mask by index is the mask by
    position -- which needs every chunk, the last included, to hold at least
    W tokens (otherwise a window row would precede retained keys).
    """
    s, hkv, d = k_bits.shape
    w = q_windows.shape[1]
    bounds = chunk_bounds(s, chunk)
    if len(q_windows) != len(bounds) or any(c1 - c0 < w for c0, c1 in bounds):
        raise ValueError("one window per chunk, and every chunk at least W tokens long")
    kept = [np.zeros(0, dtype=np.int64) for _ in range(hkv)]   # prompt indices per head
    res = None
    for b, (c0, c1) in enumerate(bounds):
        new = np.arange(c0, c1)
        acc = [np.concatenate([kept[g], new]) for g in range(hkv)]
        n_acc = acc[0].size
        k_acc = np.stack([k_bits[acc[g], g, :] for g in range(hkv)], axis=1)   # [S_acc, Hkv, D]
        v_acc = np.stack([v_bits[acc[g], g, :] for g in range(hkv)], axis=1)
        res = compress_layer(q_windows[b], k_acc, v_acc, [budget] * hkv, n_sink, n_recent,
                             scale=scale, pool=pool, score_mode=score_mode)
        kept = [acc[g][res.idx[g]] for g in range(hkv)]
        assert all(x.size == min(budget, n_acc) for x in kept)
    k_hat = np.concatenate([k_bits[kept[g], g, :] for g in range(hkv)], axis=0)
    v_hat = np.concatenate([v_bits[kept[g], g, :] for g in range(hkv)], axis=0)
    pos = np.concatenate([pos_offset + kept[g] for g in range(hkv)]).astype(np.int64)
    return LayerResult(m=res.m, z=res.z, scores=res.scores, idx=kept, k_hat=k_hat, v_hat=v_hat, pos=pos)
