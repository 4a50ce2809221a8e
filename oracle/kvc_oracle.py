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
    m: np.ndarray          # [Hq, W]
    z: np.ndarray          # [Hq, W]
    scores: np.ndarray     # [Hkv, S] (not pooled)
    idx: list              # per head, ascending int64
    k_hat: np.ndarray      # [sum K_h, D] uint16
    v_hat: np.ndarray      # [sum K_h, D] uint16
    pos: np.ndarray        # [sum K_h] int64


def compress_layer(q_bits, k_bits, v_bits, budgets, n_sink, n_recent,
                   scale=None, pool=1, pos_offset=0) -> LayerResult:
    q = bf16_to_f64(q_bits)
    k = bf16_to_f64(k_bits)
    m, z = normalizers(q, k, scale)
    sc = scores(q, k, scale)
    sel_vals = maxpool(sc, pool) if pool > 1 else sc
    idx = select(sel_vals, budgets, n_sink, n_recent)
    k_hat, v_hat, pos = gather(k_bits, v_bits, idx, pos_offset)
    return LayerResult(m=m, z=z, scores=sc, idx=idx, k_hat=k_hat, v_hat=v_hat, pos=pos)
