"""Pins for the CPU oracle: each test checks it against something other than
itself -- a closed form, an invariant, a library routine in a special case,
brute force on tiny inputs, or a value printed on the pages -- so that a
plausible mistake (dropped term, wrong sign, wrong index or head mapping,
transposed operand, off-by-one mask) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.ndimage
import scipy.special

import oracle
from synth import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_qk(rng, w, hq, hkv, d, s, spread=1.0):
    q = rng.standard_normal((w, hq, d)) * spread
    k = rng.standard_normal((s, hkv, d)) * spread
    return q, k


# ---------------------------------------------------------------- bf16 decode

def test_bf16_decode_matches_format_definition():
    with open(os.path.join(GOLDEN, "bf16_patterns.json")) as f:
        fx = json.load(f)
    bits = np.array([int(b, 16) for b, _ in fx["patterns"]], dtype=np.uint16)
    want = np.array([v for _, v in fx["patterns"]], dtype=np.float64)
    got = oracle.bf16_to_f64(bits)
    assert np.array_equal(got, want)
    assert math.copysign(1.0, oracle.bf16_to_f64(np.array([0x8000], np.uint16))[0]) == -1.0
    assert np.isinf(oracle.bf16_to_f64(np.array([0x7F80], np.uint16))[0])


# ---------------------------------------------------------------- scores: invariants

@pytest.mark.parametrize("w,hq,hkv,d,s", [(1, 1, 1, 8, 5), (4, 4, 1, 16, 40), (8, 6, 2, 8, 33), (16, 8, 2, 32, 200)])
def test_scores_sum_to_window_times_group(w, hq, hkv, d, s):
    """Each causal softmax row sums to one and the pooling is a plain sum over
    the W rows of each of the G group heads, so each head's scores sum to W*G."""
    rng = np.random.default_rng(10 + s)
    q, k = rand_qk(rng, w, hq, hkv, d, s, spread=1.5)
    sc = oracle.scores(q, k)
    assert sc.shape == (hkv, s)
    np.testing.assert_allclose(sc.sum(axis=1), w * (hq // hkv), rtol=1e-12)
    assert np.all(sc >= 0)


@pytest.mark.parametrize("w,g,s", [(1, 1, 7), (4, 2, 12), (16, 4, 64), (5, 3, 6)])
def test_identical_keys_closed_form(w, g, s):
    """All keys equal: query i (position p=S-W+i) spreads weight 1/(p+1) over
    keys 0..p. Prefix keys j <= S-W receive G*sum_i 1/(S-W+i+1); window key
    S-W+t (t>=1) is seen only by queries i>=t."""
    rng = np.random.default_rng(3)
    d = 8
    q = rng.standard_normal((w, g, d))
    krow = rng.standard_normal(d)
    k = np.broadcast_to(krow, (s, 1, d)).copy()
    sc = oracle.scores(q, k)[0]
    p = s - w + np.arange(w)
    want = np.empty(s)
    for j in range(s):
        want[j] = g * sum(1.0 / (pi + 1) for pi in p if j <= pi)
    np.testing.assert_allclose(sc, want, rtol=1e-13)
    # normalisers: every row max is the same logit, Z counts visible keys
    m, z = oracle.normalizers(q, k)
    np.testing.assert_allclose(z, np.broadcast_to(p + 1.0, (g, w)), rtol=1e-13)
    np.testing.assert_allclose(m, (q @ krow / np.sqrt(d)).T, rtol=1e-13)


def test_single_query_reduces_to_softmax():
    """W = G = 1: the only window query is the last prompt position and sees
    every key, so the scores are one softmax (scipy's routine)."""
    rng = np.random.default_rng(5)
    d, s = 16, 50
    q, k = rand_qk(rng, 1, 1, 1, d, s, spread=2.0)
    sc = oracle.scores(q, k)[0]
    want = scipy.special.softmax(k[:, 0, :] @ q[0, 0, :] / np.sqrt(d))
    np.testing.assert_allclose(sc, want, rtol=1e-12)
    m, z = oracle.normalizers(q, k)
    lse = scipy.special.logsumexp(k[:, 0, :] @ q[0, 0, :] / np.sqrt(d))
    np.testing.assert_allclose(m[0, 0] + np.log(z[0, 0]), lse, rtol=1e-13)


@pytest.mark.parametrize("a,b", [(2.0, 0.5), (-3.0, 1.0), (4.0, -2.0)])
def test_two_keys_logistic(a, b):
    """S = 2, W = 1, D = 4: q = a e0, k0 = e0, k1 = b e0 give logits a/2 and
    a*b/2 (scale 1/sqrt 4), so key 0 scores the logistic of their difference."""
    q = np.zeros((1, 1, 4)); q[0, 0, 0] = a
    k = np.zeros((2, 1, 4)); k[0, 0, 0] = 1.0; k[1, 0, 0] = b
    sc = oracle.scores(q, k)[0]
    want0 = 1.0 / (1.0 + math.exp(a * b / 2 - a / 2))
    want1 = 1.0 / (1.0 + math.exp(a / 2 - a * b / 2))
    np.testing.assert_allclose(sc, [want0, want1], rtol=1e-14)


def test_explicit_scale_is_applied():
    q = np.zeros((1, 1, 4)); q[0, 0, 0] = 1.0
    k = np.zeros((2, 1, 4)); k[0, 0, 0] = 1.0
    sc = oracle.scores(q, k, scale=3.0)[0]
    np.testing.assert_allclose(sc[0], 1.0 / (1.0 + math.exp(-3.0)), rtol=1e-14)


def test_gqa_head_to_kv_mapping():
    """Query head h reads KV head h // G. Group 0 (heads 0, 1) looks along e0,
    group 1 (heads 2, 3) along e1; KV head 0 hides key 3 along e0, KV head 1
    hides key 5 along e1. With the correct mapping every row of both groups
    finds its planted key (logit alpha * scale, all other logits 0); an
    h % Hkv mapping would pair head 1 with KV head 1 and miss it."""
    s, w, hq, hkv, d, alpha = 9, 2, 4, 2, 4, 6.0
    q = np.zeros((w, hq, d))
    q[:, 0:2, 0] = alpha
    q[:, 2:4, 1] = alpha
    k = np.zeros((s, hkv, d))
    k[3, 0, 0] = 1.0
    k[5, 1, 1] = 1.0
    sc = oracle.scores(q, k)
    x = math.exp(alpha / 2.0)  # scale 1/sqrt(4)
    p = s - w + np.arange(w)   # rows see p+1 keys each
    planted = sum(x / (x + p_i) for p_i in p) * 2      # two heads per group
    other = sum(1.0 / (x + p_i) for p_i in p) * 2
    want = np.full((hkv, s), other)
    # window key s-1 is seen only by the last query
    want[:, s - 1] = 2 * (1.0 / (x + p[-1]))
    want[0, 3] = planted
    want[1, 5] = planted
    np.testing.assert_allclose(sc, want, rtol=1e-13)


def test_causal_mask_hides_future_keys():
    """Only the last key is non-zero (logit alpha * scale for every row). Only
    the last window query may see it; earlier window queries spread weight
    uniformly over their visible keys."""
    s, w, g, d, alpha = 20, 4, 2, 4, 8.0
    q = np.zeros((w, g, d)); q[:, :, 2] = alpha
    k = np.zeros((s, 1, d)); k[s - 1, 0, 2] = 1.0
    sc = oracle.scores(q, k)[0]
    x = math.exp(alpha / 2.0)
    assert sc[s - 1] == pytest.approx(g * x / (x + s - 1), rel=1e-13)
    p = s - w + np.arange(w)
    j = 0
    want0 = g * (sum(1.0 / (p_i + 1) for p_i in p[:-1]) + 1.0 / (x + s - 1))
    assert sc[j] == pytest.approx(want0, rel=1e-13)


def test_dominant_key_tends_to_window_times_group():
    s, w, g, d = 30, 8, 4, 8
    q = np.zeros((w, g, d)); q[:, :, 0] = 1.0
    k = np.zeros((s, 1, d)); k[7, 0, 0] = 400.0
    sc = oracle.scores(q, k)[0]
    assert sc[7] == pytest.approx(w * g, rel=1e-12)


def test_permuting_heads_within_a_group_leaves_scores():
    rng = np.random.default_rng(8)
    q, k = rand_qk(rng, 6, 8, 2, 16, 40)
    perm = np.array([2, 0, 3, 1, 5, 7, 4, 6])  # stays inside each group of 4
    np.testing.assert_allclose(oracle.scores(q[:, perm, :], k), oracle.scores(q, k), rtol=1e-12)


def test_large_logits_do_not_overflow():
    """The max subtraction keeps huge logits finite: a key 1e4 logits ahead
    takes the whole row."""
    q = np.zeros((1, 1, 4)); q[0, 0, 0] = 1.0
    k = np.zeros((3, 1, 4)); k[1, 0, 0] = 2e4
    sc = oracle.scores(q, k)[0]
    assert np.all(np.isfinite(sc))
    np.testing.assert_allclose(sc, [0.0, 1.0, 0.0], atol=1e-300)


# ---------------------------------------------------------------- max-pool

@pytest.mark.parametrize("width", [1, 3, 7])
def test_maxpool_brute_force_and_scipy(width):
    rng = np.random.default_rng(width)
    x = rng.random((3, 41))
    got = oracle.maxpool(x, width)
    r = width // 2
    brute = np.array([[max(x[g, max(0, j - r): j + r + 1]) for j in range(41)] for g in range(3)])
    np.testing.assert_array_equal(got, brute)
    # a max over a window clamped at the edges equals truncation
    np.testing.assert_array_equal(got, scipy.ndimage.maximum_filter1d(x, width, axis=1, mode="nearest"))


def test_maxpool_rejects_even_width():
    with pytest.raises(ValueError):
        oracle.maxpool(np.zeros(4), 4)


# ---------------------------------------------------------------- selection

def _brute_select(values, budget, n_sink, n_recent):
    """Try every subset of candidates of the right size and keep the one whose
    members, listed by (value desc, index asc), are lexicographically best."""
    s = len(values)
    if budget >= s:
        return list(range(s))
    mand = set(range(min(n_sink, s))) | set(range(max(0, s - n_recent), s))
    cand = [j for j in range(s) if j not in mand]
    k = budget - len(mand)
    best, best_key = None, None
    for sub in itertools.combinations(cand, k):
        key = sorted(((-values[j], j) for j in sub))
        if best_key is None or key < best_key:
            best, best_key = sub, key
    return sorted(mand | set(best))


@pytest.mark.parametrize("seed", range(12))
def test_select_matches_exhaustive_search(seed):
    rng = np.random.default_rng(seed)
    s = int(rng.integers(6, 12))
    n_sink = int(rng.integers(0, 3))
    n_recent = int(rng.integers(0, 3))
    budget = int(rng.integers(n_sink + n_recent, s + 2))
    # coarse values so ties are common
    values = rng.integers(0, 4, size=s).astype(np.float64)
    got = oracle.select_head(values, budget, n_sink, n_recent)
    assert list(got) == _brute_select(values, budget, n_sink, n_recent)


def test_select_ties_take_lowest_index():
    s = 20
    values = np.ones(s)
    got = oracle.select_head(values, 8, 2, 3)
    assert list(got) == [0, 1, 2, 3, 4, 17, 18, 19]


def test_select_mandatory_always_kept_and_sizes():
    rng = np.random.default_rng(0)
    values = rng.random(100)
    values[:4] = 0.0       # sinks with the lowest scores are still kept
    values[-5:] = 0.0
    got = oracle.select_head(values, 30, 4, 5)
    assert len(got) == 30
    assert set(range(4)) <= set(got) and set(range(95, 100)) <= set(got)
    assert np.all(np.diff(got) > 0)
    chosen = [j for j in got if 4 <= j < 95]
    others = [j for j in range(4, 95) if j not in chosen]
    assert min(values[chosen]) >= max(values[others])


def test_select_budget_covering_all_keys():
    assert list(oracle.select_head(np.zeros(5), 5, 1, 1)) == [0, 1, 2, 3, 4]
    assert list(oracle.select_head(np.zeros(5), 9, 4, 4)) == [0, 1, 2, 3, 4]


def test_select_overlapping_mandatory_ranges():
    # sink and recent overlap when n_sink + n_recent > S
    assert list(oracle.mandatory(5, 3, 4)) == [0, 1, 2, 3, 4]
    assert list(oracle.mandatory(10, 0, 0)) == []


def test_select_rejects_budget_below_mandatory():
    with pytest.raises(ValueError):
        oracle.select_head(np.zeros(50), 5, 4, 4)


# ---------------------------------------------------------------- gather

def test_gather_copies_the_indexed_rows_bit_for_bit():
    """Every element's bit pattern encodes (token, head, column), so the
    gathered rows can be decoded back to the indices they came from."""
    s, hkv, d = 37, 3, 8
    j, g, c = np.meshgrid(np.arange(s), np.arange(hkv), np.arange(d), indexing="ij")
    k = (j * 97 + g * 13 + c).astype(np.uint16)
    v = (60000 - (j * 53 + g * 7 + c)).astype(np.uint16)
    idx = [np.array([0, 5, 36]), np.array([1, 2]), np.array([30])]
    kh, vh, pos = oracle.gather(k, v, idx, pos_offset=1000)
    assert kh.shape == (6, d) and kh.dtype == np.uint16
    rows = [(jj, gg) for gg, ix in enumerate(idx) for jj in ix]
    for r, (jj, gg) in enumerate(rows):
        assert list(kh[r]) == [jj * 97 + gg * 13 + cc for cc in range(d)]
        assert list(vh[r]) == [60000 - (jj * 53 + gg * 7 + cc) for cc in range(d)]
    assert list(pos) == [1000 + jj for jj, _ in rows]


# ---------------------------------------------------------------- budgets

def test_budgets_hand_example():
    # weights 2 and 4, total 10: exact 3.33 and 6.67 -> floors 3, 6 -> the
    # remaining slot goes to the larger fractional part
    assert list(oracle.inverse_stability_budgets([0.5, 0.25], 10)) == [3, 7]


def test_budgets_equal_stability_split_evenly():
    assert list(oracle.inverse_stability_budgets([0.4] * 8, 32768)) == [4096] * 8
    # 3 equal heads, total 10: floors 3,3,3; ties in the fractional part go to
    # the lower head index
    assert list(oracle.inverse_stability_budgets([0.3] * 3, 10)) == [4, 3, 3]


@pytest.mark.parametrize("seed", range(20))
def test_budgets_sum_and_proportionality(seed):
    rng = np.random.default_rng(seed)
    st = rng.uniform(0.2, 0.9, size=8)
    b = oracle.inverse_stability_budgets(st, 32768)
    assert b.sum() == 32768
    w = 1.0 / st
    exact = 32768 * w / w.sum()
    assert np.all(np.abs(b - exact) < 1.0)
    # less stable heads never get a smaller budget
    order = np.argsort(st)
    assert np.all(np.diff(b[order]) <= 0)


# ---------------------------------------------------------------- the pages' number

def test_final_cache_size_matches_tidekv():
    """At budget 4096 per KV head, 32 layers of retained bf16 K and V for the
    Llama-3.1-8B geometry make the 512-MiB final cache TideKV reports."""
    with open(os.path.join(GOLDEN, "tidekv_final_cache.json")) as f:
        fx = json.load(f)
    rng = np.random.default_rng(0)
    s, hkv, d = 5000, fx["kv_heads"], fx["head_dim"]
    k = rng.integers(0, 65535, size=(s, hkv, d), dtype=np.uint16)
    v = rng.integers(0, 65535, size=(s, hkv, d), dtype=np.uint16)
    vals = rng.random((hkv, s))
    idx = oracle.select(vals, [fx["budget_per_head"]] * hkv, 4, 32)
    kh, vh, pos = oracle.gather(k, v, idx)
    per_layer = kh.nbytes + vh.nbytes
    assert per_layer * fx["layers"] == fx["final_cache_bytes"]


# ---------------------------------------------------------------- end to end

def test_compress_layer_composes_the_steps():
    rng = np.random.default_rng(2)
    s, w, hq, hkv, d = 64, 4, 4, 2, 8
    qf = rng.standard_normal((w, hq, d)).astype(np.float32)
    kf = rng.standard_normal((s, hkv, d)).astype(np.float32)
    vf = rng.standard_normal((s, hkv, d)).astype(np.float32)
    qb, kb, vb = f32_to_bf16_bits(qf), f32_to_bf16_bits(kf), f32_to_bf16_bits(vf)
    r = oracle.compress_layer(qb, kb, vb, [10, 12], 2, 4, pool=3, pos_offset=7)
    assert [len(i) for i in r.idx] == [10, 12]
    assert r.k_hat.shape == (22, d) and r.pos.shape == (22,)
    np.testing.assert_allclose(r.scores.sum(axis=1), w * 2, rtol=1e-12)
    pooled = oracle.maxpool(r.scores, 3)
    for g in range(hkv):
        assert list(r.idx[g]) == list(oracle.select_head(pooled[g], [10, 12][g], 2, 4))


# ---------------------------------------------------------------- 50-digit brute force

@pytest.mark.parametrize("w,hq,hkv,d,s,scale,seed", [
    (1, 1, 1, 8, 2, None, 1), (3, 2, 1, 8, 5, None, 2), (4, 6, 2, 16, 9, 0.37, 3),
    (12, 3, 1, 8, 12, None, 4), (5, 4, 2, 16, 12, 1.9, 5), (7, 3, 3, 8, 11, None, 6),
])
def test_normalizers_and_scores_match_50_digit_brute_force(w, hq, hkv, d, s, scale, seed):
    """O2-O4 written out element by element in 50-digit arithmetic (mpmath):
    each logit is the exact dot product of the decoded bf16 values times the
    scale, the causal row's max and sum of exponentials, and the weights summed
    per key over the window rows and the group's heads. The fp64 oracle agrees
    to 1e-12."""
    mpmath = pytest.importorskip("mpmath")
    mp = mpmath.mp
    mp.dps = 50
    rng = np.random.default_rng(700 + seed)
    qb = f32_to_bf16_bits((rng.standard_normal((w, hq, d)) * 2.0).astype(np.float32))
    kb = f32_to_bf16_bits((rng.standard_normal((s, hkv, d)) * 2.0).astype(np.float32))
    # decode through float32 (a bf16 pattern is the top half of a float32)
    qf = (qb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    kf = (kb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    sc_mp = mp.mpf(1) / mp.sqrt(d) if scale is None else mp.mpf(scale)
    grp = hq // hkv
    want_m = np.empty((hq, w))
    want_z = np.empty((hq, w))
    want_s = [[mp.mpf(0)] * s for _ in range(hkv)]
    for h in range(hq):
        g = h // grp
        for i in range(w):
            p = s - w + i
            logits = [sc_mp * mp.fsum(mp.mpf(qf[i, h, t]) * mp.mpf(kf[j, g, t]) for t in range(d))
                      for j in range(p + 1)]
            m = max(logits)
            e = [mp.exp(x - m) for x in logits]
            z = mp.fsum(e)
            want_m[h, i] = float(m)
            want_z[h, i] = float(z)
            for j in range(p + 1):
                want_s[g][j] += e[j] / z
    q = oracle.bf16_to_f64(qb)
    k = oracle.bf16_to_f64(kb)
    got_m, got_z = oracle.normalizers(q, k, scale)
    got_s = oracle.scores(q, k, scale)
    np.testing.assert_allclose(got_m, want_m, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got_z, want_z, rtol=1e-12)
    np.testing.assert_allclose(got_s, np.array([[float(x) for x in row] for row in want_s]), rtol=1e-12)
