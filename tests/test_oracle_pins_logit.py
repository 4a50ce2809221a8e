"""Pins for the oracle's other score modes: the raw inner-product ranking
(HillInfer, Algorithmic Simplification), its INT8 form (HillInfer, Streaming
Execution and Asymmetric Precision) and the overlap coefficient (HeteroCache
summary, Key Contributions item 1). Each test checks the oracle against
something other than itself: a different route to the same number, an exact
special case, a textbook identity or brute force on tiny inputs.
"""
import numpy as np
import pytest

import oracle
from synth import f32_to_bf16_bits


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


# ---------------------------------------------------------------- logit scores

@pytest.mark.parametrize("w,hq,hkv,d,s", [(1, 1, 1, 8, 9), (4, 4, 2, 16, 20), (6, 6, 3, 8, 11)])
def test_logit_scores_equal_pooled_query_dot(w, hq, hkv, d, s):
    """Summing logits over rows equals one dot product with the summed query
    of the rows that see the key (computed here row set by row set)."""
    rng = np.random.default_rng(s)
    q = rng.standard_normal((w, hq, d))
    k = rng.standard_normal((s, hkv, d))
    got = oracle.logit_scores(q, k)
    grp = hq // hkv
    for g in range(hkv):
        for j in range(s):
            first = max(0, j - (s - w))   # rows i with S-W+i >= j
            qbar = q[first:, g * grp:(g + 1) * grp, :].sum(axis=(0, 1))
            assert got[g, j] == pytest.approx(float(qbar @ k[j, g]), rel=1e-12, abs=1e-12)


def test_logit_single_row_is_the_raw_inner_product_and_ranks_like_softmax():
    """One query row: the score is q.k (no scale), and ranking by it equals
    ranking by the softmax weight (the page's monotonicity argument)."""
    rng = np.random.default_rng(3)
    d, s = 16, 40
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((s, 1, d))
    raw = oracle.logit_scores(q, k)[0]
    np.testing.assert_allclose(raw, k[:, 0, :] @ q[0, 0], rtol=1e-13)
    soft = oracle.scores(q, k)[0]
    for budget in (5, 12, 40):
        np.testing.assert_array_equal(oracle.select_head(raw, budget, 1, 1),
                                      oracle.select_head(soft, budget, 1, 1))


def test_logit_integer_inputs_brute_force():
    """Small integer inputs: every product and sum is exact, so the oracle must
    equal a pure-Python integer brute force over (row, head, key)."""
    rng = np.random.default_rng(5)
    w, hq, hkv, d, s = 3, 4, 2, 5, 7
    q = rng.integers(-4, 5, size=(w, hq, d))
    k = rng.integers(-4, 5, size=(s, hkv, d))
    got = oracle.logit_scores(q.astype(np.float64), k.astype(np.float64))
    grp = hq // hkv
    for g in range(hkv):
        for j in range(s):
            tot = 0
            for i in range(w):
                if j > s - w + i:
                    continue
                for h in range(g * grp, (g + 1) * grp):
                    tot += sum(int(q[i, h, c]) * int(k[j, g, c]) for c in range(d))
            assert got[g, j] == tot


def test_logit_last_key_seen_by_last_row_only():
    rng = np.random.default_rng(6)
    w, hq, hkv, d, s = 5, 2, 1, 8, 12
    q = rng.standard_normal((w, hq, d))
    k = rng.standard_normal((s, hkv, d))
    got = oracle.logit_scores(q, k)[0]
    assert got[s - 1] == pytest.approx(float(q[w - 1].sum(axis=0) @ k[s - 1, 0]), rel=1e-12)
    assert got[0] == pytest.approx(float(q.sum(axis=(0, 1)) @ k[0, 0]), rel=1e-12)


def test_first_visible_row():
    np.testing.assert_array_equal(oracle.first_visible_row(6, 3), [0, 0, 0, 0, 1, 2])


# ---------------------------------------------------------------- INT8 quantisation

def test_quantize_exact_on_scaled_integer_vectors():
    """Codes times a power of two, the largest |code| 127: quantisation
    recovers the codes and the step exactly."""
    codes = np.array([[127, -64, 3, 0, -127, 55], [-127, 1, 2, 3, 4, 5]], dtype=np.int32)
    for e in (-9, 0, 4):
        x = (codes * 2.0 ** e).astype(np.float32)
        got, step = oracle.quantize_int8(x)
        np.testing.assert_array_equal(got, codes)
        np.testing.assert_array_equal(step, np.float32(2.0 ** e))


def test_quantize_rounds_half_to_even_and_is_odd_symmetric():
    x = np.array([[254.0, 1.0, 3.0, 5.0, -1.0, -3.0]], dtype=np.float32)  # 127/254 = 0.5 exactly
    got, step = oracle.quantize_int8(x)
    np.testing.assert_array_equal(got, [[127, 0, 2, 2, 0, -2]])
    assert step[0] == np.float32(2.0)
    rng = np.random.default_rng(8)
    y = rng.standard_normal((20, 32)).astype(np.float32)
    a, sa = oracle.quantize_int8(y)
    b, sb = oracle.quantize_int8(-y)
    np.testing.assert_array_equal(a, -b)
    np.testing.assert_array_equal(sa, sb)
    assert np.all(np.abs(a).max(axis=1) == 127)
    assert np.all(np.abs(a) <= 127)


def test_quantize_zero_vector():
    got, step = oracle.quantize_int8(np.zeros((2, 4), dtype=np.float32))
    assert not got.any() and not step.any()


def test_int8_scores_equal_logit_scores_when_quantisation_is_exact():
    """One query row (so the pooled query is that row) and every vector a
    power-of-two multiple of integer codes with max |code| 127: the INT8 path
    loses nothing and equals the exact logit score."""
    rng = np.random.default_rng(9)
    d, s = 16, 24

    def vec(e):
        c = rng.integers(-127, 128, size=d)
        c[rng.integers(0, d)] = 127 * (1 if rng.random() < 0.5 else -1)
        return c * 2.0 ** e

    q = np.array([[vec(-5)]], dtype=np.float64)                     # [1, 1, D]
    k = np.array([[vec(int(rng.integers(-8, 0)))] for _ in range(s)])  # [S, 1, D]
    got = oracle.logit_scores_int8(bf16(q), bf16(k))
    want = oracle.logit_scores(q, k)
    np.testing.assert_array_equal(got.astype(np.float64), want)


def test_int8_scores_close_to_logit_scores_on_random_data():
    """Each code is within half a step of the scaled value, which bounds the
    INT8 score's distance from the exact logit score."""
    rng = np.random.default_rng(10)
    w, hq, hkv, d, s = 4, 4, 2, 32, 30
    qb = bf16(rng.standard_normal((w, hq, d)))
    kb = bf16(rng.standard_normal((s, hkv, d)))
    q, k = oracle.bf16_to_f64(qb), oracle.bf16_to_f64(kb)
    got = oracle.logit_scores_int8(qb, kb).astype(np.float64)
    want = oracle.logit_scores(q, k)
    t_of = oracle.first_visible_row(s, w)
    grp = hq // hkv
    for g in range(hkv):
        for j in range(s):
            qbar = q[t_of[j]:, g * grp:(g + 1) * grp, :].sum(axis=(0, 1))
            hq_, hk_ = np.abs(qbar).max() / 254, np.abs(k[j, g]).max() / 254
            bound = (hq_ * np.abs(k[j, g]).sum() + hk_ * np.abs(qbar).sum() + d * hq_ * hk_) * 1.01 + 1e-6
            assert abs(got[g, j] - want[g, j]) <= bound


def test_pooled_query_is_the_exact_sum_rounded_once():
    rng = np.random.default_rng(11)
    qb = bf16(rng.standard_normal((5, 4, 8)))
    q = oracle.bf16_to_f64(qb)
    got = oracle.pooled_query(qb, 2, 2)
    want = np.stack([q[2:, 0:2, :].sum(axis=(0, 1)), q[2:, 2:4, :].sum(axis=(0, 1))]).astype(np.float32)
    np.testing.assert_array_equal(got, want)  # 6 bf16 terms: the float64 sum is exact


# ---------------------------------------------------------------- overlap coefficient

def test_overlap_coefficient_textbook_cases():
    assert oracle.overlap_coefficient([1, 2, 3, 4], [3, 4, 5]) == pytest.approx(2 / 3)
    assert oracle.overlap_coefficient([1, 2], [1, 2, 3, 4]) == 1.0   # a subset
    assert oracle.overlap_coefficient([1, 2], [3, 4]) == 0.0
    assert oracle.overlap_coefficient([5, 6, 7], [7, 6, 5]) == 1.0
    assert oracle.overlap_coefficient([], [1]) == 1.0


def test_compress_layer_score_modes_compose_the_steps():
    rng = np.random.default_rng(12)
    w, hq, hkv, d, s = 4, 4, 2, 16, 40
    qb = bf16(rng.standard_normal((w, hq, d)))
    kb = bf16(rng.standard_normal((s, hkv, d)))
    vb = bf16(rng.standard_normal((s, hkv, d)))
    for mode, fn in [("logit", lambda: oracle.logit_scores(oracle.bf16_to_f64(qb), oracle.bf16_to_f64(kb))),
                     ("int8", lambda: oracle.logit_scores_int8(qb, kb).astype(np.float64))]:
        r = oracle.compress_layer(qb, kb, vb, [10, 12], 2, 4, pool=3, score_mode=mode)
        assert r.m is None and r.z is None
        np.testing.assert_array_equal(r.scores, fn())
        want = oracle.select(oracle.maxpool(r.scores, 3), [10, 12], 2, 4)
        for a, b in zip(r.idx, want):
            np.testing.assert_array_equal(a, b)
    with pytest.raises(ValueError):
        oracle.compress_layer(qb, kb, vb, [10, 12], 2, 4, score_mode="nope")
