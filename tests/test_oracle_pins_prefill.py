"""Pins for the oracle of the synthetic layer-major chunked prefill (TideKV,
Fig. 2 caption; Fig. 1 caption, schedule (d)): each part checked against a
closed form, an invariant, a library routine or brute force, chosen so that a
plausible slip (a wrong pairing in the rotation, a transposed operand, a
missed causal mask, a wrong GQA head map, a chunk attending to the wrong keys)
fails one of them."""
import numpy as np
import pytest
import scipy.special

import oracle
from synth import f32_to_bf16_bits


def test_bf16_rounding_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9, 3.0e38, 0.0])
    got = oracle.bf16_to_f64(oracle.to_bf16_bits(x))
    np.testing.assert_array_equal(got, [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0, oracle.bf16_to_f64(
        oracle.to_bf16_bits(np.array([3.0e38])))[0], 0.0])
    assert got[1] == 1.0          # halfway between 1 and 1 + 2^-7: to even
    assert got[2] == 1.0 + 2 ** -6  # halfway between 1 + 2^-7 and 1 + 2^-6: to even (the latter)
    rng = np.random.default_rng(0)
    y = rng.standard_normal(1000).astype(np.float32)
    np.testing.assert_array_equal(oracle.to_bf16_bits(y.astype(np.float64)), f32_to_bf16_bits(y))


def test_rmsnorm_closed_forms():
    x = np.full((1, 8), 3.0)
    w = np.arange(1, 9, dtype=np.float64)
    np.testing.assert_allclose(oracle.rmsnorm(x, w, 0.0), w[None, :], rtol=1e-15)
    np.testing.assert_allclose(oracle.rmsnorm(x, w, 7.0), 3.0 / 4.0 * w[None, :], rtol=1e-15)
    rng = np.random.default_rng(1)
    z = rng.standard_normal((5, 16))
    y = oracle.rmsnorm(z, np.ones(16), 0.0)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(oracle.rmsnorm(4.0 * z, np.ones(16), 0.0), y, rtol=1e-13)


def test_rope_rotation_properties():
    rng = np.random.default_rng(2)
    d, base = 16, 10000.0
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    # position 0 is the identity; norms of each (i, i + D/2) pair are kept
    np.testing.assert_allclose(oracle.rope(q, np.array([0]), base), q, rtol=0, atol=0)
    r = oracle.rope(q, np.array([37]), base)
    pair = lambda a: a[..., : d // 2] ** 2 + a[..., d // 2:] ** 2  # noqa: E731
    np.testing.assert_allclose(pair(r), pair(q), rtol=1e-13)
    # scores depend on the relative position only
    for m, n in [(5, 2), (100, 40), (7, 7)]:
        a = np.sum(oracle.rope(q, np.array([m]), base) * oracle.rope(k, np.array([n]), base))
        b = np.sum(oracle.rope(q, np.array([m - n]), base) * k)
        assert a == pytest.approx(b, rel=1e-11, abs=1e-12)
    # pair 0 turns by exactly p radians (base^0 = 1), as a 2-D rotation
    e = np.zeros((1, 1, d))
    e[0, 0, 0] = 1.0
    r = oracle.rope(e, np.array([2]), base)
    assert r[0, 0, 0] == pytest.approx(np.cos(2.0)) and r[0, 0, d // 2] == pytest.approx(np.sin(2.0))
    # the last pair turns by p * base^(-(D-2)/D)
    e = np.zeros((1, 1, d))
    e[0, 0, d // 2 - 1] = 1.0
    ang = 3 * base ** (-(d - 2) / d)
    r = oracle.rope(e, np.array([3]), base)
    assert r[0, 0, d // 2 - 1] == pytest.approx(np.cos(ang)) and r[0, 0, d - 1] == pytest.approx(np.sin(ang))


def test_attention_against_brute_force():
    rng = np.random.default_rng(3)
    n, hq, hkv, d, t = 5, 4, 2, 8, 9
    q = rng.standard_normal((n, hq, d))
    k = rng.standard_normal((t, hkv, d))
    v = rng.standard_normal((t, hkv, d))
    pos = np.array([4, 5, 6, 7, 8])
    got = oracle.attention(q, k, v, pos)
    for i in range(n):
        for h in range(hq):
            g = h // 2
            logits = np.array([q[i, h] @ k[j, g] / np.sqrt(d) for j in range(pos[i] + 1)])
            p = scipy.special.softmax(logits)
            want = sum(p[j] * v[j, g] for j in range(pos[i] + 1))
            np.testing.assert_allclose(got[i, h], want, rtol=1e-12, atol=1e-14)


def test_attention_closed_forms():
    rng = np.random.default_rng(4)
    d = 8
    v = rng.standard_normal((6, 1, d))
    k = np.zeros((6, 1, d))       # equal logits: the mean of the visible values
    q = rng.standard_normal((3, 1, d))
    got = oracle.attention(q, k, v, np.array([0, 2, 5]))
    np.testing.assert_allclose(got[0, 0], v[0, 0], rtol=1e-15)   # position 0 sees key 0 only
    np.testing.assert_allclose(got[1, 0], v[:3, 0].mean(axis=0), rtol=1e-13)
    np.testing.assert_allclose(got[2, 0], v[:, 0].mean(axis=0), rtol=1e-13)
    # GQA: a one-hot key per KV head picks out that head's value
    hq, hkv = 4, 2
    k = np.zeros((2, hkv, d))
    v = np.zeros((2, hkv, d))
    k[1, 0, 0], k[1, 1, 1] = 50.0, 50.0
    v[1, 0, :], v[1, 1, :] = 1.0, 2.0
    q = np.zeros((1, hq, d))
    q[0, :2, 0] = 1.0   # heads 0, 1 (KV head 0) match key 1 of head 0
    q[0, 2:, 1] = 1.0   # heads 2, 3 (KV head 1) match key 1 of head 1
    got = oracle.attention(q, k, v, np.array([1]))
    np.testing.assert_allclose(got[0, :2, 0], 1.0, rtol=1e-6)
    np.testing.assert_allclose(got[0, 2:, 0], 2.0, rtol=1e-6)


def test_swiglu_against_scipy():
    rng = np.random.default_rng(5)
    gu = rng.standard_normal((4, 12)) * 4
    want = gu[:, :6] * scipy.special.expit(gu[:, :6]) * gu[:, 6:]
    np.testing.assert_allclose(oracle.swiglu(gu), want, rtol=1e-13)


def small_model(seed=6, layers=2, hidden=64, hq=4, hkv=2, d=16, ffn=96):
    rng = np.random.default_rng(seed)
    shp = oracle.ModelShape(hidden=hidden, hq=hq, hkv=hkv, d=d, ffn=ffn, rope_base=10000.0)

    def b(shape, scale):
        return f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))

    ws = [oracle.LayerWeights(w_attn=b(hidden, 0.1) + 0, w_qkv=b(((hq + 2 * hkv) * d, hidden), hidden ** -0.5),
                              w_o=b((hidden, hq * d), (hq * d) ** -0.5), w_mlp=b(hidden, 0.1),
                              w_gu=b((2 * ffn, hidden), hidden ** -0.5), w_down=b((hidden, ffn), ffn ** -0.5))
          for _ in range(layers)]
    for w in ws:  # norm weights around 1
        w.w_attn = f32_to_bf16_bits((1.0 + oracle.bf16_to_f64(w.w_attn)).astype(np.float32))
        w.w_mlp = f32_to_bf16_bits((1.0 + oracle.bf16_to_f64(w.w_mlp)).astype(np.float32))
    return shp, ws


@pytest.mark.parametrize("emulate", [False, True])
def test_chunked_layer_major_equals_one_shot(emulate):
    """Chunk j attends to the K/V of chunks 0..j: chunking the prompt does not
    change the result (exactly, up to float64 summation order)."""
    shp, ws = small_model()
    rng = np.random.default_rng(7)
    s, w = 48, 4
    x = f32_to_bf16_bits(rng.standard_normal((s, shp.hidden)).astype(np.float32))
    one = oracle.prefill_layer_major(x, ws, shp, s, w, [12, 12], 2, 4, emulate_bf16=emulate)
    for chunk in (8, 20):
        got = oracle.prefill_layer_major(x, ws, shp, chunk, w, [12, 12], 2, 4, emulate_bf16=emulate)
        if emulate:
            # bf16 rounding amplifies last-bit differences of the summation
            # order only rarely; compare values with one bf16 ulp of slack
            np.testing.assert_allclose(got.hidden, one.hidden, rtol=2 ** -7, atol=1e-6)
        else:
            np.testing.assert_allclose(got.hidden, one.hidden, rtol=1e-11, atol=1e-12)
            for l in range(len(ws)):
                np.testing.assert_allclose(got.k[l], one.k[l], rtol=1e-11, atol=1e-12)
                np.testing.assert_allclose(got.q_win[l], one.q_win[l], rtol=1e-11, atol=1e-12)


def test_layer_by_hand_for_one_token():
    """One token at position 0: attention returns its own value row, so the
    layer reduces to x + v-path and the MLP, written out here directly."""
    shp, ws = small_model(layers=1)
    rng = np.random.default_rng(8)
    x = oracle.bf16_to_f64(f32_to_bf16_bits(rng.standard_normal((1, shp.hidden)).astype(np.float32)))
    wt = ws[0]
    f = oracle.bf16_to_f64
    kc = np.zeros((1, shp.hkv, shp.d))
    vc = np.zeros((1, shp.hkv, shp.d))
    out, q = oracle.layer_chunk(x, wt, shp, 0, kc, vc, emulate_bf16=False)
    xn = x / np.sqrt(np.mean(x * x) + shp.eps) * f(wt.w_attn)
    qkv = xn @ f(wt.w_qkv).T
    v = qkv[0, (shp.hq + shp.hkv) * shp.d:].reshape(shp.hkv, shp.d)
    o = np.concatenate([v[h // (shp.hq // shp.hkv)] for h in range(shp.hq)])  # each query head copies its KV head's v
    h = x + o @ f(wt.w_o).T
    hn = h / np.sqrt(np.mean(h * h) + shp.eps) * f(wt.w_mlp)
    gu = hn @ f(wt.w_gu).T
    g, u = gu[0, :shp.ffn], gu[0, shp.ffn:]
    want = h + (g * scipy.special.expit(g) * u) @ f(wt.w_down).T
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(q[0], qkv[0, :shp.hq * shp.d].reshape(shp.hq, shp.d), rtol=1e-14)  # rope at 0


def test_layer_end_compression_and_window():
    shp, ws = small_model()
    rng = np.random.default_rng(9)
    s, w, chunk = 40, 6, 16
    x = f32_to_bf16_bits(rng.standard_normal((s, shp.hidden)).astype(np.float32))
    res = oracle.prefill_layer_major(x, ws, shp, chunk, w, [10, 14], 2, 4)
    for l in range(len(ws)):
        want = oracle.compress_layer(oracle.to_bf16_bits(res.q_win[l]), oracle.to_bf16_bits(res.k[l]),
                                     oracle.to_bf16_bits(res.v[l]), [10, 14], 2, 4)
        for a, b in zip(res.retained[l].idx, want.idx):
            np.testing.assert_array_equal(a, b)
        assert [len(i) for i in res.retained[l].idx] == [10, 14]
    # the window queries are the last w rows' rotated queries of each layer:
    # recompute the last layer's from its input bridge
    one = oracle.prefill_layer_major(x, ws[:1], shp, chunk, w, [10, 14], 2, 4, compress=False)
    kc = np.zeros((s, shp.hkv, shp.d))
    vc = np.zeros((s, shp.hkv, shp.d))
    _, q = oracle.layer_chunk(one.hidden, ws[1], shp, 0, kc, vc)
    np.testing.assert_allclose(res.q_win[1], q[s - w:], rtol=2 ** -7, atol=1e-6)
