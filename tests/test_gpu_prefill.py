"""GPU parity of the prefill layer pieces (kvc_prefill.h) against the CPU
oracle of the synthetic layer-major chunked prefill (TideKV, Fig. 2 caption).

Each kernel's output is bf16. The oracle computes the operation exactly
(float64) from the same bf16 inputs; the GPU computes it in fp32 (fp64 for
the rotation angles) and rounds once, so every output must lie within one
bf16 ulp (2^-7 relative) of the exact value, measured against a scale that
the operation fixes (the pair norm for the rotation, the weighted value
magnitudes for attention). Attention additionally rounds the softmax weights
to bf16 for the value sum, which adds at most 2^-8 of the weighted |v| sum
(twice: numerator and normaliser). Values that are copied must match bit for
bit, and a chunked attention must equal the one-shot attention bit for bit.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import compression_kvc_score_amd as kvc  # noqa: E402
import oracle  # noqa: E402
from synth import f32_to_bf16_bits  # noqa: E402

from gpu_util import from_dev_bits, to_dev_bf16  # noqa: E402

ULP = 2.0 ** -7


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    kvc.lib()


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def bits(rng, shape, scale=1.0):
    return f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def f64(b):
    return oracle.bf16_to_f64(b)


@pytest.mark.parametrize("rows,dim", [(37, 4096), (1, 64), (5, 200 * 8)])
def test_rmsnorm(rows, dim):
    rng = np.random.default_rng(dim)
    x, w = bits(rng, (rows, dim), 3.0), bits(rng, dim)
    y = torch.empty((rows, dim), dtype=torch.bfloat16, device="cuda")
    xd = to_dev_bf16(x)
    kvc.kvc_rmsnorm(xd, to_dev_bf16(w), y, eps=1e-5)
    torch.cuda.synchronize()
    want = oracle.rmsnorm(f64(x), f64(w), 1e-5)
    got = f64(from_dev_bits(y))
    assert np.all(np.abs(got - want) <= ULP * np.abs(want) + 1e-30)
    assert np.mean(from_dev_bits(y) != oracle.to_bf16_bits(want)) < 0.01   # almost always the nearest bf16
    kvc.kvc_rmsnorm(xd, to_dev_bf16(w), xd, eps=1e-5)                      # in place
    torch.cuda.synchronize()
    np.testing.assert_array_equal(from_dev_bits(xd), from_dev_bits(y))


@pytest.mark.parametrize("hq,hkv,d,c0,n", [(32, 8, 128, 0, 40), (4, 2, 64, 131000, 33), (8, 8, 128, 65500, 36)])
def test_rope_append(hq, hkv, d, c0, n):
    rng = np.random.default_rng(c0 + n)
    s = c0 + n + 7
    base = 500000.0
    pd = kvc.PrefillDesc(s=s, hq=hq, hkv=hkv, d=d, rope_base=base, scale=0.0)
    qkv = bits(rng, (n, (hq + 2 * hkv) * d), 2.0)
    q = torch.empty((n, hq, d), dtype=torch.bfloat16, device="cuda")
    sentinel = 0x7F7F  # a finite bf16 pattern the kernel must leave outside its rows
    kc = torch.full((s, hkv, d), 0, dtype=torch.int16, device="cuda").fill_(sentinel).view(torch.bfloat16)
    vc = torch.full((s, hkv, d), 0, dtype=torch.int16, device="cuda").fill_(sentinel).view(torch.bfloat16)
    kvc.kvc_rope_append(pd, to_dev_bf16(qkv), c0, q, kc, vc)
    torch.cuda.synchronize()
    pos = np.arange(c0, c0 + n)
    x = f64(qkv)
    for name, got, heads, off in [("q", from_dev_bits(q), hq, 0),
                                  ("k", from_dev_bits(kc)[c0:c0 + n], hkv, hq * d)]:
        src = x[:, off:off + heads * d].reshape(n, heads, d)
        want = oracle.rope(src, pos, base)
        norm = np.sqrt(src[..., : d // 2] ** 2 + src[..., d // 2:] ** 2)
        norm = np.concatenate([norm, norm], axis=-1)
        err = np.abs(f64(got) - want)
        assert np.all(err <= ULP * norm + 1e-30), f"{name}: max err/norm {np.max(err / (norm + 1e-30)):.2e}"
    np.testing.assert_array_equal(from_dev_bits(vc)[c0:c0 + n],
                                  qkv[:, (hq + hkv) * d:].reshape(n, hkv, d))
    for t in (kc, vc):
        b = from_dev_bits(t)
        assert np.all(b[:c0] == sentinel) and np.all(b[c0 + n:] == sentinel)


def attention_bound(q, k, v, pos, scale=None):
    """Per element: 2^-7 |o| + 2 * 2^-8 * sum_j p_j |v_j| (+ fp32 noise)."""
    n, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.zeros_like(q)
    j = np.arange(k.shape[0])
    for h in range(hq):
        lg = scale * (q[:, h, :] @ k[:, h // g, :].T)
        lg = np.where(j[None, :] <= pos[:, None], lg, -np.inf)
        p = np.exp(lg - lg.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ np.abs(v[:, h // g, :])
    return out


@pytest.mark.parametrize("hq,hkv,d,c0,n,s", [
    (32, 8, 128, 0, 64, 64),         # one-shot, two query tiles
    (32, 8, 128, 200, 77, 300),      # mid-prompt chunk, ragged tile, unaligned start
    (4, 1, 64, 1000, 40, 1040),      # G = 4, d = 64
    (2, 2, 128, 5, 3, 8),            # G = 1, tiny
    (16, 8, 64, 33, 64, 97),         # G = 2
    (8, 1, 128, 96, 32, 128),        # G = 8
])
def test_chunk_attention_matches_oracle(hq, hkv, d, c0, n, s):
    rng = np.random.default_rng(s + n)
    pd = kvc.PrefillDesc(s=s, hq=hq, hkv=hkv, d=d, rope_base=10000.0, scale=0.0)
    q = bits(rng, (n, hq, d), 1.5)
    k = bits(rng, (s, hkv, d), 1.5)
    v = bits(rng, (s, hkv, d))
    k[c0 + n:] = f32_to_bf16_bits(np.full((s - c0 - n, hkv, d), 1.0e4, np.float32))  # unwritten rows: never read
    o = torch.empty((n, hq, d), dtype=torch.bfloat16, device="cuda")
    kvc.kvc_chunk_attention(pd, to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), c0, o)
    torch.cuda.synchronize()
    pos = np.arange(c0, c0 + n)
    kk, vv = f64(k)[: c0 + n], f64(v)[: c0 + n]
    want = oracle.attention(f64(q), kk, vv, pos)
    bound = ULP * np.abs(want) + 2 * 2.0 ** -8 * attention_bound(f64(q), kk, vv, pos) + 1e-6
    err = np.abs(f64(from_dev_bits(o)) - want)
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3f}"


def test_chunked_attention_equals_one_shot_bitwise():
    rng = np.random.default_rng(11)
    hq, hkv, d, s = 32, 8, 128, 520
    pd = kvc.PrefillDesc(s=s, hq=hq, hkv=hkv, d=d, rope_base=10000.0, scale=0.0)
    q = to_dev_bf16(bits(rng, (s, hq, d), 2.0))
    k = to_dev_bf16(bits(rng, (s, hkv, d), 2.0))
    v = to_dev_bf16(bits(rng, (s, hkv, d)))
    one = torch.empty((s, hq, d), dtype=torch.bfloat16, device="cuda")
    kvc.kvc_chunk_attention(pd, q, k, v, 0, one)
    for chunk in (128, 100, 7):
        got = torch.empty_like(one)
        for c0 in range(0, s, chunk):
            c1 = min(c0 + chunk, s)
            out = torch.empty((c1 - c0, hq, d), dtype=torch.bfloat16, device="cuda")
            kvc.kvc_chunk_attention(pd, q[c0:c1].contiguous(), k, v, c0, out)
            got[c0:c1] = out
        torch.cuda.synchronize()
        np.testing.assert_array_equal(from_dev_bits(got), from_dev_bits(one), err_msg=f"chunk {chunk}")


def test_swiglu():
    rng = np.random.default_rng(12)
    rows, ffn = 19, 14336 // 8
    gu = bits(rng, (rows, 2 * ffn), 3.0)
    a = torch.empty((rows, ffn), dtype=torch.bfloat16, device="cuda")
    kvc.kvc_swiglu(to_dev_bf16(gu), a)
    torch.cuda.synchronize()
    want = oracle.swiglu(f64(gu))
    err = np.abs(f64(from_dev_bits(a)) - want)
    assert np.all(err <= ULP * np.abs(want) + 1e-30)
