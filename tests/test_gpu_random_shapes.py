"""Seeded sweep of random layer shapes through kvc_compress_layer, each
checked against the CPU oracle like the fixed edge cases: normalisers and
scores within their tolerances, the retained set exact outside the score tie
band, an exact top-k of the GPU's own values on every head, and the gathered
rows and positions bit for bit (TideKV, Fig. 3 caption: two-pass scoring,
top-k with mandatory keys, gather).

The shapes cover both scan designs (query rows per KV head up to 128 and up
to 256), D 64 and 128, head groups 1 to 8, short prompts against long
windows, any mandatory set, per-head budgets from below the prompt to above
it, and max-pooling. The list is drawn once from a fixed seed."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import compression_kvc_score_amd as kvc  # noqa: E402
from synth import get_config, layer_inputs  # noqa: E402

from gpu_util import desc_from, run_fused  # noqa: E402
from test_gpu_parity import check_layer, dev_inputs  # noqa: E402


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    kvc.lib()


def random_cases(n=40, seed=20261202):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2, 3, 4, 8]))
        if len(cases) % 4 == 3:  # every fourth case: more than 128 query rows per KV head
            w, g = [(32, 5), (32, 8), (64, 3), (64, 4), (48, 5)][int(rng.integers(0, 5))]
        else:
            g = int(rng.choice([1, 2, 3, 4, 5, 8]))
            w = int(rng.choice([1, 3, 8, 16, 32, 64]))
        if g * w > 256:
            continue
        s = int(rng.integers(w, 9000))
        n_sink = int(rng.integers(0, 9))
        n_recent = int(rng.integers(0, 65))
        n_mand = min(n_sink, s) + (s - max(s - n_recent, min(n_sink, s)))
        lo = max(n_mand, 1)
        budgets = [int(rng.integers(lo, s + 40)) for _ in range(hkv)]
        cases.append(dict(
            s=s, w=w, hq=g * hkv, hkv=hkv, d=d, block=int(32 * rng.integers(1, 17)),
            n_sink=n_sink, n_recent=n_recent, n_heavy=int(rng.integers(0, 1 + s // 200)),
            pool=int(rng.choice([1, 1, 1, 3, 7])), budgets=budgets, seed=int(rng.integers(1, 1 << 30))))
    return cases


CASES = random_cases()


def _case_cfg(i):
    c = dict(CASES[i])
    budgets = np.asarray(c.pop("budgets"), dtype=np.int64)
    seed = c.pop("seed")
    cfg = get_config("tiny").with_(name=f"random_{i}", sink_scale=4.0, seed_base=seed, budget=int(budgets[0]), **c)
    return cfg, budgets, seed


@pytest.mark.parametrize("i", range(len(CASES)))
def test_random_shape(i):
    cfg, budgets, _ = _case_cfg(i)
    print(f"random shape {i}: s={cfg.s} w={cfg.w} hq={cfg.hq} hkv={cfg.hkv} d={cfg.d} block={cfg.block} "
          f"sink={cfg.n_sink} recent={cfg.n_recent} pool={cfg.pool} budgets={list(budgets)}", flush=True, file=sys.stderr)
    x = layer_inputs(cfg, 0)
    q, k, v = dev_inputs(x)
    desc = desc_from(cfg, q, k, v)
    got = run_fused(desc, q, k, v, budgets)
    check_layer(x, got, budgets)



@pytest.mark.parametrize("i", range(0, len(CASES), 3))
def test_random_shape_strided_offset_and_staged(i):
    """The same layer read through strided views (K, V and Q_win embedded
    among other heads) with a position offset: the staged calls equal the
    whole-layer call bit for bit, and both equal the contiguous run with the
    positions shifted by the offset."""
    from gpu_util import from_dev_bits, run_staged, to_dev_bf16
    cfg, budgets, seed = _case_cfg(i)
    x = layer_inputs(cfg, 0)
    q, k, v = dev_inputs(x)
    base = run_fused(desc_from(cfg, q, k, v), q, k, v, budgets)
    rng = np.random.default_rng(seed)
    pos_offset = int(rng.integers(0, 1 << 20))
    g = cfg.group
    kb = torch.zeros((cfg.s, cfg.hkv + 2, cfg.d), dtype=torch.bfloat16, device="cuda")
    vb = torch.zeros_like(kb)
    qb = torch.zeros((cfg.w, cfg.hq + g, cfg.d), dtype=torch.bfloat16, device="cuda")
    kb[:, 1:1 + cfg.hkv] = k
    vb[:, 1:1 + cfg.hkv] = v
    qb[:, g:g + cfg.hq] = q
    ks, vs, qs = kb[:, 1:1 + cfg.hkv], vb[:, 1:1 + cfg.hkv], qb[:, g:g + cfg.hq]
    desc = desc_from(cfg, qs, ks, vs, pos_offset=pos_offset)
    print(f"strided case {i}: pos_offset={pos_offset}", flush=True, file=sys.stderr)
    fu = run_fused(desc, qs, ks, vs, budgets)
    st = run_staged(desc, qs, ks, vs, budgets)
    for key in ["m", "z", "scores", "idx", "k_hat", "v_hat", "pos"]:
        np.testing.assert_array_equal(fu[key], st[key], err_msg=f"staged != whole layer: {key}")
    for key in ["m", "z", "scores", "idx", "k_hat", "v_hat"]:
        np.testing.assert_array_equal(fu[key], base[key], err_msg=f"strided != contiguous: {key}")
    np.testing.assert_array_equal(fu["pos"], base["pos"] + pos_offset)


@pytest.mark.parametrize("mode", ["logit", "int8"])
@pytest.mark.parametrize("i", range(1, len(CASES), 3))
def test_random_shape_score_modes(i, mode):
    """The raw inner-product modes on the random shapes: whole layer equal to
    the staged calls, INT8 scores and selection exactly the oracle's, fp32
    scores within their rounding bound and the selection exact outside it,
    the gather bit for bit."""
    from gpu_util import split_heads
    from test_gpu_score_modes import MODES, check_selection_signed, logit_error_bound, run_staged_modes
    import oracle
    cfg, budgets, _ = _case_cfg(i)
    if cfg.s > (1 << 22):
        pytest.skip("raw modes take at most 2^22 keys")
    x = layer_inputs(cfg, 0)
    q, k, v = dev_inputs(x)
    desc = desc_from(cfg, q, k, v, score_mode=MODES[mode])
    print(f"score mode {mode} case {i}", flush=True, file=sys.stderr)
    fu = run_fused(desc, q, k, v, budgets)
    st = run_staged_modes(desc, q, k, v, budgets)
    for key in ["scores", "idx", "k_hat", "v_hat", "pos"]:
        np.testing.assert_array_equal(fu[key], st[key], err_msg=f"fused != staged: {key}")
    pool = cfg.pool
    if mode == "int8":
        want = oracle.logit_scores_int8(x.q, x.k)
        np.testing.assert_array_equal(fu["scores"], want)
        vals = oracle.maxpool(want.astype(np.float64), pool) if pool > 1 else want.astype(np.float64)
        want_idx = oracle.select(vals, budgets, cfg.n_sink, cfg.n_recent)
        np.testing.assert_array_equal(fu["idx"], np.concatenate(want_idx))
    else:
        want = oracle.logit_scores(oracle.bf16_to_f64(x.q), oracle.bf16_to_f64(x.k))
        err = logit_error_bound(x.q, x.k)
        assert np.all(np.abs(fu["scores"] - want) <= err)
        check_selection_signed(fu["idx"], fu["scores"], want, err, budgets, cfg.n_sink, cfg.n_recent, pool=pool)
    idx = split_heads(fu["idx"], fu["offsets"])
    k_hat, v_hat, pos = oracle.gather(x.k, x.v, idx)
    np.testing.assert_array_equal(fu["k_hat"], k_hat)
    np.testing.assert_array_equal(fu["v_hat"], v_hat)
    np.testing.assert_array_equal(fu["pos"], pos)


def random_long_cases(n=12, seed=20261205):
    """Long prompts (20K-300K keys): several selection chunks per head, both
    scan designs (up to 256 query rows per KV head), pooling, per-head budgets
    up to 20K."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2, 4, 8]))
        g = int(rng.choice([1, 2, 4, 5, 8]))
        w = int(rng.choice([8, 16, 32, 64]))
        if g * w > 256:
            continue
        s = int(rng.integers(20000, 300000))
        n_sink = int(rng.integers(0, 9))
        n_recent = int(rng.integers(0, 65))
        n_mand = min(n_sink, s) + (s - max(s - n_recent, min(n_sink, s)))
        budgets = [int(rng.integers(max(n_mand, 1), 20000)) for _ in range(hkv)]
        cases.append(dict(s=s, w=w, hq=g * hkv, hkv=hkv, d=d, block=int(64 * rng.integers(1, 9)),
                          n_sink=n_sink, n_recent=n_recent, n_heavy=int(rng.integers(0, 1 + s // 200)),
                          pool=int(rng.choice([1, 1, 3, 7])), budgets=budgets, seed=int(rng.integers(1, 1 << 30))))
    return cases


LONG = random_long_cases()


@pytest.mark.parametrize("i", range(len(LONG)))
def test_random_long_prompt(i):
    """A long random prompt through the whole-layer call against the oracle
    on its first and last KV head (the fp64 dense softmax over every key);
    where the plan allows the fused-selection flag, the flagged call's
    retained set and rows equal the staged selection of its own scores bit
    for bit and pass the same oracle check."""
    from test_gpu_parity import _fused_select_run, _staged_select
    c = dict(LONG[i])
    budgets = np.asarray(c.pop("budgets"), dtype=np.int64)
    seed = c.pop("seed")
    cfg = get_config("tiny").with_(name=f"random_long_{i}", sink_scale=4.0, seed_base=seed, budget=int(budgets[0]), **c)
    print(f"long prompt {i}: s={cfg.s} w={cfg.w} hq={cfg.hq} hkv={cfg.hkv} d={cfg.d} block={cfg.block} "
          f"sink={cfg.n_sink} recent={cfg.n_recent} pool={cfg.pool} budgets={list(budgets)}", flush=True, file=sys.stderr)
    x = layer_inputs(cfg, 0)
    q, k, v = dev_inputs(x)
    heads = sorted({0, cfg.hkv - 1})
    desc = desc_from(cfg, q, k, v)
    check_layer(x, run_fused(desc, q, k, v, budgets), budgets, heads=heads)
    if cfg.pool != 1:
        return
    fdesc = desc_from(cfg, q, k, v, flags=kvc.KVC_FLAG_FUSED_SELECT)
    try:
        plan = kvc.kvc_plan_layer(fdesc)
    except RuntimeError:
        return  # the flag does not take this shape (the host says why)
    if plan.fused_select != 1:
        return
    got, out = _fused_select_run(fdesc, q, k, v, budgets)
    sel = _staged_select(desc, q, k, v, out.scores, budgets)
    for key in ["idx", "k_hat", "v_hat", "pos"]:
        np.testing.assert_array_equal(got[key], sel[key], err_msg=f"fused selection: {key}")
    check_layer(x, got, budgets, heads=heads)


def random_chunked_cases(n=10, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        d = int(rng.choice([64, 128]))
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 4, 5]))
        w = int(rng.choice([2, 8, 16, 32]))
        s = int(rng.integers(4 * w, 5000))
        chunk = int(rng.integers(w, max(w + 1, s // 2)))
        if s - ((s - 1) // chunk) * chunk < w:  # the last chunk must hold a window
            continue
        n_sink = int(rng.integers(0, 5))
        n_recent = int(rng.integers(0, w + 1))
        budget = int(rng.integers(max(n_sink + n_recent, 1), max(n_sink + n_recent + 2, s // 2)))
        cases.append(dict(s=s, w=w, hq=g * hkv, hkv=hkv, d=d, block=128, n_sink=n_sink, n_recent=n_recent,
                          n_heavy=int(rng.integers(0, 1 + s // 200)), chunk=chunk, budget=budget,
                          pool=int(rng.choice([1, 1, 3])), pos_offset=int(rng.integers(0, 1 << 16)),
                          mode=str(rng.choice(["softmax", "softmax", "logit", "int8"])),
                          seed=int(rng.integers(1, 1 << 30))))
    return cases


CHUNKED = random_chunked_cases()


@pytest.mark.parametrize("i", range(len(CHUNKED)))
def test_random_immediate_eviction(i):
    """Immediate (chunk-boundary) eviction on random shapes: every boundary
    checked on the GPU's own state against the oracle, the whole-prompt call
    equal to the boundary chain, and the final cache equal to the oracle's
    chunked compressor when no boundary decision fell inside a tie band."""
    from test_gpu_chunked import check_case
    c = dict(CHUNKED[i])
    budget, pool, pos_offset, mode, seed = c.pop("budget"), c.pop("pool"), c.pop("pos_offset"), c.pop("mode"), c.pop("seed")
    cfg = get_config("tiny").with_(name=f"random_chunked_{i}", sink_scale=4.0, seed_base=seed, budget=budget, **c)
    check_case(cfg, budget, mode=mode, pool=pool, pos_offset=pos_offset)


def random_attention_cases(n=10, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        g = int(rng.choice([1, 2, 4, 8]))
        hkv = int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128]))
        c0 = int(rng.integers(0, 3000))
        n_q = int(rng.integers(1, 300))
        s = c0 + n_q + int(rng.integers(0, 50))
        out.append((g * hkv, hkv, d, c0, n_q, s, int(rng.integers(1, 1 << 30))))
    return out


@pytest.mark.parametrize("hq,hkv,d,c0,n,s,seed", random_attention_cases())
def test_random_chunk_attention(hq, hkv, d, c0, n, s, seed):
    """Causal GQA chunk attention on random shapes and offsets against the
    exact attention, within the bf16 bound of the fixed-shape test."""
    import oracle
    from test_gpu_prefill import ULP, attention_bound, bits, f64
    from gpu_util import from_dev_bits, to_dev_bf16
    rng = np.random.default_rng(seed)
    pd = kvc.PrefillDesc(s=s, hq=hq, hkv=hkv, d=d, rope_base=10000.0, scale=0.0)
    q = bits(rng, (n, hq, d), 1.5)
    k = bits(rng, (s, hkv, d), 1.5)
    v = bits(rng, (s, hkv, d))
    o = torch.empty((n, hq, d), dtype=torch.bfloat16, device="cuda")
    kvc.kvc_chunk_attention(pd, to_dev_bf16(q), to_dev_bf16(k), to_dev_bf16(v), c0, o)
    torch.cuda.synchronize()
    pos = np.arange(c0, c0 + n)
    kk, vv = f64(k)[: c0 + n], f64(v)[: c0 + n]
    want = oracle.attention(f64(q), kk, vv, pos)
    bound = ULP * np.abs(want) + 2 * 2.0 ** -8 * attention_bound(f64(q), kk, vv, pos) + 1e-6
    err = np.abs(f64(from_dev_bits(o)) - want)
    assert np.all(err <= bound), f"max err/bound {np.max(err / bound):.3f}"


@pytest.mark.parametrize("i", range(2, len(CASES), 8))
def test_random_shape_layer_sweep(i):
    """kvc_compress_layers (two layers in flight) over 1-5 layers of a random
    shape with per-layer budgets writes exactly what one kvc_compress_layer
    call per layer writes."""
    cfg, budgets, seed = _case_cfg(i)
    rng = np.random.default_rng(seed + 1)
    n_layers = int(rng.integers(1, 6))
    xs = [layer_inputs(cfg, l) for l in range(n_layers)]
    layers = [dev_inputs(x) for x in xs]
    bl = np.stack([rng.permutation(budgets) for _ in range(n_layers)])
    desc = desc_from(cfg, *layers[0])
    want = [run_fused(desc, *layers[l], bl[l], intermediates=False) for l in range(n_layers)]
    outs = [kvc.alloc_outputs(desc, bl[l], with_intermediates=False) for l in range(n_layers)]
    kvc.kvc_compress_layers(desc, layers, bl, outs, kvc.alloc_sweep_workspace(desc), aux_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    from gpu_util import from_dev_bits
    for l in range(n_layers):
        np.testing.assert_array_equal(outs[l].idx.cpu().numpy(), want[l]["idx"], err_msg=f"layer {l} idx")
        np.testing.assert_array_equal(from_dev_bits(outs[l].k_hat), want[l]["k_hat"], err_msg=f"layer {l} k_hat")
        np.testing.assert_array_equal(from_dev_bits(outs[l].v_hat), want[l]["v_hat"], err_msg=f"layer {l} v_hat")
        np.testing.assert_array_equal(outs[l].pos.cpu().numpy(), want[l]["pos"], err_msg=f"layer {l} pos")


@pytest.mark.parametrize("case", range(8))
def test_random_prefill_row_kernels(case):
    """RMSNorm, the rotary append and SwiGLU on random sizes: one bf16 ulp of
    the exact result (the pair norm for the rotation), copies bit for bit,
    and cache rows outside the written range untouched."""
    import oracle
    from test_gpu_prefill import ULP, bits, f64
    from gpu_util import from_dev_bits, to_dev_bf16
    rng = np.random.default_rng(9000 + case)
    # RMSNorm
    rows, dim = int(rng.integers(1, 70)), 8 * int(rng.integers(1, 700))
    x, w = bits(rng, (rows, dim), 3.0), bits(rng, dim)
    y = torch.empty((rows, dim), dtype=torch.bfloat16, device="cuda")
    kvc.kvc_rmsnorm(to_dev_bf16(x), to_dev_bf16(w), y, eps=1e-5)
    torch.cuda.synchronize()
    want = oracle.rmsnorm(f64(x), f64(w), 1e-5)
    assert np.all(np.abs(f64(from_dev_bits(y)) - want) <= ULP * np.abs(want) + 1e-30), "rmsnorm"
    # rotary append
    g = int(rng.choice([1, 2, 4, 8]))
    hkv, d = int(rng.choice([1, 2, 4])), int(rng.choice([64, 128]))
    hq = g * hkv
    n = int(rng.integers(1, 90))
    c0 = int(rng.integers(0, 200000))
    s = c0 + n + int(rng.integers(0, 9))
    base = float(rng.choice([10000.0, 500000.0]))
    pd = kvc.PrefillDesc(s=s, hq=hq, hkv=hkv, d=d, rope_base=base, scale=0.0)
    qkv = bits(rng, (n, (hq + 2 * hkv) * d), 2.0)
    q = torch.empty((n, hq, d), dtype=torch.bfloat16, device="cuda")
    sentinel = 0x3F80
    kc = torch.full((s, hkv, d), sentinel, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    vc = torch.full((s, hkv, d), sentinel, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    kvc.kvc_rope_append(pd, to_dev_bf16(qkv), c0, q, kc, vc)
    torch.cuda.synchronize()
    pos = np.arange(c0, c0 + n)
    xx = f64(qkv)
    for name, got, heads, off in [("q", from_dev_bits(q), hq, 0), ("k", from_dev_bits(kc)[c0:c0 + n], hkv, hq * d)]:
        src = xx[:, off:off + heads * d].reshape(n, heads, d)
        want = oracle.rope(src, pos, base)
        norm = np.sqrt(src[..., : d // 2] ** 2 + src[..., d // 2:] ** 2)
        norm = np.concatenate([norm, norm], axis=-1)
        assert np.all(np.abs(f64(got) - want) <= ULP * norm + 1e-30), name
    np.testing.assert_array_equal(from_dev_bits(vc)[c0:c0 + n], qkv[:, (hq + hkv) * d:].reshape(n, hkv, d))
    for t in (kc, vc):
        b = from_dev_bits(t)
        assert np.all(b[:c0] == sentinel) and np.all(b[c0 + n:] == sentinel)
    # SwiGLU
    rows, ffn = int(rng.integers(1, 40)), 8 * int(rng.integers(1, 400))
    gu = bits(rng, (rows, 2 * ffn), 3.0)
    a = torch.empty((rows, ffn), dtype=torch.bfloat16, device="cuda")
    kvc.kvc_swiglu(to_dev_bf16(gu), a)
    torch.cuda.synchronize()
    want = oracle.swiglu(f64(gu))
    assert np.all(np.abs(f64(from_dev_bits(a)) - want) <= ULP * np.abs(want) + 1e-30), "swiglu"


def test_positions_at_the_int32_limit():
    """pos_offset + s = 2^31 - 1 (the largest the descriptor accepts): every
    retained position is offset + index exactly, in the whole-layer call and
    in the staged gather."""
    from gpu_util import run_staged, split_heads
    cfg = get_config("tiny").with_(name="max_pos", s=2000, w=16, hq=8, hkv=2, d=64, n_sink=4, n_recent=16,
                                   n_heavy=10, budget=300)
    x = layer_inputs(cfg, 0)
    q, k, v = dev_inputs(x)
    off = (1 << 31) - 1 - cfg.s
    b = np.array([300, 2000])
    desc = desc_from(cfg, q, k, v, pos_offset=off)
    fu = run_fused(desc, q, k, v, b)
    st = run_staged(desc, q, k, v, b)
    idx = np.concatenate(split_heads(fu["idx"], fu["offsets"])).astype(np.int64)
    np.testing.assert_array_equal(fu["pos"].astype(np.int64), idx + off)
    np.testing.assert_array_equal(st["pos"], fu["pos"])
    assert int(fu["pos"].max()) == (1 << 31) - 2  # head 1 keeps every key, the last at 2^31 - 2


FSEL_CHUNKED = [i for i, c in enumerate(CHUNKED) if c["pool"] == 1 and c["mode"] == "softmax"]


@pytest.mark.parametrize("i", FSEL_CHUNKED)
def test_random_immediate_eviction_fused_select(i):
    """The random softmax boundary chains again with KVC_FLAG_FUSED_SELECT
    (every evicting boundary one launch, the scores kept on chip): every
    boundary's retained set within the tie band of the oracle's, the
    whole-prompt call equal to the chain."""
    from test_gpu_chunked import FSEL, check_case
    c = dict(CHUNKED[i])
    budget, pool, pos_offset, mode, seed = c.pop("budget"), c.pop("pool"), c.pop("pos_offset"), c.pop("mode"), c.pop("seed")
    cfg = get_config("tiny").with_(name=f"random_chunked_fsel_{i}", sink_scale=4.0, seed_base=seed, budget=budget, **c)
    check_case(cfg, budget, mode=mode, pool=pool, pos_offset=pos_offset, flags=FSEL)
