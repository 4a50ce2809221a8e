"""GPU checks of the synthetic layer-major chunked prefill driver (TideKV,
Fig. 2 caption; Fig. 4 caption: scheduler, compressor, cross-layer cache
manager, memory accountant) against the prefill oracle.

- Each layer is compared with the oracle run on the GPU's own input bridge
  (the oracle rounds every operation's output to bf16 where the GPU does):
  outputs, full K/V and window queries within a few bf16 ulps (an operation
  whose fp32 result lands on the other side of a bf16 rounding boundary
  differs by one ulp, and later operations of the layer carry that on).
- Each layer's retained cache is exactly what kvc_compress_layer makes of the
  layer's full K/V and window queries, and matches the oracle's compressor
  on them up to the tie band.
- The schedule does not change the numbers: overlapping the commit with the
  next layer, and keeping every layer's full K/V until the end (Fig. 1 (b)
  with post-prefill compression) give bit-identical caches.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import compression_kvc_score_amd as kvc  # noqa: E402
from compression_kvc_score_amd import prefill as pf  # noqa: E402
import oracle  # noqa: E402
from synth import model_weights, prompt_hidden  # noqa: E402

from gpu_util import from_dev_bits, to_dev_bf16  # noqa: E402
from parity import assert_selection_matches  # noqa: E402


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    kvc.lib()


def say(*a):
    print(*a, flush=True, file=sys.stderr)


TINY = dict(hidden=256, hq=8, hkv=2, d=64, ffn=512, layers=3)


def setup(s=512, chunk=128, w=16, seed=3, **kw):
    shape = dict(TINY)
    shape.update(kw)
    cfg = pf.ModelConfig(hidden=shape["hidden"], hq=shape["hq"], hkv=shape["hkv"], d=shape["d"],
                         ffn=shape["ffn"], layers=shape["layers"], rope_base=10000.0)
    host_w = model_weights(cfg.hidden, cfg.hq, cfg.hkv, cfg.d, cfg.ffn, cfg.layers, seed)
    x = prompt_hidden(s, cfg.hidden, seed)
    return cfg, host_w, x


def run_driver(cfg, host_w, x, s, chunk, w, budgets, overlap=True, keep_full_kv=False, per_layer=None, block=64):
    model = pf.SyntheticModel(cfg, host_weights=host_w)
    drv = pf.LayerMajorPrefill(model, s, chunk, w, budgets, 4, 16, block=block, overlap=overlap,
                               keep_full_kv=keep_full_kv)
    xb = to_dev_bf16(x)
    if per_layer is None:
        cache = drv.run(xb)
    else:
        drv.acct.hold("bridge", xb.numel() * 2)
        for l in range(cfg.layers):
            before = from_dev_bits(xb).copy()
            drv.run_layer(l, xb)
            torch.cuda.synchronize()
            i = l % len(drv.kv)
            per_layer(l, before, from_dev_bits(xb), from_dev_bits(drv.kv[i][0]), from_dev_bits(drv.kv[i][1]),
                      from_dev_bits(drv.q_win[i]))
        for ev in drv.kv_free:
            if ev is not None:
                torch.cuda.current_stream().wait_event(ev)
        cache = drv.cache
    torch.cuda.synchronize()
    return drv, cache, from_dev_bits(xb)


def close_in_ulps(got_bits, want, what, max_ulps=8.0, rms_ulps=0.5):
    """|got - want| within max_ulps bf16 ulps of the tensor's RMS at every
    element, and its RMS within rms_ulps ulps of that RMS."""
    got = oracle.bf16_to_f64(got_bits)
    rms = float(np.sqrt(np.mean(want * want)))
    err = np.abs(got - want)
    ulp = rms * 2.0 ** -7
    assert err.max() <= max_ulps * ulp, f"{what}: max error {err.max() / ulp:.2f} ulps of the RMS"
    assert np.sqrt(np.mean(err * err)) <= rms_ulps * ulp, f"{what}: RMS error {np.sqrt(np.mean(err * err)) / ulp:.3f} ulps"


def test_each_layer_matches_the_oracle_on_the_gpu_bridge():
    s, chunk, w = 512, 128, 16
    cfg, host_w, x = setup(s, chunk, w)
    budgets = [64, 96]
    shp = oracle.ModelShape(hidden=cfg.hidden, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, ffn=cfg.ffn, rope_base=cfg.rope_base)
    seen = []

    def check(l, before, after, k_bits, v_bits, qw_bits):
        kc = np.zeros((s, cfg.hkv, cfg.d))
        vc = np.zeros((s, cfg.hkv, cfg.d))
        bridge = oracle.bf16_to_f64(before)
        q_all = np.zeros((s, cfg.hq, cfg.d))
        for c0 in range(0, s, chunk):
            out, q = oracle.layer_chunk(bridge[c0:c0 + chunk], host_w[l], shp, c0, kc, vc)
            bridge[c0:c0 + chunk] = out
            q_all[c0:c0 + chunk] = q
        close_in_ulps(k_bits, kc, f"layer {l} K")
        close_in_ulps(v_bits, vc, f"layer {l} V")
        close_in_ulps(qw_bits, q_all[s - w:], f"layer {l} window queries")
        close_in_ulps(after, bridge, f"layer {l} output bridge")
        seen.append((l, k_bits, v_bits, qw_bits))

    drv, cache, _ = run_driver(cfg, host_w, x, s, chunk, w, budgets, per_layer=check)
    assert len(seen) == cfg.layers
    off = np.concatenate([[0], np.cumsum(budgets)])
    for l, k_bits, v_bits, qw_bits in seen:
        # the commit is kvc_compress_layer of this layer's K/V and window
        q, k, v = to_dev_bf16(qw_bits), to_dev_bf16(k_bits), to_dev_bf16(v_bits)
        desc = kvc.desc_for(q, k, v, block=64, n_sink=4, n_recent=16)
        out = kvc.alloc_outputs(desc, budgets, with_intermediates=False)
        kvc.compress_layer(desc, q, k, v, budgets, out, kvc.alloc_workspace(desc))
        torch.cuda.synchronize()
        np.testing.assert_array_equal(cache.idx[l].cpu().numpy(), out.idx.cpu().numpy())
        np.testing.assert_array_equal(from_dev_bits(cache.k[l]), from_dev_bits(out.k_hat))
        np.testing.assert_array_equal(from_dev_bits(cache.v[l]), from_dev_bits(out.v_hat))
        np.testing.assert_array_equal(cache.pos[l].cpu().numpy(), out.pos.cpu().numpy())
        # and the oracle's compressor agrees on the same tensors
        qf, kf = oracle.bf16_to_f64(qw_bits), oracle.bf16_to_f64(k_bits)
        sc = oracle.scores(qf, kf)
        got = cache.idx[l].cpu().numpy()
        for g in range(cfg.hkv):
            want = oracle.select_head(sc[g], budgets[g], 4, 16)
            assert_selection_matches(got[off[g]:off[g + 1]], want, sc[g], budgets[g], 4, 16)


def test_schedules_give_identical_caches():
    s, chunk, w = 384, 96, 8
    cfg, host_w, x = setup(s, chunk, w, seed=5)
    budgets = [40, 40]
    results = {}
    for name, kw in [("overlap", dict(overlap=True)), ("serial", dict(overlap=False)),
                     ("full_kv_then_compress", dict(keep_full_kv=True))]:
        drv, cache, bridge = run_driver(cfg, host_w, x, s, chunk, w, budgets, **kw)
        results[name] = (from_dev_bits(cache.k), from_dev_bits(cache.v), cache.pos.cpu().numpy(), bridge,
                         drv.acct.report())
    ref = results["overlap"]
    for name in ("serial", "full_kv_then_compress"):
        for a, b in zip(results[name][:4], ref[:4]):
            np.testing.assert_array_equal(a, b, err_msg=name)
    # memory: the layer-major schedule holds two layers' full K/V, the other all of them
    kv_layer = 2 * s * cfg.hkv * cfg.d * 2
    assert results["overlap"][4]["peak_parts"]["full_kv"] == 2 * kv_layer
    assert results["serial"][4]["peak_parts"]["full_kv"] == kv_layer
    assert results["full_kv_then_compress"][4]["peak_parts"]["full_kv"] == cfg.layers * kv_layer
    rows = sum(budgets)
    assert results["overlap"][4]["peak_parts"]["retained_cache"] == cfg.layers * rows * (2 * cfg.d * 2 + 4)


def test_chunk_size_changes_only_gemm_rounding():
    """Chunk 64 against one chunk of the whole prompt: attention and the
    row-wise kernels are chunk-invariant bit for bit; only the vendor GEMM may
    round differently for a different row count, so the final bridges agree
    to within a few ulps."""
    s, w = 256, 8
    cfg, host_w, x = setup(s, 64, w, seed=7, layers=2)
    _, c_small, b_small = run_driver(cfg, host_w, x, s, 64, w, [32, 32])
    _, c_one, b_one = run_driver(cfg, host_w, x, s, s, w, [32, 32])
    close_in_ulps(b_small, oracle.bf16_to_f64(b_one), "bridge, chunk 64 vs one shot", max_ulps=16, rms_ulps=1.0)


def test_llama8b_layer_shape_last_chunk_against_the_oracle():
    """The Llama-3.1-8B layer shape (hidden 4096, 32/8 heads of 128, FFN
    14336) through the driver; the last chunk of the layer is recomputed by the
    oracle from the GPU's own input bridge and K/V of the earlier chunks."""
    s, chunk, w = 1024, 256, 32
    cfg = pf.ModelConfig(layers=1)
    host_w = model_weights(cfg.hidden, cfg.hq, cfg.hkv, cfg.d, cfg.ffn, 1, 11)
    x = prompt_hidden(s, cfg.hidden, 11)
    shp = oracle.ModelShape(hidden=cfg.hidden, hq=cfg.hq, hkv=cfg.hkv, d=cfg.d, ffn=cfg.ffn, rope_base=cfg.rope_base)
    got = {}

    def keep(l, before, after, k_bits, v_bits, qw_bits):
        got.update(before=before, after=after, k=k_bits, v=v_bits, qw=qw_bits)

    say("llama8b layer shape: driver")
    drv, cache, _ = run_driver(cfg, host_w, x, s, chunk, w, [512] * cfg.hkv, per_layer=keep)
    c0 = s - chunk
    kc = oracle.bf16_to_f64(got["k"]).copy()
    vc = oracle.bf16_to_f64(got["v"]).copy()
    say("llama8b layer shape: oracle on the last chunk")
    out, q = oracle.layer_chunk(oracle.bf16_to_f64(got["before"][c0:]), host_w[0], shp, c0, kc, vc)
    close_in_ulps(got["k"][c0:], kc[c0:], "K rows of the last chunk")
    close_in_ulps(got["v"][c0:], vc[c0:], "V rows of the last chunk")
    close_in_ulps(got["qw"], q[chunk - w:], "window queries")
    close_in_ulps(got["after"][c0:], out, "output rows of the last chunk")
    # earlier rows of the bridge are the earlier chunks' outputs, untouched by the last chunk
    assert cache.committed[0]
