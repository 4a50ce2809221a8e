"""GPU parity of the raw inner-product score modes (HillInfer, Algorithmic
Simplification; Streaming Execution and Asymmetric Precision) and of the
overlap coefficient (HeteroCache summary, Key Contributions item 1), through
the C ABI against the CPU oracle.

- KVC_SCORE_LOGIT: fp32 dot products of bf16 keys with the pooled query, so
  each score is within a small multiple of fp32 rounding of the exact sum of
  |pooled query x key| terms; the GPU's selection equals the oracle rule
  applied to the GPU's own scores exactly, and differs from the oracle's
  selection only for keys within that error of the threshold.
- KVC_SCORE_LOGIT_INT8: the quantisation decisions and the integer dot are
  the oracle's, in the kernel's precision, so scores match bit for bit and
  the selection exactly.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import compression_kvc_score_amd as kvc  # noqa: E402
import oracle  # noqa: E402
from synth import get_config, layer_inputs  # noqa: E402

from gpu_util import desc_from, from_dev_bits, run_fused, run_staged, split_heads, to_dev_bf16  # noqa: E402

MODES = {"logit": kvc.KVC_SCORE_LOGIT, "int8": kvc.KVC_SCORE_LOGIT_INT8}


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    kvc.lib()


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def budgets_for(cfg, x):
    if cfg.hetero:
        return oracle.inverse_stability_budgets(x.s_stable, cfg.total_budget)
    return np.full(cfg.hkv, cfg.budget, dtype=np.int64)


def logit_error_bound(q_bits, k_bits):
    """Per (head, key) bound on |GPU - exact| for the fp32 logit score: the
    pooled query is rounded once to fp32 and each product and partial sum once
    more (at most D + 8 roundings), each by at most 2^-24 of the sum of
    |pooled query x key| terms."""
    q = oracle.bf16_to_f64(q_bits)
    k = oracle.bf16_to_f64(k_bits)
    w, hq, d = q.shape
    s, hkv, _ = k.shape
    grp = hq // hkv
    t_of = oracle.first_visible_row(s, w)
    out = np.empty((hkv, s))
    for g in range(hkv):
        for t in np.unique(t_of):
            keys = np.nonzero(t_of == t)[0]
            qbar = np.abs(q[t:, g * grp:(g + 1) * grp, :].sum(axis=(0, 1)))
            out[g, keys] = np.abs(k[keys, g, :]) @ qbar
    return out * (d + 8) * 2.0 ** -23 + 1e-30


def check_selection_signed(got_idx, gpu_scores, want_scores, err, budgets, n_sink, n_recent, pool=1):
    """GPU selection = the oracle rule on the GPU's scores (exact), and outside
    the error band around the threshold it agrees with the oracle's."""
    off = np.concatenate([[0], np.cumsum(np.minimum(budgets, gpu_scores.shape[1]))])
    got = split_heads(got_idx, off)
    gv = oracle.maxpool(gpu_scores.astype(np.float64), pool) if pool > 1 else gpu_scores.astype(np.float64)
    wv = oracle.maxpool(want_scores, pool) if pool > 1 else want_scores
    for g in range(gpu_scores.shape[0]):
        np.testing.assert_array_equal(got[g], oracle.select_head(gv[g], int(budgets[g]), n_sink, n_recent),
                                      err_msg=f"head {g}: selection on the GPU's own scores")
        want = oracle.select_head(wv[g], int(budgets[g]), n_sink, n_recent)
        diff = np.setxor1d(got[g], want)
        if diff.size:
            s = gpu_scores.shape[1]
            mand = oracle.mandatory(s, n_sink, n_recent)
            cand = np.setdiff1d(np.arange(s), mand)
            k_sel = int(budgets[g]) - mand.size
            tau = np.sort(wv[g][cand])[::-1][k_sel - 1]
            band = 2 * err[g].max() if pool > 1 else 2 * err[g][diff]
            assert np.all(np.abs(wv[g][diff] - tau) <= band), f"head {g}: differences outside the error band"


def dev(x):
    return to_dev_bf16(x.q), to_dev_bf16(x.k), to_dev_bf16(x.v)


CASES = [("tiny", None, 0), ("llama8b_16k", 8192, 1), ("qwen14b_hetero_64k", 8192, 2)]


@pytest.mark.parametrize("mode", ["logit", "int8"])
@pytest.mark.parametrize("name,s,layer", CASES)
def test_score_mode_full_layer_parity(mode, name, s, layer):
    cfg = get_config(name)
    if s is not None:
        cfg = cfg.with_(s=s)
    x = layer_inputs(cfg, layer)
    q, k, v = dev(x)
    b = budgets_for(cfg, x)
    desc = desc_from(cfg, q, k, v, score_mode=MODES[mode])
    say(f"{mode} {name}: fused and staged")
    fu = run_fused(desc, q, k, v, b)
    st = run_staged_modes(desc, q, k, v, b)
    for key in ["scores", "idx", "k_hat", "v_hat", "pos"]:
        np.testing.assert_array_equal(fu[key], st[key], err_msg=f"fused != staged: {key}")
    say(f"{mode} {name}: oracle")
    if mode == "int8":
        want = oracle.logit_scores_int8(x.q, x.k)
        np.testing.assert_array_equal(fu["scores"], want)
        want_idx = oracle.select(want.astype(np.float64), b, cfg.n_sink, cfg.n_recent)
        np.testing.assert_array_equal(fu["idx"], np.concatenate(want_idx))
    else:
        want = oracle.logit_scores(oracle.bf16_to_f64(x.q), oracle.bf16_to_f64(x.k))
        err = logit_error_bound(x.q, x.k)
        assert np.all(np.abs(fu["scores"] - want) <= err), float(np.max(np.abs(fu["scores"] - want) / err))
        check_selection_signed(fu["idx"], fu["scores"], want, err, b, cfg.n_sink, cfg.n_recent)
    # gather and positions of whatever was selected, bit for bit
    off = fu["offsets"]
    idx = split_heads(fu["idx"], off)
    k_hat, v_hat, pos = oracle.gather(x.k, x.v, idx)
    np.testing.assert_array_equal(fu["k_hat"], k_hat)
    np.testing.assert_array_equal(fu["v_hat"], v_hat)
    np.testing.assert_array_equal(fu["pos"], pos)


def run_staged_modes(desc, q, k, v, budgets):
    """pass 2 (the raw inner-product scan) -> select -> gather as three calls."""
    ws = kvc.alloc_workspace(desc)
    out = kvc.alloc_outputs(desc, budgets)
    kvc.kvc_score_pass2(desc, q, k, None, None, out.scores)
    kvc.kvc_select_topk(desc, out.scores, budgets, out.idx, ws)
    kvc.kvc_gather_retained(desc, k, v, out.idx, budgets, out.k_hat, out.v_hat, out.pos)
    torch.cuda.synchronize()
    return {"scores": out.scores.cpu().numpy(), "idx": out.idx.cpu().numpy(),
            "k_hat": from_dev_bits(out.k_hat), "v_hat": from_dev_bits(out.v_hat), "pos": out.pos.cpu().numpy()}


@pytest.mark.parametrize("mode", ["logit", "int8"])
def test_negative_thresholds_zero_rows_and_pooling(mode):
    """Scores mostly negative (queries negated), some keys all zero (score
    exactly 0), a max-pool of 5: the signed ranking keys, -0/+0 and pooling."""
    cfg = get_config("llama8b_16k").with_(s=5000, pool=5)
    x = layer_inputs(cfg, 3)
    qb = x.q ^ np.uint16(0x8000)                       # negate every query
    kb = x.k.copy()
    kb[100:140] = 0                                    # zero rows: score exactly 0
    kb[4000:4010] = 0x8000                             # -0 rows
    q, k, v = to_dev_bf16(qb), to_dev_bf16(kb), to_dev_bf16(x.v)
    b = np.array([600, 37, 4999, 5000, 1200, 36, 2500, 4096])
    desc = desc_from(cfg, q, k, v, score_mode=MODES[mode])
    got = run_fused(desc, q, k, v, b)
    if mode == "int8":
        want = oracle.logit_scores_int8(qb, kb)
        np.testing.assert_array_equal(got["scores"], want)
        pooled = oracle.maxpool(want.astype(np.float64), 5)
        np.testing.assert_array_equal(got["idx"], np.concatenate(oracle.select(pooled, b, cfg.n_sink, cfg.n_recent)))
    else:
        want = oracle.logit_scores(oracle.bf16_to_f64(qb), oracle.bf16_to_f64(kb))
        err = logit_error_bound(qb, kb)
        assert np.all(np.abs(got["scores"] - want) <= err)
        check_selection_signed(got["idx"], got["scores"], want, err, b, cfg.n_sink, cfg.n_recent, pool=5)
    assert np.all(got["scores"][:, 100:140] == 0.0)


@pytest.mark.parametrize("mode", ["logit", "int8"])
def test_select_on_identical_signed_values_is_exact(mode):
    """kvc_select_topk alone on given signed values (coarse, so many ties):
    equal to the oracle's selection."""
    rng = np.random.default_rng(31)
    s, hkv = 9000, 4
    vals = ((rng.integers(-60, 40, size=(hkv, s))) / 8.0).astype(np.float32)
    vals[:, rng.integers(0, s, size=300)] = -0.0
    budgets = np.array([1000, 37, 8999, 4500])
    desc = kvc.make_desc(s, 8, 8, hkv, 64, 64, n_sink=4, n_recent=32, score_mode=MODES[mode])
    scores = torch.from_numpy(vals).cuda()
    ws = kvc.alloc_workspace(desc)
    off = kvc.kvc_retained_offsets(desc, budgets)
    idx = torch.empty(int(off[-1]), dtype=torch.int32, device="cuda")
    kvc.kvc_select_topk(desc, scores, budgets, idx, ws)
    got = split_heads(idx.cpu().numpy(), off)
    for g in range(hkv):
        np.testing.assert_array_equal(got[g], oracle.select_head(vals[g].astype(np.float64), int(budgets[g]), 4, 32))


def test_overlap_coefficient_of_score_modes():
    """The retained sets of the softmax and raw inner-product modes on one
    layer, and of a set with itself: the GPU's overlap equals the oracle's."""
    cfg = get_config("llama8b_16k").with_(s=8192)
    x = layer_inputs(cfg, 4)
    q, k, v = dev(x)
    b = budgets_for(cfg, x)
    sets = {}
    for mode, sm in [("softmax", kvc.KVC_SCORE_SOFTMAX), ("logit", kvc.KVC_SCORE_LOGIT),
                     ("int8", kvc.KVC_SCORE_LOGIT_INT8)]:
        desc = desc_from(cfg, q, k, v, score_mode=sm)
        ws = kvc.alloc_workspace(desc)
        out = kvc.alloc_outputs(desc, b)
        kvc.compress_layer(desc, q, k, v, b, out, ws)
        sets[mode] = out.idx
    desc = desc_from(cfg, q, k, v)
    off = kvc.kvc_retained_offsets(desc, b)
    for a_, b_ in [("softmax", "logit"), ("logit", "int8"), ("softmax", "softmax")]:
        res = torch.empty(cfg.hkv, dtype=torch.float32, device="cuda")
        kvc.kvc_overlap_coefficient(desc, sets[a_], sets[b_], b, res)
        torch.cuda.synchronize()
        ia = split_heads(sets[a_].cpu().numpy(), off)
        ib = split_heads(sets[b_].cpu().numpy(), off)
        want = np.array([oracle.overlap_coefficient(ia[g], ib[g]) for g in range(cfg.hkv)])
        got = res.cpu().numpy()
        np.testing.assert_array_equal(np.rint(got * (off[1:] - off[:-1])), np.rint(want * (off[1:] - off[:-1])))
        np.testing.assert_allclose(got, want, rtol=1e-6)
        say(f"overlap {a_} vs {b_}: {np.round(got, 3)}")
    assert np.all(res.cpu().numpy() == 1.0)


def test_sweep_in_a_raw_inner_product_mode_equals_layer_by_layer():
    cfg = get_config("llama8b_16k").with_(s=4096)
    xs = [layer_inputs(cfg, l) for l in range(3)]
    layers = [dev(x) for x in xs]
    budgets = np.stack([budgets_for(cfg, x) for x in xs])
    desc = desc_from(cfg, *layers[0], score_mode=kvc.KVC_SCORE_LOGIT_INT8)
    want = [run_fused(desc, *layers[i], budgets[i], intermediates=False) for i in range(3)]
    outs = [kvc.alloc_outputs(desc, budgets[i], with_intermediates=False) for i in range(3)]
    ws = kvc.alloc_sweep_workspace(desc)
    kvc.kvc_compress_layers(desc, layers, budgets, outs, ws, aux_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    for i in range(3):
        np.testing.assert_array_equal(outs[i].idx.cpu().numpy(), want[i]["idx"])
        np.testing.assert_array_equal(from_dev_bits(outs[i].k_hat), want[i]["k_hat"])


def test_overlap_coefficient_synthetic_sets_both_paths():
    """Given ascending index sets (sizes below and above what the kernel keeps
    in LDS, and an empty head): the GPU's overlap equals the oracle's."""
    rng = np.random.default_rng(41)
    s, hkv = 30000, 5
    budgets = np.array([100, 15360, 15361, 20000, 0])
    desc = kvc.make_desc(s, 8, hkv, hkv, 64, 64, n_sink=0, n_recent=0)
    off = kvc.kvc_retained_offsets(desc, budgets)
    a_sets, b_sets = [], []
    for g in range(hkv):
        n = int(off[g + 1] - off[g])
        a = np.sort(rng.choice(s, size=n, replace=False))
        keep = rng.random(n) < rng.random()
        b = np.sort(np.concatenate([a[keep], rng.choice(np.setdiff1d(np.arange(s), a), size=n - keep.sum(),
                                                          replace=False)]))
        a_sets.append(a)
        b_sets.append(b)
    ia = torch.from_numpy(np.concatenate(a_sets).astype(np.int32)).cuda()
    ib = torch.from_numpy(np.concatenate(b_sets).astype(np.int32)).cuda()
    res = torch.empty(hkv, dtype=torch.float32, device="cuda")
    kvc.kvc_overlap_coefficient(desc, ia, ib, budgets, res)
    torch.cuda.synchronize()
    want = np.array([oracle.overlap_coefficient(a_sets[g], b_sets[g]) for g in range(hkv)], dtype=np.float32)
    np.testing.assert_array_equal(res.cpu().numpy(), want)


def test_logit_mode_at_its_maximum_prompt_length():
    """S = 2^22, the limit of the signed-score selection: INT8 scores and the
    selection are exact against the oracle."""
    cfg = get_config("tiny").with_(name="max_prompt_int8", s=1 << 22, w=2, hq=2, hkv=1, d=64, block=256, n_sink=4,
                                   n_recent=2, n_heavy=1000, budget=30000, sink_scale=4.0, seed_base=889)
    say("int8 max prompt: generating 2^22 keys")
    x = layer_inputs(cfg, 0)
    q, k, v = dev(x)
    b = np.array([cfg.budget])
    desc = desc_from(cfg, q, k, v, score_mode=MODES["int8"])
    say("int8 max prompt: GPU")
    got = run_fused(desc, q, k, v, b)
    want = oracle.logit_scores_int8(x.q, x.k)
    np.testing.assert_array_equal(got["scores"].astype(np.float64), want.astype(np.float64))
    np.testing.assert_array_equal(got["idx"], oracle.select_head(want[0].astype(np.float64), cfg.budget, 4, 2))
    kh, vh, pos = oracle.gather(x.k, x.v, [got["idx"]])
    np.testing.assert_array_equal(got["k_hat"], kh)
    np.testing.assert_array_equal(got["pos"], pos)
