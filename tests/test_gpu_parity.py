"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Small cases compare every output element; full-size cases (the launch
configuration the benchmark times) compare sampled KV heads against the
oracle and check properties that hold at any size on every head.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import compression_kvc_score_amd as kvc  # noqa: E402
import oracle  # noqa: E402
from synth import LayerConfig, get_config, layer_inputs  # noqa: E402

from gpu_util import desc_from, from_dev_bits, host, run_fused, run_staged, split_heads, to_dev_bf16  # noqa: E402
from parity import (  # noqa: E402
    assert_normalizers_close, assert_scores_close, assert_selection_consistent,
    assert_selection_matches,
)


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    kvc.lib()  # fails loudly if libkvc.so is missing


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def budgets_for(cfg, x):
    if cfg.hetero:
        return oracle.inverse_stability_budgets(x.s_stable, cfg.total_budget)
    return np.full(cfg.hkv, cfg.budget, dtype=np.int64)


def oracle_head(x, g, pool=1, scale=None):
    """Oracle outputs for KV head g only (its query group and key column)."""
    cfg = x.cfg
    G = cfg.group
    q = oracle.bf16_to_f64(x.q[:, g * G:(g + 1) * G, :])
    k = oracle.bf16_to_f64(x.k[:, g:g + 1, :])
    m, z = oracle.normalizers(q, k, scale)
    sc = oracle.scores(q, k, scale)[0]
    vals = oracle.maxpool(sc, pool) if pool > 1 else sc
    return m, z, sc, vals


def check_layer(x, got, budgets, heads=None, pool=None, n_sink=None, n_recent=None, scale=None):
    """Compare GPU outputs with the oracle on `heads` (default: all) and
    check gather/selection properties on every head."""
    cfg = x.cfg
    pool = cfg.pool if pool is None else pool
    n_sink = cfg.n_sink if n_sink is None else n_sink
    n_recent = cfg.n_recent if n_recent is None else n_recent
    G, hkv = cfg.group, cfg.hkv
    idx = split_heads(got["idx"], got["offsets"])
    heads = range(hkv) if heads is None else heads
    for g in heads:
        m, z, sc, vals = oracle_head(x, g, pool, scale)
        assert_normalizers_close(got["m"][g * G:(g + 1) * G], got["z"][g * G:(g + 1) * G], m, z)
        assert_scores_close(got["scores"][g], sc, what=f"scores head {g}")
        want = oracle.select_head(vals, int(budgets[g]), n_sink, n_recent)
        assert_selection_matches(idx[g], want, vals, int(budgets[g]), n_sink, n_recent)
    # every head: the choice is an exact top-k of the GPU's own values, and
    # the gather copies exactly the chosen rows
    gs = got["scores"].astype(np.float64)
    gv = oracle.maxpool(gs, pool) if pool > 1 else gs
    for g in range(hkv):
        assert_selection_consistent(idx[g], gv[g].astype(np.float32).astype(np.float64),
                                    int(budgets[g]), n_sink, n_recent)
    kh, vh, pos = oracle.gather(x.k, x.v, idx)
    np.testing.assert_array_equal(got["k_hat"], kh)
    np.testing.assert_array_equal(got["v_hat"], vh)
    np.testing.assert_array_equal(got["pos"], pos)


def dev_inputs(x):
    return to_dev_bf16(x.q), to_dev_bf16(x.k), to_dev_bf16(x.v)


# --------------------------------------------------------------------------- small, every element

def test_tiny_layer_full_parity_and_fused_equals_staged():
    cfg = get_config("tiny")
    x = layer_inputs(cfg, 0)
    q, k, v = dev_inputs(x)
    desc = desc_from(cfg, q, k, v)
    b = budgets_for(cfg, x)
    say("tiny staged")
    st = run_staged(desc, q, k, v, b)
    check_layer(x, st, b)
    # each head's scores sum to W * G
    np.testing.assert_allclose(st["scores"].sum(axis=1), cfg.w * cfg.group, rtol=1e-4)
    say("tiny fused")
    fu = run_fused(desc, q, k, v, b)
    for key in ["m", "z", "scores", "idx", "k_hat", "v_hat", "pos"]:
        np.testing.assert_array_equal(fu[key], st[key], err_msg=key)
    fu2 = run_fused(desc, q, k, v, b, intermediates=False)
    for key in ["idx", "k_hat", "v_hat", "pos"]:
        np.testing.assert_array_equal(fu2[key], st[key], err_msg=key)


def test_llama8b_16k_full_parity():
    cfg = get_config("llama8b_16k")
    x = layer_inputs(cfg, 0)
    q, k, v = dev_inputs(x)
    desc = desc_from(cfg, q, k, v)
    b = budgets_for(cfg, x)
    say("llama8b_16k fused")
    got = run_fused(desc, q, k, v, b)
    check_layer(x, got, b)


@pytest.mark.parametrize("block", [32, 64, 128, 256, 512])
def test_block_size_invariance(block):
    """The blockwise scan equals the dense definition for every block size."""
    cfg = get_config("tiny").with_(s=3001, hq=8, hkv=2, d=128, w=16, budget=300, n_heavy=20)
    x = layer_inputs(cfg, 1)
    q, k, v = dev_inputs(x)
    desc = desc_from(cfg, q, k, v, block=block)
    b = budgets_for(cfg, x)
    say(f"block {block}")
    got = run_fused(desc, q, k, v, b)
    check_layer(x, got, b)


@pytest.mark.parametrize("block", [32, 96, 224, 256, 288, 352, 416, 480, 512])
@pytest.mark.parametrize("d", [64, 128])
def test_block_size_invariance_wide_rows(block, d):
    """The per-head scans (more than 128 query rows per KV head) cover every
    key of every block, whatever the block's count of 32-key tiles (a block
    of 11 tiles once left 3 of them unscored)."""
    cfg = get_config("tiny").with_(s=3001, hq=8, hkv=1, d=d, w=32, budget=300, n_heavy=20)
    x = layer_inputs(cfg, 2)
    q, k, v = dev_inputs(x)
    desc = desc_from(cfg, q, k, v, block=block)
    b = budgets_for(cfg, x)
    say(f"wide rows, block {block}, d {d}")
    got = run_fused(desc, q, k, v, b)
    check_layer(x, got, b)
    np.testing.assert_allclose(got["scores"].sum(axis=1), cfg.w * cfg.group, rtol=1e-4)


EDGE_CASES = {
    # name: (config overrides, budgets or None for uniform, extra desc options)
    "one_key": (dict(s=1, w=1, hq=1, hkv=1, d=64, n_sink=0, n_recent=0, n_heavy=0, budget=1), None, {}),
    "window_is_prompt": (dict(s=33, w=33, hq=2, hkv=1, d=64, n_sink=1, n_recent=2, n_heavy=0, budget=10), None, {}),
    "ragged_gqa3": (dict(s=1000, w=7, hq=6, hkv=2, d=128, n_sink=3, n_recent=5, n_heavy=8, budget=77), [77, 1000], {}),
    "mha_many_heads": (dict(s=517, w=16, hq=16, hkv=16, d=64, n_sink=2, n_recent=16, n_heavy=5, budget=60),
                       None, {}),
    "max_rows": (dict(s=2048, w=64, hq=4, hkv=1, d=128, n_sink=4, n_recent=64, n_heavy=12, budget=400), None, {}),
    "max_heads": (dict(s=700, w=5, hq=64, hkv=64, d=64, n_sink=4, n_recent=5, n_heavy=4, budget=50), None, {}),
    "no_mandatory": (dict(s=1500, w=8, hq=8, hkv=2, d=128, n_sink=0, n_recent=0, n_heavy=10, budget=100), None, {}),
    "only_mandatory": (dict(s=1500, w=8, hq=8, hkv=2, d=128, n_sink=4, n_recent=8, n_heavy=10, budget=12),
                       [12, 20], {}),
    "budget_over_prompt": (dict(s=300, w=8, hq=4, hkv=2, d=64, n_sink=4, n_recent=8, n_heavy=3, budget=300),
                           [300, 1000], {}),
    "pool7": (dict(s=4000, w=16, hq=8, hkv=2, d=128, n_sink=4, n_recent=16, n_heavy=20, budget=256, pool=7),
              None, {}),
    "pool31_short": (dict(s=90, w=4, hq=4, hkv=1, d=64, n_sink=2, n_recent=4, n_heavy=3, budget=20, pool=31),
                     None, {}),
    "explicit_scale": (dict(s=1200, w=16, hq=8, hkv=2, d=128, n_sink=4, n_recent=16, n_heavy=8, budget=150),
                       None, dict(scale=0.05)),
    "hetero_budgets": (dict(s=6000, w=32, hq=40, hkv=8, d=128, n_sink=4, n_recent=32, n_heavy=60, budget=0,
                            hetero=True, total_budget=8 * 300), None, {}),
    # streaming scans with three query tiles per wavefront: 176 rows (a
    # ragged sixth row tile) and 192 rows
    "stream_176_rows": (dict(s=3001, w=44, hq=8, hkv=2, d=128, n_sink=4, n_recent=44, n_heavy=15, budget=300),
                        [300, 52], {}),
    "stream_192_rows": (dict(s=2500, w=48, hq=4, hkv=1, d=128, n_sink=4, n_recent=48, n_heavy=12, budget=256),
                        None, {}),
    # the two sides of the head-grouping rule at D = 128: 8 slots of 128 keys per
    # workgroup (one head each) and one key more (head pairs)
    "stream_one_head_32768": (dict(s=32768, w=32, hq=32, hkv=8, d=128, n_sink=4, n_recent=32, n_heavy=40,
                                   budget=2048), None, {}),
    "stream_head_pairs_32769": (dict(s=32769, w=32, hq=32, hkv=8, d=128, n_sink=4, n_recent=32, n_heavy=40,
                                     budget=2048), None, {}),
    # five row tiles with an odd KV-head count (one head per workgroup), a ragged last slot
    "stream_160_rows_odd_hkv": (dict(s=5003, w=32, hq=15, hkv=3, d=128, n_sink=4, n_recent=32, n_heavy=20,
                                     budget=700), [700, 37, 5003], {}),
}


@pytest.mark.parametrize("name", sorted(EDGE_CASES))
def test_edge_shapes(name):
    over, budgets, extra = EDGE_CASES[name]
    cfg = get_config("tiny").with_(**over).with_(name=name, sink_scale=4.0, seed_base=777)
    x = layer_inputs(cfg, 0)
    q, k, v = dev_inputs(x)
    desc = desc_from(cfg, q, k, v, **extra)
    b = np.asarray(budgets) if budgets is not None else budgets_for(cfg, x)
    say(f"edge {name} s={cfg.s} w={cfg.w} hq={cfg.hq} hkv={cfg.hkv} d={cfg.d} budgets={list(b)[:4]}")
    if name.startswith("stream_") or name == "hetero_budgets":
        plan = kvc.kvc_plan_layer(desc)
        assert plan.scan == kvc.KVC_SCAN_STREAM
        if name.startswith("stream_"):
            assert plan.fused_scans == 1  # the whole-layer call below runs both scans in one launch
        if name == "stream_one_head_32768":
            assert plan.heads_per_wg == 1
        if name == "stream_head_pairs_32769":
            assert plan.heads_per_wg == 2
    st = run_staged(desc, q, k, v, b)
    check_layer(x, st, b, scale=extra.get("scale"))
    fu = run_fused(desc, q, k, v, b)
    for key in ["m", "z", "scores", "idx", "k_hat", "v_hat", "pos"]:
        np.testing.assert_array_equal(fu[key], st[key], err_msg=key)


# --------------------------------------------------------------------------- selection and gather alone

@pytest.mark.parametrize("pool", [1, 3, 7])
def test_select_on_identical_values_is_exact(pool):
    """Given the same fp32 values, the GPU selection equals the oracle's
    selection exactly (ties included: values are coarse, so many are equal)."""
    rng = np.random.default_rng(pool)
    s, hkv = 5000, 8
    vals = (rng.integers(0, 50, size=(hkv, s)) / 64.0).astype(np.float32)
    vals[:, rng.integers(0, s, size=200)] = 1.5  # a block of exact ties near the top
    budgets = np.array([100, 36, 5000, 6000, 2000, 37, 4999, 555])
    desc = kvc.make_desc(s, 8, 8, hkv, 64, 64, n_sink=4, n_recent=32, pool=pool)
    scores = torch.from_numpy(vals).cuda()
    ws = kvc.alloc_workspace(desc)
    off = kvc.kvc_retained_offsets(desc, budgets)
    idx = torch.empty(int(off[-1]), dtype=torch.int32, device="cuda")
    kvc.kvc_select_topk(desc, scores, budgets, idx, ws)
    got = split_heads(idx.cpu().numpy(), off)
    pooled = oracle.maxpool(vals.astype(np.float64), pool)
    for g in range(hkv):
        want = oracle.select_head(pooled[g], int(budgets[g]), 4, 32)
        np.testing.assert_array_equal(got[g], want, err_msg=f"head {g}")


@pytest.mark.parametrize("case", ["all_equal", "tied_threshold_bin"])
def test_select_heavy_ties_take_the_slow_path_exactly(case):
    """More tied candidates than the threshold bin's list holds: the
    selection falls back to a radix over the whole row, with the same result."""
    rng = np.random.default_rng(11)
    s, hkv = 40000, 2
    if case == "all_equal":
        vals = np.full((hkv, s), 0.25, dtype=np.float32)
    else:
        vals = rng.random((hkv, s)).astype(np.float32)
        vals[:, 1000:30000] = np.float32(0.5)  # 29000 equal values around the threshold
    budgets = np.array([5000, 20000])
    desc = kvc.make_desc(s, 8, 8, hkv, 64, 64, n_sink=4, n_recent=32, pool=1)
    scores = torch.from_numpy(vals).cuda()
    ws = kvc.alloc_workspace(desc)
    off = kvc.kvc_retained_offsets(desc, budgets)
    idx = torch.empty(int(off[-1]), dtype=torch.int32, device="cuda")
    kvc.kvc_select_topk(desc, scores, budgets, idx, ws)
    got = split_heads(idx.cpu().numpy(), off)
    for g in range(hkv):
        want = oracle.select_head(vals[g].astype(np.float64), int(budgets[g]), 4, 32)
        np.testing.assert_array_equal(got[g], want, err_msg=f"head {g}")


@pytest.mark.parametrize("case", ["long_list", "many_chunks", "two_groups"])
def test_select_list_paths_are_exact(case):
    """Each way the compaction resolves the threshold gives the oracle's
    selection: lists held in registers (up to 32 chunks of 4096 keys), a list
    longer than one read brings (gathered through LDS), and more chunks than
    the registers hold."""
    rng = np.random.default_rng({"long_list": 21, "many_chunks": 22, "two_groups": 23}[case])
    hkv = 2
    if case == "long_list":
        s = 40000
        vals = (rng.random((hkv, s)) * 0.5).astype(np.float32)
        vals[:, 20000:20300] = 2.0 + rng.random((hkv, 300)).astype(np.float32)  # surely kept
        # 600 distinct values in one histogram bin, all inside one 4096-key chunk
        vals[:, 8200:8800] = (1.0 + np.arange(600) * 2.0 ** -16).astype(np.float32)
        budgets = np.array([36 + 300 + 250, 36 + 300 + 599])
    elif case == "many_chunks":
        s = 4096 * 36 + 123
        vals = rng.random((hkv, s)).astype(np.float32)
        budgets = np.array([4096, 30001])
    else:
        s = 4096 * 30 + 77
        vals = rng.random((hkv, s)).astype(np.float32) ** 3
        budgets = np.array([4096, 777])
    desc = kvc.make_desc(s, 8, 8, hkv, 64, 64, n_sink=4, n_recent=32, pool=1)
    scores = torch.from_numpy(vals).cuda()
    ws = kvc.alloc_workspace(desc)
    off = kvc.kvc_retained_offsets(desc, budgets)
    idx = torch.empty(int(off[-1]), dtype=torch.int32, device="cuda")
    kvc.kvc_select_topk(desc, scores, budgets, idx, ws)
    got = split_heads(idx.cpu().numpy(), off)
    for g in range(hkv):
        want = oracle.select_head(vals[g].astype(np.float64), int(budgets[g]), 4, 32)
        np.testing.assert_array_equal(got[g], want, err_msg=f"head {g}")


def test_gather_given_indices_strided_and_offset():
    rng = np.random.default_rng(4)
    s, hkv, d = 3000, 4, 128
    big_k = rng.integers(0, 65536, size=(s, 2 * hkv, d), dtype=np.uint16)  # K uses every other head slot
    big_v = rng.integers(0, 65536, size=(s, hkv, d + 64), dtype=np.uint16)  # V rows padded
    k_full, v_full = to_dev_bf16(big_k), to_dev_bf16(big_v)
    k = k_full[:, ::2, :]
    v = v_full[:, :, :d]
    k_host = big_k[:, ::2, :]
    v_host = big_v[:, :, :d]
    budgets = np.array([10, 0, 3000, 500])
    idx_l = [np.sort(rng.choice(s, size=min(int(bb), s), replace=False)) for bb in budgets]
    idx_flat = np.concatenate(idx_l).astype(np.int32)
    w = 4
    q = torch.zeros((w, hkv, d), dtype=torch.bfloat16, device="cuda")
    desc = kvc.desc_for(q, k, v, block=128, n_sink=0, n_recent=0, pos_offset=12345)
    off = kvc.kvc_retained_offsets(desc, budgets)
    rows = int(off[-1])
    k_out = torch.empty((rows, d), dtype=torch.bfloat16, device="cuda")
    v_out = torch.empty((rows, d), dtype=torch.bfloat16, device="cuda")
    pos = torch.empty(rows, dtype=torch.int32, device="cuda")
    kvc.kvc_gather_retained(desc, k, v, torch.from_numpy(idx_flat).cuda(), budgets, k_out, v_out, pos)
    kh, vh, ph = oracle.gather(k_host, v_host, idx_l, pos_offset=12345)
    np.testing.assert_array_equal(from_dev_bits(k_out), kh)
    np.testing.assert_array_equal(from_dev_bits(v_out), vh)
    np.testing.assert_array_equal(pos.cpu().numpy(), ph)


def test_strided_layer_equals_contiguous():
    cfg = get_config("tiny").with_(s=2500, hq=8, hkv=2, d=128, w=16, budget=200, n_heavy=10, sink_scale=4.0)
    x = layer_inputs(cfg, 3)
    q, k, v = dev_inputs(x)
    b = budgets_for(cfg, x)
    base = run_fused(desc_from(cfg, q, k, v), q, k, v, b)
    # the same tensors embedded in larger buffers
    qb = torch.zeros((cfg.w, cfg.hq + 3, cfg.d + 32), dtype=torch.bfloat16, device="cuda")
    qb[:, 1:1 + cfg.hq, 8:8 + cfg.d] = q
    kb = torch.zeros((cfg.s, cfg.hkv * 3, cfg.d), dtype=torch.bfloat16, device="cuda")
    kb[:, ::3, :] = k
    vb = torch.zeros((cfg.s, cfg.hkv, 2 * cfg.d), dtype=torch.bfloat16, device="cuda")
    vb[:, :, cfg.d:] = v
    qs, ks, vs = qb[:, 1:1 + cfg.hq, 8:8 + cfg.d], kb[:, ::3, :], vb[:, :, cfg.d:]
    got = run_fused(desc_from(cfg, qs, ks, vs), qs, ks, vs, b)
    for key in ["m", "z", "scores", "idx", "k_hat", "v_hat", "pos"]:
        np.testing.assert_array_equal(got[key], base[key], err_msg=key)


def test_identical_keys_exact_tie_break():
    """All keys equal: every prefix key gets the same score, and the lowest
    candidate indices must be chosen."""
    cfg = get_config("tiny").with_(s=2000, hq=4, hkv=1, d=64, w=16, budget=150, n_heavy=0)
    x = layer_inputs(cfg, 0)
    x.k[:] = x.k[5]
    q, k, v = dev_inputs(x)
    b = budgets_for(cfg, x)
    got = run_fused(desc_from(cfg, q, k, v), q, k, v, b)
    sc = got["scores"][0]
    prefix = sc[: cfg.s - cfg.w + 1]
    assert np.all(prefix == prefix[0]), "identical keys must score bitwise equal"
    want = oracle.select_head(oracle.scores(oracle.bf16_to_f64(x.q), oracle.bf16_to_f64(x.k))[0],
                              cfg.budget, cfg.n_sink, cfg.n_recent)
    np.testing.assert_array_equal(got["idx"], want)
    check_layer(x, got, b)


@pytest.mark.parametrize("log2_s", [18, 19])
def test_identical_keys_many_per_workgroup(log2_s):
    """All keys equal with 64 KV heads of D 64 and two window rows: one scan
    workgroup covers 2^17 (2^18 keys) or 2^16 (2^19 keys) keys of a head, all
    in one histogram bin. Every prefix key scores 1/(S-1) + 1/S (closed form,
    bitwise equal), and each head keeps the mandatory keys plus the lowest
    candidate indices."""
    s, hkv, d, w, budget, n_sink, n_recent = 1 << log2_s, 64, 64, 2, 4096, 4, 2
    desc = kvc.make_desc(s=s, w=w, hq=hkv, hkv=hkv, d=d, block=256, n_sink=n_sink, n_recent=n_recent)
    plan = kvc.kvc_plan_layer(desc)
    say(f"identical keys S=2^{log2_s}: {plan.keys_per_wg} keys per workgroup, histogram in scan {plan.hist_in_scan}")
    assert plan.scan == kvc.KVC_SCAN_STREAM and plan.hist_in_scan == (plan.keys_per_wg < 65536)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261202 + log2_s)
    q = torch.randn((w, hkv, d), generator=gen, device="cuda").to(torch.bfloat16)
    row = torch.randn((1, hkv, d), generator=gen, device="cuda").to(torch.bfloat16)
    k = row.expand(s, hkv, d).contiguous()
    # V rows encode (token, head, column) so the gather is checked bit for bit
    tok = torch.arange(s, device="cuda", dtype=torch.int32).view(s, 1, 1)
    code = (tok * 7 + torch.arange(hkv, device="cuda", dtype=torch.int32).view(1, hkv, 1) * 3
            + torch.arange(d, device="cuda", dtype=torch.int32).view(1, 1, d)) & 0x7F7F
    v = code.to(torch.int16).view(torch.bfloat16)
    b = np.full(hkv, budget, dtype=np.int64)
    ws = kvc.alloc_workspace(desc)
    out = kvc.alloc_outputs(desc, b)
    kvc.compress_layer(desc, q, k, v, b, out, ws)
    torch.cuda.synchronize()
    sc = out.scores.cpu().numpy()
    prefix = sc[:, : s - w + 1]
    assert np.all(prefix == prefix[:, :1]), "identical keys must score bitwise equal"
    closed = 1.0 / (s - 1) + 1.0 / s
    assert_scores_close(prefix[:, 0], np.full(hkv, closed), what="prefix score")
    want = np.concatenate([np.arange(budget - n_recent), np.arange(s - n_recent, s)]).astype(np.int32)
    idx = out.idx.cpu().numpy().reshape(hkv, budget)
    for g in range(hkv):
        np.testing.assert_array_equal(idx[g], want, err_msg=f"head {g}")
    np.testing.assert_array_equal(out.pos.cpu().numpy().reshape(hkv, budget), idx)
    kh = out.k_hat.view(hkv, budget, d)
    assert torch.equal(kh.view(torch.int16), row.view(torch.int16).view(hkv, 1, d).expand(hkv, budget, d))
    vh = out.v_hat.view(hkv, budget, d).view(torch.int16).cpu().numpy()
    wantv = v.view(torch.int16)[torch.from_numpy(want).long().cuda()].permute(1, 0, 2).cpu().numpy()
    np.testing.assert_array_equal(vh, wantv)


def test_deterministic_repeat():
    cfg = get_config("llama8b_16k").with_(s=8192)
    x = layer_inputs(cfg, 2)
    q, k, v = dev_inputs(x)
    b = budgets_for(cfg, x)
    desc = desc_from(cfg, q, k, v)
    a1 = run_fused(desc, q, k, v, b)
    a2 = run_fused(desc, q, k, v, b)
    for key in ["m", "z", "scores", "idx", "k_hat", "v_hat", "pos"]:
        np.testing.assert_array_equal(a1[key], a2[key], err_msg=key)


@pytest.mark.parametrize("name,s", [("tiny", None), ("llama8b_16k", 8192), ("llama8b_64k", None),
                                    ("qwen14b_hetero_64k", 8192)])
def test_fused_scans_need_no_workspace_init(name, s):
    """Where the scans run as one launch (pass 1, split merge, pass 2 with
    waits between workgroups), the outputs equal the staged calls' bit for
    bit whatever the workspace held before: zeros, all ones, random bytes,
    or a previous call's state."""
    cfg = get_config(name) if s is None else get_config(name).with_(s=s)
    x = layer_inputs(cfg, 5)
    q, k, v = dev_inputs(x)
    b = budgets_for(cfg, x)
    desc = desc_from(cfg, q, k, v)
    plan = kvc.kvc_plan_layer(desc)
    say(f"{name} s={cfg.s}: fused scans {plan.fused_scans}, splits {plan.splits}, heads per workgroup {plan.heads_per_wg}")
    assert plan.scan == kvc.KVC_SCAN_STREAM and plan.fused_scans == 1
    st = run_staged(desc, q, k, v, b)
    ws = kvc.alloc_workspace(desc)
    gen = torch.Generator(device="cuda").manual_seed(11)
    fills = [("zeros", lambda: ws.zero_()), ("ones", lambda: ws.fill_(255)),
             ("random", lambda: ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8, device="cuda", generator=gen))),
             ("previous call", lambda: None)]
    for label, fill in fills:
        fill()
        out = kvc.alloc_outputs(desc, b)
        kvc.compress_layer(desc, q, k, v, b, out, ws)
        torch.cuda.synchronize()
        got = host(out)
        for key in ["m", "z", "scores", "idx", "k_hat", "v_hat", "pos"]:
            np.testing.assert_array_equal(got[key], st[key], err_msg=f"{label}: {key}")


@pytest.mark.parametrize("name,over", [("tiny", {}), ("llama8b_16k", {"s": 8192}), ("llama8b_16k", {"s": 3001, "w": 64}),
                                       ("llama8b_16k", {"s": 4096, "pool": 7})])
def test_score_layer_equals_staged_and_whole_layer(name, over):
    """kvc_score_layer (both scans as the whole-layer call runs them: one
    launch where it fuses them, per-head scans for wide windows) writes the
    staged passes' m, Z and scores bit for bit, and the whole-layer call's."""
    cfg = get_config(name).with_(**over) if over else get_config(name)
    x = layer_inputs(cfg, 6)
    q, k, v = dev_inputs(x)
    b = budgets_for(cfg, x)
    desc = desc_from(cfg, q, k, v)
    plan = kvc.kvc_plan_layer(desc)
    say(f"{name} {over}: scan kind {plan.scan}, fused {plan.fused_scans}")
    st = run_staged(desc, q, k, v, b)
    fu = run_fused(desc, q, k, v, b)
    ws = kvc.alloc_workspace(desc)
    ws.fill_(255)
    out = kvc.alloc_outputs(desc, b)
    kvc.kvc_score_layer(desc, q, k, out.m, out.z, out.scores, ws)
    torch.cuda.synchronize()
    for key in ["m", "z", "scores"]:
        got = getattr(out, key).cpu().numpy()
        np.testing.assert_array_equal(got, st[key], err_msg=f"staged {key}")
        np.testing.assert_array_equal(got, fu[key], err_msg=f"whole layer {key}")
    # outputs may live in the workspace
    kvc.kvc_score_layer(desc, q, k, None, None, None, ws)
    torch.cuda.synchronize()


@pytest.mark.parametrize("name,s,n_layers", [("llama8b_16k", 8192, 5), ("qwen14b_hetero_64k", 8192, 4)])
def test_sweep_equals_layer_by_layer(name, s, n_layers):
    """kvc_compress_layers over several layers (alternating between the
    caller's two streams) writes what one kvc_compress_layer call per layer
    writes, bit for bit, and later work on the caller's stream sees all of
    it; so does a sweep on one stream."""
    cfg = get_config(name).with_(s=s)
    xs = [layer_inputs(cfg, l) for l in range(n_layers)]
    layers = [dev_inputs(x) for x in xs]
    budgets = np.stack([budgets_for(cfg, x) for x in xs])
    desc = desc_from(cfg, *layers[0])
    say(f"sweep {name}: {n_layers} layers one by one")
    want = [run_fused(desc, *layers[i], budgets[i], intermediates=False) for i in range(n_layers)]
    outs = [kvc.alloc_outputs(desc, budgets[i], with_intermediates=False) for i in range(n_layers)]
    for o in outs:  # stale contents must all be overwritten
        o.idx.fill_(-7)
        o.k_hat.view(torch.int16).fill_(-7)
    ws = kvc.alloc_sweep_workspace(desc)
    say(f"sweep {name}: one sweep call")
    kvc.kvc_compress_layers(desc, layers, budgets, outs, ws, aux_stream=torch.cuda.Stream())
    # ordered after the sweep on the caller's stream, no host synchronisation
    copies = [(o.idx.clone(), o.k_hat.clone(), o.v_hat.clone(), o.pos.clone()) for o in outs]
    torch.cuda.synchronize()
    for i in range(n_layers):
        np.testing.assert_array_equal(copies[i][0].cpu().numpy(), want[i]["idx"], err_msg=f"idx {i}")
        np.testing.assert_array_equal(from_dev_bits(copies[i][1]), want[i]["k_hat"], err_msg=f"k_hat {i}")
        np.testing.assert_array_equal(from_dev_bits(copies[i][2]), want[i]["v_hat"], err_msg=f"v_hat {i}")
        np.testing.assert_array_equal(copies[i][3].cpu().numpy(), want[i]["pos"], err_msg=f"pos {i}")
    # a second sweep into the same buffers gives the same bits again
    kvc.kvc_compress_layers(desc, layers, budgets, outs, ws, aux_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    for i in range(n_layers):
        np.testing.assert_array_equal(outs[i].idx.cpu().numpy(), want[i]["idx"], err_msg=f"repeat idx {i}")
    # one stream (the scans may then fuse, as in kvc_compress_layer)
    for o in outs:
        o.idx.fill_(-7)
    kvc.kvc_compress_layers(desc, layers, budgets, outs, ws[:kvc.kvc_workspace_size(desc)])
    torch.cuda.synchronize()
    for i in range(n_layers):
        np.testing.assert_array_equal(outs[i].idx.cpu().numpy(), want[i]["idx"], err_msg=f"one-stream idx {i}")
        np.testing.assert_array_equal(from_dev_bits(outs[i].k_hat), want[i]["k_hat"], err_msg=f"one-stream k_hat {i}")


def test_binding_errors_on_gpu():
    cfg = get_config("tiny")
    x = layer_inputs(cfg, 0)
    q, k, v = dev_inputs(x)
    desc = desc_from(cfg, q, k, v)
    b = budgets_for(cfg, x)
    out = kvc.alloc_outputs(desc, b)
    small = torch.empty(kvc.kvc_workspace_size(desc) - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(kvc.KvcError) as e:
        kvc.compress_layer(desc, q, k, v, b, out, small)
    assert e.value.status == kvc.KVC_ERR_WORKSPACE
    with pytest.raises(ValueError):
        kvc.kvc_score_pass2(desc, q.cpu(), k, out.m, out.z, out.scores)


# --------------------------------------------------------------------------- full size (sampled)

def full_size_case(name, layer, heads):
    cfg = get_config(name)
    say(f"{name} layer {layer}: generating")
    x = layer_inputs(cfg, layer)
    q, k, v = dev_inputs(x)
    b = budgets_for(cfg, x)
    if cfg.hetero:
        np.testing.assert_array_equal(kvc.kvc_budgets_inverse_stability(x.s_stable, cfg.total_budget), b)
    desc = desc_from(cfg, q, k, v)
    say(f"{name}: GPU")
    got = run_fused(desc, q, k, v, b)
    np.testing.assert_allclose(got["scores"].sum(axis=1, dtype=np.float64), cfg.w * cfg.group, rtol=1e-4)
    say(f"{name}: oracle on heads {heads}")
    check_layer(x, got, b, heads=heads)


def test_full_size_llama8b_64k_all_heads():
    full_size_case("llama8b_64k", 0, heads=list(range(8)))


def test_full_size_llama8b_128k_sampled():
    full_size_case("llama8b_128k", 0, heads=[0, 5])


def test_full_size_llama8b_128k_pool7_sampled():
    full_size_case("llama8b_128k_pool7", 0, heads=[3])


def test_full_size_qwen14b_hetero_sampled():
    full_size_case("qwen14b_hetero_64k", 1, heads=[2])


# --------------------------------------------------------------------------- the largest prompt

def test_maximum_prompt_length():
    """S = 2^23, the library's limit (every sub-chunk tag in use): one KV head
    and two window rows, so the oracle stays cheap; 20000 keys retained."""
    cfg = get_config("tiny").with_(name="max_prompt", s=1 << 23, w=2, hq=1, hkv=1, d=64, block=256, n_sink=4,
                                   n_recent=2, n_heavy=2000, budget=20000, sink_scale=4.0, seed_base=888)
    say("max prompt: generating 2^23 keys")
    x = layer_inputs(cfg, 0)
    q, k, v = dev_inputs(x)
    b = np.array([cfg.budget])
    desc = desc_from(cfg, q, k, v)
    say("max prompt: GPU")
    got = run_fused(desc, q, k, v, b)
    np.testing.assert_allclose(got["scores"].sum(axis=1, dtype=np.float64), cfg.w * cfg.group, rtol=1e-4)
    say("max prompt: oracle")
    check_layer(x, got, b)


# --------------------------------------------------------------------------- selection inside the scan launch

FSEL_CASES = [
    ("tiny", {}, None),
    ("llama8b_16k", {"s": 8192}, None),
    ("llama8b_16k", {"s": 5000}, None),
    ("llama8b_16k", {"s": 3333, "w": 7}, None),
    ("llama8b_16k", {"s": 2049, "hq": 16, "w": 16}, None),
    ("llama8b_16k", {"s": 2000}, "keep_all"),
    ("llama8b_16k", {"s": 6000}, "mandatory_only"),
    ("llama8b_16k", {"s": 9000}, "mixed"),
    ("llama8b_64k", {}, None),
    ("llama8b_64k", {"s": 131072}, None),
    # 160 and 192 query rows per KV head (five and six row tiles)
    ("qwen14b_hetero_64k", {"s": 9000}, None),
    ("llama8b_16k", {"s": 7001, "hq": 48, "hkv": 8, "w": 32}, "mixed"),
    ("llama8b_16k", {"s": 5003, "hq": 15, "hkv": 3, "w": 32}, None),
]


def _fsel_budgets(cfg, x, kind):
    b = budgets_for(cfg, x)
    if kind == "keep_all":
        return np.full(cfg.hkv, cfg.s + 5, dtype=np.int64)
    if kind == "mandatory_only":
        return np.full(cfg.hkv, cfg.n_sink + cfg.n_recent, dtype=np.int64)
    if kind == "mixed":
        rng = np.random.default_rng(7)
        m = cfg.n_sink + cfg.n_recent
        return np.array([rng.choice([m, m + 1, 700, 3000, cfg.s, cfg.s + 9]) for _ in range(cfg.hkv)], dtype=np.int64)
    return b


def _staged_select(desc, q, k, v, scores, b):
    """The staged selection and gather on given scores (a device tensor)."""
    ws = kvc.alloc_workspace(desc)
    out = kvc.alloc_outputs(desc, b)
    kvc.kvc_select_topk(desc, scores, b, out.idx, ws)
    kvc.kvc_gather_retained(desc, k, v, out.idx, b, out.k_hat, out.v_hat, out.pos)
    torch.cuda.synchronize()
    return host(out)


def _fused_select_run(fdesc, q, k, v, b, intermediates=True):
    ws = kvc.alloc_workspace(fdesc)
    ws.fill_(255)  # no initialisation needed
    out = kvc.alloc_outputs(fdesc, b, with_intermediates=intermediates)
    kvc.compress_layer(fdesc, q, k, v, b, out, ws)
    torch.cuda.synchronize()
    return host(out), out


@pytest.mark.parametrize("name,over,kind", FSEL_CASES)
def test_fused_select_equals_staged_selection(name, over, kind):
    """KVC_FLAG_FUSED_SELECT (scans, selection and gather in one launch, the
    scores kept on chip): its retained set and rows equal, bit for bit, what
    the staged selection and gather make of the same call's scores; its
    scores, m and Z match the unflagged call's to float rounding (one KV head
    per workgroup merges pass 1's partials in another order; with one KV head
    per layer the order is the same and so are the bits), and the oracle's
    within the parity tolerance."""
    cfg = get_config(name).with_(**over) if over else get_config(name)
    x = layer_inputs(cfg, 8)
    q, k, v = dev_inputs(x)
    b = _fsel_budgets(cfg, x, kind)
    desc = desc_from(cfg, q, k, v)
    fdesc = desc_from(cfg, q, k, v, flags=kvc.KVC_FLAG_FUSED_SELECT)
    plan = kvc.kvc_plan_layer(fdesc)
    say(f"fused select {name} {over} {kind}: splits {plan.splits}, keys per workgroup {plan.keys_per_wg}, "
        f"workspace {plan.workspace_bytes} B (unflagged {kvc.kvc_workspace_size(desc)} B)")
    assert plan.fused_select == 1
    got, out = _fused_select_run(fdesc, q, k, v, b)
    sel = _staged_select(desc, q, k, v, out.scores, b)
    for key in ["idx", "k_hat", "v_hat", "pos"]:
        np.testing.assert_array_equal(got[key], sel[key], err_msg=key)
    want = run_fused(desc, q, k, v, b)
    for key in ["m", "z", "scores"]:
        if cfg.hkv == 1:
            np.testing.assert_array_equal(got[key], want[key], err_msg=key)
        else:
            np.testing.assert_allclose(got[key], want[key], rtol=2e-6, atol=1e-30, err_msg=key)
    check_layer(x, got, b, heads=[0, cfg.hkv - 1])  # the fp64 oracle on two heads, full size included
    got2, _ = _fused_select_run(fdesc, q, k, v, b, intermediates=False)
    for key in ["idx", "k_hat", "v_hat", "pos"]:
        np.testing.assert_array_equal(got2[key], got[key], err_msg=f"no intermediates: {key}")


def test_fused_select_identical_keys_tie_break():
    """All keys equal: every candidate ties, and the lowest indices are kept
    (the radix rounds count ties exactly; there is no list to overflow)."""
    cfg = get_config("llama8b_16k").with_(s=12000)
    x = layer_inputs(cfg, 1)
    kk = np.repeat(x.k[:1], cfg.s, axis=0)
    q, k, v = to_dev_bf16(x.q), to_dev_bf16(kk), to_dev_bf16(x.v)
    b = np.full(cfg.hkv, 1000, dtype=np.int64)
    fdesc = desc_from(cfg, q, k, v, flags=kvc.KVC_FLAG_FUSED_SELECT)
    got, out = _fused_select_run(fdesc, q, k, v, b)
    sel = _staged_select(desc_from(cfg, q, k, v), q, k, v, out.scores, b)
    for key in ["idx", "k_hat", "v_hat", "pos"]:
        np.testing.assert_array_equal(got[key], sel[key], err_msg=key)
    n_free = 1000 - cfg.n_sink - cfg.n_recent
    expect = np.concatenate([np.arange(cfg.n_sink), np.arange(cfg.n_sink, cfg.n_sink + n_free),
                             np.arange(cfg.s - cfg.n_recent, cfg.s)])
    for g, first in enumerate(split_heads(got["idx"], got["offsets"])):
        np.testing.assert_array_equal(first, expect, err_msg=f"head {g}")


def test_fused_select_offset_noalloc_and_sweep():
    """The flag with a position offset, through the no-allocation call, and
    through the sweep (which then runs its layers on one stream): the same
    bits as one flagged kvc_compress_layer call per layer."""
    cfg = get_config("llama8b_16k").with_(s=8192)
    xs = [layer_inputs(cfg, l) for l in range(3)]
    layers = [dev_inputs(x) for x in xs]
    budgets = np.stack([budgets_for(cfg, x) for x in xs])
    fdesc = desc_from(cfg, *layers[0], pos_offset=12345, flags=kvc.KVC_FLAG_FUSED_SELECT)
    want = [_fused_select_run(fdesc, *layers[i], budgets[i], intermediates=False)[0] for i in range(3)]
    assert want[0]["pos"].min() >= 12345
    out = kvc.alloc_outputs(fdesc, budgets[0], with_intermediates=False)
    kvc.kvc_compress_layer_noalloc(fdesc, *layers[0], budgets[0], out.idx, out.k_hat, out.v_hat, out.pos)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.idx.cpu().numpy(), want[0]["idx"])
    np.testing.assert_array_equal(out.pos.cpu().numpy(), want[0]["pos"])
    np.testing.assert_array_equal(from_dev_bits(out.k_hat), want[0]["k_hat"])
    outs = [kvc.alloc_outputs(fdesc, budgets[i], with_intermediates=False) for i in range(3)]
    kvc.kvc_compress_layers(fdesc, layers, budgets, outs, kvc.alloc_sweep_workspace(fdesc),
                            aux_stream=torch.cuda.Stream())
    torch.cuda.synchronize()
    for i in range(3):
        np.testing.assert_array_equal(outs[i].idx.cpu().numpy(), want[i]["idx"], err_msg=f"sweep idx {i}")
        np.testing.assert_array_equal(from_dev_bits(outs[i].v_hat), want[i]["v_hat"], err_msg=f"sweep v_hat {i}")
        np.testing.assert_array_equal(outs[i].pos.cpu().numpy(), want[i]["pos"], err_msg=f"sweep pos {i}")


_RENDEZVOUS_SCRIPT = r"""
import sys
import numpy as np
import torch
sys.path.insert(0, sys.argv[1])
sys.path.insert(0, sys.argv[1] + "/tests")
import compression_kvc_score_amd as kvc
from synth import get_config, layer_inputs
from gpu_util import desc_from, host
out_path = sys.argv[2]
res = {}
for name, s in (("llama8b_16k", None), ("llama8b_64k", None), ("llama8b_16k", 3000)):
    cfg = get_config(name).with_(s=s) if s else get_config(name)
    x = layer_inputs(cfg, 3)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
               for a in (x.q, x.k, x.v))
    b = np.full(cfg.hkv, min(cfg.budget, cfg.s), dtype=np.int64)
    for flags in (kvc.KVC_FLAG_FUSED_SELECT, 0):
        d = desc_from(cfg, q, k, v, flags=flags)
        ws = kvc.alloc_workspace(d)
        out = kvc.alloc_outputs(d, b)
        kvc.compress_layer(d, q, k, v, b, out, ws)
        torch.cuda.synchronize()
        for key, val in host(out).items():
            res[f"{name}_{cfg.s}_{flags}_{key}"] = val
np.savez(out_path, **res)
"""


def test_rendezvous_through_l2_or_memory_same_bits(tmp_path):
    """Head groups whose workgroups all run on one XCD meet through its L2
    after their first rendezvous; KVC_XCD_LOCAL=0 makes every rendezvous go
    through device-coherent memory. The outputs (fused selection and the
    default call, m, Z, scores, indices, rows, positions) are the same bits
    either way. (The switch is read once per process: two child processes.)"""
    import os
    import subprocess
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    paths = {}
    for local in ("1", "0"):
        paths[local] = str(tmp_path / f"out_{local}.npz")
        env = dict(os.environ, KVC_XCD_LOCAL=local)
        say(f"rendezvous run with KVC_XCD_LOCAL={local}")
        subprocess.run([sys.executable, "-c", _RENDEZVOUS_SCRIPT, root, paths[local]], env=env, check=True,
                       timeout=240)
    a, b = np.load(paths["1"]), np.load(paths["0"])
    assert sorted(a.files) == sorted(b.files) and len(a.files) > 0
    for key in a.files:
        np.testing.assert_array_equal(a[key], b[key], err_msg=key)
