"""GPU parity of immediate (chunk-boundary) eviction (TideKV, Fig. 1 caption,
schedule (c); Table 8, Block-SnapKV) through the C ABI against the CPU oracle.

Every boundary is checked on the GPU's own state, after kvc_evict_chunk:
- the current arena holds the keys retained so far followed by the chunk,
  bit for bit, with their positions;
- the scores that the staged calls compute on that arena are within the
  score tolerance of the oracle's on the same keys (bit for bit in INT8);
- the next arena holds exactly the rows that the oracle's selection rule
  picks from the GPU's scores, positions carried; the oracle's own choice on
  its fp64 scores differs only inside the tie band.
When no boundary differs from the oracle's own choice, the final retained set
equals the oracle's whole-prompt result (oracle.compress_chunked) exactly. The
whole-prompt entry point kvc_compress_chunked equals the boundary-by-boundary
chain bit for bit.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import compression_kvc_score_amd as kvc  # noqa: E402
import oracle  # noqa: E402
from synth import chunk_windows, get_config, layer_inputs  # noqa: E402

from gpu_util import from_dev_bits, to_dev_bf16  # noqa: E402
from parity import assert_scores_close, assert_selection_matches  # noqa: E402

MODES = {"softmax": kvc.KVC_SCORE_SOFTMAX, "logit": kvc.KVC_SCORE_LOGIT, "int8": kvc.KVC_SCORE_LOGIT_INT8}
FSEL = kvc.KVC_FLAG_FUSED_SELECT


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    kvc.lib()


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def chunk_desc(cfg, c, pos_offset, mode, pool, flags=0):
    hq, hkv, d = cfg.hq, cfg.hkv, cfg.d
    return kvc.make_desc(c, cfg.w, hq, hkv, d, block=cfg.block, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                         pool=pool, pos_offset=pos_offset, score_mode=MODES[mode],
                         q_strides=(hq * d, d), k_strides=(hkv * d, d), v_strides=(hkv * d, d), flags=flags)


def gpu_arena_scores(cfg, q_win, arena, s_acc, cap, mode):
    """Scores of the arena's first s_acc rows by the staged calls."""
    d = cfg.d
    desc = kvc.make_desc(s_acc, cfg.w, cfg.hq, cfg.hkv, d, block=cfg.block, n_sink=cfg.n_sink,
                         n_recent=cfg.n_recent, score_mode=MODES[mode], q_strides=(cfg.hq * d, d),
                         k_strides=(d, cap * d), v_strides=(d, cap * d))
    scores = torch.empty((cfg.hkv, s_acc), dtype=torch.float32, device="cuda")
    m = z = None
    if mode == "softmax":
        ws = kvc.alloc_workspace(desc)
        m = torch.empty((cfg.hq, cfg.w), dtype=torch.float32, device="cuda")
        z = torch.empty_like(m)
        kvc.kvc_score_pass1(desc, q_win, arena[0], m, z, ws)
    kvc.kvc_score_pass2(desc, q_win, arena[0], m, z, scores)
    torch.cuda.synchronize()
    return scores.cpu().numpy()


def oracle_arena_scores(q_bits, k_acc_bits, mode):
    """Oracle scores [hkv, s_acc] of accumulated keys k_acc_bits [s_acc, hkv, d]."""
    if mode == "int8":
        return oracle.logit_scores_int8(q_bits, k_acc_bits).astype(np.float64)
    q = oracle.bf16_to_f64(q_bits)
    k = oracle.bf16_to_f64(k_acc_bits)
    return oracle.scores(q, k) if mode == "softmax" else oracle.logit_scores(q, k)


def logit_bound(q_bits, k_bits):
    """|GPU - exact| bound of fp32 logit scores (D + 8 roundings of the sum of
    |pooled query x key| terms)."""
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


def check_boundary_selection(cfg, mode, pool, budget, gs, ws_, err, k_acc, g):
    """Head g: the oracle's own selection on its scores may differ from the
    GPU's (made on the GPU's scores) only near the threshold. Returns True if
    they differ."""
    s_acc = gs.shape[1]
    gv = oracle.maxpool(gs.astype(np.float64), pool) if pool > 1 else gs.astype(np.float64)
    wv = oracle.maxpool(ws_, pool) if pool > 1 else ws_
    got = oracle.select_head(gv[g], budget, cfg.n_sink, cfg.n_recent)
    want = oracle.select_head(wv[g], budget, cfg.n_sink, cfg.n_recent)
    if mode == "softmax":
        assert_selection_matches(got, want, wv[g], budget, cfg.n_sink, cfg.n_recent)
    elif mode == "int8":
        np.testing.assert_array_equal(got, want)
    else:
        diff = np.setxor1d(got, want)
        if diff.size:
            mand = oracle.mandatory(s_acc, cfg.n_sink, cfg.n_recent)
            cand = np.setdiff1d(np.arange(s_acc), mand)
            tau = np.sort(wv[g][cand])[::-1][budget - mand.size - 1]
            band = 2 * err[g].max() if pool > 1 else 2 * err[g][diff]
            assert np.all(np.abs(wv[g][diff] - tau) <= band), f"head {g}: differences outside the error band"
    return got, not np.array_equal(got, want)


def run_chain(cfg, x, qw_bits, budget, mode="softmax", pool=1, pos_offset=0, flags=0):
    """kvc_evict_chunk boundary by boundary, each boundary checked; returns
    the final (K rows [hkv, n, d], V rows, positions [hkv, n]) and whether any
    boundary's selection differed from the oracle's own. With the fused-
    selection flag a boundary's scores stay on chip: its retained set is then
    checked against the oracle's (tie band), rows and positions against the
    arena."""
    chunk, s, w, hkv, d = cfg.chunk, cfg.s, cfg.w, cfg.hkv, cfg.d
    cap = min(budget + chunk, s)
    k_dev, v_dev, qw_dev = to_dev_bf16(x.k), to_dev_bf16(x.v), to_dev_bf16(qw_bits)
    arenas = [kvc.alloc_arena(hkv, cap, d), kvc.alloc_arena(hkv, cap, d)]
    ws = torch.empty(kvc.kvc_chunk_workspace_size(chunk_desc(cfg, min(chunk, s), pos_offset, mode, pool, flags), cap),
                     dtype=torch.uint8, device="cuda")
    cur, n_kept, flipped = 0, 0, False
    kept_k = np.zeros((hkv, 0, d), np.uint16)
    kept_v = np.zeros((hkv, 0, d), np.uint16)
    kept_p = np.zeros((hkv, 0), np.int32)
    for b, (c0, c1) in enumerate(oracle.chunk_bounds(s, chunk)):
        c, s_acc = c1 - c0, n_kept + c1 - c0
        desc = chunk_desc(cfg, c, pos_offset + c0, mode, pool, flags)
        q_win = qw_dev[b * w:(b + 1) * w]
        evict = s_acc > budget
        kvc.kvc_evict_chunk(desc, q_win, k_dev[c0:c1], v_dev[c0:c1], budget, n_kept, cap, arenas[cur],
                            arenas[1 - cur] if evict else None, ws if evict else None)
        torch.cuda.synchronize()
        ak = from_dev_bits(arenas[cur][0])[:, :s_acc]
        av = from_dev_bits(arenas[cur][1])[:, :s_acc]
        ap = arenas[cur][2].cpu().numpy()[:, :s_acc]
        # the append: retained rows untouched, the chunk behind them
        np.testing.assert_array_equal(ak[:, :n_kept], kept_k, err_msg=f"chunk {b}: retained K rows changed")
        np.testing.assert_array_equal(av[:, :n_kept], kept_v)
        np.testing.assert_array_equal(ap[:, :n_kept], kept_p)
        np.testing.assert_array_equal(ak[:, n_kept:], x.k[c0:c1].transpose(1, 0, 2), err_msg=f"chunk {b}: appended K")
        np.testing.assert_array_equal(av[:, n_kept:], x.v[c0:c1].transpose(1, 0, 2))
        np.testing.assert_array_equal(ap[:, n_kept:], np.broadcast_to(np.arange(pos_offset + c0, pos_offset + c1), (hkv, c)))
        if not evict:
            kept_k, kept_v, kept_p, n_kept = ak, av, ap, s_acc
            continue
        k_acc = np.ascontiguousarray(ak.transpose(1, 0, 2))
        q_bits = qw_bits[b * w:(b + 1) * w]
        gs = gpu_arena_scores(cfg, q_win, arenas[cur], s_acc, cap, mode)
        want = oracle_arena_scores(q_bits, k_acc, mode)
        err = None
        if mode == "softmax":
            assert_scores_close(gs, want, what=f"chunk {b} scores")
        elif mode == "int8":
            np.testing.assert_array_equal(gs.astype(np.float64), want, err_msg=f"chunk {b} INT8 scores")
        else:
            err = logit_bound(q_bits, k_acc)
            assert np.all(np.abs(gs - want) <= err), f"chunk {b}: logit scores outside the rounding bound"
        nk = from_dev_bits(arenas[1 - cur][0])[:, :budget]
        nv = from_dev_bits(arenas[1 - cur][1])[:, :budget]
        npos = arenas[1 - cur][2].cpu().numpy()[:, :budget]
        for g in range(hkv):
            if flags & FSEL:
                got = np.searchsorted(ap[g], npos[g])
                assert np.all(got < s_acc) and np.array_equal(ap[g, np.minimum(got, s_acc - 1)], npos[g]), \
                    f"chunk {b} head {g}: retained positions not among the accumulated keys"
                own = oracle.select_head(want[g], budget, cfg.n_sink, cfg.n_recent)
                assert_selection_matches(got, own, want[g], budget, cfg.n_sink, cfg.n_recent)
                diff = not np.array_equal(got, own)
            else:
                got, diff = check_boundary_selection(cfg, mode, pool, budget, gs, want, err, k_acc, g)
            flipped |= diff
            np.testing.assert_array_equal(nk[g], ak[g, got], err_msg=f"chunk {b} head {g}: retained K rows")
            np.testing.assert_array_equal(nv[g], av[g, got])
            np.testing.assert_array_equal(npos[g], ap[g, got], err_msg=f"chunk {b} head {g}: carried positions")
        kept_k, kept_v, kept_p, n_kept = nk, nv, npos, budget
        cur = 1 - cur
    return kept_k, kept_v, kept_p, flipped


def run_driver(cfg, x, qw_bits, budget, mode="softmax", pool=1, pos_offset=0, flags=0):
    hq, hkv, d = cfg.hq, cfg.hkv, cfg.d
    desc = kvc.make_desc(cfg.s, cfg.w, hq, hkv, d, block=cfg.block, n_sink=cfg.n_sink, n_recent=cfg.n_recent,
                         pool=pool, pos_offset=pos_offset, score_mode=MODES[mode], flags=flags)
    rows = min(budget, cfg.s)
    k_out = torch.empty((hkv, rows, d), dtype=torch.bfloat16, device="cuda")
    v_out = torch.empty_like(k_out)
    pos = torch.empty((hkv, rows), dtype=torch.int32, device="cuda")
    ws = torch.empty(kvc.kvc_chunked_workspace_size(desc, cfg.chunk, budget), dtype=torch.uint8, device="cuda")
    kvc.kvc_compress_chunked(desc, cfg.chunk, to_dev_bf16(qw_bits), to_dev_bf16(x.k), to_dev_bf16(x.v), budget,
                             k_out, v_out, pos, ws)
    torch.cuda.synchronize()
    return from_dev_bits(k_out), from_dev_bits(v_out), pos.cpu().numpy()


def check_case(cfg, budget, mode="softmax", pool=1, pos_offset=0, layer=0, flags=0):
    x = layer_inputs(cfg, layer)
    qw = chunk_windows(cfg, cfg.chunk, layer, q_last=x.q)
    say(f"chunked {cfg.name} s={cfg.s} C={cfg.chunk} budget={budget} {mode} pool={pool} flags={flags}: chain")
    ck, cv, cp, flipped = run_chain(cfg, x, qw, budget, mode, pool, pos_offset, flags)
    say("  driver")
    dk, dv, dp = run_driver(cfg, x, qw, budget, mode, pool, pos_offset, flags)
    np.testing.assert_array_equal(dk, ck, err_msg="driver K differs from the boundary chain")
    np.testing.assert_array_equal(dv, cv)
    np.testing.assert_array_equal(dp, cp)
    say(f"  oracle (boundary selections differed: {flipped})")
    nb = len(oracle.chunk_bounds(cfg.s, cfg.chunk))
    want = oracle.compress_chunked(qw.reshape(nb, cfg.w, cfg.hq, cfg.d), x.k, x.v, cfg.chunk, budget, cfg.n_sink,
                                   cfg.n_recent, pool=pool, pos_offset=pos_offset, score_mode=mode)
    if not flipped:
        rows = min(budget, cfg.s)
        for g in range(cfg.hkv):
            np.testing.assert_array_equal(dp[g] - pos_offset, want.idx[g], err_msg=f"head {g}: final retained set")
        np.testing.assert_array_equal(dk.reshape(-1, cfg.d), want.k_hat)
        np.testing.assert_array_equal(dv.reshape(-1, cfg.d), want.v_hat)
        np.testing.assert_array_equal(dp.reshape(-1), want.pos)
        assert dk.shape[1] == rows
    return flipped


SMALL = {
    # one KV head, ragged last chunk (1024 = 6 x 160 + 64)
    "tiny": dict(cfg=("tiny", dict(chunk=160)), budget=128),
    # max-pool 5 and a position offset, last chunk 24 tokens (>= w = 16)
    "tiny_pool5_offset": dict(cfg=("tiny", dict(chunk=100)), budget=150, pool=5, pos_offset=1000),
    # first chunk already above the budget
    "tiny_chunk_over_budget": dict(cfg=("tiny", dict(chunk=512)), budget=100),
    # Llama-3.1-8B heads (GQA 4) on a 3000-token prompt, 700-token chunks
    "gqa_3000": dict(cfg=("llama8b_16k", dict(s=3000, chunk=700, n_heavy=30)), budget=600),
}


@pytest.mark.parametrize("name", sorted(SMALL))
def test_chunked_small_softmax(name):
    c = SMALL[name]
    base, kw = c["cfg"]
    cfg = get_config(base).with_(**kw)
    check_case(cfg, c["budget"], pool=c.get("pool", 1), pos_offset=c.get("pos_offset", 0))


@pytest.mark.parametrize("mode", ["logit", "int8"])
def test_chunked_score_modes(mode):
    cfg = get_config("llama8b_16k").with_(s=3000, chunk=700, n_heavy=30)
    check_case(cfg, 600, mode=mode)


def test_chunked_budget_covering_the_prompt_keeps_everything():
    cfg = get_config("tiny").with_(chunk=200)  # last chunk 24 tokens
    x = layer_inputs(cfg, 0)
    qw = chunk_windows(cfg, cfg.chunk, 0, q_last=x.q)
    dk, dv, dp = run_driver(cfg, x, qw, cfg.s + 5)
    np.testing.assert_array_equal(dk[0], x.k[:, 0, :])
    np.testing.assert_array_equal(dv[0], x.v[:, 0, :])
    np.testing.assert_array_equal(dp[0], np.arange(cfg.s))


def test_chunked_one_chunk_equals_the_layer_compressor():
    """A single chunk is the one-shot compressor: same rows and positions as
    kvc_compress_layer."""
    cfg = get_config("llama8b_16k").with_(s=2048, chunk=2048, n_heavy=20, budget=512)
    x = layer_inputs(cfg, 0)
    dk, dv, dp = run_driver(cfg, x, x.q, cfg.budget)
    q, k, v = to_dev_bf16(x.q), to_dev_bf16(x.k), to_dev_bf16(x.v)
    desc = kvc.desc_for(q, k, v, block=cfg.block, n_sink=cfg.n_sink, n_recent=cfg.n_recent)
    b = np.full(cfg.hkv, cfg.budget)
    out = kvc.alloc_outputs(desc, b, with_intermediates=False)
    kvc.compress_layer(desc, q, k, v, b, out, kvc.alloc_workspace(desc))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dk.reshape(-1, cfg.d), from_dev_bits(out.k_hat))
    np.testing.assert_array_equal(dv.reshape(-1, cfg.d), from_dev_bits(out.v_hat))
    np.testing.assert_array_equal(dp.reshape(-1), out.pos.cpu().numpy())


def test_chunked_table8_setting_full_size():
    """The Block-SnapKV setting the benchmark times: Llama-3.1-8B layer, 16K
    prompt, 512-token chunks, 1024 keys per head, every boundary checked."""
    cfg = get_config("llama8b_16k_imm")
    check_case(cfg, cfg.budget)


@pytest.mark.parametrize("name", ["tiny", "tiny_chunk_over_budget", "gqa_3000"])
def test_chunked_fused_select(name):
    """With KVC_FLAG_FUSED_SELECT every evicting boundary is one launch
    (scans, selection and gather, the scores kept on chip): each boundary's
    retained set is the oracle's up to the tie band with rows and positions
    carried from the arena, the whole-prompt driver equals the boundary chain
    bit for bit, and with one KV head (one head per workgroup either way) the
    result equals the unflagged path's bit for bit."""
    c = SMALL[name]
    base, kw = c["cfg"]
    cfg = get_config(base).with_(**kw)
    check_case(cfg, c["budget"], flags=FSEL)
    if cfg.hkv == 1:
        x = layer_inputs(cfg, 0)
        qw = chunk_windows(cfg, cfg.chunk, 0, q_last=x.q)
        plain = run_driver(cfg, x, qw, c["budget"])
        fused = run_driver(cfg, x, qw, c["budget"], flags=FSEL)
        for a, b in zip(plain, fused):
            np.testing.assert_array_equal(a, b)


def test_chunked_fused_select_table8_setting_full_size():
    """The Block-SnapKV setting the benchmark times, every boundary as one
    launch with the scores on chip, every boundary checked."""
    cfg = get_config("llama8b_16k_imm")
    check_case(cfg, cfg.budget, flags=FSEL)
