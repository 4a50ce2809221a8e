"""Pins for the oracle's immediate (chunk-boundary) eviction (TideKV, Fig. 1
caption, schedule (c); Table 8, Block-SnapKV): special cases that reduce it to
the one-shot compressor or to keeping everything, a two-chunk case checked
against a hand-built second boundary, and invariants of every result."""
import numpy as np
import pytest

import oracle
from synth import f32_to_bf16_bits


def bits(rng, shape):
    return f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32))


def windows_of(q_all, s, chunk, w):
    """Window b: the queries at the last w positions of chunk b."""
    return np.stack([q_all[c1 - w:c1] for _, c1 in oracle.chunk_bounds(s, chunk)])


def test_chunk_bounds():
    assert oracle.chunk_bounds(10, 4) == [(0, 4), (4, 8), (8, 10)]
    assert oracle.chunk_bounds(8, 8) == [(0, 8)]


def test_one_chunk_is_the_one_shot_compressor():
    rng = np.random.default_rng(1)
    s, w, hq, hkv, d = 60, 6, 4, 2, 8
    q_all, k, v = bits(rng, (s, hq, d)), bits(rng, (s, hkv, d)), bits(rng, (s, hkv, d))
    got = oracle.compress_chunked(windows_of(q_all, s, s, w), k, v, s, 20, 2, 4, pos_offset=7)
    want = oracle.compress_layer(q_all[s - w:], k, v, [20, 20], 2, 4, pos_offset=7)
    for g in range(hkv):
        np.testing.assert_array_equal(got.idx[g], want.idx[g])
    np.testing.assert_array_equal(got.k_hat, want.k_hat)
    np.testing.assert_array_equal(got.pos, want.pos)


def test_budget_covering_the_prompt_keeps_everything():
    rng = np.random.default_rng(2)
    s, w, hq, hkv, d, chunk = 52, 4, 2, 1, 8, 12   # a ragged last chunk of 4 = W
    q_all, k, v = bits(rng, (s, hq, d)), bits(rng, (s, hkv, d)), bits(rng, (s, hkv, d))
    got = oracle.compress_chunked(windows_of(q_all, s, chunk, w), k, v, chunk, s, 1, 2)
    np.testing.assert_array_equal(got.idx[0], np.arange(s))
    np.testing.assert_array_equal(got.k_hat, k[:, 0, :])


def test_two_chunks_equal_a_hand_built_second_boundary():
    """Boundary 1 keeps the top of chunk 0; boundary 2 scores those keys
    followed by chunk 1 -- built here directly from the one-shot compressor
    on hand-assembled arrays."""
    rng = np.random.default_rng(3)
    s, w, hq, hkv, d, chunk, budget = 40, 4, 4, 2, 8, 20, 9
    q_all, k, v = bits(rng, (s, hq, d)), bits(rng, (s, hkv, d)), bits(rng, (s, hkv, d))
    got = oracle.compress_chunked(windows_of(q_all, s, chunk, w), k, v, chunk, budget, 1, 3)
    first = oracle.compress_layer(q_all[chunk - w:chunk], k[:chunk], v[:chunk], [budget] * hkv, 1, 3)
    for g in range(hkv):
        acc = np.concatenate([first.idx[g], np.arange(chunk, s)])
        kg = k[acc, g:g + 1, :]
        vg = v[acc, g:g + 1, :]
        grp = hq // hkv
        second = oracle.compress_layer(q_all[s - w:, g * grp:(g + 1) * grp], kg, vg, [budget], 1, 3)
        np.testing.assert_array_equal(got.idx[g], acc[second.idx[0]])


@pytest.mark.parametrize("s,chunk,budget", [(104, 16, 10), (100, 25, 12), (100, 64, 40)])
def test_invariants(s, chunk, budget):
    rng = np.random.default_rng(chunk)
    w, hq, hkv, d = 8, 4, 2, 8
    q_all, k, v = bits(rng, (s, hq, d)), bits(rng, (s, hkv, d)), bits(rng, (s, hkv, d))
    got = oracle.compress_chunked(windows_of(q_all, s, chunk, w), k, v, chunk, budget, 2, 8, pos_offset=3)
    for g in range(hkv):
        ix = got.idx[g]
        assert ix.size == budget and np.all(np.diff(ix) > 0)
        assert {0, 1} <= set(ix.tolist())                 # the sinks survive every boundary
        assert set(range(s - 8, s)) <= set(ix.tolist())   # the last chunk's recent keys
    off = np.concatenate([[0], np.cumsum([budget] * hkv)])
    for g in range(hkv):
        np.testing.assert_array_equal(got.k_hat[off[g]:off[g + 1]], k[got.idx[g], g, :])
        np.testing.assert_array_equal(got.pos[off[g]:off[g + 1]], got.idx[g] + 3)


def test_short_chunks_are_rejected():
    rng = np.random.default_rng(4)
    s, w, hq, hkv, d = 21, 4, 2, 1, 8
    q_all, k, v = bits(rng, (s, hq, d)), bits(rng, (s, hkv, d)), bits(rng, (s, hkv, d))
    with pytest.raises(ValueError):   # last chunk of 1 token < W
        oracle.compress_chunked(windows_of(q_all, s - 1, 10, w)[:2].repeat(2, axis=0)[:3], k, v, 10, 8, 1, 2)
    with pytest.raises(ValueError):   # window count differs from the chunk count
        oracle.compress_chunked(windows_of(q_all, 20, 10, w), k, v, 10, 8, 1, 2)
