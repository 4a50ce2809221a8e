"""The seeded input generator: determinism, bf16 rounding and the planted
structure of each workload."""
import numpy as np
import pytest

from synth import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, get_config, layer_inputs


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 lies exactly between bf16 neighbours 1 and 1 + 2^-7: ties go to
    # the even pattern (1.0); 1 + 3*2^-8 ties to 1 + 2^-6 (even).
    x = np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, 1.0 + 2**-8 + 2**-20, -2.5, 0.0], dtype=np.float32)
    b = f32_to_bf16_bits(x)
    assert list(b) == [0x3F80, 0x3F82, 0x3F81, 0xC020, 0x0000]
    np.testing.assert_array_equal(bf16_bits_to_f32(b), np.array([1.0, 1.0 + 2**-6, 1.0 + 2**-7, -2.5, 0.0], np.float32))


def test_same_seed_same_bytes_and_threads_do_not_matter():
    cfg = get_config("tiny").with_(s=9000)  # more than two K/V chunks
    a = layer_inputs(cfg, 3, threads=1)
    b = layer_inputs(cfg, 3, threads=4)
    for x, y in [(a.q, b.q), (a.k, b.k), (a.v, b.v), (a.heavy_pos, b.heavy_pos)]:
        assert np.array_equal(x, y)
    c = layer_inputs(cfg, 4)
    assert not np.array_equal(a.k, c.k)


def test_tiny_structure():
    cfg = get_config("tiny")
    x = layer_inputs(cfg, 0)
    assert x.q.shape == (16, 4, 64) and x.k.shape == (1024, 1, 64) and x.v.shape == (1024, 1, 64)
    assert x.q.dtype == np.uint16
    assert len(x.heavy_pos) == 10
    assert np.all(x.heavy_pos >= cfg.n_sink) and np.all(x.heavy_pos < cfg.s - cfg.w)
    kf = bf16_bits_to_f32(x.k).astype(np.float64)
    norms = np.linalg.norm(kf[:, 0, :], axis=1)
    # planted keys carry ~3*sqrt(D) along the mean query direction plus unit noise
    assert norms[x.heavy_pos].mean() > 2.0 * norms.mean()
    assert x.s_stable is None


@pytest.mark.parametrize("name,count", [("llama8b_16k", 164), ("llama8b_64k", 655),
                                        ("llama8b_128k", 655), ("qwen14b_hetero_64k", 655)])
def test_heavy_counts(name, count):
    assert CONFIGS[name].n_heavy == count


def test_sinks_scaled_exactly():
    cfg = get_config("llama8b_16k").with_(s=2048)
    a = layer_inputs(cfg, 0)
    b = layer_inputs(cfg.with_(sink_scale=1.0), 0)
    np.testing.assert_array_equal(bf16_bits_to_f32(a.k[:4]), 4.0 * bf16_bits_to_f32(b.k[:4]))
    np.testing.assert_array_equal(a.k[4:], b.k[4:])


def test_hetero_stabilities():
    cfg = get_config("qwen14b_hetero_64k").with_(s=4096)
    x = layer_inputs(cfg, 5)
    assert x.s_stable.shape == (8,)
    assert np.all((x.s_stable >= 0.2) & (x.s_stable < 0.9))


def test_chunk_windows_end_with_the_layer_window():
    from synth import chunk_windows
    cfg = get_config("tiny")
    x = layer_inputs(cfg, 0)
    a = chunk_windows(cfg, 200, 0)
    b = chunk_windows(cfg, 200, 0, q_last=x.q)
    n = (cfg.s + 199) // 200
    assert a.shape == (n * cfg.w, cfg.hq, cfg.d) and a.dtype == np.uint16
    np.testing.assert_array_equal(a, b)                  # deterministic, and Q is the layer's
    np.testing.assert_array_equal(a[-cfg.w:], x.q)
    assert not np.array_equal(a[:cfg.w], a[cfg.w:2 * cfg.w])
    assert not np.array_equal(a[:cfg.w], chunk_windows(cfg, 200, 1)[:cfg.w])
