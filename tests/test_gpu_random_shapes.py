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


@pytest.mark.parametrize("i", range(len(CASES)))
def test_random_shape(i):
    c = dict(CASES[i])
    budgets = np.asarray(c.pop("budgets"), dtype=np.int64)
    seed = c.pop("seed")
    cfg = get_config("tiny").with_(name=f"random_{i}", sink_scale=4.0, seed_base=seed, budget=int(budgets[0]), **c)
    print(f"random shape {i}: s={cfg.s} w={cfg.w} hq={cfg.hq} hkv={cfg.hkv} d={cfg.d} block={cfg.block} "
          f"sink={cfg.n_sink} recent={cfg.n_recent} pool={cfg.pool} budgets={list(budgets)}", flush=True, file=sys.stderr)
    x = layer_inputs(cfg, 0)
    q, k, v = dev_inputs(x)
    desc = desc_from(cfg, q, k, v)
    got = run_fused(desc, q, k, v, budgets)
    check_layer(x, got, budgets)
