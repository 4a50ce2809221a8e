"""HIP-graph capture of the whole-layer call: kvc_compress_layer enqueues
only kernels (no memsets, no allocation, no host synchronisation), so a
captured sequence of calls replays to the same outputs as the eager calls.
Each replay is checked against the eager result, with eager work of the
program's own and synchronisations between the replays."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import compression_kvc_score_amd as kvc  # noqa: E402
from synth import get_config, layer_inputs  # noqa: E402

from gpu_util import desc_from, host, to_dev_bf16  # noqa: E402


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a HIP device")
    kvc.lib()


def say(*a):
    print(*a, flush=True, file=sys.stderr)


@pytest.mark.parametrize("mode", [kvc.KVC_SCORE_SOFTMAX, kvc.KVC_SCORE_LOGIT_INT8])
def test_captured_layers_replay_like_eager_calls(mode):
    cfg = get_config("llama8b_16k").with_(s=8192, n_heavy=80)
    layers = []
    for l in range(3):
        x = layer_inputs(cfg, l)
        layers.append((to_dev_bf16(x.q), to_dev_bf16(x.k), to_dev_bf16(x.v)))
    desc = desc_from(cfg, *layers[0], score_mode=mode)
    budgets = np.full(cfg.hkv, 1024)
    ws = kvc.alloc_workspace(desc)
    eager = [kvc.alloc_outputs(desc, budgets, with_intermediates=False) for _ in layers]
    graphed = [kvc.alloc_outputs(desc, budgets, with_intermediates=False) for _ in layers]
    for (q, k, v), o in zip(layers, eager):
        kvc.compress_layer(desc, q, k, v, budgets, o, ws)
    torch.cuda.synchronize()
    want = [host(o) for o in eager]
    preps = [kvc.PreparedLayer(desc, q, k, v, budgets, o, ws) for (q, k, v), o in zip(layers, graphed)]
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):       # warm on the capture stream's side, as torch asks
        for p in preps:
            p.kvc_compress_layer()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for p in preps:
            p.kvc_compress_layer()
    for rep in range(4):
        for o in graphed:               # poison the outputs eagerly before each replay
            o.idx.fill_(-1)
            o.k_hat.zero_()
            o.pos.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(graphed):
            got = host(o)
            for key in ("idx", "k_hat", "v_hat", "pos"):
                np.testing.assert_array_equal(got[key], want[i][key], err_msg=f"replay {rep} layer {i} {key}")
        # eager work between replays, on the same workspace
        kvc.compress_layer(desc, *layers[rep % 3], budgets, eager[rep % 3], ws)
        torch.cuda.synchronize()
        say(f"replay {rep} ok")
