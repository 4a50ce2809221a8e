"""kvc_compress_layer_noalloc: the whole-layer call with the library's fixed
per-device scratch as its workspace. It must write exactly what
kvc_compress_layer writes with a caller-allocated workspace, on consecutive
calls that reuse the scratch (the second on a smaller layer), and refuse a
layer whose workspace exceeds the scratch before launching anything."""
import ctypes
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import compression_kvc_score_amd as kvc  # noqa: E402
from synth import get_config, layer_inputs  # noqa: E402


def say(*a):
    print(*a, flush=True, file=sys.stderr)


def test_noalloc_refuses_a_layer_larger_than_the_scratch():
    """Pure host path: the size check runs before any HIP call."""
    desc = kvc.make_desc(s=1 << 21, w=32, hq=32, hkv=8, d=128, block=256, n_sink=4, n_recent=32)
    assert kvc.kvc_workspace_size(desc) > kvc.KVC_NOALLOC_SCRATCH_BYTES
    lib = kvc.lib()
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced
    b = np.full(8, 4096, dtype=np.int32)
    st = lib.kvc_compress_layer_noalloc(ctypes.byref(desc), fake, fake, fake, b.ctypes.data_as(ctypes.c_void_p),
                                        None, None, None, fake, fake, fake, fake, None)
    assert st == kvc.KVC_ERR_WORKSPACE
    assert b"fixed scratch" in lib.kvc_last_error()


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _run_both(cfg, layer, pool=1):
    x = layer_inputs(cfg, layer)
    q, k, v = _dev(x.q), _dev(x.k), _dev(x.v)
    b = np.full(cfg.hkv, cfg.budget, dtype=np.int64)
    desc = kvc.desc_for(q, k, v, block=cfg.block, n_sink=cfg.n_sink, n_recent=cfg.n_recent, pool=pool)
    assert kvc.kvc_workspace_size(desc) <= kvc.KVC_NOALLOC_SCRATCH_BYTES
    want = kvc.alloc_outputs(desc, b)
    kvc.compress_layer(desc, q, k, v, b, want, kvc.alloc_workspace(desc))
    got = kvc.alloc_outputs(desc, b)
    for t in (got.m, got.z, got.scores):
        t.fill_(-3.0)
    got.idx.fill_(-7)
    got.k_hat.view(torch.int16).fill_(-7)
    kvc.kvc_compress_layer_noalloc(desc, q, k, v, b, got.idx, got.k_hat, got.v_hat, got.pos,
                                   m_out=got.m, z_out=got.z, scores_out=got.scores)
    torch.cuda.synchronize()
    for name in ("m", "z", "scores", "idx", "pos"):
        np.testing.assert_array_equal(getattr(got, name).cpu().numpy(), getattr(want, name).cpu().numpy(),
                                      err_msg=name)
    for name in ("k_hat", "v_hat"):
        assert torch.equal(getattr(got, name).view(torch.int16), getattr(want, name).view(torch.int16)), name
    return got


@pytest.mark.gpu
def test_noalloc_equals_compress_layer_on_consecutive_calls():
    if not torch.cuda.is_available():
        pytest.fail("GPU test needs a HIP device")
    say("noalloc: 64K Llama layer")
    _run_both(get_config("llama8b_64k"), 0)
    say("noalloc: the 1K tiny layer right after (the scratch holds the 64K layer's state)")
    _run_both(get_config("tiny"), 0)
    say("noalloc: 16K layer with the optional outputs in the scratch")
    cfg = get_config("llama8b_16k")
    x = layer_inputs(cfg, 1)
    q, k, v = _dev(x.q), _dev(x.k), _dev(x.v)
    b = np.full(cfg.hkv, cfg.budget, dtype=np.int64)
    desc = kvc.desc_for(q, k, v, block=cfg.block, n_sink=cfg.n_sink, n_recent=cfg.n_recent)
    want = kvc.alloc_outputs(desc, b, with_intermediates=False)
    kvc.compress_layer(desc, q, k, v, b, want, kvc.alloc_workspace(desc))
    got = kvc.alloc_outputs(desc, b, with_intermediates=False)
    kvc.kvc_compress_layer_noalloc(desc, q, k, v, b, got.idx, got.k_hat, got.v_hat, got.pos)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got.idx.cpu().numpy(), want.idx.cpu().numpy())
    assert torch.equal(got.v_hat.view(torch.int16), want.v_hat.view(torch.int16))
