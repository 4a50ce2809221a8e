"""Seeded fuzz of the library's pure host entry points (no GPU needed):
random descriptors, budgets and stabilities, including out-of-range and
extreme values, always give either a result or an error status -- never a
crash -- and every accepted result is consistent with its definition (a
workspace that is at least the score vector, packed offsets that are the
running sum of min(budget, S), inverse-stability budgets that sum to the
total and follow 1 / s_stable)."""
import ctypes

import numpy as np
import pytest

import compression_kvc_score_amd as kvc
import oracle

FIELDS_EXTREME = [0, 1, -1, 7, 31, 32, 33, 64, 128, 255, 256, 511, 512, 513, 1 << 20, (1 << 23) + 1, 2**31 - 1, -2**31]


def random_desc(rng):
    def pick(typical):
        return int(rng.choice(FIELDS_EXTREME)) if rng.random() < 0.2 else int(typical)
    hkv = pick(rng.choice([1, 2, 4, 8, 64, 65]))
    hq = pick(hkv * int(rng.choice([1, 2, 4, 5, 8])) if hkv > 0 else 1)
    return kvc.make_desc(
        s=pick(rng.integers(1, 200000)), w=pick(rng.choice([1, 8, 32, 64, 300])), hq=hq, hkv=hkv,
        d=pick(rng.choice([64, 128, 96])), block=pick(rng.choice([32, 96, 256, 512, 520])),
        scale=float(rng.choice([0.0, 0.1, -1.0, np.inf, np.nan])) if rng.random() < 0.3 else 0.0,
        n_sink=pick(rng.integers(0, 10)), n_recent=pick(rng.integers(0, 70)),
        pool=pick(rng.choice([1, 3, 7, 31, 33, 2])), pos_offset=pick(rng.integers(0, 1 << 20)),
        score_mode=pick(rng.choice([0, 1, 2, 3])))


def test_workspace_size_never_crashes_and_covers_the_scores():
    rng = np.random.default_rng(7)
    lib = kvc.lib()
    accepted = 0
    for _ in range(3000):
        d = random_desc(rng)
        n = lib.kvc_workspace_size(ctypes.byref(d))
        if n:
            accepted += 1
            assert n >= 4 * d.hkv * d.s  # at least the fp32 score vector
            assert n % 256 == 0
    assert accepted > 100


def test_retained_offsets_fuzz():
    rng = np.random.default_rng(8)
    lib = kvc.lib()
    for _ in range(2000):
        d = random_desc(rng)
        hkv = max(int(d.hkv), 0)
        nb = min(max(hkv, 1), kvc.KVC_MAX_KV_HEADS + 1)  # an invalid head count is refused before any read
        b = rng.integers(-5, min(max(int(d.s), 1), 1 << 24) + 100, size=nb).astype(np.int32)
        if rng.random() < 0.1:
            b[0] = np.int32(-2**31)
        off = np.zeros(nb + 1, dtype=np.int64)
        st = lib.kvc_retained_offsets(ctypes.byref(d), b.ctypes.data_as(ctypes.c_void_p),
                                      off.ctypes.data_as(ctypes.c_void_p))
        if st == 0:
            assert 1 <= hkv <= kvc.KVC_MAX_KV_HEADS
            s = int(d.s)
            n_mand = len(oracle.mandatory(s, int(d.n_sink), int(d.n_recent)))
            assert np.all(b[:hkv] >= 0) and np.all((b[:hkv] >= s) | (b[:hkv] >= n_mand))
            want = np.concatenate([[0], np.cumsum(np.minimum(b[:hkv].astype(np.int64), s))])
            np.testing.assert_array_equal(off[:hkv + 1], want)
        else:
            assert st < 0


def test_inverse_stability_budgets_fuzz():
    rng = np.random.default_rng(9)
    lib = kvc.lib()
    for _ in range(2000):
        hkv = int(rng.choice([0, 1, 2, 8, 64, 65, -1]))
        n = max(hkv, 1)
        st_vals = rng.uniform(0.05, 1.0, size=n)
        if rng.random() < 0.2:
            st_vals[int(rng.integers(0, n))] = float(rng.choice([0.0, -1.0, np.inf, np.nan, 1e-300, 1e-308, 1e300]))
        if rng.random() < 0.05:
            st_vals[:] = 1e-308  # weights whose sum overflows
        total = int(rng.choice([0, 1, 4096, 8 * 4096, 2**31 - 1, 2**31, -1]))
        out = np.zeros(n, dtype=np.int32)
        st = lib.kvc_budgets_inverse_stability(st_vals.ctypes.data_as(ctypes.c_void_p), hkv, total,
                                               out.ctypes.data_as(ctypes.c_void_p))
        if st == 0:
            assert hkv >= 1 and 0 <= total <= 2**31 - 1
            assert int(out[:hkv].astype(np.int64).sum()) == total
            want = oracle.inverse_stability_budgets(st_vals[:hkv], total)
            np.testing.assert_array_equal(out[:hkv], want)
        else:
            assert st < 0


def test_device_entry_points_refuse_fuzzed_arguments_before_any_launch():
    """kvc_compress_layer, the staged calls and the chunk-boundary call with
    fuzzed descriptors and pointer sets: each call lacks its workspace or an
    output (or has a misaligned one), so the host must refuse it with an
    error status before touching the device; no combination may crash."""
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("host-only fuzz: never run where kernels could launch")
    rng = np.random.default_rng(10)
    lib = kvc.lib()
    P = ctypes.c_void_p
    fake = [None, P(0x10000), P(0x10001), P(0x10004)]
    budgets = np.full(kvc.KVC_MAX_KV_HEADS + 1, 64, dtype=np.int32)
    bp = budgets.ctypes.data_as(P)
    for _ in range(3000):
        d = random_desc(rng)
        dd = ctypes.byref(d)
        ptrs = [fake[int(rng.integers(0, 4))] for _ in range(8)]
        bad = int(rng.integers(0, 3))
        if bad == 0:
            ws, wsb = None, int(rng.integers(0, 1 << 30))           # no workspace
        elif bad == 1:
            ws, wsb = P(0x10000), int(rng.integers(0, 1 << 30))
            ptrs[3] = None                                            # no idx_out
        else:
            ws, wsb = P(0x10010), int(rng.integers(0, 1 << 30))     # misaligned workspace
        st = lib.kvc_compress_layer(dd, ptrs[0], ptrs[1], ptrs[2], bp, None, None, None, ptrs[3], ptrs[4],
                                    ptrs[5], ptrs[6], ws, wsb, None)
        assert st < 0
        st = lib.kvc_score_pass1(dd, ptrs[0], ptrs[1], ptrs[2], ptrs[3], ws if bad != 1 else None, wsb, None)
        assert st < 0
        st = lib.kvc_select_topk(dd, ptrs[0], bp, ptrs[1], ws if bad != 1 else None, wsb, None)
        assert st < 0
        # no current arena: refused whether or not the boundary would evict
        st = lib.kvc_evict_chunk(dd, ptrs[0], ptrs[1], ptrs[2], int(rng.integers(-1, 5000)),
                                 int(rng.integers(-1, 5000)), int(rng.integers(-1, 20000)), None, ptrs[4],
                                 ptrs[5], ptrs[6], ptrs[7], ptrs[0], None, wsb, None)
        assert st < 0
