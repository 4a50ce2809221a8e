"""Host-side checks of bench.py: the single-GPU contract and the algorithmic
byte model that the roofline divides by (the per-layer byte counts of the
layer-end compressor: two K scans, the score vector written and read, the
retained rows read and written with their indices and positions)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import get_config  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name,budget,total", [
    # S x Hkv x D x 2 bytes of K per scan; W x Hq x D x 2 of window queries and
    # 2 x Hq x W x 4 of (m, Z) per scan; 4 bytes of score per key and head,
    # written by pass 2 and read by the selection; 4 bytes of index per kept
    # row; the kept K and V rows read and written (4 x D x 2) with a position
    ("llama8b_16k", 4096, 102_645_760),
    ("llama8b_64k", 4096, 307_118_080),
    ("llama8b_128k", 4096, 580_288_512),
    ("llama8b_128k_pool7", 4096, 580_288_512 + 2 * 8 * 131072 * 4),  # pooled values written and read
])
def test_algorithmic_bytes_per_layer(name, budget, total):
    cfg = get_config(name)
    b = bench.algorithmic_bytes(cfg, cfg.hkv * budget)
    assert sum(b.values()) == total
    k = cfg.s * cfg.hkv * cfg.d * 2
    assert b["pass1"] > k and b["pass2"] > k  # both scans read all of K
    assert b["gather"] == cfg.hkv * budget * (4 * cfg.d * 2 + 8)


def test_kernel_hash_covers_the_scan_and_selection_sources():
    h = bench.kernel_source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    for name in bench.KERNEL_SOURCES:
        assert os.path.exists(os.path.join(ROOT, "compression_kvc_score_amd", "csrc", name))
