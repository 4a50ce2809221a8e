"""Workload presets: the layer shapes the compressor is exercised on.

Shapes follow the geometry the TideKV page evaluates (Llama-3.1-8B in bf16,
physical KV budget 4096, prompts of 16K/64K/128K; TideKV Table 2) and the
Qwen2.5-14B layer the HeteroCache summary names, with the HeteroCache-style
per-KV-head budgets (HeteroCache summary, Methodology, Phase 2).
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class LayerConfig:
    name: str
    hq: int                 # query heads
    hkv: int                # KV heads (GQA group = hq // hkv)
    d: int                  # head dimension
    s: int                  # prompt length (prefix keys scored)
    w: int                  # observation window: the last w prompt queries
    block: int              # key block size b_s of the blockwise scan
    budget: int             # K_l per KV head (uniform budgets)
    n_sink: int             # mandatory leading keys
    n_recent: int           # mandatory trailing keys
    n_heavy: int            # planted high-attention key positions
    sink_scale: float       # norm multiplier of the sink keys (1 = none)
    layers: int             # layers in the layer-major sweep
    pool: int = 1           # 1-D max-pool width over scores before selection (1 = off)
    hetero: bool = False    # per-head budgets from inverse stability
    total_budget: int = 0   # sum of per-head budgets when hetero
    seed_base: int = 0
    chunk: int = 0          # prefill chunk of immediate (chunk-boundary) eviction (0: none)

    @property
    def group(self) -> int:
        return self.hq // self.hkv

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


def _heavy(frac: float, s: int) -> int:
    return int(round(frac * s))


CONFIGS: dict[str, LayerConfig] = {
    # Tiny single layer: one KV head, GQA 4, no sink scaling.
    "tiny": LayerConfig(
        name="tiny", hq=4, hkv=1, d=64, s=1024, w=16, block=128, budget=128,
        n_sink=4, n_recent=16, n_heavy=10, sink_scale=1.0, layers=1,
        seed_base=20261300),
    # Llama-3.1-8B layer geometry at a 16K prompt.
    "llama8b_16k": LayerConfig(
        name="llama8b_16k", hq=32, hkv=8, d=128, s=16384, w=32, block=256,
        budget=4096, n_sink=4, n_recent=32, n_heavy=_heavy(0.01, 16384),
        sink_scale=4.0, layers=1, seed_base=20261400),
    # The same layer at a 64K prompt, swept over the model's 32 layers.
    "llama8b_64k": LayerConfig(
        name="llama8b_64k", hq=32, hkv=8, d=128, s=65536, w=32, block=256,
        budget=4096, n_sink=4, n_recent=32, n_heavy=_heavy(0.01, 65536),
        sink_scale=4.0, layers=32, seed_base=20261500),
    # 128K prompt, 64-query window, 0.5% heavy keys.
    "llama8b_128k": LayerConfig(
        name="llama8b_128k", hq=32, hkv=8, d=128, s=131072, w=64, block=256,
        budget=4096, n_sink=4, n_recent=64, n_heavy=_heavy(0.005, 131072),
        sink_scale=4.0, layers=1, seed_base=20261600),
    # Same, with a width-7 max-pool over scores before selection.
    "llama8b_128k_pool7": LayerConfig(
        name="llama8b_128k_pool7", hq=32, hkv=8, d=128, s=131072, w=64,
        block=256, budget=4096, n_sink=4, n_recent=64,
        n_heavy=_heavy(0.005, 131072), sink_scale=4.0, layers=1, pool=7,
        seed_base=20261600),
    # Qwen2.5-14B layer geometry (GQA 5) with inverse-stability budgets
    # summing to 8 x 4096, swept over 48 layers.
    "qwen14b_hetero_64k": LayerConfig(
        name="qwen14b_hetero_64k", hq=40, hkv=8, d=128, s=65536, w=32,
        block=256, budget=4096, n_sink=4, n_recent=32,
        n_heavy=_heavy(0.01, 65536), sink_scale=4.0, layers=48, hetero=True,
        total_budget=8 * 4096, seed_base=20261700),
    # Immediate eviction after every 512-token chunk of a 16K prompt with a
    # 1024-key budget (the Block-SnapKV setting of TideKV Table 8); same
    # tensors as llama8b_16k.
    "llama8b_16k_imm": LayerConfig(
        name="llama8b_16k_imm", hq=32, hkv=8, d=128, s=16384, w=32, block=256,
        budget=1024, n_sink=4, n_recent=32, n_heavy=_heavy(0.01, 16384),
        sink_scale=4.0, layers=1, seed_base=20261400, chunk=512),
    # The 64K layer evicted after every 2048-token chunk with the 4096-key
    # budget (TideKV Table 2's chunk and budget); same tensors as llama8b_64k.
    "llama8b_64k_imm": LayerConfig(
        name="llama8b_64k_imm", hq=32, hkv=8, d=128, s=65536, w=32, block=256,
        budget=4096, n_sink=4, n_recent=32, n_heavy=_heavy(0.01, 65536),
        sink_scale=4.0, layers=1, seed_base=20261500, chunk=2048),
}


def get_config(name: str) -> LayerConfig:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}")
