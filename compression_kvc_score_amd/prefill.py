"""Synthetic layer-major chunked prefill around the layer-end compressor.

TideKV's construction schedule (Fig. 2 caption; Fig. 1 caption, schedule (d))
with the components of its reference architecture (Fig. 4 caption):

- ``LayerMajorPrefill`` -- the layer-major scheduler. For layer l it runs
  every prompt chunk j in order: RMSNorm, QKV projection, rotary embedding
  with the append of the chunk's K/V to the layer's full K/V, attention of
  the chunk over the accumulated K/V of chunks 0..j, output projection with
  the residual, RMSNorm, SwiGLU MLP with the residual; the chunk's output rows
  replace its input rows in the hidden-state bridge, which feeds layer l + 1.
  After the last chunk it commits the layer: the compressor (the C ABI's
  ``kvc_compress_layer``) turns the full K/V into the retained cache, with
  the prompt's last W queries as the window. The full K/V buffer is then free
  for layer l + 2: two buffers alternate, so the commit of layer l runs on a
  second stream while layer l + 1 computes.
- ``RetainedCacheManager`` -- the cross-layer cache manager: one arena that
  holds every layer's retained K, V and positions.
- ``MemoryAccountant`` -- records what each component keeps resident and the
  device allocator's peaks.
- ``SyntheticModel`` -- a Llama-family decoder stack with random weights (the
  pages' Llama-3.1-8B geometry by default); there are no trained weights, so
  nothing here measures quality.

The non-GEMM layer pieces and the compressor are this library's HIP kernels;
the projections are plain GEMMs, run by the vendor BLAS through torch.
``keep_full_kv=True`` gives the comparison schedule of Fig. 1 (b) followed by
post-prefill compression: every layer's full K/V stays resident until the
whole prompt is done, then all layers are compressed.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import _lib as L


@dataclass
class ModelConfig:
    hidden: int = 4096
    hq: int = 32
    hkv: int = 8
    d: int = 128
    ffn: int = 14336
    layers: int = 32
    eps: float = 1e-5
    rope_base: float = 500000.0


class SyntheticModel:
    """Random bf16 weights per layer, either drawn on the device from a seed
    or given as host bf16 bit patterns (w_attn, w_qkv, w_o, w_mlp, w_gu,
    w_down per layer, in the layouts of the prefill oracle)."""

    NAMES = ("w_attn", "w_qkv", "w_o", "w_mlp", "w_gu", "w_down")

    def __init__(self, cfg: ModelConfig, device="cuda", seed: int = 0, host_weights=None):
        import torch
        self.cfg = cfg
        self.layers = []
        if host_weights is not None:
            for lw in host_weights:
                self.layers.append({n: torch.from_numpy(np.ascontiguousarray(getattr(lw, n)).view(np.int16))
                                    .view(torch.bfloat16).to(device) for n in self.NAMES})
            return
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)
        c = cfg
        qkv_rows = (c.hq + 2 * c.hkv) * c.d

        def rnd(shape, scale):
            return (torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * scale).to(torch.bfloat16)

        for _ in range(c.layers):
            self.layers.append({
                "w_attn": (1.0 + rnd((c.hidden,), 0.1).float()).to(torch.bfloat16),
                "w_qkv": rnd((qkv_rows, c.hidden), c.hidden ** -0.5),
                "w_o": rnd((c.hidden, c.hq * c.d), (c.hq * c.d) ** -0.5),
                "w_mlp": (1.0 + rnd((c.hidden,), 0.1).float()).to(torch.bfloat16),
                "w_gu": rnd((2 * c.ffn, c.hidden), c.hidden ** -0.5),
                "w_down": rnd((c.hidden, c.ffn), c.ffn ** -0.5),
            })

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for lw in self.layers for t in lw.values())


class MemoryAccountant:
    """Bytes each component keeps resident (added and released by name) and
    the peak of their sum, next to the device allocator's own peak."""

    def __init__(self):
        import torch
        self.resident: dict[str, int] = {}
        self.peak = 0
        self.peak_parts: dict[str, int] = {}
        self.alloc_base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()

    def hold(self, name: str, nbytes: int):
        self.resident[name] = self.resident.get(name, 0) + int(nbytes)
        total = sum(self.resident.values())
        if total > self.peak:
            self.peak, self.peak_parts = total, dict(self.resident)

    def release(self, name: str, nbytes: int | None = None):
        if nbytes is None or nbytes >= self.resident.get(name, 0):
            self.resident.pop(name, None)
        else:
            self.resident[name] -= int(nbytes)

    def report(self) -> dict:
        import torch
        return {"peak_bytes": self.peak, "peak_parts": self.peak_parts,
                "allocator_peak_bytes": torch.cuda.max_memory_allocated() - self.alloc_base}


def nbytes(*ts) -> int:
    return sum(t.numel() * t.element_size() for t in ts)


class RetainedCacheManager:
    """The retained caches of all layers in one arena: K, V bf16
    [layers][sum K_h][D] and positions int32 [layers][sum K_h]."""

    def __init__(self, cfg: ModelConfig, s: int, budgets, device="cuda"):
        import torch
        self.budgets = np.asarray(budgets, dtype=np.int64)
        self.rows = int(np.minimum(self.budgets, s).sum())
        self.k = torch.empty((cfg.layers, self.rows, cfg.d), dtype=torch.bfloat16, device=device)
        self.v = torch.empty_like(self.k)
        self.pos = torch.empty((cfg.layers, self.rows), dtype=torch.int32, device=device)
        self.idx = torch.empty((cfg.layers, self.rows), dtype=torch.int32, device=device)
        self.committed = [False] * cfg.layers

    def nbytes(self) -> int:
        return nbytes(self.k, self.v, self.pos)


class LayerMajorPrefill:
    """Layer-major chunked prefill with layer-end eviction (see the module
    docstring). ``run(x)`` takes the prompt's hidden states [S, hidden] bf16
    (the bridge, updated in place) and returns the RetainedCacheManager."""

    def __init__(self, model: SyntheticModel, s: int, chunk: int, w: int, budgets, n_sink: int, n_recent: int,
                 block: int = 256, overlap: bool = True, keep_full_kv: bool = False, device="cuda",
                 accountant: MemoryAccountant | None = None, compress: bool = True):
        import torch
        c = model.cfg
        if chunk < 1 or w < 1 or w > s:
            raise ValueError("need chunk >= 1 and 1 <= w <= s")
        self.model, self.cfg, self.s, self.chunk, self.w = model, c, s, chunk, w
        self.n_sink, self.n_recent, self.block = n_sink, n_recent, block
        self.overlap, self.keep_full_kv, self.compress = overlap, keep_full_kv, compress
        self.acct = accountant or MemoryAccountant()
        self.acct.hold("weights", model.nbytes())
        self.pdesc = L.PrefillDesc(s=s, hq=c.hq, hkv=c.hkv, d=c.d, rope_base=c.rope_base, scale=0.0)
        bf = dict(dtype=torch.bfloat16, device=device)
        # chunk temporaries: sized by the chunk, not the prompt
        self.t_xn = torch.empty((chunk, c.hidden), **bf)
        self.t_qkv = torch.empty((chunk, (c.hq + 2 * c.hkv) * c.d), **bf)
        self.t_q = torch.empty((chunk, c.hq, c.d), **bf)
        self.t_o = torch.empty((chunk, c.hq, c.d), **bf)
        self.t_h = torch.empty((chunk, c.hidden), **bf)
        self.t_gu = torch.empty((chunk, 2 * c.ffn), **bf)
        self.t_a = torch.empty((chunk, c.ffn), **bf)
        self.acct.hold("chunk_temporaries", nbytes(self.t_xn, self.t_qkv, self.t_q, self.t_o, self.t_h,
                                                   self.t_gu, self.t_a))
        # full K/V of the active layer(s) and the window queries
        n_kv = c.layers if keep_full_kv else (2 if overlap else 1)
        self.kv = [(torch.empty((s, c.hkv, c.d), **bf), torch.empty((s, c.hkv, c.d), **bf)) for _ in range(n_kv)]
        self.q_win = [torch.empty((w, c.hq, c.d), **bf) for _ in range(n_kv)]
        self.kv_bytes_each = nbytes(*self.kv[0])
        self.acct.hold("full_kv", n_kv * self.kv_bytes_each)
        self.acct.hold("window_queries", nbytes(*self.q_win))
        # compressor: one workspace per buffer that can be in flight
        self.desc = L.make_desc(s, w, c.hq, c.hkv, c.d, block=block, n_sink=n_sink, n_recent=n_recent)
        n_ws = 2 if overlap and not keep_full_kv else 1
        self.ws = [L.alloc_workspace(self.desc, device) for _ in range(n_ws)]
        self.acct.hold("compressor_workspace", nbytes(*self.ws))
        self.cache = RetainedCacheManager(c, s, budgets, device)
        self.acct.hold("retained_cache", self.cache.nbytes())
        self.budgets = np.asarray(budgets, dtype=np.int32)
        self.commit_stream = torch.cuda.Stream() if overlap else None
        self.kv_free = [None] * n_kv  # event after which buffer i may be overwritten

    # -- one chunk of one layer
    def _chunk(self, lw, x, c0, k, v, q_win):
        import torch
        n = x.shape[0]
        c = self.cfg
        xn, qkv, q, o = self.t_xn[:n], self.t_qkv[:n], self.t_q[:n], self.t_o[:n]
        h, gu, a = self.t_h[:n], self.t_gu[:n], self.t_a[:n]
        L.kvc_rmsnorm(x, lw["w_attn"], xn, c.eps)
        torch.matmul(xn, lw["w_qkv"].t(), out=qkv)
        L.kvc_rope_append(self.pdesc, qkv, c0, q, k, v)
        L.kvc_chunk_attention(self.pdesc, q, k, v, c0, o)
        torch.addmm(x, o.view(n, c.hq * c.d), lw["w_o"].t(), out=h)
        L.kvc_rmsnorm(h, lw["w_mlp"], xn, c.eps)
        torch.matmul(xn, lw["w_gu"].t(), out=gu)
        L.kvc_swiglu(gu, a)
        torch.addmm(h, a, lw["w_down"].t(), out=x)   # the chunk's rows of the bridge, in place
        w0 = self.s - self.w             # first position of the observation window
        lo = max(c0, w0)
        if lo < c0 + n:
            q_win[lo - w0:c0 + n - w0].copy_(q[lo - c0:])

    def _commit(self, l, k, v, q_win, ws):
        cm = self.cache
        L.kvc_compress_layer(self.desc, q_win, k, v, self.budgets, cm.idx[l], cm.k[l], cm.v[l], cm.pos[l], ws)
        cm.committed[l] = True

    def run_layer(self, l: int, x):
        """Layer l over all chunks, then its commit (on the commit stream when
        overlapping). Returns (start, end) events of the layer's chunks."""
        import torch
        main = torch.cuda.current_stream()
        i = l if self.keep_full_kv else l % len(self.kv)
        if self.kv_free[i] is not None:
            main.wait_event(self.kv_free[i])   # the commit that last read buffer i is done
        k, v = self.kv[i]
        q_win = self.q_win[i]
        e0 = torch.cuda.Event(enable_timing=True)
        e0.record(main)
        for c0 in range(0, self.s, self.chunk):
            c1 = min(c0 + self.chunk, self.s)
            self._chunk(self.model.layers[l], x[c0:c1], c0, k, v, q_win)
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record(main)
        if self.keep_full_kv or not self.compress:
            return e0, e1, None
        ws = self.ws[i % len(self.ws)]
        if self.commit_stream is not None:
            self.commit_stream.wait_event(e1)
            with torch.cuda.stream(self.commit_stream):
                self._commit(l, k, v, q_win, ws)
                done = torch.cuda.Event(enable_timing=True)
                done.record(self.commit_stream)
        else:
            self._commit(l, k, v, q_win, ws)
            done = torch.cuda.Event(enable_timing=True)
            done.record(main)
        self.kv_free[i] = done
        return e0, e1, done

    def run(self, x):
        """All layers; returns the cache manager once every commit has been
        ordered before later work on the current stream."""
        import torch
        main = torch.cuda.current_stream()
        self.acct.hold("bridge", nbytes(x))
        self.kv_free = [None] * len(self.kv)
        self.layer_events = []
        for l in range(self.cfg.layers):
            self.layer_events.append(self.run_layer(l, x))
        if self.keep_full_kv and self.compress:
            # post-prefill compression of every layer (Fig. 1 (b) then compression)
            for l in range(self.cfg.layers):
                k, v = self.kv[l]
                self._commit(l, k, v, self.q_win[l], self.ws[0])
        else:
            for ev in self.kv_free:
                if ev is not None:
                    main.wait_event(ev)
        self.acct.release("bridge")
        return self.cache
