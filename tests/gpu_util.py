"""Helpers of the GPU tests: moving synthetic bf16 bit patterns to and from
the device and running the library's entry points (staged or fused)."""
from __future__ import annotations

import numpy as np
import torch

import compression_kvc_score_amd as kvc


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def from_dev_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def desc_from(cfg, q, k, v=None, **kw):
    opts = dict(block=cfg.block, n_sink=cfg.n_sink, n_recent=cfg.n_recent, pool=cfg.pool)
    opts.update(kw)
    return kvc.desc_for(q, k, v, **opts)


def run_staged(desc, q, k, v, budgets):
    """pass 1 -> pass 2 -> select -> gather as four calls; returns host arrays."""
    ws = kvc.alloc_workspace(desc)
    out = kvc.alloc_outputs(desc, budgets)
    kvc.kvc_score_pass1(desc, q, k, out.m, out.z, ws)
    kvc.kvc_score_pass2(desc, q, k, out.m, out.z, out.scores)
    kvc.kvc_select_topk(desc, out.scores, budgets, out.idx, ws)
    kvc.kvc_gather_retained(desc, k, v, out.idx, budgets, out.k_hat, out.v_hat, out.pos)
    torch.cuda.synchronize()
    return host(out)


def run_fused(desc, q, k, v, budgets, intermediates=True):
    ws = kvc.alloc_workspace(desc)
    out = kvc.alloc_outputs(desc, budgets, with_intermediates=intermediates)
    kvc.compress_layer(desc, q, k, v, budgets, out, ws)
    torch.cuda.synchronize()
    return host(out)


def host(out):
    h = {
        "idx": out.idx.cpu().numpy(),
        "k_hat": from_dev_bits(out.k_hat),
        "v_hat": from_dev_bits(out.v_hat),
        "pos": out.pos.cpu().numpy(),
        "offsets": out.offsets,
    }
    if out.m is not None:
        h["m"] = out.m.cpu().numpy()
        h["z"] = out.z.cpu().numpy()
        h["scores"] = out.scores.cpu().numpy()
    return h


def split_heads(flat: np.ndarray, offsets: np.ndarray):
    return [flat[offsets[g]:offsets[g + 1]] for g in range(len(offsets) - 1)]
