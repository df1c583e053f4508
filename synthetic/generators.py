"""Seeded Gaussian inputs.

Every draw comes from NumPy's PCG64 seeded with SeedSequence([seed, layer,
chunk, stream]); stream 0 = latent-path weights, 1 = layer input x, 2 = query,
3 = dense-comparison weights, 4 = the attention block's query and output
projections and the latent's normalisation gain.  Values are drawn in float64 and rounded to the
storage dtype by torch's own dtype conversion (round to nearest even), so the
arrays handed to the GPU and to the oracle hold identical values.

Distributions: x ~ N(0, 1); q ~ N(0, 1) (the distribution a query projection
with N(0, 1/hidden) weights gives for unit-variance x); weights ~ N(0, 1/fan_in)
with fan_in = hidden for the down-projections and d_c for the up-projections.
"""

from __future__ import annotations

import numpy as np
import torch

_TORCH_DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def _rng(seed, layer, chunk, stream):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, chunk, stream])))


def to_storage_tensor(a, dtype):
    """float64 array -> CPU torch tensor in the storage dtype."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(_TORCH_DTYPES[dtype])


def layer_weights(cfg, layer=0, seed=None):
    """Latent-path weights of one layer as CPU tensors in cfg.dtype.

    w_dkr [d_c + d_rope, hidden] (rows < d_c: down-projection, rest: k^R
    projection), w_uk [n_h, d_nope, d_c], w_uv [n_h, d_v, d_c].
    """
    seed = cfg.seed if seed is None else seed
    g = _rng(seed, layer, 0, 0)
    w_dkr = g.standard_normal((cfg.d_c + cfg.d_rope, cfg.hidden)) / np.sqrt(cfg.hidden)
    w_uk = g.standard_normal((cfg.n_heads, cfg.d_nope, cfg.d_c)) / np.sqrt(cfg.d_c)
    w_uv = g.standard_normal((cfg.n_heads, cfg.d_v, cfg.d_c)) / np.sqrt(cfg.d_c)
    return {k: to_storage_tensor(v, cfg.dtype)
            for k, v in (("w_dkr", w_dkr), ("w_uk", w_uk), ("w_uv", w_uv))}


def block_weights(cfg, layer=0, seed=None):
    """Weights around the latent path: w_q [n_h * (d_nope + d_rope), hidden]
    (query projection, N(0, 1/hidden)), w_o [hidden, n_h * d_v] (output
    projection, N(0, 1/(n_h d_v))), kv_gamma [d_c] (RMS-norm gain of the
    latent, 1 + N(0, 1/16))."""
    seed = cfg.seed if seed is None else seed
    g = _rng(seed, layer, 0, 4)
    w_q = g.standard_normal((cfg.n_heads * cfg.d_qk, cfg.hidden)) / np.sqrt(cfg.hidden)
    w_o = g.standard_normal((cfg.hidden, cfg.n_heads * cfg.d_v)) / np.sqrt(cfg.n_heads * cfg.d_v)
    gamma = 1.0 + 0.25 * g.standard_normal(cfg.d_c)
    return {k: to_storage_tensor(v, cfg.dtype) for k, v in (("w_q", w_q), ("w_o", w_o), ("kv_gamma", gamma))}


def dense_weights(cfg, layer=0, seed=None):
    """Dense-comparison projections w_k, w_v [n_h * d_h, hidden]."""
    seed = cfg.seed if seed is None else seed
    g = _rng(seed, layer, 0, 3)
    n = cfg.n_heads * cfg.d_qk
    w_k = g.standard_normal((n, cfg.hidden)) / np.sqrt(cfg.hidden)
    w_v = g.standard_normal((n, cfg.hidden)) / np.sqrt(cfg.hidden)
    return {"w_k": to_storage_tensor(w_k, cfg.dtype), "w_v": to_storage_tensor(w_v, cfg.dtype)}


def chunk_x(cfg, n_frames, batch=None, layer=0, chunk=0, seed=None):
    """Layer input for n_frames whole latent frames: [B, n_frames*T, hidden]."""
    seed = cfg.seed if seed is None else seed
    B = cfg.batch if batch is None else batch
    g = _rng(seed, layer, chunk, 1)
    return to_storage_tensor(g.standard_normal((B, n_frames * cfg.T, cfg.hidden)), cfg.dtype)


def chunk_q(cfg, Lq, batch=None, layer=0, chunk=0, seed=None):
    """Per-head queries [B, Lq, n_h, d_nope + d_rope], q^R part un-rotated."""
    seed = cfg.seed if seed is None else seed
    B = cfg.batch if batch is None else batch
    g = _rng(seed, layer, chunk, 2)
    return to_storage_tensor(g.standard_normal((B, Lq, cfg.n_heads, cfg.d_qk)), cfg.dtype)
