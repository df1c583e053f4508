"""Shared helpers of the GPU parity tests: drive the HIP library and the oracle
through the same window schedule on the same seeded inputs, and compare."""

from __future__ import annotations

import math

import numpy as np
import torch

from oracle import mla as O
from synthetic import chunk_q, chunk_x, dense_weights, layer_weights

# Acceptance bar for bf16 storage with fp32 accumulation against the fp64 oracle.
BF16_MAX_REL = 1e-2      # max |gpu - ref| <= 1e-2 * max |ref|
BF16_MEAN_REL = 2e-3     # sum |gpu - ref| <= 2e-3 * sum |ref|
# fp32 path: fp32 rounding of O(100)-term sums, well inside these.
F32_MAX_REL = 1e-5
F32_MEAN_REL = 1e-6


def parity_stats(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    return float(err.max() / np.abs(ref).max()), float(err.sum() / np.abs(ref).sum())


# bf16 ring (split operands): the gate with a 25% margin.
BF16_RING_MEAN_REL = 1.5e-3


def assert_parity(got, ref, dtype="bf16", what="", mean_lim=None):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    mx, mean = parity_stats(got, ref)
    lim = (BF16_MAX_REL, BF16_MEAN_REL) if dtype == "bf16" else (F32_MAX_REL, F32_MEAN_REL)
    if mean_lim is not None:
        lim = (lim[0], min(lim[1], mean_lim))
    print(f"[parity] {what}: max_rel={mx:.3e} mean_rel={mean:.3e} (limits {lim[0]:.0e}/{lim[1]:.0e})",
          flush=True)
    assert mx <= lim[0] and mean <= lim[1], (what, mx, mean)
    return mx, mean


def dev(t):
    return t.to("cuda")


NAN_BITS = {"bf16": 0x7FC0, "f16": 0x7E00}
E4M3_NAN = 0x7F


def nan_fill_(storage, dtype):
    """Fill ring storage with NaN in the storage dtype."""
    if dtype == "e4m3":
        storage.view(torch.uint8).fill_(E4M3_NAN)
    elif dtype in NAN_BITS:
        storage.view(torch.int16).fill_(NAN_BITS[dtype])
    else:
        storage.view(torch.float32).fill_(float("nan"))


class LatentRun:
    """A latent cache driven in lock step on the GPU and in the oracle."""

    def __init__(self, cfg, poison=False, layer=0, storage_round=None, path=None):
        from rank_latent_kv_absorbed_amd import LatentCache
        self.cfg = cfg
        self.layer = layer
        self.w = layer_weights(cfg, layer=layer)
        self.wd = {k: dev(v) for k, v in self.w.items()}
        self.gpu = LatentCache(cfg)
        if path is not None:
            self.gpu.set_attend_path(path)
        if poison:
            nan_fill_(self.gpu.storage, cfg.cache_dtype)
        self.ring = O.RingModel(cfg.window_frames, cfg.T)
        self.store = O.new_store(cfg.batch, cfg.window_frames, cfg.T, cfg.width,
                                 fill=np.nan if poison else 0.0)
        self.rnd = storage_round or cfg.cache_dtype
        self.n_ops = 0
        self.last_frame0 = None
        self.q_norm = None

    def write(self, frame0, n_frames, x=None):
        if x is None:
            x = chunk_x(self.cfg, n_frames, layer=self.layer, chunk=self.n_ops)
        self.n_ops += 1
        self.gpu.write(dev(x), self.wd["w_dkr"], frame0, n_frames)
        O.cache_write(self.store, self.ring, x.double().numpy(), self.w["w_dkr"].double().numpy(),
                      frame0, n_frames, self.cfg, storage=self.rnd)
        self.last_frame0 = frame0
        return x

    def evict(self, n):
        self.gpu.evict(n)
        O.cache_evict(self.ring, n)

    def fill(self, oldest, newest, rows):
        """Make frames oldest..newest resident with the given stored rows
        [B, n_frames*T, width] (values exact in the cache type), on the GPU
        ring (set_state + copy into the resident slots) and in the oracle."""
        self.gpu.set_state(oldest, newest)
        self.ring.oldest, self.ring.newest = oldest, newest
        slots = self.ring.resident_slots()
        self.store[:, slots, :] = rows
        ring = self.gpu.ring()
        t = torch.from_numpy(np.ascontiguousarray(rows)).to(ring.dtype)
        if ring.dtype == torch.float8_e4m3fn:   # one-byte codes, copied as bytes
            ring, t = ring.view(torch.uint8), t.view(torch.uint8)
        ring[:, torch.from_numpy(slots)] = t.to(ring.device)
        torch.cuda.synchronize()

    def query(self, Lq, chunk=1000):
        return chunk_q(self.cfg, Lq, layer=self.layer, chunk=chunk)

    def set_query_norm(self, gamma, eps):
        """Query RMS norm on the GPU handle and in the oracle (gamma: CPU tensor
        in the input dtype, or None to switch it off)."""
        if gamma is None:
            self.gpu.set_query_norm(None)
            self.q_norm = None
            return
        self.gpu.set_query_norm(dev(gamma), eps)
        self.q_norm = (gamma.double().numpy(), eps)

    def attend(self, q, q_token0, key_splits=0, rows=None, workspace=None):
        out = self.gpu.attend(dev(q), q_token0, self.wd["w_uk"], self.wd["w_uv"],
                              key_splits=key_splits, workspace=workspace)
        torch.cuda.synchronize()
        ref = O.attend(self.store, self.ring, q.double().numpy(), q_token0,
                       self.w["w_uk"].double().numpy(), self.w["w_uv"].double().numpy(), self.cfg,
                       rows=rows, q_norm=self.q_norm)
        got = out.cpu().numpy()
        if rows is not None:
            got = got[:, rows]
        return got, ref, out


class DenseRun:
    """Dense per-head cache driven in lock step on the GPU and in the oracle."""

    def __init__(self, cfg, layer=0):
        from rank_latent_kv_absorbed_amd import DenseCache
        self.cfg = cfg
        self.w = dense_weights(cfg, layer=layer)
        self.wd = {k: dev(v) for k, v in self.w.items()}
        self.gpu = DenseCache(cfg)
        self.ring = O.RingModel(cfg.window_frames, cfg.T)
        d_h = cfg.d_qk
        self.split = O.default_rope_split(d_h)
        self.store = np.zeros((cfg.batch, cfg.window_frames * cfg.T, 2, cfg.n_heads, d_h))
        self.layer = layer
        self.n_ops = 0

    def write(self, frame0, n_frames):
        x = chunk_x(self.cfg, n_frames, layer=self.layer, chunk=self.n_ops)
        self.n_ops += 1
        self.gpu.write(dev(x), self.wd["w_k"], self.wd["w_v"], frame0, n_frames)
        O.mha_cache_write(self.store, self.ring, x.double().numpy(), self.w["w_k"].double().numpy(),
                          self.w["w_v"].double().numpy(), frame0, n_frames, self.cfg, self.split,
                          storage=self.cfg.cache_dtype)

    def evict(self, n):
        self.gpu.evict(n)
        O.cache_evict(self.ring, n)

    def attend(self, q, q_token0, rows=None):
        out = self.gpu.attend(dev(q), q_token0)
        torch.cuda.synchronize()
        ref = O.mha_attend(self.store, self.ring, q.double().numpy(), q_token0, self.cfg, self.split,
                           rows=rows)
        got = out.cpu().numpy()
        if rows is not None:
            got = got[:, rows]
        return got, ref


def sample_rows(Lq, n, seed=0):
    """Query rows to check at full size: first, last, the ragged tail and a spread."""
    rng = np.random.default_rng(seed)
    pick = {0, 1, Lq - 1, Lq - 2} | set(range(max(0, (Lq // 32) * 32 - 2), Lq))
    pick |= set(rng.choice(Lq, size=min(n, Lq), replace=False).tolist())
    return np.array(sorted(pick), dtype=np.int64)


def log2e_scale(d):
    return math.log2(math.e) / math.sqrt(d)
