"""Workload shapes: a tiny fp32 case and Wan-1.3B-shaped attention layers.

The Wan-1.3B head shape (12 heads of 128, latent 192, positional key 32) is the
one the VideoMLA technical summary uses for its default setting; the latent
frame grid of 30 x 52 tokens and the 21-frame window are the sliding-window
setting named in its problem definition.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class LayerConfig:
    name: str
    hidden: int
    n_heads: int
    d_nope: int
    d_rope: int
    d_v: int
    d_c: int
    grid_h: int
    grid_w: int
    window_frames: int
    batch: int = 1
    rope_split: tuple = None          # pairs per axis (t, h, w); None -> default
    rope_base: float = 10000.0
    dtype: str = "bf16"               # inputs (x, q, weights); accumulation is fp32
    cache_dtype: str = None           # ring storage; None -> fp16 for bf16 inputs, fp32 for fp32
    prefill_frames: int = 0           # frames written before the measured chunk
    evict_frames: int = 0             # frames evicted before the chunk is written
    chunk_frames: int = 3             # frames in the query chunk (written, then attended)
    seed: int = 0

    def __post_init__(self):
        if self.cache_dtype is None:
            object.__setattr__(self, "cache_dtype", "f32" if self.dtype == "f32" else "f16")
        if self.rope_split is None:
            p = self.d_rope // 2
            object.__setattr__(self, "rope_split", (p - 2 * (p // 3), p // 3, p // 3))

    @property
    def T(self):
        return self.grid_h * self.grid_w

    @property
    def d_qk(self):
        return self.d_nope + self.d_rope

    @property
    def width(self):
        """Scalars per cached token: d_c + d_rope."""
        return self.d_c + self.d_rope

    @property
    def Lq(self):
        return self.chunk_frames * self.T

    @property
    def chunk_frame0(self):
        return self.prefill_frames

    @property
    def Lk(self):
        return (self.prefill_frames - self.evict_frames + self.chunk_frames) * self.T

    def with_(self, **kw):
        return replace(self, **kw)


WAN = dict(hidden=1536, n_heads=12, d_nope=96, d_rope=32, d_v=128, d_c=192,
           grid_h=30, grid_w=52, window_frames=21)

CONFIGS = {
    # Tiny fp32 layer: 2 cached frames, then a 1-frame chunk; every query
    # attends to all 3 resident frames.
    "tiny": LayerConfig("tiny", hidden=64, n_heads=2, d_nope=24, d_rope=8, d_v=32, d_c=16,
                        grid_h=4, grid_w=4, window_frames=3, dtype="f32",
                        prefill_frames=2, chunk_frames=1),
    # One Wan-shaped layer, window not yet full: 6 cached frames + 3-frame chunk.
    "wan_layer": LayerConfig("wan_layer", **WAN, prefill_frames=6, chunk_frames=3),
    # Full 21-frame window: prefill 21, evict 3, write the 3-frame chunk, attend.
    "wan_window": LayerConfig("wan_window", **WAN, prefill_frames=21, evict_frames=3,
                              chunk_frames=3),
}


def config(name, **overrides):
    return CONFIGS[name].with_(**overrides) if overrides else CONFIGS[name]
