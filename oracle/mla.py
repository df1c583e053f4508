"""fp64 reference for the VideoMLA cache-write / attend / evict path.

TEST INFRASTRUCTURE ONLY (see the package docstring): never imported by the
product path.

What the pages fix (VideoMLA technical summary, gist.science, section 手法
"method", items 1-4; abstract on chatpaper.ai):
  1. each token's content is compressed by a down-projection W^KV_down into one
     latent c^KV_t shared by all heads, with d_c much smaller than n_h*d_h;
  2. during attention, each head's content key k^nope_{t,h} and value v_{t,h}
     are rebuilt from that latent with head-specific up-projections
     W^K_up and W^V_up;
  3. each head's q.k width is split into a content part d^nope_h and a
     positional part d^rope_h; a single positional key k^R_t shared by all
     heads is computed and rotated by 3D-RoPE; the cache stores the pair
     (c^KV_t, k^R_t) per token instead of dense per-head keys and values;
  4. per-token cache state drops from 2*n_h*d_h scalars to d_c + d^rope_h
     (92.7% at d_c=192, d^rope_h=32).
The surrounding setting (problem definition section and abstract): a
fixed-size sliding-window KV cache of latent frames, rolled out chunk by chunk.

Conventions (matrix-times-column-vector, as the pages write W c):
  w_dkr : [d_c + d_rope, hidden]   rows < d_c are W^KV_down, the rest W^KR
  w_uk  : [n_h, d_nope, d_c]       k^nope_{t,h} = w_uk[h] @ c_t
  w_uv  : [n_h, d_v, d_c]          v_{t,h}      = w_uv[h] @ c_t
  x     : [B, tokens, hidden]      tokens of whole latent frames, row-major (h, w)
  q     : [B, Lq, n_h, d_nope + d_rope]   per-head [q^nope | q^R], q^R un-rotated
  out   : [B, Lq, n_h, d_v]
Readings the pages leave open (each one listed with its reason in the design
notes): score scale 1/sqrt(d_nope + d_rope); RoPE pairs are adjacent
elements, grouped t then h then w, frequencies base^(-i/P_axis); positions are
(absolute latent-frame index, row, column); k^R comes from the layer input x;
no biases, and norms only where asked for (an RMS norm of the latent c in the
cache write; an RMS norm of each head's query row [q^nope | q^R] before its
rotation); the stored cache is rounded to the storage dtype (RNE).

Everything is float64 NumPy; a matmul is the only library primitive used as a
step.  Plain loops are used where they make the definition clearer.
"""

from __future__ import annotations

import math

import numpy as np

# ----------------------------------------------------------------------------
# Rounding of stored values (the cache dtype is part of the method: the pages'
# 92.7% and ~6.0 GB figures count stored scalars at 2 bytes each).
# ----------------------------------------------------------------------------


def round_to_bf16(a):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits (1 implicit + 7 stored) and the float32
    exponent range.  Written from the format's definition: scale the value so
    that the bits to keep form the integer part, round half to even
    (np.rint), scale back.  Subnormals keep a fixed quantum of 2^-133.
    Values beyond the largest finite bfloat16 become +-inf; NaN stays NaN.
    """
    a = np.asarray(a, dtype=np.float64)
    out = np.array(a, copy=True)
    finite = np.isfinite(a) & (a != 0.0)
    v = a[finite]
    _, e = np.frexp(v)                      # v = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                 # below 2^-126 the quantum stops shrinking
    q = np.ldexp(np.rint(np.ldexp(v, 8 - e)), e - 8)
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    q = np.where(np.abs(q) > bf16_max, np.copysign(np.inf, q), q)
    out[finite] = q
    return out


def round_to_f32(a):
    """Round float64 values to float32 (NumPy's cast is round-to-nearest-even)."""
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_to_f16(a):
    """Round float64 values to IEEE binary16 (NumPy's cast: nearest even,
    with binary16 subnormals and overflow to inf)."""
    with np.errstate(over="ignore"):  # overflow to inf is the intended result
        return np.asarray(a, dtype=np.float64).astype(np.float16).astype(np.float64)


def round_to_e4m3(a):
    """Round float64 values to the OCP 8-bit float E4M3 ('fn' variant), ties
    to even, saturating.

    E4M3 keeps 4 significant bits (1 implicit + 3 stored), exponent bias 7,
    no infinities: the largest finite magnitude is 1.75 * 2^8 = 448, the
    smallest normal 2^-6, and below it subnormals keep a fixed quantum of
    2^-9.  Written from the format's definition like round_to_bf16.  Values
    whose magnitude rounds past 448 saturate to +-448 (the format's saturating
    conversion; its only other choice is NaN); NaN stays NaN.
    """
    a = np.asarray(a, dtype=np.float64)
    out = np.array(a, copy=True)
    finite = np.isfinite(a) & (a != 0.0)
    v = a[finite]
    _, e = np.frexp(v)                      # v = m * 2^e, 0.5 <= |m| < 1
    e = np.maximum(e, -5)                   # below 2^-6 the quantum stops shrinking
    q = np.ldexp(np.rint(np.ldexp(v, 4 - e)), e - 4)
    out[finite] = np.clip(q, -448.0, 448.0)
    inf = np.isinf(a)
    out[inf] = np.copysign(448.0, a[inf])
    return out


def round_storage(a, dtype):
    """Round to the cache storage dtype: 'bf16', 'f16', 'e4m3', 'f32', or None
    (keep fp64)."""
    if dtype is None:
        return np.asarray(a, dtype=np.float64)
    if dtype == "bf16":
        return round_to_bf16(a)
    if dtype == "f16":
        return round_to_f16(a)
    if dtype == "e4m3":
        return round_to_e4m3(a)
    if dtype == "f32":
        return round_to_f32(a)
    raise ValueError(f"unknown storage dtype {dtype!r}")


# ----------------------------------------------------------------------------
# 3D-RoPE (technical summary, 手法 item 3: the shared positional key is rotated
# by 3D-RoPE over the frame, height and width axes).  The pages give no
# formula; the reading here is the standard rotary embedding applied per axis.
# ----------------------------------------------------------------------------


def default_rope_split(d_rope):
    """Pairs per axis (t, h, w): h and w get floor(P/3) pairs, t the rest."""
    if d_rope % 2:
        raise ValueError("d_rope must be even")
    p = d_rope // 2
    return (p - 2 * (p // 3), p // 3, p // 3)


def rope_pair_table(split, base):
    """For every rotated pair, in storage order: (axis, inverse frequency).

    Axis 0 = latent frame t, 1 = grid row h, 2 = grid column w.  Inside an axis
    group of P_a pairs, pair i turns at base^(-i / P_a) radians per position.
    """
    table = []
    for axis, n_pairs in enumerate(split):
        for i in range(n_pairs):
            table.append((axis, float(base) ** (-i / n_pairs)))
    return table


def rope3d(v, pos, split, base):
    """Rotate the last axis of ``v`` (2*sum(split) wide) at positions ``pos``.

    v   : [..., 2P] float64
    pos : [..., 3]  integer (t, h, w), broadcast against v's leading axes
    Pair p = (v[2p], v[2p+1]) turns by angle = pos[axis_p] * inv_freq_p:
        (a, b) -> (a cos - b sin, a sin + b cos).
    """
    v = np.asarray(v, dtype=np.float64)
    table = rope_pair_table(split, base)
    if v.shape[-1] != 2 * len(table):
        raise ValueError("rope width does not match the axis split")
    pos = np.asarray(pos)
    out = np.empty_like(v)
    for p, (axis, inv_freq) in enumerate(table):
        ang = pos[..., axis].astype(np.float64) * inv_freq
        c, s = np.cos(ang), np.sin(ang)
        a, b = v[..., 2 * p], v[..., 2 * p + 1]
        out[..., 2 * p] = a * c - b * s
        out[..., 2 * p + 1] = a * s + b * c
    return out


def token_position(g, grid_h, grid_w):
    """Global token index -> (latent frame, row, column); rows are row-major."""
    g = np.asarray(g, dtype=np.int64)
    t_per_frame = grid_h * grid_w
    tau = g % t_per_frame
    return np.stack([g // t_per_frame, tau // grid_w, tau % grid_w], axis=-1)


# ----------------------------------------------------------------------------
# The sliding window (abstract: a fixed-size sliding-window KV cache; problem
# definition: a cache of 21 latent frames).  Whole frames enter at the newest
# end and leave from the oldest end; a frame's tokens live at a fixed slot.
# ----------------------------------------------------------------------------


class RingError(Exception):
    """A write or eviction that the window cannot take."""


class RingModel:
    """Which latent frames are resident, and where each token is stored.

    Slot of token tau of frame f: (f mod W) * T + tau, with W the capacity in
    frames and T tokens per frame.  Writes must continue the newest frame and
    fit in the free capacity; evictions remove the oldest frames.
    """

    def __init__(self, window_frames, tokens_per_frame):
        if window_frames <= 0 or tokens_per_frame <= 0:
            raise ValueError("window and frame size must be positive")
        self.W = int(window_frames)
        self.T = int(tokens_per_frame)
        self.oldest = 0
        self.newest = -1

    @property
    def n_resident(self):
        return self.newest - self.oldest + 1

    def write(self, frame0, n_frames):
        if n_frames <= 0:
            raise RingError("write of no frames")
        if frame0 < 0:
            raise RingError("negative frame index")
        if self.n_resident > 0 and frame0 != self.newest + 1:
            raise RingError("frames must continue the newest resident frame")
        if self.n_resident + n_frames > self.W:
            raise RingError("window full")
        if self.n_resident == 0:
            self.oldest = frame0
        self.newest = frame0 + n_frames - 1

    def evict(self, n_frames):
        if n_frames < 0 or n_frames > self.n_resident:
            raise RingError("evicting more frames than are resident")
        self.oldest += n_frames

    def slot(self, frame, tau):
        return (int(frame) % self.W) * self.T + int(tau)

    def resident_frames(self):
        return list(range(self.oldest, self.newest + 1))

    def resident_slots(self):
        """Slots of every resident token, oldest frame first, tau ascending."""
        return np.array([self.slot(f, tau) for f in self.resident_frames()
                         for tau in range(self.T)], dtype=np.int64)

    def resident_tokens(self):
        """Global token index of every resident token, in resident_slots order."""
        return np.array([f * self.T + tau for f in self.resident_frames()
                         for tau in range(self.T)], dtype=np.int64)


# ----------------------------------------------------------------------------
# Cache write (手法 items 1 and 3): c = W^KV_down x, k^R = RoPE3D(W^KR x), the
# pair stored, rounded to the cache dtype, at the token's ring slot.
# ----------------------------------------------------------------------------


def new_store(batch, window_frames, tokens_per_frame, width, fill=0.0):
    return np.full((batch, window_frames * tokens_per_frame, width), fill, dtype=np.float64)


def rms_norm(v, gamma, eps):
    """Root-mean-square normalisation over the last axis:
    gamma * v / sqrt(mean(v^2) + eps)."""
    v = np.asarray(v, dtype=np.float64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return np.asarray(gamma, dtype=np.float64) * v / np.sqrt(ms + eps)


def cache_write(store, ring, x, w_dkr, frame0, n_frames, cfg, storage="bf16", kv_norm=None):
    """Write n_frames whole latent frames of layer input x into the ring.

    store   : [B, W*T, d_c + d_rope] float64, updated in place
    x       : [B, n_frames*T, hidden]
    kv_norm : optional (gamma [d_c], eps): the latent c is RMS-normalised
              (rms_norm) before it is stored; k^R is not.
    Returns the (unrounded) rows [B, n_frames*T, d_c + d_rope] for inspection.
    """
    T = cfg.grid_h * cfg.grid_w
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w_dkr, dtype=np.float64)
    assert x.shape[1] == n_frames * T and w.shape == (cfg.d_c + cfg.d_rope, cfg.hidden)
    ring.write(frame0, n_frames)
    y = x @ w.T                                          # [B, n*T, d_c + d_rope]
    c = y[..., :cfg.d_c]
    if kv_norm is not None:
        c = rms_norm(c, kv_norm[0], kv_norm[1])
    g = frame0 * T + np.arange(n_frames * T)
    kr = rope3d(y[..., cfg.d_c:], token_position(g, cfg.grid_h, cfg.grid_w),
                cfg.rope_split, cfg.rope_base)
    rows = np.concatenate([c, kr], axis=-1)
    for i, gi in enumerate(g):
        store[:, ring.slot(gi // T, gi % T), :] = round_storage(rows[:, i, :], storage)
    return rows


def cache_evict(ring, n_frames):
    """Drop the n oldest resident frames (bookkeeping only; no values change)."""
    ring.evict(n_frames)


# ----------------------------------------------------------------------------
# Attend (手法 item 2, explicit on-demand rebuild): for each head, rebuild
# k^nope = W^K_up c and v = W^V_up c for every resident token, score with the
# shared rotated k^R, softmax over the whole window, weight the values.
# ----------------------------------------------------------------------------


def attend(store, ring, q, q_token0, w_uk, w_uv, cfg, rows=None, block=512, q_norm=None):
    """Attention of query chunk q over every resident token, per head.

    Keys are all tokens of all resident frames (no mask inside the window).
    Query i sits at global token q_token0 + i; its q^R is rotated there.
    rows: optional array of query indices to evaluate (default: all).
    q_norm: optional (gamma [d_nope + d_rope], eps): each head's query row
    [q^nope | q^R] is RMS-normalised (rms_norm over its d_nope + d_rope values,
    the same gain for every head) before anything else, the rotation included.
    Returns float64 [B, len(rows), n_h, d_v].
    """
    q = np.asarray(q, dtype=np.float64)
    B, Lq, n_h, dq = q.shape
    assert n_h == cfg.n_heads and dq == cfg.d_nope + cfg.d_rope
    if q_norm is not None:
        q = rms_norm(q, q_norm[0], q_norm[1])
    if ring.n_resident <= 0:
        raise RingError("attend on an empty window")
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    slots = ring.resident_slots()
    C = store[:, slots, :cfg.d_c]                         # [B, Lk, d_c]
    KR = store[:, slots, cfg.d_c:]                        # [B, Lk, d_rope]
    scale = 1.0 / math.sqrt(cfg.d_nope + cfg.d_rope)
    out = np.empty((B, len(rows), n_h, cfg.d_v), dtype=np.float64)
    for h in range(n_h):
        w_k = np.asarray(w_uk[h], dtype=np.float64)        # [d_nope, d_c]
        w_v = np.asarray(w_uv[h], dtype=np.float64)        # [d_v, d_c]
        K_nope = C @ w_k.T                                 # [B, Lk, d_nope]
        V = C @ w_v.T                                      # [B, Lk, d_v]
        for r0 in range(0, len(rows), block):
            rb = rows[r0:r0 + block]
            qn = q[:, rb, h, :cfg.d_nope]
            pos = token_position(q_token0 + rb, cfg.grid_h, cfg.grid_w)
            qr = rope3d(q[:, rb, h, cfg.d_nope:], pos, cfg.rope_split, cfg.rope_base)
            s = (qn @ K_nope.transpose(0, 2, 1) + qr @ KR.transpose(0, 2, 1)) * scale
            s = s - s.max(axis=-1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=-1, keepdims=True)
            out[:, r0:r0 + len(rb), h, :] = p @ V
    return out


# ----------------------------------------------------------------------------
# The attention block from the layer input to model width.  Around the steps
# above sit the layer's query projection (each head's [q^nope | q^R], the
# split of 手法 item 3) and its output projection W^O over the heads'
# concatenated outputs; the pages print neither, and the readings here are the
# plain ones: q = W_q x, out = W_O [o_1; ...; o_n_h].
#   w_q : [n_h * (d_nope + d_rope), hidden]   head h's rows are [W^nope_q,h ; W^R_q,h]
#   w_o : [hidden, n_h * d_v]                 head h's columns follow o_h
# ----------------------------------------------------------------------------


def query_projection(x, w_q, cfg):
    """Per-head queries [B, L, n_h, d_nope + d_rope] (q^R not yet rotated)."""
    x = np.asarray(x, dtype=np.float64)
    B, L, _ = x.shape
    return (x @ np.asarray(w_q, dtype=np.float64).T).reshape(B, L, cfg.n_heads, cfg.d_nope + cfg.d_rope)


def attend_block(store, ring, x, q_token0, w_q, w_uk, w_uv, w_o, cfg, rows=None):
    """Query tokens' layer input x [B, Lq, hidden] -> [B, len(rows), hidden]:
    queries from the projection, attention over the window exactly as in
    attend (explicit per-head rebuild), then W_O over the heads' outputs."""
    q = query_projection(x, w_q, cfg)
    o = attend(store, ring, q, q_token0, w_uk, w_uv, cfg, rows=rows)
    B, R = o.shape[:2]
    return o.reshape(B, R, cfg.n_heads * cfg.d_v) @ np.asarray(w_o, dtype=np.float64).T


# ----------------------------------------------------------------------------
# Dense per-head MHA (problem definition: every cached token stores full keys
# and values for every head).  The in-run comparison for the cache-byte claim.
# Keys are rotated by 3D-RoPE over the whole head width.
# ----------------------------------------------------------------------------


def mha_cache_write(store, ring, x, w_k, w_v, frame0, n_frames, cfg, split, storage="bf16"):
    """Dense cache write: per head k = RoPE3D((W_K x)_h), v = (W_V x)_h.

    store : [B, W*T, 2, n_h, d_h] float64; w_k, w_v : [n_h*d_h, hidden]
    """
    T = cfg.grid_h * cfg.grid_w
    n_h, d_h = cfg.n_heads, cfg.d_nope + cfg.d_rope
    x = np.asarray(x, dtype=np.float64)
    ring.write(frame0, n_frames)
    g = frame0 * T + np.arange(n_frames * T)
    pos = token_position(g, cfg.grid_h, cfg.grid_w)
    k = (x @ np.asarray(w_k, np.float64).T).reshape(x.shape[0], -1, n_h, d_h)
    v = (x @ np.asarray(w_v, np.float64).T).reshape(x.shape[0], -1, n_h, d_h)
    k = rope3d(k, pos[None, :, None, :], split, cfg.rope_base)
    for i, gi in enumerate(g):
        s = ring.slot(gi // T, gi % T)
        store[:, s, 0] = round_storage(k[:, i], storage)
        store[:, s, 1] = round_storage(v[:, i], storage)


def mha_attend(store, ring, q, q_token0, cfg, split, rows=None, block=512):
    """Textbook per-head softmax attention over the dense window.

    q is rotated over the whole head width at its token's position.
    Returns float64 [B, len(rows), n_h, d_h].
    """
    q = np.asarray(q, dtype=np.float64)
    B, Lq, n_h, d_h = q.shape
    rows = np.arange(Lq) if rows is None else np.asarray(rows, dtype=np.int64)
    slots = ring.resident_slots()
    scale = 1.0 / math.sqrt(d_h)
    out = np.empty((B, len(rows), n_h, d_h), dtype=np.float64)
    for h in range(n_h):
        K = store[:, slots, 0, h, :]
        V = store[:, slots, 1, h, :]
        for r0 in range(0, len(rows), block):
            rb = rows[r0:r0 + block]
            pos = token_position(q_token0 + rb, cfg.grid_h, cfg.grid_w)
            qr = rope3d(q[:, rb, h, :], pos, split, cfg.rope_base)
            s = (qr @ K.transpose(0, 2, 1)) * scale
            s = s - s.max(axis=-1, keepdims=True)
            p = np.exp(s)
            p /= p.sum(axis=-1, keepdims=True)
            out[:, r0:r0 + len(rb), h, :] = p @ V
    return out


# ----------------------------------------------------------------------------
# Byte accounting (手法 item 4; problem definition's ~6.0 GB dense cache).
# ----------------------------------------------------------------------------


def latent_scalars_per_token(cfg):
    """Scalars stored per token per cached layer: d_c + d^rope_h."""
    return cfg.d_c + cfg.d_rope


def dense_scalars_per_token(cfg):
    """Dense per-head state per token per cached layer: 2 * n_h * d_h."""
    return 2 * cfg.n_heads * (cfg.d_nope + cfg.d_rope)


def kv_reduction(cfg):
    """Fraction of per-token KV memory removed at every cached layer."""
    return 1.0 - latent_scalars_per_token(cfg) / dense_scalars_per_token(cfg)


def cache_bytes(scalars_per_token, tokens, layers=1, bytes_per_scalar=2, batch=1):
    return int(scalars_per_token) * int(tokens) * int(layers) * int(bytes_per_scalar) * int(batch)
