"""Pins for the fp64 oracle: each test checks it against something other than
itself -- numbers printed on the VideoMLA pages, library routines it reduces to,
closed forms, invariants of rotations and of softmax, and brute force.

A plausible slip anywhere in the oracle (a dropped term, a wrong sign or index,
a transposed operand, a wrong slot) fails at least one of these.
"""

import cmath
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import mla as O
from synthetic import config

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "paper_numbers.json")))


# --------------------------------------------------------------------------
# Numbers printed on the pages
# --------------------------------------------------------------------------

def test_kv_reduction_matches_printed_percentage():
    wan = config("wan_window")
    assert wan.d_c == GOLDEN["default_d_c"]["value"]
    assert wan.d_rope == GOLDEN["default_d_rope"]["value"]
    assert O.latent_scalars_per_token(wan) == 224
    assert O.dense_scalars_per_token(wan) == 3072
    pct = 100.0 * O.kv_reduction(wan)
    g = GOLDEN["kv_reduction_percent"]
    assert abs(pct - g["value"]) <= g["printed_precision"], pct
    assert O.kv_reduction(wan) == 1.0 - 224.0 / 3072.0


def test_head_shape_from_the_pages():
    wan = config("wan_window")
    assert wan.n_heads == GOLDEN["wan_heads"]["value"]
    assert wan.d_qk == GOLDEN["wan_head_dim"]["value"]
    assert wan.n_heads * wan.d_qk == GOLDEN["wan_heads_times_head_dim"]["value"]
    assert wan.d_c == GOLDEN["analogy_latent_width"]["value"]


def test_dense_cache_size_matches_printed_gigabytes():
    wan = config("wan_window")
    frames = GOLDEN["window_latent_frames"]["value"]
    dense = O.cache_bytes(O.dense_scalars_per_token(wan), frames * wan.T, layers=30)
    assert dense == 6_038_323_200
    g = GOLDEN["dense_cache_21_frames_gb"]
    assert abs(dense / 1e9 - g["value"]) <= g["printed_precision"]
    latent = O.cache_bytes(O.latent_scalars_per_token(wan), frames * wan.T, layers=30)
    assert latent == 440_294_400
    for d_c, want in ((128, 314_496_000), (64, 188_697_600)):
        assert O.cache_bytes(d_c + 32, frames * wan.T, layers=30) == want


# --------------------------------------------------------------------------
# Storage rounding against torch's own dtype conversion
# --------------------------------------------------------------------------

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    v = rng.standard_normal(20000) * np.exp2(rng.integers(-40, 40, 20000))
    v = v.astype(np.float32)
    # exact ties: a bf16 value plus half its quantum, both parities of the last bit
    base = torch.from_numpy(v[:2000]).to(torch.bfloat16).to(torch.float32).numpy()
    _, e = np.frexp(base.astype(np.float64))
    ties = (base.astype(np.float64) + np.ldexp(1.0, e - 9)).astype(np.float32)
    tiny = (rng.standard_normal(500) * 2.0 ** -130).astype(np.float32)   # subnormal range
    allv = np.concatenate([v, ties, tiny, np.float32([0.0, -0.0, 1.0, -3.5])])
    want = torch.from_numpy(allv).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_to_bf16(allv.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_f16_rounding_matches_torch():
    rng = np.random.default_rng(9)
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 18, 20000))).astype(np.float32)
    want = torch.from_numpy(v).to(torch.float16).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_to_f16(v.astype(np.float64)), want)


def test_f16_rounding_overflows_to_infinity_past_the_range():
    """IEEE binary16: the largest finite value is 65504; values round to it up
    to half an ulp (16) past it, and to infinity from 65520 on."""
    v = np.array([65504.0, 65519.99, 65520.0, 1e6, -65520.0, -65504.0])
    got = O.round_to_f16(v)
    np.testing.assert_array_equal(got, [65504.0, 65504.0, np.inf, np.inf, -np.inf, -65504.0])
    want = torch.from_numpy(v.astype(np.float32)).to(torch.float16).to(torch.float64).numpy()
    np.testing.assert_array_equal(got, want)


def test_e4m3_rounding_matches_torch():
    """OCP E4M3 against torch's float8_e4m3fn conversion, inside the range
    where the two agree (|v| <= 464: torch turns larger values into NaN)."""
    rng = np.random.default_rng(21)
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-14, 8, 20000))).astype(np.float32)
    v = v[np.abs(v) <= 464.0]
    # every finite code, and the exact midpoints between neighbouring codes
    # (both parities of the last stored bit)
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    codes = np.unique(codes[np.isfinite(codes)])
    mids = (codes[:-1] + codes[1:]) / 2.0
    allv = np.concatenate([v.astype(np.float64), codes, mids, [0.0, -0.0, 464.0, -464.0, 447.9]])
    want = torch.from_numpy(allv.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_to_e4m3(allv), want)


def test_e4m3_code_table_closed_forms():
    """The representable magnitudes are m * 2^-9 (m = 0..7, subnormal) and
    (1 + k/8) * 2^(e-7) for e = 1..15, k = 0..7 except e = 15, k = 7 (NaN):
    253 finite non-negative values up to 448; each rounds to itself."""
    sub = np.arange(8) * 2.0 ** -9
    norm = np.array([(1 + k / 8) * 2.0 ** (e - 7) for e in range(1, 16) for k in range(8)
                     if not (e == 15 and k == 7)])
    table = np.concatenate([sub, norm])
    assert table.size == 127 and table.max() == 448.0 and norm.min() == 2.0 ** -6
    both = np.concatenate([table, -table])
    np.testing.assert_array_equal(O.round_to_e4m3(both), both)
    # a value between two codes goes to the nearer one
    np.testing.assert_array_equal(O.round_to_e4m3(table[1:] - 0.3 * np.diff(table)), table[1:])
    np.testing.assert_array_equal(O.round_to_e4m3(table[:-1] + 0.3 * np.diff(table)), table[:-1])


def test_e4m3_saturates_past_the_range():
    """Magnitudes that round past 448 saturate to +-448 (the format has no
    infinity); NaN stays NaN."""
    v = np.array([448.0, 463.99, 464.0, 465.0, 1e6, np.inf, -np.inf, -500.0, np.nan])
    got = O.round_to_e4m3(v)
    np.testing.assert_array_equal(got[:-1], [448.0, 448.0, 448.0, 448.0, 448.0, 448.0, -448.0, -448.0])
    assert np.isnan(got[-1])


def test_f32_rounding_matches_torch():
    v = np.random.default_rng(2).standard_normal(1000) * 1e3
    want = torch.from_numpy(v).to(torch.float32).to(torch.float64).numpy()
    np.testing.assert_array_equal(O.round_to_f32(v), want)


# --------------------------------------------------------------------------
# 3D-RoPE: rotation invariants and the textbook 1D case
# --------------------------------------------------------------------------

SPLIT = (6, 5, 5)


def _rand_pos(rng, n):
    return np.stack([rng.integers(0, 300, n), rng.integers(0, 30, n), rng.integers(0, 52, n)], -1)


def test_default_axis_split():
    assert O.default_rope_split(32) == (6, 5, 5)
    assert O.default_rope_split(8) == (2, 1, 1)
    assert O.default_rope_split(128) == (22, 21, 21)
    assert config("wan_window").rope_split == (6, 5, 5)
    assert config("tiny").rope_split == (2, 1, 1)


def test_rope_preserves_norm_and_identity_at_origin():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((64, 32))
    pos = _rand_pos(rng, 64)
    r = O.rope3d(v, pos, SPLIT, 10000.0)
    np.testing.assert_allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(v, axis=-1), rtol=1e-13)
    np.testing.assert_array_equal(O.rope3d(v, np.zeros((64, 3), int), SPLIT, 10000.0), v)


def test_rope_composes_additively():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((32, 32))
    p1, p2 = _rand_pos(rng, 32), _rand_pos(rng, 32)
    a = O.rope3d(O.rope3d(v, p1, SPLIT, 10000.0), p2, SPLIT, 10000.0)
    b = O.rope3d(v, p1 + p2, SPLIT, 10000.0)
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_rope_inner_product_depends_on_offset_only():
    rng = np.random.default_rng(5)
    a, b = rng.standard_normal((16, 32)), rng.standard_normal((16, 32))
    p, pp, s = _rand_pos(rng, 16), _rand_pos(rng, 16), _rand_pos(rng, 16)
    d1 = np.sum(O.rope3d(a, p, SPLIT, 1e4) * O.rope3d(b, pp, SPLIT, 1e4), -1)
    d2 = np.sum(O.rope3d(a, p + s, SPLIT, 1e4) * O.rope3d(b, pp + s, SPLIT, 1e4), -1)
    np.testing.assert_allclose(d1, d2, rtol=1e-11, atol=1e-11)


def test_rope_single_axis_is_textbook_rotary():
    # One axis holding every pair: pair i of a d-wide vector turns by
    # t * base^(-2i/d), i.e. multiplication by exp(1j * angle) in the complex plane.
    rng = np.random.default_rng(6)
    d, base = 16, 10000.0
    v = rng.standard_normal((10, d))
    t = rng.integers(0, 500, 10)
    pos = np.stack([t, rng.integers(0, 9, 10), rng.integers(0, 9, 10)], -1)
    got = O.rope3d(v, pos, (d // 2, 0, 0), base)
    for n in range(10):
        for i in range(d // 2):
            z = complex(v[n, 2 * i], v[n, 2 * i + 1]) * cmath.exp(1j * t[n] * base ** (-2.0 * i / d))
            assert abs(got[n, 2 * i] - z.real) < 1e-12 and abs(got[n, 2 * i + 1] - z.imag) < 1e-12
    # the h and w groups read their own axes: with only an h group, t and w do not matter
    got_h = O.rope3d(v, pos, (0, d // 2, 0), base)
    pos2 = pos.copy()
    pos2[:, 0] += 7
    pos2[:, 2] += 3
    np.testing.assert_array_equal(got_h, O.rope3d(v, pos2, (0, d // 2, 0), base))


def test_token_position_row_major():
    p = O.token_position(np.array([0, 1, 51, 52, 1559, 1560, 3 * 1560 + 2 * 52 + 5]), 30, 52)
    assert p.tolist() == [[0, 0, 0], [0, 0, 1], [0, 0, 51], [0, 1, 0], [0, 29, 51], [1, 0, 0], [3, 2, 5]]


# --------------------------------------------------------------------------
# Sliding window: slot map and scripted minute-scale schedule
# --------------------------------------------------------------------------

def test_ring_rollout_schedule_closed_form():
    W, T, F = 21, 1560, 3
    ring = O.RingModel(W, T)
    for k in range(80):
        ring.evict(max(0, ring.n_resident + F - W))
        ring.write(F * k, F)
        assert ring.oldest == max(0, F * k + F - W)
        assert ring.newest == F * k + F - 1
        assert ring.n_resident == min(F * (k + 1), W)
        slots = ring.resident_slots()
        assert len(np.unique(slots)) == len(slots) == ring.n_resident * T
        assert slots.min() >= 0 and slots.max() < W * T
        f = np.repeat(np.arange(ring.oldest, ring.newest + 1), T)
        tau = np.tile(np.arange(T), ring.n_resident)
        np.testing.assert_array_equal(slots, (f % W) * T + tau)


def test_ring_errors_leave_state_unchanged():
    ring = O.RingModel(3, 4)
    with pytest.raises(O.RingError):
        ring.evict(1)
    ring.write(5, 2)
    for bad in ((8, 1), (7, 2), (6, 1), (7, 0), (-1, 1)):
        with pytest.raises(O.RingError):
            ring.write(*bad)
        assert (ring.oldest, ring.newest) == (5, 6)
    with pytest.raises(O.RingError):
        ring.evict(3)
    ring.evict(2)
    assert ring.n_resident == 0
    ring.write(40, 3)            # an empty window takes any start frame
    assert ring.resident_frames() == [40, 41, 42]


# --------------------------------------------------------------------------
# Cache write: exact-integer placement fixture
# --------------------------------------------------------------------------

def test_cache_write_exact_placement():
    cfg = config("tiny").with_(dtype="bf16")
    T = cfg.T
    rng = np.random.default_rng(7)
    w = O.round_to_bf16(rng.standard_normal((cfg.width, cfg.hidden)))
    w[cfg.d_c:] = 0.0                                  # k^R rows zero: rope output exactly 0
    ring = O.RingModel(cfg.window_frames, T)
    store = O.new_store(1, cfg.window_frames, T, cfg.width, fill=np.nan)
    frame0, n = 4, 2                                   # frames 4, 5 -> slots of frames 1, 2
    x = np.zeros((1, n * T, cfg.hidden))
    ks = rng.permutation(cfg.hidden)[: n * T]
    es = rng.integers(-3, 4, n * T)
    for i in range(n * T):
        x[0, i, ks[i]] = 2.0 ** es[i]
    O.cache_write(store, ring, x, w, frame0, n, cfg, storage="bf16")
    for i in range(n * T):
        f, tau = frame0 + i // T, i % T
        slot = (f % cfg.window_frames) * T + tau
        np.testing.assert_array_equal(store[0, slot, : cfg.d_c], 2.0 ** es[i] * w[: cfg.d_c, ks[i]])
        np.testing.assert_array_equal(store[0, slot, cfg.d_c:], 0.0)
    assert np.isnan(store[0, :T]).all()                # frame slot 0 never written


# --------------------------------------------------------------------------
# Attention: absorption, reduction to MHA, softmax special cases, brute force
# --------------------------------------------------------------------------

def _setup(cfg, frames_before=2, chunk=1, storage=None, seed=0, fill=0.0, frame_offset=0):
    rng = np.random.default_rng(seed)
    T = cfg.T
    w = rng.standard_normal((cfg.width, cfg.hidden)) / math.sqrt(cfg.hidden)
    w_uk = rng.standard_normal((cfg.n_heads, cfg.d_nope, cfg.d_c)) / math.sqrt(cfg.d_c)
    w_uv = rng.standard_normal((cfg.n_heads, cfg.d_v, cfg.d_c)) / math.sqrt(cfg.d_c)
    ring = O.RingModel(cfg.window_frames, T)
    store = O.new_store(cfg.batch, cfg.window_frames, T, cfg.width, fill=fill)
    n = frames_before + chunk
    x = rng.standard_normal((cfg.batch, n * T, cfg.hidden))
    O.cache_write(store, ring, x[:, : frames_before * T], w, frame_offset, frames_before, cfg, storage)
    O.cache_write(store, ring, x[:, frames_before * T:], w, frame_offset + frames_before, chunk, cfg,
                  storage)
    q = rng.standard_normal((cfg.batch, chunk * T, cfg.n_heads, cfg.d_qk))
    return dict(store=store, ring=ring, q=q, q_token0=(frame_offset + frames_before) * T,
                w_uk=w_uk, w_uv=w_uv, w=w, x=x)


def _softmax(s):
    s = s - s.max(-1, keepdims=True)
    p = np.exp(s)
    return p / p.sum(-1, keepdims=True)


def test_absorbed_form_equals_explicit_rebuild():
    cfg = config("tiny").with_(batch=2)
    st = _setup(cfg, storage="bf16")
    ref = O.attend(st["store"], st["ring"], st["q"], st["q_token0"], st["w_uk"], st["w_uv"], cfg)
    # absorbed: fold W^K_up into the query, attend in latent space, apply W^V_up after
    slots = st["ring"].resident_slots()
    C, KR = st["store"][:, slots, : cfg.d_c], st["store"][:, slots, cfg.d_c:]
    Lq = st["q"].shape[1]
    pos = O.token_position(st["q_token0"] + np.arange(Lq), cfg.grid_h, cfg.grid_w)
    out = np.empty_like(ref)
    for h in range(cfg.n_heads):
        q_lat = st["q"][:, :, h, : cfg.d_nope] @ st["w_uk"][h]            # [B, Lq, d_c]
        q_r = O.rope3d(st["q"][:, :, h, cfg.d_nope:], pos, cfg.rope_split, cfg.rope_base)
        s = (q_lat @ C.transpose(0, 2, 1) + q_r @ KR.transpose(0, 2, 1)) / math.sqrt(cfg.d_qk)
        o_lat = _softmax(s) @ C                                             # [B, Lq, d_c]
        out[:, :, h] = o_lat @ st["w_uv"][h].T
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def _sdpa(q, k, v, scale):
    """torch's CPU scaled-dot-product attention in float64."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    return torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), scale=scale).numpy()


@pytest.mark.parametrize("d_rope", [0, 8])
def test_reduces_to_standard_mha_with_block_selector_up_projections(d_rope):
    # d_c = n_h * (d_nope + d_v): the latent holds every head's key and value
    # block; W^K_up,h and W^V_up,h are selectors of head h's blocks.
    n_h, d_nope, d_v = 2, 8, 6
    d_c = n_h * (d_nope + d_v)
    cfg = config("tiny").with_(d_c=d_c, d_nope=d_nope, d_v=d_v, d_rope=d_rope, n_heads=n_h,
                               rope_split=None, batch=2, dtype="f32")
    st = _setup(cfg, storage=None, seed=11)
    w_uk = np.zeros((n_h, d_nope, d_c))
    w_uv = np.zeros((n_h, d_v, d_c))
    for h in range(n_h):
        o = h * (d_nope + d_v)
        w_uk[h][:, o:o + d_nope] = np.eye(d_nope)
        w_uv[h][:, o + d_nope:o + d_nope + d_v] = np.eye(d_v)
    got = O.attend(st["store"], st["ring"], st["q"], st["q_token0"], w_uk, w_uv, cfg)
    # textbook MHA on keys/values projected directly from x
    x, w = st["x"], st["w"]
    Lq = st["q"].shape[1]
    T = cfg.T
    kv = x @ w[:d_c].T                                                     # [B, Lk, d_c]
    kr = O.rope3d(x @ w[d_c:].T, O.token_position(np.arange(x.shape[1]), cfg.grid_h, cfg.grid_w),
                  cfg.rope_split, cfg.rope_base)
    pos = O.token_position(st["q_token0"] + np.arange(Lq), cfg.grid_h, cfg.grid_w)
    for h in range(n_h):
        o = h * (d_nope + d_v)
        k = np.concatenate([kv[..., o:o + d_nope], kr], -1)
        v = kv[..., o + d_nope:o + d_nope + d_v]
        qh = np.concatenate([st["q"][:, :, h, :d_nope],
                             O.rope3d(st["q"][:, :, h, d_nope:], pos, cfg.rope_split, cfg.rope_base)], -1)
        want = _sdpa(qh, k, v, 1.0 / math.sqrt(d_nope + d_rope))
        np.testing.assert_allclose(got[:, :, h], want, rtol=1e-11, atol=1e-12)
    assert T == 16


def test_single_key_returns_its_value():
    cfg = config("tiny").with_(grid_h=1, grid_w=1, window_frames=1)
    rng = np.random.default_rng(12)
    ring = O.RingModel(1, 1)
    store = O.new_store(1, 1, 1, cfg.width)
    w = rng.standard_normal((cfg.width, cfg.hidden))
    x = rng.standard_normal((1, 1, cfg.hidden))
    O.cache_write(store, ring, x, w, 9, 1, cfg, storage=None)
    w_uk = rng.standard_normal((cfg.n_heads, cfg.d_nope, cfg.d_c))
    w_uv = rng.standard_normal((cfg.n_heads, cfg.d_v, cfg.d_c))
    q = rng.standard_normal((1, 1, cfg.n_heads, cfg.d_qk)) * 30.0
    out = O.attend(store, ring, q, 9, w_uk, w_uv, cfg)
    c = x[0, 0] @ w[: cfg.d_c].T
    for h in range(cfg.n_heads):
        np.testing.assert_allclose(out[0, 0, h], w_uv[h] @ c, rtol=1e-13)


def test_identical_keys_and_zero_queries_give_plain_means():
    cfg = config("tiny")
    st = _setup(cfg, storage=None, seed=13)
    slots = st["ring"].resident_slots()
    C = st["store"][0, slots, : cfg.d_c]
    # q = 0: uniform weights, the output is the mean of the rebuilt values
    out = O.attend(st["store"], st["ring"], np.zeros_like(st["q"]), st["q_token0"], st["w_uk"],
                   st["w_uv"], cfg)
    for h in range(cfg.n_heads):
        np.testing.assert_allclose(out[0, :, h], np.broadcast_to((C @ st["w_uv"][h].T).mean(0),
                                                                 out[0, :, h].shape), rtol=1e-12)
    # identical latents and zero k^R: every key equal, output = that key's value
    store = st["store"].copy()
    store[:, :, : cfg.d_c] = C[0]
    store[:, :, cfg.d_c:] = 0.0
    out = O.attend(store, st["ring"], st["q"] * 10, st["q_token0"], st["w_uk"], st["w_uv"], cfg)
    for h in range(cfg.n_heads):
        np.testing.assert_allclose(out[0, :, h], np.broadcast_to(st["w_uv"][h] @ C[0],
                                                                 out[0, :, h].shape), rtol=1e-12)


def test_frame_shift_invariance():
    # Relative positions only: shifting every frame index by a constant leaves
    # the (unrounded) attention output unchanged.
    cfg = config("tiny")
    a = _setup(cfg, storage=None, seed=14, frame_offset=0)
    b = _setup(cfg, storage=None, seed=14, frame_offset=123)
    oa = O.attend(a["store"], a["ring"], a["q"], a["q_token0"], a["w_uk"], a["w_uv"], cfg)
    ob = O.attend(b["store"], b["ring"], b["q"], b["q_token0"], b["w_uk"], b["w_uv"], cfg)
    np.testing.assert_allclose(oa, ob, rtol=1e-10, atol=1e-12)


def test_key_order_and_unresident_slots_do_not_matter():
    # Filling every slot outside the window with NaN must not change the output.
    cfg = config("tiny").with_(window_frames=5)
    a = _setup(cfg, storage=None, seed=15, fill=0.0)
    b = _setup(cfg, storage=None, seed=15, fill=np.nan)
    oa = O.attend(a["store"], a["ring"], a["q"], a["q_token0"], a["w_uk"], a["w_uv"], cfg)
    ob = O.attend(b["store"], b["ring"], b["q"], b["q_token0"], b["w_uk"], b["w_uv"], cfg)
    np.testing.assert_array_equal(oa, ob)


def test_brute_force_scalar_loops_on_tiny_config():
    """The whole write -> attend path as scalar loops, rotations via complex numbers."""
    cfg = config("tiny")
    st = _setup(cfg, storage="f32", seed=16)
    got = O.attend(st["store"], st["ring"], st["q"], st["q_token0"], st["w_uk"], st["w_uv"], cfg)
    T, gw = cfg.T, cfg.grid_w
    P = cfg.d_rope // 2
    groups = []
    for axis, n in enumerate(cfg.rope_split):
        groups += [(axis, i, n) for i in range(n)]

    def rot(vec, g):
        pos = (g // T, (g % T) // gw, g % gw)
        outv = []
        for p in range(P):
            axis, i, n = groups[p]
            z = complex(vec[2 * p], vec[2 * p + 1]) * cmath.exp(1j * pos[axis] * cfg.rope_base ** (-i / n))
            outv += [z.real, z.imag]
        return outv

    x, w = st["x"][0], st["w"]
    keys = []
    for g in range(x.shape[0]):
        y = [sum(w[r, k] * x[g, k] for k in range(cfg.hidden)) for r in range(cfg.width)]
        c = [float(np.float32(v)) for v in y[: cfg.d_c]]
        kr = [float(np.float32(v)) for v in rot(y[cfg.d_c:], g)]
        keys.append((c, kr))
    for i in range(st["q"].shape[1]):
        g = st["q_token0"] + i
        for h in range(cfg.n_heads):
            qv = st["q"][0, i, h]
            qr = rot(list(qv[cfg.d_nope:]), g)
            scores, vals = [], []
            for c, kr in keys:
                kn = [sum(st["w_uk"][h][n, j] * c[j] for j in range(cfg.d_c)) for n in range(cfg.d_nope)]
                s = sum(qv[n] * kn[n] for n in range(cfg.d_nope)) + sum(qr[p] * kr[p] for p in range(cfg.d_rope))
                scores.append(s / math.sqrt(cfg.d_qk))
                vals.append([sum(st["w_uv"][h][v, j] * c[j] for j in range(cfg.d_c)) for v in range(cfg.d_v)])
            m = max(scores)
            e = [math.exp(s - m) for s in scores]
            z = sum(e)
            want = [sum(e[j] * vals[j][v] for j in range(len(keys))) / z for v in range(cfg.d_v)]
            np.testing.assert_allclose(got[0, i, h], want, rtol=1e-10, atol=1e-12)


def test_dense_mha_oracle_against_torch_sdpa():
    cfg = config("tiny").with_(batch=2)
    split = O.default_rope_split(cfg.d_qk)
    rng = np.random.default_rng(17)
    T, n_h, d_h = cfg.T, cfg.n_heads, cfg.d_qk
    w_k = rng.standard_normal((n_h * d_h, cfg.hidden)) / 8
    w_v = rng.standard_normal((n_h * d_h, cfg.hidden)) / 8
    ring = O.RingModel(cfg.window_frames, T)
    store = np.full((2, cfg.window_frames * T, 2, n_h, d_h), np.nan)
    x = rng.standard_normal((2, 3 * T, cfg.hidden))
    O.mha_cache_write(store, ring, x, w_k, w_v, 0, 3, cfg, split, storage=None)
    q = rng.standard_normal((2, T, n_h, d_h))
    got = O.mha_attend(store, ring, q, 2 * T, cfg, split)
    pos_k = O.token_position(np.arange(3 * T), cfg.grid_h, cfg.grid_w)
    pos_q = O.token_position(2 * T + np.arange(T), cfg.grid_h, cfg.grid_w)
    for h in range(n_h):
        k = O.rope3d((x @ w_k.T)[..., h * d_h:(h + 1) * d_h], pos_k, split, cfg.rope_base)
        v = (x @ w_v.T)[..., h * d_h:(h + 1) * d_h]
        qh = O.rope3d(q[:, :, h], pos_q, split, cfg.rope_base)
        np.testing.assert_allclose(got[:, :, h], _sdpa(qh, k, v, 1 / math.sqrt(d_h)), rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------
# Steps around the path: latent RMS normalisation, the attention block
# --------------------------------------------------------------------------

def test_rms_norm_matches_torch_and_its_invariants():
    rng = np.random.default_rng(31)
    v = rng.standard_normal((7, 192)) * 3.0
    gamma = 1.0 + 0.25 * rng.standard_normal(192)
    got = O.rms_norm(v, gamma, 1e-6)
    want = torch.nn.functional.rms_norm(torch.from_numpy(v), (192,), torch.from_numpy(gamma), 1e-6).numpy()
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-14)
    unit = O.rms_norm(v, np.ones(192), 0.0)
    np.testing.assert_allclose(np.mean(unit * unit, axis=-1), 1.0, rtol=1e-14)     # unit mean square
    np.testing.assert_allclose(O.rms_norm(37.5 * v, gamma, 0.0), O.rms_norm(v, gamma, 0.0), rtol=1e-13)


def test_cache_write_with_latent_norm_normalises_only_c():
    cfg = config("tiny").with_(batch=2)
    rng = np.random.default_rng(32)
    x = rng.standard_normal((2, cfg.T, cfg.hidden))
    w = rng.standard_normal((cfg.width, cfg.hidden)) / math.sqrt(cfg.hidden)
    plain, normed = (O.new_store(2, cfg.window_frames, cfg.T, cfg.width) for _ in range(2))
    r1, r2 = O.RingModel(cfg.window_frames, cfg.T), O.RingModel(cfg.window_frames, cfg.T)
    O.cache_write(plain, r1, x, w, 0, 1, cfg, storage=None)
    O.cache_write(normed, r2, x, w, 0, 1, cfg, storage=None, kv_norm=(np.ones(cfg.d_c), 0.0))
    slots = r1.resident_slots()
    np.testing.assert_array_equal(normed[:, slots, cfg.d_c:], plain[:, slots, cfg.d_c:])  # k^R untouched
    c = normed[:, slots, :cfg.d_c]
    np.testing.assert_allclose(np.mean(c * c, axis=-1), 1.0, rtol=1e-13)
    # direction kept: the normalised row is a positive multiple of the plain one
    ratio = c / plain[:, slots, :cfg.d_c]
    np.testing.assert_allclose(ratio, ratio[..., :1] * np.ones_like(ratio), rtol=1e-12)
    assert (ratio > 0).all()


def _qnorm_case(seed):
    cfg = config("tiny").with_(batch=2)
    rng = np.random.default_rng(seed)
    store = O.round_storage(rng.standard_normal((2, cfg.window_frames * cfg.T, cfg.width)), "f32")
    ring = O.RingModel(cfg.window_frames, cfg.T)
    ring.write(0, 3)
    w_uk = rng.standard_normal((cfg.n_heads, cfg.d_nope, cfg.d_c)) / math.sqrt(cfg.d_c)
    w_uv = rng.standard_normal((cfg.n_heads, cfg.d_v, cfg.d_c)) / math.sqrt(cfg.d_c)
    # rows of very different sizes, so that the norm changes the attention
    q = rng.standard_normal((2, 5, cfg.n_heads, cfg.d_qk)) * np.exp(rng.standard_normal((2, 5, cfg.n_heads, 1)))
    return cfg, rng, store, ring, w_uk, w_uv, q


def test_query_norm_is_identity_on_rows_of_unit_rms():
    """gamma = 1, eps = 0: rows already of mean square 1 over d_nope + d_rope
    come out unchanged, so the attention equals the plain one; rows normalised
    over the content part only, or over all heads, do not (the axis is pinned)."""
    cfg, rng, store, ring, w_uk, w_uv, q = _qnorm_case(41)
    unit = q / np.sqrt(np.mean(q * q, axis=-1, keepdims=True))
    ones = (np.ones(cfg.d_qk), 0.0)
    plain = O.attend(store, ring, unit, 2 * cfg.T, w_uk, w_uv, cfg)
    np.testing.assert_allclose(O.attend(store, ring, unit, 2 * cfg.T, w_uk, w_uv, cfg, q_norm=ones), plain,
                               rtol=1e-12, atol=1e-13)
    for other in (q / np.sqrt(np.mean(q[..., :cfg.d_nope] ** 2, axis=-1, keepdims=True)),
                  q / np.sqrt(np.mean(q * q, axis=(-2, -1), keepdims=True))):
        a = O.attend(store, ring, other, 2 * cfg.T, w_uk, w_uv, cfg, q_norm=ones)
        b = O.attend(store, ring, other, 2 * cfg.T, w_uk, w_uv, cfg)
        assert np.abs(a - b).max() > 1e-3


def test_query_norm_removes_each_rows_scale():
    """eps = 0: multiplying each (token, head) row by its own positive factor
    changes nothing; without the norm it does."""
    cfg, rng, store, ring, w_uk, w_uv, q = _qnorm_case(42)
    gamma = 1.0 + 0.3 * rng.standard_normal(cfg.d_qk)
    f = np.exp(2.0 * rng.standard_normal(q.shape[:-1] + (1,)))
    a = O.attend(store, ring, q, 2 * cfg.T, w_uk, w_uv, cfg, q_norm=(gamma, 0.0))
    b = O.attend(store, ring, f * q, 2 * cfg.T, w_uk, w_uv, cfg, q_norm=(gamma, 0.0))
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)
    assert np.abs(O.attend(store, ring, f * q, 2 * cfg.T, w_uk, w_uv, cfg) - a).max() > 1e-3


def test_query_norm_acts_on_the_unrotated_query():
    """The gain meets q^R before its rotation: the normalised attention is the
    plain attention of torch's rms_norm(q, gamma, eps).  The gain differs
    inside every rotary pair, where scaling and rotating do not commute, so an
    oracle that applied it after the rotation would fail this."""
    cfg, rng, store, ring, w_uk, w_uv, q = _qnorm_case(43)
    gamma = 1.0 + 0.5 * rng.standard_normal(cfg.d_qk)
    assert np.abs(gamma[cfg.d_nope::2] - gamma[cfg.d_nope + 1::2]).min() > 1e-3
    eps = 1e-3
    pre = torch.nn.functional.rms_norm(torch.from_numpy(q), (cfg.d_qk,), torch.from_numpy(gamma), eps).numpy()
    got = O.attend(store, ring, q, 2 * cfg.T, w_uk, w_uv, cfg, q_norm=(gamma, eps))
    np.testing.assert_allclose(got, O.attend(store, ring, pre, 2 * cfg.T, w_uk, w_uv, cfg), rtol=1e-11, atol=1e-13)


def test_attention_block_with_identity_projections_is_the_attention():
    """hidden = n_h * d_qk = n_h * d_v and identity W_q, W_O: the block is the
    per-head attention of x read as queries, the heads concatenated."""
    cfg = config("tiny").with_(hidden=2 * 32)
    assert cfg.n_heads * cfg.d_qk == cfg.hidden == cfg.n_heads * cfg.d_v
    rng = np.random.default_rng(33)
    store = O.round_storage(rng.standard_normal((1, cfg.window_frames * cfg.T, cfg.width)), "f32")
    ring = O.RingModel(cfg.window_frames, cfg.T)
    ring.write(0, 3)
    x = rng.standard_normal((1, 5, cfg.hidden))
    w_uk = rng.standard_normal((cfg.n_heads, cfg.d_nope, cfg.d_c))
    w_uv = rng.standard_normal((cfg.n_heads, cfg.d_v, cfg.d_c))
    eye = np.eye(cfg.hidden)
    got = O.attend_block(store, ring, x, 40, eye, w_uk, w_uv, eye, cfg)
    want = O.attend(store, ring, x.reshape(1, 5, cfg.n_heads, cfg.d_qk), 40, w_uk, w_uv, cfg)
    np.testing.assert_allclose(got, want.reshape(1, 5, cfg.hidden), rtol=1e-13, atol=1e-13)


def test_weight_level_folds_give_the_same_block():
    """The folds the library applies at the weight level -- W^K_up folded into
    the query projection (q_lat,h = (W_uk,h^T W^nope_q,h) x) and W^V_up into
    W^O (out = sum_h (W^O_h W_uv,h) o_lat,h) -- compute the explicit block."""
    cfg = config("tiny")
    rng = np.random.default_rng(34)
    store = O.round_storage(rng.standard_normal((1, cfg.window_frames * cfg.T, cfg.width)), "f32")
    ring = O.RingModel(cfg.window_frames, cfg.T)
    ring.write(0, 3)
    n_h, dq, dn, dv, dc = cfg.n_heads, cfg.d_qk, cfg.d_nope, cfg.d_v, cfg.d_c
    x = rng.standard_normal((1, 6, cfg.hidden))
    w_q = rng.standard_normal((n_h * dq, cfg.hidden))
    w_o = rng.standard_normal((cfg.hidden, n_h * dv))
    w_uk = rng.standard_normal((n_h, dn, dc))
    w_uv = rng.standard_normal((n_h, dv, dc))
    want = O.attend_block(store, ring, x, 33, w_q, w_uk, w_uv, w_o, cfg)
    # folded weights: per head [W_uk,h^T W^nope_q,h ; W^R_q,h] and W^O_h W_uv,h
    wq = w_q.reshape(n_h, dq, cfg.hidden)
    w_qf = np.concatenate([np.einsum("hni,hnk->hik", w_uk, wq[:, :dn]), wq[:, dn:]], axis=1)
    w_fo = np.einsum("chv,hvi->chi", w_o.reshape(cfg.hidden, n_h, dv), w_uv)
    # absorbed attention with the folded weights, written out directly
    slots = ring.resident_slots()
    C, KR = store[0, slots, :dc], store[0, slots, dc:]
    pos = O.token_position(33 + np.arange(6), cfg.grid_h, cfg.grid_w)
    got = np.zeros((6, cfg.hidden))
    for h in range(n_h):
        qh = x[0] @ w_qf[h].T                                  # [6, d_c + d_rope]
        qr = O.rope3d(qh[:, dc:], pos, cfg.rope_split, cfg.rope_base)
        s = (qh[:, :dc] @ C.T + qr @ KR.T) / math.sqrt(dq)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        got += (p @ C) @ w_fo[:, h, :].T
    np.testing.assert_allclose(got, want[0], rtol=1e-11, atol=1e-11)
