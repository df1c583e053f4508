"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded inputs.  Small and mid sizes compare every output element; the
Wan-sized window compares sampled query rows at full size.

Bars: bf16 inputs with fp32 accumulation -> max|err| <= 1e-2 max|ref| and
sum|err| <= 2e-3 sum|ref| (for both 2-byte ring types; a bf16 ring, whose
attention runs on split operands, is held to sum|err| <= 1.5e-3 sum|ref|);
fp32 path -> 1e-5 / 1e-6; cache placement and the window's slot map are
bit-exact.
"""

import math

import numpy as np
import pytest
import torch

from oracle import mla as O
from synthetic import config, chunk_q, chunk_x
from tests.parity_util import (BF16_RING_MEAN_REL, NAN_BITS, DenseRun, LatentRun, assert_parity, dev,
                               nan_fill_, parity_stats, sample_rows)

TORCH_T = {"bf16": torch.bfloat16, "f16": torch.float16}
SIG_BITS = {"bf16": 8, "f16": 11}

pytestmark = pytest.mark.gpu

WAN_HEADS = dict(hidden=1536, n_heads=12, d_nope=96, d_rope=32, d_v=128, d_c=192)


def mid_cfg(**kw):
    base = dict(hidden=256, n_heads=4, d_nope=32, d_rope=32, d_v=64, d_c=64, grid_h=6, grid_w=10,
                window_frames=5, batch=2, rope_split=None, dtype="bf16")
    base.update(kw)
    return config("wan_layer").with_(**base)


def wan_small(**kw):
    base = dict(WAN_HEADS, grid_h=5, grid_w=13, window_frames=6, batch=2, rope_split=None,
                dtype="bf16")
    base.update(kw)
    return config("wan_layer").with_(**base)


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.manual_seed(0)


def _ring_bits(run):
    return run.gpu.ring().view(torch.int16).cpu().numpy()


def _oracle_bits(store, cache_dtype):
    t = torch.from_numpy(store).to(TORCH_T[cache_dtype])
    return t.view(torch.int16).numpy()


def _onehot_x(cfg, n_frames, seed):
    """Rows 2^e * onehot(k) with distinct (k, e) per token: every product of
    the cache-write GEMM is exact, so the stored rows are known exactly."""
    rng = np.random.default_rng(seed)
    n = n_frames * cfg.T
    x = np.zeros((cfg.batch, n, cfg.hidden))
    for b in range(cfg.batch):
        ks = rng.integers(0, cfg.hidden, n)
        es = rng.integers(-4, 5, n)
        x[b, np.arange(n), ks] = 2.0 ** es
    return torch.from_numpy(x).to(torch.bfloat16)


# --------------------------------------------------------------------------
# cache write
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cache_dtype", ["f16", "bf16"])
def test_cache_write_exact_placement_and_untouched_slots(cache_dtype):
    cfg = mid_cfg(cache_dtype=cache_dtype)
    run = LatentRun(cfg, poison=True)
    run.w["w_dkr"][cfg.d_c:] = 0          # k^R rows zero: every stored value is exact
    run.wd["w_dkr"] = dev(run.w["w_dkr"])
    run.write(7, 2, x=_onehot_x(cfg, 2, 1))   # frames 7, 8 -> ring frames 2, 3
    torch.cuda.synchronize()
    got = _ring_bits(run)
    want = _oracle_bits(run.store, cache_dtype)
    written = np.zeros(cfg.window_frames * cfg.T, bool)
    written[2 * cfg.T:4 * cfg.T] = True
    np.testing.assert_array_equal(got[:, written], want[:, written])
    assert (got[:, ~written] == NAN_BITS[cache_dtype]).all(), "kernel wrote outside the chunk's slots"


@pytest.mark.parametrize("cache_dtype", ["f16", "bf16"])
def test_cache_write_values_within_one_ulp(cache_dtype):
    """Stored rows are the oracle's rounded values or a neighbour: the GPU sums
    in fp32, so a value may round the other way when the fp64 sum lies within
    the fp32 summation error of a rounding boundary."""
    cfg = wan_small(batch=1, cache_dtype=cache_dtype)
    run = LatentRun(cfg)
    x = run.write(0, 4)
    torch.cuda.synchronize()
    got = run.gpu.ring().double().cpu().numpy()
    ref = run.store
    written = np.zeros(cfg.window_frames * cfg.T, bool)
    written[:4 * cfg.T] = True
    g, r = got[:, written], ref[:, written]
    ulp = np.ldexp(1.0, np.frexp(np.abs(r))[1] - SIG_BITS[cache_dtype])
    # fp32 accumulation bound of the 1536-term products (rotation adds a few ulp of fp32)
    mag = np.abs(x.double().numpy()[0]) @ np.abs(run.w["w_dkr"].double().numpy()).T
    acc = 1536 * 2.0 ** -24 * np.concatenate([mag[:, :cfg.d_c], np.repeat(
        mag[:, cfg.d_c:].reshape(-1, cfg.d_rope // 2, 2).sum(-1), 2, axis=-1)], -1)
    assert (np.abs(g - r)[0] <= ulp[0] + acc).all()
    assert np.mean(g == r) > 0.97


@pytest.mark.parametrize("batch", [1, 2])
def test_cache_write_wan_chunk_values_and_placement(batch):
    """A 3-frame Wan chunk (4680 tokens per sequence) into the 21-frame ring:
    at B = 1 each 32-token tile's 7 column tiles are split over two
    workgroups of 4 (the 8th tile past the row is loaded but never written),
    at B = 2 one workgroup of 7 takes them all.  Stored rows are the oracle's
    rounded values or a neighbour (fp32 summation), and no slot outside the
    chunk is touched."""
    cfg = config("wan_window").with_(batch=batch)
    run = LatentRun(cfg, poison=True)
    f0 = cfg.chunk_frame0
    x = run.write(f0, cfg.chunk_frames)
    torch.cuda.synchronize()
    got = run.gpu.ring().double().cpu().numpy()
    ref = run.store
    slot0 = (f0 % cfg.window_frames) * cfg.T
    written = np.zeros(cfg.window_frames * cfg.T, bool)
    written[slot0:slot0 + cfg.chunk_frames * cfg.T] = True
    assert np.isnan(got[:, ~written]).all(), "kernel wrote outside the chunk's slots"
    g, r = got[:, written], ref[:, written]
    ulp = np.ldexp(1.0, np.frexp(np.abs(r))[1] - SIG_BITS[cfg.cache_dtype])
    for b in range(batch):
        mag = np.abs(x.double().numpy()[b]) @ np.abs(run.w["w_dkr"].double().numpy()).T
        acc = cfg.hidden * 2.0 ** -24 * np.concatenate([mag[:, :cfg.d_c], np.repeat(
            mag[:, cfg.d_c:].reshape(-1, cfg.d_rope // 2, 2).sum(-1), 2, axis=-1)], -1)
        assert (np.abs(g[b] - r[b]) <= ulp[b] + acc).all(), f"sequence {b}"
    assert np.mean(g == r) > 0.97


@pytest.mark.parametrize("cache_dtype", ["f16", "bf16"])
def test_rollout_ring_bit_exact_through_wraps(cache_dtype):
    """A 12-chunk rollout through a 5-frame window (the ring wraps four times):
    after every chunk the resident rows match the oracle bit for bit."""
    cfg = mid_cfg(batch=1, cache_dtype=cache_dtype)
    run = LatentRun(cfg, poison=True)
    run.w["w_dkr"][cfg.d_c:] = 0
    run.wd["w_dkr"] = dev(run.w["w_dkr"])
    for k in range(12):
        n_ev = max(0, run.ring.n_resident + 2 - cfg.window_frames)
        run.evict(n_ev)
        run.write(2 * k, 2, x=_onehot_x(cfg, 2, 100 + k))
        torch.cuda.synchronize()
        info = run.gpu.info()
        assert (info["oldest_frame"], info["newest_frame"]) == (run.ring.oldest, run.ring.newest)
        slots = run.ring.resident_slots()
        np.testing.assert_array_equal(_ring_bits(run)[:, slots],
                                      _oracle_bits(run.store, cache_dtype)[:, slots])
        for f in (run.ring.oldest, run.ring.newest):
            assert run.gpu.slot(f, 7) == run.ring.slot(f, 7)


# --------------------------------------------------------------------------
# attention, every element
# --------------------------------------------------------------------------

def test_attend_tiny_fp32_path():
    cfg = config("tiny")
    run = LatentRun(cfg)
    run.write(0, 2)
    run.write(2, 1)
    q = run.query(cfg.T)
    got, ref, _ = run.attend(q, 2 * cfg.T)
    assert_parity(got, ref, "f32", "tiny fp32")


@pytest.mark.parametrize("key_splits", [0, 1, 3])
def test_attend_mid_ragged_with_wrap(key_splits):
    cfg = mid_cfg()
    run = LatentRun(cfg)
    run.write(0, 4)
    run.evict(2)
    run.write(4, 2)       # frames 2..5 resident, ring wrapped (frame 5 -> slot 0)
    run.evict(1)
    run.write(6, 2)       # frames 3..7, Lk = 300 keys: 4 full key tiles + a ragged one
    q = run.query(2 * cfg.T)
    got, ref, _ = run.attend(q, 6 * cfg.T, key_splits=key_splits)
    assert_parity(got, ref, "bf16", f"mid splits={key_splits}")


# Lq * n_heads = 12 rows: one-wave blocks on 32-key tiles; 80 rows: four-wave
# blocks with a wave of padding; 132 rows: eight-wave blocks with three padding
# waves.  300 keys leave a ragged last tile; forced splits put several blocks
# on each row group.
@pytest.mark.parametrize("Lq,key_splits", [(3, 0), (3, 4), (20, 0), (20, 2), (33, 0), (33, 3)])
def test_attend_narrow_blocks_ragged_with_wrap(Lq, key_splits):
    cfg = mid_cfg()
    run = LatentRun(cfg)
    run.write(0, 4)
    run.evict(2)
    run.write(4, 2)
    run.evict(1)
    run.write(6, 2)       # frames 3..7 resident through a ring wrap, Lk = 300
    q = run.query(Lq)
    got, ref, _ = run.attend(q, 8 * cfg.T - Lq, key_splits=key_splits)
    assert_parity(got, ref, "bf16", f"narrow blocks Lq={Lq} splits={key_splits}")


@pytest.mark.parametrize("cache_dtype", ["f16", "bf16", "e4m3"])
@pytest.mark.parametrize("window_frames,n_frames", [(3, 3), (40, 37)])
def test_ring_shorter_than_a_key_tile(cache_dtype, window_frames, n_frames):
    """One token per frame: a 3-row ring is shorter than every key tile, so a
    tile's keys past the window wrap around it more than once (their scores
    are masked); a 40-row ring is shorter than the 64-key tiles of the chunk
    shape.  Every element, 1 and 130 queries."""
    cfg = mid_cfg(grid_h=1, grid_w=1, window_frames=window_frames, batch=3, cache_dtype=cache_dtype)
    run = LatentRun(cfg)
    run.write(0, n_frames)
    for Lq in (1, 130):
        q = run.query(Lq, chunk=Lq)
        got, ref, _ = run.attend(q, n_frames - 1)
        assert_parity(got, ref, "bf16", f"{window_frames}-row ring {cache_dtype} Lq={Lq}",
                      mean_lim=ring_lim(cfg))


@pytest.mark.parametrize("d_c", [64, 128, 192])
def test_attend_wan_heads_latent_widths(d_c):
    cfg = wan_small(d_c=d_c)
    run = LatentRun(cfg)
    run.write(0, 4)
    run.evict(1)
    run.write(4, 2)
    q = run.query(2 * cfg.T)
    got, ref, _ = run.attend(q, 4 * cfg.T)
    assert_parity(got, ref, "bf16", f"wan heads d_c={d_c}")


def ring_lim(cfg):
    """Mean-error limit of a ring type: the bf16 ring's gate has a 25% margin."""
    return BF16_RING_MEAN_REL if cfg.cache_dtype == "bf16" else None


@pytest.mark.parametrize("cache_dtype", ["f16", "bf16"])
@pytest.mark.parametrize("Lq", [1, 4, 8])
def test_attend_small_queries_cache_bound_shapes(Lq, cache_dtype):
    cfg = config("wan_layer").with_(window_frames=3, batch=3, cache_dtype=cache_dtype)
    run = LatentRun(cfg)
    run.write(0, 3)       # Lk = 4680
    q = run.query(Lq)
    got, ref, _ = run.attend(q, 3 * cfg.T - Lq)
    assert_parity(got, ref, "bf16", f"small query Lq={Lq} {cache_dtype}", mean_lim=ring_lim(cfg))


# Few-token prologue and per-row epilogue at every latent width; batch 3
# puts Lq = 8 (288 rows) on the lean epilogue and Lq = 1 on the wide one.
@pytest.mark.parametrize("d_c", [64, 128])
@pytest.mark.parametrize("Lq", [1, 8])
def test_attend_small_queries_latent_widths(Lq, d_c):
    cfg = config("wan_layer").with_(window_frames=3, batch=3, d_c=d_c, cache_dtype="f16")
    run = LatentRun(cfg)
    run.write(0, 3)
    q = run.query(Lq)
    got, ref, _ = run.attend(q, 3 * cfg.T - Lq)
    assert_parity(got, ref, "bf16", f"small query Lq={Lq} d_c={d_c}")


@pytest.mark.parametrize("cache_dtype,path", [("f16", "absorbed"), ("f16", "expand"), ("bf16", "absorbed"),
                                              ("bf16", "expand"), ("e4m3", "absorbed"), ("e4m3", "expand")])
def test_degenerate_softmax_closed_forms(cache_dtype, path):
    """Two windows whose attention has a closed form, 300 keys through a wrap:
    zero queries weight every key equally, so each head's output is W^V_up,h
    applied to the mean stored latent; a window of identical rows gives
    W^V_up,h c for any query.  Checked against the closed forms (fp64, from
    the stored values) and the oracle."""
    cfg = mid_cfg(d_nope=96, d_rope=32, d_v=128, d_c=192, cache_dtype=cache_dtype)
    run = LatentRun(cfg, path=path)
    run.write(0, 4)
    run.evict(2)
    run.write(4, 2)
    run.evict(1)
    run.write(6, 2)
    slots = run.ring.resident_slots()
    w_uv = run.w["w_uv"].double().numpy()
    for Lq in (20, 130):
        q = torch.zeros((cfg.batch, Lq, cfg.n_heads, cfg.d_qk), dtype=torch.bfloat16)
        got, ref, _ = run.attend(q, 8 * cfg.T - Lq)
        cbar = run.store[:, slots, :cfg.d_c].mean(axis=1)                 # [B, d_c]
        want = np.einsum("hvc,bc->bhv", w_uv, cbar)[:, None].repeat(Lq, axis=1)
        assert_parity(got, want, "bf16", f"zero queries {cache_dtype} {path} Lq={Lq}", mean_lim=ring_lim(cfg))
        assert_parity(ref, want, "f32", "oracle, zero queries")
    # every resident row equal to one stored row
    row = run.store[:, slots[:1]]
    run.fill(run.ring.oldest, run.ring.newest, np.repeat(row, len(slots), axis=1))
    q = run.query(40)
    got, ref, _ = run.attend(q, 8 * cfg.T - 40)
    want = np.einsum("hvc,bc->bhv", w_uv, row[:, 0, :cfg.d_c])[:, None].repeat(40, axis=1)
    assert_parity(got, want, "bf16", f"identical keys {cache_dtype} {path}", mean_lim=ring_lim(cfg))
    assert_parity(ref, want, "f32", "oracle, identical keys")


def test_nan_poison_determinism_and_split_agreement():
    cfg = wan_small()
    runs = [LatentRun(cfg, poison=p) for p in (False, True)]
    for r in runs:
        r.write(0, 4)
        r.evict(2)
        r.write(4, 2)
    q = runs[0].query(2 * cfg.T)
    outs = []
    for r in runs:
        for _ in range(2):
            outs.append(r.gpu.attend(dev(q), 4 * cfg.T, r.wd["w_uk"], r.wd["w_uv"]).cpu())
    for o in outs[1:]:
        assert torch.equal(o, outs[0]), "results differ between runs or with NaN-filled free slots"
    got, ref, _ = runs[1].attend(q, 4 * cfg.T, key_splits=5)
    assert_parity(got, ref, "bf16", "5 key ranges")
    mx, mean = parity_stats(got, outs[0].numpy())
    assert mx < 2e-3 and mean < 5e-4


def test_frame_shift_changes_nothing_beyond_rounding():
    cfg = wan_small(batch=1)
    outs = []
    for off in (0, 100):
        run = LatentRun(cfg)
        run.write(off, 3, x=chunk_x(cfg, 3, chunk=0))
        q = run.query(cfg.T)
        got, ref, _ = run.attend(q, (off + 2) * cfg.T)
        assert_parity(got, ref, "bf16", f"frame offset {off}")
        outs.append(got)
    mx, mean = parity_stats(outs[1], outs[0])
    assert mx < 1e-2 and mean < 4e-3


# --------------------------------------------------------------------------
# attention at Wan sizes, sampled rows
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cache_dtype,path", [("f16", "absorbed"), ("f16", "expand"), ("bf16", "absorbed"),
                                              ("bf16", "auto")])
def test_wan_layer_sampled_rows(cache_dtype, path):
    cfg = config("wan_layer").with_(cache_dtype=cache_dtype)
    run = LatentRun(cfg, path=path)
    run.write(0, cfg.prefill_frames)
    run.write(cfg.chunk_frame0, cfg.chunk_frames)
    q = run.query(cfg.Lq)
    rows = sample_rows(cfg.Lq, 96)
    taken = run.gpu.attend_path(cfg.Lq)
    assert taken == (path if path != "auto" else "expand")
    got, ref, _ = run.attend(q, cfg.chunk_frame0 * cfg.T, rows=rows)
    assert_parity(got, ref, "bf16", f"wan layer (6+3 frames) sampled {cache_dtype} {taken}",
                  mean_lim=ring_lim(cfg))


# A bf16 ring's expansion: bf16 products of the stored values, the rebuilt
# keys and values in fp16 like an fp16 ring's, mid sizes through a wrap with
# the shapes of the fp16 expand cases, every element.
@pytest.mark.parametrize("Lq,d_c,n_heads", [(3, 192, 4), (33, 64, 4), (120, 128, 6), (300, 192, 4)])
def test_bf16_ring_expand_mid_ragged_with_wrap(Lq, d_c, n_heads):
    cfg = mid_cfg(d_nope=96, d_rope=32, d_v=128, d_c=d_c, n_heads=n_heads, cache_dtype="bf16")
    run = LatentRun(cfg, path="expand")
    run.write(0, 4)
    run.evict(2)
    run.write(4, 2)
    run.evict(1)
    run.write(6, 2)       # frames 3..7 resident, Lk = 300
    assert run.gpu.attend_path(Lq) == "expand"
    q = run.query(Lq)
    got, ref, _ = run.attend(q, 8 * cfg.T - Lq)
    assert_parity(got, ref, "bf16", f"bf16 ring expand Lq={Lq} d_c={d_c} n_h={n_heads}", mean_lim=ring_lim(cfg))
    mx, mean = parity_stats(got, ref)
    assert mean < 1e-3, mean      # fp16 rebuilt keys and values: an fp16 ring's error, not bf16's


@pytest.mark.parametrize("batch,cache_dtype,path",
                         [(1, "f16", "absorbed"), (2, "f16", "absorbed"), (1, "bf16", "absorbed"),
                          (1, "f16", "expand"), (2, "bf16", "auto"), (1, "bf16", "expand"), (1, "f16", "auto")])
def test_full_window_sampled_rows(batch, cache_dtype, path):
    cfg = config("wan_window").with_(batch=batch, cache_dtype=cache_dtype)
    run = LatentRun(cfg, path=path)
    run.write(0, cfg.prefill_frames)
    run.evict(cfg.evict_frames)
    run.write(cfg.chunk_frame0, cfg.chunk_frames)
    assert run.gpu.info()["n_resident_frames"] == 21
    q = run.query(cfg.Lq)
    rows = sample_rows(cfg.Lq, 48 if batch == 1 else 24)
    got, ref, _ = run.attend(q, cfg.chunk_frame0 * cfg.T, rows=rows)
    assert_parity(got, ref, "bf16", f"21-frame window B={batch} {cache_dtype} {path} sampled",
                  mean_lim=ring_lim(cfg))


# Expand-then-attend on mid sizes, every element: Wan head widths on a small
# frame grid (60 tokens); 300 resident keys through a ring wrap leave ragged
# 32- and 64-key tiles and a ragged last 128-key rebuild block; the query
# counts reach all three attention block shapes (3 -> 32-row blocks, 33 and
# 120 -> 128-row blocks, 200 and 300 -> 256-row blocks with padded rows).
# 6 heads: the rebuild's last head group is partial (4 + 2 heads).
@pytest.mark.parametrize("Lq,d_c,n_heads", [(3, 192, 4), (33, 64, 4), (120, 128, 6), (200, 192, 4),
                                            (300, 64, 4)])
def test_expand_mid_ragged_with_wrap(Lq, d_c, n_heads):
    cfg = mid_cfg(d_nope=96, d_rope=32, d_v=128, d_c=d_c, n_heads=n_heads)
    run = LatentRun(cfg, path="expand")
    run.write(0, 4)
    run.evict(2)
    run.write(4, 2)
    run.evict(1)
    run.write(6, 2)       # frames 3..7 resident, Lk = 300
    assert run.gpu.attend_path(Lq) == "expand"
    q = run.query(Lq)
    got, ref, _ = run.attend(q, 8 * cfg.T - Lq)
    assert_parity(got, ref, "bf16", f"expand Lq={Lq} d_c={d_c} n_h={n_heads}")


@pytest.mark.parametrize("cache_dtype", ["f16", "bf16"])
def test_expand_poisoned_free_slots_and_agreement(cache_dtype):
    """Expand path: NaN in every free ring slot changes nothing (only resident
    keys are rebuilt), repeated calls agree bit for bit, and the two paths agree
    to within their rounding."""
    cfg = wan_small(cache_dtype=cache_dtype)
    runs = [LatentRun(cfg, poison=p, path="expand") for p in (False, True)]
    for r in runs:
        r.write(0, 4)
        r.evict(2)
        r.write(4, 2)
    q = runs[0].query(2 * cfg.T)
    outs = []
    for r in runs:
        for _ in range(2):
            outs.append(r.gpu.attend(dev(q), 4 * cfg.T, r.wd["w_uk"], r.wd["w_uv"]).cpu())
    for o in outs[1:]:
        assert torch.equal(o, outs[0]), "expand results differ between runs or with NaN free slots"
    got, ref, _ = runs[1].attend(q, 4 * cfg.T)
    assert_parity(got, ref, "bf16", f"expand, poisoned {cache_dtype} ring", mean_lim=ring_lim(cfg))
    runs[1].gpu.set_attend_path("absorbed")
    absorbed = runs[1].gpu.attend(dev(q), 4 * cfg.T, runs[1].wd["w_uk"], runs[1].wd["w_uv"]).cpu()
    mx, mean = parity_stats(outs[0].numpy(), absorbed.numpy())
    assert mx < 1e-2 and mean < 2e-3, (mx, mean)


@pytest.mark.parametrize("Lq,path,cache_dtype", [(1, "absorbed", "f16"), (8, "absorbed", "f16"), (1, "expand", "f16"),
                                                (8, "expand", "bf16")])
def test_small_queries_full_window(Lq, path, cache_dtype):
    """Decode-like shapes on the full 21-frame window: each sequence's few rows
    spread over many key ranges (about a hundred partials per row)."""
    cfg = config("wan_window").with_(batch=2, cache_dtype=cache_dtype)
    run = LatentRun(cfg, path=path)
    run.write(0, cfg.prefill_frames)
    run.evict(cfg.evict_frames)
    run.write(cfg.chunk_frame0, cfg.chunk_frames)
    q = run.query(Lq)
    got, ref, _ = run.attend(q, (cfg.chunk_frame0 + cfg.chunk_frames) * cfg.T - Lq)
    assert_parity(got, ref, "bf16", f"21-frame window small query Lq={Lq} {path} {cache_dtype}",
                  mean_lim=ring_lim(cfg))


# --------------------------------------------------------------------------
# dense comparison path
# --------------------------------------------------------------------------

def test_dense_mha_full_small():
    cfg = wan_small()
    run = DenseRun(cfg)
    run.write(0, 4)
    run.evict(1)
    run.write(4, 2)
    q = chunk_q(cfg, 2 * cfg.T, chunk=7)
    got, ref = run.attend(q, 4 * cfg.T)
    assert_parity(got, ref, "bf16", "dense small")


# one-wave blocks (1 row per head), four-wave blocks with padding (40),
# eight-wave blocks with padding waves (129)
@pytest.mark.parametrize("Lq", [1, 40, 129])
def test_dense_mha_small_queries(Lq):
    cfg = wan_small()
    run = DenseRun(cfg)
    run.write(0, 4)
    run.evict(1)
    run.write(4, 2)
    q = chunk_q(cfg, Lq, chunk=5)
    got, ref = run.attend(q, 6 * cfg.T - Lq)
    assert_parity(got, ref, "bf16", f"dense small query Lq={Lq}")


def test_dense_mha_tiny_fp32():
    cfg = config("tiny").with_(batch=2)
    run = DenseRun(cfg)
    run.write(0, 3)
    q = chunk_q(cfg, cfg.T, chunk=3)
    got, ref = run.attend(q, 2 * cfg.T)
    assert_parity(got, ref, "f32", "dense tiny fp32")


def test_dense_mha_window_sampled():
    cfg = config("wan_window")
    run = DenseRun(cfg)
    run.write(0, cfg.prefill_frames)
    run.evict(cfg.evict_frames)
    run.write(cfg.chunk_frame0, cfg.chunk_frames)
    q = chunk_q(cfg, cfg.Lq, chunk=9)
    rows = sample_rows(cfg.Lq, 32)
    got, ref = run.attend(q, cfg.chunk_frame0 * cfg.T, rows=rows)
    assert_parity(got, ref, "bf16", "dense 21-frame window sampled")


def test_dense_mha_ring_wrap():
    """Dense cache through a ring wrap: 6-frame window, frames 2..7 resident
    (frames 6 and 7 in slots 0 and 1), 390 keys (a ragged last 64-key tile)."""
    cfg = wan_small()
    run = DenseRun(cfg)
    run.write(0, 6)
    run.evict(2)
    run.write(6, 2)
    q = chunk_q(cfg, 2 * cfg.T, chunk=11)
    got, ref = run.attend(q, 6 * cfg.T)
    assert_parity(got, ref, "bf16", "dense ring wrap")


# ---------------------------------------------------------------------------
# expand-then-attend: path choice, batches, workspace reuse
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cache_dtype,Lq,first", [("f16", 511, 512), ("f16", 512, 512), ("bf16", 127, 128),
                                                 ("bf16", 128, 128)])
def test_auto_path_threshold_batch3_wrap(cache_dtype, Lq, first):
    """Three sequences through a ring wrap; on automatic an fp16 ring expands
    from 512 queries and a bf16 ring (split-operand absorbed core) from 128,
    both sides of each threshold against the oracle."""
    cfg = mid_cfg(d_nope=96, d_rope=32, d_v=128, d_c=192, n_heads=6, batch=3, cache_dtype=cache_dtype)
    run = LatentRun(cfg)
    run.write(0, 4)
    run.evict(2)
    run.write(4, 2)
    run.evict(1)
    run.write(6, 2)       # frames 3..7 resident through a wrap, Lk = 300
    assert run.gpu.attend_path(Lq) == ("expand" if Lq >= first else "absorbed")
    q = run.query(Lq)
    rows = sample_rows(Lq, 64)
    got, ref, _ = run.attend(q, 8 * cfg.T, rows=rows)
    assert_parity(got, ref, "bf16", f"auto path {cache_dtype} Lq={Lq} B=3", mean_lim=ring_lim(cfg))


def test_expand_workspace_reused_as_window_fills():
    """One workspace, sized once, serves the expand path while the window
    fills, is full, and wraps; every call is checked against the oracle."""
    from rank_latent_kv_absorbed_amd import LatentCache  # noqa: F401
    cfg = wan_small(batch=1)
    run = LatentRun(cfg, path="expand")
    Lq = cfg.T
    ws = None
    frame = 0
    for n_new, n_ev in ((2, 0), (3, 0), (1, 0), (2, 2), (3, 3)):
        run.evict(n_ev)
        run.write(frame, n_new)
        frame += n_new
        need = run.gpu.workspace_bytes(Lq)
        if ws is None:
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        assert need == ws.numel()      # sized for the full window from the start
        q = run.query(Lq, chunk=frame)
        out = run.gpu.attend(dev(q), frame * cfg.T - Lq, run.wd["w_uk"], run.wd["w_uv"], workspace=ws)
        torch.cuda.synchronize()
        ref = O.attend(run.store, run.ring, q.double().numpy(), frame * cfg.T - Lq,
                       run.w["w_uk"].double().numpy(), run.w["w_uv"].double().numpy(), cfg)
        assert_parity(out.cpu().numpy(), ref, "bf16", f"expand, {run.ring.n_resident} frames resident")


def test_expand_reuse_across_attends_and_after_write():
    """Reuse of the rebuilt window: three attends with different queries on
    one window state (one rebuild), then a new chunk is written and the next
    attend must see it; every result against the oracle."""
    cfg = wan_small(batch=2)
    run = LatentRun(cfg, path="expand")
    run.gpu.set_expand_reuse(True)
    run.write(0, 4)
    Lq = cfg.T
    ws = torch.empty(run.gpu.workspace_bytes(Lq), dtype=torch.uint8, device="cuda")
    for step, (frame0, n_new, n_ev) in enumerate(((None, 0, 0), (None, 0, 0), (None, 0, 0),
                                                  (4, 2, 1), (None, 0, 0))):
        if frame0 is not None:
            run.evict(n_ev)
            run.write(frame0, n_new)
        newest = run.ring.newest
        q = run.query(Lq, chunk=50 + step)
        out = run.gpu.attend(dev(q), (newest + 1) * cfg.T - Lq, run.wd["w_uk"], run.wd["w_uv"],
                             workspace=ws)
        torch.cuda.synchronize()
        ref = O.attend(run.store, run.ring, q.double().numpy(), (newest + 1) * cfg.T - Lq,
                       run.w["w_uk"].double().numpy(), run.w["w_uv"].double().numpy(), cfg)
        assert_parity(out.cpu().numpy(), ref, "bf16", f"expand reuse, call {step}")


# ---------------------------------------------------------------------------
# bf16 ring: split operands, every element at a few hundred keys
# ---------------------------------------------------------------------------

# 300 resident keys through a ring wrap (a ragged last tile); the query counts
# reach every core shape of the split-operand core: 12 rows (one 16-row wave),
# 80 (four 32-row waves on 32-key tiles), 132 (four waves on 64-key tiles),
# 1200 (several row groups); forced key splits merge partials.
@pytest.mark.parametrize("Lq,key_splits", [(3, 0), (20, 0), (33, 0), (33, 3), (300, 0)])
def test_bf16_ring_every_element_ragged_with_wrap(Lq, key_splits):
    cfg = mid_cfg(d_nope=96, d_rope=32, d_v=128, d_c=192, cache_dtype="bf16")
    run = LatentRun(cfg)
    run.write(0, 4)
    run.evict(2)
    run.write(4, 2)
    run.evict(1)
    run.write(6, 2)       # frames 3..7 resident through a wrap, Lk = 300
    q = run.query(Lq)
    got, ref, _ = run.attend(q, 8 * cfg.T - Lq, key_splits=key_splits)
    assert_parity(got, ref, "bf16", f"bf16 ring Lq={Lq} splits={key_splits}",
                  mean_lim=BF16_RING_MEAN_REL)


@pytest.mark.parametrize("d_c", [64, 128])
def test_bf16_ring_latent_widths_every_element(d_c):
    cfg = wan_small(d_c=d_c, cache_dtype="bf16")
    run = LatentRun(cfg)
    run.write(0, 4)
    run.evict(1)
    run.write(4, 2)       # 325 keys
    q = run.query(2 * cfg.T)
    got, ref, _ = run.attend(q, 4 * cfg.T)
    assert_parity(got, ref, "bf16", f"bf16 ring d_c={d_c}", mean_lim=BF16_RING_MEAN_REL)


@pytest.mark.parametrize("Lq", [1, 40, 129])
def test_dense_mha_bf16_ring_every_element(Lq):
    cfg = wan_small(cache_dtype="bf16")
    run = DenseRun(cfg)
    run.write(0, 4)
    run.evict(1)
    run.write(4, 2)
    q = chunk_q(cfg, Lq, chunk=5)
    got, ref = run.attend(q, 6 * cfg.T - Lq)
    assert_parity(got, ref, "bf16", f"dense bf16 ring Lq={Lq}", mean_lim=BF16_RING_MEAN_REL)


# ---------------------------------------------------------------------------
# batch sizes of the batch-scaling and rollout workloads (full window, sampled
# rows of every sequence, the first and the last included)
# ---------------------------------------------------------------------------

def _prefill_full_window(run, cfg):
    for f0 in range(0, cfg.prefill_frames, 3):      # 3 frames at a time bounds host memory
        run.write(f0, min(3, cfg.prefill_frames - f0))
    run.evict(cfg.evict_frames)
    run.write(cfg.chunk_frame0, cfg.chunk_frames)


@pytest.mark.parametrize("batch,cache_dtype,path",
                         [(4, "f16", "absorbed"), (4, "f16", "expand"), (8, "f16", "auto"),
                          (8, "bf16", "auto"), (11, "f16", "absorbed"), (11, "f16", "expand")])
def test_batches_full_window_sampled_rows(batch, cache_dtype, path):
    cfg = config("wan_window").with_(batch=batch, cache_dtype=cache_dtype)
    run = LatentRun(cfg, path=path)
    _prefill_full_window(run, cfg)
    q = run.query(cfg.Lq)
    rows = sample_rows(cfg.Lq, 8)
    got, ref, _ = run.attend(q, cfg.chunk_frame0 * cfg.T, rows=rows)
    for b in (0, batch - 1):
        assert_parity(got[b], ref[b], "bf16", f"B={batch} sequence {b} {cache_dtype} {path}",
                      mean_lim=ring_lim(cfg))
    assert_parity(got, ref, "bf16", f"B={batch} {cache_dtype} {run.gpu.attend_path(cfg.Lq)}",
                  mean_lim=ring_lim(cfg))


@pytest.mark.parametrize("path", ["auto", "absorbed"])
def test_batch64_full_window_sampled_sequences(path):
    """64 sequences over the full window (the expanded window alone holds
    6.4e9 elements, past 2^32): random stored rows placed straight into the
    ring (frames 10..30 resident, so it wraps), the whole chunk attended,
    sampled rows of the first, a middle and the last sequence against the
    oracle on those sequences."""
    cfg = config("wan_window").with_(batch=64)
    run = LatentRun(cfg, path=path)
    rng = np.random.default_rng(64)
    rows = O.round_storage(rng.standard_normal((cfg.batch, cfg.window_frames * cfg.T, cfg.width)),
                           cfg.cache_dtype)
    run.fill(10, 30, rows)
    del rows
    q = run.query(cfg.Lq)
    q_token0 = 28 * cfg.T
    out = run.gpu.attend(dev(q), q_token0, run.wd["w_uk"], run.wd["w_uv"])
    torch.cuda.synchronize()
    taken = run.gpu.attend_path(cfg.Lq)
    assert taken == ("expand" if path == "auto" else "absorbed")
    one = cfg.with_(batch=1)
    sel = sample_rows(cfg.Lq, 8)
    for b in (0, 31, 63):
        ref = O.attend(run.store[b:b + 1], run.ring, q[b:b + 1].double().numpy(), q_token0,
                       run.w["w_uk"].double().numpy(), run.w["w_uv"].double().numpy(), one, rows=sel)
        got = out[b:b + 1, torch.from_numpy(sel)].cpu().numpy()
        assert_parity(got, ref, "bf16", f"B=64 sequence {b} {taken}")
    del out


@pytest.mark.parametrize("Lq", [1, 8])
def test_batch11_small_queries_full_window(Lq):
    cfg = config("wan_window").with_(batch=11)
    run = LatentRun(cfg)
    _prefill_full_window(run, cfg)
    q = run.query(Lq)
    got, ref, _ = run.attend(q, (cfg.chunk_frame0 + cfg.chunk_frames) * cfg.T - Lq)
    assert_parity(got, ref, "bf16", f"B=11 small query Lq={Lq}")


# ---------------------------------------------------------------------------
# minute-scale rollout at the Wan shape: 80 chunks of 3 frames through the
# 21-frame window (the ring wraps 11 times)
# ---------------------------------------------------------------------------

ROLLOUT_CHECK = (0, 6, 7, 79)


@pytest.mark.parametrize("d_c", [64, 128, 192])
def test_rollout_80_chunks_ring_bit_exact(d_c):
    """Exact-integer inputs (every cache-write product exact, k^R = 0): after
    every one of the 80 chunks the resident ring rows equal the oracle's bit
    for bit and the window bookkeeping matches; at chunks 0, 6, 7 and 79 the
    chunk's sampled query rows match the oracle's attention."""
    cfg = config("wan_window").with_(d_c=d_c)
    run = LatentRun(cfg, poison=True)
    run.w["w_dkr"][cfg.d_c:] = 0
    run.wd["w_dkr"] = dev(run.w["w_dkr"])
    rows = sample_rows(cfg.Lq, 16)
    for k in range(80):
        res = run.ring.n_resident
        run.evict(max(0, res + 3 - cfg.window_frames))
        run.write(3 * k, 3, x=_onehot_x(cfg, 3, 1000 + k))
        torch.cuda.synchronize()
        info = run.gpu.info()
        assert (info["oldest_frame"], info["newest_frame"]) == (run.ring.oldest, run.ring.newest)
        assert (run.ring.oldest, run.ring.newest) == (max(0, 3 * k + 3 - 21), 3 * k + 2)
        slots = run.ring.resident_slots()
        np.testing.assert_array_equal(_ring_bits(run)[:, slots],
                                      _oracle_bits(run.store, cfg.cache_dtype)[:, slots],
                                      err_msg=f"chunk {k}")
        if k in ROLLOUT_CHECK:
            q = run.query(cfg.Lq, chunk=k)
            got, ref, _ = run.attend(q, 3 * k * cfg.T, rows=rows)
            assert_parity(got, ref, "bf16", f"exact rollout d_c={d_c} chunk {k}")


@pytest.mark.parametrize("d_c,cache_dtype", [(64, "f16"), (128, "f16"), (192, "f16"), (192, "bf16")])
def test_rollout_80_chunks_gaussian_sampled_rows(d_c, cache_dtype):
    """The same rollout on Gaussian inputs (seeded per chunk), attention on the
    library's automatic path, sampled rows checked at chunks 0, 6, 7, 79 (a
    bf16 ring expands into fp16 keys and values there)."""
    cfg = config("wan_window").with_(d_c=d_c, cache_dtype=cache_dtype)
    run = LatentRun(cfg)
    rows = sample_rows(cfg.Lq, 16)
    ws = torch.empty(run.gpu.workspace_bytes(cfg.Lq), dtype=torch.uint8, device="cuda")
    for k in range(80):
        run.evict(max(0, run.ring.n_resident + 3 - cfg.window_frames))
        run.write(3 * k, 3, x=chunk_x(cfg, 3, chunk=k))
        if k in ROLLOUT_CHECK:
            q = run.query(cfg.Lq, chunk=k)
            got, ref, _ = run.attend(q, 3 * k * cfg.T, rows=rows, workspace=ws)
            assert_parity(got, ref, "bf16",
                          f"gaussian rollout d_c={d_c} {cache_dtype} chunk {k} {run.gpu.attend_path(cfg.Lq)}",
                          mean_lim=ring_lim(cfg))


# ---------------------------------------------------------------------------
# sharp attention: the running maximum climbs across the window
# ---------------------------------------------------------------------------

def _climbing_window(cfg, step_log2, seed=0):
    """Stored rows of a full window whose scores climb frame by frame: Gaussian
    [c | k^R], plus, in k^R's slowest-turning frame-axis pair, a value growing
    with the key's frame.  Queries put A in the same pair, so each frame's
    keys score about step_log2 (log2 units) above the previous frame's."""
    rng = np.random.default_rng(seed)
    B, W, T = cfg.batch, cfg.window_frames, cfg.T
    rows = rng.standard_normal((B, W * T, cfg.width))
    pair = cfg.rope_split[0] - 1                    # last (slowest) pair of the frame axis
    col = cfg.d_c + 2 * pair
    A = 8.0
    scale_log2 = math.log2(math.e) / math.sqrt(cfg.d_qk)
    per_frame = step_log2 / (A * scale_log2)
    for f in range(W):
        rows[:, f * T:(f + 1) * T, col] = per_frame * f
        rows[:, f * T:(f + 1) * T, col + 1] = 0.0
    return rows, col - cfg.d_c, A


@pytest.mark.parametrize("cache_dtype,path", [("f16", "absorbed"), ("f16", "expand"), ("bf16", "absorbed"),
                                              ("bf16", "expand"), ("e4m3", "absorbed"), ("e4m3", "expand")])
def test_sharp_attention_running_max_climbs(cache_dtype, path):
    """Every frame's keys score about 9 log2 units above the previous frame's,
    so each row's running maximum jumps by more than the lazy-rescale
    threshold (8) at every frame boundary, 20 times across the 21-frame
    window (resident from the middle of the ring, so the climb also crosses
    the ring's end)."""
    cfg = config("wan_window").with_(cache_dtype=cache_dtype)
    run = LatentRun(cfg, path=path)
    stored, qcol, A = _climbing_window(cfg, 9.0)
    stored = O.round_storage(stored, cache_dtype)
    oldest = 10                                     # frames 10..30: slots wrap after frame 20
    # resident order is oldest first: frame oldest + i holds the i-th climb step
    order = np.concatenate([np.arange(i * cfg.T, (i + 1) * cfg.T) for i in range(cfg.window_frames)])
    run.fill(oldest, oldest + cfg.window_frames - 1, stored[:, order])
    q = run.query(cfg.Lq).double().numpy()
    q[..., cfg.d_nope + qcol] = A
    q[..., cfg.d_nope + qcol + 1] = 0.0
    q = torch.from_numpy(q).to(torch.bfloat16)
    rows = sample_rows(cfg.Lq, 32)
    got, ref, _ = run.attend(q, (oldest + 18) * cfg.T, rows=rows)
    assert_parity(got, ref, "bf16", f"sharp attention {cache_dtype} {path}", mean_lim=ring_lim(cfg))


# ---------------------------------------------------------------------------
# fp16 ring range: values past 65504 are stored as infinity (IEEE rounding)
# ---------------------------------------------------------------------------

def test_f16_ring_overflow_stores_infinity():
    cfg = mid_cfg(cache_dtype="f16", batch=1)
    run = LatentRun(cfg)
    run.w["w_dkr"][cfg.d_c:] = 0
    run.wd["w_dkr"] = dev(run.w["w_dkr"])
    x = _onehot_x(cfg, 1, 5).double() * 2.0 ** 20      # 2^16 .. 2^24 times a weight
    run.write(0, 1, x=x.to(torch.bfloat16))
    torch.cuda.synchronize()
    got = _ring_bits(run)[:, :cfg.T]
    want = _oracle_bits(run.store, "f16")[:, :cfg.T]
    assert np.isinf(run.store[:, :cfg.T]).any(), "fixture must overflow the fp16 range"
    np.testing.assert_array_equal(got, want)
