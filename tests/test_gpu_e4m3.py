"""GPU parity of the one-byte latent ring (OCP E4M3), through the C ABI, against
the fp64 oracle on the same seeded inputs.

The oracle rounds its cache rows to E4M3 as the storage step (round_to_e4m3:
nearest even, saturating at +-448) and then computes in fp64 from those stored
values, so the comparison isolates the path's own arithmetic: fp32 sums and
fp16 query and probability operands, as for an fp16 ring.

  * cache write: stored codes bit-exact on an exact-product fixture (with
    saturation, and free slots untouched), within one E4M3 step plus the fp32
    summation bound on Gaussian inputs, and through an 80-chunk rollout;
  * widening: every finite code passes through the attention unchanged
    (one-key windows, identity value up-projection), in a ring shorter than
    one key tile;
  * attention: every element at mid sizes through ring wraps (all core shapes,
    key splits, d_c in {64, 128, 192}); sampled rows of the Wan layer, of the
    21-frame window at batch 1, 2, 4, 8 and 11, of small queries over the full
    window, and of an 80-chunk rollout for each latent width; the
    expand-then-attend path (rows widened as the per-head keys and values are
    rebuilt) every element at mid sizes and sampled at the Wan shapes.

Bars as for the fp16 ring: max|err| <= 1e-2 max|ref|, sum|err| <= 2e-3 sum|ref|.
"""

import numpy as np
import pytest
import torch

from oracle import mla as O
from synthetic import chunk_x, config
from rank_latent_kv_absorbed_amd.mla import ERR_INVALID_ARG, MlaError
from tests.parity_util import E4M3_NAN, LatentRun, assert_parity, dev, sample_rows

pytestmark = pytest.mark.gpu

E8 = torch.float8_e4m3fn


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def mid_cfg(**kw):
    base = dict(hidden=256, n_heads=4, d_nope=32, d_rope=32, d_v=64, d_c=64, grid_h=6, grid_w=10,
                window_frames=5, batch=2, rope_split=None, dtype="bf16", cache_dtype="e4m3")
    base.update(kw)
    return config("wan_layer").with_(**base)


def ring_codes(run):
    return run.gpu.ring().view(torch.uint8).cpu().numpy()


def oracle_codes(store):
    return torch.from_numpy(np.ascontiguousarray(store)).to(E8).view(torch.uint8).numpy()


def e4m3_step(v):
    """Spacing of E4M3 values at |v|: 2^(e-3) for v in [2^(e-1), 2^e), at least
    the subnormal quantum 2^-9."""
    _, e = np.frexp(np.abs(v))
    return np.maximum(np.ldexp(1.0, e - 4), 2.0 ** -9)


def onehot_x(cfg, n_frames, seed, e_lo=-4, e_hi=5):
    """Rows 2^e * onehot(k): every product of the cache-write GEMM is exact."""
    rng = np.random.default_rng(seed)
    n = n_frames * cfg.T
    x = np.zeros((cfg.batch, n, cfg.hidden))
    for b in range(cfg.batch):
        x[b, np.arange(n), rng.integers(0, cfg.hidden, n)] = 2.0 ** rng.integers(e_lo, e_hi, n)
    return torch.from_numpy(x).to(torch.bfloat16)


def wrapped_window(run):
    run.write(0, 4)
    run.evict(2)
    run.write(4, 2)
    run.evict(1)
    run.write(6, 2)       # frames 3..7 resident through a wrap


# --------------------------------------------------------------------------
# cache write
# --------------------------------------------------------------------------

def test_cache_write_exact_codes_saturation_and_untouched_slots():
    cfg = mid_cfg()
    run = LatentRun(cfg, poison=True)
    run.w["w_dkr"][cfg.d_c:] = 0          # k^R rows zero: every stored value is exact
    run.wd["w_dkr"] = dev(run.w["w_dkr"])
    # exponents up to 2^13: some products pass 448 and saturate
    run.write(7, 2, x=onehot_x(cfg, 2, 5, e_lo=-10, e_hi=14))
    torch.cuda.synchronize()
    got, want = ring_codes(run), oracle_codes(run.store)
    written = np.zeros(cfg.window_frames * cfg.T, bool)
    written[2 * cfg.T:4 * cfg.T] = True
    np.testing.assert_array_equal(got[:, written], want[:, written])
    assert ((got[:, written] & 0x7F) == 0x7E).sum() > 50, "fixture reaches saturation"
    assert ((got[:, written] & 0x7F) < 8).sum() > 50, "fixture reaches subnormals"
    assert (got[:, ~written] == E4M3_NAN).all(), "kernel wrote outside the chunk's slots"


@pytest.mark.parametrize("d_c", [64, 192])
def test_cache_write_values_within_one_step(d_c):
    """Stored values are the oracle's rounded values or a neighbour: the GPU
    sums in fp32, so a value may round the other way when the fp64 sum lies
    within the fp32 summation error of a rounding boundary."""
    cfg = config("wan_layer").with_(d_c=d_c, grid_h=5, grid_w=13, window_frames=6, batch=2,
                                    cache_dtype="e4m3")
    run = LatentRun(cfg)
    x = run.write(0, 4)
    torch.cuda.synchronize()
    got = run.gpu.ring().cpu().double().numpy()[:, :4 * cfg.T]
    ref = run.store[:, :4 * cfg.T]
    for b in range(cfg.batch):
        mag = np.abs(x.double().numpy()[b]) @ np.abs(run.w["w_dkr"].double().numpy()).T
        acc = cfg.hidden * 2.0 ** -24 * np.concatenate([mag[:, :cfg.d_c], np.repeat(
            mag[:, cfg.d_c:].reshape(-1, cfg.d_rope // 2, 2).sum(-1), 2, axis=-1)], -1)
        assert (np.abs(got[b] - ref[b]) <= e4m3_step(ref[b]) + acc).all(), f"sequence {b}"
    assert np.mean(got == ref) > 0.999


def test_rollout_80_chunks_codes_bit_exact():
    """Exact-product inputs through the 21-frame Wan window for 80 chunks: after
    every chunk the resident codes equal the oracle's; sampled attention rows
    at chunks 0, 7 and 79."""
    cfg = config("wan_window").with_(cache_dtype="e4m3")
    run = LatentRun(cfg, poison=True)
    run.w["w_dkr"][cfg.d_c:] = 0
    run.wd["w_dkr"] = dev(run.w["w_dkr"])
    rows = sample_rows(cfg.Lq, 16)
    for k in range(80):
        run.evict(max(0, run.ring.n_resident + 3 - cfg.window_frames))
        run.write(3 * k, 3, x=onehot_x(cfg, 3, 2000 + k))
        torch.cuda.synchronize()
        slots = run.ring.resident_slots()
        np.testing.assert_array_equal(ring_codes(run)[:, slots], oracle_codes(run.store)[:, slots],
                                      err_msg=f"chunk {k}")
        if k in (0, 7, 79):
            q = run.query(cfg.Lq, chunk=k)
            got, ref, _ = run.attend(q, 3 * k * cfg.T, rows=rows)
            assert_parity(got, ref, "bf16", f"e4m3 exact rollout chunk {k}")


# --------------------------------------------------------------------------
# widening inside the attention
# --------------------------------------------------------------------------

def test_every_code_widens_exactly_in_a_tiny_ring():
    """Each of 4 sequences holds one key whose 64 latent values are 64 of the
    254 finite codes (the two NaN codes replaced by zeros); with one key the
    softmax weight is exactly 1, and with W^V_up = I the output is the stored
    row itself.  The ring (2 rows) is shorter than a key tile, so the tile's
    other keys wrap past it more than once."""
    cfg = config("wan_layer").with_(hidden=64, n_heads=2, d_nope=32, d_rope=32, d_v=64, d_c=64,
                                    grid_h=1, grid_w=1, window_frames=2, batch=4, rope_split=None,
                                    cache_dtype="e4m3")
    run = LatentRun(cfg)
    eye = torch.eye(64, dtype=torch.bfloat16)
    run.w["w_uv"] = torch.stack([eye, eye])
    run.wd["w_uv"] = dev(run.w["w_uv"])
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0
    vals = torch.from_numpy(codes).view(E8).double().numpy().reshape(4, 1, 64)
    kr = np.random.default_rng(3).standard_normal((4, 1, 32))
    rows = np.concatenate([vals, O.round_to_e4m3(kr)], axis=-1)
    run.fill(5, 5, rows)
    q = run.query(1)
    got, ref, _ = run.attend(q, 5)
    want = np.broadcast_to(vals.reshape(4, 1, 1, 64), got.shape)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(ref, want)


# --------------------------------------------------------------------------
# attention, every element
# --------------------------------------------------------------------------

# 300 resident keys through a wrap (ragged 32- and 64-key tiles); query counts
# reach every core shape: 3 (16-row waves), 8 and 20 (one 32-row wave), 33
# (four-wave blocks), 130 and 300 (the eight-wave chunk blocks).
@pytest.mark.parametrize("d_c", [64, 128, 192])
@pytest.mark.parametrize("Lq", [3, 33, 130, 300])
def test_expand_every_element_ragged_with_wrap(d_c, Lq):
    cfg = mid_cfg(d_nope=96, d_v=128, d_c=d_c)
    run = LatentRun(cfg, path="expand")
    wrapped_window(run)
    q = run.query(Lq)
    got, ref, _ = run.attend(q, 8 * cfg.T - Lq)
    assert_parity(got, ref, "bf16", f"e4m3 expand d_c={d_c} Lq={Lq}")


@pytest.mark.parametrize("d_c", [64, 128, 192])
@pytest.mark.parametrize("Lq,key_splits", [(3, 0), (8, 0), (20, 2), (33, 3), (130, 0), (300, 0)])
def test_attend_every_element_ragged_with_wrap(d_c, Lq, key_splits):
    cfg = mid_cfg(d_nope=96, d_v=128, d_c=d_c)
    run = LatentRun(cfg)
    wrapped_window(run)
    q = run.query(Lq)
    got, ref, _ = run.attend(q, 8 * cfg.T - Lq, key_splits=key_splits)
    assert_parity(got, ref, "bf16", f"e4m3 d_c={d_c} Lq={Lq} splits={key_splits}")


def test_attend_tiny_bf16_inputs():
    """The tiny head shape (4x4 grid, 2 cached frames + a 1-frame chunk) with
    bf16 inputs and the one-byte ring, every element."""
    cfg = config("tiny").with_(dtype="bf16", cache_dtype="e4m3", hidden=64, d_nope=32, d_rope=32,
                               d_v=64, d_c=64, rope_split=None)
    run = LatentRun(cfg)
    run.write(0, 3)
    q = run.query(cfg.T)
    got, ref, _ = run.attend(q, 2 * cfg.T)
    assert_parity(got, ref, "bf16", "e4m3 tiny")


# --------------------------------------------------------------------------
# Wan shapes, sampled rows
# --------------------------------------------------------------------------

@pytest.mark.parametrize("path", ["absorbed", "auto"])
def test_wan_layer_sampled_rows(path):
    cfg = config("wan_layer").with_(cache_dtype="e4m3")
    run = LatentRun(cfg, path=path)
    run.write(0, cfg.prefill_frames)
    run.write(cfg.chunk_frame0, cfg.chunk_frames)
    assert run.gpu.attend_path(cfg.Lq) == ("absorbed" if path == "absorbed" else "expand")
    q = run.query(cfg.Lq)
    rows = sample_rows(cfg.Lq, 64)
    got, ref, _ = run.attend(q, cfg.chunk_frame0 * cfg.T, rows=rows)
    assert_parity(got, ref, "bf16", f"e4m3 wan layer sampled {path}")


def _full_window(run, cfg):
    for f0 in range(0, cfg.prefill_frames, 3):
        run.write(f0, min(3, cfg.prefill_frames - f0))
    run.evict(cfg.evict_frames)
    run.write(cfg.chunk_frame0, cfg.chunk_frames)
    assert run.gpu.info()["n_resident_frames"] == 21


@pytest.mark.parametrize("batch,path", [(1, "auto"), (2, "auto"), (4, "auto"), (8, "auto"), (11, "auto"),
                                        (1, "absorbed"), (4, "absorbed")])
def test_full_window_sampled_rows(batch, path):
    cfg = config("wan_window").with_(batch=batch, cache_dtype="e4m3")
    run = LatentRun(cfg, path=path)
    _full_window(run, cfg)
    q = run.query(cfg.Lq)
    rows = sample_rows(cfg.Lq, 32 if batch <= 2 else 8)
    got, ref, _ = run.attend(q, cfg.chunk_frame0 * cfg.T, rows=rows)
    for b in (0, batch - 1):
        assert_parity(got[b], ref[b], "bf16", f"e4m3 B={batch} sequence {b} {path}")
    assert_parity(got, ref, "bf16", f"e4m3 21-frame window B={batch} {run.gpu.attend_path(cfg.Lq)}")


@pytest.mark.parametrize("d_c,Lq,path", [(64, 1, "auto"), (128, 1, "auto"), (192, 1, "auto"),
                                         (64, 8, "auto"), (128, 8, "auto"), (192, 8, "auto"),
                                         (192, 1, "expand")])
def test_small_queries_full_window_batch11(d_c, Lq, path):
    cfg = config("wan_window").with_(batch=11, d_c=d_c, cache_dtype="e4m3")
    run = LatentRun(cfg, path=path)
    _full_window(run, cfg)
    q = run.query(Lq)
    got, ref, _ = run.attend(q, (cfg.chunk_frame0 + cfg.chunk_frames) * cfg.T - Lq)
    assert_parity(got, ref, "bf16", f"e4m3 B=11 d_c={d_c} small query Lq={Lq} {path}")


@pytest.mark.parametrize("d_c", [64, 128, 192])
def test_rollout_80_chunks_gaussian_sampled_rows(d_c):
    cfg = config("wan_window").with_(d_c=d_c, cache_dtype="e4m3")
    run = LatentRun(cfg)
    rows = sample_rows(cfg.Lq, 16)
    ws = torch.empty(run.gpu.workspace_bytes(cfg.Lq), dtype=torch.uint8, device="cuda")
    for k in range(80):
        run.evict(max(0, run.ring.n_resident + 3 - cfg.window_frames))
        run.write(3 * k, 3, x=chunk_x(cfg, 3, chunk=k))
        if k in (0, 6, 7, 79):
            q = run.query(cfg.Lq, chunk=k)
            got, ref, _ = run.attend(q, 3 * k * cfg.T, rows=rows, workspace=ws)
            assert_parity(got, ref, "bf16", f"e4m3 gaussian rollout d_c={d_c} chunk {k}")


# --------------------------------------------------------------------------
# what the one-byte ring refuses
# --------------------------------------------------------------------------

def test_path_choice_and_no_dense_cache():
    from rank_latent_kv_absorbed_amd import DenseCache
    cfg = config("wan_layer").with_(cache_dtype="e4m3")
    run = LatentRun(cfg)
    assert run.gpu.attend_path(4680) == "expand" and run.gpu.attend_path(8) == "absorbed"
    run.gpu.set_attend_path("expand")
    assert run.gpu.attend_path(8) == "expand"
    with pytest.raises(MlaError) as e:
        DenseCache(cfg)
    assert e.value.status == ERR_INVALID_ARG
