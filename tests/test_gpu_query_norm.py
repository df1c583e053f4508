"""GPU parity of the query-side RMS norm (mla_cache_set_query_norm) against
the fp64 oracle on the same seeded inputs: each head's query row
[q^nope | q^R] is normalised over its d_nope + d_rope values with one gain
for every head, before its rotation and the fold of W^K_up.

The query rows are drawn with very different sizes (a log-normal factor per
(token, head) row), so that the norm changes the attention.  Covered: the
few-token prologue (fp32 arithmetic) and the chunk prologue (the gained query
as two bf16 parts on the matrix units) of the absorbed path, the per-head
prologue of the expand path, every ring type, every element on mid sizes
through a ring wrap, sampled rows over the full 21-frame window, single-token
queries at the full window, the norm switched off again, and the attention
block's refusal while it is set.

Bars as in the other parity tests: max|err| <= 1e-2 max|ref| and
sum|err| <= 2e-3 sum|ref| (1.5e-3 for a bf16 ring).
"""

import numpy as np
import pytest
import torch

from rank_latent_kv_absorbed_amd.mla import ERR_UNSUPPORTED, MlaError
from synthetic import block_weights, chunk_x, config
from tests.parity_util import BF16_RING_MEAN_REL, LatentRun, assert_parity, dev, sample_rows

pytestmark = pytest.mark.gpu

EPS = 1e-6


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def mid_cfg(**kw):
    base = dict(hidden=256, n_heads=4, d_nope=96, d_rope=32, d_v=128, d_c=192, grid_h=6, grid_w=10,
                window_frames=5, batch=2, rope_split=None, dtype="bf16")
    base.update(kw)
    return config("wan_layer").with_(**base)


def ring_lim(cfg):
    return BF16_RING_MEAN_REL if cfg.cache_dtype == "bf16" else None


def gain(cfg, seed=5):
    g = torch.Generator().manual_seed(seed)
    return (1.0 + 0.25 * torch.randn(cfg.d_qk, generator=g, dtype=torch.float64)).to(torch.bfloat16)


def uneven_query(run, Lq, seed=7, chunk=1000):
    """The run's seeded queries, each (token, head) row scaled by its own
    factor exp(N(0, 1)) (rounded back to bf16)."""
    q = run.query(Lq, chunk=chunk).double()
    g = torch.Generator().manual_seed(seed)
    f = torch.exp(torch.randn(q.shape[:-1] + (1,), generator=g, dtype=torch.float64))
    return (q * f).to(torch.bfloat16)


def wrapped_mid_run(cache_dtype, path):
    cfg = mid_cfg(cache_dtype=cache_dtype)
    run = LatentRun(cfg, path=path)
    run.write(0, 4)
    run.evict(2)
    run.write(4, 2)
    run.evict(1)
    run.write(6, 2)       # frames 3..7 resident through a wrap, Lk = 300
    return cfg, run


@pytest.mark.parametrize("cache_dtype", ["f16", "bf16", "e4m3"])
@pytest.mark.parametrize("path", ["absorbed", "expand"])
@pytest.mark.parametrize("Lq", [3, 130])
def test_query_norm_every_element(cache_dtype, path, Lq):
    cfg, run = wrapped_mid_run(cache_dtype, path)
    run.set_query_norm(gain(cfg), EPS)
    assert run.gpu.attend_path(Lq) == path
    q = uneven_query(run, Lq)
    got, ref, _ = run.attend(q, 8 * cfg.T - Lq)
    assert_parity(got, ref, "bf16", f"query norm {cache_dtype} {path} Lq={Lq}", mean_lim=ring_lim(cfg))


@pytest.mark.parametrize("path", ["absorbed", "expand"])
def test_query_norm_full_window_sampled_rows(path):
    cfg = config("wan_window")
    run = LatentRun(cfg, path=path)
    run.write(0, cfg.prefill_frames)
    run.evict(cfg.evict_frames)
    run.write(cfg.chunk_frame0, cfg.chunk_frames)
    run.set_query_norm(gain(cfg, seed=6), 1e-5)
    q = uneven_query(run, cfg.Lq, seed=8)
    rows = sample_rows(cfg.Lq, 32)
    got, ref, _ = run.attend(q, cfg.chunk_frame0 * cfg.T, rows=rows)
    assert_parity(got, ref, "bf16", f"query norm, 21-frame window, {path}")


@pytest.mark.parametrize("cache_dtype", ["f16", "e4m3"])
def test_query_norm_single_token_full_window(cache_dtype):
    cfg = config("wan_window").with_(batch=2, cache_dtype=cache_dtype)
    run = LatentRun(cfg)
    run.write(0, cfg.prefill_frames)
    run.evict(cfg.evict_frames)
    run.write(cfg.chunk_frame0, cfg.chunk_frames)
    run.set_query_norm(gain(cfg, seed=9), EPS)
    q = uneven_query(run, 1, seed=10)
    got, ref, _ = run.attend(q, (cfg.chunk_frame0 + cfg.chunk_frames) * cfg.T - 1)
    assert_parity(got, ref, "bf16", f"query norm, one token, {cache_dtype}")


def test_query_norm_off_again_and_block_refusal():
    cfg, run = wrapped_mid_run("f16", None)
    q = uneven_query(run, 40)
    run.set_query_norm(gain(cfg), EPS)
    normed, ref_n, _ = run.attend(q, 8 * cfg.T - 40)
    assert_parity(normed, ref_n, "bf16", "query norm on")
    # the attention block never forms per-head queries: refused while set
    bw = {k: dev(v) for k, v in block_weights(cfg).items()}
    w_qf = run.gpu.fold_query_weights(bw["w_q"], run.wd["w_uk"])
    w_fo = run.gpu.fold_output_weights(bw["w_o"], run.wd["w_uv"])
    xq = dev(chunk_x(cfg, 1, chunk=3)[:, :16].contiguous())
    with pytest.raises(MlaError) as e:
        run.gpu.attend_block(xq, 8 * cfg.T - 16, w_qf, w_fo)
    assert e.value.status == ERR_UNSUPPORTED
    run.set_query_norm(None, 0.0)
    plain, ref_p, _ = run.attend(q, 8 * cfg.T - 40)
    assert_parity(plain, ref_p, "bf16", "query norm off again")
    assert np.abs(ref_p - ref_n).max() > 1e-2 * np.abs(ref_p).max()   # the norm mattered
    run.gpu.attend_block(xq, 8 * cfg.T - 16, w_qf, w_fo)
    torch.cuda.synchronize()


def test_query_norm_key_splits_and_noalloc():
    """With the norm set: forced key splits against the oracle, and the
    allocation-free entry bit for bit against mla_attend (same path and
    schedule)."""
    cfg, run = wrapped_mid_run("f16", "absorbed")
    run.set_query_norm(gain(cfg), EPS)
    q = uneven_query(run, 40)
    got, ref, _ = run.attend(q, 8 * cfg.T - 40, key_splits=3)
    assert_parity(got, ref, "bf16", "query norm, 3 key ranges")
    _, _, out = run.attend(q, 8 * cfg.T - 40)
    o2 = torch.empty_like(out)
    run.gpu.attend_noalloc(dev(q), 8 * cfg.T - 40, run.wd["w_uk"], run.wd["w_uv"], o2)
    torch.cuda.synchronize()
    assert torch.equal(o2, out)


@pytest.mark.parametrize("path", ["absorbed", "expand"])
def test_query_norm_zero_row_with_zero_eps_stays_in_its_row(path):
    """eps = 0 and one all-zero query row: that (token, head) row has no scale
    and comes out NaN, as in the oracle (0 / 0); every other row is untouched
    and matches the oracle."""
    cfg, run = wrapped_mid_run("f16", path)
    run.set_query_norm(gain(cfg), 0.0)
    q = uneven_query(run, 130)
    q[1, 17, 2] = 0.0
    with np.errstate(invalid="ignore", divide="ignore"):      # the oracle's 0 / 0
        got, ref, _ = run.attend(q, 8 * cfg.T - 130)
    assert np.isnan(ref[1, 17, 2]).all() and np.isnan(got[1, 17, 2]).all()
    keep = np.ones(got.shape[:3], dtype=bool)
    keep[1, 17, 2] = False
    assert np.isfinite(got[keep]).all()
    assert_parity(got[keep], ref[keep], "bf16", f"query norm, zero row elsewhere, {path}")
