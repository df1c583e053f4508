"""GPU parity of the steps around the latent path, through the C ABI, against
the fp64 oracle on the same seeded inputs:

  * the cache write with the latent RMS-normalised (mla_cache_write_norm):
    stored rows within one ring ulp of the oracle's rounded values (plus the
    fp32 summation bound), and attention over a normalised window;
  * the weight-level folds (mla_fold_query_weights, mla_fold_output_weights):
    the two bf16 parts sum to the fp64 products within 2^-15 of each value;
  * the attention block (mla_attend_block) from the query tokens' layer input
    to model width, every element on mid sizes and sampled rows at the Wan
    shape, every ring type.

Bars as in the other parity tests: max|err| <= 1e-2 max|ref| and
sum|err| <= 2e-3 sum|ref| (1.5e-3 for a bf16 ring).
"""


import numpy as np
import pytest
import torch

from oracle import mla as O
from synthetic import block_weights, chunk_x, config
from tests.parity_util import (BF16_RING_MEAN_REL, LatentRun, assert_parity, dev, sample_rows)

pytestmark = pytest.mark.gpu

SIG_BITS = {"bf16": 8, "f16": 11, "e4m3": 4}
EPS = 1e-6


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def mid_cfg(**kw):
    base = dict(hidden=256, n_heads=4, d_nope=32, d_rope=32, d_v=64, d_c=64, grid_h=6, grid_w=10,
                window_frames=5, batch=2, rope_split=None, dtype="bf16")
    base.update(kw)
    return config("wan_layer").with_(**base)


def ring_lim(cfg):
    return BF16_RING_MEAN_REL if cfg.cache_dtype == "bf16" else None


class BlockRun(LatentRun):
    """A latent cache whose writes normalise the latent (optional) and whose
    attention runs as the model-width block with folded weights."""

    def __init__(self, cfg, norm=False, **kw):
        super().__init__(cfg, **kw)
        self.bw = block_weights(cfg)
        self.bwd = {k: dev(v) for k, v in self.bw.items()}
        self.norm = norm

    def write(self, frame0, n_frames, x=None):
        if not self.norm:
            return super().write(frame0, n_frames, x)
        if x is None:
            x = chunk_x(self.cfg, n_frames, layer=self.layer, chunk=self.n_ops)
        self.n_ops += 1
        self.gpu.write_norm(dev(x), self.wd["w_dkr"], self.bwd["kv_gamma"], EPS, frame0, n_frames)
        O.cache_write(self.store, self.ring, x.double().numpy(), self.w["w_dkr"].double().numpy(), frame0,
                      n_frames, self.cfg, storage=self.rnd,
                      kv_norm=(self.bw["kv_gamma"].double().numpy(), EPS))
        return x

    def folds(self):
        w_qf = self.gpu.fold_query_weights(self.bwd["w_q"], self.wd["w_uk"])
        w_fo = self.gpu.fold_output_weights(self.bwd["w_o"], self.wd["w_uv"])
        return w_qf, w_fo

    def attend_block(self, xq, q_token0, rows=None, key_splits=0):
        w_qf, w_fo = self.folds()
        out = self.gpu.attend_block(dev(xq), q_token0, w_qf, w_fo, key_splits=key_splits)
        torch.cuda.synchronize()
        ref = O.attend_block(self.store, self.ring, xq.double().numpy(), q_token0,
                             self.bw["w_q"].double().numpy(), self.w["w_uk"].double().numpy(),
                             self.w["w_uv"].double().numpy(), self.bw["w_o"].double().numpy(), self.cfg,
                             rows=rows)
        got = out.cpu().numpy()
        return (got if rows is None else got[:, rows]), ref


# --------------------------------------------------------------------------
# cache write with the latent normalised
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cache_dtype,d_c", [("f16", 64), ("bf16", 128), ("f16", 192), ("e4m3", 192)])
def test_cache_write_norm_values(cache_dtype, d_c):
    cfg = mid_cfg(cache_dtype=cache_dtype, d_c=d_c, batch=2) if d_c < 192 else \
        config("wan_layer").with_(grid_h=5, grid_w=13, window_frames=6, batch=2, cache_dtype=cache_dtype)
    run = BlockRun(cfg, norm=True)
    x = run.write(0, 3)
    torch.cuda.synchronize()
    got = run.gpu.ring().cpu().double().numpy()[:, :3 * cfg.T]
    ref = run.store[:, :3 * cfg.T]
    ulp = np.ldexp(1.0, np.frexp(np.abs(ref))[1] - SIG_BITS[cache_dtype])
    if cache_dtype == "e4m3":
        ulp = np.maximum(ulp, 2.0 ** -9)          # the subnormal quantum
    # fp32 summation of the hidden-wide products (scaled like the stored value)
    # and of the row's sum of squares
    raw = np.abs(x.double().numpy()) @ np.abs(run.w["w_dkr"].double().numpy()).T
    c_raw = x.double().numpy() @ run.w["w_dkr"].double().numpy().T
    rms = np.sqrt(np.mean(c_raw[..., :cfg.d_c] ** 2, axis=-1, keepdims=True) + EPS)
    gam = np.abs(run.bw["kv_gamma"].double().numpy())
    acc = cfg.hidden * 2.0 ** -24 * raw
    acc[..., :cfg.d_c] = acc[..., :cfg.d_c] * gam / rms + 4 * 2.0 ** -24 * np.abs(ref[..., :cfg.d_c])
    acc[..., cfg.d_c:] = 4 * acc[..., cfg.d_c:]
    assert (np.abs(got - ref) <= ulp + acc).all()
    assert np.mean(got == ref) > 0.95


def test_attend_over_normalised_window_with_wrap():
    cfg = mid_cfg(d_nope=96, d_rope=32, d_v=128, d_c=192)
    run = BlockRun(cfg, norm=True)
    run.write(0, 4)
    run.evict(2)
    run.write(4, 2)
    run.evict(1)
    run.write(6, 2)       # frames 3..7 resident through a wrap, Lk = 300
    q = run.query(40)
    got, ref, _ = run.attend(q, 8 * cfg.T - 40)
    assert_parity(got, ref, "bf16", "attend over RMS-normalised latents")


# --------------------------------------------------------------------------
# weight-level folds
# --------------------------------------------------------------------------

def test_folded_weights_match_fp64_products():
    cfg = config("wan_layer").with_(grid_h=5, grid_w=13, window_frames=6, batch=1)
    run = BlockRun(cfg)
    w_qf, w_fo = run.folds()
    torch.cuda.synchronize()
    n_h, dq, dn, dv, dc = cfg.n_heads, cfg.d_qk, cfg.d_nope, cfg.d_v, cfg.d_c
    wq = run.bw["w_q"].double().numpy().reshape(n_h, dq, cfg.hidden)
    w_uk = run.w["w_uk"].double().numpy()
    w_uv = run.w["w_uv"].double().numpy()
    want_q = np.concatenate([np.einsum("hni,hnk->hik", w_uk, wq[:, :dn]), wq[:, dn:]], axis=1)
    w_o = run.bw["w_o"].double().numpy().reshape(cfg.hidden, n_h, dv)
    want_o = np.einsum("chv,hvi->chi", w_o, w_uv).reshape(cfg.hidden, n_h * dc)
    # fp32 accumulation bound of each dot product (n terms: n 2^-24 sum |a_i b_i|)
    bound_q = np.concatenate([dn * 2.0 ** -24 * np.einsum("hni,hnk->hik", np.abs(w_uk), np.abs(wq[:, :dn])),
                              np.zeros_like(wq[:, dn:])], axis=1)
    bound_o = (dv * 2.0 ** -24 * np.einsum("chv,hvi->chi", np.abs(w_o), np.abs(w_uv))).reshape(cfg.hidden, n_h * dc)
    for got_t, want, bound, what in ((w_qf, want_q, bound_q, "query"), (w_fo, want_o, bound_o, "output")):
        parts = got_t.double().cpu().numpy()
        got = parts[0] + parts[1]
        # the two bf16 parts carry the fp32 result to within 2^-16 of it
        tol = 2.0 ** -15 * np.abs(want) + 2 * bound
        assert (np.abs(got - want) <= tol).all(), what
        assert (parts[0] == torch.from_numpy(want).to(torch.bfloat16).double().numpy()).mean() > 0.99, what


# --------------------------------------------------------------------------
# the attention block, model width
# --------------------------------------------------------------------------

# Mid sizes through a ring wrap (300 keys, ragged tiles); query counts reach
# the narrow and chunk core shapes; forced key splits merge partials.
@pytest.mark.parametrize("cache_dtype", ["f16", "bf16", "e4m3"])
@pytest.mark.parametrize("Lq,key_splits", [(3, 0), (20, 0), (33, 3), (130, 0)])
def test_attend_block_every_element(cache_dtype, Lq, key_splits):
    cfg = mid_cfg(d_nope=96, d_rope=32, d_v=128, d_c=64, cache_dtype=cache_dtype)
    run = BlockRun(cfg)
    run.write(0, 4)
    run.evict(2)
    run.write(4, 2)
    run.evict(1)
    run.write(6, 2)
    xq = chunk_x(cfg, 3, chunk=77)[:, :Lq].contiguous()
    got, ref = run.attend_block(xq, 8 * cfg.T - Lq, key_splits=key_splits)
    assert_parity(got, ref, "bf16", f"block {cache_dtype} Lq={Lq} splits={key_splits}", mean_lim=ring_lim(cfg))


@pytest.mark.parametrize("cache_dtype,norm", [("f16", False), ("bf16", False), ("f16", True), ("e4m3", True)])
def test_attend_block_wan_layer_sampled_rows(cache_dtype, norm):
    cfg = config("wan_layer").with_(cache_dtype=cache_dtype)
    run = BlockRun(cfg, norm=norm)
    run.write(0, cfg.prefill_frames)
    run.write(cfg.chunk_frame0, cfg.chunk_frames)
    xq = chunk_x(cfg, cfg.chunk_frames, chunk=88)
    rows = sample_rows(cfg.Lq, 24)
    got, ref = run.attend_block(xq, cfg.chunk_frame0 * cfg.T, rows=rows)
    assert_parity(got, ref, "bf16", f"block wan layer {cache_dtype} norm={norm}", mean_lim=ring_lim(cfg))


@pytest.mark.parametrize("Lq", [1, 8])
def test_attend_block_small_queries(Lq):
    cfg = config("wan_layer").with_(window_frames=3, batch=3)
    run = BlockRun(cfg)
    run.write(0, 3)
    xq = chunk_x(cfg, 1, chunk=99)[:, :Lq].contiguous()
    got, ref = run.attend_block(xq, 3 * cfg.T - Lq)
    assert_parity(got, ref, "bf16", f"block small query Lq={Lq}")
