"""mla_attend_noalloc: the allocation-free variant of mla_attend (workspace in
the library's static device scratch).

CPU: through the host library compiled against the recording launcher, the
variant hands the kernels the scratch's address as their workspace, takes the
same path and schedule as mla_attend, and refuses (MLA_ERR_SCRATCH, nothing
enqueued) a call whose workspace would exceed the scratch.
GPU: through the C ABI, two calls in a row (the second with fewer queries)
give the same output as mla_attend with a caller workspace, bit for bit, and
match the fp64 oracle.
"""

import ctypes
import os
import subprocess

import numpy as np
import pytest
import torch

from synthetic import config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rank_latent_kv_absorbed_amd", "csrc")
SCRATCH_FAKE = 3 << 40          # the recording launcher's stand-in scratch address
P = ctypes.c_void_p


@pytest.fixture(scope="module")
def sim(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("hostsim_noalloc") / "libmla_hostsim.so")
    cmd = ["g++", "-O1", "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "mla_host.cpp"), os.path.join(ROOT, "tests", "hostsim", "fake_launch.cpp"),
           "-o", out]
    subprocess.run(cmd, check=True, capture_output=True)
    L = ctypes.CDLL(out)
    from rank_latent_kv_absorbed_amd.mla import SIGNATURES
    for name, (res, args) in SIGNATURES.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    return L


def _handle(L, **kw):
    from rank_latent_kv_absorbed_amd.mla import _HANDLE, make_config
    c = make_config(config("wan_window", **kw))
    h = _HANDLE()
    assert L.mla_cache_create(ctypes.byref(c), P(1 << 40), L.mla_cache_bytes(ctypes.byref(c)),
                              ctypes.byref(h)) == 0
    return h


def _attend_ptrs(L):
    a = (ctypes.c_longlong * 4)()
    L.fake_attend_ptrs(a)
    return list(a)


def _attend_info(L):
    a = (ctypes.c_longlong * 20)()
    L.fake_attend_info(a)
    return list(a)


def test_noalloc_uses_the_scratch_and_refuses_oversized_calls(sim):
    from rank_latent_kv_absorbed_amd.mla import ERR_EMPTY, ERR_SCRATCH
    assert sim.mla_attend_noalloc_max_bytes() == 64 << 20
    for cache_dtype in ("f16", "bf16"):
        h = _handle(sim, batch=11, cache_dtype=cache_dtype)
        assert sim.mla_attend_noalloc(h, P(1 << 41), 0, 1, P(1 << 41), P(1 << 41), P(1 << 41), 0,
                                      None) == ERR_EMPTY
        assert sim.mla_cache_set_state(h, 3, 23) == 0
        for Lq in (1, 8, 16):
            n = sim.fake_count()
            assert sim.mla_attend_noalloc(h, P(1 << 41), 23 * 1560, Lq, P(1 << 41), P(1 << 41),
                                          P(1 << 41), 0, None) == 0
            assert sim.fake_count() == n + 1
            noalloc = (_attend_info(sim), _attend_ptrs(sim))
            assert noalloc[1][0] == SCRATCH_FAKE            # queries at the scratch's start
            ws = 1 << 42
            need = sim.mla_attend_workspace_bytes(h, Lq, 0)
            assert need <= 64 << 20
            assert sim.mla_attend(h, P(1 << 41), 23 * 1560, Lq, P(1 << 41), P(1 << 41), P(1 << 41), 0,
                                  P(ws), need, None) == 0
            info, ptrs = _attend_info(sim), _attend_ptrs(sim)
            assert info == noalloc[0]                       # same schedule and arguments
            assert [p - ws if p else 0 for p in ptrs] == [p - SCRATCH_FAKE if p else 0 for p in noalloc[1]]
        # a full 4680-query chunk needs far more than the scratch: refused, nothing enqueued
        n = sim.fake_count()
        assert sim.mla_attend_noalloc(h, P(1 << 41), 0, 4680, P(1 << 41), P(1 << 41), P(1 << 41), 0,
                                      None) == ERR_SCRATCH
        assert sim.fake_count() == n
        sim.mla_cache_destroy(h)


@pytest.mark.gpu
@pytest.mark.parametrize("cache_dtype", ["f16", "bf16", "e4m3"])
def test_noalloc_matches_mla_attend_twice(cache_dtype):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from tests.parity_util import LatentRun, assert_parity, dev
    from oracle import mla as O
    cfg = config("wan_layer").with_(grid_h=5, grid_w=13, window_frames=6, batch=3,
                                    cache_dtype=cache_dtype)
    run = LatentRun(cfg)
    run.write(0, 4)
    run.evict(1)
    run.write(4, 2)                       # 5 frames resident through a wrap: 325 keys
    for Lq in (40, 3):                    # the second call is smaller
        q = run.query(Lq, chunk=Lq)
        out_na = torch.full((cfg.batch, Lq, cfg.n_heads, cfg.d_v), float("nan"), device="cuda")
        run.gpu.attend_noalloc(dev(q), 6 * cfg.T - Lq, run.wd["w_uk"], run.wd["w_uv"], out_na)
        ws = torch.empty(run.gpu.workspace_bytes(Lq), dtype=torch.uint8, device="cuda")
        out_ws = run.gpu.attend(dev(q), 6 * cfg.T - Lq, run.wd["w_uk"], run.wd["w_uv"], workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_ws), f"Lq={Lq}: noalloc and workspace results differ"
        ref = O.attend(run.store, run.ring, q.double().numpy(), 6 * cfg.T - Lq,
                       run.w["w_uk"].double().numpy(), run.w["w_uv"].double().numpy(), cfg)
        assert_parity(out_na.cpu().numpy(), ref, "bf16", f"noalloc {cache_dtype} Lq={Lq}",
                      mean_lim=1.5e-3 if cache_dtype == "bf16" else None)
