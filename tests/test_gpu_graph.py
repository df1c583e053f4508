"""mla_attend and mla_attend_noalloc under HIP graph capture.

The library enqueues only kernels on the caller's stream (no memset, no
allocation, no host synchronisation), so a call can be captured into a
graph.  A captured call keeps the arguments of its capture: the query,
weight, output and workspace pointers and the window state (resident key
count and first slot), so it is replayed for new query contents in the same
buffers and re-captured after a write or an eviction.

Each case captures one call, then replays it several times with eager work
and synchronisations in between, and checks every replay bit for bit
against the eager call on the same inputs; the last replays run after the
query buffer was refilled in place.  Cases: the absorbed path with the chunk
and the few-token prologues, the expand path, and the allocation-free entry.
"""

import numpy as np
import pytest
import torch

from synthetic import config
from tests.parity_util import LatentRun, assert_parity, dev

pytestmark = pytest.mark.gpu


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def mid_run(path):
    cfg = config("wan_layer").with_(hidden=256, n_heads=4, d_nope=96, d_rope=32, d_v=128, d_c=192, grid_h=6,
                                    grid_w=10, window_frames=5, batch=2, rope_split=None, dtype="bf16")
    run = LatentRun(cfg, path=path)
    run.write(0, 4)
    run.evict(2)
    run.write(4, 2)
    run.evict(1)
    run.write(6, 2)       # frames 3..7 resident through a wrap, Lk = 300
    return cfg, run


@pytest.mark.parametrize("path,Lq,noalloc", [("absorbed", 130, False), ("absorbed", 3, False),
                                             ("expand", 200, False), ("absorbed", 40, True)])
def test_captured_attend_replays_match_eager(path, Lq, noalloc):
    cfg, run = mid_run(path)
    assert run.gpu.attend_path(Lq) == path
    q0 = run.query(Lq, chunk=21)
    q1 = run.query(Lq, chunk=22)
    qd = dev(q0)
    q_token0 = 8 * cfg.T - Lq
    w_uk, w_uv = run.wd["w_uk"], run.wd["w_uv"]
    out = torch.empty((cfg.batch, Lq, cfg.n_heads, cfg.d_v), dtype=torch.float32, device="cuda")
    ws = None if noalloc else torch.empty(run.gpu.workspace_bytes(Lq), dtype=torch.uint8, device="cuda")

    def call():
        if noalloc:
            run.gpu.attend_noalloc(qd, q_token0, w_uk, w_uv, out)
        else:
            run.gpu.attend(qd, q_token0, w_uk, w_uv, out=out, workspace=ws)

    # eager references on both query contents (and the library's one-time set-up)
    eager = []
    for qc in (q0, q1):
        qd.copy_(dev(qc))
        call()
        torch.cuda.synchronize()
        eager.append(out.clone())
    # the eager result is the attention (the oracle), for the first contents
    got, ref, _ = run.attend(q0, q_token0)
    assert_parity(eager[0].cpu().numpy(), ref, "bf16", f"graph case {path} Lq={Lq} eager")

    qd.copy_(dev(q0))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for rep, k in enumerate((0, 0, 1, 1, 0)):
        qd.copy_(dev((q0, q1)[k]))
        out.fill_(float("nan"))
        scratch.mul_(1.0001)                       # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[k]), f"replay {rep} ({'second' if k else 'first'} query contents)"
    del g
