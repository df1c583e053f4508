#!/usr/bin/env python3
"""Benchmark of the latent-KV hot path on one MI355X.

A step is one pass of the whole path for one layer: evict the 3 oldest frames
of that layer's 21-frame window, fused cache write of the new 3-frame chunk
(4680 tokens), attention of the chunk's 4680 queries over the 32760 resident
keys (the library's choice of path for this chunk length: expand-then-attend,
which rebuilds the window's per-head keys and values from the latent and runs
per-head attention; --path absorbed times the latent-space form instead).
Steps cycle over the windows of 30 layers (440 MB of latent cache, more than
the 256 MB last-level cache).  Printed metric: attended query tokens/s per
layer = batch * 4680 / step time, plus MFMA utilisation.

Also reported: the main attention kernel alone (HIP events recorded by the
library on its stream) against the bf16 MFMA roofline, the other path's step
time, the dense per-head MHA comparison on the same shape, a cache-bound
small-query case against HBM bandwidth, and the fp64 CPU oracle timed on a
bounded sample.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attended query tokens/s per layer (21-frame window, 4680-q chunk) + MFMA util %"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
# Hardware traffic counters of each path's attention core (written from
# rocprofv3 runs of this script), valid while the core's sources are unchanged.
TRAFFIC_FILES = {"absorbed": os.path.join(ROOT, "profiles", "attend_core_wan_window_traffic.json"),
                 "expand": os.path.join(ROOT, "profiles", "attend_expand_wan_window_traffic.json")}
CORE_SOURCES = {
    "absorbed": ["rank_latent_kv_absorbed_amd/csrc/mla_attn_core.h",
                 "rank_latent_kv_absorbed_amd/csrc/mla_attend.hip",
                 "rank_latent_kv_absorbed_amd/csrc/mla_device.h"],
    "expand": ["rank_latent_kv_absorbed_amd/csrc/mla_attn_core.h",
               "rank_latent_kv_absorbed_amd/csrc/mha_attend.hip",
               "rank_latent_kv_absorbed_amd/csrc/mla_expand.hip",
               "rank_latent_kv_absorbed_amd/csrc/mla_device.h"],
}
CORE_KERNELS = {"absorbed": "attn_core_kernel<E, 224, 192, ...> (latent scores and value sums)",
                "expand": "attn_core_kernel<E, 128, 128, ...> (per-head attention over the "
                          "rebuilt keys and values)"}


def core_source_sha(path="absorbed"):
    h = hashlib.sha256()
    for p in CORE_SOURCES[path]:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def core_flop(cfg, path, B, Lq, Lk):
    """Algorithmic FLOP of one launch of the path's attention core."""
    if path == "expand":
        return B * cfg.n_heads * Lq * Lk * 2 * (cfg.d_qk + cfg.d_v)
    return B * cfg.n_heads * Lq * Lk * (2 * (cfg.d_c + cfg.d_rope) + 2 * cfg.d_c)


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime (for the library's profiling hook)."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self):
        e = ctypes.c_void_p()
        assert self.rt.hipEventCreate(ctypes.byref(e)) == 0
        self.made.append(e.value)
        return e.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.rt.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def close(self):
        for e in self.made:
            self.rt.hipEventDestroy(e)
        self.made = []


def cpu_baseline(cfg, x_chunk, w, q, repeats=3):
    """The fp64 oracle, untuned, on one full step of the workload at batch 1:
    evict 3 frames, cache write of the 3-frame chunk into the 21-frame window,
    attention of all of the chunk's queries; median of `repeats` runs."""
    import numpy as np
    from oracle import mla as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    T = cfg.T
    rng = np.random.default_rng(0)
    xs = x_chunk[:1].double().numpy()
    wd = {k: v.double().numpy() for k, v in w.items()}
    qs = q[:1].double().numpy()
    times = []
    for _ in range(repeats):
        store = O.round_storage(rng.standard_normal((1, cfg.window_frames * T, cfg.width)),
                                cfg.cache_dtype)
        ring = O.RingModel(cfg.window_frames, T)
        ring.write(0, cfg.window_frames)
        t0 = time.perf_counter()
        O.cache_evict(ring, cfg.chunk_frames)
        O.cache_write(store, ring, xs, wd["w_dkr"], cfg.window_frames, cfg.chunk_frames, cfg,
                      storage=cfg.cache_dtype)
        O.attend(store, ring, qs, cfg.window_frames * T, wd["w_uk"], wd["w_uv"], cfg)
        times.append(time.perf_counter() - t0)
    t_step = sorted(times)[len(times) // 2]
    return {
        "value": cfg.Lq / t_step, "unit": "query tokens/s per layer", "cores": int(threads),
        "kind": "oracle",
        "sample": (f"one full step at batch 1 (evict {cfg.chunk_frames} frames, cache write of "
                   f"{cfg.Lq} tokens, attention of {cfg.Lq} queries x {cfg.n_heads} heads over "
                   f"{cfg.window_frames * T} keys), fp64 NumPy oracle, median of {repeats} runs"),
        "seconds_measured": round(sum(times), 2),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--layers", type=int, default=30)
    ap.add_argument("--path", choices=["auto", "absorbed", "expand"], default="auto",
                    help="attention path of every layer's handle (auto: the library's choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip dense and small-query cases")
    ap.add_argument("--rollout", action="store_true",
                    help="full rollout sweep: latent widths 64/128/192 x batch 1/4/8/11 (default "
                         "extras run latent width 192 at batch 1 only)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device-to-device copy of this size first (a known-byte "
                         "kernel for scaling hardware traffic counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)

    import torch
    from rank_latent_kv_absorbed_amd import LatentCache, DenseCache, attend_flops, attend_bytes
    from rank_latent_kv_absorbed_amd.mla import expand_attend_flops, mha_attend_flops
    from synthetic import chunk_q, chunk_x, config, dense_weights, layer_weights

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cfg = config("wan_window").with_(batch=args.batch)
    B, T, Lq, W = cfg.batch, cfg.T, cfg.Lq, cfg.window_frames
    Lk = W * T
    L = args.layers

    # inputs resident in HBM before timing
    x_chunk_cpu = chunk_x(cfg, cfg.chunk_frames, chunk=1)
    q_cpu = chunk_q(cfg, Lq, chunk=1)
    x_chunk = x_chunk_cpu.to(dev)
    q = q_cpu.to(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    x_pre = torch.randn((B, W * T, cfg.hidden), generator=gen, device=dev).to(torch.bfloat16)
    weights_cpu = [layer_weights(cfg, layer=l) for l in range(L)]
    weights = [{k: v.to(dev) for k, v in w.items()} for w in weights_cpu]
    caches = []
    for l in range(L):
        c = LatentCache(cfg, device=dev)
        c.set_attend_path(args.path)
        c.write(x_pre, weights[l]["w_dkr"], 0, W)
        caches.append(c)
    path = caches[0].attend_path(Lq)
    newest = [W - 1] * L
    out = torch.empty((B, Lq, cfg.n_heads, cfg.d_v), dtype=torch.float32, device=dev)
    ws_bytes = max(caches[0].workspace_bytes(Lq), 1)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ev = HipEvents()
    state = {"i": 0}

    def step(core_events=None):
        l = state["i"] % L
        state["i"] += 1
        c, w = caches[l], weights[l]
        c.evict(cfg.chunk_frames)
        f0 = newest[l] + 1
        c.write(x_chunk, w["w_dkr"], f0, cfg.chunk_frames)
        newest[l] = f0 + cfg.chunk_frames - 1
        if core_events is not None:
            c.set_profile_events(*core_events)
        c.attend(q, f0 * T, w["w_uk"], w["w_uv"], out=out, workspace=ws)
        if core_events is not None:
            c.set_profile_events(None, None)

    def timed(n_steps):
        """(ms per step, mean core-kernel ms) over n_steps steps."""
        core_ev = [(ev.create(), ev.create()) for _ in range(n_steps)]
        t_start = torch.cuda.Event(enable_timing=True)
        t_stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t_start.record()
        for k in range(n_steps):
            step(core_ev[k])
        t_stop.record()
        torch.cuda.synchronize()
        core_ms = [ev.elapsed_ms(a, b) for a, b in core_ev]
        return t_start.elapsed_time(t_stop) / n_steps, sum(core_ms) / len(core_ms)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms_step, core_avg = timed(args.steps)

    # algorithmic work of the path that ran
    c_flop = core_flop(cfg, path, B, Lq, Lk)
    if path == "expand":
        att_flop = expand_attend_flops(cfg.n_heads, Lq, Lk, cfg.d_c, cfg.d_rope, cfg.d_nope,
                                       cfg.d_v, B)
    else:
        att_flop = attend_flops(cfg.n_heads, Lq, Lk, cfg.d_c, cfg.d_rope, cfg.d_nope, cfg.d_v, B)
    write_flop = 2 * B * Lq * cfg.hidden * cfg.width
    step_flop = att_flop + write_flop
    absorbed_step_flop = write_flop + attend_flops(cfg.n_heads, Lq, Lk, cfg.d_c, cfg.d_rope,
                                                   cfg.d_nope, cfg.d_v, B)
    value = B * Lq / (ms_step / 1e3)
    mfma_pct = 100.0 * step_flop / (ms_step / 1e3) / (PEAK_BF16_TFLOPS * 1e12)
    absorbed_pct = 100.0 * absorbed_step_flop / (ms_step / 1e3) / (PEAK_BF16_TFLOPS * 1e12)
    achieved = c_flop / (core_avg / 1e3) / 1e12

    traffic = None
    if os.path.exists(TRAFFIC_FILES[path]):
        tr = json.load(open(TRAFFIC_FILES[path]))
        if tr.get("kernel_source_sha") == core_source_sha(path) and tr.get("batch") == B:
            traffic = tr.get("hbm_bytes_per_launch")

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "query tokens/s per layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "wan_window: per layer, evict 3 frames + fused cache write of a "
                               "3-frame chunk + latent-KV attention of its queries over a 21-frame "
                               "window; 30 layer windows cycled",
                   "attend_path": path,
                   "global_batch": B, "query_tokens": Lq, "resident_keys": Lk, "n_heads": cfg.n_heads,
                   "d_c": cfg.d_c, "d_rope": cfg.d_rope, "d_nope": cfg.d_nope, "d_v": cfg.d_v,
                   "hidden": cfg.hidden, "grid": [cfg.grid_h, cfg.grid_w], "layers_cycled": L,
                   "parallelism": "none (1 GPU)"},
        "mfma_util_pct": round(mfma_pct, 2),
        "mfma_util_pct_absorbed_form": round(absorbed_pct, 2),
        "roofline": {"bound": "mfma", "kernel": CORE_KERNELS[path],
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "avg_launch_ms": round(core_avg, 4),
                     "algorithmic_flop_per_launch": c_flop},
        "step_flop": step_flop,
        "breakdown_ms": {"step": round(ms_step, 4), "attend_core": round(core_avg, 4)},
        "cache_bytes": {"latent_per_layer": caches[0].nbytes, "latent_30_layers": caches[0].nbytes * 30,
                        "dense_per_layer": None},
    }

    if not args.no_extras:
        # the other attention path on the same steps
        other = "absorbed" if path == "expand" else "expand"
        try:
            for c in caches:
                c.set_attend_path(other)
        except Exception as e:          # the handle cannot take that path
            result["other_path"] = {"path": other, "error": str(e)}
        else:
            need = caches[0].workspace_bytes(Lq)
            if need > ws.numel():
                ws = torch.empty(need, dtype=torch.uint8, device=dev)
            for _ in range(5):
                step()
            o_step, o_core = timed(min(args.steps, 20))
            result["other_path"] = {"path": other, "ms_per_step": round(o_step, 4),
                                    "attend_core_ms": round(o_core, 4),
                                    "core_tflops": round(core_flop(cfg, other, B, Lq, Lk)
                                                         / (o_core / 1e3) / 1e12, 1),
                                    "value": round(B * Lq / (o_step / 1e3), 1)}
            for c in caches:
                c.set_attend_path(args.path)

        # several attends per written chunk (denoising steps): with reuse on, the
        # expand path rebuilds the window once per chunk
        if path == "expand":
            c = caches[0]
            reuse = {}
            for flag in (False, True):
                c.set_expand_reuse(flag)
                for _ in range(3):
                    c.attend(q, newest[0] * T, weights[0]["w_uk"], weights[0]["w_uv"], out=out, workspace=ws)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record()
                for _ in range(10):
                    c.attend(q, newest[0] * T, weights[0]["w_uk"], weights[0]["w_uv"], out=out, workspace=ws)
                e1.record()
                torch.cuda.synchronize()
                reuse["reuse_on" if flag else "reuse_off"] = round(e0.elapsed_time(e1) / 10, 4)
            c.set_expand_reuse(False)
            result["attend_ms_repeated_on_one_window"] = reuse

        # dense per-head MHA on the same shape (one layer), for time and cache bytes
        dcache = DenseCache(cfg, device=dev)
        dw = {k: v.to(dev) for k, v in dense_weights(cfg).items()}
        dcache.write(x_pre, dw["w_k"], dw["w_v"], 0, W)
        dcache.evict(cfg.chunk_frames)
        dcache.write(x_chunk, dw["w_k"], dw["w_v"], W, cfg.chunk_frames)
        dout = torch.empty((B, Lq, cfg.n_heads, cfg.d_qk), dtype=torch.float32, device=dev)
        dws = torch.empty(dcache.workspace_bytes(Lq), dtype=torch.uint8, device=dev)
        for _ in range(3):
            dcache.attend(q, W * T, out=dout, workspace=dws)
        dev_ev = [(ev.create(), ev.create()) for _ in range(10)]
        torch.cuda.synchronize()
        for a_, b_ in dev_ev:
            dcache.set_profile_events(a_, b_)
            dcache.attend(q, W * T, out=dout, workspace=dws)
        torch.cuda.synchronize()
        d_ms = sum(ev.elapsed_ms(a_, b_) for a_, b_ in dev_ev) / len(dev_ev)
        d_flop = mha_attend_flops(cfg.n_heads, Lq, Lk, cfg.d_qk, B)
        result["dense_mha"] = {"attend_core_ms": round(d_ms, 4),
                               "tflops": round(d_flop / (d_ms / 1e3) / 1e12, 2),
                               "cache_bytes_per_layer": dcache.nbytes,
                               "latent_vs_dense_attend_time": round(core_avg / d_ms, 3),
                               "cache_capacity_ratio": round(dcache.nbytes / caches[0].nbytes, 3)}
        result["cache_bytes"]["dense_per_layer"] = dcache.nbytes
        del dcache, dws, dout

        # cache-bound small-query shapes: Lq queries per sequence over the full
        # window, latent widths 64 / 128 / 192, batch 8 and 11, 30 layer windows
        # cycled (3.5-4.8 GB of windows, far above the last-level cache)
        sq = {}
        for d_c in (192, 128, 64):
            for Bs in (8, 11):
                scfg = cfg.with_(batch=Bs, d_c=d_c)
                sw = [layer_weights(scfg, layer=l) for l in range(2)]
                sw = [{k: v.to(dev) for k, v in w_.items()} for w_ in sw]
                scaches = []
                for l in range(L):
                    c = LatentCache(scfg, device=dev)
                    c.ring().copy_(torch.randn(c.ring().shape, generator=gen, device=dev).to(c.ring().dtype))
                    c.set_state(0, W - 1)
                    scaches.append(c)
                for Lqs in (1, 4, 8):
                    qs = torch.randn((Bs, Lqs, cfg.n_heads, cfg.d_qk), generator=gen, device=dev).to(torch.bfloat16)
                    so = torch.empty((Bs, Lqs, cfg.n_heads, cfg.d_v), dtype=torch.float32, device=dev)
                    sws = torch.empty(max(scaches[0].workspace_bytes(Lqs), 1), dtype=torch.uint8, device=dev)
                    for l in range(L):
                        scaches[l].attend(qs, Lk - Lqs, sw[l % 2]["w_uk"], sw[l % 2]["w_uv"], out=so, workspace=sws)
                    # whole calls back to back (no profiling events), then the
                    # core kernel alone by the library's events
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    torch.cuda.synchronize()
                    e0.record()
                    for i in range(2 * L):
                        scaches[i % L].attend(qs, Lk - Lqs, sw[i % 2]["w_uk"], sw[i % 2]["w_uv"], out=so,
                                              workspace=sws)
                    e1.record()
                    torch.cuda.synchronize()
                    call_ms = e0.elapsed_time(e1) / (2 * L)
                    sev = [(ev.create(), ev.create()) for _ in range(2 * L)]
                    for i, (a_, b_) in enumerate(sev):
                        c = scaches[i % L]
                        c.set_profile_events(a_, b_)
                        c.attend(qs, Lk - Lqs, sw[i % 2]["w_uk"], sw[i % 2]["w_uv"], out=so, workspace=sws)
                        c.set_profile_events(None, None)
                    torch.cuda.synchronize()
                    kms = sum(ev.elapsed_ms(a_, b_) for a_, b_ in sev) / len(sev)
                    win = Bs * Lk * (d_c + cfg.d_rope) * 2
                    nbytes = attend_bytes(cfg.n_heads, Lqs, Lk, d_c, cfg.d_rope, cfg.d_nope, cfg.d_v, Bs)
                    sq[f"dc{d_c}_Lq{Lqs}_B{Bs}"] = {
                        "attend_ms": round(call_ms, 4), "core_kernel_ms": round(kms, 4),
                        "algorithmic_bytes": nbytes,
                        "core_GBps": round(win / (kms / 1e3) / 1e9, 1),
                        "call_GBps": round(nbytes / (call_ms / 1e3) / 1e9, 1),
                        "hbm_frac_call": round(nbytes / (call_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                        "query_tokens_per_s": round(Bs * Lqs / (call_ms / 1e3), 1)}
                    del sws, so, qs
                del scaches, sw
        result["small_query_cache_bound"] = sq

        # batch scaling of the chunk step (evict + write + attend), 4 layer
        # windows cycled per batch size
        scale = {}
        for Bb in (1, 2, 4, 8):
            bcfg = cfg.with_(batch=Bb)
            bw = [{k: v.to(dev) for k, v in layer_weights(bcfg, layer=l).items()} for l in range(2)]
            bx = torch.randn((Bb, W * T, cfg.hidden), generator=gen, device=dev).to(torch.bfloat16)
            bxc = bx[:, :Lq].contiguous()
            bq = torch.randn((Bb, Lq, cfg.n_heads, cfg.d_qk), generator=gen, device=dev).to(torch.bfloat16)
            bcs = []
            for l in range(4):
                c = LatentCache(bcfg, device=dev)
                c.set_attend_path(args.path)
                c.write(bx, bw[l % 2]["w_dkr"], 0, W)
                bcs.append(c)
            bnew = [W - 1] * 4
            bout = torch.empty((Bb, Lq, cfg.n_heads, cfg.d_v), dtype=torch.float32, device=dev)
            bws = torch.empty(max(bcs[0].workspace_bytes(Lq), 1), dtype=torch.uint8, device=dev)
            del bx

            def bstep(k):
                l = k % 4
                c = bcs[l]
                c.evict(cfg.chunk_frames)
                f0 = bnew[l] + 1
                c.write(bxc, bw[l % 2]["w_dkr"], f0, cfg.chunk_frames)
                bnew[l] = f0 + cfg.chunk_frames - 1
                c.attend(bq, f0 * T, bw[l % 2]["w_uk"], bw[l % 2]["w_uv"], out=bout, workspace=bws)

            for k in range(4):
                bstep(k)
            n_b = 12
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for k in range(n_b):
                bstep(k)
            e1.record()
            torch.cuda.synchronize()
            b_ms = e0.elapsed_time(e1) / n_b
            bflop = (attend_flops(cfg.n_heads, Lq, Lk, cfg.d_c, cfg.d_rope, cfg.d_nope, cfg.d_v, Bb)
                     + 2 * Bb * Lq * cfg.hidden * cfg.width)
            scale[f"B{Bb}"] = {"ms_per_step": round(b_ms, 4),
                               "query_tokens_per_s": round(Bb * Lq / (b_ms / 1e3), 1),
                               "path": bcs[0].attend_path(Lq),
                               "mfma_util_pct_absorbed_form": round(100.0 * bflop / (b_ms / 1e3)
                                                                    / (PEAK_BF16_TFLOPS * 1e12), 2)}
            del bcs, bws, bout, bq, bxc, bw
        result["batch_scaling"] = scale

        # rollout: 80 chunks of 3 frames through every layer's 21-frame window
        # (evict to make room, write the chunk, attend its 4680 queries), the
        # whole loop bracketed by events; the window grows over the first 7
        # chunks, so the keys per attend average 1617 / 80 frames
        def rollout(d_c, Bb, n_chunks=80):
            rcfg = cfg.with_(batch=Bb, d_c=d_c)
            rw = [{k: v.to(dev) for k, v in layer_weights(rcfg, layer=l).items()} for l in range(L)]
            rx = torch.randn((Bb, Lq, cfg.hidden), generator=gen, device=dev).to(torch.bfloat16)
            rq = torch.randn((Bb, Lq, cfg.n_heads, cfg.d_qk), generator=gen, device=dev).to(torch.bfloat16)
            rcs = [LatentCache(rcfg, device=dev) for _ in range(L)]
            for c in rcs:
                c.set_attend_path(args.path)
            rout = torch.empty((Bb, Lq, cfg.n_heads, cfg.d_v), dtype=torch.float32, device=dev)
            rws = torch.empty(max(rcs[0].workspace_bytes(Lq), 1), dtype=torch.uint8, device=dev)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for k in range(n_chunks):
                for l in range(L):
                    c = rcs[l]
                    res = 0 if k == 0 else min(3 * k, W)
                    c.evict(max(0, res + cfg.chunk_frames - W))
                    c.write(rx, rw[l]["w_dkr"], 3 * k, cfg.chunk_frames)
                    c.attend(rq, 3 * k * T, rw[l]["w_uk"], rw[l]["w_uv"], out=rout, workspace=rws)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            frames = sum(min(3 * (k + 1), W) for k in range(n_chunks))
            flop = L * (sum(attend_flops(cfg.n_heads, Lq, min(3 * (k + 1), W) * T, d_c, cfg.d_rope,
                                         cfg.d_nope, cfg.d_v, Bb) for k in range(n_chunks))
                        + n_chunks * 2 * Bb * Lq * cfg.hidden * (d_c + cfg.d_rope))
            out = {"ms_total": round(ms, 2), "chunks": n_chunks, "layers": L,
                   "resident_frames_summed": frames,
                   "query_tokens_per_s_per_layer": round(Bb * Lq * n_chunks * L / (ms / 1e3), 1),
                   "mfma_util_pct_absorbed_form": round(100.0 * flop / (ms / 1e3) / (PEAK_BF16_TFLOPS * 1e12), 2)}
            del rcs, rws, rout, rw, rx, rq
            return out

        sweep = [(d, b_) for d in (192, 128, 64) for b_ in (1, 4, 8, 11)] if args.rollout else [(192, 1)]
        result["rollout"] = {}
        for d, b_ in sweep:
            result["rollout"][f"dc{d}_B{b_}"] = rollout(d, b_)
            print(f"rollout d_c={d} B={b_}: {result['rollout'][f'dc{d}_B{b_}']}", file=sys.stderr,
                  flush=True)

    ev.close()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, x_chunk_cpu, weights_cpu[0], q_cpu)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
