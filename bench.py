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

Also reported on the same JSON line: the main attention kernel alone (HIP
events recorded by the library on its stream) against the MFMA roofline; the
other path's step time; the same step with a bf16 ring (both paths) and with
the query norm set; the
dense per-head MHA comparison (same shape, and at the largest batch whose
30-layer dense cache fits the GPU, with the measured batch capacity of both
caches); cache-bound small-query cases against HBM bandwidth; batch scaling;
the 80-chunk rollout at latent widths 192 / 128 / 64; measured copy and read
bandwidth ceilings; and the fp64 CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

# The fp64 oracle's matrix products run on OpenBLAS threads: one per host core
# this process may run on, set before numpy is first imported.
HOST_CORES = len(os.sched_getaffinity(0))
os.environ["OPENBLAS_NUM_THREADS"] = str(HOST_CORES)

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attended query tokens/s per layer (21-frame window, 4680-q chunk) + MFMA util %"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
PAGES_BATCH_RATIO = 8.0     # largest batch vs dense MHA at d_c = 192 (technical summary, results)
# Hardware traffic counters and the sustained clock of each path's attention
# core (written from rocprofv3 runs of this script), valid while the core's
# sources are unchanged.
TRAFFIC_FILES = {"absorbed": os.path.join(ROOT, "profiles", "attend_core_wan_window_traffic.json"),
                 "expand": os.path.join(ROOT, "profiles", "attend_expand_wan_window_traffic.json")}
CORE_SOURCES = {
    "absorbed": ["rank_latent_kv_absorbed_amd/csrc/mla_attn_core.h",
                 "rank_latent_kv_absorbed_amd/csrc/mla_attend.hip",
                 "rank_latent_kv_absorbed_amd/csrc/mla_device.h",
                 "rank_latent_kv_absorbed_amd/csrc/mla_launch.h"],
    "expand": ["rank_latent_kv_absorbed_amd/csrc/mla_attn_core.h",
               "rank_latent_kv_absorbed_amd/csrc/mha_attend.hip",
               "rank_latent_kv_absorbed_amd/csrc/mla_expand.hip",
               "rank_latent_kv_absorbed_amd/csrc/mla_device.h",
               "rank_latent_kv_absorbed_amd/csrc/mla_launch.h"],
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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
        threads = HOST_CORES
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
    # the cache-bound case beside it: one query token of 8 sequences over the
    # full window (the oracle's explicit per-head rebuild of every key)
    sq_cfg = cfg.with_(batch=8)
    sq_store = O.round_storage(rng.standard_normal((8, cfg.window_frames * T, cfg.width)), cfg.cache_dtype)
    sq_ring = O.RingModel(cfg.window_frames, T)
    sq_ring.write(0, cfg.window_frames)
    sq_q = rng.standard_normal((8, 1, cfg.n_heads, cfg.d_qk))
    sq_times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        O.attend(sq_store, sq_ring, sq_q, cfg.window_frames * T - 1, wd["w_uk"], wd["w_uv"], sq_cfg)
        sq_times.append(time.perf_counter() - t0)
    t_sq = sorted(sq_times)[len(sq_times) // 2]
    return {
        "value": cfg.Lq / t_step, "unit": "query tokens/s per layer", "cores": int(threads),
        "kind": "oracle",
        "sample": (f"one full step at batch 1 (evict {cfg.chunk_frames} frames, cache write of "
                   f"{cfg.Lq} tokens, attention of {cfg.Lq} queries x {cfg.n_heads} heads over "
                   f"{cfg.window_frames * T} keys), fp64 NumPy oracle, median of {repeats} runs"),
        "seconds_measured": round(sum(times) + sum(sq_times), 2),
        "small_query": {"value": 8 / t_sq, "unit": "query tokens/s per layer",
                        "sample": (f"attention of 1 query x {cfg.n_heads} heads in each of 8 sequences over "
                                   f"{cfg.window_frames * T} keys, fp64 NumPy oracle, median of {repeats} runs")},
        "cpu_model": cpu_model(), "host_cores": HOST_CORES,
        "openblas_num_threads": os.environ.get("OPENBLAS_NUM_THREADS"),
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
    ap.add_argument("--no-extras", action="store_true",
                    help="only the headline step (no comparison or sweep cases)")
    ap.add_argument("--rollout", action="store_true",
                    help="full rollout sweep: batch 1/4/8/11 at every latent width (default "
                         "extras run batch 1 and 11)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device-to-device copy of this size first (a known-byte "
                         "kernel for scaling hardware traffic counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs the path on one GPU; --gpus must be 1",
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

    def make_caches(c_cfg, path):
        out_ = []
        for l in range(L):
            c = LatentCache(c_cfg, device=dev)
            c.set_attend_path(path)
            c.write(x_pre, weights[l]["w_dkr"], 0, W)
            out_.append(c)
        return out_

    caches = make_caches(cfg, args.path)
    path = caches[0].attend_path(Lq)
    out = torch.empty((B, Lq, cfg.n_heads, cfg.d_v), dtype=torch.float32, device=dev)
    ws = torch.empty(max(caches[0].workspace_bytes(Lq), 1), dtype=torch.uint8, device=dev)
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

    class Stepper:
        """Steps (evict, write, attend) cycling over one set of layer windows."""

        def __init__(self, cs, ws_):
            self.cs, self.ws, self.i = cs, ws_, 0
            self.newest = [c.info()["newest_frame"] for c in cs]

        def step(self, core_events=None):
            l = self.i % len(self.cs)
            self.i += 1
            c, w = self.cs[l], weights[l]
            c.evict(cfg.chunk_frames)
            f0 = self.newest[l] + 1
            c.write(x_chunk, w["w_dkr"], f0, cfg.chunk_frames)
            self.newest[l] = f0 + cfg.chunk_frames - 1
            if core_events is not None:
                c.set_profile_events(*core_events)
            c.attend(q, f0 * T, w["w_uk"], w["w_uv"], out=out, workspace=self.ws)
            if core_events is not None:
                c.set_profile_events(None, None)

        def timed(self, n_steps):
            """(ms per step, mean core-kernel ms) over n_steps steps; the
            per-step and per-launch times are kept in self.last."""
            core_ev = [(ev.create(), ev.create()) for _ in range(n_steps)]
            marks = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps + 1)]
            torch.cuda.synchronize()
            marks[0].record()
            for k in range(n_steps):
                self.step(core_ev[k])
                marks[k + 1].record()
            torch.cuda.synchronize()
            core_ms = [ev.elapsed_ms(a, b) for a, b in core_ev]
            self.last = {"step_ms": [marks[k].elapsed_time(marks[k + 1]) for k in range(n_steps)],
                         "core_ms": core_ms}
            return marks[0].elapsed_time(marks[n_steps]) / n_steps, sum(core_ms) / len(core_ms)

    main_steps = Stepper(caches, ws)
    for _ in range(args.warmup):
        main_steps.step()
    torch.cuda.synchronize()
    ms_step, core_avg = main_steps.timed(args.steps)

    def pct(v, p):
        v = sorted(v)
        return v[min(len(v) - 1, int(round(p / 100.0 * (len(v) - 1))))]
    spread = {k: [round(pct(v, p), 4) for p in (10, 50, 90)] for k, v in main_steps.last.items()}

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

    traffic, clock = None, None
    if os.path.exists(TRAFFIC_FILES[path]):
        tr = json.load(open(TRAFFIC_FILES[path]))
        if tr.get("kernel_source_sha") == core_source_sha(path) and tr.get("batch") == B:
            traffic = tr.get("hbm_bytes_per_launch")
            clock = tr.get("sustained_clock_ghz")

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "query tokens/s per layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"bf16 in; {cfg.cache_dtype} ring and {cfg.cache_dtype} MFMA operands, fp32 accumulation",
        "data": "synthetic",
        "config": {"workload": "wan_window: per layer, evict 3 frames + fused cache write of a "
                               "3-frame chunk + latent-KV attention of its queries over a 21-frame "
                               "window; 30 layer windows cycled",
                   "attend_path": path, "cache_dtype": cfg.cache_dtype,
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
                     "algorithmic_flop_per_launch": c_flop,
                     "sustained_clock_ghz": clock,
                     "frac_at_sustained_clock": (round(achieved / (PEAK_BF16_TFLOPS * clock / 2.4), 4)
                                                 if clock else None)},
        "step_flop": step_flop,
        "breakdown_ms": {"step": round(ms_step, 4), "attend_core": round(core_avg, 4)},
        "p10_p50_p90_ms": {"step": spread["step_ms"], "attend_core": spread["core_ms"]},
        "cache_bytes": {"latent_per_layer": caches[0].nbytes, "latent_30_layers": caches[0].nbytes * 30,
                        "dense_per_layer": None},
    }

    def log(name):
        print(f"[bench] {name} done at {time.perf_counter() - t_begin:.1f} s", file=sys.stderr, flush=True)

    t_begin = time.perf_counter()
    if not args.no_extras:
        run_extras(args, result, torch, dev, cfg, caches, weights, x_pre, x_chunk, q, out, ws, gen, ev,
                   Stepper, make_caches, core_avg, log,
                   (LatentCache, DenseCache, attend_flops, attend_bytes, mha_attend_flops, chunk_x,
                    dense_weights, layer_weights))

    ev.close()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, x_chunk_cpu, weights_cpu[0], q_cpu)
    print(json.dumps(result), flush=True)


def run_extras(args, result, torch, dev, cfg, caches, weights, x_pre, x_chunk, q, out, ws, gen, ev,
               Stepper, make_caches, core_avg, log, lib):
    (LatentCache, DenseCache, attend_flops, attend_bytes, mha_attend_flops, chunk_x, dense_weights,
     layer_weights) = lib
    B, T, Lq, W = cfg.batch, cfg.T, cfg.Lq, cfg.window_frames
    Lk = W * T
    L = args.layers
    path = caches[0].attend_path(Lq)

    def event_ms(fn, n):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # ---- measured bandwidth ceilings: a plain 1 GiB device copy (read + write)
    # and a 1 GiB read-only reduction
    buf = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(buf)
    acc = torch.empty((), dtype=torch.float32, device=dev)
    for _ in range(2):
        dst.copy_(buf)
        torch.sum(buf, dim=0, out=acc)
    copy_ms = event_ms(lambda i: dst.copy_(buf), 10)
    read_ms = event_ms(lambda i: torch.sum(buf, dim=0, out=acc), 10)
    result["hbm_measured"] = {"copy_GBps": round(2 * buf.numel() * 4 / (copy_ms / 1e3) / 1e9, 1),
                              "read_GBps": round(buf.numel() * 4 / (read_ms / 1e3) / 1e9, 1),
                              "how": "1 GiB torch copy (bytes read + written) and 1 GiB torch.sum "
                                     "(bytes read), mean of 10"}
    del buf, dst, acc
    log("bandwidth ceilings")

    # ---- the other attention path on the same steps
    other = "absorbed" if path == "expand" else "expand"
    try:
        for c in caches:
            c.set_attend_path(other)
    except Exception as e:          # the handle cannot take that path
        result["other_path"] = {"path": other, "error": str(e)}
    else:
        need = caches[0].workspace_bytes(Lq)
        ws2 = ws if need <= ws.numel() else torch.empty(need, dtype=torch.uint8, device=dev)
        st = Stepper(caches, ws2)
        for _ in range(5):
            st.step()
        o_step, o_core = st.timed(min(args.steps, 20))
        result["other_path"] = {"path": other, "ms_per_step": round(o_step, 4),
                                "attend_core_ms": round(o_core, 4),
                                "core_tflops": round(core_flop(cfg, other, B, Lq, Lk) / (o_core / 1e3) / 1e12, 1),
                                "value": round(B * Lq / (o_step / 1e3), 1)}
        for c in caches:
            c.set_attend_path(args.path)
        del ws2, st
    log("other path")

    # ---- the Wan-layer configuration: the chunk's queries over 9 resident
    # frames (6 earlier + the 3 of the chunk, 14 040 keys), attention only,
    # 30 layer windows cycled (each window narrowed to its newest 9 frames and
    # restored afterwards)
    saved = [c.info() for c in caches]
    for c, inf in zip(caches, saved):
        c.set_state(inf["newest_frame"] - 8, inf["newest_frame"])
    Lk9 = 9 * T
    p9 = caches[0].attend_path(Lq)

    def call9(i):
        l = i % L
        caches[l].attend(q, (saved[l]["newest_frame"] - 2) * T, weights[l]["w_uk"], weights[l]["w_uv"],
                         out=out, workspace=ws)

    for i in range(L):
        call9(i)
    ms9 = event_ms(call9, 2 * L)
    ev9 = [(ev.create(), ev.create()) for _ in range(2 * L)]
    for i, (a_, b_) in enumerate(ev9):
        caches[i % L].set_profile_events(a_, b_)
        call9(i)
        caches[i % L].set_profile_events(None, None)
    torch.cuda.synchronize()
    core9 = sum(ev.elapsed_ms(a_, b_) for a_, b_ in ev9) / len(ev9)
    for c, inf in zip(caches, saved):
        c.set_state(inf["oldest_frame"], inf["newest_frame"])
    f9 = core_flop(cfg, p9, B, Lq, Lk9)
    result["wan_layer_9_frames"] = {
        "path": p9, "resident_keys": Lk9, "attend_ms": round(ms9, 4), "attend_core_ms": round(core9, 4),
        "query_tokens_per_s": round(B * Lq / (ms9 / 1e3), 1),
        "core_frac": round(f9 / (core9 / 1e3) / (PEAK_BF16_TFLOPS * 1e12), 4),
        "mfma_util_pct_absorbed_form": round(100.0 * attend_flops(cfg.n_heads, Lq, Lk9, cfg.d_c, cfg.d_rope,
                                                                  cfg.d_nope, cfg.d_v, B)
                                             / (ms9 / 1e3) / (PEAK_BF16_TFLOPS * 1e12), 2)}
    log("wan layer, 9 frames")

    # ---- the same step with a bf16 ring, on its automatic path (the rebuild
    # multiplies the bf16 rows on bf16 matrix units into fp16 keys and values)
    # and on the absorbed path (split operands: query and probabilities as two
    # bf16 parts, twice the products)
    bcfg = cfg.with_(cache_dtype="bf16")
    bcaches = make_caches(bcfg, "absorbed")
    b_need = bcaches[0].workspace_bytes(Lq)
    bcaches[0].set_attend_path("auto")
    bws = torch.empty(max(b_need, bcaches[0].workspace_bytes(Lq), 1), dtype=torch.uint8, device=dev)
    bres = {}
    for bpath in ("auto", "absorbed"):
        for c in bcaches:
            c.set_attend_path(bpath)
        st = Stepper(bcaches, bws)
        for _ in range(5):
            st.step()
        b_step, b_core = st.timed(min(args.steps, 20))
        taken = bcaches[0].attend_path(Lq)
        b_flop = core_flop(bcfg, taken, B, Lq, Lk)
        r = {"path": taken, "ms_per_step": round(b_step, 4), "value": round(B * Lq / (b_step / 1e3), 1),
             "attend_core_ms": round(b_core, 4),
             "core_frac_algorithmic": round(b_flop / (b_core / 1e3) / (PEAK_BF16_TFLOPS * 1e12), 4)}
        if taken == "absorbed":
            r["core_frac_executed"] = round(2 * b_flop / (b_core / 1e3) / (PEAK_BF16_TFLOPS * 1e12), 4)
            r["note"] = ("bf16 MFMA on split operands: every score and value product is issued twice "
                         "(leading part and remainder), so executed matrix work is twice the algorithmic")
        else:
            r["note"] = "rebuild on bf16 MFMA into fp16 keys and values, then the fp16 per-head core"
        bres[bpath] = r
        del st
    result["bf16_ring"] = dict(bres["auto"], absorbed=bres["absorbed"]) if bres["auto"]["path"] != "absorbed" \
        else bres["absorbed"]
    del bcaches, bws
    torch.cuda.empty_cache()
    log("bf16 ring")

    # ---- the same step with a one-byte E4M3 ring (half the cache bytes),
    # on the handle's automatic path (the rebuild widens the rows)
    ecfg = cfg.with_(cache_dtype="e4m3")
    ecaches = make_caches(ecfg, "auto")
    ews = torch.empty(max(ecaches[0].workspace_bytes(Lq), 1), dtype=torch.uint8, device=dev)
    st = Stepper(ecaches, ews)
    for _ in range(5):
        st.step()
    e_step, e_core = st.timed(min(args.steps, 20))
    e_path = ecaches[0].attend_path(Lq)
    e_flop = core_flop(ecfg, e_path, B, Lq, Lk)
    result["e4m3_ring"] = {
        "path": e_path, "ms_per_step": round(e_step, 4), "value": round(B * Lq / (e_step / 1e3), 1),
        "attend_core_ms": round(e_core, 4),
        "core_frac": round(e_flop / (e_core / 1e3) / (PEAK_BF16_TFLOPS * 1e12), 4),
        "cache_bytes_per_layer": ecaches[0].nbytes,
        "note": "E4M3 storage (1 byte per scalar), widened to fp16 for the arithmetic"}
    del ecaches, ews, st
    torch.cuda.empty_cache()
    log("e4m3 ring")

    # ---- the same step with the query RMS norm set on every layer window
    # (gain 1 + 0.25 N(0, 1)): its cost over the plain step
    # Plain and normed steps alternate (three rounds each), so that clock
    # drift over the run does not enter the comparison.
    qn_gain = (1.0 + 0.25 * torch.randn(cfg.d_qk, generator=gen, device=dev)).to(torch.bfloat16)
    st = Stepper(caches, ws)
    timing = {False: [], True: []}
    for _ in range(3):
        for norm in (False, True):
            for c in caches:
                c.set_query_norm(qn_gain if norm else None, 1e-6)
            for _ in range(3):
                st.step()
            timing[norm].append(st.timed(min(args.steps, 10))[0])
    for c in caches:
        c.set_query_norm(None)
    qn_step, plain_step = min(timing[True]), min(timing[False])
    result["query_norm"] = {"ms_per_step": round(qn_step, 4), "value": round(B * Lq / (qn_step / 1e3), 1),
                            "plain_ms_per_step_alternating": round(plain_step, 4),
                            "overhead_pct": round(100.0 * (qn_step / plain_step - 1.0), 2), "path": path,
                            "note": "each head's query row RMS-normalised before the rotation and the fold; "
                                    "best of three rounds, alternating with plain steps"}
    del st
    log("query norm")

    # ---- several attends per written chunk (denoising steps): with reuse on,
    # the expand path rebuilds the window once per chunk
    if path == "expand":
        c = caches[0]
        newest = c.info()["newest_frame"]
        reuse = {}
        for flag in (False, True):
            c.set_expand_reuse(flag)
            for _ in range(3):
                c.attend(q, (newest - 2) * T, weights[0]["w_uk"], weights[0]["w_uv"], out=out, workspace=ws)
            reuse["reuse_on" if flag else "reuse_off"] = round(event_ms(
                lambda i: c.attend(q, (newest - 2) * T, weights[0]["w_uk"], weights[0]["w_uv"], out=out,
                                   workspace=ws), 10), 4)
        c.set_expand_reuse(False)
        result["attend_ms_repeated_on_one_window"] = reuse
    log("denoising reuse")

    # ---- dense per-head MHA on the same shape: 30 dense layer windows cycled
    # (6.04 GB), core kernel timed by the library's events
    dw = {k: v.to(dev) for k, v in dense_weights(cfg).items()}
    dcs = []
    for l in range(L):
        d = DenseCache(cfg, device=dev)
        d.write(x_pre, dw["w_k"], dw["w_v"], 0, W)
        dcs.append(d)
    dout = torch.empty((B, Lq, cfg.n_heads, cfg.d_qk), dtype=torch.float32, device=dev)
    dws = torch.empty(dcs[0].workspace_bytes(Lq), dtype=torch.uint8, device=dev)
    for i in range(3):
        dcs[i].attend(q, (W - 3) * T, out=dout, workspace=dws)
    dev_ev = [(ev.create(), ev.create()) for _ in range(L)]
    torch.cuda.synchronize()
    for i, (a_, b_) in enumerate(dev_ev):
        dcs[i].set_profile_events(a_, b_)
        dcs[i].attend(q, (W - 3) * T, out=dout, workspace=dws)
        dcs[i].set_profile_events(None, None)
    torch.cuda.synchronize()
    d_ms = sum(ev.elapsed_ms(a_, b_) for a_, b_ in dev_ev) / len(dev_ev)
    d_flop = mha_attend_flops(cfg.n_heads, Lq, Lk, cfg.d_qk, B)
    dense_layer = dcs[0].nbytes
    result["dense_mha"] = {"attend_core_ms": round(d_ms, 4), "layers_cycled": L,
                           "tflops": round(d_flop / (d_ms / 1e3) / 1e12, 2),
                           "cache_bytes_per_layer": dense_layer,
                           "latent_vs_dense_attend_time": round(core_avg / d_ms, 3),
                           "cache_bytes_ratio": round(dense_layer / caches[0].nbytes, 3)}
    result["cache_bytes"]["dense_per_layer"] = dense_layer
    del dcs, dws, dout
    torch.cuda.empty_cache()
    log("dense same shape")

    # ---- batch capacity (30 layers, 21-frame windows) of both caches in the
    # memory free on this GPU, and the dense attention at its largest batch
    result["batch_capacity"] = batch_capacity(torch, dev, cfg, W, T, Lq, L, x_chunk, q, dw, gen, ev,
                                              caches, DenseCache, LatentCache, mha_attend_flops, log)
    del dw
    torch.cuda.empty_cache()

    # ---- cache-bound small-query shapes: Lq queries per sequence over the full
    # window, latent widths 192 / 128 / 64, batch 8 and 11, 30 layer windows
    # cycled (1.5-4.8 GB of windows, far above the last-level cache); the
    # one-byte E4M3 ring at d_c = 192 (half the window bytes)
    host_gen = torch.Generator().manual_seed(5)

    def small_queries(sq, d_c, Bs, cache_dtype, suffix=""):
        scfg = cfg.with_(batch=Bs, d_c=d_c, cache_dtype=cache_dtype)
        sw = [{k: v.to(dev) for k, v in layer_weights(scfg, layer=l).items()} for l in range(2)]
        scaches = []
        staged = None
        for l in range(L):
            c = LatentCache(scfg, device=dev)
            r = c.ring()
            if r.dtype == torch.float8_e4m3fn:
                # Gaussian values rounded to E4M3 on the host, staged once
                if staged is None:
                    staged = torch.randn(r.shape, generator=host_gen).to(r.dtype).view(torch.uint8).to(dev)
                r.view(torch.uint8).copy_(staged)
            else:
                r.copy_(torch.randn(r.shape, generator=gen, device=dev).to(r.dtype))
            c.set_state(0, W - 1)
            scaches.append(c)
        del staged
        elem = scaches[0].ring().element_size()
        for Lqs in (1, 4, 8):
            qs = torch.randn((Bs, Lqs, cfg.n_heads, cfg.d_qk), generator=gen, device=dev).to(torch.bfloat16)
            so = torch.empty((Bs, Lqs, cfg.n_heads, cfg.d_v), dtype=torch.float32, device=dev)
            sws = torch.empty(max(scaches[0].workspace_bytes(Lqs), 1), dtype=torch.uint8, device=dev)

            def call(i):
                scaches[i % L].attend(qs, Lk - Lqs, sw[i % 2]["w_uk"], sw[i % 2]["w_uv"], out=so,
                                      workspace=sws)

            for i in range(L):
                call(i)
            call_ms = event_ms(call, 2 * L)
            sev = [(ev.create(), ev.create()) for _ in range(2 * L)]
            for i, (a_, b_) in enumerate(sev):
                c = scaches[i % L]
                c.set_profile_events(a_, b_)
                call(i)
                c.set_profile_events(None, None)
            torch.cuda.synchronize()
            kms = sum(ev.elapsed_ms(a_, b_) for a_, b_ in sev) / len(sev)
            win = Bs * Lk * (d_c + cfg.d_rope) * elem
            nbytes = attend_bytes(cfg.n_heads, Lqs, Lk, d_c, cfg.d_rope, cfg.d_nope, cfg.d_v, Bs,
                                  cache_elem=elem)
            sq[f"dc{d_c}_Lq{Lqs}_B{Bs}{suffix}"] = {
                "attend_ms": round(call_ms, 4), "core_kernel_ms": round(kms, 4),
                "algorithmic_bytes": nbytes,
                "core_GBps": round(win / (kms / 1e3) / 1e9, 1),
                "call_GBps": round(nbytes / (call_ms / 1e3) / 1e9, 1),
                "hbm_frac_call": round(nbytes / (call_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                "query_tokens_per_s": round(Bs * Lqs / (call_ms / 1e3), 1)}
            del sws, so, qs
        del scaches, sw
        torch.cuda.empty_cache()

    sq = {}
    for d_c in (192, 128, 64):
        for Bs in (8, 11):
            small_queries(sq, d_c, Bs, cfg.cache_dtype)
    sq8 = {}
    for Bs in (8, 11):
        small_queries(sq8, 192, Bs, "e4m3", "_e4m3")
    for k, v in sq8.items():
        base = sq.get(k[:-len("_e4m3")])
        if base is not None:
            v["speedup_vs_2byte_ring"] = round(base["attend_ms"] / v["attend_ms"], 3)
    result["small_query_e4m3"] = sq8
    result["small_query_cache_bound"] = sq
    log("small queries")

    # ---- batch scaling of the chunk step (evict + write + attend) over 30
    # layer windows per batch size
    scale = {}
    for Bb in (1, 2, 4, 8):
        bcfg = cfg.with_(batch=Bb)
        bx = torch.randn((Bb, W * T, cfg.hidden), generator=gen, device=dev).to(torch.bfloat16)
        bxc = bx[:, :Lq].contiguous()
        bq = torch.randn((Bb, Lq, cfg.n_heads, cfg.d_qk), generator=gen, device=dev).to(torch.bfloat16)
        bcs = []
        for l in range(L):
            c = LatentCache(bcfg, device=dev)
            c.set_attend_path(args.path)
            c.write(bx, weights[l]["w_dkr"], 0, W)
            bcs.append(c)
        del bx
        bnew = [W - 1] * L
        bout = torch.empty((Bb, Lq, cfg.n_heads, cfg.d_v), dtype=torch.float32, device=dev)
        bws = torch.empty(max(bcs[0].workspace_bytes(Lq), 1), dtype=torch.uint8, device=dev)

        def bstep(k):
            l = k % L
            c = bcs[l]
            c.evict(cfg.chunk_frames)
            f0 = bnew[l] + 1
            c.write(bxc, weights[l]["w_dkr"], f0, cfg.chunk_frames)
            bnew[l] = f0 + cfg.chunk_frames - 1
            c.attend(bq, f0 * T, weights[l]["w_uk"], weights[l]["w_uv"], out=bout, workspace=bws)

        for k in range(4):
            bstep(k)
        n_b = 30 if Bb <= 2 else 15
        b_ms = event_ms(lambda k: bstep(k + 4), n_b)
        bflop = (attend_flops(cfg.n_heads, Lq, Lk, cfg.d_c, cfg.d_rope, cfg.d_nope, cfg.d_v, Bb)
                 + 2 * Bb * Lq * cfg.hidden * cfg.width)
        scale[f"B{Bb}"] = {"ms_per_step": round(b_ms, 4),
                           "query_tokens_per_s": round(Bb * Lq / (b_ms / 1e3), 1),
                           "path": bcs[0].attend_path(Lq), "layers_cycled": L,
                           "mfma_util_pct_absorbed_form": round(100.0 * bflop / (b_ms / 1e3)
                                                                / (PEAK_BF16_TFLOPS * 1e12), 2)}
        del bcs, bws, bout, bq, bxc
        torch.cuda.empty_cache()
    result["batch_scaling"] = scale
    log("batch scaling")

    # ---- rollout: 80 chunks of 3 frames through every layer's 21-frame window
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

        def chunk(k):
            for l in range(L):
                c = rcs[l]
                res = 0 if k == 0 else min(3 * k, W)
                c.evict(max(0, res + cfg.chunk_frames - W))
                c.write(rx, rw[l]["w_dkr"], 3 * k, cfg.chunk_frames)
                c.attend(rq, 3 * k * T, rw[l]["w_uk"], rw[l]["w_uv"], out=rout, workspace=rws)

        ms = event_ms(chunk, n_chunks) * n_chunks
        frames = sum(min(3 * (k + 1), W) for k in range(n_chunks))
        flop = L * (sum(attend_flops(cfg.n_heads, Lq, min(3 * (k + 1), W) * T, d_c, cfg.d_rope,
                                     cfg.d_nope, cfg.d_v, Bb) for k in range(n_chunks))
                    + n_chunks * 2 * Bb * Lq * cfg.hidden * (d_c + cfg.d_rope))
        res_ = {"ms_total": round(ms, 2), "chunks": n_chunks, "layers": L, "batch": Bb, "d_c": d_c,
                "path": rcs[0].attend_path(Lq), "resident_frames_summed": frames,
                "query_tokens_per_s_per_layer": round(Bb * Lq * n_chunks * L / (ms / 1e3), 1),
                "mfma_util_pct_absorbed_form": round(100.0 * flop / (ms / 1e3) / (PEAK_BF16_TFLOPS * 1e12), 2)}
        del rcs, rws, rout, rw, rx, rq
        torch.cuda.empty_cache()
        return res_

    batches = (1, 4, 8, 11) if args.rollout else (1, 11)
    result["rollout"] = {}
    for d in (192, 128, 64):
        for b_ in batches:
            result["rollout"][f"dc{d}_B{b_}"] = rollout(d, b_)
            log(f"rollout d_c={d} B={b_}")


def batch_capacity(torch, dev, cfg, W, T, Lq, L, x_chunk, q, dw, gen, ev, caches, DenseCache, LatentCache,
                   mha_attend_flops, log):
    """How many sequences' 30-layer, 21-frame caches fit in the memory free on
    the GPU (after this process's other allocations are released), for the
    dense per-head cache and the latent cache, cache storage only and with the
    4680-query attention workspace of one layer call; then the dense MHA runs
    at its largest batch with all 30 of its layer caches allocated."""
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    free, total = torch.cuda.mem_get_info(dev)
    reserve = 4 << 30          # held back for the runtime and the step's inputs and outputs
    usable = free - reserve
    per_seq = {}
    for kind, cls in (("dense", DenseCache), ("latent", LatentCache)):
        c1 = cls(cfg.with_(batch=1), device=dev)
        c8 = cls(cfg.with_(batch=8), device=dev)
        c1.set_state(0, W - 1)
        c8.set_state(0, W - 1)
        w1, w8 = c1.workspace_bytes(Lq), c8.workspace_bytes(Lq)
        per_seq[kind] = {"cache_bytes_30_layers": 30 * c1.nbytes, "workspace_per_seq": (w8 - w1) / 7,
                         "workspace_fixed": w1 - (w8 - w1) / 7}
        del c1, c8
    out = {"free_bytes_measured": free, "total_bytes": total, "reserve_bytes": reserve}
    for kind, p in per_seq.items():
        cache_only = int(usable // p["cache_bytes_30_layers"])
        with_ws = int((usable - p["workspace_fixed"]) // (p["cache_bytes_30_layers"] + p["workspace_per_seq"]))
        out[kind] = {"cache_bytes_30_layers_per_seq": p["cache_bytes_30_layers"],
                     "attend_workspace_per_seq": int(p["workspace_per_seq"]),
                     "max_batch_cache_only": cache_only, "max_batch_with_workspace": with_ws}
    out["ratio_cache_only"] = round(out["latent"]["max_batch_cache_only"] / max(1, out["dense"]["max_batch_cache_only"]), 2)
    out["ratio_with_workspace"] = round(out["latent"]["max_batch_with_workspace"]
                                        / max(1, out["dense"]["max_batch_with_workspace"]), 2)
    out["pages_ratio"] = PAGES_BATCH_RATIO
    out["pages_note"] = ("the pages' 8.0x (d_c = 192) was measured on a B200 under a fixed memory "
                         "budget of a whole video model; the ratios here count 30 attention layers' "
                         "caches (and the attention workspace) only")
    log("capacity")

    # the dense MHA at its largest batch: every one of its 30 layer caches
    # allocated, the first layer's window written, its attention timed
    Bd = out["dense"]["max_batch_with_workspace"]
    dcfg = cfg.with_(batch=Bd)
    try:
        layers = []
        for l in range(30):
            layers.append(DenseCache(dcfg, device=dev))
        d0 = layers[0]
        xb = x_chunk[:1].expand(Bd, -1, -1).contiguous()
        for f0 in range(0, W, 3):
            d0.write(xb, dw["w_k"], dw["w_v"], f0, 3)
        qb = q[:1].expand(Bd, -1, -1, -1).contiguous()
        dout = torch.empty((Bd, Lq, cfg.n_heads, cfg.d_qk), dtype=torch.float32, device=dev)
        dws = torch.empty(d0.workspace_bytes(Lq), dtype=torch.uint8, device=dev)
        d0.attend(qb, (W - 3) * T, out=dout, workspace=dws)
        e = [(ev.create(), ev.create()) for _ in range(3)]
        torch.cuda.synchronize()
        for a_, b_ in e:
            d0.set_profile_events(a_, b_)
            d0.attend(qb, (W - 3) * T, out=dout, workspace=dws)
            d0.set_profile_events(None, None)
        torch.cuda.synchronize()
        ms = sum(ev.elapsed_ms(a_, b_) for a_, b_ in e) / len(e)
        flop = mha_attend_flops(cfg.n_heads, Lq, W * T, cfg.d_qk, Bd)
        out["dense_at_max_batch"] = {
            "batch": Bd, "layers_allocated": 30,
            "bytes_allocated": sum(x.nbytes for x in layers) + dws.numel() + dout.numel() * 4,
            "attend_core_ms_one_layer": round(ms, 3),
            "query_tokens_per_s_per_layer": round(Bd * Lq / (ms / 1e3), 1),
            "tflops": round(flop / (ms / 1e3) / 1e12, 1)}
        del layers, d0, xb, qb, dout, dws
    except torch.cuda.OutOfMemoryError as e:
        out["dense_at_max_batch"] = {"batch": Bd, "error": f"out of memory: {e}"[:300]}
    torch.cuda.empty_cache()
    log("dense at max batch")
    return out


if __name__ == "__main__":
    main()
