"""CPU tests of the C ABI: the built library loads and exports every function
include/mla.h declares, and the host logic (validation, window bookkeeping,
launch arguments, workspace sizes, error codes) is checked against the
oracle's ring model.  Host logic runs from the same mla_host.cpp compiled with
g++ against a recording launcher (tests/hostsim/fake_launch.cpp), so no GPU
and no kernel is involved.
"""

import ctypes
import math
import os
import re
import subprocess

import numpy as np
import pytest

from oracle import mla as O
from synthetic import config

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")
CSRC = os.path.join(ROOT, "rank_latent_kv_absorbed_amd", "csrc")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b((?:mla|mha)_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def real_lib():
    from rank_latent_kv_absorbed_amd import mla as binding
    if not os.path.exists(binding.LIB_PATH):
        from rank_latent_kv_absorbed_amd import build
        build.build()
    return ctypes.CDLL(binding.LIB_PATH)


def test_library_exports_every_declared_function(real_lib):
    names = header_functions()
    assert len(names) >= 17
    for n in names:
        assert hasattr(real_lib, n), n
    from rank_latent_kv_absorbed_amd.mla import SIGNATURES
    assert sorted(SIGNATURES) == names


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from rank_latent_kv_absorbed_amd import mla as binding
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(binding, "_lib", None)
    with pytest.raises(binding.LibraryMissing):
        binding.lib()


# --------------------------------------------------------------------------
# host logic against the recording launcher
# --------------------------------------------------------------------------

@pytest.fixture(scope="module")
def sim(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("hostsim") / "libmla_hostsim.so")
    cmd = ["g++", "-O1", "-std=c++17", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(CSRC, "mla_host.cpp"), os.path.join(ROOT, "tests", "hostsim", "fake_launch.cpp"),
           "-o", out]
    # MLA_HOSTSIM_SANITIZE=1 builds the host library with AddressSanitizer and
    # UBSan (run with the sanitizer runtimes in LD_PRELOAD, e.g.
    # LD_PRELOAD=$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so)
    # ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1).
    if os.environ.get("MLA_HOSTSIM_SANITIZE"):
        cmd[1:1] = ["-g", "-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
    subprocess.run(cmd, check=True, capture_output=True)
    L = ctypes.CDLL(out)
    from rank_latent_kv_absorbed_amd.mla import SIGNATURES
    for name, (res, args) in SIGNATURES.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    L.fake_attend_qscale.restype = ctypes.c_float
    L.fake_qnorm_gamma.restype = ctypes.c_longlong
    L.fake_qnorm_eps.restype = ctypes.c_float
    return L


FAKE_STORAGE = 1 << 40          # host never dereferences storage; any aligned address works
FAKE_PTR = 1 << 41


def _cfg(name="wan_window", **kw):
    from rank_latent_kv_absorbed_amd.mla import make_config
    return make_config(config(name, **kw))


def _create(L, c, dense=False, nbytes=None):
    from rank_latent_kv_absorbed_amd.mla import _HANDLE
    h = _HANDLE()
    size = (L.mha_cache_bytes if dense else L.mla_cache_bytes)(ctypes.byref(c))
    st = (L.mha_cache_create if dense else L.mla_cache_create)(
        ctypes.byref(c), ctypes.c_void_p(FAKE_STORAGE), size if nbytes is None else nbytes,
        ctypes.byref(h))
    return st, h


def _info(L, h):
    from rank_latent_kv_absorbed_amd.mla import CacheInfoC
    i = CacheInfoC()
    assert L.mla_cache_query(h, ctypes.byref(i)) == 0
    return i.oldest_frame, i.newest_frame, i.n_resident_frames, i.capacity_frames


def _write_info(L):
    a = (ctypes.c_longlong * 10)()
    L.fake_write_info(a)
    return list(a)


def _attend_info(L):
    a = (ctypes.c_longlong * 20)()
    L.fake_attend_info(a)
    keys = ["key_slot0", "Lk", "B", "Lq", "q_token0", "ring_rows", "n_h", "d_c", "n_rg", "n_kt",
            "n_groups", "n_blocks", "full_rounds", "rem", "main_len", "tpb", "n_slots",
            "block_rows", "key_tile", "stages"]
    return dict(zip(keys, list(a)))


def _mha_info(L):
    a = (ctypes.c_longlong * 17)()
    L.fake_mha_info(a)
    keys = ["key_slot0", "Lk", "B", "Lq", "q_token0", "n_rg", "n_kt", "n_groups", "n_blocks",
            "full_rounds", "rem", "main_len", "tpb", "n_slots", "block_rows", "key_tile",
            "stages"]
    return dict(zip(keys, list(a)))


# Core shapes (block rows, key tile, LDS stages) by rows per row unit, and how
# many blocks of each fit one compute unit (stages LDS tiles of
# key_tile * chunks * 16 bytes in 160 KiB; at most eight waves, or four for
# the split-operand cores of a bf16 ring, whose chunk shape has four waves).
def expected_shape(rows, chunks_per_key=28, split=False):
    if rows <= 16:
        br, kt, ns, waves = 16, 32, 2, 1                # one wave of 16 rows (16x16x32 MFMAs)
    elif rows <= 32:
        br, kt, ns, waves = 32, 32, 2, 1
    elif rows <= 64:
        br, kt, ns, waves = 64, 32, 4, 4               # four waves of 16 rows
    elif rows <= 128:
        br, kt, ns, waves = 128, 32, 4, 4
    elif split:
        br, kt, ns, waves = 128, 64, 3, 4
    else:
        br, kt, ns, waves = 256, 64, 3, 8
    spans = kt * chunks_per_key // 64 // waves         # tile loads per wave
    return br, kt, min(ns, 1 + 63 // spans)           # in-flight loads fit a 6-bit counter


def blocks_per_cu(shape, chunks_per_key, split=False):
    br, kt, ns = shape
    waves = 1 if br <= 32 else (4 if br == 64 else br // 32)
    return min(160 * 1024 // (ns * kt * chunks_per_key * 16), (4 if split else 8) // waves)


# Steps charged per segment start by the library's schedule (latent, dense).
SEG_COST = (3, 6)


def _block_segments(L, which, g, n):
    out = (ctypes.c_int * 5)()
    k = 0
    for i in range(n):
        L.fake_sched_decode(which, g, i, out)
        k += out[3]
    return k


def check_schedule(L, info, R, which=0):
    """Walk the last attend's schedule exactly as the kernel decodes it: every
    (row group, key tile) step runs once; each block's steps form segments
    flagged first/last; a group's segments use slots 0..k-1 with k the count
    the merge reads, k <= the workspace's slot count; block work is balanced."""
    n_rg, n_kt, nb = info["n_rg"], info["n_kt"], info["n_blocks"]
    br, kt = info["block_rows"], info["key_tile"]
    assert n_rg == -(-R // br) and n_kt == -(-info["Lk"] // kt)
    groups = info["B"] * n_rg
    seen = np.zeros((groups, n_kt), np.int32)
    slots = {}
    out = (ctypes.c_int * 5)()
    steps = [L.fake_sched_steps(which, g) for g in range(nb)]
    for g in range(nb):
        prev = None
        for i in range(steps[g]):
            L.fake_sched_decode(which, g, i, out)
            grp, kt, slot, first, last = list(out)
            seen[grp, kt] += 1
            if prev is None or prev[4]:
                assert first, (g, i)
                slots.setdefault(grp, set()).add(slot)
            else:
                assert not first and grp == prev[0] and kt == prev[1] + 1 and slot == prev[2]
            prev = (grp, kt, slot, first, last)
        assert prev is None or prev[4]
    assert (seen == 1).all()
    for grp in range(groups):
        k = L.fake_sched_group_slots(which, grp)
        assert slots[grp] == set(range(k)) and k <= info["n_slots"]
    # balanced once every segment start counts SEG_COST[which] steps
    seg_cost = SEG_COST[which]
    segs = [L.fake_sched_steps(which, g) and _block_segments(L, which, g, steps[g]) for g in range(nb)]
    busy = [s for s in steps if s > 0]
    assert max(busy) <= -(-groups * n_kt // nb) + seg_cost * max(segs) + 1
    costs = [s + seg_cost * k for s, k in zip(steps, segs) if s > 0]
    # (every data-parallel round adds one segment start to every block)
    assert max(costs) <= min(max(busy), -(-groups * n_kt // nb)) + (2 + info["full_rounds"]) * seg_cost + 1
    # the kernels walk the same steps incrementally
    assert L.fake_sched_cursor_mismatches(which) == 0


P = ctypes.c_void_p


def test_cache_bytes_closed_forms(sim):
    c = _cfg()
    assert sim.mla_cache_bytes(ctypes.byref(c)) == 14_676_480
    assert sim.mha_cache_bytes(ctypes.byref(c)) == 201_277_440
    c.batch = 8
    assert sim.mla_cache_bytes(ctypes.byref(c)) == 8 * 14_676_480
    c.batch, c.d_c = 1, 64
    assert sim.mla_cache_bytes(ctypes.byref(c)) == 6_289_920
    t = _cfg("tiny")
    assert sim.mla_cache_bytes(ctypes.byref(t)) == 3 * 16 * 24 * 4


def test_invalid_configs_rejected(sim):
    for field, val in (("d_rope", 7), ("rope_pairs_t", 5), ("hidden", 0), ("window_frames", 0),
                       ("dtype", 3), ("batch", -1), ("grid_w", 0)):
        c = _cfg()
        setattr(c, field, val)
        assert sim.mla_cache_bytes(ctypes.byref(c)) == 0, field
        st, _ = _create(sim, c, nbytes=1 << 30)
        assert st == 1, field
    c = _cfg()
    st, _ = _create(sim, c, nbytes=14_676_480 - 1)
    assert st == 2
    # one sequence's ring must stay below 2^31 elements (32-bit offsets in the kernels)
    c = _cfg(window_frames=6146)                   # 9 587 760 rows x 224 >= 2^31
    assert sim.mla_cache_bytes(ctypes.byref(c)) == 0
    c = _cfg(window_frames=6145)                   # 9 586 200 rows x 224 < 2^31
    assert sim.mla_cache_bytes(ctypes.byref(c)) == 9_586_200 * 224 * 2
    c = _cfg(window_frames=449)                    # dense: 700 440 rows x 3072 > 2^31
    assert sim.mha_cache_bytes(ctypes.byref(c)) == 0
    c = _cfg(window_frames=448)
    assert sim.mha_cache_bytes(ctypes.byref(c)) == 448 * 1560 * 3072 * 2


def test_rollout_schedule_matches_ring_model(sim):
    """80 chunks of 3 frames through a 21-frame window: window state, write
    launch arguments, attend key range and slot map agree with the oracle."""
    c = _cfg()
    st, h = _create(sim, c)
    assert st == 0 and sim.mla_cache_set_attend_path(h, 1) == 0
    ring = O.RingModel(21, 1560)
    for k in range(80):
        n_ev = max(0, ring.n_resident + 3 - 21)
        assert sim.mla_cache_evict(h, n_ev) == 0
        ring.evict(n_ev)
        assert sim.mla_cache_write(h, P(FAKE_PTR), P(FAKE_PTR), 3 * k, 3, None) == 0
        ring.write(3 * k, 3)
        w = _write_info(sim)
        assert w[:8] == [3 * k, 3 * 1560, 3 * 1560, 224, 21 * 1560, 192, 224, 32]
        assert _info(sim, h) == (ring.oldest, ring.newest, ring.n_resident, 21)
        assert sim.mla_attend(h, P(FAKE_PTR), 3 * k * 1560, 4680, P(FAKE_PTR), P(FAKE_PTR),
                              P(FAKE_PTR), 0, P(FAKE_PTR), 1 << 40, None) == 0
        a = _attend_info(sim)
        slots = ring.resident_slots()
        assert a["key_slot0"] == slots[0] and a["Lk"] == len(slots)
        # keys are the contiguous (mod ring) run of slots starting at key_slot0
        np.testing.assert_array_equal((a["key_slot0"] + np.arange(a["Lk"])) % (21 * 1560), slots)
        for f in (ring.oldest, ring.newest):
            for tau in (0, 777, 1559):
                assert sim.mla_cache_slot(h, f, tau) == ring.slot(f, tau)
    sim.mla_cache_destroy(h)


def test_write_errors_leave_state_unchanged(sim):
    c = _cfg()
    st, h = _create(sim, c)
    assert sim.mla_cache_write(h, P(FAKE_PTR), P(FAKE_PTR), 10, 18, None) == 0
    before = _info(sim, h)
    n = sim.fake_count()
    assert sim.mla_cache_write(h, P(FAKE_PTR), P(FAKE_PTR), 28, 4, None) == 3     # full
    assert sim.mla_cache_write(h, P(FAKE_PTR), P(FAKE_PTR), 29, 1, None) == 4     # gap
    assert sim.mla_cache_write(h, P(FAKE_PTR), P(FAKE_PTR), 27, 1, None) == 4     # overlap
    assert sim.mla_cache_write(h, P(FAKE_PTR), P(FAKE_PTR), 28, 0, None) == 1
    assert sim.mla_cache_write(h, P(FAKE_PTR + 2), P(FAKE_PTR), 28, 1, None) == 1  # misaligned
    assert sim.mla_cache_write(h, None, P(FAKE_PTR), 28, 1, None) == 1
    assert sim.mla_cache_evict(h, 19) == 5
    assert sim.mla_cache_evict(h, -1) == 5
    assert _info(sim, h) == before and sim.fake_count() == n
    # a launch failure is reported and does not commit the frames
    sim.fake_fail_next()
    assert sim.mla_cache_write(h, P(FAKE_PTR), P(FAKE_PTR), 28, 3, None) == 10
    assert _info(sim, h) == before
    assert sim.mla_cache_write(h, P(FAKE_PTR), P(FAKE_PTR), 28, 3, None) == 0
    assert _info(sim, h) == (10, 30, 21, 21)
    # empty window: attend refuses, a write may start anywhere
    assert sim.mla_cache_evict(h, 21) == 0
    assert sim.mla_attend(h, P(FAKE_PTR), 0, 16, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR), 0,
                          P(FAKE_PTR), 1 << 40, None) == 6
    assert sim.mla_cache_write(h, P(FAKE_PTR), P(FAKE_PTR), 500, 2, None) == 0
    assert _info(sim, h)[:3] == (500, 501, 2)


def test_attend_arguments_and_workspace(sim):
    c = _cfg()
    st, h = _create(sim, c)
    assert sim.mla_cache_set_state(h, 3, 23) == 0
    assert sim.mla_cache_set_attend_path(h, 1) == 0
    need = sim.mla_attend_workspace_bytes(h, 4680, 0)
    R = 4680 * 12
    assert need >= R * 224 * 2 + R * 192 * 4 + R * 8
    ws = 1 << 40
    assert sim.mla_attend(h, P(FAKE_PTR), 21 * 1560, 4680, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR),
                          0, P(ws), 256, None) == 7
    assert sim.mla_attend(h, P(FAKE_PTR), 21 * 1560, 4680, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR),
                          0, P(ws + 64), need, None) == 7                      # misaligned
    assert sim.mla_attend(h, P(FAKE_PTR), 21 * 1560, 4680, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR),
                          0, P(ws), need, None) == 0
    a = _attend_info(sim)
    assert a["key_slot0"] == (3 % 21) * 1560 and a["Lk"] == 21 * 1560 and a["Lq"] == 4680
    assert a["q_token0"] == 21 * 1560
    assert sim.fake_attend_qscale() == np.float32(math.log2(math.e) / math.sqrt(128))
    # full window, one sequence: 220 main blocks walk key tiles 0..442 in
    # lockstep, 36 tail blocks share tiles 443..511 of every group, 422 each
    # (a tail run starts about 7 segments, 3 steps each, so it gets fewer
    # tiles than the 440 of an even split)
    assert (a["block_rows"], a["key_tile"]) == (256, 64)
    assert (a["n_blocks"], a["n_rg"], a["n_kt"], a["rem"], a["main_len"], a["tpb"]) == \
        (256, 220, 512, 220, 443, 422)
    check_schedule(sim, a, R)
    # forced key splits: every row group gets about that many pieces
    for s in (1, 2, 7, 64):
        need = sim.mla_attend_workspace_bytes(h, 8, s)
        assert sim.mla_attend(h, P(FAKE_PTR), 0, 8, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR), s,
                              P(ws), need, None) == 0
        a = _attend_info(sim)
        assert a["n_blocks"] == a["n_groups"] * s
        check_schedule(sim, a, 8 * 12)
    # small and large query counts: narrow blocks on short key tiles for a few
    # rows, several per compute unit; at least 8 key tiles per block
    for Lq in (1, 2, 3, 8, 10, 11, 100, 4680):
        assert sim.mla_attend(h, P(FAKE_PTR), 0, Lq, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR), 0,
                              P(ws), 1 << 40, None) == 0
        a = _attend_info(sim)
        shape = expected_shape(Lq * 12)
        assert (a["block_rows"], a["key_tile"], a["stages"]) == shape
        check_schedule(sim, a, Lq * 12)
        resident = 256 * blocks_per_cu(shape, 224 // 8)
        assert a["n_blocks"] == min(resident, -(-a["n_groups"] * a["n_kt"] // 8))


def _expand_info(L):
    a = (ctypes.c_longlong * 13)()
    L.fake_expand_info(a)
    keys = ["B", "ring_rows", "key_slot0", "Lk", "n_h", "d_nope", "d_rope", "d_c", "d_v",
            "cache_type", "kv", "ring", "w_uk"]
    return dict(zip(keys, list(a)))


def _mha_ptrs(L):
    a = (ctypes.c_longlong * 10)()
    L.fake_mha_ptrs(a)
    return dict(zip(["ring_rows", "d_h", "ring", "qrot", "opart", "ml", "q", "out", "qscale_u",
                     "qrot_lo"], list(a)))


def _attend_ptrs(L):
    a = (ctypes.c_longlong * 4)()
    L.fake_attend_ptrs(a)
    return dict(zip(["qcat", "qcat_lo", "opart", "ml"], list(a)))


def test_bf16_ring_split_operands_and_fp16_expansion(sim):
    """A bf16 ring runs the absorbed core on split operands: the workspace
    carries the query remainders after the queries and the chunk shape has
    four waves (one per SIMD).  Its expansion rebuilds into the same fp16
    window as an fp16 ring's, so the per-head attention behind it takes plain
    operands (no remainders, the 8-wave chunk shape).  fp16 rings do not
    split."""
    ws = 1 << 40
    for cache_dtype in ("bf16", "f16"):
        split = cache_dtype == "bf16"
        st, h = _create(sim, _cfg(cache_dtype=cache_dtype))
        assert st == 0 and sim.mla_cache_set_state(h, 3, 23) == 0
        assert sim.mla_attend_path(h, 4680, 0) == 2
        need = sim.mla_attend_workspace_bytes(h, 4680, 0)
        assert sim.mla_attend(h, P(FAKE_PTR), 21 * 1560 - 4680, 4680, P(FAKE_PTR), P(FAKE_PTR),
                              P(FAKE_PTR), 0, P(ws), need, None) == 0
        a, p = _mha_info(sim), _mha_ptrs(sim)
        assert (a["block_rows"], a["key_tile"], a["stages"]) == expected_shape(4680, 32, False)
        assert p["qrot_lo"] == 0
        t = (ctypes.c_int * 5)()
        sim.fake_type_info(t)
        assert t[3] == (1 if split else 2) and t[4] == 2
        assert sim.mla_cache_set_attend_path(h, 2) == 0
        assert sim.mla_cache_set_attend_path(h, 1) == 0
        for Lq in (1, 4, 8, 11, 100, 4680):
            R = Lq * 12
            need = sim.mla_attend_workspace_bytes(h, Lq, 0)
            assert sim.mla_attend(h, P(FAKE_PTR), 21 * 1560, Lq, P(FAKE_PTR), P(FAKE_PTR),
                                  P(FAKE_PTR), 0, P(ws), need, None) == 0
            a = _attend_info(sim)
            shape = expected_shape(R, split=split)
            assert (a["block_rows"], a["key_tile"], a["stages"]) == shape, (cache_dtype, Lq)
            check_schedule(sim, a, R)
            resident = 256 * blocks_per_cu(shape, 224 // 8, split)
            assert a["n_blocks"] == min(resident, -(-a["n_groups"] * a["n_kt"] // 8))
            p = _attend_ptrs(sim)
            qbytes = -(-R * 224 * 2 // 256) * 256
            assert p["qcat"] == ws
            if split:
                assert p["qcat_lo"] == ws + qbytes and p["opart"] == ws + 2 * qbytes
            else:
                assert p["qcat_lo"] == 0 and p["opart"] == ws + qbytes
            slots = a["n_slots"]
            assert p["ml"] == p["opart"] + -(-slots * R * 192 * 4 // 256) * 256
            assert need >= p["ml"] - ws + slots * R * 8
        st, d = _create(sim, _cfg(cache_dtype=cache_dtype), dense=True)
        assert sim.mla_cache_set_state(d, 0, 20) == 0
        for Lq in (1, 40, 129, 4680):
            need = sim.mha_attend_workspace_bytes(d, Lq)
            assert sim.mha_attend(d, P(FAKE_PTR), 0, Lq, P(FAKE_PTR), P(ws), need, None) == 0
            a, p = _mha_info(sim), _mha_ptrs(sim)
            shape = expected_shape(Lq, 32, split)
            assert (a["block_rows"], a["key_tile"], a["stages"]) == shape
            lq_pad = -(-Lq // shape[0]) * shape[0]
            qbytes = -(-12 * lq_pad * 128 * 2 // 256) * 256
            assert p["qrot"] == ws
            assert p["qrot_lo"] == (ws + qbytes if split else 0)
            assert p["opart"] == ws + (2 if split else 1) * qbytes
            check_schedule(sim, a, 12 * lq_pad, which=1)


def test_attend_path_choice(sim):
    c = _cfg()
    st, h = _create(sim, c)
    assert st == 0 and sim.mla_cache_set_state(h, 0, 20) == 0
    # automatic: long chunks expand, short ones and forced key splits stay absorbed
    assert sim.mla_attend_path(h, 4680, 0) == 2
    assert sim.mla_attend_path(h, 511, 0) == 1 and sim.mla_attend_path(h, 512, 0) == 2
    assert sim.mla_attend_path(h, 4680, 3) == 1
    assert sim.mla_attend_path(h, 0, 0) == -1 and sim.mla_attend_path(h, 8, -1) == -1
    assert sim.mla_cache_set_attend_path(h, 2) == 0
    assert sim.mla_attend_path(h, 1, 0) == 2 and sim.mla_attend_path(h, 1, 2) == 1
    assert sim.mla_cache_set_attend_path(h, 1) == 0
    assert sim.mla_attend_path(h, 4680, 0) == 1
    assert sim.mla_cache_set_attend_path(h, 3) == 1 and sim.mla_cache_set_attend_path(h, -1) == 1
    assert sim.mla_cache_set_attend_path(h, 0) == 0
    # handles the expansion cannot serve: fp32, other head widths, dense handles
    # (449 frames: the expanded window would pass 2^31 elements per sequence)
    for kw in ({"dtype": "f32", "cache_dtype": "f32"}, {"d_nope": 64}, {"d_v": 64},
               {"d_nope": 112, "d_rope": 16, "rope_split": (4, 2, 2)}, {"window_frames": 449}):
        st, g = _create(sim, _cfg(**kw))
        assert st == 0, kw
        assert sim.mla_cache_set_attend_path(g, 2) == 8, kw
        assert sim.mla_attend_path(g, 4680, 0) == 1, kw
    st, g = _create(sim, _cfg(window_frames=448))
    assert sim.mla_cache_set_attend_path(g, 2) == 0
    # narrower latents: the latent form needs few enough products to stay on
    # automatic (2 (d_c + 32) + 2 d_c < 1.5 * 512), yet the expansion can be chosen
    for d_c in (64, 128):
        st, g = _create(sim, _cfg(d_c=d_c))
        assert st == 0 and sim.mla_attend_path(g, 4680, 0) == 1, d_c
        assert sim.mla_cache_set_attend_path(g, 2) == 0 and sim.mla_attend_path(g, 4680, 0) == 2
    # bf16 rings (the absorbed core issues every product twice): expand from
    # 128 / 256 / 384 queries at d_c 192 / 128 / 64
    for d_c, first in ((192, 128), (128, 256), (64, 384)):
        st, g = _create(sim, _cfg(d_c=d_c, cache_dtype="bf16"))
        assert st == 0 and sim.mla_cache_set_state(g, 0, 20) == 0
        assert sim.mla_attend_path(g, first - 1, 0) == 1, d_c
        assert sim.mla_attend_path(g, first, 0) == 2 and sim.mla_attend_path(g, 4680, 0) == 2, d_c
        assert sim.mla_attend_path(g, 4680, 2) == 1, d_c
    st, d = _create(sim, c, dense=True)
    assert sim.mla_cache_set_attend_path(d, 1) == 9 and sim.mla_attend_path(d, 16, 0) == -1


def test_expand_attend_arguments_and_workspace(sim):
    """The expand path: workspace = expanded window, dense attention
    workspace, in that order and disjoint; the rebuild reads the
    resident keys from the ring, the dense attention reads the expanded window
    from key 0 with the latent path's scale and a rotation that leaves the
    d_nope content dimensions alone."""
    c = _cfg()
    st, h = _create(sim, c)
    assert sim.mla_cache_set_state(h, 3, 23) == 0
    ws = 1 << 40
    for Lq, (oldest, newest) in ((4680, (3, 23)), (512, (40, 44)), (2000, (7, 7))):
        assert sim.mla_cache_set_state(h, oldest, newest) == 0
        Lk = (newest - oldest + 1) * 1560
        need = sim.mla_attend_workspace_bytes(h, Lq, 0)
        kv = 21 * 1560 * 2 * 12 * 128 * 2                 # sized for the full window
        shape = expected_shape(Lq, 32)
        lq_pad = -(-Lq // shape[0]) * shape[0]
        R = 12 * lq_pad
        assert need >= kv + R * 128 * 2 + R * 128 * 4 + R * 8
        assert sim.mla_attend(h, P(FAKE_PTR), 0, Lq, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR), 0,
                              P(ws), 256, None) == 7
        n = sim.fake_count()
        assert sim.mla_attend(h, P(FAKE_PTR), 77, Lq, P(FAKE_PTR + 256), P(FAKE_PTR + 512),
                              P(FAKE_PTR + 768), 0, P(ws), need, None) == 0
        assert sim.fake_count() == n + 2 and sim.fake_kind() == 5
        e = _expand_info(sim)
        assert (e["B"], e["ring_rows"], e["key_slot0"], e["Lk"]) == \
            (1, 21 * 1560, (oldest % 21) * 1560, Lk)
        assert (e["n_h"], e["d_nope"], e["d_rope"], e["d_c"], e["d_v"], e["cache_type"]) == \
            (12, 96, 32, 192, 128, 2)
        assert e["ring"] == FAKE_STORAGE and e["w_uk"] == FAKE_PTR + 256
        assert e["kv"] == ws
        m = _mha_info(sim)
        p = _mha_ptrs(sim)
        assert (m["key_slot0"], m["Lk"], m["Lq"], m["q_token0"]) == (0, Lk, Lq, 77)
        assert p["ring"] == e["kv"] and p["ring_rows"] == Lk and p["d_h"] == 128
        assert p["q"] == FAKE_PTR and p["out"] == FAKE_PTR + 768
        assert p["qscale_u"] == round(float(np.float32(math.log2(math.e) / math.sqrt(128))) * 1e6)
        # disjoint regions inside the workspace
        assert e["kv"] + kv <= p["qrot"] < p["opart"] < p["ml"] < ws + need
        assert p["opart"] - p["qrot"] >= R * 128 * 2 and p["ml"] - p["opart"] >= R * 128 * 4
        assert (m["block_rows"], m["key_tile"], m["stages"]) == shape
        check_schedule(sim, m, R, which=1)
    # rotation of the expanded queries: identity on the content pairs, the
    # latent path's 3D table on the positional ones
    axis = (ctypes.c_int * 64)()
    inv = (ctypes.c_double * 64)()
    n = sim.fake_rope(2, axis, inv)
    want = O.rope_pair_table((6, 5, 5), 10000.0)
    assert n == 48 + 16
    assert all(inv[p] == 0.0 for p in range(48))
    assert [(axis[48 + p], inv[48 + p]) for p in range(16)] == [(a, f) for a, f in want]
    # a failed rebuild launch is reported and the attention is not launched
    n = sim.fake_count()
    sim.fake_fail_next()
    assert sim.mla_attend(h, P(FAKE_PTR), 0, 2000, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR), 0,
                          P(ws), 1 << 40, None) == 10
    assert sim.fake_count() == n + 1 and sim.fake_kind() == 7


@pytest.mark.parametrize("path,dense", [(1, False), (2, False), (0, True)])
def test_workspace_sized_once_serves_every_window_state(sim, path, dense):
    """The workspace size does not depend on how many frames are resident: a
    buffer of that size is accepted as the window fills, slides and wraps,
    and is the largest any state needs (a smaller one fails in some state)."""
    c = _cfg()
    st, h = _create(sim, c, dense=dense)
    assert st == 0
    if not dense:
        assert sim.mla_cache_set_attend_path(h, path) == 0
    ws = 1 << 40
    for Lq in (1, 100, 1024, 4680):
        sizes = set()
        ok_all = True
        for oldest, newest in ((0, 0), (0, 2), (0, 10), (0, 20), (5, 25), (30, 33)):
            assert sim.mla_cache_set_state(h, oldest, newest) == 0
            need = (sim.mha_attend_workspace_bytes(h, Lq) if dense
                    else sim.mla_attend_workspace_bytes(h, Lq, 0))
            sizes.add(need)
            if dense:
                ok_all &= sim.mha_attend(h, P(FAKE_PTR), 0, Lq, P(FAKE_PTR), P(ws), need, None) == 0
            else:
                ok_all &= sim.mla_attend(h, P(FAKE_PTR), 0, Lq, P(FAKE_PTR), P(FAKE_PTR),
                                         P(FAKE_PTR), 0, P(ws), need, None) == 0
        assert len(sizes) == 1 and ok_all, (Lq, sizes)
        need = sizes.pop()
        too_small = []
        for f in range(1, 22):
            assert sim.mla_cache_set_state(h, 0, f - 1) == 0
            if dense:
                too_small.append(sim.mha_attend(h, P(FAKE_PTR), 0, Lq, P(FAKE_PTR), P(ws), need - 1, None))
            else:
                too_small.append(sim.mla_attend(h, P(FAKE_PTR), 0, Lq, P(FAKE_PTR), P(FAKE_PTR),
                                                P(FAKE_PTR), 0, P(ws), need - 1, None))
        assert 7 in too_small, (Lq, too_small)


def test_expand_reuse_skips_rebuild_only_while_unchanged(sim):
    """With reuse on, a second expand-path attend on the same window state,
    workspace and weights launches no rebuild; a write, an eviction, a state
    change, another workspace, other weights, an absorbed attend in between
    or switching reuse off again bring the rebuild back."""
    c = _cfg()
    st, h = _create(sim, c)
    assert sim.mla_cache_set_state(h, 0, 17) == 0 and sim.mla_cache_set_attend_path(h, 2) == 0
    ws, ws2 = 1 << 40, (1 << 40) + (1 << 36)
    wuk, wuv = FAKE_PTR + 256, FAKE_PTR + 512

    def attend(w=ws, uk=wuk, uv=wuv, Lq=4680):
        n = sim.fake_count()
        assert sim.mla_attend(h, P(FAKE_PTR), 0, Lq, P(uk), P(uv), P(FAKE_PTR), 0, P(w), 1 << 40,
                              None) == 0
        return sim.fake_count() - n      # 2 with a rebuild, 1 without

    assert attend() == 2 and attend() == 2          # reuse off by default
    assert sim.mla_cache_set_expand_reuse(h, 1) == 0
    assert attend() == 2 and attend() == 1 and attend(Lq=1000) == 1
    assert sim.mla_cache_write(h, P(FAKE_PTR), P(FAKE_PTR), 18, 3, None) == 0
    assert attend() == 2 and attend() == 1
    assert sim.mla_cache_evict(h, 3) == 0
    assert attend() == 2 and attend() == 1
    assert sim.mla_cache_set_state(h, 3, 20) == 0
    assert attend() == 2 and attend() == 1
    assert attend(w=ws2) == 2 and attend(w=ws) == 2 and attend() == 1
    assert attend(uk=wuk + 256) == 2 and attend() == 2
    assert sim.mla_cache_set_attend_path(h, 1) == 0 and attend() == 1   # one absorbed launch
    assert sim.mla_cache_set_attend_path(h, 2) == 0 and attend() == 2 and attend() == 1
    assert sim.mla_cache_set_expand_reuse(h, 0) == 0 and attend() == 2 and attend() == 2
    assert sim.mla_cache_set_expand_reuse(h, 2) == 1
    st, d = _create(sim, c, dense=True)
    assert sim.mla_cache_set_expand_reuse(d, 1) == 9


def test_expand_reuse_sees_writes_by_other_handles(sim):
    """Expand reuse is process-wide aware of the workspace: another handle's
    attend (latent expand or absorbed, or dense) on the same or an overlapping
    workspace between two attends of handle A forces A to rebuild; another
    handle on a disjoint workspace does not."""
    c = _cfg()
    _, a = _create(sim, c)
    _, b = _create(sim, c)
    _, d = _create(sim, c, dense=True)
    for h in (a, b, d):
        assert sim.mla_cache_set_state(h, 0, 20) == 0
    assert sim.mla_cache_set_attend_path(a, 2) == 0 and sim.mla_cache_set_expand_reuse(a, 1) == 0
    ws = 1 << 40
    other = ws + (1 << 37)
    wuk, wuv = FAKE_PTR + 256, FAKE_PTR + 512

    def attend_a():
        n = sim.fake_count()
        assert sim.mla_attend(a, P(FAKE_PTR), 0, 4680, P(wuk), P(wuv), P(FAKE_PTR), 0, P(ws),
                              1 << 36, None) == 0
        return sim.fake_count() - n      # 2 with a rebuild, 1 without

    def attend_b(w, path):
        assert sim.mla_cache_set_attend_path(b, path) == 0
        assert sim.mla_attend(b, P(FAKE_PTR), 0, 4680, P(wuk), P(wuv), P(FAKE_PTR), 0, P(w),
                              1 << 36, None) == 0

    assert attend_a() == 2 and attend_a() == 1
    attend_b(ws, 2)                      # B expands into A's workspace
    assert attend_a() == 2 and attend_a() == 1
    attend_b(ws, 1)                      # B's absorbed attend overwrites it
    assert attend_a() == 2 and attend_a() == 1
    attend_b(ws + 4096, 2)               # overlapping range
    assert attend_a() == 2 and attend_a() == 1
    need = sim.mha_attend_workspace_bytes(d, 16)
    assert sim.mha_attend(d, P(FAKE_PTR), 0, 16, P(FAKE_PTR), P(ws + 256), need, None) == 0
    assert attend_a() == 2 and attend_a() == 1
    attend_b(other, 2)                   # a disjoint workspace leaves A's window alone
    attend_b(other, 1)
    assert attend_a() == 1
    sim.mla_cache_destroy(b)
    sim.mla_cache_destroy(d)
    assert attend_a() == 1
    sim.mla_cache_destroy(a)


def test_dense_attend_schedule(sim):
    c = _cfg()
    st, h = _create(sim, c, dense=True)
    assert st == 0 and sim.mla_cache_set_state(h, 0, 20) == 0
    ws = 1 << 40
    for Lq in (1, 31, 32, 33, 128, 129, 4680):
        need = sim.mha_attend_workspace_bytes(h, Lq)
        shape = expected_shape(Lq, 32)
        lq_pad = -(-Lq // shape[0]) * shape[0]
        R = 12 * lq_pad
        assert need >= R * 128 * 2 + R * 128 * 4 + R * 8
        assert sim.mha_attend(h, P(FAKE_PTR), 0, Lq, P(FAKE_PTR), P(ws), 256, None) == 7
        assert sim.mha_attend(h, P(FAKE_PTR), 21 * 1560, Lq, P(FAKE_PTR), P(ws), need, None) == 0
        a = _mha_info(sim)
        assert (a["block_rows"], a["key_tile"], a["stages"]) == shape
        assert a["Lk"] == 21 * 1560 and a["Lq"] == Lq and a["q_token0"] == 21 * 1560
        check_schedule(sim, a, R, which=1)
        resident = 256 * blocks_per_cu(shape, 2 * 128 // 8)
        assert a["n_blocks"] == min(resident, -(-a["n_groups"] * a["n_kt"] // 8))


def test_wrong_kind_and_unsupported(sim):
    c = _cfg()
    st, dense = _create(sim, c, dense=True)
    assert st == 0
    assert sim.mla_cache_write(dense, P(FAKE_PTR), P(FAKE_PTR), 0, 1, None) == 9
    st, lat = _create(sim, c)
    assert sim.mha_cache_write(lat, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR), 0, 1, None) == 9
    c2 = _cfg(d_c=96)
    st, h = _create(sim, c2)
    assert st == 0
    assert sim.mla_cache_write(h, P(FAKE_PTR), P(FAKE_PTR), 0, 1, None) == 0
    assert sim.mla_attend(h, P(FAKE_PTR), 0, 8, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR), 0,
                          P(1 << 40), 1 << 40, None) == 8


def test_rope_tables_match_oracle(sim):
    c = _cfg()
    st, h = _create(sim, c)
    sim.mla_cache_write(h, P(FAKE_PTR), P(FAKE_PTR), 0, 3, None)
    axis = (ctypes.c_int * 64)()
    inv = (ctypes.c_double * 64)()
    n = sim.fake_rope(0, axis, inv)
    want = O.rope_pair_table((6, 5, 5), 10000.0)
    assert n == len(want) == 16
    for p, (ax, f) in enumerate(want):
        assert axis[p] == ax and inv[p] == f
    st, d = _create(sim, c, dense=True)
    sim.mha_cache_write(d, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR), 0, 3, None)
    n = sim.fake_rope(0, axis, inv)
    want = O.rope_pair_table(O.default_rope_split(128), 10000.0)
    assert n == 64 and [axis[p] for p in range(64)] == [a for a, _ in want]
    assert [inv[p] for p in range(64)] == [f for _, f in want]
    w = _write_info(sim)
    assert w[3] == 3072 and w[5:9] == [0, 1536, 128, 1536]


def test_set_state_and_slot_validation(sim):
    c = _cfg()
    st, h = _create(sim, c)
    assert sim.mla_cache_set_state(h, 5, 3) == 1
    assert sim.mla_cache_set_state(h, 5, 26) == 1
    assert sim.mla_cache_set_state(h, -1, 3) == 1
    assert sim.mla_cache_set_state(h, 5, 25) == 0
    assert _info(sim, h) == (5, 25, 21, 21)
    assert sim.mla_cache_set_state(h, 7, 6) == 0       # empty
    assert _info(sim, h)[2] == 0
    assert sim.mla_cache_slot(h, 22, 1560) == -1
    assert sim.mla_cache_slot(h, -1, 0) == -1
    assert sim.mla_cache_slot(h, 43, 5) == (43 % 21) * 1560 + 5


def _proj_info(L, which):
    a = (ctypes.c_longlong * 15)()
    L.fake_proj_info(which, a)
    keys = ["M", "tokens_per_batch", "hidden", "width", "rot_begin", "rot_end", "rot_group", "rot_skip",
            "passes", "w_part1", "x_part2", "q_token0", "ring", "out_lo", "x"]
    return dict(zip(keys, list(a)))


def test_attend_block_arguments_and_workspace(sim):
    """mla_attend_block: the folded query projection writes [q_lat | q^R] rows
    of every head (rotation past d_c in each 224-wide head group, two weight
    parts) into the workspace's query block, the core and the latent merge
    follow, and the folded output projection (three passes of two-part
    operands, K = n_h * d_c) writes model-width rows to `out`."""
    for cache_dtype in ("f16", "bf16"):
        c = _cfg(cache_dtype=cache_dtype)
        st, h = _create(sim, c)
        assert sim.mla_cache_set_state(h, 3, 23) == 0
        Lq = 4680
        need = sim.mla_attend_block_workspace_bytes(h, Lq, 0)
        ws, out, x = 1 << 40, FAKE_PTR + 4096, FAKE_PTR + 8192
        assert sim.mla_attend_block(h, P(x), 21 * 1560, Lq, P(FAKE_PTR), P(FAKE_PTR), P(out), 0, P(ws),
                                    need - 1, None) == 7
        n = sim.fake_count()
        assert sim.mla_attend_block(h, P(x), 21 * 1560, Lq, P(FAKE_PTR), P(FAKE_PTR), P(out), 0, P(ws),
                                    need, None) == 0
        assert sim.fake_count() == n + 4                  # projection, core, merge, projection
        qp, op, at = _proj_info(sim, 0), _proj_info(sim, 1), _attend_info(sim)
        p_ = _attend_ptrs(sim)
        ptrs = [p_["qcat"], p_["qcat_lo"], p_["opart"], p_["ml"]]
        assert (qp["M"], qp["tokens_per_batch"], qp["hidden"], qp["width"]) == (Lq, Lq, 1536, 12 * 224)
        assert (qp["rot_begin"], qp["rot_end"], qp["rot_group"], qp["rot_skip"]) == (0, 12 * 224, 224, 192)
        assert (qp["passes"], qp["w_part1"], qp["q_token0"], qp["x"]) == (2, 12 * 224 * 1536 * 2, 21 * 1560, x)
        assert qp["ring"] == ptrs[0] == ws and qp["out_lo"] == ptrs[1]
        assert (ptrs[1] != 0) == (cache_dtype == "bf16")
        assert (op["M"], op["hidden"], op["width"], op["passes"]) == (Lq, 12 * 192, 1536, 3)
        assert op["w_part1"] == 1536 * 12 * 192 * 2 and op["ring"] == out
        o_bytes = -(-Lq * 12 * 192 * 2 // 256) * 256
        assert op["x_part2"] == o_bytes and ws < op["x"] and op["x"] + 2 * o_bytes <= ws + need
        assert op["x"] >= ptrs[3] + at["n_slots"] * Lq * 12 * 8    # after the max/sum block
        assert (at["block_rows"], at["key_tile"]) == expected_shape(Lq * 12, split=cache_dtype == "bf16")[:2]
        assert sim.mla_fold_query_bytes(h) == 2 * 12 * 224 * 1536 * 2
        assert sim.mla_fold_output_bytes(h) == 2 * 1536 * 12 * 192 * 2
        assert sim.mla_fold_query_weights(h, P(FAKE_PTR), P(FAKE_PTR), P(ws), 1 << 30, None) == 0
        assert sim.mla_fold_query_weights(h, P(FAKE_PTR), P(FAKE_PTR), P(ws), 1024, None) == 1
        assert sim.mla_fold_output_weights(h, P(FAKE_PTR), P(FAKE_PTR), P(ws), 1 << 30, None) == 0
    # fp32 handles and dense handles have no block
    st, g = _create(sim, _cfg(dtype="f32", cache_dtype="f32"))
    assert sim.mla_attend_block_workspace_bytes(g, 16, 0) == 0
    assert sim.mla_attend_block(g, P(FAKE_PTR), 0, 16, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR), 0,
                                P(1 << 40), 1 << 30, None) in (6, 8)
    st, d = _create(sim, _cfg(), dense=True)
    assert sim.mla_attend_block(d, P(FAKE_PTR), 0, 16, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR), 0,
                                P(1 << 40), 1 << 30, None) == 9


def test_cache_write_norm_arguments(sim):
    c = _cfg()
    st, h = _create(sim, c)
    sim.fake_write_eps.restype = ctypes.c_float
    assert sim.mla_cache_write_norm(h, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR), ctypes.c_float(-1.0), 0, 3,
                                    None) == 1
    assert sim.mla_cache_write_norm(h, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR), ctypes.c_float(1e-6), 0, 3,
                                    None) == 0
    assert sim.fake_kind() == 10 + 1 and sim.fake_write_norm_cols() == 192
    assert abs(sim.fake_write_eps() - 1e-6) < 1e-12
    assert _info(sim, h)[:3] == (0, 2, 3)
    assert sim.mla_cache_write_norm(h, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR), ctypes.c_float(1e-6), 5, 3,
                                    None) == 4                       # not contiguous
    st, g = _create(sim, _cfg(dtype="f32", cache_dtype="f32"))
    assert sim.mla_cache_write_norm(g, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR), ctypes.c_float(0.0), 0, 1,
                                    None) == 8


def test_e4m3_ring_rules(sim):
    """A one-byte (E4M3) ring: latent caches with bf16 inputs only, one byte
    per stored scalar; writes and attends carry the type; the expansion reads
    the one-byte rows and hands an fp16 window to the per-head attention; the
    core's LDS holds the raw tiles plus one fp16 decode tile, which sets the
    blocks per compute unit; the attention block's query projection writes
    fp16 operands."""
    E4M3 = 3
    c = _cfg(cache_dtype="e4m3")
    assert sim.mla_cache_bytes(ctypes.byref(c)) == 21 * 1560 * 224
    assert sim.mha_cache_bytes(ctypes.byref(c)) == 0
    assert _create(sim, c, dense=True)[0] == 1
    f32 = _cfg(cache_dtype="e4m3")
    f32.dtype = 0
    assert sim.mla_cache_bytes(ctypes.byref(f32)) == 0
    st, h = _create(sim, c)
    assert st == 0
    assert sim.mla_cache_write(h, P(FAKE_PTR), P(FAKE_PTR), 0, 3, None) == 0
    t = (ctypes.c_int * 5)()
    sim.fake_type_info(t)
    assert t[0] == E4M3
    assert sim.mla_cache_set_state(h, 3, 23) == 0
    ws = 1 << 40
    assert sim.mla_attend_path(h, 4680, 0) == 2 and sim.mla_attend_path(h, 8, 0) == 1
    need = sim.mla_attend_workspace_bytes(h, 4680, 0)
    assert sim.mla_attend(h, P(FAKE_PTR), 21 * 1560 - 4680, 4680, P(FAKE_PTR), P(FAKE_PTR),
                          P(FAKE_PTR), 0, P(ws), need, None) == 0
    sim.fake_type_info(t)
    assert t[3] == E4M3 and t[4] == 2        # one-byte rows in, fp16 window to the per-head core
    assert sim.mla_cache_set_attend_path(h, 2) == 0
    assert sim.mla_cache_set_attend_path(h, 1) == 0
    for Lq in (1, 4, 8, 11, 100, 4680):
        R = Lq * 12
        need = sim.mla_attend_workspace_bytes(h, Lq, 0)
        assert sim.mla_attend(h, P(FAKE_PTR), 21 * 1560, Lq, P(FAKE_PTR), P(FAKE_PTR),
                              P(FAKE_PTR), 0, P(ws), need, None) == 0
        sim.fake_type_info(t)
        assert t[1] == E4M3
        a = _attend_info(sim)
        shape = expected_shape(R, chunks_per_key=14)      # raw rows: 224 bytes
        assert (a["block_rows"], a["key_tile"], a["stages"]) == shape, Lq
        check_schedule(sim, a, R)
        br, kt, ns = shape
        waves = 1 if br <= 32 else (4 if br == 64 else br // 32)
        per_cu = min(160 * 1024 // ((ns * 14 + 28) * kt * 16), 8 // waves)
        assert a["n_blocks"] == min(256 * per_cu, -(-a["n_groups"] * a["n_kt"] // 8))
        p = _attend_ptrs(sim)
        qbytes = -(-R * 224 * 2 // 256) * 256
        assert p["qcat_lo"] == 0 and p["opart"] == ws + qbytes
    bw = sim.mla_attend_block_workspace_bytes(h, 40, 0)
    assert sim.mla_attend_block(h, P(FAKE_PTR), 21 * 1560 - 40, 40, P(FAKE_PTR), P(FAKE_PTR),
                                P(FAKE_PTR), 0, P(ws), bw, None) == 0
    sim.fake_type_info(t)
    assert t[2] == 2 and t[1] == E4M3


def test_block_placement_is_a_permutation_with_tails_beside_their_groups(sim):
    """Hardware workgroup -> logical block (dealt round-robin over 8 dies) is a
    permutation of the blocks; with a balanced tail, each die runs a
    proportional share of the main blocks and of the tail blocks, and the
    groups its tail blocks finish are within a die's worth of the groups its
    main blocks start."""
    ws = 1 << 40
    for name, kw, Lq in (("wan_window", {}, 4680), ("wan_window", {"batch": 11}, 1),
                         ("wan_window", {"batch": 3}, 8), ("wan_layer", {}, 4680)):
        for path in (1, 2):
            st, h = _create(sim, _cfg(name, **kw))
            assert st == 0
            c = _cfg(name, **kw)
            assert sim.mla_cache_set_state(h, 0, c.window_frames - 1) == 0
            if sim.mla_cache_set_attend_path(h, path) != 0:
                continue
            need = sim.mla_attend_workspace_bytes(h, Lq, 0)
            assert sim.mla_attend(h, P(FAKE_PTR), c.window_frames * 1560 - Lq, Lq, P(FAKE_PTR),
                                  P(FAKE_PTR), P(FAKE_PTR), 0, P(ws), need, None) == 0
            which = 1 if path == 2 else 0
            a = _mha_info(sim) if which else _attend_info(sim)
            nb, rem = a["n_blocks"], a["rem"]
            g = [sim.fake_sched_block_of(which, hw) for hw in range(nb)]
            assert sorted(g) == list(range(nb)), (name, kw, Lq, path)
            if rem == 0 or a["main_len"] >= a["n_kt"]:
                continue
            tl = a["n_kt"] - a["main_len"]
            for x in range(8):
                mine = [g[hw] for hw in range(x, nb, 8)]
                mains = [b for b in mine if b < rem]
                tails = [b - rem for b in mine if b >= rem]
                assert abs(len(mains) - len(mine) * rem / nb) <= 1.0
                if mains and tails:
                    first_grp = min(tails) * a["tpb"] // tl
                    assert abs(first_grp - min(mains)) <= -(-rem // 8) + 1, (name, kw, Lq, path, x)


def test_query_norm_state_reaches_both_paths_and_the_block_refuses(sim):
    """mla_cache_set_query_norm: argument checks, the gain and epsilon carried
    by the latent (absorbed) and per-head (expand) attends, switched off by
    NULL, refused on dense and fp32 handles, and mla_attend_block refuses
    while it is set (nothing launched)."""
    gam = FAKE_PTR + 4096
    st, h = _create(sim, _cfg())
    assert st == 0 and sim.mla_cache_set_state(h, 0, 20) == 0
    f32 = ctypes.c_float
    assert sim.mla_cache_set_query_norm(None, P(gam), f32(1e-6)) == 1
    assert sim.mla_cache_set_query_norm(h, P(gam + 8), f32(1e-6)) == 1      # misaligned
    assert sim.mla_cache_set_query_norm(h, P(gam), f32(-1.0)) == 1
    assert sim.mla_cache_set_query_norm(h, P(gam), f32(float("inf"))) == 1
    assert sim.mla_cache_set_query_norm(h, P(gam), f32(float("nan"))) == 1
    assert sim.mla_cache_set_query_norm(h, P(gam), f32(1e-5)) == 0
    ws = 1 << 40
    for path, which in ((1, 0), (2, 1)):
        assert sim.mla_cache_set_attend_path(h, path) == 0
        need = sim.mla_attend_workspace_bytes(h, 4680, 0)
        assert sim.mla_attend(h, P(FAKE_PTR), 21 * 1560 - 4680, 4680, P(FAKE_PTR), P(FAKE_PTR),
                              P(FAKE_PTR), 0, P(ws), need, None) == 0
        assert sim.fake_qnorm_gamma(which) == gam
        assert sim.fake_qnorm_eps(which) == np.float32(1e-5)
    # the attention block never forms per-head queries: refused, nothing launched
    assert sim.mla_cache_set_attend_path(h, 0) == 0
    n0 = sim.fake_count()
    need = sim.mla_attend_block_workspace_bytes(h, 64, 0)
    assert sim.mla_attend_block(h, P(FAKE_PTR), 0, 64, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR), 0,
                                P(ws), need, None) == 8
    assert sim.fake_count() == n0
    # off again: attends carry no gain, the block runs
    assert sim.mla_cache_set_query_norm(h, None, f32(0.0)) == 0
    assert sim.mla_attend(h, P(FAKE_PTR), 0, 64, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR), 0, P(ws),
                          sim.mla_attend_workspace_bytes(h, 64, 0), None) == 0
    assert sim.fake_qnorm_gamma(0) == 0
    assert sim.mla_attend_block(h, P(FAKE_PTR), 0, 64, P(FAKE_PTR), P(FAKE_PTR), P(FAKE_PTR), 0,
                                P(ws), need, None) == 0
    # dense and fp32 handles
    st, d = _create(sim, _cfg(), dense=True)
    assert st == 0 and sim.mla_cache_set_query_norm(d, P(gam), f32(1e-6)) == 9
    st, g = _create(sim, _cfg(dtype="f32", cache_dtype="f32"))
    assert st == 0 and sim.mla_cache_set_query_norm(g, P(gam), f32(1e-6)) == 8
    assert sim.mla_cache_set_query_norm(g, None, f32(0.0)) == 0
