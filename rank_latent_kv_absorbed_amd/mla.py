"""Python binding of libmla (ctypes).  Argument marshalling only: every step of
the cache-write / attend path runs in the library's gfx950 kernels.  PyTorch
supplies device memory and the current HIP stream.

The library must have been built (``python -m rank_latent_kv_absorbed_amd.build``);
importing this module without it raises ``LibraryMissing``: there is no
fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmla.so")


class LibraryMissing(ImportError):
    pass


class MlaError(RuntimeError):
    def __init__(self, status, what):
        self.status = int(status)
        super().__init__(f"{what}: {status_str(status)} (status {int(status)})")


# status codes (include/mla.h)
OK, ERR_INVALID_ARG, ERR_STORAGE_TOO_SMALL, ERR_FULL, ERR_NOT_CONTIGUOUS, ERR_EVICT_RANGE, \
    ERR_EMPTY, ERR_WORKSPACE, ERR_UNSUPPORTED, ERR_WRONG_KIND, ERR_HIP, ERR_SCRATCH = range(12)
F32, BF16, F16, E4M3 = 0, 1, 2, 3
_DTYPES = {"f32": (F32, torch.float32), "bf16": (BF16, torch.bfloat16), "f16": (F16, torch.float16),
           "e4m3": (E4M3, torch.float8_e4m3fn)}


class LayerConfigC(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32), ("d_nope", ctypes.c_int32),
        ("d_rope", ctypes.c_int32), ("d_v", ctypes.c_int32), ("d_c", ctypes.c_int32),
        ("grid_h", ctypes.c_int32), ("grid_w", ctypes.c_int32), ("window_frames", ctypes.c_int32),
        ("batch", ctypes.c_int32), ("rope_pairs_t", ctypes.c_int32),
        ("rope_pairs_h", ctypes.c_int32), ("rope_pairs_w", ctypes.c_int32),
        ("rope_base", ctypes.c_float), ("dtype", ctypes.c_int32), ("cache_dtype", ctypes.c_int32),
    ]


class CacheInfoC(ctypes.Structure):
    _fields_ = [("oldest_frame", ctypes.c_int64), ("newest_frame", ctypes.c_int64),
                ("n_resident_frames", ctypes.c_int32), ("capacity_frames", ctypes.c_int32)]


_VP, _SZ, _I32, _I64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
_CFGP = ctypes.POINTER(LayerConfigC)
_HANDLE = ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/mla.h
SIGNATURES = {
    "mla_cache_bytes": (_SZ, [_CFGP]),
    "mha_cache_bytes": (_SZ, [_CFGP]),
    "mla_cache_create": (_I32, [_CFGP, _VP, _SZ, ctypes.POINTER(_HANDLE)]),
    "mha_cache_create": (_I32, [_CFGP, _VP, _SZ, ctypes.POINTER(_HANDLE)]),
    "mla_cache_destroy": (None, [_HANDLE]),
    "mla_cache_write": (_I32, [_HANDLE, _VP, _VP, _I64, _I32, _VP]),
    "mla_cache_write_norm": (_I32, [_HANDLE, _VP, _VP, _VP, ctypes.c_float, _I64, _I32, _VP]),
    "mla_fold_query_bytes": (_SZ, [_HANDLE]),
    "mla_fold_output_bytes": (_SZ, [_HANDLE]),
    "mla_fold_query_weights": (_I32, [_HANDLE, _VP, _VP, _VP, _SZ, _VP]),
    "mla_fold_output_weights": (_I32, [_HANDLE, _VP, _VP, _VP, _SZ, _VP]),
    "mla_attend_block_workspace_bytes": (_SZ, [_HANDLE, _I32, _I32]),
    "mla_attend_block": (_I32, [_HANDLE, _VP, _I64, _I32, _VP, _VP, _VP, _I32, _VP, _SZ, _VP]),
    "mha_cache_write": (_I32, [_HANDLE, _VP, _VP, _VP, _I64, _I32, _VP]),
    "mla_cache_evict": (_I32, [_HANDLE, _I32]),
    "mla_cache_query": (_I32, [_HANDLE, ctypes.POINTER(CacheInfoC)]),
    "mla_cache_set_state": (_I32, [_HANDLE, _I64, _I64]),
    "mla_cache_slot": (_I64, [_HANDLE, _I64, _I32]),
    "mla_attend_workspace_bytes": (_SZ, [_HANDLE, _I32, _I32]),
    "mla_attend": (_I32, [_HANDLE, _VP, _I64, _I32, _VP, _VP, _VP, _I32, _VP, _SZ, _VP]),
    "mla_attend_noalloc": (_I32, [_HANDLE, _VP, _I64, _I32, _VP, _VP, _VP, _I32, _VP]),
    "mla_attend_noalloc_max_bytes": (_SZ, []),
    "mha_attend_workspace_bytes": (_SZ, [_HANDLE, _I32]),
    "mha_attend": (_I32, [_HANDLE, _VP, _I64, _I32, _VP, _VP, _SZ, _VP]),
    "mla_cache_set_profile_events": (_I32, [_HANDLE, _VP, _VP]),
    "mla_cache_set_attend_path": (_I32, [_HANDLE, _I32]),
    "mla_attend_path": (_I32, [_HANDLE, _I32, _I32]),
    "mla_cache_set_expand_reuse": (_I32, [_HANDLE, _I32]),
    "mla_cache_set_query_norm": (_I32, [_HANDLE, _VP, ctypes.c_float]),
    "mla_status_str": (ctypes.c_char_p, [_I32]),
    "mla_version": (ctypes.c_char_p, []),
}

_lib = None


def lib():
    """The loaded libmla (raises LibraryMissing if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryMissing(
                f"{LIB_PATH} not built; run `python -m rank_latent_kv_absorbed_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_str(status):
    return lib().mla_status_str(int(status)).decode()


def _check(status, what):
    if status != OK:
        raise MlaError(status, what)


def default_rope_split(d_rope):
    p = d_rope // 2
    return (p - 2 * (p // 3), p // 3, p // 3)


def make_config(cfg, batch=None):
    """ctypes config from any object with the layer attributes (hidden, n_heads,
    d_nope, d_rope, d_v, d_c, grid_h, grid_w, window_frames, batch, rope_split,
    rope_base, dtype in {'bf16', 'f32'}, cache_dtype in {'bf16', 'f16', 'e4m3', 'f32'}; a
    missing cache_dtype means fp16 storage for bf16 inputs, fp32 for fp32)."""
    split = getattr(cfg, "rope_split", None) or default_rope_split(cfg.d_rope)
    c = LayerConfigC()
    c.hidden, c.n_heads, c.d_nope, c.d_rope = cfg.hidden, cfg.n_heads, cfg.d_nope, cfg.d_rope
    c.d_v, c.d_c, c.grid_h, c.grid_w = cfg.d_v, cfg.d_c, cfg.grid_h, cfg.grid_w
    c.window_frames = cfg.window_frames
    c.batch = cfg.batch if batch is None else batch
    c.rope_pairs_t, c.rope_pairs_h, c.rope_pairs_w = split
    c.rope_base = float(getattr(cfg, "rope_base", 10000.0))
    c.dtype = _DTYPES[cfg.dtype][0]
    c.cache_dtype = _DTYPES[cache_dtype_of(cfg)][0]
    return c


def cache_dtype_of(cfg):
    cd = getattr(cfg, "cache_dtype", None)
    if cd is None:
        cd = "f32" if cfg.dtype == "f32" else "f16"
    return cd


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _alloc(nbytes_or_shape, dtype, device, stream):
    """A new tensor whose memory the caching allocator ties to `stream` (the
    stream the library's kernels use), so that it is not handed out again
    while those kernels may still run."""
    if stream is None or stream == torch.cuda.current_stream(device):
        return torch.empty(nbytes_or_shape, dtype=dtype, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(nbytes_or_shape, dtype=dtype, device=device)


def _need(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {dtype} {tuple(shape)}, got "
                         f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, the cache is on {device}")


class _CacheBase:
    _dense = False

    def __init__(self, cfg, storage=None, device="cuda", batch=None):
        self.cfg = cfg
        self.c = make_config(cfg, batch)
        self.batch = self.c.batch
        self.T = cfg.grid_h * cfg.grid_w
        self.tdtype = _DTYPES[cfg.dtype][1]           # inputs
        self.cdtype = _DTYPES[cache_dtype_of(cfg)][1]  # ring storage
        self.device = torch.device(device)
        if self.device.type == "cuda" and self.device.index is None:
            self.device = torch.device("cuda", torch.cuda.current_device())
        L = lib()
        nbytes = (L.mha_cache_bytes if self._dense else L.mla_cache_bytes)(ctypes.byref(self.c))
        if nbytes == 0:
            raise MlaError(ERR_INVALID_ARG, "cache_bytes")
        self.nbytes = nbytes
        if storage is None:
            storage = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.storage = storage
        h = _HANDLE()
        create = L.mha_cache_create if self._dense else L.mla_cache_create
        _check(create(ctypes.byref(self.c), _ptr(storage), storage.numel() * storage.element_size(),
                      ctypes.byref(h)), "cache_create")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.mla_cache_destroy(h)
            self._h = None

    # window bookkeeping (host-only)
    def evict(self, n_frames):
        _check(lib().mla_cache_evict(self._h, int(n_frames)), "cache_evict")

    def info(self):
        i = CacheInfoC()
        _check(lib().mla_cache_query(self._h, ctypes.byref(i)), "cache_query")
        return {"oldest_frame": i.oldest_frame, "newest_frame": i.newest_frame,
                "n_resident_frames": i.n_resident_frames, "capacity_frames": i.capacity_frames}

    def set_state(self, oldest_frame, newest_frame):
        _check(lib().mla_cache_set_state(self._h, int(oldest_frame), int(newest_frame)), "set_state")

    def slot(self, frame, tau):
        return lib().mla_cache_slot(self._h, int(frame), int(tau))

    def set_profile_events(self, start, stop):
        """Raw hipEvent_t handles (ints) recorded around the main attention
        kernel of later attend calls; (None, None) switches it off."""
        _check(lib().mla_cache_set_profile_events(self._h, ctypes.c_void_p(start),
                                                  ctypes.c_void_p(stop)), "set_profile_events")


# mla_attend_path_kind
ATTEND_PATHS = {"auto": 0, "absorbed": 1, "expand": 2}


class LatentCache(_CacheBase):
    """One cached layer's sliding window of (c^KV, k^R) rows."""

    @property
    def width(self):
        return self.cfg.d_c + self.cfg.d_rope

    def ring(self):
        """The ring storage viewed as [batch, window_frames*T, d_c + d_rope]."""
        n = self.batch * self.cfg.window_frames * self.T * self.width
        return self.storage.view(self.cdtype)[:n].view(self.batch, self.cfg.window_frames * self.T,
                                                       self.width)

    def write(self, x, w_dkr, frame0, n_frames, stream=None):
        cfg = self.cfg
        _need(x, "x", self.tdtype, (self.batch, n_frames * self.T, cfg.hidden), self.device)
        _need(w_dkr, "w_dkr", self.tdtype, (self.width, cfg.hidden), self.device)
        _check(lib().mla_cache_write(self._h, _ptr(x), _ptr(w_dkr), int(frame0), int(n_frames),
                                     _stream(stream)), "cache_write")

    def write_norm(self, x, w_dkr, gamma, eps, frame0, n_frames, stream=None):
        """Cache write with the latent RMS-normalised (mla_cache_write_norm)."""
        cfg = self.cfg
        _need(x, "x", self.tdtype, (self.batch, n_frames * self.T, cfg.hidden), self.device)
        _need(w_dkr, "w_dkr", self.tdtype, (self.width, cfg.hidden), self.device)
        _need(gamma, "gamma", self.tdtype, (cfg.d_c,), self.device)
        _check(lib().mla_cache_write_norm(self._h, _ptr(x), _ptr(w_dkr), _ptr(gamma), float(eps),
                                          int(frame0), int(n_frames), _stream(stream)), "cache_write_norm")

    def fold_query_weights(self, w_q, w_uk, stream=None):
        """[2, n_h, d_c + d_rope, hidden] bf16: W^K_up folded into the query
        projection, as value and remainder parts (mla_fold_query_weights)."""
        cfg = self.cfg
        _need(w_q, "w_q", self.tdtype, (cfg.n_heads * (cfg.d_nope + cfg.d_rope), cfg.hidden), self.device)
        _need(w_uk, "w_uk", self.tdtype, (cfg.n_heads, cfg.d_nope, cfg.d_c), self.device)
        out = _alloc((2, cfg.n_heads, cfg.d_c + cfg.d_rope, cfg.hidden), self.tdtype, self.device, stream)
        _check(lib().mla_fold_query_weights(self._h, _ptr(w_q), _ptr(w_uk), _ptr(out),
                                            out.numel() * out.element_size(), _stream(stream)),
               "fold_query_weights")
        return out

    def fold_output_weights(self, w_o, w_uv, stream=None):
        """[2, hidden, n_h * d_c] bf16: W^V_up folded into W^O, as value and
        remainder parts (mla_fold_output_weights)."""
        cfg = self.cfg
        _need(w_o, "w_o", self.tdtype, (cfg.hidden, cfg.n_heads * cfg.d_v), self.device)
        _need(w_uv, "w_uv", self.tdtype, (cfg.n_heads, cfg.d_v, cfg.d_c), self.device)
        out = _alloc((2, cfg.hidden, cfg.n_heads * cfg.d_c), self.tdtype, self.device, stream)
        _check(lib().mla_fold_output_weights(self._h, _ptr(w_o), _ptr(w_uv), _ptr(out),
                                             out.numel() * out.element_size(), _stream(stream)),
               "fold_output_weights")
        return out

    def block_workspace_bytes(self, Lq, key_splits=0):
        return lib().mla_attend_block_workspace_bytes(self._h, int(Lq), int(key_splits))

    def attend_block(self, x, q_token0, w_qf, w_fo, out=None, key_splits=0, workspace=None, stream=None):
        """Model-width attention block of the query tokens' layer input x
        [batch, Lq, hidden] with folded weights (mla_attend_block)."""
        cfg = self.cfg
        Lq = x.shape[1]
        _need(x, "x", self.tdtype, (self.batch, Lq, cfg.hidden), self.device)
        _need(w_qf, "w_qf", self.tdtype, (2, cfg.n_heads, cfg.d_c + cfg.d_rope, cfg.hidden), self.device)
        _need(w_fo, "w_fo", self.tdtype, (2, cfg.hidden, cfg.n_heads * cfg.d_c), self.device)
        if out is None:
            out = _alloc((self.batch, Lq, cfg.hidden), torch.float32, self.device, stream)
        _need(out, "out", torch.float32, (self.batch, Lq, cfg.hidden), self.device)
        need = self.block_workspace_bytes(Lq, key_splits)
        if workspace is None and need > 0:
            workspace = _alloc(need, torch.uint8, self.device, stream)
        wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib().mla_attend_block(self._h, _ptr(x), int(q_token0), int(Lq), _ptr(w_qf), _ptr(w_fo),
                                      _ptr(out), int(key_splits), _ptr(workspace), wbytes,
                                      _stream(stream)), "attend_block")
        return out

    def workspace_bytes(self, Lq, key_splits=0):
        return lib().mla_attend_workspace_bytes(self._h, int(Lq), int(key_splits))

    def set_attend_path(self, path):
        """'auto', 'absorbed' or 'expand' (see ATTEND_PATHS)."""
        _check(lib().mla_cache_set_attend_path(self._h, ATTEND_PATHS[path]), "set_attend_path")

    def set_expand_reuse(self, enable=True):
        """Let expand-path attends reuse the rebuilt window while it is unchanged
        (same workspace and weights; see mla_cache_set_expand_reuse)."""
        _check(lib().mla_cache_set_expand_reuse(self._h, 1 if enable else 0), "set_expand_reuse")

    def set_query_norm(self, gamma, eps=1e-6):
        """RMS-normalise each head's query row with gain `gamma` [d_nope + d_rope]
        (input dtype, on this device) in later attends; None switches it off
        (see mla_cache_set_query_norm).  The handle keeps a reference to gamma
        while the norm is set."""
        if gamma is None:
            _check(lib().mla_cache_set_query_norm(self._h, None, 0.0), "set_query_norm")
            self._qn_gamma = None
            return
        cfg = self.cfg
        _need(gamma, "gamma", self.tdtype, (cfg.d_nope + cfg.d_rope,), self.device)
        _check(lib().mla_cache_set_query_norm(self._h, _ptr(gamma), float(eps)), "set_query_norm")
        self._qn_gamma = gamma

    def attend_path(self, Lq, key_splits=0):
        """Name of the path an attend of Lq queries takes on this handle."""
        k = lib().mla_attend_path(self._h, int(Lq), int(key_splits))
        if k < 0:
            raise ValueError(f"attend_path: bad arguments Lq={Lq} key_splits={key_splits}")
        return {v: n for n, v in ATTEND_PATHS.items()}[k]

    def attend(self, q, q_token0, w_uk, w_uv, out=None, key_splits=0, workspace=None, stream=None):
        cfg = self.cfg
        Lq = q.shape[1]
        _need(q, "q", self.tdtype, (self.batch, Lq, cfg.n_heads, cfg.d_nope + cfg.d_rope), self.device)
        _need(w_uk, "w_uk", self.tdtype, (cfg.n_heads, cfg.d_nope, cfg.d_c), self.device)
        _need(w_uv, "w_uv", self.tdtype, (cfg.n_heads, cfg.d_v, cfg.d_c), self.device)
        if out is None:
            out = _alloc((self.batch, Lq, cfg.n_heads, cfg.d_v), torch.float32, self.device, stream)
        _need(out, "out", torch.float32, (self.batch, Lq, cfg.n_heads, cfg.d_v), self.device)
        need = self.workspace_bytes(Lq, key_splits)
        if workspace is None and need > 0:
            workspace = _alloc(need, torch.uint8, self.device, stream)
        wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib().mla_attend(self._h, _ptr(q), int(q_token0), int(Lq), _ptr(w_uk), _ptr(w_uv),
                                _ptr(out), int(key_splits), _ptr(workspace), wbytes,
                                _stream(stream)), "attend")
        return out


    def attend_noalloc(self, q, q_token0, w_uk, w_uv, out, key_splits=0, stream=None):
        """mla_attend_noalloc: the workspace comes from the library's static
        device scratch; `out` must be given (nothing is allocated)."""
        cfg = self.cfg
        Lq = q.shape[1]
        _need(q, "q", self.tdtype, (self.batch, Lq, cfg.n_heads, cfg.d_nope + cfg.d_rope), self.device)
        _need(w_uk, "w_uk", self.tdtype, (cfg.n_heads, cfg.d_nope, cfg.d_c), self.device)
        _need(w_uv, "w_uv", self.tdtype, (cfg.n_heads, cfg.d_v, cfg.d_c), self.device)
        _need(out, "out", torch.float32, (self.batch, Lq, cfg.n_heads, cfg.d_v), self.device)
        _check(lib().mla_attend_noalloc(self._h, _ptr(q), int(q_token0), int(Lq), _ptr(w_uk),
                                        _ptr(w_uv), _ptr(out), int(key_splits), _stream(stream)),
               "attend_noalloc")
        return out


class DenseCache(_CacheBase):
    """Dense per-head K/V window (comparison path)."""

    _dense = True

    @property
    def d_h(self):
        return self.cfg.d_nope + self.cfg.d_rope

    def ring(self):
        """[batch, window_frames*T, 2, n_heads, d_h]."""
        n_h, d_h = self.cfg.n_heads, self.d_h
        n = self.batch * self.cfg.window_frames * self.T * 2 * n_h * d_h
        return self.storage.view(self.cdtype)[:n].view(self.batch, self.cfg.window_frames * self.T,
                                                       2, n_h, d_h)

    def write(self, x, w_k, w_v, frame0, n_frames, stream=None):
        cfg = self.cfg
        n = cfg.n_heads * self.d_h
        _need(x, "x", self.tdtype, (self.batch, n_frames * self.T, cfg.hidden), self.device)
        _need(w_k, "w_k", self.tdtype, (n, cfg.hidden), self.device)
        _need(w_v, "w_v", self.tdtype, (n, cfg.hidden), self.device)
        _check(lib().mha_cache_write(self._h, _ptr(x), _ptr(w_k), _ptr(w_v), int(frame0),
                                     int(n_frames), _stream(stream)), "mha_cache_write")

    def workspace_bytes(self, Lq):
        return lib().mha_attend_workspace_bytes(self._h, int(Lq))

    def attend(self, q, q_token0, out=None, workspace=None, stream=None):
        cfg = self.cfg
        Lq = q.shape[1]
        _need(q, "q", self.tdtype, (self.batch, Lq, cfg.n_heads, self.d_h), self.device)
        if out is None:
            out = _alloc((self.batch, Lq, cfg.n_heads, self.d_h), torch.float32, self.device, stream)
        _need(out, "out", torch.float32, (self.batch, Lq, cfg.n_heads, self.d_h), self.device)
        need = self.workspace_bytes(Lq)
        if workspace is None and need > 0:
            workspace = _alloc(need, torch.uint8, self.device, stream)
        wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        _check(lib().mha_attend(self._h, _ptr(q), int(q_token0), int(Lq), _ptr(out),
                                _ptr(workspace), wbytes, _stream(stream)), "mha_attend")
        return out


def attend_flops(n_heads, Lq, Lk, d_c, d_rope, d_nope, d_v, batch=1):
    """Algorithmic FLOP of one absorbed attend call: scores over [c | k^R],
    latent value sums, the W^K_up query fold and the W^V_up epilogue."""
    R = batch * n_heads * Lq
    return R * Lk * (2 * (d_c + d_rope) + 2 * d_c) + R * (2 * d_nope * d_c + 2 * d_c * d_v)


def attend_bytes(n_heads, Lq, Lk, d_c, d_rope, d_nope, d_v, batch=1, elem=2, cache_elem=None):
    """Algorithmic HBM bytes of one attend call: the window read once (at
    cache_elem bytes per scalar, default elem), queries in, fp32 output out,
    and the up-projection weights."""
    ce = elem if cache_elem is None else cache_elem
    return batch * (Lk * (d_c + d_rope) * ce + Lq * n_heads * (d_nope + d_rope) * elem
                    + Lq * n_heads * d_v * 4) + n_heads * (d_nope + d_v) * d_c * elem


def expand_attend_flops(n_heads, Lq, Lk, d_c, d_rope, d_nope, d_v, batch=1):
    """Algorithmic FLOP of one expand-then-attend call: the window's per-head
    keys and values rebuilt once, then per-head scores (d_nope + d_rope) and
    value sums (d_v)."""
    rebuild = batch * Lk * n_heads * 2 * d_c * (d_nope + d_v)
    return rebuild + batch * n_heads * Lq * Lk * 2 * (d_nope + d_rope + d_v)


def mha_attend_flops(n_heads, Lq, Lk, d_h, batch=1):
    return batch * n_heads * Lq * Lk * 4 * d_h

