"""ctypes binding of libshadowkv.so (include/shadowkv.h).

Argument marshalling only: every step of the decode path runs in the HIP
library.  The module-level functions carry the C names; ``Layer`` and
``HostBuffer`` marshal torch tensors (device memory and streams) into them and
check every tensor's shape, dtype, device and contiguity before a call, so a
kernel never sees a buffer smaller than its grid assumes.  The library must be
built (``python -m sparse_kv_cache_step_amd.build``); loading fails loudly
otherwise.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libshadowkv.so")

SKV_F32, SKV_BF16 = 0, 1
SKV_OK, SKV_E_INVAL, SKV_E_SHAPE, SKV_E_STATE, SKV_E_NOMEM, SKV_E_HIP = 0, -1, -2, -3, -4, -5
(SKV_T_LANDMARKS, SKV_T_MIN_COS, SKV_T_OUTLIERS, SKV_T_CAND_MASK, SKV_T_SCORES, SKV_T_GROUP_SCORES,
 SKV_T_SELECTION, SKV_T_SLOT_CHUNKS, SKV_T_CACHE_V, SKV_T_K_OUT, SKV_T_V_OUT, SKV_T_K_LOC,
 SKV_T_V_LOC, SKV_T_SELECTION_SLOTS, SKV_T_V_CODES) = range(15)
KERNELS = ("score", "select", "fetch", "qk", "pv", "attn")
SKV_K_COUNT = len(KERNELS)

EXPORTS = (
    "shadowkv_layer_create", "shadowkv_layer_destroy", "shadowkv_prefill_meta", "shadowkv_load_meta",
    "shadowkv_append", "shadowkv_snapkv_select", "shadowkv_decode_step", "shadowkv_decode_step_noalloc",
    "shadowkv_reset_cache", "shadowkv_get_stats", "shadowkv_reset_stats",
    "shadowkv_tensor_bytes", "shadowkv_read", "shadowkv_set_overlap", "shadowkv_set_timing",
    "shadowkv_get_timing",
    "shadowkv_host_alloc", "shadowkv_host_free", "shadowkv_last_error", "shadowkv_equiv_bandwidth",
    "shadowkv_probe_hbm_read", "shadowkv_factorize", "shadowkv_probe_host_copies",
)


class skv_config(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads_q", ctypes.c_int32), ("heads_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("seq_len", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("n_outlier", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("local_window", ctypes.c_int32), ("rope_base", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("max_new", ctypes.c_int32), ("cache_chunks", ctypes.c_int32)]


class skv_stats(ctypes.Structure):
    _fields_ = [("steps", ctypes.c_int64), ("hits", ctypes.c_int64), ("misses", ctypes.c_int64),
                ("bytes_h2d", ctypes.c_int64)]


class ShadowKVError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"shadowkv error {code}: {msg}")
        self.code = code


_VP = ctypes.c_void_p
_lib_handle = None


def lib() -> ctypes.CDLL:
    """Load libshadowkv.so (never builds it; raises if it is missing)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m sparse_kv_cache_step_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "shadowkv_layer_create": (ctypes.c_int, [ctypes.POINTER(skv_config), ctypes.POINTER(_VP)]),
            "shadowkv_layer_destroy": (None, [_VP]),
            "shadowkv_prefill_meta": (ctypes.c_int, [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
            "shadowkv_load_meta": (ctypes.c_int, [_VP] * 11),
            "shadowkv_append": (ctypes.c_int, [_VP, _VP, _VP, _VP]),
            "shadowkv_snapkv_select": (ctypes.c_int, [_VP, _VP, ctypes.c_int, ctypes.c_int, _VP]),
            "shadowkv_decode_step": (ctypes.c_int, [_VP, _VP, _VP, _VP]),
            "shadowkv_decode_step_noalloc": (ctypes.c_int, [_VP, _VP, _VP, _VP]),
            "shadowkv_reset_cache": (ctypes.c_int, [_VP, _VP]),
            "shadowkv_get_stats": (ctypes.c_int, [_VP, ctypes.POINTER(skv_stats)]),
            "shadowkv_reset_stats": (ctypes.c_int, [_VP]),
            "shadowkv_tensor_bytes": (ctypes.c_size_t, [_VP, ctypes.c_int]),
            "shadowkv_read": (ctypes.c_int, [_VP, ctypes.c_int, _VP, ctypes.c_size_t, _VP]),
            "shadowkv_set_overlap": (ctypes.c_int, [_VP, ctypes.c_int]),
            "shadowkv_set_timing": (ctypes.c_int, [_VP, ctypes.c_int]),
            "shadowkv_get_timing": (ctypes.c_int, [_VP, ctypes.POINTER(ctypes.c_double),
                                                   ctypes.POINTER(ctypes.c_int64)]),
            "shadowkv_host_alloc": (ctypes.c_int, [ctypes.c_size_t, ctypes.POINTER(_VP)]),
            "shadowkv_host_free": (ctypes.c_int, [_VP]),
            "shadowkv_last_error": (ctypes.c_char_p, []),
            "shadowkv_equiv_bandwidth": (ctypes.c_double, [ctypes.c_double] * 7),
            "shadowkv_probe_hbm_read": (ctypes.c_int, [_VP, ctypes.c_size_t, ctypes.c_int, _VP,
                                                       ctypes.POINTER(ctypes.c_double)]),
            "shadowkv_factorize": (ctypes.c_int, [ctypes.c_int] * 6 + [_VP, _VP, _VP, _VP,
                                                                        ctypes.POINTER(ctypes.c_int)]),
            "shadowkv_probe_host_copies": (ctypes.c_int, [_VP, ctypes.c_size_t, _VP, ctypes.c_size_t, ctypes.c_int,
                                                          _VP, ctypes.c_int, _VP, ctypes.POINTER(ctypes.c_double),
                                                          ctypes.POINTER(ctypes.c_double)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib_handle = L
    return _lib_handle


def _check(rc: int) -> None:
    if rc != SKV_OK:
        raise ShadowKVError(rc, shadowkv_last_error())


# ---- C entry points under their own names --------------------------------
def shadowkv_last_error() -> str:
    return lib().shadowkv_last_error().decode()


def shadowkv_equiv_bandwidth(S, C, K, O, alpha, b_gpu, b_pcie) -> float:
    return lib().shadowkv_equiv_bandwidth(S, C, K, O, alpha, b_gpu, b_pcie)


def shadowkv_probe_hbm_read(buf, nbytes: int, reps: int, stream) -> float:
    """Streaming-read ceiling (GB/s) over `nbytes` of device memory at `buf`."""
    out = ctypes.c_double()
    rc = lib().shadowkv_probe_hbm_read(buf, nbytes, reps, stream, ctypes.byref(out))
    if rc != SKV_OK:
        raise ShadowKVError(rc, "read probe failed")
    return out.value


def shadowkv_probe_host_copies(host, host_bytes: int, dev, chunk_bytes: int, host_chunks, reps: int,
                               stream) -> tuple[float, float]:
    """Host-issued chunk copies (GB/s): one hipMemcpyAsync per chunk, and one
    hipMemcpyBatchAsync; host_chunks is a sequence of chunk indices."""
    n = len(host_chunks)
    arr = (ctypes.c_int64 * n)(*host_chunks)
    each, batch = ctypes.c_double(), ctypes.c_double()
    rc = lib().shadowkv_probe_host_copies(host, host_bytes, dev, chunk_bytes, n, arr, reps, stream,
                                          ctypes.byref(each), ctypes.byref(batch))
    if rc != SKV_OK:
        raise ShadowKVError(rc, "host-copy probe failed")
    return each.value, batch.value


def shadowkv_layer_create(cfg: skv_config) -> int:
    h = _VP()
    _check(lib().shadowkv_layer_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h.value


def shadowkv_layer_destroy(h: int) -> None:
    lib().shadowkv_layer_destroy(h)


def shadowkv_prefill_meta(h, k_pre, k_rope, v, A, B, v_host, stream) -> None:
    _check(lib().shadowkv_prefill_meta(h, k_pre, k_rope, v, A, B, v_host, stream))


def shadowkv_load_meta(h, landmarks, outliers, k_out, v_out, k_loc, v_loc, A, B, v_host, stream) -> None:
    _check(lib().shadowkv_load_meta(h, landmarks, outliers, k_out, v_out, k_loc, v_loc, A, B, v_host, stream))


def shadowkv_append(h, k_new, v_new, stream) -> None:
    _check(lib().shadowkv_append(h, k_new, v_new, stream))


def shadowkv_snapkv_select(h, q_obs, w_obs, pool, stream) -> None:
    _check(lib().shadowkv_snapkv_select(h, q_obs, int(w_obs), int(pool), stream))


def shadowkv_decode_step(h, q, out, stream) -> None:
    _check(lib().shadowkv_decode_step(h, q, out, stream))


def shadowkv_decode_step_noalloc(h, q, out, stream) -> None:
    _check(lib().shadowkv_decode_step_noalloc(h, q, out, stream))


def shadowkv_reset_cache(h, stream) -> None:
    _check(lib().shadowkv_reset_cache(h, stream))


def shadowkv_get_stats(h) -> skv_stats:
    st = skv_stats()
    _check(lib().shadowkv_get_stats(h, ctypes.byref(st)))
    return st


def shadowkv_reset_stats(h) -> None:
    _check(lib().shadowkv_reset_stats(h))


def shadowkv_tensor_bytes(h, which: int) -> int:
    return lib().shadowkv_tensor_bytes(h, which)


def shadowkv_read(h, which: int, dst, nbytes: int, stream) -> None:
    _check(lib().shadowkv_read(h, which, dst, nbytes, stream))


def shadowkv_set_overlap(h, enable: bool) -> None:
    _check(lib().shadowkv_set_overlap(h, int(bool(enable))))


def shadowkv_set_timing(h, enable: bool) -> None:
    _check(lib().shadowkv_set_timing(h, int(bool(enable))))


def shadowkv_get_timing(h) -> tuple[list[float], int]:
    ms = (ctypes.c_double * SKV_K_COUNT)()
    steps = ctypes.c_int64()
    _check(lib().shadowkv_get_timing(h, ms, ctypes.byref(steps)))
    return list(ms), steps.value


def shadowkv_host_alloc(nbytes: int) -> int:
    p = _VP()
    _check(lib().shadowkv_host_alloc(nbytes, ctypes.byref(p)))
    return p.value


def shadowkv_host_free(ptr: int) -> None:
    _check(lib().shadowkv_host_free(ptr))


# ---- torch marshalling ----------------------------------------------------
def _torch():
    import torch
    return torch


def _stream_ptr(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def factorize(k_pre, rank: int, stream=None, return_sweeps: bool = False):
    """Low-rank key factors on k_pre's GPU (shadowkv_factorize): k_pre
    (b, h_kv, s, d), bfloat16 or binary32, contiguous.  Returns A (b, s, rank)
    and B (b, h_kv, rank, d) in k_pre's dtype (and the eigensolver's sweep
    count with return_sweeps)."""
    torch = _torch()
    if k_pre.dim() != 4 or not k_pre.is_cuda or not k_pre.is_contiguous():
        raise ValueError("k_pre must be a contiguous (b, h_kv, s, d) device tensor")
    if k_pre.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"k_pre: dtype {k_pre.dtype} is neither bfloat16 nor float32")
    b, hkv, s, d = k_pre.shape
    A = torch.empty((b, s, rank), dtype=k_pre.dtype, device=k_pre.device)
    B = torch.empty((b, hkv, rank, d), dtype=k_pre.dtype, device=k_pre.device)
    sweeps = ctypes.c_int()
    with torch.cuda.device(k_pre.device):
        _check(lib().shadowkv_factorize(SKV_BF16 if k_pre.dtype == torch.bfloat16 else SKV_F32, b, hkv, s, d, rank,
                                        k_pre.data_ptr(), A.data_ptr(), B.data_ptr(), _stream_ptr(stream),
                                        ctypes.byref(sweeps)))
    return (A, B, sweeps.value) if return_sweeps else (A, B)


class HostBuffer:
    """Pinned, device-readable host memory owned by the caller (the layer
    borrows it).  ``tensor(dtype, shape)`` is a CPU torch view of it."""

    def __init__(self, nbytes: int):
        self.nbytes = int(nbytes)
        self.ptr = shadowkv_host_alloc(self.nbytes)

    def tensor(self, dtype, shape):
        torch = _torch()
        count = 1
        for x in shape:
            count *= x
        if count * torch.empty((), dtype=dtype).element_size() > self.nbytes:
            raise ValueError("view larger than the buffer")
        raw = (ctypes.c_uint8 * self.nbytes).from_address(self.ptr)
        return torch.frombuffer(raw, dtype=dtype, count=count).view(*shape)

    def free(self) -> None:
        if self.ptr:
            shadowkv_host_free(self.ptr)
            self.ptr = 0

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


class Layer:
    """One model layer's ShadowKV state on the current GPU."""

    def __init__(self, *, batch, heads_q, heads_kv, head_dim, seq_len, chunk, rank, n_outlier, top_k,
                 local_window, rope_base=10000.0, bf16=True, max_new=0, cache_chunks=0):
        torch = _torch()
        self.cfg = skv_config(batch, heads_q, heads_kv, head_dim, seq_len, chunk, rank, n_outlier, top_k,
                              local_window, float(rope_base), SKV_BF16 if bf16 else SKV_F32, max_new, cache_chunks)
        self.cap = cache_chunks if cache_chunks > 0 else top_k  # V cache slots per (sequence, KV head)
        self.dtype = torch.bfloat16 if bf16 else torch.float32
        self.n = seq_len // chunk if chunk > 0 else 0
        self.device = torch.device("cuda", torch.cuda.current_device())
        self.h = shadowkv_layer_create(self.cfg)
        self._v_host = None

    # shapes -----------------------------------------------------------------
    def _shape(self, name):
        c = self.cfg
        b, hq, hkv, d, s, ch = c.batch, c.heads_q, c.heads_kv, c.head_dim, c.seq_len, c.chunk
        return {
            "k_pre": (b, hkv, s, d), "k_rope": (b, hkv, s, d), "v": (b, hkv, s, d),
            "A": (b, s, c.rank), "B": (b, hkv, c.rank, d), "q": (b, hq, d), "out": (b, hq, d),
            "landmarks": (b, hkv, self.n, d), "outliers": (b, hkv, c.n_outlier),
            "k_out": (b, hkv, c.n_outlier * ch, d), "v_out": (b, hkv, c.n_outlier * ch, d),
            "k_loc": (b, hkv, c.local_window, d), "v_loc": (b, hkv, c.local_window, d),
            "k_new": (b, hkv, d), "v_new": (b, hkv, d),
        }[name]

    def _dev(self, name, t, dtype=None, optional=False, shape=None):
        torch = _torch()
        if t is None:
            if optional:
                return None
            raise ValueError(f"{name} is required")
        dtype = self.dtype if dtype is None else dtype
        shape = self._shape(name) if shape is None else shape
        if tuple(t.shape) != shape:
            raise ValueError(f"{name}: shape {tuple(t.shape)} != {shape}")
        if t.dtype != dtype:
            raise ValueError(f"{name}: dtype {t.dtype} != {dtype}")
        if t.device != self.device:
            raise ValueError(f"{name}: must be on {self.device}, got {t.device}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous")
        return t.data_ptr()

    def _host(self, v_host: HostBuffer):
        c = self.cfg
        need = c.batch * c.heads_kv * c.seq_len * c.head_dim * (2 if c.dtype == SKV_BF16 else 4)
        if not isinstance(v_host, HostBuffer) or v_host.nbytes < need:
            raise ValueError(f"v_host must be a HostBuffer of at least {need} bytes")
        return v_host.ptr

    def host_buffer(self) -> HostBuffer:
        c = self.cfg
        return HostBuffer(c.batch * c.heads_kv * c.seq_len * c.head_dim * (2 if c.dtype == SKV_BF16 else 4))

    # entry points -------------------------------------------------------------
    def prefill_meta(self, k_pre, v, A, B, v_host: HostBuffer, k_rope=None, stream=None):
        kp = self._dev("k_pre", k_pre, optional=k_rope is not None)
        kr = self._dev("k_rope", k_rope, optional=True)
        shadowkv_prefill_meta(self.h, kp, kr, self._dev("v", v), self._dev("A", A), self._dev("B", B),
                              self._host(v_host), _stream_ptr(stream))
        self._v_host = v_host

    def load_meta(self, landmarks, outliers, k_out, v_out, k_loc, v_loc, A, B, v_host: HostBuffer, stream=None):
        torch = _torch()
        shadowkv_load_meta(self.h, self._dev("landmarks", landmarks), self._dev("outliers", outliers, torch.int32),
                           self._dev("k_out", k_out), self._dev("v_out", v_out), self._dev("k_loc", k_loc),
                           self._dev("v_loc", v_loc), self._dev("A", A), self._dev("B", B), self._host(v_host),
                           _stream_ptr(stream))
        self._v_host = v_host

    def append(self, k_new, v_new, stream=None):
        shadowkv_append(self.h, self._dev("k_new", k_new), self._dev("v_new", v_new), _stream_ptr(stream))

    def snapkv_select(self, q_obs, pool: int, stream=None):
        """q_obs: (b, h_q, w_obs, d) post-RoPE window queries."""
        c = self.cfg
        if q_obs is None or q_obs.dim() != 4 or tuple(q_obs.shape[:2]) != (c.batch, c.heads_q) \
                or q_obs.shape[3] != c.head_dim:
            raise ValueError(f"q_obs: shape must be ({c.batch}, {c.heads_q}, w_obs, {c.head_dim})")
        w_obs = int(q_obs.shape[2])
        shadowkv_snapkv_select(self.h, self._dev("q_obs", q_obs, shape=tuple(q_obs.shape)), w_obs, pool,
                               _stream_ptr(stream))

    def decode_step(self, q, out, stream=None):
        shadowkv_decode_step(self.h, self._dev("q", q), self._dev("out", out), _stream_ptr(stream))

    def decode_step_noalloc(self, q, out, stream=None):
        shadowkv_decode_step_noalloc(self.h, self._dev("q", q), self._dev("out", out), _stream_ptr(stream))

    def reset_cache(self, stream=None):
        shadowkv_reset_cache(self.h, _stream_ptr(stream))

    def stats(self) -> dict:
        s = shadowkv_get_stats(self.h)
        return {"steps": s.steps, "hits": s.hits, "misses": s.misses, "bytes_h2d": s.bytes_h2d}

    def reset_stats(self):
        shadowkv_reset_stats(self.h)

    def read(self, which: int, stream=None):
        """Copy of the layer's tensor `which` (SKV_T_*) as a device tensor."""
        torch = _torch()
        c = self.cfg
        b, hq, hkv, d, k, ch = c.batch, c.heads_q, c.heads_kv, c.head_dim, c.top_k, c.chunk
        dt = self.dtype
        spec = {
            SKV_T_LANDMARKS: (dt, (b, hkv, self.n, d)), SKV_T_MIN_COS: (torch.float32, (b, hkv, self.n)),
            SKV_T_OUTLIERS: (torch.int32, (b, hkv, c.n_outlier)),
            SKV_T_CAND_MASK: (torch.int32, (b, hkv, (self.n + 31) // 32)),
            SKV_T_SCORES: (torch.float32, (b, hkv, self.n, hq // hkv)),
            SKV_T_GROUP_SCORES: (torch.float32, (b, hkv, self.n)),
            SKV_T_SELECTION: (torch.int32, (b, hkv, k)), SKV_T_SLOT_CHUNKS: (torch.int32, (b, hkv, self.cap)),
            SKV_T_CACHE_V: (dt, (b, hkv, self.cap * ch, d)), SKV_T_K_OUT: (dt, (b, hkv, c.n_outlier * ch, d)),
            SKV_T_V_OUT: (dt, (b, hkv, c.n_outlier * ch, d)), SKV_T_K_LOC: (dt, (b, hkv, c.local_window + c.max_new, d)),
            SKV_T_V_LOC: (dt, (b, hkv, c.local_window + c.max_new, d)),
            SKV_T_SELECTION_SLOTS: (torch.int32, (b, hkv, k)),
            SKV_T_V_CODES: (torch.int32, (b, hkv, self.n)),
        }[which]
        t = torch.empty(spec[1], dtype=spec[0], device=self.device)
        nbytes = t.numel() * t.element_size()
        if nbytes != shadowkv_tensor_bytes(self.h, which):
            raise RuntimeError("tensor size mismatch between binding and library")
        if nbytes:
            shadowkv_read(self.h, which, t.data_ptr(), nbytes, _stream_ptr(stream))
        return t

    def set_overlap(self, enable: bool):
        shadowkv_set_overlap(self.h, enable)

    def set_timing(self, enable: bool):
        shadowkv_set_timing(self.h, enable)

    def get_timing(self) -> tuple[dict, int]:
        ms, steps = shadowkv_get_timing(self.h)
        return dict(zip(KERNELS, ms)), steps

    def close(self):
        if self.h:
            shadowkv_layer_destroy(self.h)
            self.h = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
