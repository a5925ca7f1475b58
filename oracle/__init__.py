"""ShadowKV sparse decode step -- CPU oracle (Python side).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
CPU-baseline leg of the benchmark import this package.  It never imports the
HIP library or anything from the product package, and the product package
never imports it.

The arithmetic lives in ``shadowkv_oracle.c`` (double precision, one plain
loop nest per step of the review page's Algorithms 1 and 2).  This wrapper
adds the two steps that are library routines or pure bookkeeping:

* ``svd_factors`` -- Algorithm 1 step 1, ``A, B <- SVD(K)`` on the pre-RoPE
  keys, done with LAPACK's SVD (numpy) in double precision.  The page fixes
  only the shapes, A (b, s, r) shared by all KV heads and B (b, h_kv, r, d);
  the reading taken is: per sequence, K is the s x (h_kv*d) matrix whose
  column h*d+i is head h's dimension i, A = U_r Sigma_r and B = V_r^T split by
  head.
* ``CacheSim`` -- the per-layer set-difference cache of the Telegram write-up
  ("Часть II"): at step t only I_t \\ I_{t-1} is loaded, the rest is reused.
  The attended set is always I_t, so the cache changes no output; the
  simulation yields the hit count that defines the hit rate alpha.  A larger
  least-recently-used capacity is the same cache keeping more than one step's
  chunks (a reading: the pages size the cache only by the selection).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "shadowkv_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_D = ctypes.POINTER(ctypes.c_double)
_I32 = ctypes.POINTER(ctypes.c_int32)
_U8 = ctypes.POINTER(ctypes.c_uint8)


class _Cfg(ctypes.Structure):
    _fields_ = [
        ("b", ctypes.c_int32), ("h_q", ctypes.c_int32), ("h_kv", ctypes.c_int32),
        ("d", ctypes.c_int32), ("s", ctypes.c_int32), ("c", ctypes.c_int32),
        ("r", ctypes.c_int32), ("o", ctypes.c_int32), ("k", ctypes.c_int32),
        ("w", ctypes.c_int32), ("rope_base", ctypes.c_double), ("bf16", ctypes.c_int32),
        ("n_app", ctypes.c_int32), ("plant", ctypes.c_int32),
    ]


# Deliberate mistakes orc_attend can plant in the rebuilt-key block; only the
# tests that show a parity case discriminates use them.  PLANT_BF16_REBUILT is
# no mistake: the rebuilt, rotated keys rounded to bfloat16 before the logits,
# as the bfloat16 kernels do (the share of the error bar that rounding uses).
(PLANT_NONE, PLANT_ZERO_REBUILT, PLANT_NO_ROPE_REBUILT, PLANT_POS_PLUS_ONE, PLANT_NO_OUTLIERS,
 PLANT_BF16_REBUILT) = range(6)


@dataclass(frozen=True)
class Shape:
    """Sizes of one layer (the review page's Algorithm 1 input list)."""
    b: int
    h_q: int
    h_kv: int
    d: int
    s: int
    c: int
    r: int
    o: int
    k: int
    w: int
    rope_base: float = 10000.0
    bf16: bool = False

    @property
    def n(self) -> int:
        return self.s // self.c

    def _c(self, n_app: int = 0, plant: int = PLANT_NONE) -> _Cfg:
        return _Cfg(self.b, self.h_q, self.h_kv, self.d, self.s, self.c, self.r,
                    self.o, self.k, self.w, float(self.rope_base), int(self.bf16), int(n_app), int(plant))


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, IEEE arithmetic, OpenMP)."""
    if force or not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(_SRC):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        build()
        lib = ctypes.CDLL(LIB_PATH)
        lib.orc_round_bf16.restype = ctypes.c_double
        lib.orc_round_bf16.argtypes = [ctypes.c_double]
        lib.orc_round_bf16_n.restype = None
        lib.orc_round_bf16_n.argtypes = [_D, ctypes.c_int64]
        lib.orc_rope_row.restype = None
        lib.orc_rope_row.argtypes = [_D, _D, ctypes.c_int32, ctypes.c_double, ctypes.c_double]
        lib.orc_topk.restype = ctypes.c_int
        lib.orc_topk.argtypes = [_D, _U8, ctypes.c_int32, ctypes.c_int32, _I32]
        lib.orc_prefill.restype = ctypes.c_int
        lib.orc_prefill.argtypes = [ctypes.POINTER(_Cfg), _D, _D, _D, _D, _I32, _D, _D, _D, _D, _U8]
        lib.orc_attend.restype = ctypes.c_int
        lib.orc_attend.argtypes = [ctypes.POINTER(_Cfg), _D, _I32, _D, _D, _D, _D, _D, _D, _D, _D]
        lib.orc_decode.restype = ctypes.c_int
        lib.orc_decode.argtypes = [ctypes.POINTER(_Cfg), _D, _D, _U8, _D, _D, _D, _D, _D, _D, _D,
                                   _D, _D, _I32, _D]
        lib.orc_equiv_bandwidth.restype = ctypes.c_double
        lib.orc_equiv_bandwidth.argtypes = [ctypes.c_double] * 7
        _lib_handle = lib
    return _lib_handle


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


# --------------------------------------------------------------------------
# Small building blocks (exposed for the pins)
# --------------------------------------------------------------------------
def round_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of each element, as float64."""
    y = np.array(x, dtype=np.float64, order="C", copy=True)
    _lib().orc_round_bf16_n(_p(y, _D), y.size)
    return y


def round_store(x, bf16: bool) -> np.ndarray:
    """Round to the storage type: bfloat16 or binary32."""
    return round_bf16(x) if bf16 else _f64(x).astype(np.float32).astype(np.float64)


def rope(x, pos: float, base: float = 10000.0) -> np.ndarray:
    """Rotate-half RoPE of one vector at one position, double precision."""
    x = _f64(x)
    y = np.empty_like(x)
    _lib().orc_rope_row(_p(x, _D), _p(y, _D), x.shape[-1], float(pos), float(base))
    return y


def topk(key, k: int, valid=None) -> np.ndarray:
    """Indices of the k largest keys (ties to the lower index), ascending."""
    key = _f64(key)
    v = None if valid is None else np.ascontiguousarray(valid, dtype=np.uint8)
    out = np.empty(k, dtype=np.int32)
    rc = _lib().orc_topk(_p(key, _D), None if v is None else _p(v, _U8), key.size, k, _p(out, _I32))
    _check(rc, "topk")
    return out


def equiv_bandwidth(S, C, K, O, alpha, b_gpu, b_pcie) -> float:
    """Equivalent bandwidth of section 三's 核心公式 (same unit as b_gpu)."""
    return _lib().orc_equiv_bandwidth(S, C, K, O, alpha, b_gpu, b_pcie)


# --------------------------------------------------------------------------
# Algorithm 1 step 1: truncated SVD of the pre-RoPE keys (LAPACK via numpy)
# --------------------------------------------------------------------------
def svd_factors(shape: Shape, k_pre) -> tuple[np.ndarray, np.ndarray]:
    """A (b, s, r) and B (b, h_kv, r, d) with A[b] @ B[b, h] the rank-r
    approximation of head h's keys; both rounded to the storage type."""
    k_pre = _f64(k_pre)
    b, hkv, s, d = k_pre.shape
    r = shape.r
    A = np.zeros((b, s, r))
    B = np.zeros((b, hkv, r, d))
    for bi in range(b):
        M = k_pre[bi].transpose(1, 0, 2).reshape(s, hkv * d)
        U, S, Vt = np.linalg.svd(M, full_matrices=False)
        rr = min(r, S.size)
        A[bi, :, :rr] = U[:, :rr] * S[:rr]
        B[bi, :, :rr, :] = Vt[:rr].reshape(rr, hkv, d).transpose(1, 0, 2)
    return round_store(A, shape.bf16), round_store(B, shape.bf16)


# --------------------------------------------------------------------------
# Algorithm 1 steps 2-5
# --------------------------------------------------------------------------
def prefill(shape: Shape, k_pre, v) -> dict:
    k_pre, v = _f64(k_pre), _f64(v)
    b, hkv, d, n, o, c, w = shape.b, shape.h_kv, shape.d, shape.n, shape.o, shape.c, shape.w
    assert k_pre.shape == (b, hkv, shape.s, d) and v.shape == k_pre.shape
    out = dict(
        landmarks=np.empty((b, hkv, n, d)), min_cos=np.empty((b, hkv, n)),
        outliers=np.empty((b, hkv, o), dtype=np.int32),
        k_out=np.empty((b, hkv, o * c, d)), v_out=np.empty((b, hkv, o * c, d)),
        k_loc=np.empty((b, hkv, w, d)), v_loc=np.empty((b, hkv, w, d)),
        cand=np.empty((b, hkv, n), dtype=np.uint8),
    )
    cfg = shape._c()
    rc = _lib().orc_prefill(ctypes.byref(cfg), _p(k_pre, _D), _p(v, _D),
                            _p(out["landmarks"], _D), _p(out["min_cos"], _D),
                            _p(out["outliers"], _I32), _p(out["k_out"], _D), _p(out["v_out"], _D),
                            _p(out["k_loc"], _D), _p(out["v_loc"], _D), _p(out["cand"], _U8))
    _check(rc, "prefill")
    return out


# --------------------------------------------------------------------------
# Decode-token append: the token generated at position s + t joins the dense
# local block (the third key block of Algorithm 2 step 4), its key rotated at
# that position like every other stored key and rounded once to storage.
# --------------------------------------------------------------------------
def append(shape: Shape, meta: dict, k_new, v_new) -> dict:
    """meta with the new token's key (pre-RoPE, (b, h_kv, d)) and value
    appended to k_loc / v_loc; the token's position is s plus the number of
    tokens appended before it."""
    k_new, v_new = _f64(k_new), _f64(v_new)
    b, hkv, d = shape.b, shape.h_kv, shape.d
    assert k_new.shape == (b, hkv, d) and v_new.shape == (b, hkv, d)
    pos = shape.s + _n_app(shape, meta)
    k_rot = np.empty_like(k_new)
    for bi in range(b):
        for h in range(hkv):
            k_rot[bi, h] = rope(k_new[bi, h], pos, shape.rope_base)
    out = dict(meta)
    out["k_loc"] = np.concatenate([_f64(meta["k_loc"]), round_store(k_rot, shape.bf16)[:, :, None, :]], axis=2)
    out["v_loc"] = np.concatenate([_f64(meta["v_loc"]), v_new[:, :, None, :]], axis=2)
    return out


def _n_app(shape: Shape, meta: dict) -> int:
    n = meta["k_loc"].shape[2] - shape.w
    assert n >= 0 and meta["v_loc"].shape[2] == shape.w + n
    return n


# --------------------------------------------------------------------------
# Algorithm 2
# --------------------------------------------------------------------------
def attend(shape: Shape, q, sel, A, B, v_host, meta: dict, plant: int = PLANT_NONE) -> np.ndarray:
    """Algorithm 2 steps 3-4 for a given selection (b, h_kv, k).  `plant`
    (tests only) plants one of the PLANT_* mistakes."""
    q, A, B, v_host = _f64(q), _f64(A), _f64(B), _f64(v_host)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    assert sel.shape == (shape.b, shape.h_kv, shape.k)
    out = np.empty((shape.b, shape.h_q, shape.d))
    cfg = shape._c(_n_app(shape, meta), plant)
    m = {key: _f64(meta[key]) for key in ("k_out", "v_out", "k_loc", "v_loc")}
    rc = _lib().orc_attend(ctypes.byref(cfg), _p(q, _D), _p(sel, _I32), _p(A, _D), _p(B, _D),
                           _p(v_host, _D), _p(m["k_out"], _D), _p(m["v_out"], _D),
                           _p(m["k_loc"], _D), _p(m["v_loc"], _D), _p(out, _D))
    _check(rc, "attend")
    return out


def decode(shape: Shape, q, meta: dict, A, B, v_host) -> dict:
    """One decode step: P, S2, the selection I and the attention output."""
    q, A, B, v_host = _f64(q), _f64(A), _f64(B), _f64(v_host)
    b, hq, hkv, n, d, k = shape.b, shape.h_q, shape.h_kv, shape.n, shape.d, shape.k
    assert q.shape == (b, hq, d)
    res = dict(P=np.empty((b, hq, n)), S2=np.empty((b, hkv, n)),
               sel=np.empty((b, hkv, k), dtype=np.int32), out=np.empty((b, hq, d)))
    m = {key: _f64(meta[key]) for key in ("landmarks", "k_out", "v_out", "k_loc", "v_loc")}
    cand = np.ascontiguousarray(meta["cand"], dtype=np.uint8)
    cfg = shape._c(_n_app(shape, meta))
    rc = _lib().orc_decode(ctypes.byref(cfg), _p(q, _D), _p(m["landmarks"], _D), _p(cand, _U8),
                           _p(A, _D), _p(B, _D), _p(v_host, _D), _p(m["k_out"], _D),
                           _p(m["v_out"], _D), _p(m["k_loc"], _D), _p(m["v_loc"], _D),
                           _p(res["P"], _D), _p(res["S2"], _D), _p(res["sel"], _I32),
                           _p(res["out"], _D))
    _check(rc, "decode")
    return res


# --------------------------------------------------------------------------
# SnapKV-style selection (the SnapKV review page, 核心公式: importance =
# attention summed over the heads and the observation window's queries, then
# average pooling, then Top-K), at chunk level against the landmarks: the
# selection is made once from a window of queries and then kept.
# --------------------------------------------------------------------------
def snapkv_scores(shape: Shape, q_obs, meta: dict) -> np.ndarray:
    """(b, h_kv, n): for each KV head, the softmax over selectable chunks of
    q . L^T / sqrt(d), summed over the group's query heads and the window's
    queries (0 elsewhere).  q_obs: (b, h_q, w_obs, d) post-RoPE."""
    q_obs = _f64(q_obs)
    b, hq, w_obs, d = q_obs.shape
    assert (b, hq, d) == (shape.b, shape.h_q, shape.d)
    # each (query head, window position) pair as a query head of its group:
    # the decode step's group score of these heads is their mean softmax
    virt = Shape(b=shape.b, h_q=hq * w_obs, h_kv=shape.h_kv, d=d, s=shape.s, c=shape.c, r=shape.r, o=shape.o,
                 k=shape.k, w=shape.w, rope_base=shape.rope_base, bf16=shape.bf16)
    q = q_obs.reshape(b, hq * w_obs, d)
    res = dict(P=np.empty((b, hq * w_obs, shape.n)), S2=np.empty((b, shape.h_kv, shape.n)),
               sel=np.empty((b, shape.h_kv, shape.k), dtype=np.int32), out=np.empty((b, hq * w_obs, d)))
    m = {key: _f64(meta[key]) for key in ("landmarks", "k_out", "v_out", "k_loc", "v_loc")}
    cand = np.ascontiguousarray(meta["cand"], dtype=np.uint8)
    zero_a = np.zeros((b, shape.s, shape.r))
    zero_b = np.zeros((b, shape.h_kv, shape.r, d))
    zero_v = np.zeros((b, shape.h_kv, shape.s, d))
    cfg = virt._c(_n_app(shape, meta))
    rc = _lib().orc_decode(ctypes.byref(cfg), _p(q, _D), _p(m["landmarks"], _D), _p(cand, _U8),
                           _p(zero_a, _D), _p(zero_b, _D), _p(zero_v, _D), _p(m["k_out"], _D),
                           _p(m["v_out"], _D), _p(m["k_loc"], _D), _p(m["v_loc"], _D),
                           _p(res["P"], _D), _p(res["S2"], _D), _p(res["sel"], _I32), _p(res["out"], _D))
    _check(rc, "snapkv scores")
    return res["S2"] * (hq // shape.h_kv) * w_obs


def snapkv_select(shape: Shape, q_obs, meta: dict, pool: int) -> dict:
    """The importance of snapkv_scores, average-pooled over `pool` (odd)
    neighbouring chunks (zero padding, divided by `pool`), then the k
    selectable chunks of largest pooled importance (ties to the lower index,
    decided on binary32 values like the decode step), ascending."""
    assert pool >= 1 and pool % 2 == 1
    S = snapkv_scores(shape, q_obs, meta)
    half = pool // 2
    pad = np.pad(S, ((0, 0), (0, 0), (half, half)))
    pooled = sum(pad[:, :, i:i + shape.n] for i in range(pool)) / pool
    cand = meta["cand"].astype(bool)
    pooled = np.where(cand, pooled, 0.0)
    sel = np.empty((shape.b, shape.h_kv, shape.k), dtype=np.int32)
    for bi in range(shape.b):
        for h in range(shape.h_kv):
            key = pooled[bi, h].astype(np.float32).astype(np.float64)
            sel[bi, h] = topk(key, shape.k, cand[bi, h])
    return dict(S=S, pooled=pooled, sel=sel)


class CacheSim:
    """Per-layer resident set of the V cache.  With capacity None (the
    set-difference cache of the ShadowKV review page: adjacent decoding steps
    share chunks) R_t = I_t, and step t loads only I_t \\ R_{t-1}.  With a
    capacity C >= k chunks per (sequence, KV head) the cache is least recently
    used: R_t holds I_t and, of R_{t-1} \\ I_t, the C - k chunks selected most
    recently (equal steps: the lower chunk index stays).  Capacity k is the
    set-difference cache."""

    def __init__(self, b: int, h_kv: int, capacity: int | None = None):
        self.capacity = capacity
        self.step_no = 0
        # per row: chunk -> the last step that selected it
        self.resident = [[{} for _ in range(h_kv)] for _ in range(b)]

    def step(self, sel) -> tuple[int, int]:
        """Returns (hits, misses) summed over sequences and KV heads."""
        sel = np.asarray(sel)
        self.step_no += 1
        hits = misses = 0
        for bi, row in enumerate(self.resident):
            for h in range(len(row)):
                cur = set(int(x) for x in sel[bi, h])
                hit = len(cur & row[h].keys())
                hits += hit
                misses += len(cur) - hit
                cap = len(cur) if self.capacity is None else self.capacity
                assert cap >= len(cur)
                others = sorted((j for j in row[h] if j not in cur), key=lambda j: (-row[h][j], j))
                kept = {j: row[h][j] for j in others[:cap - len(cur)]}
                kept.update({j: self.step_no for j in cur})
                row[h] = kept
        return hits, misses

    def reset(self) -> None:
        for row in self.resident:
            for h in range(len(row)):
                row[h] = {}
