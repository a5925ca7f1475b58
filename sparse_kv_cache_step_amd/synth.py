"""Seeded synthetic workloads for the ShadowKV decode step.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no RoPE, no landmarks, no SVD, no attention).  Both the
HIP path and the CPU oracle consume exactly the arrays it returns.

Workloads mirror the shapes of the review page's throughput table
(section 五, 吞吐量评估: Llama-3-8B-1M at 60K with batch 48, 128K, GLM-4-9B at
244K with batch 12) and its key-parameter table (chunk 8, rank 160, 48
outlier chunks, a 1.56 % budget).  The page's accuracy suites are not used:
the arrays below stand in for shapes only.

Pre-RoPE keys are a seeded low-rank factor product plus Gaussian noise,
    K_pre[b, h, t, :] = (U_b W_b)[t, h*d:(h+1)*d] + sigma * N(0, 1),
with U_b (s x R) and W_b (R x h_kv*d) entries N(0,1)/sqrt(R).  Values and
queries are N(0, 1).  Queries drift between steps as
    Q_t = rho Q_{t-1} + sqrt(1 - rho^2) N(0, 1),
so consecutive steps select overlapping chunk sets.  A workload may scale the
queries by a constant (q_scale) after drawing them: with N(0,1) queries and
keys of norm ~1 the logits q.k/sqrt(d) have a spread of ~0.1 and attention is
nearly uniform, so a larger scale makes outputs depend sharply on every key.

Seeds: numpy SeedSequence([workload, layer, sequence, tag]) with tag 0 = U,
1 = W, 2 = noise, 3 = V, 4 = Q_0, 5 = Q innovations, 6 = special-chunk choice.
Two generators exist: ``numpy`` (bit-reproducible on any host; used by the
tests) and ``torch`` on a device (for the full-size workloads whose host
generation would take minutes).  They draw different streams from the same
seeds; each is deterministic.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np

TAG_U, TAG_W, TAG_NOISE, TAG_V, TAG_Q0, TAG_QINNOV, TAG_SPECIAL = range(7)


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # seed namespace
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
    bf16: bool
    steps: int
    layers: int
    true_rank: int | tuple[int, int]   # fixed rank, or inclusive range drawn per sequence
    noise: float
    rho: float                # query drift between steps (0: i.i.d.)
    sink_tokens: int = 0      # leading tokens whose K_pre is scaled
    sink_scale: float = 1.0
    n_scaled_chunks: int = 0  # chunks whose whole K_pre is scaled
    chunk_scale: float = 1.0
    n_noisy_chunks: int = 0   # chunks whose noise term is scaled
    noisy_scale: float = 1.0
    rope_base: float = 10000.0
    q_scale: float = 1.0      # every query is drawn, then multiplied by this (sharper attention)

    @property
    def n(self) -> int:
        return self.s // self.c

    @property
    def n_loc(self) -> int:
        return self.w // self.c

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads.  Budget k = n / 64 (1.5625 %) except the tiny one.
TINY_FP32 = Workload("tiny-fp32", 1, b=1, h_q=8, h_kv=2, d=64, s=1024, c=8, r=32, o=4, k=8, w=32,
                     bf16=False, steps=1, layers=1, true_rank=24, noise=0.01, rho=0.0,
                     n_scaled_chunks=4, chunk_scale=5.0)
LLAMA_32K = Workload("llama3-8b-32k-b1", 2, b=1, h_q=32, h_kv=8, d=128, s=32768, c=8, r=160, o=48,
                     k=64, w=32, bf16=True, steps=16, layers=1, true_rank=120, noise=0.02, rho=0.0,
                     sink_tokens=4, sink_scale=8.0)
LLAMA_128K = Workload("llama3-8b-128k-b8", 3, b=8, h_q=32, h_kv=8, d=128, s=131072, c=8, r=160, o=48,
                      k=256, w=32, bf16=True, steps=64, layers=32, true_rank=120, noise=0.02, rho=0.9,
                      sink_tokens=4, sink_scale=8.0)
LLAMA_60K_B48 = Workload("llama3-8b-60k-b48", 4, b=48, h_q=32, h_kv=8, d=128, s=61440, c=8, r=160,
                         o=48, k=120, w=32, bf16=True, steps=32, layers=32, true_rank=(80, 150),
                         noise=0.02, rho=0.9, sink_tokens=4, sink_scale=8.0)
GLM_244K = Workload("glm4-9b-244k-b12", 5, b=12, h_q=32, h_kv=2, d=128, s=249856, c=8, r=160, o=48,
                    k=488, w=32, bf16=True, steps=32, layers=40, true_rank=140, noise=0.02, rho=0.85,
                    n_noisy_chunks=94, noisy_scale=4.0)

WORKLOADS = {w.name: w for w in (TINY_FP32, LLAMA_32K, LLAMA_128K, LLAMA_60K_B48, GLM_244K)}


def _rng(wl: Workload, layer: int, seq: int, tag: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([wl.wid, layer, seq, tag]))


def seed_int(wl: Workload, layer: int, seq: int, tag: int) -> int:
    """A 63-bit integer seed derived from the same SeedSequence."""
    return int(np.random.SeedSequence([wl.wid, layer, seq, tag]).generate_state(2, np.uint64)[0] >> 1)


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """float32 array -> float32 array holding the nearest bfloat16 values
    (round to nearest, ties to even), i.e. the stored inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = ((u + (((u >> 16) & 1) + 0x7FFF)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32)


def _store(wl: Workload, x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return to_bf16_values(x) if wl.bf16 else x


def _true_rank(wl: Workload, layer: int, seq: int) -> int:
    if isinstance(wl.true_rank, tuple):
        lo, hi = wl.true_rank
        return int(_rng(wl, layer, seq, TAG_SPECIAL).integers(lo, hi + 1))
    return int(wl.true_rank)


def special_chunks(wl: Workload, layer: int, seq: int) -> tuple[np.ndarray, np.ndarray]:
    """(scaled chunks, noisy chunks), drawn among chunks outside the local window."""
    g = _rng(wl, layer, seq, TAG_SPECIAL)
    g.integers(0, 2)  # keep this stream independent of the rank draw's position
    pool = wl.n - wl.n_loc
    scaled = np.sort(g.choice(pool, size=wl.n_scaled_chunks, replace=False)) if wl.n_scaled_chunks else np.zeros(0, np.int64)
    noisy = np.sort(g.choice(pool, size=wl.n_noisy_chunks, replace=False)) if wl.n_noisy_chunks else np.zeros(0, np.int64)
    return scaled, noisy


# --------------------------------------------------------------------------
# numpy generator (host)
# --------------------------------------------------------------------------
def k_pre_numpy(wl: Workload, layer: int = 0) -> np.ndarray:
    """(b, h_kv, s, d) pre-RoPE keys in the storage type's values (float32)."""
    out = np.empty((wl.b, wl.h_kv, wl.s, wl.d), dtype=np.float32)
    hd = wl.h_kv * wl.d
    for seq in range(wl.b):
        R = _true_rank(wl, layer, seq)
        U = _rng(wl, layer, seq, TAG_U).standard_normal((wl.s, R)) / np.sqrt(R)
        W = _rng(wl, layer, seq, TAG_W).standard_normal((R, hd)) / np.sqrt(R)
        noise = _rng(wl, layer, seq, TAG_NOISE).standard_normal((wl.s, hd)) * wl.noise
        scaled, noisy = special_chunks(wl, layer, seq)
        for j in noisy:
            noise[j * wl.c:(j + 1) * wl.c] *= wl.noisy_scale
        K = U @ W + noise
        for j in scaled:
            K[j * wl.c:(j + 1) * wl.c] *= wl.chunk_scale
        if wl.sink_tokens:
            K[:wl.sink_tokens] *= wl.sink_scale
        out[seq] = _store(wl, K.reshape(wl.s, wl.h_kv, wl.d).transpose(1, 0, 2))
    return out


def v_numpy(wl: Workload, layer: int = 0) -> np.ndarray:
    out = np.empty((wl.b, wl.h_kv, wl.s, wl.d), dtype=np.float32)
    for seq in range(wl.b):
        out[seq] = _store(wl, _rng(wl, layer, seq, TAG_V).standard_normal((wl.h_kv, wl.s, wl.d)))
    return out


def queries_numpy(wl: Workload, layer: int = 0, steps: int | None = None) -> np.ndarray:
    """(steps, b, h_q, d) post-RoPE queries, drifting with rho."""
    steps = wl.steps if steps is None else steps
    out = np.empty((steps, wl.b, wl.h_q, wl.d), dtype=np.float32)
    for seq in range(wl.b):
        q = _rng(wl, layer, seq, TAG_Q0).standard_normal((wl.h_q, wl.d))
        innov = _rng(wl, layer, seq, TAG_QINNOV)
        for t in range(steps):
            if t > 0:
                q = wl.rho * q + np.sqrt(1.0 - wl.rho ** 2) * innov.standard_normal((wl.h_q, wl.d))
            out[t, seq] = _store(wl, q * wl.q_scale)
    return out


# --------------------------------------------------------------------------
# torch generator (device), for the full-size workloads
# --------------------------------------------------------------------------
def _tgen(torch, device, wl, layer, seq, tag):
    g = torch.Generator(device=device)
    g.manual_seed(seed_int(wl, layer, seq, tag))
    return g


def _tstore(torch, wl, x):
    return x.to(torch.bfloat16) if wl.bf16 else x.to(torch.float32)


def k_pre_torch(wl: Workload, layer: int, device, seqs=None):
    """Like k_pre_numpy but drawn with torch's generator on `device`; returns a
    (len(seqs), h_kv, s, d) tensor in the storage dtype."""
    import torch
    seqs = range(wl.b) if seqs is None else seqs
    hd = wl.h_kv * wl.d
    out = torch.empty((len(seqs), wl.h_kv, wl.s, wl.d), dtype=torch.bfloat16 if wl.bf16 else torch.float32,
                      device=device)
    for i, seq in enumerate(seqs):
        R = _true_rank(wl, layer, seq)
        U = torch.randn((wl.s, R), generator=_tgen(torch, device, wl, layer, seq, TAG_U), device=device) / R ** 0.5
        W = torch.randn((R, hd), generator=_tgen(torch, device, wl, layer, seq, TAG_W), device=device) / R ** 0.5
        K = torch.randn((wl.s, hd), generator=_tgen(torch, device, wl, layer, seq, TAG_NOISE), device=device)
        K.mul_(wl.noise)
        scaled, noisy = special_chunks(wl, layer, seq)
        for j in noisy:
            K[j * wl.c:(j + 1) * wl.c] *= wl.noisy_scale
        K.addmm_(U, W)
        for j in scaled:
            K[j * wl.c:(j + 1) * wl.c] *= wl.chunk_scale
        if wl.sink_tokens:
            K[:wl.sink_tokens] *= wl.sink_scale
        out[i] = _tstore(torch, wl, K.view(wl.s, wl.h_kv, wl.d).transpose(0, 1))
        del U, W, K
    return out


def v_torch(wl: Workload, layer: int, device, seqs=None):
    import torch
    seqs = range(wl.b) if seqs is None else seqs
    out = torch.empty((len(seqs), wl.h_kv, wl.s, wl.d), dtype=torch.bfloat16 if wl.bf16 else torch.float32,
                      device=device)
    for i, seq in enumerate(seqs):
        g = _tgen(torch, device, wl, layer, seq, TAG_V)
        for h in range(wl.h_kv):
            out[i, h] = _tstore(torch, wl, torch.randn((wl.s, wl.d), generator=g, device=device))
    return out


def queries_torch(wl: Workload, layer: int, device, steps: int | None = None):
    """(steps, b, h_q, d) drifting queries in the storage dtype on `device`."""
    import torch
    steps = wl.steps if steps is None else steps
    out = torch.empty((steps, wl.b, wl.h_q, wl.d), dtype=torch.bfloat16 if wl.bf16 else torch.float32,
                      device=device)
    a = float(np.sqrt(1.0 - wl.rho ** 2))
    for seq in range(wl.b):
        q = torch.randn((wl.h_q, wl.d), generator=_tgen(torch, device, wl, layer, seq, TAG_Q0), device=device)
        g = _tgen(torch, device, wl, layer, seq, TAG_QINNOV)
        for t in range(steps):
            if t > 0:
                q = wl.rho * q + a * torch.randn((wl.h_q, wl.d), generator=g, device=device)
            out[t, seq] = _tstore(torch, wl, q * wl.q_scale)
    return out
