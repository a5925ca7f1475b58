"""The device factorisation (shadowkv_factorize; the ShadowKV review page,
section 三, Algorithm 1 step 1, A, B <- SVD(K_pre)) against the oracle's
LAPACK SVD of the same keys.

Reference: the oracle's factors stored in binary32 (``oracle.svd_factors`` of
a binary32 shape), whose products A . B are the rank-r approximations of the
heads' keys to ~1e-7.  Checked per sequence:
  * A . B per head, in relative Frobenius norm; for bfloat16 factors the bar
    is what correctly rounded factors reach (the oracle's own bfloat16
    factors) plus a margin;
  * the singular values (column norms of A);
  * orthonormal rows of B (all heads together);
  * zero columns of A and rows of B past n = h_kv * d;
  * batches of more than the eight sequences solved at once;
  * the eigensolver's round forms (super-blocks of 32 and of 64 indices,
    single index pairs);
  * all-zero keys (the degenerate case: A = 0, orthonormal B, finite).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from parity_helpers import log, oracle_shape, tdtype, to_dev, to_np
from sparse_kv_cache_step_amd import binding as skv
from sparse_kv_cache_step_amd import synth

pytestmark = pytest.mark.gpu

CASES = {
    "tiny-fp32": synth.TINY_FP32,
    "tiny-fp32-rank-past-n": synth.TINY_FP32.with_(h_kv=1, s=512, r=96, true_rank=40),
    "fp32-b10": synth.TINY_FP32.with_(b=10, s=256, r=16, true_rank=12),
    "bf16-llama-32k": synth.LLAMA_32K,
    "bf16-glm-shape": synth.GLM_244K.with_(b=2, s=8192),
    # the largest n the call takes (h_kv * d = 2048): 128 block places, 64 super-blocks
    "bf16-n2048": synth.LLAMA_32K.with_(b=1, h_kv=16, s=4096),
}


def _products(A, B):
    """A (b, s, r), B (b, h, r, d) -> (b, h, s, d) in float64."""
    return np.einsum("bsr,bhrd->bhsd", A, B)


# The eigensolver's round forms: super-blocks of 32 indices (blocks of 16,
# the default), of 64 indices (blocks of 32, asked for), and single index
# pairs.
PATHS = {"block": "1", "block32": "32", "single": "0"}
PARAMS = ([(c, "block") for c in CASES] + [("tiny-fp32", "block32"), ("bf16-glm-shape", "block32"),
                                           ("bf16-llama-32k", "block32")]
          + [("tiny-fp32", "single"), ("bf16-glm-shape", "single")])


@pytest.mark.parametrize("case,path", PARAMS, ids=[f"{c}-{p}" for c, p in PARAMS])
def test_factorize_matches_the_oracle_svd(case, path, monkeypatch):
    monkeypatch.setenv("SKV_FACTOR_BLOCK", PATHS[path])
    wl = CASES[case]
    k_pre = synth.k_pre_numpy(wl)
    b, hkv, s, d = k_pre.shape
    n, r = hkv * d, wl.r
    rr = min(r, n)
    log(f"[{case}/{path}] b={b} h_kv={hkv} s={s} d={d} r={r} n={n} dtype={'bf16' if wl.bf16 else 'f32'}")
    A_g, B_g, sweeps = skv.factorize(to_dev(k_pre, tdtype(wl)), r, return_sweeps=True)
    torch.cuda.synchronize()
    A_g, B_g = to_np(A_g), to_np(B_g)
    log(f"[{case}] device factors in {sweeps} Jacobi sweeps")
    assert 1 <= sweeps <= 30
    shape32 = dataclasses.replace(oracle_shape(wl), bf16=False)
    A_o, B_o = oracle.svd_factors(shape32, k_pre)
    P_o = _products(A_o, B_o)
    P_g = _products(A_g, B_g)
    if wl.bf16:
        A_r, B_r = oracle.svd_factors(oracle_shape(wl), k_pre)  # correctly rounded factors
        P_r = _products(A_r, B_r)
    for bi in range(b):
        ref = np.linalg.norm(P_o[bi])
        err = np.linalg.norm(P_g[bi] - P_o[bi]) / ref
        bar = 1e-6
        if wl.bf16:
            rounded = np.linalg.norm(P_r[bi] - P_o[bi]) / ref
            bar = 1.5 * rounded + 1e-5
            log(f"[{case}] seq {bi}: |AB - AB_oracle| / |AB_oracle| = {err:.3g} (rounded oracle factors: {rounded:.3g})")
        else:
            log(f"[{case}] seq {bi}: |AB - AB_oracle| / |AB_oracle| = {err:.3g}")
        assert err <= bar
        # singular values: column norms of A
        sv_o = np.linalg.norm(A_o[bi, :, :rr], axis=0)
        sv_g = np.linalg.norm(A_g[bi, :, :rr], axis=0)
        sv_tol = 4e-3 if wl.bf16 else 1e-5
        assert np.all(np.abs(sv_g - sv_o) <= sv_tol * sv_o[0])
        assert np.all(np.diff(sv_g) <= sv_tol * sv_o[0])  # leading first
        # orthonormal rows of B over all heads
        Bm = B_g[bi, :, :rr, :].transpose(1, 0, 2).reshape(rr, n)
        gram = Bm @ Bm.T
        assert np.max(np.abs(gram - np.eye(rr))) <= (1.6e-2 if wl.bf16 else 1e-5)
        # nothing past n
        assert np.all(A_g[bi, :, rr:] == 0) and np.all(B_g[bi, :, rr:, :] == 0)
    if r >= n:
        # full rank: the factors reproduce the keys
        M = k_pre.astype(np.float64)
        assert np.max(np.abs(P_g - M)) <= 1e-5 * np.max(np.abs(M))


@pytest.mark.parametrize("path", list(PATHS))
def test_factorize_zero_keys(path, monkeypatch):
    """All-zero keys: the Gram matrix is zero, every rotation is skipped and
    the first sweep's measure (0 of 0) decides; the factors are A = 0 and
    orthonormal rows of B (the singular vectors of a zero matrix are any
    orthonormal set), with nothing non-finite."""
    monkeypatch.setenv("SKV_FACTOR_BLOCK", PATHS[path])
    b, hkv, s, d, r = 2, 2, 256, 64, 24
    k_pre = torch.zeros((b, hkv, s, d), dtype=torch.float32, device="cuda")
    A_g, B_g, sweeps = skv.factorize(k_pre, r, return_sweeps=True)
    torch.cuda.synchronize()
    A_g, B_g = to_np(A_g), to_np(B_g)
    log(f"[zero keys/{path}] {sweeps} sweeps")
    assert 1 <= sweeps <= 2
    assert np.all(np.isfinite(A_g)) and np.all(np.isfinite(B_g))
    assert np.all(A_g == 0)
    n = hkv * d
    for bi in range(b):
        Bm = B_g[bi].transpose(1, 0, 2).reshape(r, n)
        assert np.max(np.abs(Bm @ Bm.T - np.eye(r))) <= 1e-6
