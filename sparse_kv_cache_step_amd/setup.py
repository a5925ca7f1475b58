"""Low-rank pre-RoPE key factors (Algorithm 1 step 1), computed once per
sequence outside the decode path.

The review page ("ShadowKV ...", section 三, Algorithm 1 step 1) gives only
the shapes: A (b, s, r) shared by the KV heads and B (b, h_kv, r, d) per head.
Per sequence the keys form the s x (h_kv*d) matrix M whose column h*d+i is
head h's dimension i.  Its rank-r truncated SVD M ~ U_r S_r V_r^T gives
A = U_r S_r = M V_r and B = V_r^T split by head.  V_r is taken from the
eigenvectors of the Gram matrix M^T M (double precision; the Gram product
and the (h_kv*d)^2 eigenproblems run on M's device, or the eigenproblems on
the host with host_eigh=True), which gives the same subspace as the SVD.
This is setup, not part of the decode step: its results are inputs of
shadowkv_prefill_meta.
"""
from __future__ import annotations


def svd_factors(k_pre, rank: int, dtype=None, batch_eigh: int = 8, host_eigh: bool = False):
    """k_pre: (b, h_kv, s, d) tensor (any float dtype, any device).
    Returns (A (b, s, r), B (b, h_kv, r, d)) on k_pre's device in `dtype`
    (default: k_pre's dtype)."""
    import torch

    b, hkv, s, d = k_pre.shape
    hd = hkv * d
    dtype = k_pre.dtype if dtype is None else dtype
    dev = k_pre.device
    A = torch.empty((b, s, rank), dtype=dtype, device=dev)
    B = torch.zeros((b, hkv, rank, d), dtype=dtype, device=dev)
    rr = min(rank, hd)
    for b0 in range(0, b, batch_eigh):
        seqs = range(b0, min(b, b0 + batch_eigh))
        grams = []
        for bi in seqs:
            M = k_pre[bi].transpose(0, 1).reshape(s, hd).to(torch.float64)
            gram = torch.mm(M.t().contiguous(), M)
            grams.append(gram.cpu() if host_eigh else gram)
            del M
        _, vecs = torch.linalg.eigh(torch.stack(grams))  # ascending eigenvalues
        for i, bi in enumerate(seqs):
            V = vecs[i, :, hd - rr:].flip(-1).to(dev)     # (hd, rr), leading first
            M = k_pre[bi].transpose(0, 1).reshape(s, hd).to(torch.float64)
            Ab = torch.mm(M, V)
            if rr < rank:
                Ab = torch.cat([Ab, torch.zeros((s, rank - rr), dtype=Ab.dtype, device=dev)], dim=1)
            A[bi] = Ab.to(dtype)
            B[bi, :, :rr, :] = V.t().reshape(rr, hkv, d).transpose(0, 1).to(dtype)
            del M, Ab
    return A, B
