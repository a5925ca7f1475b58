"""shadowkv_decode_step_noalloc (the step's scratch in the library's static
device array) against shadowkv_decode_step (the layer's own scratch), called
through the C ABI on identical layers: two calls in a row, the second on a
smaller layer, must give the same selections, cache contents, hit counts
and outputs within the bfloat16 bar (the same kernels run, so equality is
expected); a layer whose step needs more scratch than the array holds is
refused before any work is enqueued."""
import numpy as np
import pytest
import torch

from parity_helpers import OUT_TOL, layer_kwargs, log, tdtype, to_dev
from sparse_kv_cache_step_amd import binding as skv
from sparse_kv_cache_step_amd import synth

pytestmark = pytest.mark.gpu


def _pair(wl):
    """Two layers prefilled from the same inputs."""
    dt = tdtype(wl)
    k_pre, v = synth.k_pre_numpy(wl), synth.v_numpy(wl)
    k_d, v_d = to_dev(k_pre, dt), to_dev(v, dt)
    A, B = skv.factorize(k_d, wl.r)
    out = []
    for _ in range(2):
        lay = skv.Layer(**layer_kwargs(wl))
        hb = lay.host_buffer()
        lay.prefill_meta(k_d, v_d, A, B, hb)
        out.append((lay, hb))
    torch.cuda.synchronize()
    return out


def test_noalloc_matches_decode_step_two_calls():
    # 64 (sequence, KV head) rows: one-pass selection, GQA 4: fused attention
    big = synth.LLAMA_32K.with_(b=8, s=8192, k=16, steps=3, rho=0.9)
    # 1 row pair: two-pass selection, GQA 16: separate QK + PV kernels
    small = synth.GLM_244K.with_(b=1, s=4096, o=6, k=9, steps=3, rho=0.85)
    for wl in (big, small):
        (ref, hb1), (nal, hb2) = _pair(wl)
        qs = synth.queries_numpy(wl)
        for t in range(wl.steps):
            q = to_dev(qs[t], tdtype(wl))
            o_ref, o_nal = torch.empty_like(q), torch.empty_like(q)
            ref.decode_step(q, o_ref)
            nal.decode_step_noalloc(q, o_nal)
            torch.cuda.synchronize()
            err = float((o_ref.float() - o_nal.float()).abs().max())
            log(f"[noalloc {wl.name} b={wl.b} s={wl.s}] step {t}: max|noalloc - decode_step| = {err:.3g}, "
                f"bitwise {torch.equal(o_ref, o_nal)}")
            assert err <= OUT_TOL[wl.bf16]
            assert torch.equal(ref.read(skv.SKV_T_SELECTION), nal.read(skv.SKV_T_SELECTION))
            assert torch.equal(ref.read(skv.SKV_T_SLOT_CHUNKS), nal.read(skv.SKV_T_SLOT_CHUNKS))
            assert torch.equal(ref.read(skv.SKV_T_CACHE_V), nal.read(skv.SKV_T_CACHE_V))
        assert ref.stats() == nal.stats()
        for lay, hb in ((ref, hb1), (nal, hb2)):
            lay.close()
            hb.free()


def test_noalloc_refuses_a_step_larger_than_its_scratch():
    # one-token chunks: U alone is 4 x 8 x 131072 x 16 x 4 B = 268 MB.  The
    # size is checked before anything else, so no prefill (and no kernel) is
    # needed to see the refusal.
    lay = skv.Layer(batch=4, heads_q=128, heads_kv=8, head_dim=64, seq_len=131072, chunk=1, rank=32,
                    n_outlier=8, top_k=64, local_window=32, bf16=True)
    q = torch.zeros((4, 128, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(skv.ShadowKVError) as e:
        lay.decode_step_noalloc(q, torch.empty_like(q))
    assert e.value.code == skv.SKV_E_SHAPE and "static scratch" in str(e.value)
    # a layer that fits but has no prefill yet is refused as before
    small = skv.Layer(batch=1, heads_q=8, heads_kv=2, head_dim=64, seq_len=1024, chunk=8, rank=32,
                      n_outlier=4, top_k=8, local_window=32, bf16=True)
    q2 = torch.zeros((1, 8, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(skv.ShadowKVError) as e:
        small.decode_step_noalloc(q2, torch.empty_like(q2))
    assert e.value.code == skv.SKV_E_STATE
    lay.close()
    small.close()
