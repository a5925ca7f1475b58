"""CPU-side checks of the C ABI: the library loads without a GPU, exports
every function include/shadowkv.h declares, evaluates the page's bandwidth
formula, and rejects invalid layer sizes before touching the device."""
import os
import re
import subprocess

import pytest

from sparse_kv_cache_step_amd import binding as skv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "shadowkv.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(skv.LIB_PATH):
        from sparse_kv_cache_step_amd import build
        build.build(force=False)
    return skv.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(shadowkv_\w+)\s*\(", text)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(skv.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", skv.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\bT (shadowkv_\w+)", out.stdout))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_config_struct_matches_the_header():
    """The binding's skv_config fields are the header's, in order, with the
    same widths."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{([^}]*)\} skv_config;", text).group(1)
    fields = re.findall(r"\b(int32_t|float)\s+(\w+);", body)
    ctype = {"int32_t": "c_int", "float": "c_float"}
    got = [(name, t.__name__) for name, t in skv.skv_config._fields_]
    assert got == [(name, ctype[t]) for t, name in fields]


def test_equiv_bandwidth_closed_form(lib):
    bw = skv.shadowkv_equiv_bandwidth(131072, 8, 256, 48, 0.6, 2e12, 31.5e9)
    assert round(bw / 1e12, 1) == 7.2


def _cfg(**kw):
    base = dict(batch=1, heads_q=8, heads_kv=2, head_dim=64, seq_len=1024, chunk=8, rank=32, n_outlier=4, top_k=8,
                local_window=32, rope_base=10000.0, dtype=skv.SKV_F32)
    base.update(kw)
    return skv.skv_config(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), skv.SKV_E_INVAL),
    (dict(head_dim=96), skv.SKV_E_SHAPE),
    (dict(heads_q=6, heads_kv=4), skv.SKV_E_SHAPE),
    (dict(heads_q=34, heads_kv=2), skv.SKV_E_SHAPE),       # group of 17
    (dict(seq_len=1020), skv.SKV_E_SHAPE),                  # not a multiple of the chunk
    (dict(local_window=12), skv.SKV_E_SHAPE),
    (dict(n_outlier=125), skv.SKV_E_SHAPE),                 # > n - n_loc
    (dict(top_k=121), skv.SKV_E_SHAPE),                     # > n - n_loc - o
    (dict(rank=0), skv.SKV_E_SHAPE),
    (dict(rank=257), skv.SKV_E_SHAPE),
    (dict(rank=100, dtype=skv.SKV_BF16), skv.SKV_E_SHAPE),  # bfloat16 rank not a multiple of 8
    (dict(chunk=65, seq_len=65 * 16, local_window=0), skv.SKV_E_SHAPE),
    (dict(n_outlier=0, top_k=0, local_window=0), skv.SKV_E_SHAPE),  # nothing to attend
    (dict(rope_base=0.0), skv.SKV_E_SHAPE),
    (dict(cache_chunks=7), skv.SKV_E_SHAPE),                # below top_k
    (dict(cache_chunks=-1), skv.SKV_E_SHAPE),
    (dict(cache_chunks=121), skv.SKV_E_SHAPE),              # > n - n_loc - o selectable chunks
    (dict(max_new=-1), skv.SKV_E_SHAPE),
])
def test_invalid_sizes_are_rejected_before_the_device(lib, kw, code):
    with pytest.raises(skv.ShadowKVError) as e:
        skv.shadowkv_layer_create(_cfg(**kw))
    assert e.value.code == code
    assert skv.shadowkv_last_error()


def test_null_arguments(lib):
    assert lib.shadowkv_layer_create(None, None) == skv.SKV_E_INVAL
    assert lib.shadowkv_decode_step(None, None, None, None) == skv.SKV_E_INVAL
    assert lib.shadowkv_tensor_bytes(None, 0) == 0


@pytest.mark.parametrize("args, code", [
    ((skv.SKV_BF16, 1, 8, 1024, 128, 160, None, 1, 1), skv.SKV_E_INVAL),   # null k_pre
    ((7, 1, 8, 1024, 128, 160, 1, 1, 1), skv.SKV_E_INVAL),                  # dtype
    ((skv.SKV_BF16, 0, 8, 1024, 128, 160, 1, 1, 1), skv.SKV_E_SHAPE),       # batch
    ((skv.SKV_BF16, 1, 8, 0, 128, 160, 1, 1, 1), skv.SKV_E_SHAPE),          # seq_len
    ((skv.SKV_BF16, 1, 8, 1024, 96, 160, 1, 1, 1), skv.SKV_E_SHAPE),        # head_dim
    ((skv.SKV_BF16, 1, 8, 1024, 128, 0, 1, 1, 1), skv.SKV_E_SHAPE),         # rank
    ((skv.SKV_BF16, 1, 8, 1024, 128, 257, 1, 1, 1), skv.SKV_E_SHAPE),       # rank
    ((skv.SKV_BF16, 1, 32, 1024, 128, 160, 1, 1, 1), skv.SKV_E_SHAPE),      # n = 4096 > 2048
])
def test_factorize_rejects_bad_arguments_before_the_device(lib, args, code):
    # the pointer arguments are never dereferenced on these paths
    assert lib.shadowkv_factorize(*args, None, None) == code
    assert skv.shadowkv_last_error()
