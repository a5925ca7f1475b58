"""The host-V chunk forms the header documents under shadowkv_prefill_meta,
checked on the CPU: chunks laid out by hand from that description decode
(parity_helpers.decode_host_v_chunks, which the GPU tests use to read the
pinned host buffer) to their values bit for bit.  The layout is written here
from the description, not from the library's encoder."""
import numpy as np
import pytest
import torch

from parity_helpers import decode_host_v_chunks, host_v_form


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _class_form(vals: np.ndarray, N: int):
    """One chunk in the class form: (slot bytes, code word), or None past 64 escapes."""
    e = ((vals.astype(np.int64) >> 7) & 0xff)
    top = max(int(e.max()) - 1, 0)
    d = top - e
    cls = np.where((d >= 0) & (d <= 2), d, 3)
    codes, esc = [], []
    for v in np.flatnonzero(cls == 3):
        dv = int(d[v])
        xc = 0 if e[v] == top + 1 else (dv - 2 if 3 <= dv <= 8 else 7)
        codes.append(xc)
        if xc == 7:
            esc.append((int(v) << 8) | int(e[v]))
    if len(esc) > 64:
        return None
    S = (3 * len(codes) + 31) // 32 * 4
    bits = np.zeros(8 * S, dtype=np.uint8)
    for m, xc in enumerate(codes):
        bits[3 * m:3 * m + 3] = [(xc >> j) & 1 for j in range(3)]
    slot = np.zeros(2 * N, dtype=np.uint8)
    slot[:N] = ((vals >> 8) & 0x80) | (vals & 0x7f)
    for j in range(4):
        slot[N:N + N // 4] |= (cls[j::4] << (2 * j)).astype(np.uint8)
    slot[N + N // 4:N + N // 4 + S] = np.packbits(bits, bitorder="little")
    ent = np.array(esc, dtype=np.uint32).view(np.uint8)
    slot[N + N // 4 + S:N + N // 4 + S + ent.size] = ent
    return slot, 0xC0000000 | ((S // 4) << 20) | (len(esc) << 8) | top


def _twelve_bit_form(vals: np.ndarray, N: int):
    e = ((vals.astype(np.int64) >> 7) & 0xff)
    base = max(int(e.max()) - 14, 0)
    esc = [(int(v) << 8) | int(e[v]) for v in np.flatnonzero(e < base)]
    if len(esc) > 64:
        return None
    off = np.where(e < base, 15, e - base).astype(np.uint8)
    slot = np.zeros(2 * N, dtype=np.uint8)
    slot[:N] = ((vals >> 8) & 0x80) | (vals & 0x7f)
    slot[N:N + N // 2] = off[0::2] | (off[1::2] << 4)
    ent = np.array(esc, dtype=np.uint32).view(np.uint8)
    slot[3 * N // 2:3 * N // 2 + ent.size] = ent
    return slot, 0x80000000 | (len(esc) << 16) | base


@pytest.mark.parametrize("N", [512, 1024, 2048])
def test_documented_chunk_forms_decode_bit_for_bit(N):
    rng = np.random.default_rng(N)
    cases = [rng.standard_normal(N), np.zeros(N), rng.standard_normal(N) * 2.0 ** 40,
             rng.standard_normal(N) * 2.0 ** -40]
    x = rng.standard_normal(N)
    x[rng.choice(N, 30, replace=False)] = 2.0 ** -50  # escapes in both forms
    cases.append(x)
    x = rng.standard_normal(N)
    x[:5] = 0.0
    x[5] = 7.5  # a value above top + 1 of the rest: an escape in the class form
    cases.append(x)
    slots, words, want = [], [], []
    for v in cases:
        bits = _bf16_bits(v).astype(np.uint32)
        for make in (_class_form, _twelve_bit_form):
            r = make(bits, N)
            assert r is not None
            slots.append(r[0]); words.append(r[1]); want.append(bits.astype(np.uint16))
    raw = _bf16_bits(np.exp2(rng.uniform(-100, 100, N)))
    slots.append(raw.view(np.uint8).copy()); words.append(0); want.append(raw)
    got = decode_host_v_chunks(np.stack(slots), np.array(words, dtype=np.int64), N)
    np.testing.assert_array_equal(got, np.stack(want))
    assert [host_v_form(w)[0] for w in words[:2]] == ["class", "12-bit"] and host_v_form(0) == ("raw", 0)


def test_class_form_size_on_normal_values():
    """About 10.6 bits a value on normally distributed values: the class form
    is at least 9 % smaller than the 12-bit form on them."""
    rng = np.random.default_rng(5)
    N = 1024
    tot_c = tot_12 = 0
    for _ in range(50):
        bits = _bf16_bits(rng.standard_normal(N)).astype(np.uint32)
        sc, wc = _class_form(bits, N)
        s12, w12 = _twelve_bit_form(bits, N)
        tot_c += N + N // 4 + 4 * ((wc >> 20) & 0xff) + 4 * ((wc >> 8) & 0xff)
        tot_12 += 3 * N // 2 + 4 * ((w12 >> 16) & 0xff)
    assert tot_c <= 0.91 * tot_12
