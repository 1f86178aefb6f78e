"""Pins of the oracle's fp8 input quantization (oracle/quant.py), no GPU.

The encoder is pinned to the OCP E4M3 definition (every finite code round
trips, every tie between neighbours goes to the even code, near-ties go to the
nearer one) and to torch's CPU float8_e4m3fn conversion; the block
quantization to properties any correct implementation has (the largest
element lands on 448, power-of-two scaling only moves the scale, half a grid
step of error); the paged store to the indexer's own key reader.
"""
import numpy as np
import pytest
import torch

from oracle import decode_e4m3fn, gather_index_keys, indexer_logits_row
from oracle.quant import encode_e4m3fn, quant_index_q, quant_rows, store_index_k


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def _bf16_bits(x32):
    return torch.from_numpy(_f32(x32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    vals = decode_e4m3fn(codes).astype(np.float32)
    assert np.array_equal(encode_e4m3fn(vals), codes.astype(np.uint8))


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_ties_to_even_and_near_ties_to_nearest(sign):
    for c in range(0x7E):
        lo, hi = decode_e4m3fn(c), decode_e4m3fn(c + 1)
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2                    # exact in fp32
        even = c if c % 2 == 0 else c + 1
        s = 0x80 if sign < 0 else 0
        assert encode_e4m3fn(sign * mid)[()] == even | s, hex(c)
        up = np.nextafter(mid, np.float32(np.inf))
        dn = np.nextafter(mid, np.float32(0))
        assert encode_e4m3fn(sign * up)[()] == (c + 1) | s, hex(c)
        assert encode_e4m3fn(sign * dn)[()] == c | s, hex(c)


def test_range_end_reading():
    assert encode_e4m3fn(_f32(448.0))[()] == 0x7E
    assert encode_e4m3fn(_f32(464.0))[()] == 0x7E            # tie with the NaN step: even code
    assert encode_e4m3fn(np.nextafter(_f32(464.0), _f32(np.inf)))[()] == 0x7F
    for v in (480.0, 1e6, np.inf):
        assert encode_e4m3fn(_f32(v))[()] == 0x7F
        assert encode_e4m3fn(_f32(-v))[()] == 0xFF
    assert encode_e4m3fn(_f32(np.nan))[()] & 0x7F == 0x7F
    assert encode_e4m3fn(_f32(0.0))[()] == 0x00
    assert encode_e4m3fn(_f32(-0.0))[()] == 0x80


def test_matches_torch_conversion():
    rng = np.random.default_rng(5)
    n = 1_000_000
    mag = np.exp2(rng.uniform(-13.0, np.log2(470.0), size=n))
    x = _f32(mag * rng.choice([-1.0, 1.0], size=n))
    mids = (decode_e4m3fn(np.arange(0x7E)) + decode_e4m3fn(np.arange(1, 0x7F))) / 2
    x = np.concatenate([x, _f32(mids), _f32(-mids), _f32([0.0, -0.0, 448.0, 464.0, 470.0])])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = encode_e4m3fn(x)
    nan_ref = (ref & 0x7F) == 0x7F
    assert np.array_equal(nan_ref, (got & 0x7F) == 0x7F)
    assert np.array_equal(ref[~nan_ref], got[~nan_ref])


def test_block_quant_properties():
    rng = np.random.default_rng(6)
    x = _f32(rng.standard_normal((500, 128)) * np.exp2(rng.uniform(-8, 8, size=(500, 1))))
    codes, s = quant_rows(x)
    # the element of largest magnitude lands on +-448
    top = np.abs(x).argmax(axis=1)
    assert np.all((codes[np.arange(500), top] & 0x7F) == 0x7E)
    # error of at most half a grid step: 2**-4 relative for normals, 2**-10 absolute below 2**-6
    y = x / s[:, None].astype(np.float64)
    err = np.abs(decode_e4m3fn(codes) - y)
    bound = np.maximum(np.abs(y) * 2.0 ** -4, 2.0 ** -10)
    assert np.all(err <= bound)
    # power-of-two scaling only moves the scale
    for k in (-20, -3, 5, 40):
        c2, s2 = quant_rows(x * np.float32(2.0 ** k))
        assert np.array_equal(c2, codes)
        assert np.array_equal(s2, _f32(s * np.float32(2.0 ** k)))


def test_zero_block_uses_the_floor():
    codes, s = quant_rows(np.zeros((2, 128), np.float32) * _f32([[1.0], [-1.0]]))
    assert s[0] == np.float32(np.float32(1e-30) / np.float32(448.0))
    assert np.all(codes[0] == 0x00) and np.all(codes[1] == 0x80)


def test_quant_q_folds_scale_and_keeps_scores():
    rng = np.random.default_rng(7)
    T, H, D = 3, 64, 128
    q = rng.standard_normal((T, H, D))
    q_bits = _bf16_bits(q)
    w = _f32(rng.standard_normal((T, H)) / 8.0)
    codes, w_eff, s = quant_index_q(q_bits, w)
    assert codes.shape == (T, H, D) and w_eff.dtype == np.float32
    assert np.array_equal(w_eff, _f32(w * s))
    # scores from the quantized (q8, w_eff) stay within the quantization error
    # of the scores from the bf16 query and the plain gates
    keys = rng.standard_normal((40, D))
    sig = np.ones(40)
    qb = torch.from_numpy(q_bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    for t in range(T):
        a = indexer_logits_row(decode_e4m3fn(codes[t]), w_eff[t].astype(np.float64), keys, sig)
        b = indexer_logits_row(qb[t], w[t].astype(np.float64), keys, sig)
        scale = np.abs(w[t]).sum() * np.abs(qb[t]).max() * np.abs(keys).sum(axis=1)
        assert np.all(np.abs(a - b) <= 2.0 ** -4 * scale)


def test_store_index_k_reads_back_through_the_indexer_reader():
    rng = np.random.default_rng(8)
    P, D, pages = 16, 128, 6
    cache = rng.integers(0, 256, size=(pages, P * D + 4 * P), dtype=np.uint8)
    n = 20
    slots = rng.choice(pages * P, size=n, replace=False).astype(np.int64)
    slots[3] = -1
    slots[11] = pages * P + 5                                 # past the pool: skipped
    key = rng.standard_normal((n, D)) * 3.0
    key_bits = _bf16_bits(key)
    out = store_index_k(cache, key_bits, slots, P)
    codes, s = quant_rows(torch.from_numpy(key_bits.view(np.int16)).view(torch.bfloat16).float().numpy())
    keys, sigma = gather_index_keys(out, np.arange(pages), pages * P, P, D, "fp8")
    written = set()
    for i in range(n):
        if slots[i] < 0 or slots[i] >= pages * P:
            continue
        written.add(int(slots[i]))
        assert np.array_equal(keys[slots[i]], decode_e4m3fn(codes[i]))
        assert sigma[slots[i]] == np.float64(s[i])
        deq = keys[slots[i]] * sigma[slots[i]]
        kb = torch.from_numpy(key_bits[i].view(np.int16)).view(torch.bfloat16).double().numpy()
        assert np.all(np.abs(deq - kb) <= np.maximum(np.abs(kb) * 2.0 ** -4, 2.0 ** -10 * s[i]))
    # every other byte is untouched
    mask = np.zeros_like(cache, dtype=bool)
    for slot in written:
        page, pos = divmod(slot, P)
        mask[page, pos * D:(pos + 1) * D] = True
        mask[page, P * D + 4 * pos:P * D + 4 * pos + 4] = True
    assert np.array_equal(out[~mask], cache[~mask])
