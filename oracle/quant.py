"""fp8 quantization of the indexer's inputs: the step just before the scores.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What the pages do (SGLang indexer page, "dsa_indexer.py"):

* `Indexer.forward_cuda` (the decode branch with two streams) turns the bf16
  index query into `(q_fp8, q_scale)` with `act_quant(query, block_size,
  scale_fmt)`, and `_get_logits_head_gate` multiplies the head gates by
  `q_scale` (after the `n_heads ** -0.5` factor; the softmax scale joins the
  same product);
* `Indexer._store_index_k_cache` quantizes the step's new index keys the same
  way (its fallback path: `act_quant(key, ...)`) and writes `(k_fp8, k_scale)`
  into the paged index-K buffer at `out_cache_loc` (`set_index_k_scale_buffer`).

`act_quant` itself is not on the pages. Reading taken (the plainest one the
rest supports: the block is the 128-wide head dimension, so one fp32 scale per
head row or per key, as the 132-byte token of the cache holds):

    s      = max(max_d |x_d|, 1e-30) / 448        fp32 (448 = largest E4M3 value)
    code_d = E4M3FN(x_d / s)                      the fp32 quotient, rounded to
                                                  the nearest code, ties to even

E4M3FN rounding (OCP 8-bit floating point, E4M3): the finite codes 0x00..0x7E
of one sign form an increasing grid (subnormals m * 2**-9, then normals);
rounding picks the nearest grid value, ties to the code with an even mantissa
(an even code). The format has no infinity: a magnitude that rounds past 448
becomes NaN (0x7F, i.e. the grid continued by one step to 480 and read as NaN;
anything at or above 480 is NaN as well). This is the non-saturating
conversion; with the scales above no finite input reaches it. NaN in gives
NaN out, the sign is kept (so -0.0 is 0x80).

Parity status: pinned (tests/test_oracle_quant.py): round trip of every
finite code, ties and near-ties between every pair of neighbours, agreement
with torch's CPU float8_e4m3fn conversion on a million values, the amax
element landing on 448, power-of-two scale invariance, the error bound of
half a grid step, and the paged store read back through
`dsa.gather_index_keys`.
"""

import numpy as np

from .formats import decode_bf16, e4m3fn_table

F8_MAX = 448.0
SCALE_FLOOR = 1e-30

# non-negative grid: codes 0x00..0x7E, plus 0x7F standing at 480 (read as NaN)
_GRID = np.concatenate([e4m3fn_table()[:0x7F], [480.0]])


def encode_e4m3fn(x):
    """Round float32 values to OCP E4M3FN codes (uint8), nearest, ties to even."""
    v = np.asarray(x, dtype=np.float32).astype(np.float64)   # exact
    a = np.abs(v)
    hi = np.clip(np.searchsorted(_GRID, a, side="left"), 0, 0x7F)   # first grid value >= a
    lo = np.clip(hi - 1, 0, 0x7F)
    d_lo = a - _GRID[lo]
    d_hi = _GRID[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= 480.0, 0x7F, code)
    code = np.where(np.isnan(v), 0x7F, code)
    code = code | (np.signbit(v).astype(np.int64) << 7)
    return code.astype(np.uint8)


def quant_rows(x32):
    """Quantize the last axis of float32 `x32` as one block: (codes, scales)."""
    x32 = np.asarray(x32, dtype=np.float32)
    amax = np.abs(x32).max(axis=-1)
    s = (np.maximum(amax, np.float32(SCALE_FLOOR)) / np.float32(F8_MAX)).astype(np.float32)
    q = (x32 / s[..., None]).astype(np.float32)              # IEEE float32 division
    return encode_e4m3fn(q), s


def quant_index_q(q_bf16_bits, w):
    """Index queries [T, H, D] (bf16 bits) and gates [T, H] -> (q8 codes, w_eff, s).

    w_eff = w * s in float32: the gate then carries the query's scale, so the
    scores use the fp8 codes directly (the head-gate fold of the SGLang page).
    """
    x = decode_bf16(q_bf16_bits).astype(np.float32)           # bf16 -> fp32 is exact
    codes, s = quant_rows(x)
    w_eff = (np.asarray(w, dtype=np.float32) * s).astype(np.float32)
    return codes, w_eff, s


def store_index_k(index_cache, key_bf16_bits, slot_mapping, page_size):
    """Quantize new keys [N, D] (bf16 bits) per token and write them into a
    copy of the paged cache [num_pages, P * D + 4 * P] (uint8) at their slots.

    Slot i goes to page slot // P, position slot % P: its D codes at byte
    position * D, its fp32 scale at byte P * D + 4 * position (the layout the
    indexer reads). Negative slots and slots past the pool are skipped.
    """
    cache = np.array(index_cache, dtype=np.uint8, copy=True)
    keys = decode_bf16(key_bf16_bits).astype(np.float32)
    n, d = keys.shape
    codes, s = quant_rows(keys)
    P = int(page_size)
    num_pages = cache.shape[0]
    for i in range(n):
        slot = int(slot_mapping[i])
        if slot < 0 or slot >= num_pages * P:
            continue
        page, pos = divmod(slot, P)
        cache[page, pos * d:(pos + 1) * d] = codes[i]
        cache[page, P * d + 4 * pos:P * d + 4 * pos + 4] = np.frombuffer(
            np.float32(s[i]).tobytes(), dtype=np.uint8)
    return cache
