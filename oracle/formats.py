"""Exact decoding of the storage formats the DSA step reads.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The SGLang indexer page stores the index keys as fp8 (it views the cache as
`torch.float8_e4m3fn` in `Indexer.forward_indexer`) and notes that the fp8
flavour differs by platform; the OCP 8-bit floating-point specification
defines E4M3 ("fn": finite, no infinities) as:

* 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
* exponent field 0: subnormal, value = mantissa * 2**-9;
* exponent field 1..15: value = (1 + mantissa/8) * 2**(exponent - 7);
* the two codes with all exponent and mantissa bits set (0x7F, 0xFF) are NaN;
  every other code is finite, the largest magnitude being 448 (0x7E).

bfloat16 is the upper half of an IEEE binary32 word.
"""

import numpy as np


def e4m3fn_table():
    """Float64 value of each of the 256 OCP E4M3 codes, from the definition."""
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if (code >> 7) & 1 else 1.0
        exponent = (code >> 3) & 0xF
        mantissa = code & 0x7
        if exponent == 0xF and mantissa == 0x7:
            table[code] = np.nan
        elif exponent == 0:
            table[code] = sign * mantissa * 2.0 ** -9
        else:
            table[code] = sign * (1.0 + mantissa / 8.0) * 2.0 ** (exponent - 7)
    return table


_E4M3FN = e4m3fn_table()


def decode_e4m3fn(codes):
    """Decode an array of E4M3 bytes (any integer dtype) to float64."""
    codes = np.asarray(codes)
    return _E4M3FN[codes.astype(np.uint8)]


def decode_bf16(bits):
    """Decode an array of bfloat16 bit patterns (uint16/int16) to float64."""
    bits = np.asarray(bits).astype(np.uint16).astype(np.uint32)
    with np.errstate(invalid="ignore"):   # signalling-NaN patterns stay NaN
        return (bits << np.uint32(16)).view(np.float32).astype(np.float64)
