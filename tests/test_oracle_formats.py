"""Pins of the oracle's exact input decoding (no GPU)."""
import json
import os

import numpy as np
import torch

from oracle import decode_bf16, decode_e4m3fn, e4m3fn_table


def test_e4m3fn_code_points_from_the_format_definition(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "e4m3fn_codes.json")))
    table = e4m3fn_table()
    for entry in spec["codes"]:
        code = int(entry["code"], 16)
        want = float(entry["value"])
        got = table[code]
        if np.isnan(want):
            assert np.isnan(got), entry
        else:
            assert got == want, entry
            assert np.signbit(got) == np.signbit(want), entry


def test_e4m3fn_table_matches_torch_exhaustively():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    got = decode_e4m3fn(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))
    assert nan.sum() == 2 and np.nanmax(got) == 448.0


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2 ** 16, size=20000, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = decode_bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
