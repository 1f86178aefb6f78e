"""Host logic of bench.py (no GPU): visible lengths, algorithmic work, bounds,
and that the measurement path does not use the oracle."""
import ast
import os

import numpy as np

import bench
from dsa_workloads import CONFIGS, generate

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_visible_lengths():
    vis, seq = bench.visible_lengths(np.array([10, 7]), None)
    assert vis.tolist() == [10, 7] and seq.tolist() == [0, 1]
    vis, seq = bench.visible_lengths(np.array([10, 7, 3]), np.array([0, 3, 4, 6]))
    assert vis.tolist() == [8, 9, 10, 7, 2, 3]
    assert seq.tolist() == [0, 0, 0, 1, 2, 2]


def _work(name):
    return bench.algorithmic_work(generate(CONFIGS[name], with_mla=False, with_indexer=False))


def test_ragged_decode_work():
    w = _work("decode_b64_ragged")
    # 1,237,475 keys x (132 B cache + 4 B logit) + 64 rows x (8,192 B q + 256 B w)
    assert w["indexer"]["bytes"] == 1237475 * 136 + 64 * 8448
    assert w["indexer"]["bound"] == "hbm"
    # 64 rows x 2,048 selected rows x 1,152 B + 64 x (q 147,456 + out 131,072 + idx 8,192 + lse 512)
    assert w["sparse_mla"]["bytes"] == 64 * 2048 * 1152 + 64 * 287232
    assert w["sparse_mla"]["bound"] == "hbm"
    assert w["topk"]["bytes"] == 1237475 * 4 + 64 * 8192


def test_prefill_work_counts_shared_keys_once():
    w = _work("prefill_4k_on_16k")
    rows_vis = np.arange(16385, 20481)
    # the request's 20,480 keys are read once for its 4,096 rows
    assert w["indexer"]["bytes"] == 20480 * 132 + int(rows_vis.sum()) * 4 + 4096 * 8448
    assert w["indexer"]["flops"] == int(rows_vis.sum()) * 16384
    assert w["indexer"]["bound"] == "mfma" and w["indexer"]["peak_tflops"] == bench.FP8_PEAK_TFLOPS
    # attention: at most the 20,480 cached rows come from HBM; the per-row gather is cache traffic
    assert w["sparse_mla"]["bytes"] == 20480 * 1152 + 4096 * 287232
    assert w["sparse_mla"]["gather_bytes"] == 4096 * 2048 * 1152 + 4096 * 287232
    assert w["sparse_mla"]["bound"] == "mfma" and w["sparse_mla"]["peak_tflops"] == bench.BF16_PEAK_TFLOPS


def test_multi_token_decode_reads_keys_once_per_request():
    w = _work("mtp_b64x2_ragged")
    lens = generate(CONFIGS["mtp_b64x2_ragged"], with_mla=False, with_indexer=False).seq_lens_k.astype(np.int64)
    assert w["indexer"]["bytes"] == int(lens.sum()) * 132 + int((2 * lens - 1).sum()) * 4 + 128 * 8448


def test_measurement_path_does_not_use_the_oracle():
    """Only cpu_baseline (the timed oracle leg) may import the oracle."""
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    for fn in tree.body:
        names = set()
        for node in ast.walk(fn):
            if isinstance(node, ast.Import):
                names |= {a.name.split(".")[0] for a in node.names}
            elif isinstance(node, ast.ImportFrom) and node.module:
                names.add(node.module.split(".")[0])
        if "oracle" in names:
            assert isinstance(fn, ast.FunctionDef) and fn.name == "cpu_baseline", getattr(fn, "name", fn)
