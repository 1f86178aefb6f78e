"""Pins of the oracle's lightning-indexer score (no GPU)."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import gather_index_keys, indexer_logits, indexer_logits_row
from dsa_workloads import CONFIGS, generate, small_config
from tests.packing import pack_index_cache_f32, scatter_tokens


def _hand_example(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "indexer_hand_example.json")))
    q = np.array(ex["q"], dtype=np.float32)[None]           # [T=1, H, D]
    w = np.array(ex["w"], dtype=np.float32)[None]
    keys = np.array(ex["keys"], dtype=np.float32)
    sigma = np.array(ex["sigma"], dtype=np.float32)
    bt = np.array([[1, 0]], dtype=np.int32)
    kp = scatter_tokens(keys, bt[0], 2, 2)
    sp = scatter_tokens(sigma, bt[0], 2, 2)
    cache = pack_index_cache_f32(kp, sp)
    return ex, q, w, cache, bt


def test_hand_worked_example(golden_dir):
    ex, q, w, cache, bt = _hand_example(golden_dir)
    got = indexer_logits(q, w, cache, bt, np.array([4]), None, 2, "f32")[0]
    assert np.array_equal(got, np.array(ex["expected_logits"]))
    assert list(oracle.topk_row(got, 4, 2)[:2]) == ex["expected_top2"]
    assert list(oracle.topk_row(got, 4, 3)[:3]) == ex["expected_top3"]


@pytest.mark.parametrize("variant", ["relu_after_weight", "no_weight", "transposed", "sigma_outside_sum_squared"])
def test_hand_example_rejects_plausible_mistakes(golden_dir, variant, monkeypatch):
    """Plant a mistake in the oracle (on the CPU) and check the golden example catches it."""
    ex, q, w, cache, bt = _hand_example(golden_dir)

    def wrong(q_row, w_row, keys, sigma):
        dots = keys @ q_row.T
        if variant == "relu_after_weight":
            return np.maximum(0.0, sigma[:, None] * dots * w_row[None]).sum(1)
        if variant == "no_weight":
            return np.maximum(0.0, sigma[:, None] * dots).sum(1)
        if variant == "transposed":
            return np.maximum(0.0, sigma[:, None] * (keys @ q_row)) @ w_row
        return (np.maximum(0.0, sigma[:, None] * dots) @ w_row) * sigma

    monkeypatch.setattr(oracle.dsa, "indexer_logits_row", wrong)
    got = oracle.dsa.indexer_logits(q, w, cache, bt, np.array([4]), None, 2, "f32")[0]
    assert not np.allclose(got, np.array(ex["expected_logits"]))


def _brute(q, w, cache, bt, seq_lens, cu, P, kind):
    """Triple loop over rows, keys and heads, D-loop dot products."""
    rows = oracle.row_layout(seq_lens, cu)
    qf = oracle.decode_e4m3fn(q) if kind == "fp8" else q.astype(np.float64)
    out = {}
    for t, r in enumerate(rows):
        keys, sigma = gather_index_keys(cache, bt[r.seq], r.visible, P, q.shape[2], kind)
        vals = []
        for p in range(r.visible):
            acc = 0.0
            for h in range(q.shape[1]):
                dot = 0.0
                for d in range(q.shape[2]):
                    dot += qf[t, h, d] * keys[p, d]
                acc += float(w[t, h]) * max(0.0, sigma[p] * dot)
            vals.append(acc)
        out[t] = np.array(vals)
    return out


def test_vectorized_equals_brute_force_tiny_config():
    wl = generate(CONFIGS["tiny"], with_mla=False)
    got = indexer_logits(wl.q_idx, wl.w, wl.index_cache, wl.block_table, wl.seq_lens_k,
                         wl.cu_seqlens_q, wl.cfg.page_size, "f32")
    ref = _brute(wl.q_idx, wl.w, wl.index_cache, wl.block_table, wl.seq_lens_k,
                 wl.cu_seqlens_q, wl.cfg.page_size, "f32")
    np.testing.assert_allclose(got[0], ref[0], rtol=1e-12, atol=1e-12)
    assert len(got[0]) == 256


def test_vectorized_equals_brute_force_fp8_prefill_two_pages():
    cfg = small_config("bf_fp8", seed=21, lens=[70], q_lens=[3], page_size=64, idx_heads=8, idx_dim=16)
    wl = generate(cfg, with_mla=False)
    got = indexer_logits(wl.q_idx, wl.w, wl.index_cache, wl.block_table, wl.seq_lens_k,
                         wl.cu_seqlens_q, 64, "fp8")
    ref = _brute(wl.q_idx, wl.w, wl.index_cache, wl.block_table, wl.seq_lens_k,
                 wl.cu_seqlens_q, 64, "fp8")
    for t in range(3):
        assert len(got[t]) == 68 + t                     # bottom-right causal rows
        np.testing.assert_allclose(got[t], ref[t], rtol=1e-12, atol=1e-12)


def test_single_head_unit_scale_is_a_matrix_product():
    """H = 1, w = 1, sigma = 1 and non-negative q, k: relu is the identity and
    the score is the textbook product k @ q."""
    rng = np.random.default_rng(3)
    n, D, P = 37, 8, 16
    keys = np.abs(rng.standard_normal((n, D))).astype(np.float32)
    q = np.abs(rng.standard_normal((1, 1, D))).astype(np.float32)
    bt = np.array([[2, 0, 1]], dtype=np.int32)
    cache = pack_index_cache_f32(scatter_tokens(keys, bt[0], 3, P), scatter_tokens(np.ones(n, np.float32), bt[0], 3, P))
    got = indexer_logits(q, np.ones((1, 1), np.float32), cache, bt, np.array([n]), None, P, "f32")[0]
    want = np.matmul(keys.astype(np.float64), q[0, 0].astype(np.float64))
    np.testing.assert_allclose(got, want, rtol=1e-13)


def test_page_permutation_invariance():
    """Paging is a bijection: the same tokens behind a different block table give bitwise-equal logits."""
    rng = np.random.default_rng(4)
    n, H, D, P = 100, 4, 32, 16
    keys = rng.standard_normal((n, D)).astype(np.float32)
    sig = rng.uniform(0.5, 2.0, n).astype(np.float32)
    q = rng.standard_normal((1, H, D)).astype(np.float32)
    w = rng.standard_normal((1, H)).astype(np.float32)
    res = []
    for perm_seed in (0, 1):
        bt = np.random.default_rng(perm_seed).permutation(7).astype(np.int32)[None]
        cache = pack_index_cache_f32(scatter_tokens(keys, bt[0], 7, P), scatter_tokens(sig, bt[0], 7, P))
        res.append(indexer_logits(q, w, cache, bt, np.array([n]), None, P, "f32")[0])
    assert np.array_equal(res[0], res[1])


def test_zero_weight_heads_leave_logits_unchanged():
    """Padding q heads with zero weight (as done to reach an MMA-friendly head count) changes nothing."""
    rng = np.random.default_rng(5)
    n, D = 50, 16
    keys = rng.standard_normal((n, D))
    sig = rng.uniform(0.1, 1.0, n)
    q = rng.standard_normal((4, D))
    w = rng.standard_normal(4)
    q_pad = np.concatenate([q, rng.standard_normal((12, D))])
    w_pad = np.concatenate([w, np.zeros(12)])
    a = indexer_logits_row(q, w, keys, sig)
    b = indexer_logits_row(q_pad, w_pad, keys, sig)
    np.testing.assert_allclose(a, b, rtol=1e-14, atol=1e-14)


def test_positive_scale_commutes_with_relu():
    """relu(c x) = c relu(x) for c > 0: scaling sigma by c scales every logit by c."""
    rng = np.random.default_rng(6)
    keys = rng.standard_normal((40, 16))
    sig = rng.uniform(0.1, 1.0, 40)
    q = rng.standard_normal((4, 16))
    w = rng.standard_normal(4)
    a = indexer_logits_row(q, w, keys, sig * 3.0)
    b = 3.0 * indexer_logits_row(q, w, keys, sig)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


def test_canaries_are_never_read():
    """Rows only see positions below their visible length; the NaN canary slots
    after the last token and the poison page never reach a logit."""
    cfg = small_config("canary", seed=7, lens=[100, 33], page_size=16, idx_kind="f32")
    wl = generate(cfg, with_mla=False)
    got = indexer_logits(wl.q_idx, wl.w, wl.index_cache, wl.block_table, wl.seq_lens_k, None, 16, "f32")
    assert len(got[0]) == 100 and len(got[1]) == 33
    assert all(np.isfinite(v).all() for v in got.values())


@pytest.mark.parametrize("bad_page", [-1, 2, 1 << 20])
def test_absent_page_scores_minus_inf(golden_dir, bad_page):
    """A block-table entry outside [0, num_pages) names no page: its positions
    score -inf and the others keep the hand-worked values. Logical page 1
    (positions 2, 3) is made absent; the pool has 2 pages."""
    ex, q, w, cache, bt = _hand_example(golden_dir)
    bt_bad = bt.copy()
    bt_bad[0, 1] = bad_page
    got = indexer_logits(q, w, cache, bt_bad, np.array([4]), None, 2, "f32")[0]
    want = np.array(ex["expected_logits"][:2] + [-np.inf, -np.inf])
    assert np.array_equal(got, want)
    assert list(oracle.topk_row(got, 4, 3)[:3]) == [0, 1, 2]   # -inf ties go to the lower position

