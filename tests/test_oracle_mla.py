"""Pins of the oracle's sparse MLA attention and LSE merge (no GPU)."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import dense_mla, lse_merge, sparse_mla, sparse_mla_row
from dsa_workloads import generate, small_config
from tests.packing import scatter_tokens


def test_hand_worked_example(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "mla_hand_example.json")))
    rows = np.array(ex["cache_rows"], dtype=np.float32)
    bt = np.array([[1, 0]], dtype=np.int32)
    latent = scatter_tokens(rows, bt[0], 2, 2)            # page size 2, logical page 0 in physical 1
    q = np.array(ex["q"], dtype=np.float32)[None]
    idx = np.array([ex["topk"]])
    res = sparse_mla(q, latent, idx, bt, np.array([3]), None, 2, 2, 1.0, "f32")[0]
    # the cache holds float32, so ln 3 is stored to ~6e-8 relative
    np.testing.assert_allclose(res[0], np.array(ex["expected_out"]), rtol=1e-7, atol=1e-7)
    np.testing.assert_allclose(res[1], np.array(ex["expected_lse"]), rtol=1e-7)


@pytest.mark.parametrize("bad_page", [-1, 2, 99])
def test_hand_example_skips_absent_pages(golden_dir, bad_page):
    """Entries whose page is outside the pool are skipped like -1: with the
    hand example's row 0 on an absent page, only row 2 remains, which is the
    one-index closed form out = C[:Dl], lse = z."""
    ex = json.load(open(os.path.join(golden_dir, "mla_hand_example.json")))
    rows = np.array(ex["cache_rows"], dtype=np.float32)
    bt = np.array([[1, 0]], dtype=np.int32)
    latent = scatter_tokens(rows, bt[0], 2, 2)
    q = np.array(ex["q"], dtype=np.float32)[None]
    bt_bad = np.array([[bad_page, 0]], dtype=np.int32)     # logical page 0 (rows 0, 1) absent
    idx = np.array([[2, -1, 0, 1, 0]])
    out, lse = sparse_mla(q, latent, idx, bt_bad, np.array([3]), None, 2, 2, 1.0, "f32")[0]
    np.testing.assert_allclose(out, [[0.0, 1.0]], rtol=0, atol=0)
    np.testing.assert_allclose(lse, [np.float32(1.0986122886681098)], rtol=1e-7)


def test_hand_example_duplicates_and_order():
    """Duplicate entries count twice (two copies of row 2 against one of row
    0: weights 6/7 and 1/7); the order of the entries does not matter."""
    rows = np.array([[1.0, 0.0, 0.0], [5.0, 5.0, 5.0], [0.0, 1.0, np.log(3.0)]], dtype=np.float64)
    bt = np.array([[1, 0]], dtype=np.int32)
    latent = scatter_tokens(rows, bt[0], 2, 2)
    q = np.array([[[0.0, 0.0, 1.0]]])
    for order in ([2, 0, 2], [0, 2, 2], [2, 2, 0, -1]):
        out, lse = sparse_mla(q, latent, np.array([order]), bt, np.array([3]), None, 2, 2, 1.0, "f64")[0]
        np.testing.assert_allclose(out, [[1.0 / 7.0, 6.0 / 7.0]], rtol=1e-15)
        np.testing.assert_allclose(lse, [np.log(7.0)], rtol=1e-15)


def test_lse_merge_hand_example(golden_dir):
    ex = json.load(open(os.path.join(golden_dir, "lse_merge_hand_example.json")))
    o, l = lse_merge(np.array(ex["o1"]), np.array(ex["lse1"]), np.array(ex["o2"]), np.array(ex["lse2"]))
    np.testing.assert_allclose(o, ex["expected_o"], rtol=1e-15)
    np.testing.assert_allclose(l, ex["expected_lse"], rtol=1e-15)


def test_softmax_weights_sum_to_one():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((8, 80))
    c = rng.standard_normal((50, 80))
    _, _, probs = sparse_mla_row(q, c, 64, 0.3, return_probs=True)
    np.testing.assert_allclose(probs.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    assert (probs >= 0).all()


def test_single_index_closed_form():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((4, 12))
    c = rng.standard_normal((1, 12))
    out, lse = sparse_mla_row(q, c, 8, 0.7)
    np.testing.assert_allclose(out, np.repeat(c[:, :8], 4, axis=0), rtol=1e-15)
    np.testing.assert_allclose(lse, 0.7 * (q @ c[0]), rtol=1e-13)


def test_zero_query_closed_form():
    rng = np.random.default_rng(3)
    c = rng.standard_normal((9, 12))
    out, lse = sparse_mla_row(np.zeros((2, 12)), c, 8, 1.3)
    np.testing.assert_allclose(out, np.repeat(c[:, :8].mean(0, keepdims=True), 2, 0), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(9.0), rtol=1e-14)


def test_empty_selection():
    out, lse = sparse_mla_row(np.ones((3, 6)), np.zeros((0, 6)), 4, 1.0)
    assert (out == 0).all() and np.isneginf(lse).all()


@pytest.mark.parametrize("kind", ["f32", "bf16"])
def test_sparse_equals_dense_when_k_covers_the_context(kind):
    """With k >= visible every visible token is selected, so the sparse step
    must equal dense attention over the whole context."""
    cfg = small_config("dense_eq", seed=8, lens=[45], page_size=16, topk=64, idx_kind="f32",
                       mla_kind=kind, mla_heads=4, d_latent=16, d_rope=8)
    wl = generate(cfg, with_indexer=False)
    idx = oracle.topk_row(np.zeros(45), 45, 64)[None]    # short row: 0..44 then -1
    res = sparse_mla(wl.q_mla, wl.latent, idx, wl.block_table, wl.seq_lens_k, None, 16, 16,
                     cfg.softmax_scale, kind)[0]
    rows = oracle.gather_latent_rows(wl.latent, wl.block_table[0], range(45), 16, kind)
    q_row = oracle.decode_bf16(wl.q_mla[0]) if kind == "bf16" else wl.q_mla[0].astype(np.float64)
    d_out, d_lse = dense_mla(q_row, rows, 16, cfg.softmax_scale)
    np.testing.assert_allclose(res[0], d_out, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(res[1], d_lse, rtol=1e-12)


def test_split_and_merge_equals_one_pass():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((6, 20))
    c = rng.standard_normal((33, 20))
    full = sparse_mla_row(q, c, 16, 0.5)
    a = sparse_mla_row(q, c[:10], 16, 0.5)
    b = sparse_mla_row(q, c[10:], 16, 0.5)
    o, l = lse_merge(a[0], a[1], b[0], b[1])
    np.testing.assert_allclose(o, full[0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l, full[1], rtol=1e-13)
    # merging with an empty part is the identity
    e = sparse_mla_row(q, c[:0], 16, 0.5)
    o2, l2 = lse_merge(full[0], full[1], e[0], e[1])
    np.testing.assert_allclose(o2, full[0], rtol=1e-15)
    np.testing.assert_allclose(l2, full[1], rtol=1e-15)


def test_absorbed_form_equals_per_head_projection():
    """q_nope . (W_UK c) = (q_nope W_UK) . c and the per-head value up-projection
    commutes with the weighted sum, so attention over the latent with absorbed
    queries equals multi-head attention with projected keys and values."""
    rng = np.random.default_rng(5)
    H, dn, dl, dr, dv, n = 3, 6, 10, 4, 5, 17
    W_UK = rng.standard_normal((H, dn, dl))
    W_UV = rng.standard_normal((H, dl, dv))
    q_nope = rng.standard_normal((H, dn))
    q_pe = rng.standard_normal((H, dr))
    lat = rng.standard_normal((n, dl))
    k_pe = rng.standard_normal((n, dr))
    scale = 0.4
    # absorbed
    ql = np.einsum("hd,hdl->hl", q_nope, W_UK)
    out_l, _ = sparse_mla_row(np.concatenate([ql, q_pe], 1), np.concatenate([lat, k_pe], 1), dl, scale)
    absorbed = np.einsum("hl,hlv->hv", out_l, W_UV)
    # explicit multi-head attention
    mha = np.empty((H, dv))
    for h in range(H):
        keys = lat @ W_UK[h].T                      # [n, dn]
        vals = lat @ W_UV[h]                        # [n, dv]
        z = scale * (keys @ q_nope[h] + k_pe @ q_pe[h])
        p = np.exp(z - z.max())
        p /= p.sum()
        mha[h] = p @ vals
    np.testing.assert_allclose(absorbed, mha, rtol=1e-11, atol=1e-12)


def test_minus_one_and_out_of_range_entries_are_skipped():
    rng = np.random.default_rng(6)
    rows = rng.standard_normal((5, 6)).astype(np.float32)
    bt = np.array([[0]], dtype=np.int32)
    latent = scatter_tokens(rows, bt[0], 1, 8)
    q = rng.standard_normal((1, 2, 6)).astype(np.float32)
    a = sparse_mla(q, latent, np.array([[3, -1, 1, 9, -1]]), bt, np.array([5]), None, 8, 4, 1.0, "f32")[0]
    b = sparse_mla(q, latent, np.array([[3, 1]]), bt, np.array([5]), None, 8, 4, 1.0, "f32")[0]
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


@pytest.mark.parametrize("variant", ["rope_in_value", "no_scale", "value_from_tail"])
def test_hand_example_rejects_plausible_mistakes(golden_dir, variant, monkeypatch):
    ex = json.load(open(os.path.join(golden_dir, "mla_hand_example.json")))
    real = oracle.dsa.sparse_mla_row

    def wrong(q_row, rows_c, d_latent, scale, return_probs=False):
        if variant == "rope_in_value":
            out, lse = real(q_row, rows_c, d_latent + 1, scale)
            return out[:, 1:], lse
        if variant == "no_scale":
            return real(q_row, rows_c, d_latent, 2.0)
        z = scale * (q_row @ rows_c.T)
        p = np.exp(z - z.max(1, keepdims=True))
        p /= p.sum(1, keepdims=True)
        return p @ rows_c[:, -d_latent:], np.log(np.exp(z).sum(1))

    monkeypatch.setattr(oracle.dsa, "sparse_mla_row", wrong)
    rows = np.array(ex["cache_rows"], dtype=np.float32)
    bt = np.array([[1, 0]], dtype=np.int32)
    latent = scatter_tokens(rows, bt[0], 2, 2)
    res = oracle.dsa.sparse_mla(np.array(ex["q"], np.float32)[None], latent, np.array([ex["topk"]]), bt,
                                np.array([3]), None, 2, 2, 1.0, "f32")[0]
    ok = np.allclose(res[0], ex["expected_out"]) and np.allclose(res[1], ex["expected_lse"])
    assert not ok


def _fp8_case(seed, n_pages=6, P=16, Hm=8, Dl=64, Dr=16, k=40):
    rng = np.random.default_rng(seed)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    latent = rng.choice(finite, size=(n_pages, P, Dl + Dr))
    q = rng.choice(finite, size=(2, Hm, Dl + Dr))
    bt = rng.permutation(n_pages).astype(np.int32).reshape(2, n_pages // 2)
    lens = np.array([P * (n_pages // 2) - 5, P * (n_pages // 2)])
    idx = np.stack([rng.choice(int(n), size=k, replace=False) for n in lens]).astype(np.int32)
    idx[0, :3] = -1
    return latent, q, idx, bt, lens, P, Dl


def test_fp8_cache_reduces_to_the_float_path():
    """With power-of-two scales the dequantized values are exact in float32,
    so the fp8 path must give exactly the float path's results on them."""
    latent, q, idx, bt, lens, P, Dl = _fp8_case(21)
    qs, ks = 2.0 ** -5, 2.0 ** -3
    lat_f = (oracle.decode_e4m3fn(latent) * ks).astype(np.float32)
    q_f = (oracle.decode_e4m3fn(q) * qs).astype(np.float32)
    a = sparse_mla(q, latent, idx, bt, lens, None, P, Dl, 0.11, "fp8", q_scale=qs, kv_scale=ks)
    b = sparse_mla(q_f, lat_f, idx, bt, lens, None, P, Dl, 0.11, "f32")
    for t in a:
        assert np.array_equal(a[t][0], b[t][0]) and np.array_equal(a[t][1], b[t][1])


def test_fp8_scale_invariances():
    """Only scale * q_scale * kv_scale reaches the scores and only kv_scale the
    values: moving a factor between the scales leaves lse alone and scales
    the output by what moved into kv_scale."""
    latent, q, idx, bt, lens, P, Dl = _fp8_case(22)
    base = sparse_mla(q, latent, idx, bt, lens, None, P, Dl, 0.05, "fp8", q_scale=0.02, kv_scale=0.3)
    kvx = sparse_mla(q, latent, idx, bt, lens, None, P, Dl, 0.05 / 3.0, "fp8", q_scale=0.02, kv_scale=0.9)
    qx = sparse_mla(q, latent, idx, bt, lens, None, P, Dl, 0.05 / 7.0, "fp8", q_scale=0.14, kv_scale=0.3)
    for t in base:
        np.testing.assert_allclose(kvx[t][0], 3.0 * base[t][0], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(kvx[t][1], base[t][1], rtol=1e-12)
        np.testing.assert_allclose(qx[t][0], base[t][0], rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(qx[t][1], base[t][1], rtol=1e-12)
