"""Comparison rules between the HIP path and the oracle.

Tolerances (stated once, used by every parity test):

* indexer logits: |L_gpu - L_orc| <= 1e-3 * max(|L_orc|, A), where
  A = sum_h |w_h| relu(sigma (q_h . k)) is the magnitude of the terms being
  summed (the relative 1e-3 of the logits, measured against the sum's own
  scale because signed head weights can cancel toward 0). Infinite oracle
  values (-inf on absent pages, +inf at forced positions) must be matched
  exactly.
* top-k on identical logits: bit-exact (same positions, same order).
* top-k end to end (GPU logits vs oracle logits): the GPU row holds exactly
  min(k, visible) distinct positions in [0, visible) in ascending order, then
  -1; every position in the symmetric difference with the oracle's set has an
  oracle logit within 1e-3 * max(|tau|, 1) of tau, the oracle's k-th largest.
* attention, on the GPU's own indices: |o_gpu - o_orc| <= 2e-2 + 1e-2 |o_orc|
  (bf16 output), lse within 1e-3 + 1e-3 |lse|; fp32 output paths use
  1e-4 + 1e-4 |o| and 1e-5 + 1e-5 |lse|.
"""
import numpy as np

import oracle

LOGIT_RTOL = 1e-3
TIE_RTOL = 1e-3


def logits_tolerance_scale(wl, rows):
    """A per (row, position) for the listed rows (oracle with |w|)."""
    absw = np.abs(wl.w)
    return oracle.indexer_logits(wl.q_idx, absw, wl.index_cache, wl.block_table, wl.seq_lens_k,
                                 wl.cu_seqlens_q, wl.cfg.page_size, wl.cfg.idx_kind, rows=rows)


def check_logits(gpu_logits, wl, rows, ref=None):
    ref = ref if ref is not None else oracle.indexer_logits(
        wl.q_idx, wl.w, wl.index_cache, wl.block_table, wl.seq_lens_k, wl.cu_seqlens_q,
        wl.cfg.page_size, wl.cfg.idx_kind, rows=rows)
    scale = logits_tolerance_scale(wl, rows)
    worst = 0.0
    for t in rows:
        n = len(ref[t])
        got = np.asarray(gpu_logits[t][:n], dtype=np.float64)
        # an infinite oracle value (a position on an absent page, -inf; a
        # forced position, +inf) must come out as exactly that value
        inf = ~np.isfinite(ref[t])
        if not np.array_equal(got[inf], ref[t][inf]):
            i = int(np.nonzero(inf & (got != ref[t]))[0][0])
            raise AssertionError(f"row {t}: position {i} should be {ref[t][i]!r}, gpu {got[i]!r}")
        fin = ~inf
        bound = np.zeros(n)
        bound[fin] = LOGIT_RTOL * np.maximum(np.abs(ref[t][fin]), scale[t][fin])
        err = np.zeros(n)
        err[fin] = np.abs(got[fin] - ref[t][fin])
        bad = ~(err <= bound)
        if bad.any():
            i = int(np.argmax(bad))
            raise AssertionError(f"row {t}: logits differ at {int(bad.sum())} of {n} positions; "
                                 f"first at {i}: gpu {got[i]!r} oracle {ref[t][i]!r} bound {bound[i]!r}")
        if n:
            worst = max(worst, float((err / np.maximum(bound, 1e-300)).max()))
    return ref, worst


def visible_of(wl):
    return [r.visible for r in oracle.row_layout(wl.seq_lens_k, wl.cu_seqlens_q)]


def check_topk_exact(gpu_idx_rows, gpu_logits_rows, visible, k, rows):
    """GPU top-k on the GPU's logits vs the oracle's top-k on the same values."""
    for t in rows:
        want = oracle.topk_row(np.asarray(gpu_logits_rows[t], dtype=np.float64), visible[t], k)
        got = np.asarray(gpu_idx_rows[t], dtype=np.int64)
        if not np.array_equal(got, want):
            diff = np.nonzero(got != want)[0]
            raise AssertionError(f"row {t}: top-k differs at {len(diff)} slots, first {diff[0]}: "
                                 f"gpu {got[diff[0]]} oracle {want[diff[0]]}")


def check_topk_near_ties(gpu_idx_row, ref_logits_row, visible, k):
    """End-to-end rule: set equality up to near-ties at the k-th score."""
    got = np.asarray(gpu_idx_row, dtype=np.int64)
    n_sel = min(k, visible)
    sel = got[:n_sel]
    assert (got[n_sel:] == -1).all(), "tail after the selected positions must be -1"
    assert ((sel >= 0) & (sel < visible)).all(), "selected positions must be visible"
    assert len(np.unique(sel)) == n_sel, "selected positions must be distinct"
    assert np.all(np.diff(sel) > 0), "selected positions must be ascending"
    want = oracle.topk_row(ref_logits_row, visible, k)[:n_sel]
    if visible <= k:
        assert np.array_equal(sel, want)
        return 0
    vals = np.asarray(ref_logits_row[:visible], dtype=np.float64)
    tau = np.sort(vals)[::-1][k - 1]
    sym = np.setxor1d(sel, want)
    tol = TIE_RTOL * max(abs(tau), 1.0)
    far = sym[np.abs(vals[sym] - tau) > tol]
    assert len(far) == 0, f"{len(far)} positions differ beyond the near-tie window (tau {tau})"
    return len(sym)


def check_attention(gpu_out, gpu_lse, wl, gpu_idx, rows, fp32=False):
    res = oracle.sparse_mla(wl.q_mla, wl.latent, gpu_idx, wl.block_table, wl.seq_lens_k,
                            wl.cu_seqlens_q, wl.cfg.page_size, wl.cfg.d_latent,
                            wl.cfg.softmax_scale, wl.cfg.mla_kind, rows=rows,
                            q_scale=wl.extras.get("q_scale", 1.0), kv_scale=wl.extras.get("kv_scale", 1.0))
    atol, rtol = (1e-4, 1e-4) if fp32 else (2e-2, 1e-2)
    latol, lrtol = (1e-5, 1e-5) if fp32 else (1e-3, 1e-3)
    worst = 0.0
    for t in rows:
        o_ref, l_ref = res[t]
        o = np.asarray(gpu_out[t], dtype=np.float64)
        l = np.asarray(gpu_lse[t], dtype=np.float64)
        bound = atol + rtol * np.abs(o_ref)
        err = np.abs(o - o_ref)
        if not (err <= bound).all():
            h, d = np.unravel_index(int(np.argmax(err - bound)), err.shape)
            raise AssertionError(f"row {t}: out differs at head {h} dim {d}: gpu {o[h, d]} oracle {o_ref[h, d]}")
        finite = np.isfinite(l_ref)
        assert np.array_equal(finite, np.isfinite(l)), f"row {t}: lse finiteness differs"
        assert (np.isneginf(l[~finite])).all()
        lb = latol + lrtol * np.abs(l_ref[finite])
        assert (np.abs(l[finite] - l_ref[finite]) <= lb).all(), f"row {t}: lse differs"
        worst = max(worst, float((err / bound).max()))
    return worst
