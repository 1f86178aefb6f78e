"""Pin of the oracle's init/local-token forcing (no GPU).

The expected forced positions come from `tests/golden/init_local_hand_example.json`,
worked by hand from the SGLang indexer page's `Indexer._mask_init_and_local_tokens`
in its ragged and paged layouts. The oracle is run on a batch of those lengths
(decode rows and prefill rows of different visible lengths, both windows longer
than some rows), and two plausible mistakes planted in the oracle must be
rejected by the same fixture.
"""
import json
import os

import numpy as np
import pytest

import oracle
from tests.packing import pack_index_cache_f32

PAGE = 16
H, D = 2, 4


def _golden(golden_dir):
    return json.load(open(os.path.join(golden_dir, "init_local_hand_example.json")))


def _batch(ex):
    """f32 keys on one page per request (identity block table), random q, w."""
    rng = np.random.default_rng(2024)
    lens = np.array(ex["seq_lens_k"], dtype=np.int32)
    cu = np.concatenate([[0], np.cumsum(ex["q_lens"])]).astype(np.int32)
    B, T = len(lens), int(cu[-1])
    keys = rng.standard_normal((B, PAGE, D)).astype(np.float32)
    sigma = np.ones((B, PAGE), dtype=np.float32)
    cache = pack_index_cache_f32(keys, sigma)
    bt = np.arange(B, dtype=np.int32)[:, None]
    q = rng.standard_normal((T, H, D)).astype(np.float32)
    w = rng.standard_normal((T, H)).astype(np.float32)
    return dict(q=q, w=w, index_cache=cache, block_table=bt, seq_lens_k=lens, cu_seqlens_q=cu,
                page_size=PAGE, kind="f32")


def _forced_sets(logits_by_row):
    return {t: sorted(int(i) for i in np.nonzero(np.isposinf(v))[0]) for t, v in logits_by_row.items()}


def _matches_golden(ex, logits_by_row, plain_by_row):
    """True when every row has the golden visible length, exactly the golden
    forced positions, and its other positions untouched."""
    for r in ex["rows"]:
        t = r["row"]
        got = logits_by_row[t]
        if len(got) != r["visible"]:
            return False
        if _forced_sets({t: got})[t] != r["forced"]:
            return False
        keep = np.ones(len(got), dtype=bool)
        keep[r["forced"]] = False
        if not np.array_equal(got[keep], plain_by_row[t][keep]):
            return False
    return True


def _run(ex, b):
    return oracle.indexer_logits(b["q"], b["w"], b["index_cache"], b["block_table"], b["seq_lens_k"],
                                 b["cu_seqlens_q"], b["page_size"], b["kind"],
                                 num_init=ex["num_init"], num_local=ex["num_local"])


def test_forcing_matches_hand_worked_rows(golden_dir):
    ex = _golden(golden_dir)
    b = _batch(ex)
    plain = oracle.indexer_logits(b["q"], b["w"], b["index_cache"], b["block_table"], b["seq_lens_k"],
                                  b["cu_seqlens_q"], b["page_size"], b["kind"])
    assert not any(np.isinf(v).any() for v in plain.values())
    forced = _run(ex, b)
    assert [r.visible for r in oracle.row_layout(b["seq_lens_k"], b["cu_seqlens_q"])] == \
        [r["visible"] for r in ex["rows"]]
    assert _matches_golden(ex, forced, plain)


def _local_off_by_one(logits_row, visible, num_init, num_local):
    """Planted mistake: the local window ends one past the row (length - i)."""
    out = np.array(logits_row, dtype=np.float64, copy=True)
    n = int(visible)
    for i in range(int(num_init)):
        if i < n:
            out[i] = np.inf
    for i in range(int(num_local)):
        pos = max(n - i, 0)
        if pos < n:
            out[pos] = np.inf
    return out


def test_golden_rejects_local_window_off_by_one(golden_dir, monkeypatch):
    ex = _golden(golden_dir)
    b = _batch(ex)
    plain = _run({"num_init": 0, "num_local": 0}, b)
    monkeypatch.setattr(oracle.dsa, "mask_init_and_local", _local_off_by_one)
    assert not _matches_golden(ex, _run(ex, b), plain)


def test_golden_rejects_window_anchored_at_request_length(golden_dir, monkeypatch):
    """Planted mistake: the local window of a prefill row is placed at the
    end of the request's keys (seq_lens_k) rather than at the row's own
    visible length."""
    ex = _golden(golden_dir)
    b = _batch(ex)
    plain = _run({"num_init": 0, "num_local": 0}, b)
    real_mask = oracle.dsa.mask_init_and_local
    real_layout = oracle.dsa.row_layout
    rows = real_layout(b["seq_lens_k"], b["cu_seqlens_q"])
    calls = iter(range(len(rows)))

    def anchored(logits_row, visible, num_init, num_local):
        t = next(calls)
        seq_len = int(b["seq_lens_k"][rows[t].seq])
        padded = np.concatenate([logits_row, np.zeros(seq_len - int(visible))])
        return real_mask(padded, seq_len, num_init, num_local)[:int(visible)]

    monkeypatch.setattr(oracle.dsa, "mask_init_and_local", anchored)
    assert not _matches_golden(ex, _run(ex, b), plain)


@pytest.mark.parametrize("k", [1, 3, 5, 8])
def test_forced_positions_are_selected(golden_dir, k):
    """Top-k over forced logits holds every forced position (the lower ones
    when more are forced than k) and fills the rest by value."""
    ex = _golden(golden_dir)
    b = _batch(ex)
    plain = _run({"num_init": 0, "num_local": 0}, b)
    forced = _run(ex, b)
    for r in ex["rows"]:
        t, n = r["row"], r["visible"]
        chosen = [int(x) for x in oracle.topk_row(forced[t], n, k) if x >= 0]
        want_forced = r["forced"]
        if len(want_forced) >= min(k, n):
            assert chosen == want_forced[:min(k, n)]
        else:
            assert set(want_forced) <= set(chosen)
            rest = sorted((i for i in range(n) if i not in want_forced), key=lambda i: (-plain[t][i], i))
            assert set(chosen) - set(want_forced) == set(rest[:min(k, n) - len(want_forced)])
