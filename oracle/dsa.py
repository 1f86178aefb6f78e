"""Float64 reference for the three stages of the DSA step.

TEST INFRASTRUCTURE ONLY (see the package docstring). Plain definitions, no
blocking or fusion: every value is computed in float64 from exactly decoded
inputs, one query row at a time.

Storage conventions (the inputs are the same bytes the HIP library reads):

* Index-K cache: one record per page. A page holds `P*D` key elements of the
  key dtype (fp8 E4M3 bytes, or little-endian float32), token-major, followed
  by `P` little-endian float32 scales, one per token. With P = 64, D = 128 and
  fp8 keys that is the 132 bytes per token of the SGLang indexer page
  (`_get_topk_paged` views the cache as [pages, 64, 1, 132]).
* Latent cache: [pages, P, Dl + Dr] rows; the first Dl elements are the
  compressed latent `c`, the last Dr the rope key. Key = whole row, value =
  first Dl elements (Ascend SFA page, `_execute_sparse_flash_attention_process`
  passes the same cache as key and value; vLLM MLA page splits the cached row
  512 | 64).
* Block table: [B, max_pages] physical page ids; logical position `p` of
  request `b` lives at page `block_table[b, p // P]`, slot `p % P` (SGLang
  page, `forward_indexer` builds it from `req_to_token` strided by the page
  size).
"""

from dataclasses import dataclass

import numpy as np

from .formats import decode_bf16, decode_e4m3fn


@dataclass(frozen=True)
class RowInfo:
    seq: int       # request the row belongs to
    visible: int   # number of keys the row may see: positions [0, visible)


def row_layout(seq_lens_k, cu_seqlens_q=None):
    """Query rows of a batch and how many keys each one may see.

    Decode (`cu_seqlens_q is None`): one row per request, and the row sees
    the whole cache of its request, its own key included (the SGLang page
    stores the new index key before scoring, `Indexer.forward_cuda`).

    Prefill / extend: request b owns rows `cu[b] .. cu[b+1]-1`. Causality is
    bottom-right aligned (`sparse_mode=3` on the Ascend SFA page; the SGLang
    context-parallel split gives row i the key end `start + i + 1`): the j-th
    of `q_len` rows sees `seq_lens_k[b] - q_len + j + 1` keys.
    """
    rows = []
    seq_lens_k = np.asarray(seq_lens_k)
    if cu_seqlens_q is None:
        for b, n in enumerate(seq_lens_k):
            rows.append(RowInfo(b, max(0, int(n))))
    else:
        cu = np.asarray(cu_seqlens_q)
        for b in range(len(seq_lens_k)):
            q_len = int(cu[b + 1] - cu[b])
            for j in range(q_len):
                rows.append(RowInfo(b, max(0, int(seq_lens_k[b]) - q_len + j + 1)))
    return rows


def _decode_keys(raw, kind):
    if kind == "fp8":
        return decode_e4m3fn(raw)
    if kind == "f32":
        return raw.view("<f4").astype(np.float64)
    raise ValueError(f"unknown key kind {kind!r}")


def page_of(block_table_row, p, page_size, num_pages):
    """Physical page of logical position `p`, or None when the position names
    no page of the pool.

    The pages always hand the kernels well-formed tables. The library states
    what happens otherwise, and the oracle follows it: a table entry outside
    [0, num_pages) is an absent page. The indexer then scores the position
    -inf and attention skips it. (A position past the table row's width has
    no entry at all; callers keep seq_lens_k within the table, and the oracle
    only guards against indexing past the row.)
    """
    slot = int(p) // page_size
    if slot >= len(block_table_row):
        return None
    page = int(block_table_row[slot])
    if page < 0 or page >= num_pages:
        return None
    return page


def gather_index_keys(index_cache, block_table_row, n, page_size, head_dim, kind):
    """Keys k[p] (float64 [n, D]) and scales sigma[p] (float64 [n]) of
    positions 0..n-1 of one request, walked through its block-table row.
    A position on an absent page (`page_of`) gets NaN for its key and scale."""
    elem = 1 if kind == "fp8" else 4
    keys = np.empty((n, head_dim), dtype=np.float64)
    sigma = np.empty(n, dtype=np.float64)
    for p in range(n):
        page = page_of(block_table_row, p, page_size, len(index_cache))
        if page is None:
            keys[p] = np.nan
            sigma[p] = np.nan
            continue
        slot = p % page_size
        record = index_cache[page]
        k_raw = record[slot * head_dim * elem:(slot + 1) * head_dim * elem]
        keys[p] = _decode_keys(k_raw, kind)
        s_off = page_size * head_dim * elem + 4 * slot
        sigma[p] = record[s_off:s_off + 4].view("<f4").astype(np.float64)[0]
    return keys, sigma


def indexer_logits_row(q_row, w_row, keys, sigma):
    """Lightning-indexer score of one query row over the given keys.

        L[p] = sum_h w[h] * relu(sigma[p] * (q[h] . k[p]))

    q_row [H, D], w_row [H] (the head gate with the q scale folded in, as
    `_get_logits_head_gate` returns it), keys [n, D], sigma [n]. The scale
    sits inside the relu, as the formula states it.
    """
    dots = keys @ q_row.T                          # [n, H]: q[h] . k[p]
    gated = np.maximum(0.0, sigma[:, None] * dots)  # relu(sigma_p * dot)
    return gated @ w_row                            # sum over heads


def mask_init_and_local(logits_row, visible, num_init, num_local):
    """Force the first `num_init` and the last `num_local` visible positions
    into the selection by giving them +inf (SGLang indexer page,
    `Indexer._mask_init_and_local_tokens`).

    On the page a row's keys start at column `row_start` of the logits. The
    init columns are `row_start + i` for i < num_init, clamped to the last
    column; the local columns are `row_start + length - 1 - i` for
    i < num_local, clamped at column 0. Here every row starts at position 0
    and `visible` is the row's own length (for a prefill row, the keys that
    row may see, not the request's). Columns that land outside
    [0, visible) after those clamps belong to no key of the row, and top-k
    never reads them. So the forced set is [0, min(num_init, visible)) and
    [max(visible - num_local, 0), visible). Returns a new array.
    """
    out = np.array(logits_row, dtype=np.float64, copy=True)
    n = int(visible)
    for i in range(int(num_init)):
        if i < n:
            out[i] = np.inf
    for i in range(int(num_local)):
        pos = max(n - 1 - i, 0)
        if pos < n:
            out[pos] = np.inf
    return out


def indexer_logits(q, w, index_cache, block_table, seq_lens_k, cu_seqlens_q,
                   page_size, kind, rows=None, num_init=0, num_local=0):
    """Logits for every query row (or only the listed `rows`).

    q: [T, H, D] fp8 codes (uint8) for kind "fp8", float32 for kind "f32".
    w: [T, H] float32. Returns {row: float64 [visible]}; columns at or past a
    row's visible length are not defined by the method (the CUDA kernels on
    the SGLang page are called with `clean_logits=False`).
    """
    info = row_layout(seq_lens_k, cu_seqlens_q)
    head_dim = q.shape[2]
    wanted = list(range(len(info)) if rows is None else rows)
    # keys of each request are gathered once, up to the longest row that needs them
    longest = {}
    for t in wanted:
        longest[info[t].seq] = max(longest.get(info[t].seq, 0), info[t].visible)
    gathered = {b: gather_index_keys(index_cache, block_table[b], n, page_size, head_dim, kind)
                for b, n in longest.items()}
    absent = {b: np.array([page_of(block_table[b], p, page_size, len(index_cache)) is None
                           for p in range(n)], dtype=bool)
              for b, n in longest.items()}
    out = {}
    for t in wanted:
        r = info[t]
        keys, sigma = gathered[r.seq]
        q_row = decode_e4m3fn(q[t]) if kind == "fp8" else np.asarray(q[t], dtype=np.float64)
        w_row = np.asarray(w[t], dtype=np.float64)
        out[t] = indexer_logits_row(q_row, w_row, keys[:r.visible], sigma[:r.visible])
        out[t][absent[r.seq][:r.visible]] = -np.inf     # absent page: no key to score
        if num_init or num_local:
            out[t] = mask_init_and_local(out[t], r.visible, num_init, num_local)
    return out


def topk_row(logits_row, visible, k):
    """Top-k positions of one row, stored ascending, padded with -1 to k.

    * visible <= k: every visible position, `[0, 1, .., visible-1]` then -1
      (the short-row rule the SGLang page relies on in
      `_forward_cuda_k_only`, and `forward_indexer` taking
      `topk(min(topk, seq_len))` then padding with -1).
    * otherwise the k positions with the largest logits. Ties at the k-th
      value go to the lower position (the pages are silent on ties).
    The pages treat the result as a set: the SGLang indexer page lets each
    attention backend rewrite the top-k output in `topk_transform`, so no
    order is part of the method. The oracle stores the set in ascending
    position order, a canonical form in which two equal sets are equal
    arrays.
    """
    out = np.full(k, -1, dtype=np.int64)
    if visible <= k:
        out[:visible] = np.arange(visible)
        return out
    vals = np.asarray(logits_row[:visible], dtype=np.float64)
    positions = np.arange(visible)
    order = np.lexsort((positions, -vals))   # by value descending, then position
    chosen = np.sort(order[:k])
    out[:k] = chosen
    return out


def topk(logits_by_row, visible_by_row, k):
    """{row: indices} for the rows of `logits_by_row`."""
    return {t: topk_row(logits_by_row[t], visible_by_row[t], k) for t in logits_by_row}


def _decode_latent(raw, kind):
    if kind == "bf16":
        return decode_bf16(raw)
    if kind == "fp8":
        return decode_e4m3fn(raw)
    return np.asarray(raw, dtype=np.float64)


def gather_latent_rows(latent_cache, block_table_row, positions, page_size, kind):
    """Latent rows C[p] (float64 [len(positions), Dl+Dr]) through the block
    table; for kind "fp8" the decoded E4M3 codes (the caller applies the scale)."""
    rows = []
    for p in positions:
        page = int(block_table_row[int(p) // page_size])
        slot = int(p) % page_size
        raw = latent_cache[page, slot]
        rows.append(_decode_latent(raw, kind))
    if not rows:
        return np.zeros((0, latent_cache.shape[-1]), dtype=np.float64)
    return np.stack(rows)


def _valid_positions(idx_row, seq_len, block_table_row, page_size, num_pages):
    """Entries that name a token of the request, in list order, duplicates
    kept. -1 (the pages pad unused top-k slots with it) and anything outside
    [0, seq_len) are skipped, and so is a position on an absent page
    (`page_of`)."""
    keep = []
    for p in np.asarray(idx_row).tolist():
        if 0 <= p < seq_len and page_of(block_table_row, p, page_size, num_pages) is not None:
            keep.append(p)
    return np.asarray(keep, dtype=np.int64)


def sparse_mla_row(q_row, rows_c, d_latent, scale, return_probs=False):
    """Attention of one query row over the gathered latent rows.

    q_row [Hm, Dl+Dr] (absorbed no-rope part followed by the rope part),
    rows_c [n, Dl+Dr]. Per head h:
        z_i = scale * (q[h] . C_i)
        out[h] = sum_i softmax(z)_i * C_i[:Dl],   lse[h] = log sum_i exp(z_i)
    An empty selection gives out = 0 and lse = -inf.
    """
    n_heads = q_row.shape[0]
    if rows_c.shape[0] == 0:
        out = np.zeros((n_heads, d_latent))
        lse = np.full(n_heads, -np.inf)
        return (out, lse, np.zeros((n_heads, 0))) if return_probs else (out, lse)
    z = scale * (q_row @ rows_c.T)               # [Hm, n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    s = e.sum(axis=1, keepdims=True)
    probs = e / s
    out = probs @ rows_c[:, :d_latent]
    lse = (m + np.log(s))[:, 0]
    return (out, lse, probs) if return_probs else (out, lse)


def sparse_mla(q, latent_cache, topk_idx, block_table, seq_lens_k, cu_seqlens_q,
               page_size, d_latent, scale, kind, rows=None, q_scale=1.0, kv_scale=1.0):
    """Sparse MLA for every query row (or the listed rows).

    q: [T, Hm, Dqk] bf16 bits (uint16) for kind "bf16", float32 for "f32",
    E4M3 codes (uint8) for "fp8".
    topk_idx: [T, k] logical positions, -1 = empty slot.
    Returns {row: (out float64 [Hm, Dl], lse float64 [Hm])}.

    fp8 (vLLM MLA page, the decode path under `fp8_attention`: the absorbed
    query goes through `scaled_fp8_quant` with the layer's q scale, and the
    cache is written in fp8 with the layer's k scale): one scale per tensor,
    so the query is codes * q_scale and every cached row codes * kv_scale;
    the attention is then the same as for the other kinds, on those values.
    """
    info = row_layout(seq_lens_k, cu_seqlens_q)
    wanted = range(len(info)) if rows is None else rows
    res = {}
    for t in wanted:
        b = info[t].seq
        pos = _valid_positions(topk_idx[t], int(seq_lens_k[b]), block_table[b], page_size,
                               len(latent_cache))
        rows_c = gather_latent_rows(latent_cache, block_table[b], pos, page_size, kind)
        q_row = _decode_latent(q[t], kind)
        if kind == "fp8":
            rows_c = rows_c * float(kv_scale)
            q_row = q_row * float(q_scale)
        res[t] = sparse_mla_row(q_row, rows_c, d_latent, scale)
    return res


def dense_mla(q_row, all_rows_c, d_latent, scale):
    """Dense attention of one row over all its visible latent rows, coded
    without the max-subtraction route used above: per head, weights are
    computed one key at a time against the log-sum-exp from scipy. This is
    the dense counterpart the sparse step must equal when k >= context."""
    from scipy.special import logsumexp

    n_heads = q_row.shape[0]
    out = np.zeros((n_heads, d_latent))
    lse = np.empty(n_heads)
    for h in range(n_heads):
        z = np.array([scale * float(np.dot(q_row[h], c)) for c in all_rows_c])
        lse[h] = logsumexp(z)
        for i, c in enumerate(all_rows_c):
            out[h] += np.exp(z[i] - lse[h]) * c[:d_latent]
    return out, lse


def lse_merge(o1, lse1, o2, lse2):
    """Merge two partial attention results over disjoint key sets
    (`merge_attn_states` on the vLLM MLA page):

        lse = log(exp(lse1) + exp(lse2))
        o   = (exp(lse1) * o1 + exp(lse2) * o2) / exp(lse)

    evaluated relative to the larger lse. Both empty -> o = 0, lse = -inf.
    """
    lse1 = np.asarray(lse1, dtype=np.float64)
    lse2 = np.asarray(lse2, dtype=np.float64)
    m = np.maximum(lse1, lse2)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    a1 = np.exp(lse1 - safe_m)
    a2 = np.exp(lse2 - safe_m)
    tot = a1 + a2
    with np.errstate(invalid="ignore", divide="ignore"):
        o = (a1[..., None] * o1 + a2[..., None] * o2) / tot[..., None]
        lse = safe_m + np.log(tot)
    empty = tot == 0
    o = np.where(empty[..., None], 0.0, o)
    lse = np.where(empty, -np.inf, lse)
    return o, lse
