"""Float64 CPU oracle for the DeepSeek-Sparse-Attention (DSA) step.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: it exists so that `tests/`, the smoke check in
`__graft_entry__.py` and the `cpu_baseline` leg of `bench.py` can compare the
HIP kernels against a plain, slow, obviously correct definition of what the
step computes. It shares no code, tables, headers or constants with the HIP
library, and imports nothing from it.

Sources (web pages, cited by title and section):

* "sglang/srt/layers/attention/dsa/dsa_indexer.py" (the SGLang lightning
  indexer page): `Indexer.forward_indexer` (per-request score + `topk`),
  `Indexer._get_topk_paged` / `_get_topk_ragged` (paged fp8 index-K cache,
  132 bytes per token, weights squeezed to [T, H]), `_forward_cuda_k_only`
  (short rows give `[0 .. len-1, -1 ...]`), `_get_logits_head_gate`
  (q scale folded into the head weights).
* "vllm_ascend/attention/sfa_v1.py" (the Ascend SFA page):
  `_execute_sparse_flash_attention_process` (key = value = latent cache,
  rope part passed separately, token-granular sparse indices, causal
  `sparse_mode=3`), `indexer_select_post_process` (`sparse_count=2048`).
* "vllm.v1.attention.backends.mla.common" (the vLLM MLA API page):
  `merge_attn_states` use in `_compute_prefill_context` (LSE merge), the
  decode path returning `(attn_out, lse)`, the 512 | 64 split of the latent
  row.

Every function states the plain definition it implements. Where the pages are
silent the reading taken is stated in the function's docstring.

Parity status per function (what pins it; see tests/test_oracle_*.py):

* formats.e4m3fn_table / decode_bf16 ... pinned (format definition code points,
  exhaustive agreement with torch's CPU conversion).
* dsa.indexer_logits ..................... pinned (hand-worked golden example,
  brute-force loops, textbook matmul special case, page-permutation and
  zero-weight-head invariances).
* dsa.mask_init_and_local ................ pinned (hand-worked golden example
  of the SGLang page's init/local windows over decode and prefill rows, which
  rejects an off-by-one local window and a window anchored at the request's
  length; forced positions always selected, the rest ranked as before).
* dsa.page_of (absent pages) ............. pinned (the indexer hand example with
  a page id outside the pool: -inf there, the hand-worked values elsewhere;
  the attention hand example reduced to its one-index closed form).
* dsa.topk ............................... pinned (brute-force full sort,
  short-row rule, order-statistic property, affine invariance).
* dsa.sparse_mla ......................... pinned (closed forms for one index
  and q = 0, softmax sums to one, equality with an independently coded dense
  attention when k >= context, split + LSE merge, absorption identity).
* dsa.sparse_mla, fp8 latent cache ........ pinned (exact reduction to the
  float path with power-of-two scales; moving factors between the softmax,
  query and cache scales).
* dsa.lse_merge .......................... pinned (associativity against a
  single pass, closed form for equal halves).
* quant.encode_e4m3fn / quant_rows /
  quant_index_q / store_index_k .......... pinned (every finite code round
  trips, ties and near-ties between all neighbours, torch's CPU conversion on
  a million values, amax lands on 448, power-of-two scale invariance, half-step
  error bound, paged store read back through dsa.gather_index_keys).
"""

from .formats import decode_bf16, decode_e4m3fn, e4m3fn_table  # noqa: F401
from .dsa import (  # noqa: F401
    RowInfo,
    dense_mla,
    gather_index_keys,
    gather_latent_rows,
    indexer_logits,
    indexer_logits_row,
    lse_merge,
    mask_init_and_local,
    page_of,
    row_layout,
    sparse_mla,
    sparse_mla_row,
    topk,
    topk_row,
)
from .quant import encode_e4m3fn, quant_index_q, quant_rows, store_index_k  # noqa: F401
