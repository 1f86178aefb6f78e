"""One DSA step of one layer on one stream: indexer logits -> top-k -> sparse MLA.

Allocates the intermediate buffers once (logits, indices, output, lse,
workspace) and replays the three library calls. Allocation happens here, in
the constructor; `run()` itself allocates nothing. With `fused=True` the
indexer and the top-k are one call (dsa_indexer_topk, fp8 indexer only) and no
logits buffer exists.
"""
import torch

from . import (DSA_BF16, DSA_F32, DSA_FP8_E4M3, DSA_OP_INDEXER_TOPK, DSA_OP_MLA_DECODE, DSA_OP_MLA_PREFILL,
               DSA_OP_TOPK, dsa_indexer_logits, dsa_indexer_topk, dsa_topk, dsa_workspace_bytes, make_batch,
               sparse_mla_decode, sparse_mla_decode_fp8, sparse_mla_prefill, sparse_mla_prefill_fp8)


class DsaStep:
    def __init__(self, *, block_table, seq_lens_k, cu_seqlens_q, page_size, num_pages,
                 max_seq_len_k, max_seq_len_q, num_rows, q_idx, w, index_cache, q_mla, kv_cache,
                 topk, softmax_scale, d_latent, mla_scales=None, num_init_tokens=0, num_local_tokens=0,
                 fused=False):
        self.prefill = cu_seqlens_q is not None
        self.batch = make_batch(block_table, seq_lens_k, cu_seqlens_q, page_size=page_size,
                                num_pages=num_pages, max_seq_len_k=max_seq_len_k,
                                max_seq_len_q=max_seq_len_q, num_rows=num_rows)
        dev = q_mla.device
        self.q_idx, self.w, self.index_cache = q_idx, w, index_cache
        self.num_init_tokens, self.num_local_tokens = int(num_init_tokens), int(num_local_tokens)
        self.q_mla, self.kv_cache = q_mla, kv_cache
        self.topk, self.softmax_scale, self.d_latent = int(topk), float(softmax_scale), int(d_latent)
        T, Hm = num_rows, int(q_mla.shape[1])
        self.fused = bool(fused)
        if self.fused and q_idx.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise ValueError("the fused indexer + top-k call takes the fp8 indexer inputs only")
        stride = max(1, (max_seq_len_k + 3) // 4 * 4)
        self.logits = None if self.fused else torch.empty((T, stride), dtype=torch.float32, device=dev)
        self.topk_idx = torch.empty((T, self.topk), dtype=torch.int32, device=dev)
        # an fp8 latent cache (E4M3 codes) comes with its (q_scale, kv_scale)
        self.fp8 = q_mla.dtype in (torch.uint8, torch.float8_e4m3fn)
        if self.fp8 and mla_scales is None:
            raise ValueError("an fp8 latent cache needs mla_scales=(q_scale, kv_scale)")
        self.mla_scales = tuple(float(x) for x in mla_scales) if self.fp8 else None
        out_dtype = torch.float32 if q_mla.dtype == torch.float32 else torch.bfloat16
        self.out = torch.empty((T, Hm, self.d_latent), dtype=out_dtype, device=dev)
        self.lse = torch.empty((T, Hm), dtype=torch.float32, device=dev)
        mla_dtype = DSA_F32 if q_mla.dtype == torch.float32 else (DSA_FP8_E4M3 if self.fp8 else DSA_BF16)
        op = DSA_OP_MLA_PREFILL if self.prefill else DSA_OP_MLA_DECODE
        nbytes = dsa_workspace_bytes(op, self.batch, self.topk, Hm, self.d_latent, mla_dtype)
        self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev) if nbytes else None
        tk_op = DSA_OP_INDEXER_TOPK if self.fused else DSA_OP_TOPK
        tk_bytes = dsa_workspace_bytes(tk_op, self.batch, self.topk, Hm, self.d_latent, mla_dtype)
        self.topk_workspace = torch.empty(tk_bytes, dtype=torch.uint8, device=dev) if tk_bytes else None

    def indexer(self, stream=None):
        dsa_indexer_logits(self.batch, self.q_idx, self.w, self.index_cache, self.logits,
                           num_init_tokens=self.num_init_tokens, num_local_tokens=self.num_local_tokens,
                           stream=stream)

    def select(self, stream=None):
        dsa_topk(self.batch, self.logits, self.topk, self.topk_idx, self.topk_workspace, stream=stream)

    def index_select(self, stream=None):
        """topk_idx from the indexer inputs: one fused call, or the scores then their top-k."""
        if self.fused:
            dsa_indexer_topk(self.batch, self.q_idx, self.w, self.index_cache, self.topk, self.topk_idx,
                             self.topk_workspace, num_init_tokens=self.num_init_tokens,
                             num_local_tokens=self.num_local_tokens, stream=stream)
            return
        self.indexer(stream)
        self.select(stream)

    def attend(self, stream=None, topk_idx=None):
        idx = self.topk_idx if topk_idx is None else topk_idx
        if self.fp8:
            fn = sparse_mla_prefill_fp8 if self.prefill else sparse_mla_decode_fp8
            q_scale, kv_scale = self.mla_scales
            fn(self.batch, self.q_mla, q_scale, self.kv_cache, kv_scale, idx, self.softmax_scale, self.out,
               self.lse, self.workspace, stream=stream)
            return
        fn = sparse_mla_prefill if self.prefill else sparse_mla_decode
        fn(self.batch, self.q_mla, self.kv_cache, idx, self.softmax_scale, self.out, self.lse,
           self.workspace, d_latent=self.d_latent, stream=stream)

    def run(self, stream=None):
        self.index_select(stream)
        self.attend(stream)
