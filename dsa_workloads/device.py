"""Copy a generated Workload to a torch device and wrap it in a DsaStep."""
import torch


def upload(wl, device="cuda"):
    """Device tensors with the same bytes as the host arrays of `wl`."""
    def t(a, dtype=None):
        x = torch.from_numpy(a)
        if dtype is not None:
            x = x.view(dtype)
        return x.to(device)

    cfg = wl.cfg
    d = {
        "block_table": t(wl.block_table),
        "seq_lens_k": t(wl.seq_lens_k),
        "cu_seqlens_q": None if wl.cu_seqlens_q is None else t(wl.cu_seqlens_q),
        "index_cache": t(wl.index_cache),
        "q_idx": t(wl.q_idx, torch.float8_e4m3fn) if cfg.idx_kind == "fp8" else t(wl.q_idx),
        "w": t(wl.w),
        "kv_cache": t(wl.latent.view("int16"), torch.bfloat16) if cfg.mla_kind == "bf16" else t(wl.latent),
        "q_mla": t(wl.q_mla.view("int16"), torch.bfloat16) if cfg.mla_kind == "bf16" else t(wl.q_mla),
    }
    return d


def make_step(wl, device="cuda", fused=False):
    from sparse_mla_attention_dsa_amd.step import DsaStep

    d = upload(wl, device)
    cfg = wl.cfg
    return DsaStep(block_table=d["block_table"], seq_lens_k=d["seq_lens_k"],
                   cu_seqlens_q=d["cu_seqlens_q"], page_size=cfg.page_size, num_pages=wl.num_pages,
                   max_seq_len_k=wl.max_seq_len_k, max_seq_len_q=wl.max_seq_len_q,
                   num_rows=wl.num_rows, q_idx=d["q_idx"], w=d["w"], index_cache=d["index_cache"],
                   q_mla=d["q_mla"], kv_cache=d["kv_cache"], topk=cfg.topk,
                   softmax_scale=cfg.softmax_scale, d_latent=cfg.d_latent,
                   mla_scales=(wl.extras["q_scale"], wl.extras["kv_scale"]) if cfg.mla_kind == "fp8" else None,
                   fused=fused)
