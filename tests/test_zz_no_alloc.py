"""sparse_mla_decode_noalloc (split partials in the library's static per-GPU
scratch) against sparse_mla_decode with a caller workspace, through the C ABI:
two calls in a row, the second on a smaller batch, must give the same bytes."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from dsa_workloads import generate, small_config  # noqa: E402

pytestmark = pytest.mark.gpu


def _case(name, seed, lens, kind="bf16"):
    from dsa_workloads.device import make_step
    cfg = small_config(name, seed=seed, lens=lens, mla_kind=kind,
                       **({"idx_kind": "f32", "page_size": 16} if kind == "f32" else {}))
    wl = generate(cfg, with_indexer=False)
    step = make_step(wl)
    rng = np.random.default_rng(seed)
    idx = np.full((wl.num_rows, cfg.topk), -1, dtype=np.int32)
    for t, n in enumerate(wl.seq_lens_k):
        m = min(int(n), cfg.topk)
        idx[t, :m] = np.sort(rng.choice(int(n), size=m, replace=False))
    return cfg, step, torch.from_numpy(idx).cuda()


def _both(cfg, step, idx):
    import sparse_mla_attention_dsa_amd as dsa
    step.attend(topk_idx=idx)
    ref_out, ref_lse = step.out.clone(), step.lse.clone()
    out = torch.full_like(step.out, float("nan"))
    lse = torch.full_like(step.lse, float("nan"))
    dsa.sparse_mla_decode_noalloc(step.batch, step.q_mla, step.kv_cache, idx, cfg.softmax_scale, out, lse,
                                  d_latent=cfg.d_latent)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out,
                       ref_out.view(torch.int16) if ref_out.dtype == torch.bfloat16 else ref_out)
    assert torch.equal(lse, ref_lse)


@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_noalloc_matches_workspace_call_twice(kind):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mla_attention_dsa_amd as dsa
    lens = [int(x) for x in np.random.default_rng(900).integers(2100, 5000, size=64)]
    big = _case(f"na_big_{kind}", 901, lens, kind)
    small = _case(f"na_small_{kind}", 902, [3000, 700, 4500], kind)
    for cfg, step, idx in (big, small):
        need = dsa.dsa_workspace_bytes(dsa.DSA_OP_MLA_DECODE, step.batch, cfg.topk, cfg.mla_heads, cfg.d_latent,
                                       dsa.DSA_BF16 if kind == "bf16" else dsa.DSA_F32)
        print(f"\n[noalloc] {cfg.name}: rows {len(cfg.ctx)} partials {need} bytes", flush=True)
        if kind == "bf16":
            assert need > 0
        _both(cfg, step, idx)
