"""GPU parity of the documented entry rules, on hand-built inputs.

Attention (`sparse_mla_decode` / `_prefill`, bf16, fp8 and fp32 caches) is fed
top-k lists that the library's own top-k never produces: -1 in the middle of
the list, positions at or past the request's length, positions on pages whose
block-table entry lies outside [0, num_pages) (-1 and num_pages and beyond),
duplicates (counted twice), descending and shuffled order, and a row with no
valid entry at all. k = 2048, so the entries of a row are cut into several
splits and the invalid ones land in different splits, some of which end up
empty. The indexer (stream, two-row stream, prefill, general and fp32 kernels)
is run on block tables with absent pages under visible positions: those
positions must score -inf, the others keep the parity rule, and top-k on the
result must be exact. Everything is compared with the oracle, which
implements the same rules.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from dsa_workloads import generate, small_config  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _break_pages(wl, rng, per_request=2):
    """Point some block-table entries that hold visible positions outside the
    pool: -1, num_pages, and a large id. Returns {request: [logical pages]}."""
    bad = {}
    ids = [-1, wl.num_pages, wl.num_pages + 1000, -7]
    P = wl.cfg.page_size
    for b, n in enumerate(wl.seq_lens_k):
        used = -(-int(n) // P)
        if used < 3:
            continue
        pages = sorted(rng.choice(np.arange(1, used), size=min(per_request, used - 1), replace=False).tolist())
        for i, lp in enumerate(pages):
            wl.block_table[b, lp] = ids[(b + i) % len(ids)]
        bad[b] = pages
    return bad


def _crafted_row(rng, seq_len, k, bad_pages, P, kind):
    """A k-entry list mixing valid positions (shuffled), duplicates, -1 in the
    middle, positions >= seq_len and positions on absent pages."""
    n_valid = min(seq_len, k // 2)
    valid = rng.choice(seq_len, size=n_valid, replace=False) if seq_len else np.zeros(0, dtype=np.int64)
    dups = rng.choice(valid, size=min(len(valid), k // 16), replace=True) if len(valid) else valid
    beyond = np.array([seq_len, seq_len + 1, seq_len + 63, 1 << 20, (1 << 31) - 1], dtype=np.int64)
    on_bad = np.concatenate([np.arange(lp * P, min((lp + 1) * P, seq_len)) for lp in bad_pages]) \
        if bad_pages else np.zeros(0, dtype=np.int64)
    on_bad = on_bad[:k // 8]
    parts = [valid, dups, beyond, on_bad, np.full(k // 16, -1), np.array([-5, -(1 << 30)])]
    row = np.concatenate(parts).astype(np.int64)
    row = row[:k]
    row = np.concatenate([row, np.full(k - len(row), -1)])
    if kind == "descending":
        row = np.sort(row)[::-1]
    else:
        rng.shuffle(row)
    return row.astype(np.int32)


def _all_invalid_row(rng, seq_len, k, bad_pages, P):
    on_bad = np.concatenate([np.arange(lp * P, min((lp + 1) * P, seq_len)) for lp in bad_pages]) \
        if bad_pages else np.zeros(0, dtype=np.int64)
    row = np.concatenate([on_bad, [seq_len, seq_len + 3, -1, -2]]).astype(np.int64)
    row = np.resize(row, k)
    rng.shuffle(row)
    return row.astype(np.int32)


MLA_CASES = [
    ("bf16_decode", dict(lens=[3000, 2600, 700, 4100], mla_kind="bf16")),
    ("bf16_prefill", dict(lens=[3000, 2600], q_lens=[3, 2], mla_kind="bf16")),
    ("fp8_decode", dict(lens=[3000, 2600, 700, 4100], mla_kind="fp8")),
    ("fp8_prefill", dict(lens=[3000, 2600], q_lens=[3, 2], mla_kind="fp8")),
    ("f32_decode", dict(lens=[3000, 2600, 700, 4100], mla_kind="f32", idx_kind="f32", page_size=16)),
    ("f32_prefill", dict(lens=[3000, 2600], q_lens=[3, 2], mla_kind="f32", idx_kind="f32", page_size=16)),
]


@pytest.mark.parametrize("name,kw", MLA_CASES, ids=[c[0] for c in MLA_CASES])
def test_attention_entry_rules(name, kw):
    _need_gpu()
    from dsa_workloads.device import make_step
    seed = 700 + [c[0] for c in MLA_CASES].index(name)
    rng = np.random.default_rng(seed)
    cfg = small_config(f"rules_{name}", seed=seed, topk=2048, **kw)
    wl = generate(cfg, with_indexer=False)
    bad = _break_pages(wl, rng)
    P, k = cfg.page_size, cfg.topk
    vis = parity.visible_of(wl)
    seqs = [r for r in range(len(wl.seq_lens_k))]
    row_seq = np.repeat(seqs, np.diff(wl.cu_seqlens_q)) if wl.cu_seqlens_q is not None else np.array(seqs)
    idx = np.empty((wl.num_rows, k), dtype=np.int32)
    for t in range(wl.num_rows):
        b = int(row_seq[t])
        L = int(wl.seq_lens_k[b])
        if t == wl.num_rows - 1:
            idx[t] = _all_invalid_row(rng, L, k, bad.get(b, []), P)
        else:
            idx[t] = _crafted_row(rng, L, k, bad.get(b, []), P, "descending" if t % 2 else "shuffled")
    step = make_step(wl)
    print(f"\n[rules] {name}: rows {wl.num_rows}, absent pages {bad}, visible {vis}", flush=True)
    step.attend(topk_idx=torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    out = step.out.float().cpu().numpy()
    lse = step.lse.cpu().numpy()
    worst = parity.check_attention(out, lse, wl, idx, list(range(wl.num_rows)), fp32=cfg.mla_kind == "f32")
    last = wl.num_rows - 1
    assert (out[last] == 0).all() and np.isneginf(lse[last]).all(), "a row with no valid entry gives 0 / -inf"
    print(f"[rules] {name}: attention err/bound {worst:.3f}", flush=True)


INDEXER_CASES = [
    ("stream_decode", dict(lens=[3000, 2600, 700, 4100, 64])),
    ("two_row_stream", dict(lens=[3000, 2600, 700], q_lens=[2, 2, 2])),
    ("prefill", dict(lens=[3000, 2600], q_lens=[40, 9])),
    ("f32", dict(lens=[900, 300, 77], idx_kind="f32", mla_kind="f32", page_size=16, topk=64)),
]


@pytest.mark.parametrize("name,kw", INDEXER_CASES, ids=[c[0] for c in INDEXER_CASES])
def test_indexer_absent_pages(name, kw):
    _need_gpu()
    from dsa_workloads.device import make_step
    seed = 720 + [c[0] for c in INDEXER_CASES].index(name)
    rng = np.random.default_rng(seed)
    kw = dict(kw)
    kw.setdefault("topk", 512)
    cfg = small_config(f"absent_{name}", seed=seed, **kw)
    wl = generate(cfg)
    bad = _break_pages(wl, rng)
    step = make_step(wl)
    print(f"\n[rules] indexer {name}: rows {wl.num_rows}, absent pages {bad}", flush=True)
    step.indexer()
    step.select()
    torch.cuda.synchronize()
    logits = step.logits.cpu().numpy()
    idx = step.topk_idx.cpu().numpy()
    rows = list(range(wl.num_rows))
    ref, worst = parity.check_logits(logits, wl, rows)
    vis = parity.visible_of(wl)
    n_neg = sum(int(np.isneginf(ref[t]).sum()) for t in rows)
    assert n_neg > 0, "the broken pages must hold visible positions"
    parity.check_topk_exact(idx, logits, vis, cfg.topk, rows)
    print(f"[rules] indexer {name}: -inf positions {n_neg}, logits err/bound {worst:.3f}", flush=True)


def test_indexer_logits_row_stride_beyond_the_stream_kernel():
    """A logits row stride of more than 2^29 floats (a 2 GiB row) takes the
    general fp8 kernel instead of the stream kernel, whose per-row store range
    must fit 32 bits; both give the same scores (same contraction, same
    summation order)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_mla_attention_dsa_amd as dsa
    wl = generate(small_config("wide_stride", seed=231, lens=[3000]), with_mla=False)
    dev = "cuda"
    bt = torch.from_numpy(wl.block_table).to(dev)
    lens = torch.from_numpy(wl.seq_lens_k).to(dev)
    batch = dsa.make_batch(bt, lens, page_size=wl.cfg.page_size, num_pages=wl.index_cache.shape[0],
                           max_seq_len_k=int(wl.seq_lens_k.max()))
    q = torch.from_numpy(wl.q_idx).to(dev).view(torch.float8_e4m3fn)
    w = torch.from_numpy(wl.w).to(dev)
    cache = torch.from_numpy(wl.index_cache).to(dev)
    n = int(wl.seq_lens_k[0])
    narrow = torch.empty((1, n), dtype=torch.float32, device=dev)
    dsa.dsa_indexer_logits(batch, q, w, cache, narrow)
    wide = torch.empty((1, (1 << 29) + 64), dtype=torch.float32, device=dev)
    print(f"\n[entry] logits row stride {wide.stride(0)} floats", flush=True)
    dsa.dsa_indexer_logits(batch, q, w, cache, wide)
    torch.cuda.synchronize()
    assert torch.equal(wide[0, :n], narrow[0]), "wide-stride scores differ"
    parity.check_logits(narrow.cpu().numpy(), wl, [0])
    del wide
    torch.cuda.empty_cache()


SCALE_CASES = [("bf16", 0.0), ("bf16", -0.06), ("bf16", 0.3), ("bf16", 1e-39), ("fp8", 0.0), ("fp8", -0.06), ("fp8", 0.3), ("fp8", 1e-39)]


@pytest.mark.parametrize("kind,scale", SCALE_CASES, ids=[f"{k}_{s}" for k, s in SCALE_CASES])
def test_attention_any_softmax_scale(kind, scale):
    """The attention takes any finite softmax scale: zero (uniform weights over
    the valid entries), negative (the smallest scores dominate), positive ones
    (the kernels take a separate path for positive normal scales, with the
    scale folded into the exponent) and a subnormal one (the general path), on
    decode and prefill rows whose last tiles are partial, against the oracle."""
    _need_gpu()
    from dsa_workloads.device import make_step
    seed = 740 + SCALE_CASES.index((kind, scale))
    rng = np.random.default_rng(seed)
    cfg = small_config(f"scale_{kind}_{scale}", seed=seed, topk=2048, lens=[3000, 2600, 700], q_lens=[2, 1, 3],
                       mla_kind=kind, softmax_scale=scale)
    wl = generate(cfg, with_indexer=False)
    vis = parity.visible_of(wl)
    k = cfg.topk
    idx = np.full((wl.num_rows, k), -1, dtype=np.int32)
    for t in range(wl.num_rows):
        n = min(int(vis[t]), k)
        idx[t, :n] = np.sort(rng.choice(int(vis[t]), size=n, replace=False))
    step = make_step(wl)
    print(f"\n[scale] {kind} softmax_scale={scale}: rows {wl.num_rows}, visible {vis}", flush=True)
    step.attend(topk_idx=torch.from_numpy(idx).cuda())
    torch.cuda.synchronize()
    out = step.out.float().cpu().numpy()
    lse = step.lse.cpu().numpy()
    worst = parity.check_attention(out, lse, wl, idx, list(range(wl.num_rows)))
    print(f"[scale] {kind} softmax_scale={scale}: attention err/bound {worst:.3f}", flush=True)
