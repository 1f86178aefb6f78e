"""GPU parity: the HIP library (through its C ABI) against the float64 oracle.

Small workloads are compared element by element; the full-size workloads are
compared on sampled rows the oracle computes one at a time, in the same launch
configuration the benchmark times.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from dsa_workloads import CONFIGS, generate, small_config  # noqa: E402
import oracle  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(cfg):
    _need_gpu()
    from dsa_workloads.device import make_step
    print(f"\n[parity] {cfg.name}: generating", flush=True)
    wl = generate(cfg)
    step = make_step(wl)
    print(f"[parity] {cfg.name}: running T={wl.num_rows} max_len={wl.max_seq_len_k}", flush=True)
    step.run()
    torch.cuda.synchronize()
    host = {
        "logits": step.logits.cpu().numpy(),
        "topk": step.topk_idx.cpu().numpy(),
        "out": step.out.float().cpu().numpy(),
        "lse": step.lse.cpu().numpy(),
    }
    return wl, step, host


def _full_check(cfg, rows=None):
    wl, step, h = _run(cfg)
    rows = list(range(wl.num_rows)) if rows is None else rows
    ref, worst_l = parity.check_logits(h["logits"], wl, rows)
    vis = parity.visible_of(wl)
    parity.check_topk_exact(h["topk"], h["logits"], vis, cfg.topk, rows)
    n_near = sum(parity.check_topk_near_ties(h["topk"][t], ref[t], vis[t], cfg.topk) for t in rows)
    worst_o = parity.check_attention(h["out"], h["lse"], wl, h["topk"], rows, fp32=cfg.mla_kind == "f32")
    print(f"[parity] {cfg.name}: rows {len(rows)} logits err/bound {worst_l:.3f} "
          f"near-tie swaps {n_near} attention err/bound {worst_o:.3f}", flush=True)
    return wl, step, h


SMALL = [
    CONFIGS["tiny"],
    small_config("dec3_p64", seed=101, lens=[100, 2100, 5000]),
    small_config("dec2_p16_k256", seed=102, lens=[700, 1500], page_size=16, topk=256),
    small_config("dec4_ragged_tail", seed=103, lens=[2049, 3333, 64, 4097]),
    small_config("pre2_p64", seed=104, lens=[300, 2500], q_lens=[37, 64]),
    small_config("pre2_k128", seed=105, lens=[400, 1000], q_lens=[50, 21], topk=128),
    small_config("pre1_k4096", seed=106, lens=[5000], q_lens=[40], topk=4096),
    small_config("pre3_p16_ragged", seed=109, lens=[900, 64, 3000], q_lens=[17, 1, 100], page_size=16,
                 topk=512),
    small_config("dec_f32", seed=107, lens=[90, 300], page_size=16, topk=64, idx_kind="f32", mla_kind="f32"),
    small_config("pre_f32", seed=108, lens=[120, 77], q_lens=[9, 13], page_size=16, topk=32,
                 idx_kind="f32", mla_kind="f32"),
    small_config("dec_k1", seed=109, lens=[500, 33], topk=1),
    small_config("dec_empty_row", seed=110, lens=[0, 700], page_size=64, topk=256),
    # multi-token decode (next_n rows per request, causal inside the request)
    small_config("mtp_x2", seed=111, lens=[2049, 3000, 130, 5000], q_lens=[2, 2, 2, 2]),
    small_config("mtp_x4_p16", seed=112, lens=[700, 4100, 2047], q_lens=[4, 4, 4], page_size=16,
                 topk=512),
    small_config("mtp_x3_short", seed=113, lens=[3, 2050, 64], q_lens=[3, 3, 3], topk=2048),
    # fp8 latent cache (per-tensor query and cache scales)
    small_config("dec3_fp8", seed=114, lens=[100, 2100, 5000], mla_kind="fp8"),
    small_config("pre2_fp8", seed=115, lens=[300, 2500], q_lens=[37, 64], mla_kind="fp8"),
    small_config("dec_fp8_k4096", seed=116, lens=[5000, 4097], topk=4096, mla_kind="fp8"),
    small_config("dec_fp8_empty_p16", seed=117, lens=[0, 700, 65], page_size=16, topk=256, mla_kind="fp8"),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_small_workloads_match_oracle(cfg):
    _full_check(cfg)


def test_full_single_decode_8k():
    _full_check(CONFIGS["decode_b1_8k"])


def test_full_ragged_batch64_sampled():
    """Logits and attention on sampled rows (the shortest and longest requests
    and the quartiles of the lengths); top-k bit-exact on the GPU's own logits
    for all 64 rows (the oracle's selection is cheap)."""
    cfg = CONFIGS["decode_b64_ragged"]
    wl = generate(cfg, with_mla=False)
    lens = wl.seq_lens_k
    order = np.argsort(lens, kind="stable")
    rows = sorted({int(order[0]), int(order[len(order) // 4]), int(order[len(order) // 2]),
                   int(order[3 * len(order) // 4]), int(order[-1]), 17})
    wl, _, h = _full_check(cfg, rows=rows)
    parity.check_topk_exact(h["topk"], h["logits"], parity.visible_of(wl), cfg.topk, range(wl.num_rows))


def test_full_all_32k_batch64_sampled():
    """The literal "ctx 32k" batch: 64 rows of 32,768 keys each."""
    cfg = CONFIGS["decode_b64_32k"]
    wl, _, h = _full_check(cfg, rows=[0, 31, 63])
    parity.check_topk_exact(h["topk"], h["logits"], parity.visible_of(wl), cfg.topk, range(wl.num_rows))


def test_full_multi_token_decode_x4_sampled():
    """next_n = 4 over the ragged batch: the four rows of the shortest and the
    longest request, and one more."""
    cfg = CONFIGS["mtp_b64x4_ragged"]
    wl = generate(cfg, with_mla=False)
    lens = wl.seq_lens_k
    b_min, b_max = int(np.argmin(lens)), int(np.argmax(lens))
    rows = sorted({*range(4 * b_min, 4 * b_min + 4), *range(4 * b_max, 4 * b_max + 4), 101})
    wl, _, h = _full_check(cfg, rows=rows)
    parity.check_topk_exact(h["topk"], h["logits"], parity.visible_of(wl), cfg.topk, range(wl.num_rows))


def test_full_long_context_128k_sampled():
    """Logits and attention on two of the eight 131,072-key rows; top-k (the
    two-phase selection) bit-exact on the GPU's own logits for all eight."""
    cfg = CONFIGS["decode_b8_128k"]
    wl, _, h = _full_check(cfg, rows=[0, 5])
    parity.check_topk_exact(h["topk"], h["logits"], parity.visible_of(wl), cfg.topk, range(wl.num_rows))


def test_full_multi_token_decode_sampled():
    cfg = CONFIGS["mtp_b64x2_ragged"]
    wl = generate(cfg, with_mla=False)
    lens = wl.seq_lens_k
    b_min, b_max = int(np.argmin(lens)), int(np.argmax(lens))
    rows = sorted({2 * b_min, 2 * b_min + 1, 2 * b_max, 2 * b_max + 1, 35})
    wl, _, h = _full_check(cfg, rows=rows)
    parity.check_topk_exact(h["topk"], h["logits"], parity.visible_of(wl), cfg.topk, range(wl.num_rows))


def test_full_ragged_batch64_fp8_cache_sampled():
    cfg = CONFIGS["decode_b64_ragged_fp8"]
    wl = generate(cfg, with_mla=False)
    lens = wl.seq_lens_k
    rows = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 40})
    wl, _, h = _full_check(cfg, rows=rows)
    parity.check_topk_exact(h["topk"], h["logits"], parity.visible_of(wl), cfg.topk, range(wl.num_rows))


def test_decode_batch32_four_splits_sampled():
    """32 decode rows: the attention plans four splits per row (the unrolled
    four-way merge), bf16 and fp8 latent caches."""
    lens = [int(x) for x in np.random.default_rng(118).integers(2049, 4000, size=32)]
    for kind, seed in (("bf16", 118), ("fp8", 119)):
        _full_check(small_config(f"dec32_{kind}", seed=seed, lens=lens, mla_kind=kind), rows=[0, 13, 31])


def test_full_prefill_sampled():
    """Logits and attention on sampled rows; top-k bit-exact on the GPU's own
    logits for all 4,096 rows (about 2 ms of CPU per row)."""
    cfg = CONFIGS["prefill_4k_on_16k"]
    wl, _, h = _full_check(cfg, rows=[0, 1, 2047, 4094, 4095])
    parity.check_topk_exact(h["topk"], h["logits"], parity.visible_of(wl), cfg.topk, range(wl.num_rows))


def _shared_pool_indexer(seed, lens, q_lens=None, pool=320, check_rows=(), absent=False):
    """The fp8 indexer on rows whose block tables name pages of one shared pool
    (as shared prefixes do), so that large batches need little memory; the
    listed rows (and the first, last and longest) against the oracle. With
    `absent`, one block-table entry in five names no page of the pool (-1 or
    an id at or past the pool size): those positions must score -inf."""
    _need_gpu()
    import types
    import sparse_mla_attention_dsa_amd as dsa
    from dsa_workloads import _to_e4m3fn_bytes
    rng = np.random.default_rng(seed)
    P, H, D = 64, 64, 128
    lens = np.asarray(lens, dtype=np.int32)
    B = len(lens)
    cu = None if q_lens is None else np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    T = B if cu is None else int(cu[-1])
    max_len = int(lens.max())
    bt = rng.integers(0, pool, size=(B, -(-max_len // P))).astype(np.int32)
    if absent:
        holes = rng.random(bt.shape) < 0.2
        bt[holes] = rng.choice(np.array([-1, pool, pool + 77], dtype=np.int32), size=int(holes.sum()))
    keys = rng.standard_normal((pool * P, D)).astype(np.float32)
    sig = (np.abs(keys).max(axis=1) / 448.0).astype(np.float32)
    codes = _to_e4m3fn_bytes(keys / sig[:, None])
    cache = np.concatenate([codes.reshape(pool, P * D), sig.reshape(pool, P).view(np.uint8).reshape(pool, 4 * P)],
                           axis=1)
    q8 = _to_e4m3fn_bytes(rng.standard_normal((T, H, D)).astype(np.float32))
    w = (rng.standard_normal((T, H)) / 8.0).astype(np.float32)
    print(f"\n[parity] shared-pool indexer: {B} requests, {T} rows, keys {int(lens.sum())}", flush=True)
    batch = dsa.make_batch(torch.from_numpy(bt).cuda(), torch.from_numpy(lens).cuda(),
                           None if cu is None else torch.from_numpy(cu).cuda(), page_size=P, num_pages=pool,
                           max_seq_len_k=max_len, max_seq_len_q=1 if q_lens is None else int(max(q_lens)),
                           num_rows=T)
    logits = torch.empty((T, max_len), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_logits(batch, torch.from_numpy(q8).cuda(), torch.from_numpy(w).cuda(),
                           torch.from_numpy(cache).cuda(), logits)
    torch.cuda.synchronize()
    wl = types.SimpleNamespace(q_idx=q8, w=w, index_cache=cache, block_table=bt, seq_lens_k=lens,
                               cu_seqlens_q=cu, cfg=types.SimpleNamespace(page_size=P, idx_kind="fp8"))
    longest = int(np.argmax(lens)) if cu is None else int(cu[int(np.argmax(lens)) + 1]) - 1
    rows = sorted({0, T - 1, longest, *check_rows})
    _, worst = parity.check_logits(logits.cpu().numpy(), wl, rows)
    print(f"[parity] shared-pool indexer: rows {rows} logits err/bound {worst:.3f}", flush=True)


def test_indexer_chunk_records_in_rounds():
    """1,024 decode rows of 15-20k keys: every work-group of the stream
    indexer owns more chunks than its LDS record table holds (1,024) and takes
    them in two rounds."""
    lens = np.random.default_rng(620).integers(15000, 20001, size=1024)
    _shared_pool_indexer(620, lens, check_rows=(1, 511, 1022))


def test_indexer_more_rows_than_stream_units():
    """1,100 decode rows (more than the stream kernel's 1,024 units): the
    general fp8 kernel, one work-group per (row, 512 keys)."""
    lens = np.random.default_rng(621).integers(1, 3001, size=1100)
    _shared_pool_indexer(621, lens, check_rows=(7, 1024, 1025))


def test_indexer_general_kernel_absent_pages():
    """The general fp8 kernel (1,100 decode rows) on block tables with absent pages."""
    lens = np.random.default_rng(623).integers(1, 3001, size=1100)
    _shared_pool_indexer(623, lens, check_rows=(3, 1024, 1099), absent=True)


def test_indexer_more_requests_than_prefill_blocks():
    """1,030 two-row requests (more than the two-row stream kernel's 512 and
    the prefill kernel's 1,024 requests): the general fp8 kernel with causal
    visible lengths per row."""
    rng = np.random.default_rng(622)
    lens = rng.integers(2, 2500, size=1030)
    _shared_pool_indexer(622, lens, q_lens=[2] * 1030, check_rows=(2, 3, 2057))


def test_empty_batch_launches_nothing():
    _need_gpu()
    import sparse_mla_attention_dsa_amd as dsa
    dev = "cuda"
    bt = torch.zeros((1, 1), dtype=torch.int32, device=dev)
    sl = torch.zeros((0,), dtype=torch.int32, device=dev)
    batch = dsa.make_batch(bt, sl, page_size=64, num_pages=1, max_seq_len_k=0, max_seq_len_q=1)
    logits = torch.empty((0, 1), dtype=torch.float32, device=dev)
    idx = torch.empty((0, 16), dtype=torch.int32, device=dev)
    dsa.dsa_topk(batch, logits, 16, idx)
    torch.cuda.synchronize()



@pytest.mark.parametrize("cfg,n_init,n_local", [
    (small_config("force_dec", seed=118, lens=[3000, 700, 2100, 5]), 4, 64),
    (small_config("force_pre", seed=119, lens=[2500, 300], q_lens=[40, 9]), 16, 3),
    (small_config("force_many", seed=120, lens=[2500], topk=128), 100, 100),
], ids=["decode", "prefill", "more_than_k"])
def test_init_and_local_forcing(cfg, n_init, n_local):
    """The forced positions come out of the indexer as +inf and are always
    selected; every other logit keeps the parity rule, and top-k is exact on
    the GPU's logits."""
    _need_gpu()
    from dsa_workloads.device import make_step
    wl = generate(cfg)
    step = make_step(wl)
    step.num_init_tokens, step.num_local_tokens = n_init, n_local
    print(f"\n[parity] {cfg.name}: forcing {n_init} init, {n_local} local", flush=True)
    step.run()
    torch.cuda.synchronize()
    logits = step.logits.cpu().numpy()
    idx = step.topk_idx.cpu().numpy()
    vis = parity.visible_of(wl)
    rows = list(range(wl.num_rows))
    ref = oracle.indexer_logits(wl.q_idx, wl.w, wl.index_cache, wl.block_table, wl.seq_lens_k,
                                wl.cu_seqlens_q, cfg.page_size, cfg.idx_kind, rows=rows,
                                num_init=n_init, num_local=n_local)
    plain = {t: np.where(np.isinf(ref[t]) & (ref[t] > 0), 0.0, ref[t]) for t in rows}
    for t in rows:
        n = vis[t]
        forced = np.isposinf(ref[t])
        assert np.array_equal(np.isposinf(logits[t][:n]), forced), f"row {t}: forced positions differ"
        got = logits[t][:n].copy()
        got[forced] = 0.0
        parity.check_logits({t: got}, wl, [t], ref={t: plain[t]})
    parity.check_topk_exact(idx, logits, vis, cfg.topk, rows)
    for t in rows:
        forced = set(np.nonzero(np.isposinf(ref[t]))[0].tolist())
        chosen = set(int(x) for x in idx[t] if x >= 0)
        if len(forced) <= cfg.topk:
            assert forced <= chosen, f"row {t}: a forced position was not selected"
        else:
            assert chosen == set(sorted(forced)[:cfg.topk])


if __name__ == "__main__":
    sys.exit(pytest.main([__file__, "-v"]))
