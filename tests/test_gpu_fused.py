"""GPU tests of dsa_indexer_topk: the indexer scores and their top-k in one
call, with no score matrix in memory.

Every case runs the fused call and the two-call path (dsa_indexer_logits, then
dsa_topk) on the same device inputs and requires the same lists, bit for bit,
on every row. The two-call path is itself pinned to the oracle on the same
rows: its logits under the logits rule, its selection bit-exact against
oracle.topk_row of those logits; and the fused lists are also checked end to
end against the oracle's own logits (the near-tie rule). Decode, multi-token
decode and prefill rows, ragged tails, several chunks per row, rows shorter
than k, forcing, absent pages, k from 1 to 4096 and rows long enough for the
merge to run from global memory are covered.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from dsa_workloads import CONFIGS, _to_e4m3fn_bytes, generate, small_config  # noqa: E402
import oracle  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


class _Inputs:
    """Device copies of the indexer inputs of a workload-like object."""

    def __init__(self, wl, k):
        import sparse_mla_attention_dsa_amd as dsa
        cu = wl.cu_seqlens_q
        self.T = int(wl.q_idx.shape[0])
        self.k = int(k)
        self.max_len = int(wl.seq_lens_k.max()) if len(wl.seq_lens_k) else 0
        max_q = 1 if cu is None else int(np.diff(cu).max())
        self.bt = torch.from_numpy(np.ascontiguousarray(wl.block_table)).cuda()
        self.lens = torch.from_numpy(np.ascontiguousarray(wl.seq_lens_k)).cuda()
        self.cu = None if cu is None else torch.from_numpy(np.ascontiguousarray(cu)).cuda()
        self.batch = dsa.make_batch(self.bt, self.lens, self.cu, page_size=wl.cfg.page_size,
                                    num_pages=int(wl.index_cache.shape[0]), max_seq_len_k=self.max_len,
                                    max_seq_len_q=max_q, num_rows=self.T)
        self.q = torch.from_numpy(wl.q_idx).cuda().view(torch.float8_e4m3fn)
        self.w = torch.from_numpy(wl.w).cuda()
        self.cache = torch.from_numpy(wl.index_cache).cuda()

    def two_call(self, n_init=0, n_local=0):
        import sparse_mla_attention_dsa_amd as dsa
        stride = max(1, (self.max_len + 3) // 4 * 4)
        logits = torch.empty((self.T, stride), dtype=torch.float32, device="cuda")
        idx = torch.empty((self.T, self.k), dtype=torch.int32, device="cuda")
        dsa.dsa_indexer_logits(self.batch, self.q, self.w, self.cache, logits, num_init_tokens=n_init,
                               num_local_tokens=n_local)
        nb = dsa.dsa_workspace_bytes(dsa.DSA_OP_TOPK, self.batch, self.k, 128, 512, dsa.DSA_BF16)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda") if nb else None
        dsa.dsa_topk(self.batch, logits, self.k, idx, ws)
        torch.cuda.synchronize()
        return logits.cpu().numpy(), idx.cpu().numpy()

    def fused(self, n_init=0, n_local=0, fill=None):
        import sparse_mla_attention_dsa_amd as dsa
        idx = torch.full((self.T, self.k), -7 if fill is None else fill, dtype=torch.int32, device="cuda")
        nb = dsa.dsa_workspace_bytes(dsa.DSA_OP_INDEXER_TOPK, self.batch, self.k, 128, 512, dsa.DSA_BF16)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        dsa.dsa_indexer_topk(self.batch, self.q, self.w, self.cache, self.k, idx, ws, num_init_tokens=n_init,
                             num_local_tokens=n_local)
        torch.cuda.synchronize()
        return idx.cpu().numpy()


def _check(wl, k, oracle_rows, n_init=0, n_local=0, label=""):
    """Fused == two-call on every row; both pinned to the oracle on `oracle_rows`."""
    _need_gpu()
    x = _Inputs(wl, k)
    print(f"\n[fused] {label}: T={x.T} max_len={x.max_len} k={k} init={n_init} local={n_local}", flush=True)
    logits, idx2 = x.two_call(n_init, n_local)
    idxf = x.fused(n_init, n_local)
    if not np.array_equal(idxf, idx2):
        bad = np.nonzero((idxf != idx2).any(axis=1))[0]
        t = int(bad[0])
        j = int(np.nonzero(idxf[t] != idx2[t])[0][0])
        raise AssertionError(f"{label}: fused lists differ from the two-call path on {len(bad)} rows; "
                             f"row {t} slot {j}: fused {idxf[t, j]} two-call {idx2[t, j]}")
    vis = parity.visible_of(wl)
    rows = sorted(set(int(r) for r in oracle_rows))
    ref = oracle.indexer_logits(wl.q_idx, wl.w, wl.index_cache, wl.block_table, wl.seq_lens_k,
                                wl.cu_seqlens_q, wl.cfg.page_size, "fp8", rows=rows, num_init=n_init,
                                num_local=n_local)
    if n_init == 0 and n_local == 0:
        parity.check_logits(logits, wl, rows, ref=ref)
    parity.check_topk_exact(idx2, logits, vis, k, rows)
    n_near = sum(parity.check_topk_near_ties(idxf[t], ref[t], vis[t], k) for t in rows)
    print(f"[fused] {label}: {x.T} rows identical; oracle rows {rows}, near-tie swaps {n_near}", flush=True)
    return idxf


SMALL = [
    small_config("dec3_p64", seed=201, lens=[100, 2100, 5000]),
    small_config("dec4_ragged_tail", seed=202, lens=[2049, 3333, 64, 4097, 8193, 12289]),
    small_config("dec2_p16_k256", seed=203, lens=[700, 1500], page_size=16, topk=256),
    small_config("dec_k1", seed=204, lens=[500, 33, 9000], topk=1),
    small_config("dec_k7_p32", seed=205, lens=[4100, 40], page_size=32, topk=7),
    small_config("dec_k4096", seed=206, lens=[5000, 4097, 20000, 100], topk=4096),
    small_config("dec_empty_rows", seed=207, lens=[0, 700, 0, 2500], topk=256),
    small_config("dec_k1024_chunks", seed=208, lens=[30000, 16384, 16385, 8191], topk=1024),
    small_config("pre2_p64", seed=209, lens=[300, 2500], q_lens=[37, 64]),
    small_config("pre2_k128", seed=210, lens=[400, 9000], q_lens=[50, 21], topk=128),
    small_config("pre1_k4096", seed=211, lens=[5000], q_lens=[40], topk=4096),
    small_config("pre3_p16_ragged", seed=212, lens=[900, 64, 3000], q_lens=[17, 1, 100], page_size=16,
                 topk=512),
    small_config("mtp_x2", seed=213, lens=[2049, 3000, 130, 5000], q_lens=[2, 2, 2, 2]),
    small_config("mtp_x4_p16", seed=214, lens=[700, 4100, 2047], q_lens=[4, 4, 4], page_size=16, topk=512),
    small_config("mtp_x3_short", seed=215, lens=[3, 2050, 64], q_lens=[3, 3, 3]),
]


@pytest.mark.parametrize("cfg", SMALL, ids=[c.name for c in SMALL])
def test_small_workloads(cfg):
    wl = generate(cfg, with_mla=False)
    _check(wl, cfg.topk, range(wl.q_idx.shape[0]), label=cfg.name)


@pytest.mark.parametrize("cfg,n_init,n_local", [
    (small_config("force_dec", seed=216, lens=[3000, 700, 2100, 5, 9000]), 4, 64),
    (small_config("force_pre", seed=217, lens=[2500, 300], q_lens=[40, 9]), 16, 3),
    (small_config("force_many", seed=218, lens=[2500, 10000], topk=128), 100, 100),
    (small_config("force_mtp", seed=219, lens=[5000, 2100], q_lens=[3, 3]), 1, 1),
], ids=["decode", "prefill", "more_than_k", "mtp"])
def test_init_and_local_forcing(cfg, n_init, n_local):
    wl = generate(cfg, with_mla=False)
    idx = _check(wl, cfg.topk, range(wl.q_idx.shape[0]), n_init=n_init, n_local=n_local, label=cfg.name)
    vis = parity.visible_of(wl)
    for t in range(wl.q_idx.shape[0]):
        n = vis[t]
        forced = sorted(set(range(min(n_init, n))) | set(range(max(n - n_local, 0), n)))
        chosen = set(int(v) for v in idx[t] if v >= 0)
        if len(forced) <= cfg.topk:
            assert set(forced) <= chosen, f"row {t}: a forced position was not selected"
        else:
            assert chosen == set(forced[:cfg.topk])


def _shared_pool(seed, lens, q_lens=None, pool=320, absent=False, k=2048):
    """Decode or prefill rows over one shared pool of fp8 index pages (so that
    long rows need little memory); with `absent`, one block-table entry in five
    names no page of the pool."""
    import types
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
    return types.SimpleNamespace(q_idx=q8, w=w, index_cache=cache, block_table=bt, seq_lens_k=lens,
                                 cu_seqlens_q=cu, cfg=types.SimpleNamespace(page_size=P, idx_kind="fp8"))


def test_absent_pages_decode():
    lens = np.random.default_rng(220).integers(1, 40000, size=48)
    wl = _shared_pool(220, lens, absent=True)
    _check(wl, 2048, (0, int(np.argmax(lens)), 47), label="absent pages, decode")


def test_absent_pages_prefill():
    wl = _shared_pool(221, [9000, 3000], q_lens=[30, 5], absent=True, k=512)
    _check(wl, 512, (0, 29, 30, 34), label="absent pages, prefill")


def test_merge_beyond_the_lds_cache():
    """Rows whose candidates outgrow the merge's 32,768-key LDS cache (200k
    keys at k = 2048: 25 chunks; 70k keys at k = 4096: 9 chunks), so the merge
    re-reads them from global memory."""
    wl = _shared_pool(222, [200000, 150000, 3000])
    _check(wl, 2048, (0, 1, 2), label="200k rows, k 2048")
    wl = _shared_pool(223, [70000, 65537])
    _check(wl, 4096, (0, 1), label="70k rows, k 4096")


def test_many_rows():
    """1,100 decode rows (one fused work-group per (row, chunk); short rows are
    the merge's alone)."""
    lens = np.random.default_rng(224).integers(1, 12000, size=1100)
    wl = _shared_pool(224, lens)
    _check(wl, 2048, (3, int(np.argmax(lens)), 1099), label="1100 rows")


@pytest.mark.parametrize("name,rows", [
    ("decode_b64_ragged", (0, 17, 63)),
    ("decode_b64_32k", (0, 63)),
    ("decode_b8_128k", (0, 5)),
    ("mtp_b64x4_ragged", (0, 1, 2, 3, 255)),
    ("decode_b1_8k", (0,)),
])
def test_full_size(name, rows):
    """The benchmark's decode workloads: every row equal to the two-call path,
    sampled rows against the oracle."""
    cfg = CONFIGS[name]
    wl = generate(cfg, with_mla=False)
    _check(wl, cfg.topk, rows, label=name)


def test_full_prefill():
    cfg = CONFIGS["prefill_4k_on_16k"]
    wl = generate(cfg, with_mla=False)
    _check(wl, cfg.topk, (0, 2047, 4095), label=cfg.name)


def test_two_calls_in_a_row_reuse_the_workspace():
    """A second call with a smaller batch over the same workspace gives its own
    lists (no state kept between calls)."""
    _need_gpu()
    import sparse_mla_attention_dsa_amd as dsa
    big = _Inputs(_shared_pool(225, [30000, 17000, 9000]), 2048)
    small = _Inputs(_shared_pool(226, [9000, 2500]), 2048)
    nb = dsa.dsa_workspace_bytes(dsa.DSA_OP_INDEXER_TOPK, big.batch, 2048, 128, 512, dsa.DSA_BF16)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = []
    for x in (big, small):
        idx = torch.empty((x.T, 2048), dtype=torch.int32, device="cuda")
        dsa.dsa_indexer_topk(x.batch, x.q, x.w, x.cache, 2048, idx, ws)
        torch.cuda.synchronize()
        out.append(idx.cpu().numpy())
        assert np.array_equal(out[-1], x.two_call()[1])


if __name__ == "__main__":
    sys.exit(pytest.main([__file__, "-v"]))
