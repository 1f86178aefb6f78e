"""GPU parity of the indexer's input side: dsa_quant_index_q and dsa_store_index_k.

Both produce integer codes and fp32 scales decided in fp32 on both sides, so
the comparison with the oracle (oracle/quant.py) is bit for bit: every code
byte, every scale and gate, and every byte of the paged cache the store
leaves (untouched slots included). The last test runs the indexer on what the
GPU produced and holds its scores to the oracle's on the same bytes.
"""
import types

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle.quant import quant_index_q, store_index_k  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bf16(x, device="cuda"):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(device)


def _bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def _q_with_edges(rng, T, H):
    q = rng.standard_normal((T, H, 128)) * np.exp2(rng.uniform(-10, 10, size=(T, H, 1)))
    rows = q.reshape(-1, 128)                           # a view: edits land in q
    if len(rows) >= 5:
        rows[0] = 0.0                                   # zero block: the scale floor
        rows[1] = -0.0
        rows[2] = 1e-6                                  # everything but one element subnormal in fp8
        rows[2, 5] = 3.0e4
        rows[3, :64] = 448.0                            # ties and exact grid values after scaling
        rows[3, 64:] = np.linspace(-448.0, 448.0, 64)
        rows[4] = np.exp2(np.arange(128) % 30 - 20.0) * np.where(np.arange(128) % 2, -1.0, 1.0)
    return q


@pytest.mark.parametrize("T,H", [(1, 64), (64, 64), (130, 3), (5, 1)])
def test_quant_index_q_bit_exact(T, H):
    _need_gpu()
    import sparse_mla_attention_dsa_amd as dsa
    rng = np.random.default_rng(400 + T + H)
    print(f"\n[quant q] T={T} H={H}", flush=True)
    q = _bf16(_q_with_edges(rng, T, H))
    w = torch.from_numpy((rng.standard_normal((T, H)) / 8.0).astype(np.float32)).cuda()
    q8 = torch.empty((T, H, 128), dtype=torch.uint8, device="cuda")
    w_eff = torch.empty((T, H), dtype=torch.float32, device="cuda")
    dsa.dsa_quant_index_q(q, w, q8, w_eff)
    torch.cuda.synchronize()
    codes, w_ref, _ = quant_index_q(_bits(q), w.cpu().numpy())
    got = q8.cpu().numpy()
    if not np.array_equal(got, codes):
        i = np.argwhere(got != codes)[0]
        raise AssertionError(f"code differs at {tuple(i)}: gpu {got[tuple(i)]:#x} oracle {codes[tuple(i)]:#x}")
    assert np.array_equal(w_eff.cpu().numpy().view(np.uint32), w_ref.view(np.uint32))


def test_quant_index_q_in_place_gates_and_non_finite_blocks():
    _need_gpu()
    import sparse_mla_attention_dsa_amd as dsa
    rng = np.random.default_rng(431)
    x = rng.standard_normal((2, 4, 128))
    x[0, 1, 7] = np.nan
    x[1, 2, 9] = np.inf
    q = _bf16(x)
    w = torch.from_numpy(rng.standard_normal((2, 4)).astype(np.float32)).cuda()
    w_in = w.cpu().numpy().copy()
    q8 = torch.empty((2, 4, 128), dtype=torch.uint8, device="cuda")
    dsa.dsa_quant_index_q(q, w, q8, w)                  # w_eff written over w
    torch.cuda.synchronize()
    codes, w_ref, _ = quant_index_q(_bits(q), w_in)
    got, w_got = q8.cpu().numpy(), w.cpu().numpy()
    finite = np.ones((2, 4), bool)
    finite[0, 1] = finite[1, 2] = False
    assert np.array_equal(got[finite], codes[finite])
    assert np.array_equal(w_got[finite].view(np.uint32), w_ref[finite].view(np.uint32))
    # NaN block: NaN scale, every code NaN (sign unspecified)
    assert np.isnan(w_got[0, 1]) and np.all((got[0, 1] & 0x7F) == 0x7F)
    # inf block: infinite scale, the inf element NaN, the finite ones zero of their sign
    assert np.isinf(w_got[1, 2])
    assert (got[1, 2, 9] & 0x7F) == 0x7F
    others = np.delete(np.arange(128), 9)
    assert np.array_equal(got[1, 2, others], codes[1, 2, others])


@pytest.mark.parametrize("P,pages,n", [(64, 9, 200), (16, 40, 333), (64, 2, 1)])
def test_store_index_k_bit_exact(P, pages, n):
    _need_gpu()
    import sparse_mla_attention_dsa_amd as dsa
    rng = np.random.default_rng(500 + P + n)
    print(f"\n[store k] P={P} pages={pages} n={n}", flush=True)
    cache_h = rng.integers(0, 256, size=(pages, 132 * P), dtype=np.uint8)
    n_slots = min(n, pages * P)
    slots = rng.choice(pages * P, size=n_slots, replace=False).astype(np.int64)
    if n_slots > 4:
        slots[1] = -1                                   # padding token
        slots[2] = pages * P + 3                        # past the pool
    key = _bf16(_q_with_edges(rng, n_slots, 1)[:, 0, :])
    cache = torch.from_numpy(cache_h).cuda()
    dsa.dsa_store_index_k(key, torch.from_numpy(slots).cuda(), cache, P)
    torch.cuda.synchronize()
    want = store_index_k(cache_h, _bits(key), slots, P)
    got = cache.cpu().numpy()
    if not np.array_equal(got, want):
        i = np.argwhere(got != want)[0]
        raise AssertionError(f"cache byte differs at {tuple(i)}: gpu {got[tuple(i)]} oracle {want[tuple(i)]}")


def test_gpu_inputs_feed_the_indexer():
    """dsa_store_index_k fills a paged cache token by token, dsa_quant_index_q
    prepares the queries, and dsa_indexer_logits scores them: the bytes equal
    the oracle's quantization and the scores pass the indexer parity rule."""
    _need_gpu()
    import sparse_mla_attention_dsa_amd as dsa
    rng = np.random.default_rng(611)
    P, H, lens = 64, 64, np.array([100, 700, 1500, 64], dtype=np.int32)
    B = len(lens)
    n_pages = [-(-int(n) // P) for n in lens]
    pool = rng.permutation(sum(n_pages) + 2)             # two pages stay unused
    bt = np.full((B, max(n_pages)), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(n_pages):
        bt[b, :n] = pool[off:off + n]
        off += n
    num_pages = len(pool)
    slots = np.concatenate([bt[b, np.arange(lens[b]) // P].astype(np.int64) * P + np.arange(lens[b]) % P
                            for b in range(B)])
    keys = _bf16(rng.standard_normal((len(slots), 128)))
    cache = torch.zeros((num_pages, 132 * P), dtype=torch.uint8, device="cuda")
    dsa.dsa_store_index_k(keys, torch.from_numpy(slots).cuda(), cache, P)
    q = _bf16(rng.standard_normal((B, H, 128)))
    w = torch.from_numpy((rng.standard_normal((B, H)) / 8.0).astype(np.float32)).cuda()
    q8 = torch.empty((B, H, 128), dtype=torch.uint8, device="cuda")
    w_eff = torch.empty((B, H), dtype=torch.float32, device="cuda")
    dsa.dsa_quant_index_q(q, w, q8, w_eff)
    torch.cuda.synchronize()
    cache_h = cache.cpu().numpy()
    assert np.array_equal(cache_h, store_index_k(np.zeros_like(cache_h), _bits(keys), slots, P))
    codes, w_ref, _ = quant_index_q(_bits(q), w.cpu().numpy())
    assert np.array_equal(q8.cpu().numpy(), codes)

    bt_d = torch.from_numpy(bt).cuda()
    sl_d = torch.from_numpy(lens).cuda()
    batch = dsa.make_batch(bt_d, sl_d, page_size=P, num_pages=num_pages, max_seq_len_k=int(lens.max()))
    logits = torch.empty((B, int(lens.max())), dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_logits(batch, q8, w_eff, cache, logits)
    torch.cuda.synchronize()
    wl = types.SimpleNamespace(q_idx=codes, w=w_ref, index_cache=cache_h, block_table=bt, seq_lens_k=lens,
                               cu_seqlens_q=None, cfg=types.SimpleNamespace(page_size=P, idx_kind="fp8"))
    _, worst = parity.check_logits(logits.cpu().numpy(), wl, list(range(B)))
    print(f"[quant e2e] logits err/bound {worst:.3f}", flush=True)
