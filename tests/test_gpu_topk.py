"""GPU top-k against the oracle on crafted logits, bit for bit.

dsa_topk is called directly (no indexer) on rows whose lengths cover the
short-row rule (visible <= k), rows cached in LDS, rows cut into chunks for
the two-phase selection of few-row batches, and rows longer than the LDS key
cache. Values come from a small set with +0 and -0 mixed in, so the k-th value
is shared by many positions and the lower-position rule decides the set.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from tests import parity  # noqa: E402

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _run(lengths, k, values, seed):
    _need_gpu()
    import sparse_mla_attention_dsa_amd as dsa
    rng = np.random.default_rng(seed)
    B = len(lengths)
    maxlen = max(lengths)
    stride = (maxlen + 3) // 4 * 4
    page = 64
    logits = np.full((B, stride), np.nan, dtype=np.float32)   # columns past a row's length are never read
    for t, n in enumerate(lengths):
        logits[t, :n] = values(rng, n)
    dev = "cuda"
    lg = torch.from_numpy(logits).to(dev)
    bt = torch.zeros((B, (maxlen + page - 1) // page), dtype=torch.int32, device=dev)
    sl = torch.tensor(lengths, dtype=torch.int32, device=dev)
    batch = dsa.make_batch(bt, sl, page_size=page, num_pages=1, max_seq_len_k=maxlen, max_seq_len_q=1)
    nbytes = dsa.dsa_workspace_bytes(dsa.DSA_OP_TOPK, batch, k, 0, 0, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None
    idx = torch.full((B, k), -7, dtype=torch.int32, device=dev)
    print(f"\n[topk] B={B} k={k} max_len={maxlen} workspace={nbytes}", flush=True)
    dsa.dsa_topk(batch, lg, k, idx, ws)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    parity.check_topk_exact(got, logits.astype(np.float64), list(lengths), k, range(B))
    return nbytes


def _ties(rng, n):
    v = rng.integers(-3, 4, size=n).astype(np.float32) * np.float32(0.5)
    zeros = rng.random(n) < 0.2
    v[zeros] = np.where(rng.random(int(zeros.sum())) < 0.5, np.float32(0.0), np.float32(-0.0))
    return v


def _normal(rng, n):
    return rng.standard_normal(n).astype(np.float32)


MIXED = [100, 2048, 2049, 8191, 8192, 12288, 20000, 32768, 40000, 131072]


@pytest.mark.parametrize("values", [_ties, _normal], ids=["ties", "normal"])
def test_two_phase_rows_match_oracle(values):
    nbytes = _run(MIXED, 2048, values, seed=11)
    assert nbytes > 0                       # a few long rows: chunks, then their candidates


def test_two_phase_k4096():
    assert _run([5000, 30000, 70000, 4096, 4097], 4096, _ties, seed=12) > 0


@pytest.mark.parametrize("k", [1, 7])
def test_small_odd_k(k):
    _run([1, 5, 9000, 20000, 50000], k, _ties, seed=13 + k)


def test_many_rows_single_phase():
    rng = np.random.default_rng(17)
    lengths = [int(x) for x in rng.integers(1, 6000, size=300)]
    assert _run(lengths, 512, _ties, seed=18) == 0   # enough rows: one work-group per row


def test_many_long_rows_uncached():
    """300 tie-heavy rows of 33k-70k positions: enough rows for one work-group
    per row, and too long for the LDS key cache, so every pass re-reads the
    row (the uncached selection and its variable-length output runs)."""
    rng = np.random.default_rng(19)
    lengths = [int(x) for x in rng.integers(33000, 70001, size=300)]
    assert _run(lengths, 2048, _ties, seed=20) == 0


def test_merge_of_more_candidates_than_the_cache():
    """k = 3000 over 340k positions: eleven 32,768-position chunks give 33,000
    candidates, more than the merge's LDS key cache, so the merge selection
    runs uncached."""
    assert _run([340000, 100000, 5000], 3000, _ties, seed=21) > 0


# Whole-row selections of rows up to 32,768 long (held in LDS), on value
# distributions that stress the digit passes: ties on every fourth position,
# values spread over 80 binary orders of magnitude with infinities, constant
# rows, and every k regime (short rows, the rank path of the last digit, the
# last-digit histogram).
REG_LENGTHS = [1, 2047, 2048, 2049, 4096, 8192, 8193, 9000, 16384, 20000, 24576, 32767, 32768]


@pytest.mark.parametrize("values", [_ties, _normal], ids=["ties", "normal"])
def test_whole_rows_in_lds(values):
    assert _run(REG_LENGTHS, 2048, values, seed=31) == 0


@pytest.mark.parametrize("k", [1, 7, 256, 4096])
def test_whole_rows_in_lds_k(k):
    _run([3, 5000, 16385, 20000, 32768], k, _normal, seed=32 + k)


def _low_every_fourth(rng, n):
    """Positions 0 mod 4 far below the rest."""
    v = rng.standard_normal(n).astype(np.float32)
    s = np.arange(n) % 4 == 0
    v[s] = np.float32(-100.0) + rng.standard_normal(int(s.sum())).astype(np.float32)
    return v


def _high_every_fourth(rng, n):
    """Positions 0 mod 4 equal and far above the rest: the k winners are the
    first k of their ties."""
    v = rng.standard_normal(n).astype(np.float32)
    v[np.arange(n) % 4 == 0] = np.float32(100.0)
    return v


def _shifted_every_fourth(rng, n):
    """Positions 0 mod 4 a quarter of a standard deviation above the rest."""
    v = rng.standard_normal(n).astype(np.float32)
    s = np.arange(n) % 4 == 0
    v[s] += np.float32(0.25)
    return v


def _wide_exponents(rng, n):
    """Magnitudes 2^U, U uniform in [-40, 40], random signs, some infinities:
    the keys spread over many first-digit bins."""
    v = (np.exp2(rng.uniform(-40, 40, size=n)) * np.where(rng.random(n) < 0.5, -1, 1)).astype(np.float32)
    v[rng.random(n) < 0.01] = np.float32(np.inf)
    v[rng.random(n) < 0.01] = np.float32(-np.inf)
    return v


def _constant(rng, n):
    return np.full(n, np.float32(0.25))


@pytest.mark.parametrize("values", [_low_every_fourth, _high_every_fourth, _shifted_every_fourth, _wide_exponents, _constant],
                         ids=["low-every-fourth", "high-every-fourth", "shifted-every-fourth", "wide-exponents", "constant"])
def test_whole_rows_skewed_values(values):
    assert _run([16384, 24576, 32768, 20000, 9000, 8193], 2048, values, seed=41) == 0


@pytest.mark.parametrize("values", [_low_every_fourth, _normal], ids=["low-every-fourth", "normal"])
def test_chunks_and_merge_skewed_values(values):
    """Few long rows: the 16,384-position chunks and the merge of their
    candidates on the same value patterns."""
    assert _run([131072, 70000, 40000], 2048, values, seed=43) > 0
