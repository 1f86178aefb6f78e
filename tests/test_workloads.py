"""The seeded input generator (no GPU)."""
import numpy as np

from dsa_workloads import CONFIGS, generate, small_config


def test_ragged_batch_lengths_are_reproducible():
    cfg = CONFIGS["decode_b64_ragged"]
    rng = np.random.default_rng(cfg.seed)
    lens = rng.integers(4096, 32768, size=64, endpoint=True)
    assert (int(lens.sum()), int(lens.min()), int(lens.max())) == (1237475, 5236, 32564)


def test_generation_is_deterministic_and_canaried():
    cfg = small_config("det", seed=3, lens=[100, 64, 1], page_size=16)
    a = generate(cfg)
    b = generate(cfg)
    for name in ("block_table", "index_cache", "q_idx", "w", "latent", "q_mla"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    P = 16
    # every request's pages are distinct and unused slots point at the poison page
    used = [a.block_table[i, :(-(-int(n) // P))] for i, n in enumerate(a.seq_lens_k)]
    flat = np.concatenate(used)
    assert len(set(flat.tolist())) == len(flat)
    assert (a.block_table[1, 4:] == a.num_pages - 1).all()
    # slot 4 of request 0's last page (position 100) is a NaN canary in both caches
    page = a.block_table[0, 100 // P]
    assert (a.latent[page, 100 % P] == 0x7FC0).all()
    assert (a.index_cache[page, (100 % P) * 128:(100 % P + 1) * 128] == 0x7F).all()


def test_prefill_rows():
    cfg = small_config("pf", seed=4, lens=[300], q_lens=[40], page_size=64)
    wl = generate(cfg, with_mla=False)
    assert wl.num_rows == 40 and list(wl.cu_seqlens_q) == [0, 40]
    assert wl.max_seq_len_q == 40 and wl.max_seq_len_k == 300
