"""Seeded synthetic inputs for the DSA step, shared by the tests, the smoke
check and the benchmark.

This module only draws random numbers and packs them into the byte layouts
the library and the oracle both read. It holds none of the step's arithmetic
(no scores, no selection, no attention). The one transformation it applies is
the input convention of the indexer: the SGLang indexer page quantizes the
index query per 128-wide row with `act_quant(..., block_size=128)` and folds
the resulting scale into the head weights (`_get_logits_head_gate`), and
stores each index key as fp8 plus one fp32 scale (`_store_index_k_cache`).
Those quantizations happen before the step and are done here on the CPU with
torch's float8_e4m3fn conversion so that both sides consume identical bytes.

Random streams (numpy PCG64), fixed so the bytes are reproducible:
* `default_rng(seed)`: 1. context lengths (only for configs with a length
  range); 2. the page permutation of the pool (unused block-table slots point
  at one extra poison page filled with NaN);
* every large array is drawn in float32 from its own streams
  `default_rng([seed, array_id, chunk])`, one per chunk of the leading
  dimension, so chunks can be filled in parallel and the bytes do not depend
  on the number of threads: 3. index keys [pages, P, D] (array 1);
  4. index queries [T, H, D] (2); 5. head weights [T, H] / sqrt(H) (3);
  6. latent cache [pages, P, Dl + Dr] (4); 7. MLA queries [T, Hm, Dl + Dr] (5).
Slots past a request's length inside its last page are NaN canaries.
"""

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
import math
import os

import numpy as np

F8_MAX = 448.0
NAN_F8 = 0x7F
NAN_BF16 = 0x7FC0


@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    batch: int
    ctx: tuple = ()                 # fixed key lengths per request (decode) or ()
    ctx_range: tuple = ()           # (lo, hi) inclusive uniform lengths when ctx == ()
    q_lens: tuple = ()              # rows per request; () = decode (one row each)
    page_size: int = 64
    idx_heads: int = 64
    idx_dim: int = 128
    idx_kind: str = "fp8"           # "fp8" (quantized) or "f32"
    topk: int = 2048
    mla_heads: int = 128
    d_latent: int = 512
    d_rope: int = 64
    mla_kind: str = "bf16"          # "bf16" or "f32"
    softmax_scale: float = 1.0 / math.sqrt(192.0)
    note: str = ""

    @property
    def is_prefill(self):
        return len(self.q_lens) > 0


# The five workloads the step is specified on, the literal "ctx 32k" variant
# of the ragged decode batch, and multi-token decode (speculative verification:
# next_n query rows per request, row i of a request seeing len - next_n + i + 1
# keys) over the ragged batch's lengths, pages and keys (same seed).
CONFIGS = {
    "tiny": Config("tiny", seed=0, batch=1, ctx=(256,), page_size=16, idx_heads=4,
                   idx_dim=32, idx_kind="f32", topk=64, mla_heads=8, d_latent=64,
                   d_rope=16, mla_kind="f32", softmax_scale=1.0 / math.sqrt(80.0),
                   note="batch 1 decode, ctx 256, fp32, 4x32 indexer, 8-head 80-d MLA"),
    "decode_b1_8k": Config("decode_b1_8k", seed=1, batch=1, ctx=(8192,),
                           note="DeepSeek-V3.2-shaped single decode, ctx 8192"),
    "decode_b64_ragged": Config("decode_b64_ragged", seed=2, batch=64, ctx_range=(4096, 32768),
                                note="ragged batch-64 decode, ctx U[4096, 32768]"),
    "decode_b8_128k": Config("decode_b8_128k", seed=3, batch=8, ctx=(131072,) * 8,
                             note="batch-8 decode, ctx 131072"),
    "prefill_4k_on_16k": Config("prefill_4k_on_16k", seed=4, batch=1, ctx=(20480,), q_lens=(4096,),
                                note="chunked prefill: 4096 rows on a 16384 prefix"),
    "decode_b64_32k": Config("decode_b64_32k", seed=5, batch=64, ctx=(32768,) * 64,
                             note="batch-64 decode, every ctx 32768"),
    "decode_b64_ragged_fp8": Config("decode_b64_ragged_fp8", seed=2, batch=64, ctx_range=(4096, 32768),
                                    mla_kind="fp8",
                                    note="ragged batch-64 decode over an fp8 latent cache (per-tensor scales)"),
    "mtp_b64x2_ragged": Config("mtp_b64x2_ragged", seed=2, batch=64, ctx_range=(4096, 32768),
                               q_lens=(2,) * 64,
                               note="multi-token decode, next_n 2, ragged batch 64, ctx U[4096, 32768]"),
    "mtp_b64x4_ragged": Config("mtp_b64x4_ragged", seed=2, batch=64, ctx_range=(4096, 32768),
                               q_lens=(4,) * 64,
                               note="multi-token decode, next_n 4, ragged batch 64, ctx U[4096, 32768]"),
}


@dataclass
class Workload:
    cfg: Config
    seq_lens_k: np.ndarray          # int32 [B]
    cu_seqlens_q: object            # int32 [B+1] or None (decode)
    block_table: np.ndarray         # int32 [B, max_pages]
    num_pages: int                  # pages in the pool, poison page included
    index_cache: np.ndarray         # uint8 [num_pages, page_bytes]
    q_idx: np.ndarray               # uint8 fp8 codes or float32 [T, H, D]
    w: np.ndarray                   # float32 [T, H] (q scale folded in)
    latent: np.ndarray              # uint16 bf16 bits or float32 [num_pages, P, Dqk]
    q_mla: np.ndarray               # uint16 bf16 bits or float32 [T, Hm, Dqk]
    extras: dict = field(default_factory=dict)

    @property
    def num_rows(self):
        return self.q_idx.shape[0]

    @property
    def max_seq_len_k(self):
        return int(self.seq_lens_k.max()) if len(self.seq_lens_k) else 0

    @property
    def max_seq_len_q(self):
        if self.cu_seqlens_q is None:
            return 1
        return int(np.diff(self.cu_seqlens_q).max()) if len(self.seq_lens_k) else 0


def _to_bf16_bits(x32):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bf16_bits_to_f32(bits):
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _to_e4m3fn_bytes(x32):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _per_tensor_e4m3(bits16, rows=4096):
    """E4M3 codes of a bf16 array with one fp32 scale (absmax / 448) for all of it."""
    flat = bits16.reshape(bits16.shape[0], -1)
    starts = list(range(0, flat.shape[0], rows))
    with ThreadPoolExecutor(_THREADS) as ex:
        amax = max(ex.map(lambda s: float(np.abs(_bf16_bits_to_f32(flat[s:s + rows])).max()), starts))
    scale = np.float32(max(amax, 1e-30) / F8_MAX)
    codes = np.empty(flat.shape, dtype=np.uint8)

    def work(s):
        codes[s:s + rows] = _to_e4m3fn_bytes(_bf16_bits_to_f32(flat[s:s + rows]) / scale)

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(work, starts))
    return codes.reshape(bits16.shape), float(scale)


def _fill(shape, seed, array_id, chunk_rows, dtype, convert=lambda x: x):
    """Standard normal float32 values of `shape`, chunk i of the leading dim
    drawn from default_rng([seed, array_id, i]) and passed through `convert`."""
    out = np.empty(shape, dtype=dtype)
    starts = list(range(0, shape[0], chunk_rows))

    def work(i):
        s = starts[i]
        e = min(shape[0], s + chunk_rows)
        g = np.random.default_rng([seed, array_id, i])
        out[s:e] = convert(g.standard_normal((e - s,) + tuple(shape[1:]), dtype=np.float32))

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(work, range(len(starts))))
    return out


def generate(cfg, with_mla=True, with_indexer=True):
    """Build the seeded inputs of `cfg` (a Config or a CONFIGS key)."""
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    rng = np.random.default_rng(cfg.seed)
    B, P = cfg.batch, cfg.page_size

    # 1. context lengths
    if cfg.ctx:
        lens = np.asarray(cfg.ctx, dtype=np.int64)
    else:
        lo, hi = cfg.ctx_range
        lens = rng.integers(lo, hi, size=B, endpoint=True)
    assert len(lens) == B
    if cfg.is_prefill:
        q_lens = np.asarray(cfg.q_lens, dtype=np.int64)
        cu = np.zeros(B + 1, dtype=np.int32)
        cu[1:] = np.cumsum(q_lens)
        T = int(cu[-1])
    else:
        cu = None
        T = B

    # 2. pages
    n_pages = [max(1, -(-int(n) // P)) for n in lens]
    total = int(sum(n_pages))
    poison = total
    pool = rng.permutation(total)
    max_pages = max(n_pages)
    block_table = np.full((B, max_pages), poison, dtype=np.int32)
    off = 0
    for b, n in enumerate(n_pages):
        block_table[b, :n] = pool[off:off + n]
        off += n
    num_pages = total + 1
    # slots that hold no token: the tail of each request's last page, and the
    # whole poison page -> (page, first dead slot)
    dead = [(poison, 0)]
    for b in range(B):
        used = int(lens[b]) - (n_pages[b] - 1) * P
        if used < P:
            dead.append((int(block_table[b, n_pages[b] - 1]), max(0, used)))

    def poison_slots(arr, value):
        for page, first in dead:
            arr[page, first:] = value

    H, D = cfg.idx_heads, cfg.idx_dim
    # 3. index keys (+ per-token scale)
    if with_indexer:
        keys = _fill((num_pages, P, D), cfg.seed, 1, 256, np.float32)
        if cfg.idx_kind == "fp8":
            page_bytes = P * D + 4 * P
            cache = np.empty((num_pages, page_bytes), dtype=np.uint8)
            codes = cache[:, :P * D]
            sig_all = cache[:, P * D:].view(np.float32)
            bounds = list(range(0, num_pages, 1024))

            def quant(s):
                e = min(num_pages, s + 1024)
                amax = np.abs(keys[s:e]).max(axis=2)
                sig = (np.maximum(amax, np.float32(1e-30)) / np.float32(F8_MAX)).astype(np.float32)
                sig_all[s:e] = sig
                codes[s:e] = _to_e4m3fn_bytes(keys[s:e] / sig[:, :, None]).reshape(e - s, P * D)

            with ThreadPoolExecutor(_THREADS) as ex:
                list(ex.map(quant, bounds))
            # canaries: NaN keys and scales in dead slots and in the poison page
            for page, first in dead:
                cache[page, first * D:P * D] = NAN_F8
                sig_all[page, first:] = np.nan
        else:
            page_bytes = 4 * P * D + 4 * P
            cache = np.empty((num_pages, page_bytes), dtype=np.uint8)
            poison_slots(keys, np.nan)
            sf = np.ones((num_pages, P), dtype=np.float32)
            poison_slots(sf, np.nan)
            cache[:, :4 * P * D] = keys.reshape(num_pages, -1).view(np.uint8)
            cache[:, 4 * P * D:] = sf.view(np.uint8)
        del keys

        # 4. index queries, 5. head weights
        qn = _fill((T, H, D), cfg.seed, 2, 1024, np.float32)
        wn = (_fill((T, H), cfg.seed, 3, 1 << 30, np.float32) / np.float32(math.sqrt(H))).astype(np.float32)
        if cfg.idx_kind == "fp8":
            qb = _bf16_bits_to_f32(_to_bf16_bits(qn))           # q is bf16 before quantization
            amax = np.abs(qb).max(axis=2)
            s_q = (np.maximum(amax, np.float32(1e-30)) / np.float32(F8_MAX)).astype(np.float32)
            q_idx = np.empty((T, H, D), dtype=np.uint8)
            for s in range(0, T, 1024):
                e = min(T, s + 1024)
                q_idx[s:e] = _to_e4m3fn_bytes(qb[s:e] / s_q[s:e, :, None])
            w = (wn * s_q).astype(np.float32)                   # fold the q scale into the gate
        else:
            q_idx = qn.astype(np.float32)
            w = wn
        del qn
    else:
        cache = np.zeros((num_pages, 0), dtype=np.uint8)
        q_idx = np.zeros((T, H, D), dtype=np.uint8 if cfg.idx_kind == "fp8" else np.float32)
        w = np.zeros((T, H), dtype=np.float32)

    # 6. latent cache, 7. MLA queries
    Dqk = cfg.d_latent + cfg.d_rope
    Hm = cfg.mla_heads
    extras = {}
    if with_mla:
        if cfg.mla_kind == "bf16":
            latent = _fill((num_pages, P, Dqk), cfg.seed, 4, 128, np.uint16, _to_bf16_bits)
            poison_slots(latent, NAN_BF16)
            q_mla = _fill((T, Hm, Dqk), cfg.seed, 5, 64, np.uint16, _to_bf16_bits)
        elif cfg.mla_kind == "fp8":
            # the bf16 rows and queries of the bf16 workload, quantized with
            # one scale per tensor (absmax / 448 over the live rows)
            lat16 = _fill((num_pages, P, Dqk), cfg.seed, 4, 128, np.uint16, _to_bf16_bits)
            poison_slots(lat16, 0)
            q16 = _fill((T, Hm, Dqk), cfg.seed, 5, 64, np.uint16, _to_bf16_bits)
            latent, kv_scale = _per_tensor_e4m3(lat16)
            q_mla, q_scale = _per_tensor_e4m3(q16)
            del lat16, q16
            poison_slots(latent, NAN_F8)
            extras = {"q_scale": q_scale, "kv_scale": kv_scale}
        else:
            latent = _fill((num_pages, P, Dqk), cfg.seed, 4, 128, np.float32)
            poison_slots(latent, np.nan)
            q_mla = _fill((T, Hm, Dqk), cfg.seed, 5, 64, np.float32)
    else:
        latent = np.zeros((num_pages, P, 0), dtype=np.uint16)
        q_mla = np.zeros((T, Hm, 0), dtype=np.uint16)

    return Workload(cfg=cfg, seq_lens_k=lens.astype(np.int32), cu_seqlens_q=cu,
                    block_table=block_table, num_pages=num_pages, index_cache=cache,
                    q_idx=q_idx, w=w, latent=latent, q_mla=q_mla, extras=extras)


def small_config(name, seed, lens, q_lens=(), page_size=64, topk=2048, idx_kind="fp8",
                 mla_kind="bf16", **kw):
    """A reduced workload with the DeepSeek shapes (or fp32 shapes) and the
    given lengths, for parity tests the oracle finishes in seconds."""
    if idx_kind == "f32":
        kw.setdefault("idx_heads", 4)
        kw.setdefault("idx_dim", 32)
    if mla_kind == "f32":
        kw.setdefault("mla_heads", 8)
        kw.setdefault("d_latent", 64)
        kw.setdefault("d_rope", 16)
        kw.setdefault("softmax_scale", 1.0 / math.sqrt(80.0))
    return Config(name, seed=seed, batch=len(lens), ctx=tuple(int(x) for x in lens),
                  q_lens=tuple(int(x) for x in q_lens), page_size=page_size, topk=topk,
                  idx_kind=idx_kind, mla_kind=mla_kind, **kw)
