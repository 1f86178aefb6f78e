"""The C ABI on the host: the library loads, exports every symbol declared in
include/dsa.h, and rejects invalid arguments before touching a device.
None of these calls launches a kernel (no GPU needed)."""
import ctypes
import os
import re
import subprocess

import pytest

import sparse_mla_attention_dsa_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dsa.library_path()):
        from sparse_mla_attention_dsa_amd.build import build
        build()
    return dsa.lib()


def _declared():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(\w+)\s*\([^;]*\)\s*;", text)) - {"if", "while"})


def test_every_declared_symbol_is_exported(L):
    declared = _declared()
    assert set(declared) == set(dsa.EXPORTED_SYMBOLS), declared
    out = subprocess.run(["nm", "-D", "--defined-only", dsa.library_path()], capture_output=True, text=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in declared:
        assert name in exported, name
        assert hasattr(L, name)


def test_version_and_status_strings(L):
    assert re.fullmatch(r"\d+\.\d+\.\d+", dsa.dsa_version())
    for st in range(5):
        assert L.dsa_status_string(st)
    assert L.dsa_status_string(99) == b"unknown status"


class FakeTensor:
    """A host-side stand-in with a data_ptr and strides; never dereferenced."""

    def __init__(self, shape, dtype=None, ptr=0x1000):
        self.shape = shape
        self.dtype = dtype
        self._ptr = ptr

    def data_ptr(self):
        return self._ptr

    def stride(self, i):
        s = 1
        for d in self.shape[i + 1:]:
            s *= d
        return s


def _batch(**kw):
    args = dict(num_seqs=1, num_rows=1, page_size=64, max_pages_per_seq=4, num_pages=8,
                max_seq_len_k=256, max_seq_len_q=1, block_table=0x2000, seq_lens_k=0x3000,
                cu_seqlens_q=None)
    args.update(kw)
    return dsa.DsaBatch(**args)


def _idx(L, batch, k=2048, stride=256):
    return L.dsa_topk(ctypes.byref(batch), ctypes.c_void_p(0x4000), stride, k,
                      ctypes.c_void_p(0x5000), None, 0, None)


@pytest.mark.parametrize("field,value", [
    ("page_size", 0), ("page_size", 24), ("page_size", -16), ("max_pages_per_seq", 0),
    ("num_pages", 0), ("num_seqs", -1), ("num_rows", 2), ("max_seq_len_k", -5),
    ("block_table", None), ("seq_lens_k", None), ("max_seq_len_q", 3),
])
def test_topk_rejects_bad_batches(L, field, value):
    assert _idx(L, _batch(**{field: value})) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert L.dsa_last_error()


@pytest.mark.parametrize("k", [0, -1, 4097])
def test_topk_rejects_bad_k(L, k):
    assert _idx(L, _batch(), k=k) == dsa.DSA_ERR_INVALID_ARGUMENT


def test_contexts_beyond_2_pow_24_are_unsupported(L):
    assert _idx(L, _batch(max_seq_len_k=(1 << 24) + 1)) == dsa.DSA_ERR_UNSUPPORTED
    assert _logits(L, _batch(max_seq_len_k=(1 << 24) + 1), stride=(1 << 24) + 1) == dsa.DSA_ERR_UNSUPPORTED


def test_null_batch(L):
    assert L.dsa_topk(None, None, 1, 1, None, None, 0, None) == dsa.DSA_ERR_INVALID_ARGUMENT


def test_huge_pool_is_unsupported(L):
    assert _idx(L, _batch(num_pages=2 ** 30)) == dsa.DSA_ERR_UNSUPPORTED


def test_empty_batch_is_ok_without_launch(L):
    b = _batch(num_seqs=0, num_rows=0, block_table=None, seq_lens_k=None)
    assert _idx(L, b) == dsa.DSA_OK


def _logits(L, batch, qd=dsa.DSA_FP8_E4M3, kd=dsa.DSA_FP8_E4M3, H=64, D=128, stride=256, nullq=False,
            n_init=0, n_local=0):
    return L.dsa_indexer_logits(ctypes.byref(batch), None if nullq else ctypes.c_void_p(0x100), qd,
                                ctypes.c_void_p(0x200), ctypes.c_void_p(0x300), kd, H, D,
                                ctypes.c_void_p(0x400), stride, n_init, n_local, None)


def test_indexer_validation(L):
    b = _batch()
    assert _logits(L, b, H=32) == dsa.DSA_ERR_UNSUPPORTED
    assert _logits(L, b, D=64) == dsa.DSA_ERR_UNSUPPORTED
    assert _logits(L, b, kd=dsa.DSA_F32) == dsa.DSA_ERR_UNSUPPORTED
    assert _logits(L, b, qd=dsa.DSA_BF16, kd=dsa.DSA_BF16) == dsa.DSA_ERR_UNSUPPORTED
    assert _logits(L, b, qd=dsa.DSA_F32, kd=dsa.DSA_F32, H=65, D=8) == dsa.DSA_ERR_UNSUPPORTED
    assert _logits(L, b, stride=255) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert _logits(L, b, nullq=True) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert _logits(L, b, H=0) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert _logits(L, _batch(num_rows=0, num_seqs=0)) == dsa.DSA_OK
    assert _logits(L, b, n_init=-1) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert _logits(L, b, n_local=-2) == dsa.DSA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("which", ["q", "w", "cache"])
def test_fp8_indexer_rejects_misaligned_pointers(L, which):
    ptr = {"q": 0x100, "w": 0x200, "cache": 0x300}
    ptr[which] += 4
    V = ctypes.c_void_p
    st = L.dsa_indexer_logits(ctypes.byref(_batch()), V(ptr["q"]), dsa.DSA_FP8_E4M3, V(ptr["w"]), V(ptr["cache"]),
                              dsa.DSA_FP8_E4M3, 64, 128, V(0x400), 256, 0, 0, None)
    assert st == dsa.DSA_ERR_INVALID_ARGUMENT


def _mla(L, batch, decode=True, dtype=dsa.DSA_BF16, H=128, Dl=512, Dr=64, k=2048, ws=None, wsb=0,
         scale=0.07, nullout=False):
    fn = L.sparse_mla_decode if decode else L.sparse_mla_prefill
    return fn(ctypes.byref(batch), ctypes.c_void_p(0x10), ctypes.c_void_p(0x20), dtype,
              ctypes.c_void_p(0x30), k, H, Dl, Dr, scale, None if nullout else ctypes.c_void_p(0x40),
              None, ws, wsb, None)


def test_mla_validation(L):
    dec = _batch(num_seqs=64, num_rows=64)
    need = L.dsa_workspace_bytes(dsa.DSA_OP_MLA_DECODE, ctypes.byref(dec), 2048, 128, 512, dsa.DSA_BF16)
    # split-KV partials for a 64-row decode: 2 splits x 128 heads per row, a bf16
    # O / l of 512 values and an fp32 lse each
    assert need == 64 * 2 * 128 * (512 * 2 + 4)
    assert _mla(L, dec, ws=None, wsb=0) == dsa.DSA_ERR_WORKSPACE_TOO_SMALL
    assert _mla(L, dec, ws=None, wsb=need) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert _mla(L, dec, H=96, ws=ctypes.c_void_p(0x50), wsb=need) == dsa.DSA_ERR_UNSUPPORTED
    assert _mla(L, dec, Dl=256, ws=ctypes.c_void_p(0x50), wsb=need) == dsa.DSA_ERR_UNSUPPORTED
    assert _mla(L, dec, dtype=dsa.DSA_FP8_E4M3) == dsa.DSA_ERR_UNSUPPORTED
    assert _mla(L, dec, k=0) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert _mla(L, dec, scale=float("nan")) == dsa.DSA_ERR_INVALID_ARGUMENT
    # finite, but the kernels' base-2 scale (times log2(e)) would overflow
    assert _mla(L, dec, scale=3e38) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert _mla(L, dec, scale=-3e38) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert _mla(L, dec, nullout=True, ws=ctypes.c_void_p(0x50), wsb=need) == dsa.DSA_ERR_INVALID_ARGUMENT
    # decode needs cu_seqlens_q == NULL, prefill needs it
    pre = _batch(num_seqs=1, num_rows=4096, max_seq_len_q=4096, cu_seqlens_q=0x6000)
    assert _mla(L, pre, decode=True) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert _mla(L, dec, decode=False) == dsa.DSA_ERR_INVALID_ARGUMENT
    # a long prefill needs no partials
    assert L.dsa_workspace_bytes(dsa.DSA_OP_MLA_PREFILL, ctypes.byref(pre), 2048, 128, 512, dsa.DSA_BF16) == 0
    assert _mla(L, dsa.DsaBatch(**{**{f: getattr(pre, f) for f, _ in dsa.DsaBatch._fields_},
                                   "num_rows": 0, "num_seqs": 1}), decode=False) == dsa.DSA_OK


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("which", ["q", "kv", "out", "ws"])
def test_attention_rejects_misaligned_pointers(L, fp8, which):
    dec = _batch(num_seqs=64, num_rows=64)
    dt = dsa.DSA_FP8_E4M3 if fp8 else dsa.DSA_BF16
    need = L.dsa_workspace_bytes(dsa.DSA_OP_MLA_DECODE, ctypes.byref(dec), 2048, 128, 512, dt)
    ptr = {"q": 0x10, "kv": 0x20, "out": 0x40, "ws": 0x1000}
    ptr[which] += 8
    V = ctypes.c_void_p
    if fp8:
        st = L.sparse_mla_decode_fp8(ctypes.byref(dec), V(ptr["q"]), 0.02, V(ptr["kv"]), 0.01, V(0x30), 2048,
                                     128, 512, 64, 0.07, V(ptr["out"]), None, V(ptr["ws"]), need, None)
    else:
        st = L.sparse_mla_decode(ctypes.byref(dec), V(ptr["q"]), V(ptr["kv"]), dt, V(0x30), 2048, 128, 512, 64,
                                 0.07, V(ptr["out"]), None, V(ptr["ws"]), need, None)
    assert st == dsa.DSA_ERR_INVALID_ARGUMENT


def test_topk_workspace_for_few_long_rows(L):
    few_long = _batch(num_seqs=8, num_rows=8, max_pages_per_seq=2048, max_seq_len_k=131072)
    need = L.dsa_workspace_bytes(dsa.DSA_OP_TOPK, ctypes.byref(few_long), 2048, 0, 0, 0)
    # 8 chunks of 16384 per row, 2048 (key, position) candidates of 8 bytes each
    assert need == 8 * 8 * 2048 * 8
    assert _idx(L, few_long, stride=131072) == dsa.DSA_ERR_WORKSPACE_TOO_SMALL
    many = _batch(num_seqs=4096, num_rows=4096, max_pages_per_seq=2048, max_seq_len_k=131072)
    assert L.dsa_workspace_bytes(dsa.DSA_OP_TOPK, ctypes.byref(many), 2048, 0, 0, 0) == 0


def test_workspace_bytes_errors(L):
    b = _batch()
    assert L.dsa_workspace_bytes(7, ctypes.byref(b), 16, 128, 512, dsa.DSA_BF16) == ctypes.c_size_t(-1).value
    assert L.dsa_workspace_bytes(dsa.DSA_OP_TOPK, ctypes.byref(b), 0, 0, 0, 0) == ctypes.c_size_t(-1).value
    assert L.dsa_workspace_bytes(dsa.DSA_OP_TOPK, ctypes.byref(b), 16, 0, 0, 0) == 0
    with pytest.raises(dsa.DsaError):
        dsa.dsa_workspace_bytes(dsa.DSA_OP_TOPK, dsa.Batch(b, ()), 0, 0, 0, 0)


def test_python_binding_raises_on_errors(L):
    bt = FakeTensor((1, 4))
    sl = FakeTensor((1,))
    batch = dsa.make_batch(bt, sl, page_size=24, num_pages=4, max_seq_len_k=10)
    logits = FakeTensor((1, 16))
    idx = FakeTensor((1, 8))
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_topk(batch, logits, 8, idx, stream=0)
    assert e.value.status == dsa.DSA_ERR_INVALID_ARGUMENT
    assert "page_size" in str(e.value)


def test_quant_entry_points_validate_on_the_host(L):
    V = ctypes.c_void_p
    ok = dsa.DSA_OK
    assert L.dsa_quant_index_q(None, None, 0, 64, 128, None, None, None) == ok      # nothing to do
    assert L.dsa_quant_index_q(V(0x100), V(0x200), 4, 64, 64, V(0x300), V(0x400), None) == dsa.DSA_ERR_UNSUPPORTED
    assert L.dsa_quant_index_q(None, V(0x200), 4, 64, 128, V(0x300), V(0x400), None) == \
        dsa.DSA_ERR_INVALID_ARGUMENT
    assert L.dsa_quant_index_q(V(0x108), V(0x200), 4, 64, 128, V(0x300), V(0x400), None) == \
        dsa.DSA_ERR_INVALID_ARGUMENT                                                 # q misaligned
    assert L.dsa_quant_index_q(V(0x100), V(0x200), -1, 64, 128, V(0x300), V(0x400), None) == \
        dsa.DSA_ERR_INVALID_ARGUMENT
    assert L.dsa_store_index_k(None, 0, 128, None, 64, 4, None, None) == ok
    assert L.dsa_store_index_k(V(0x100), 3, 128, V(0x200), 48 + 1, 4, V(0x300), None) == \
        dsa.DSA_ERR_INVALID_ARGUMENT                                                 # page size
    assert L.dsa_store_index_k(V(0x100), 3, 96, V(0x200), 64, 4, V(0x300), None) == dsa.DSA_ERR_UNSUPPORTED
    assert L.dsa_store_index_k(V(0x100), 3, 128, None, 64, 4, V(0x300), None) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert L.dsa_store_index_k(V(0x100), 3, 128, V(0x200), 64, 4, V(0x308), None) == \
        dsa.DSA_ERR_INVALID_ARGUMENT                                                 # cache misaligned


def test_fp8_attention_entry_points_validate_on_the_host(L):
    b = _batch()
    V = ctypes.c_void_p

    def call(q_scale=0.02, kv_scale=0.01, H=128, Dl=512, Dr=64, ws=None, wsb=0, scale=0.07):
        return L.sparse_mla_decode_fp8(ctypes.byref(b), V(0x10), q_scale, V(0x20), kv_scale, V(0x30), 2048,
                                       H, Dl, Dr, scale, V(0x40), None, ws, wsb, None)
    need = L.dsa_workspace_bytes(dsa.DSA_OP_MLA_DECODE, ctypes.byref(b), 2048, 128, 512, dsa.DSA_FP8_E4M3)
    rows = b.num_rows
    assert need >= rows * 2 * 128 * (512 * 2 + 4)                      # at least two splits
    assert call(q_scale=0.0, ws=V(0x1000), wsb=need) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert call(kv_scale=float("inf"), ws=V(0x1000), wsb=need) == dsa.DSA_ERR_INVALID_ARGUMENT
    # each scale finite, their product with log2(e) not
    assert call(q_scale=1e20, kv_scale=1e20, ws=V(0x1000), wsb=need) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert call(scale=3e38, q_scale=1.0, kv_scale=1.0, ws=V(0x1000), wsb=need) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert call(H=96, ws=V(0x1000), wsb=need) == dsa.DSA_ERR_UNSUPPORTED
    assert call(Dr=32, ws=V(0x1000), wsb=need) == dsa.DSA_ERR_UNSUPPORTED
    assert call(ws=V(0x1000), wsb=need - 1) == dsa.DSA_ERR_WORKSPACE_TOO_SMALL
    # the plain entry point does not take an fp8 cache (it has no scales)
    assert L.sparse_mla_decode(ctypes.byref(b), V(0x10), V(0x20), dsa.DSA_FP8_E4M3, V(0x30), 2048, 128, 512, 64,
                               0.07, V(0x40), None, V(0x1000), need, None) == dsa.DSA_ERR_UNSUPPORTED


def test_noalloc_rejects_partials_beyond_the_scratch(L):
    """1,024 rows at k = 4096 need two splits each: 1024 x 2 x 128 heads x
    (512 bf16 + fp32 lse) bytes of partials, far above the 32 MiB scratch. The
    call is rejected on the host before any device work."""
    bt = FakeTensor((1024, 64), ptr=0x10000)
    sl = FakeTensor((1024,), ptr=0x20000)
    batch = dsa.make_batch(bt, sl, page_size=64, num_pages=100, max_seq_len_k=4096, max_seq_len_q=1)
    need = dsa.dsa_workspace_bytes(dsa.DSA_OP_MLA_DECODE, batch, 4096, 128, 512, dsa.DSA_BF16)
    assert need > 32 << 20
    q = FakeTensor((1024, 128, 576), ptr=0x30000)
    idx = FakeTensor((1024, 4096), ptr=0x40000)
    out = FakeTensor((1024, 128, 512), ptr=0x50000)
    st = L.sparse_mla_decode_noalloc(batch.ref(), ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(0x60000),
                                     dsa.DSA_BF16, ctypes.c_void_p(idx.data_ptr()), 4096, 128, 512, 64,
                                     ctypes.c_float(0.07), ctypes.c_void_p(out.data_ptr()), None, None)
    assert st == dsa.DSA_ERR_UNSUPPORTED
    assert b"static scratch" in L.dsa_last_error()


def test_noalloc_reports_the_plain_calls_status(L):
    """An unsupported head count gives the same status as sparse_mla_decode (no launch)."""
    bt = FakeTensor((4, 8), ptr=0x10000)
    sl = FakeTensor((4,), ptr=0x20000)
    batch = dsa.make_batch(bt, sl, page_size=64, num_pages=100, max_seq_len_k=512, max_seq_len_q=1)
    V = ctypes.c_void_p
    args = (batch.ref(), V(0x30000), V(0x60000), dsa.DSA_BF16, V(0x40000), 2048, 96, 512, 64, ctypes.c_float(0.07),
            V(0x50000), None)
    assert L.sparse_mla_decode_noalloc(*args, None) == dsa.DSA_ERR_UNSUPPORTED
    assert L.sparse_mla_decode(*args, V(0x1000), 1 << 20, None) == dsa.DSA_ERR_UNSUPPORTED
    bad = args[:5] + (0,) + args[6:]                      # k = 0
    assert L.sparse_mla_decode_noalloc(*bad, None) == dsa.DSA_ERR_INVALID_ARGUMENT


def _fused(L, batch, H=64, D=128, k=2048, n_init=0, n_local=0, ws=0x600, wsb=1 << 30, q=0x100, w=0x200,
           cache=0x300, idx=0x400):
    V = ctypes.c_void_p
    return L.dsa_indexer_topk(ctypes.byref(batch), V(q) if q else None, V(w) if w else None,
                              V(cache) if cache else None, H, D, n_init, n_local, k, V(idx) if idx else None,
                              V(ws) if ws else None, wsb, None)


def test_fused_indexer_topk_validation(L):
    b = _batch()
    assert _fused(L, b, H=32) == dsa.DSA_ERR_UNSUPPORTED
    assert _fused(L, b, D=64) == dsa.DSA_ERR_UNSUPPORTED
    for k in (0, -3, 4097):
        assert _fused(L, b, k=k) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert _fused(L, b, n_init=-1) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert _fused(L, b, n_local=-1) == dsa.DSA_ERR_INVALID_ARGUMENT
    for which in ("q", "w", "cache", "idx"):
        assert _fused(L, b, **{which: 0}) == dsa.DSA_ERR_INVALID_ARGUMENT, which
    for which in ("q", "w", "cache"):
        assert _fused(L, b, **{which: 0x108}) == dsa.DSA_ERR_INVALID_ARGUMENT, which
    assert _fused(L, _batch(page_size=24)) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert _fused(L, _batch(max_seq_len_k=(1 << 24) + 1)) == dsa.DSA_ERR_UNSUPPORTED
    assert _fused(L, b, H=16) == dsa.DSA_ERR_UNSUPPORTED
    assert "64 fp8 heads" in _last(L)
    # an empty batch needs nothing and launches nothing
    empty = _batch(num_seqs=0, num_rows=0, block_table=None, seq_lens_k=None)
    assert _fused(L, empty, ws=0, wsb=0, q=0, w=0, cache=0, idx=0) == dsa.DSA_OK


def _last(L):
    return L.dsa_last_error().decode()


def test_fused_indexer_topk_workspace(L):
    # 64 rows of up to 32,564 keys: 8,192-key chunks would give 256 work-groups
    # (fewer than two per CU), so chunks of 4,096: 8 per row, k pairs of 8 bytes each
    b = _batch(num_seqs=64, num_rows=64, max_pages_per_seq=509, max_seq_len_k=32564)
    need = L.dsa_workspace_bytes(dsa.DSA_OP_INDEXER_TOPK, ctypes.byref(b), 2048, 0, 0, 0)
    assert need == 64 * 8 * 2048 * 8
    assert _fused(L, b, wsb=need - 1) == dsa.DSA_ERR_WORKSPACE_TOO_SMALL
    assert _fused(L, b, ws=0, wsb=need) == dsa.DSA_ERR_INVALID_ARGUMENT
    # 4,096 prefill rows of up to 20,480 keys: chunks of 8,192 (3 per row)
    pre = _batch(num_seqs=1, num_rows=4096, max_pages_per_seq=320, max_seq_len_k=20480, max_seq_len_q=4096,
                 cu_seqlens_q=0x7000)
    assert L.dsa_workspace_bytes(dsa.DSA_OP_INDEXER_TOPK, ctypes.byref(pre), 2048, 0, 0, 0) == 4096 * 3 * 2048 * 8
    # k above a quarter of 8,192 keeps the 8,192-key chunks
    assert L.dsa_workspace_bytes(dsa.DSA_OP_INDEXER_TOPK, ctypes.byref(b), 4096, 0, 0, 0) == 64 * 4 * 4096 * 8
    assert L.dsa_workspace_bytes(dsa.DSA_OP_INDEXER_TOPK, ctypes.byref(b), 0, 0, 0, 0) == ctypes.c_size_t(-1).value
