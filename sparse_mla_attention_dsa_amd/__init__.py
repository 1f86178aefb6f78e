"""Python binding of the DSA C ABI (`include/dsa.h`, `libdsa.so`).

Argument marshalling only: torch tensors become device pointers, the current
torch stream becomes the HIP stream, and every computation happens in the HIP
kernels of libdsa.so. There is no fallback: if the library is not built, or a
call fails, an exception is raised.

    batch = make_batch(block_table, seq_lens_k, cu_seqlens_q, page_size=64,
                       num_pages=..., max_seq_len_k=..., max_seq_len_q=1)
    dsa_indexer_logits(batch, q_fp8, w, index_cache, logits)
    dsa_topk(batch, logits, k, topk_idx)
    sparse_mla_decode(batch, q, kv_cache, topk_idx, softmax_scale, out, lse, workspace)
"""
import ctypes
import os

__all__ = [
    "DSA_OK", "DSA_F32", "DSA_BF16", "DSA_FP8_E4M3", "DSA_OP_TOPK", "DSA_OP_MLA_DECODE",
    "DSA_OP_MLA_PREFILL", "DSA_OP_INDEXER_TOPK", "DsaError", "DsaBatch", "lib", "library_path", "make_batch",
    "dsa_indexer_logits", "dsa_topk", "dsa_indexer_topk", "sparse_mla_decode", "sparse_mla_prefill",
    "dsa_quant_index_q", "dsa_store_index_k", "sparse_mla_decode_fp8", "sparse_mla_prefill_fp8",
    "sparse_mla_decode_noalloc", "dsa_workspace_bytes", "dsa_version", "EXPORTED_SYMBOLS",
]

DSA_OK, DSA_ERR_INVALID_ARGUMENT, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE_TOO_SMALL, DSA_ERR_HIP = range(5)
DSA_F32, DSA_BF16, DSA_FP8_E4M3 = range(3)
DSA_OP_TOPK, DSA_OP_MLA_DECODE, DSA_OP_MLA_PREFILL, DSA_OP_INDEXER_TOPK = range(4)

EXPORTED_SYMBOLS = (
    "dsa_indexer_logits", "dsa_topk", "dsa_indexer_topk", "sparse_mla_decode", "sparse_mla_prefill",
    "dsa_quant_index_q", "dsa_store_index_k", "sparse_mla_decode_fp8", "sparse_mla_prefill_fp8",
    "sparse_mla_decode_noalloc", "dsa_workspace_bytes", "dsa_status_string", "dsa_last_error",
    "dsa_version",
)

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path():
    return os.path.join(_HERE, "libdsa.so")


class DsaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"dsa status {status}: {message}")
        self.status = status


class DsaBatch(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("num_rows", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("max_seq_len_k", ctypes.c_int32),
        ("max_seq_len_q", ctypes.c_int32),
        ("block_table", ctypes.c_void_p),
        ("seq_lens_k", ctypes.c_void_p),
        ("cu_seqlens_q", ctypes.c_void_p),
    ]


_LIB = None


def lib():
    """Load libdsa.so (once). Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -m sparse_mla_attention_dsa_amd.build` "
                           "(or __graft_entry__.build()) first")
    L = ctypes.CDLL(path)
    P, I32, I64, SZ, F32, V = (ctypes.POINTER(DsaBatch), ctypes.c_int32, ctypes.c_int64,
                               ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p)
    L.dsa_indexer_logits.argtypes = [P, V, I32, V, V, I32, I32, I32, V, I64, I32, I32, V]
    L.dsa_indexer_logits.restype = I32
    L.dsa_topk.argtypes = [P, V, I64, I32, V, V, SZ, V]
    L.dsa_topk.restype = I32
    L.dsa_indexer_topk.argtypes = [P, V, V, V, I32, I32, I32, I32, I32, V, V, SZ, V]
    L.dsa_indexer_topk.restype = I32
    for name in ("sparse_mla_decode", "sparse_mla_prefill"):
        f = getattr(L, name)
        f.argtypes = [P, V, V, I32, V, I32, I32, I32, I32, F32, V, V, V, SZ, V]
        f.restype = I32
    L.sparse_mla_decode_noalloc.argtypes = [P, V, V, I32, V, I32, I32, I32, I32, F32, V, V, V]
    L.sparse_mla_decode_noalloc.restype = I32
    for name in ("sparse_mla_decode_fp8", "sparse_mla_prefill_fp8"):
        f = getattr(L, name)
        f.argtypes = [P, V, F32, V, F32, V, I32, I32, I32, I32, F32, V, V, V, SZ, V]
        f.restype = I32
    L.dsa_quant_index_q.argtypes = [V, V, I32, I32, I32, V, V, V]
    L.dsa_quant_index_q.restype = I32
    L.dsa_store_index_k.argtypes = [V, I32, I32, V, I32, I32, V, V]
    L.dsa_store_index_k.restype = I32
    L.dsa_workspace_bytes.argtypes = [I32, P, I32, I32, I32, I32]
    L.dsa_workspace_bytes.restype = SZ
    L.dsa_status_string.argtypes = [I32]
    L.dsa_status_string.restype = ctypes.c_char_p
    L.dsa_last_error.argtypes = []
    L.dsa_last_error.restype = ctypes.c_char_p
    L.dsa_version.argtypes = []
    L.dsa_version.restype = ctypes.c_char_p
    _LIB = L
    return L


def _check(status):
    if status != DSA_OK:
        L = lib()
        raise DsaError(status, f"{L.dsa_status_string(status).decode()}: {L.dsa_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    handle = getattr(stream, "cuda_stream", stream)
    return ctypes.c_void_p(int(handle))


def _dtype_code(t):
    import torch
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return DSA_FP8_E4M3
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return DSA_BF16
    raise TypeError(f"no DSA dtype for torch dtype {t.dtype}")


class Batch:
    """A dsa_batch_t plus references to the device tensors it points into."""

    def __init__(self, struct, tensors):
        self.struct = struct
        self._tensors = tensors

    def ref(self):
        return ctypes.byref(self.struct)


def make_batch(block_table, seq_lens_k, cu_seqlens_q=None, *, page_size, num_pages,
               max_seq_len_k, max_seq_len_q=1, num_rows=None):
    """Build the batch descriptor. Tensors are int32 device tensors; the max
    lengths are host integers the caller already knows (nothing is read back)."""
    B = int(seq_lens_k.shape[0])
    if num_rows is None:
        num_rows = B if cu_seqlens_q is None else None
    if num_rows is None:
        raise ValueError("num_rows is required with cu_seqlens_q (it is not read back from the device)")
    s = DsaBatch(B, int(num_rows), int(page_size), int(block_table.shape[1]), int(num_pages),
                 int(max_seq_len_k), int(max_seq_len_q), _ptr(block_table).value,
                 _ptr(seq_lens_k).value, None if cu_seqlens_q is None else _ptr(cu_seqlens_q).value)
    return Batch(s, (block_table, seq_lens_k, cu_seqlens_q))


def dsa_indexer_logits(batch, q, w, index_cache, logits, *, num_heads=None, head_dim=None, num_init_tokens=0,
                       num_local_tokens=0, stream=None):
    """logits[t, s] = sum_h w[t,h] relu(sigma_s (q[t,h] . k_s)) for s < visible(t), then +inf at the
    first num_init_tokens and the last num_local_tokens visible positions of each row."""
    code = _dtype_code(q)
    H = int(q.shape[1]) if num_heads is None else num_heads
    D = int(q.shape[2]) if head_dim is None else head_dim
    _check(lib().dsa_indexer_logits(batch.ref(), _ptr(q), code, _ptr(w), _ptr(index_cache), code,
                                    H, D, _ptr(logits), int(logits.stride(0)), int(num_init_tokens),
                                    int(num_local_tokens), _stream(stream)))


def dsa_topk(batch, logits, k, topk_idx, workspace=None, stream=None):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsa_topk(batch.ref(), _ptr(logits), int(logits.stride(0)), int(k), _ptr(topk_idx),
                          _ptr(workspace), nbytes, _stream(stream)))


def dsa_indexer_topk(batch, q, w, index_cache, k, topk_idx, workspace=None, *, num_init_tokens=0,
                     num_local_tokens=0, stream=None):
    """dsa_indexer_logits (fp8, 64 x 128) followed by dsa_topk, without the
    logits in memory; `workspace` holds dsa_workspace_bytes(DSA_OP_INDEXER_TOPK)."""
    H, D = int(q.shape[1]), int(q.shape[2])
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().dsa_indexer_topk(batch.ref(), _ptr(q), _ptr(w), _ptr(index_cache), H, D, int(num_init_tokens),
                                  int(num_local_tokens), int(k), _ptr(topk_idx), _ptr(workspace), nbytes,
                                  _stream(stream)))


def _mla(fn, batch, q, kv_cache, topk_idx, softmax_scale, out, lse, workspace, d_latent, stream):
    code = _dtype_code(q)
    Hm, Dqk = int(q.shape[1]), int(q.shape[2])
    Dl = int(out.shape[2]) if d_latent is None else d_latent
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(batch.ref(), _ptr(q), _ptr(kv_cache), code, _ptr(topk_idx), int(topk_idx.shape[1]),
              Hm, Dl, Dqk - Dl, float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace),
              nbytes, _stream(stream)))


def sparse_mla_decode(batch, q, kv_cache, topk_idx, softmax_scale, out, lse=None, workspace=None,
                      *, d_latent=None, stream=None):
    _mla(lib().sparse_mla_decode, batch, q, kv_cache, topk_idx, softmax_scale, out, lse, workspace,
         d_latent, stream)


def sparse_mla_prefill(batch, q, kv_cache, topk_idx, softmax_scale, out, lse=None, workspace=None,
                       *, d_latent=None, stream=None):
    _mla(lib().sparse_mla_prefill, batch, q, kv_cache, topk_idx, softmax_scale, out, lse, workspace,
         d_latent, stream)


def sparse_mla_decode_noalloc(batch, q, kv_cache, topk_idx, softmax_scale, out, lse=None, *, d_latent=None,
                              stream=None):
    """sparse_mla_decode with its split partials in the library's static
    per-GPU scratch (no workspace argument, nothing allocated)."""
    code = _dtype_code(q)
    Hm, Dqk = int(q.shape[1]), int(q.shape[2])
    Dl = int(out.shape[2]) if d_latent is None else d_latent
    _check(lib().sparse_mla_decode_noalloc(batch.ref(), _ptr(q), _ptr(kv_cache), code, _ptr(topk_idx),
                                           int(topk_idx.shape[1]), Hm, Dl, Dqk - Dl, float(softmax_scale),
                                           _ptr(out), _ptr(lse), _stream(stream)))


def _mla_fp8(fn, batch, q, q_scale, kv_cache, kv_scale, topk_idx, softmax_scale, out, lse, workspace, stream):
    Hm, Dqk = int(q.shape[1]), int(q.shape[2])
    Dl = int(out.shape[2])
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(fn(batch.ref(), _ptr(q), float(q_scale), _ptr(kv_cache), float(kv_scale), _ptr(topk_idx),
              int(topk_idx.shape[1]), Hm, Dl, Dqk - Dl, float(softmax_scale), _ptr(out), _ptr(lse),
              _ptr(workspace), nbytes, _stream(stream)))


def sparse_mla_decode_fp8(batch, q, q_scale, kv_cache, kv_scale, topk_idx, softmax_scale, out, lse=None,
                          workspace=None, *, stream=None):
    """Sparse MLA over an fp8 latent cache: q, kv_cache E4M3 codes (uint8) with
    per-tensor scales; out [T, Hm, 512] bf16."""
    _mla_fp8(lib().sparse_mla_decode_fp8, batch, q, q_scale, kv_cache, kv_scale, topk_idx, softmax_scale,
             out, lse, workspace, stream)


def sparse_mla_prefill_fp8(batch, q, q_scale, kv_cache, kv_scale, topk_idx, softmax_scale, out, lse=None,
                           workspace=None, *, stream=None):
    _mla_fp8(lib().sparse_mla_prefill_fp8, batch, q, q_scale, kv_cache, kv_scale, topk_idx, softmax_scale,
             out, lse, workspace, stream)


def dsa_quant_index_q(q, w, q8, w_eff, stream=None):
    """q [T, H, 128] bf16 -> q8 [T, H, 128] fp8 codes and w_eff = w * per-head scale."""
    T, H, D = (int(x) for x in q.shape)
    _check(lib().dsa_quant_index_q(_ptr(q), _ptr(w), T, H, D, _ptr(q8), _ptr(w_eff), _stream(stream)))


def dsa_store_index_k(key, slot_mapping, index_cache, page_size, stream=None):
    """Quantize key [N, 128] bf16 per token and store it at slot_mapping [N] int64
    into the paged index cache [num_pages, 132 * page_size] (uint8)."""
    N, D = (int(x) for x in key.shape)
    _check(lib().dsa_store_index_k(_ptr(key), N, D, _ptr(slot_mapping), int(page_size),
                                   int(index_cache.shape[0]), _ptr(index_cache), _stream(stream)))


def dsa_workspace_bytes(op, batch, k, num_heads, d_latent, dtype):
    n = lib().dsa_workspace_bytes(int(op), batch.ref(), int(k), int(num_heads), int(d_latent), int(dtype))
    if n == ctypes.c_size_t(-1).value:
        raise DsaError(DSA_ERR_INVALID_ARGUMENT, lib().dsa_last_error().decode())
    return int(n)


def dsa_version():
    return lib().dsa_version().decode()
