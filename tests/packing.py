"""Byte packing for hand-made test inputs (the layouts the library reads)."""
import numpy as np


def pack_index_cache_f32(keys_by_page, sigma_by_page):
    """keys_by_page [pages, P, D] float32, sigma_by_page [pages, P] -> uint8 [pages, P*D*4 + P*4]."""
    keys = np.ascontiguousarray(keys_by_page, dtype=np.float32)
    sig = np.ascontiguousarray(sigma_by_page, dtype=np.float32)
    pages, P, D = keys.shape
    out = np.empty((pages, 4 * P * D + 4 * P), dtype=np.uint8)
    out[:, :4 * P * D] = keys.reshape(pages, -1).view(np.uint8)
    out[:, 4 * P * D:] = sig.view(np.uint8).reshape(pages, -1)
    return out


def pack_index_cache_fp8(codes_by_page, sigma_by_page):
    codes = np.ascontiguousarray(codes_by_page, dtype=np.uint8)
    sig = np.ascontiguousarray(sigma_by_page, dtype=np.float32)
    pages, P, D = codes.shape
    out = np.empty((pages, P * D + 4 * P), dtype=np.uint8)
    out[:, :P * D] = codes.reshape(pages, -1)
    out[:, P * D:] = sig.view(np.uint8).reshape(pages, -1)
    return out


def scatter_tokens(tokens, block_table_row, num_pages, page_size, fill=np.nan):
    """Place per-token rows [n, ...] into pages [num_pages, P, ...] through a block-table row."""
    tokens = np.asarray(tokens)
    out = np.full((num_pages, page_size) + tokens.shape[1:], fill, dtype=tokens.dtype)
    for p in range(tokens.shape[0]):
        out[block_table_row[p // page_size], p % page_size] = tokens[p]
    return out
