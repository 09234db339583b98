"""fp64 reference of decode over a KV cache with paging and in-place append
(test infrastructure only).

[FA] "Examples" (flash_attn_with_kvcache): q attends to the cached keys and
values of its batch row, k_cache / v_cache are updated in place with the new
keys / values k, v, cache_seqlens gives the cache lengths, cache_batch_idx
indexes the cache's batch rows, and block_table addresses a paged cache.  The
pages print only the argument list; the readings used here are:

  * new keys/values of batch b go to cache rows [L_b, L_b + S_new) of that
    sequence (L_b = cache_seqlens[b]) and the query then attends to the first
    L_b + S_new rows (the cache lengths themselves are not changed: the caller
    advances them);
  * a paged cache is [num_pages, page_size, Hkv, D]; row r of sequence b is
    row r % page_size of page block_table[b, r // page_size];
  * cache_batch_idx[b] is the batch row of a contiguous cache that sequence b
    uses (identity when absent); it is not combined with paging.

Everything else is the decode definition of ``attention.decode``.
"""

import numpy as np

from .attention import decode


def cache_rows(cache, b, n, block_table=None, page_size=None, cache_batch_idx=None):
    """Rows [0, n) of sequence b's cache as a contiguous [n, Hkv, D] array."""
    if block_table is None:
        row = int(cache_batch_idx[b]) if cache_batch_idx is not None else b
        return cache[row, :n]
    out = np.empty((n,) + cache.shape[2:], dtype=cache.dtype)
    for r in range(n):
        out[r] = cache[int(block_table[b, r // page_size]), r % page_size]
    return out


def kvcache_append(k_cache, v_cache, k_new, v_new, cache_seqlens, block_table=None,
                   page_size=None, cache_batch_idx=None):
    """Copies of the caches with rows [L_b, L_b + S_new) of every sequence b
    replaced by k_new[b], v_new[b] ([B, S_new, Hkv, D])."""
    kc, vc = k_cache.copy(), v_cache.copy()
    B, S_new = k_new.shape[:2]
    for b in range(B):
        L = int(cache_seqlens[b])
        for t in range(S_new):
            r = L + t
            if block_table is None:
                row = int(cache_batch_idx[b]) if cache_batch_idx is not None else b
                kc[row, r], vc[row, r] = k_new[b, t], v_new[b, t]
            else:
                page = int(block_table[b, r // page_size])
                kc[page, r % page_size], vc[page, r % page_size] = k_new[b, t], v_new[b, t]
    return kc, vc


def decode_kvcache(q, k_cache, v_cache, cache_seqlens, block_table=None, page_size=None,
                   cache_batch_idx=None, k_new=None, v_new=None, scale=None, softcap=0.0,
                   causal=False):
    """Append (when k_new / v_new are given), then attend each sequence's
    queries to the first cache_seqlens[b] + S_new rows of its cache (with
    ``causal``, bottom-right aligned: the last query sees every row, query t
    of Sq the first cache_seqlens[b] + S_new - Sq + 1 + t).

    Returns O [B, Sq, Hq, D], LSE [B, Hq, Sq] and the updated caches."""
    B = q.shape[0]
    lens = np.asarray(cache_seqlens, dtype=np.int64)
    if k_new is not None:
        k_cache, v_cache = kvcache_append(k_cache, v_cache, k_new, v_new, lens, block_table,
                                          page_size, cache_batch_idx)
        lens = lens + k_new.shape[1]
    n_max = max(int(lens.max()) if B else 0, 1)
    kc = np.zeros((B, n_max) + k_cache.shape[2:], dtype=np.float64)
    vc = np.zeros((B, n_max) + v_cache.shape[2:], dtype=np.float64)
    for b in range(B):
        n = int(lens[b])
        kc[b, :n] = cache_rows(k_cache, b, n, block_table, page_size, cache_batch_idx)
        vc[b, :n] = cache_rows(v_cache, b, n, block_table, page_size, cache_batch_idx)
    O, L = decode(q, kc, vc, lens, scale=scale, softcap=softcap, causal=causal)
    return O, L, (k_cache, v_cache)
