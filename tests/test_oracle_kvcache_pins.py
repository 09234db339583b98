"""Pins of the KV-cache oracle (paged cache, cache_batch_idx, in-place append;
[FA] "Examples", flash_attn_with_kvcache) against independent constructions:
a paged cache built by scattering a contiguous cache through a random block
table must decode exactly like the contiguous cache (decode itself is pinned
in test_oracle_pins.py), appended rows are checked element by element, and
the decode after an append must equal decode over the explicitly
concatenated rows."""

import numpy as np
import pytest

import oracle


def _case(seed, B=3, Smax=96, Hq=4, Hkv=2, D=16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, 1, Hq, D))
    k = rng.standard_normal((B, Smax, Hkv, D))
    v = rng.standard_normal((B, Smax, Hkv, D))
    lens = np.array([Smax, 1, 37][:B], dtype=np.int64)
    return rng, q, k, v, lens


def _scatter_paged(rng, k, page_size, spare=3):
    """Scatter a contiguous [B, Smax, ...] cache into pages in random order."""
    B, Smax = k.shape[:2]
    nblk = -(-Smax // page_size)
    num_pages = B * nblk + spare
    perm = rng.permutation(num_pages)[: B * nblk].reshape(B, nblk)
    pages = rng.standard_normal((num_pages, page_size) + k.shape[2:])  # junk in unused rows
    for b in range(B):
        for r in range(Smax):
            pages[perm[b, r // page_size], r % page_size] = k[b, r]
    return pages, perm.astype(np.int32)


@pytest.mark.parametrize("page_size", [32, 64, 7])
def test_paged_equals_contiguous(page_size):
    rng, q, k, v, lens = _case(21)
    kp, bt = _scatter_paged(rng, k, page_size)
    vp = np.empty_like(kp)
    # the same block table for V (pages hold both at the same index)
    for b in range(k.shape[0]):
        for r in range(k.shape[1]):
            vp[bt[b, r // page_size], r % page_size] = v[b, r]
    O, L = oracle.decode(q, k, v, lens, scale=0.3)
    Op, Lp, _ = oracle.decode_kvcache(q, kp, vp, lens, block_table=bt, page_size=page_size, scale=0.3)
    np.testing.assert_array_equal(Op, O)
    np.testing.assert_array_equal(Lp, L)


def test_cache_rows_identity_table():
    rng, q, k, v, lens = _case(22)
    B, Smax, Hkv, D = k.shape
    ps = 32
    pages = k.reshape(B * (Smax // ps), ps, Hkv, D)  # page p of b is b * nblk + p
    bt = np.arange(B * (Smax // ps)).reshape(B, Smax // ps)
    for b in range(B):
        np.testing.assert_array_equal(oracle.cache_rows(pages, b, Smax, bt, ps), k[b])


def test_cache_batch_idx():
    rng, q, k, v, lens = _case(23)
    idx = np.array([2, 0, 1])
    O, L = oracle.decode(q, k[idx], v[idx], lens, softcap=2.0)
    Oi, Li, _ = oracle.decode_kvcache(q, k, v, lens, cache_batch_idx=idx, softcap=2.0)
    np.testing.assert_array_equal(Oi, O)
    np.testing.assert_array_equal(Li, L)


@pytest.mark.parametrize("paged", [False, True])
def test_append_rows_and_decode(paged):
    rng, q, k, v, lens = _case(24, Smax=128)
    lens = np.array([5, 0, 90], dtype=np.int64)
    B, Smax, Hkv, D = k.shape
    S_new = 3
    kn = rng.standard_normal((B, S_new, Hkv, D))
    vn = rng.standard_normal((B, S_new, Hkv, D))
    if paged:
        ps = 32
        kc, bt = _scatter_paged(rng, k, ps)
        vc = np.empty_like(kc)
        for b in range(B):
            for r in range(Smax):
                vc[bt[b, r // ps], r % ps] = v[b, r]
        kw = dict(block_table=bt, page_size=ps)
    else:
        kc, vc, kw = k, v, {}
    k2, v2 = oracle.kvcache_append(kc, vc, kn, vn, lens, **kw)
    # element by element: new rows where they belong, everything else unchanged
    for b in range(B):
        for r in range(Smax):
            if paged:
                loc = (kw["block_table"][b, r // 32], r % 32)
            else:
                loc = (b, r)
            want_k = kn[b, r - lens[b]] if lens[b] <= r < lens[b] + S_new else kc[loc]
            want_v = vn[b, r - lens[b]] if lens[b] <= r < lens[b] + S_new else vc[loc]
            np.testing.assert_array_equal(k2[loc], want_k)
            np.testing.assert_array_equal(v2[loc], want_v)
    # the input caches are not modified
    assert not np.shares_memory(k2, kc)
    # decode after append == decode over old rows followed by the new rows
    cat_k = np.zeros((B, Smax, Hkv, D))
    cat_v = np.zeros((B, Smax, Hkv, D))
    for b in range(B):
        n = lens[b]
        cat_k[b, :n], cat_v[b, :n] = k[b, :n], v[b, :n]
        cat_k[b, n:n + S_new], cat_v[b, n:n + S_new] = kn[b], vn[b]
    O, L = oracle.decode(q, cat_k, cat_v, lens + S_new, scale=0.25)
    Oa, La, _ = oracle.decode_kvcache(q, kc, vc, lens, k_new=kn, v_new=vn, scale=0.25, **kw)
    np.testing.assert_allclose(Oa, O, rtol=0, atol=1e-13)
    np.testing.assert_allclose(La, L, rtol=0, atol=1e-13)
