"""Pins of the fp64 CPU oracle against things other than itself.

Each test names what fixes the expected value: a closed form, a library
routine (scipy), brute-force pure-Python loops with exact summation
(math.fsum) on tiny inputs, finite differences, or an invariant of the
mathematics.  They are chosen so that a plausible slip in the oracle (a
dropped term, a wrong sign or index, a transposed operand, an off-by-one in a
mask bound) fails at least one of them.
"""

import math
import zlib

import numpy as np
import pytest
import scipy.special

import oracle
from exact_attention_10_amd import inputs

RNG = np.random.default_rng(1234)


def rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------------------
# brute-force mini oracle: pure Python loops, exact sums, no key-range cuts


def brute_allowed(i, j, Sq, Sk, causal, window, dq, dk, kv_len):
    d = Sk - Sq
    if causal and not j <= i + d:
        return False
    if window[0] >= 0 and not j >= i + d - window[0]:
        return False
    if window[1] >= 0 and not j <= i + d + window[1]:
        return False
    if dq is not None and dq[i] != dk[j]:
        return False
    if kv_len is not None and not j < kv_len:
        return False
    return True


def brute_fwd(q, k, v, scale, causal=False, window=(-1, -1), slopes=None,
              softcap=0.0, doc=None, kv_len=None):
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, Dv = v.shape
    G = Hq // Hkv
    O = np.zeros((B, Sq, Hq, Dv))
    L = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(Sq):
                us = []
                for j in range(Sk):
                    if not brute_allowed(i, j, Sq, Sk, causal, window,
                                         None if doc is None else doc[b],
                                         None if doc is None else doc[b],
                                         kv_len):
                        continue
                    s = scale * math.fsum(float(q[b, i, h, x]) * float(k[b, j, g, x])
                                          for x in range(D))
                    if softcap > 0:
                        s = softcap * math.tanh(s / softcap)
                    if slopes is not None:
                        # (Hq,) slopes, or (B, Hq): one row per batch row
                        a = slopes[h] if np.ndim(slopes) == 1 else slopes[b][h]
                        s -= float(a) * abs(i + (Sk - Sq) - j)
                    us.append((j, s))
                if not us:
                    continue
                m = max(u for _, u in us)
                z = math.fsum(math.exp(u - m) for _, u in us)
                lse = m + math.log(z)
                L[b, h, i] = lse
                for x in range(Dv):
                    O[b, i, h, x] = math.fsum(math.exp(u - lse) * float(v[b, j, g, x])
                                              for j, u in us)
    return O, L


# ---------------------------------------------------------------------------
# forward


@pytest.mark.parametrize("case", [
    dict(),
    dict(causal=True),
    dict(causal=True, window=(3, 0)),
    dict(window=(2, 5)),
    dict(window=(-1, 1)),
    dict(softcap=1.5),
    dict(slopes=True),
    dict(slopes=True, softcap=2.0, causal=True),
    dict(slopes2d=True, causal=True),
    dict(slopes2d=True, window=(3, 2)),
    dict(doc=True, causal=True),
    dict(kv_len=4),
])
@pytest.mark.parametrize("shape", [(2, 7, 7, 4, 2, 5), (1, 9, 13, 2, 1, 8),
                                   (1, 13, 6, 3, 3, 4)])
def test_fwd_matches_brute_force(case, shape):
    """[P7] fp64 vectorised oracle == pure-Python loops with math.fsum."""
    B, Sq, Sk, Hq, Hkv, D = shape
    rng = np.random.default_rng(zlib.crc32(repr((sorted(case), shape)).encode()))
    q, k, v = rand(B, Sq, Hq, D, rng=rng), rand(B, Sk, Hkv, D, rng=rng), rand(B, Sk, Hkv, D, rng=rng)
    kw = {}
    doc = None
    slopes = None
    if case.get("doc"):
        if Sq != Sk:
            pytest.skip("document masks are self-attention")
        doc = np.stack([np.sort(rng.integers(0, 3, Sq)) for _ in range(B)])
        kw.update(doc_q=doc, doc_k=doc)
    if case.get("slopes"):
        slopes = rng.uniform(0.1, 1.0, Hq)
        kw["alibi_slopes"] = slopes
    if case.get("slopes2d"):
        # per-batch slopes [B, Hq]; every entry distinct, so a swapped
        # [h, b] index or a flattened-index slip changes the result
        slopes = rng.uniform(0.1, 1.0, (B, Hq)) + 0.01 * np.arange(B * Hq).reshape(B, Hq)
        kw["alibi_slopes"] = slopes
    for name in ("causal", "window", "softcap", "kv_len"):
        if name in case:
            kw[name] = case[name]
    O, L = oracle.attention_fwd(q, k, v, scale=0.37, row_chunk=4, **kw)
    Ob, Lb = brute_fwd(q, k, v, 0.37, case.get("causal", False),
                       case.get("window", (-1, -1)), slopes,
                       case.get("softcap", 0.0), doc, case.get("kv_len"))
    np.testing.assert_array_equal(np.isinf(L), np.isinf(Lb))
    fin = np.isfinite(Lb)
    np.testing.assert_allclose(L[fin], Lb[fin], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O, Ob, rtol=1e-12, atol=1e-12)


def test_single_key_returns_v0():
    """[P1] With one key, softmax weight 1: O_i = v_0 exactly, LSE_i = u_i0."""
    q, k, v = rand(2, 5, 3, 8), rand(2, 1, 3, 8), rand(2, 1, 3, 8)
    O, L = oracle.attention_fwd(q, k, v, scale=0.5)
    np.testing.assert_allclose(O, np.broadcast_to(v, O.shape), rtol=0, atol=1e-15)
    expect = 0.5 * np.einsum("bihd,bhd->bhi", q, k[:, 0])
    np.testing.assert_allclose(L, expect, rtol=1e-14, atol=1e-14)
    # the bias of a single key at distance |i + delta - 0| = |i - 4|
    slopes = np.array([0.5, 0.25, 0.125])
    _, La = oracle.attention_fwd(q, k, v, scale=0.5, alibi_slopes=slopes)
    dist = np.abs(np.arange(5) - 4.0)
    np.testing.assert_allclose(La, expect - slopes[None, :, None] * dist[None, None, :],
                               rtol=1e-14, atol=1e-14)


def test_identical_v_rows():
    """[P2] Any convex combination of identical rows is that row."""
    q, k = rand(1, 9, 4, 6), rand(1, 11, 2, 6)
    row = rand(6)
    v = np.broadcast_to(row, (1, 11, 2, 6)).copy()
    O, _ = oracle.attention_fwd(q, k, v, scale=0.9, causal=True, window=(4, 1),
                                alibi_slopes=np.array([.1, .2, .3, .4]), softcap=3.0)
    np.testing.assert_allclose(O, np.broadcast_to(row, O.shape), rtol=0, atol=1e-14)


def test_causal_row0():
    """[P3] Causal square attention: row 0 sees only key 0."""
    q, k, v = rand(1, 6, 2, 4), rand(1, 6, 2, 4), rand(1, 6, 2, 4)
    O, L = oracle.attention_fwd(q, k, v, scale=0.3, causal=True)
    np.testing.assert_allclose(O[0, 0], v[0, 0], atol=1e-15)
    np.testing.assert_allclose(L[0, :, 0], 0.3 * (q[0, 0] * k[0, 0]).sum(-1), rtol=1e-14)


def test_probabilities_are_softmax_via_scipy():
    """[P4, P5] With one-hot value rows the output row is the probability row:
    it must equal scipy.special.softmax of the allowed scores (so it sums to
    1), and LSE must equal scipy.special.logsumexp of them."""
    Sq, Sk, D = 7, 10, 5
    q, k = rand(1, Sq, 1, D), rand(1, Sk, 1, D)
    v = np.eye(Sk).reshape(1, Sk, 1, Sk)
    O, L = oracle.attention_fwd(q, k, v, scale=0.8, causal=True, window=(5, 2))
    for i in range(Sq):
        js = [j for j in range(Sk) if j <= i + 3 and j >= i + 3 - 5]
        s = np.array([0.8 * float(q[0, i, 0] @ k[0, j, 0]) for j in js])
        np.testing.assert_allclose(L[0, 0, i], scipy.special.logsumexp(s), rtol=1e-14)
        p = np.zeros(Sk)
        p[js] = scipy.special.softmax(s)
        np.testing.assert_allclose(O[0, i, 0], p, atol=1e-15)
        assert abs(O[0, i, 0].sum() - 1.0) < 1e-14


def _window_count(i, Sq, Sk, causal, left, right):
    """Closed-form number of allowed keys for row i (no document mask)."""
    d = Sk - Sq
    hi = Sk - 1
    if causal:
        hi = min(hi, i + d)
    if right >= 0:
        hi = min(hi, i + d + right)
    lo = 0 if left < 0 else max(0, i + d - left)
    return max(0, hi - lo + 1)


@pytest.mark.parametrize("Sq,Sk,causal,window", [
    (16, 16, True, (-1, -1)), (9, 20, True, (-1, -1)), (20, 9, True, (-1, -1)),
    (30, 30, True, (7, 0)), (30, 30, False, (3, 5)), (12, 25, False, (0, 0)),
    (25, 12, True, (4, -1)), (8, 8, False, (-1, 2)),
])
def test_zero_q_counts_allowed_keys(Sq, Sk, causal, window):
    """[P6] Q = 0 makes every allowed score 0: O_i is the plain mean of the
    allowed value rows and LSE_i = log(#allowed), with #allowed from the
    closed-form interval length; empty rows give O = 0, LSE = -inf."""
    q = np.zeros((1, Sq, 2, 3))
    k, v = rand(1, Sk, 1, 3), rand(1, Sk, 1, 3)
    O, L = oracle.attention_fwd(q, k, v, scale=1.0, causal=causal, window=window, row_chunk=5)
    d = Sk - Sq
    for i in range(Sq):
        n = _window_count(i, Sq, Sk, causal, *window)
        if n == 0:
            assert np.isneginf(L[0, 0, i]) and np.all(O[0, i] == 0)
            continue
        lo = 0 if window[0] < 0 else max(0, i + d - window[0])
        np.testing.assert_allclose(L[0, :, i], math.log(n), rtol=1e-14)
        np.testing.assert_allclose(O[0, i, 0], v[0, lo:lo + n, 0].mean(0), atol=1e-14)


def test_zero_q_long_window_closed_form():
    """[P6] At the 16384-token causal + (4096, 0) window shape:
    LSE_i = log(min(i, 4096) + 1) for every row (D reduced to 2: the
    predicate does not involve D)."""
    S = 16384
    q = np.zeros((1, S, 1, 2))
    k, v = rand(1, S, 1, 2), rand(1, S, 1, 2)
    _, L = oracle.attention_fwd(q, k, v, scale=1.0, causal=True, window=(4096, 0),
                                row_chunk=2048)
    i = np.arange(S)
    np.testing.assert_allclose(L[0, 0], np.log(np.minimum(i, 4096) + 1.0), rtol=1e-13)


def test_zero_q_document_mask():
    """[P6] Document + causal mask, Q = 0: LSE_i = log(i - start(doc(i)) + 1)."""
    rng = np.random.default_rng(7)
    lens = inputs.doc_lengths(rng, 300, 10, 60)
    doc = inputs.doc_ids(lens)[None]
    q = np.zeros((1, 300, 1, 2))
    k, v = rand(1, 300, 1, 2), rand(1, 300, 1, 2)
    O, L = oracle.attention_fwd(q, k, v, scale=1.0, causal=True, doc_q=doc, doc_k=doc,
                                row_chunk=64)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    start_of = np.repeat(starts, lens)
    i = np.arange(300)
    np.testing.assert_allclose(L[0, 0], np.log(i - start_of + 1.0), rtol=1e-14)
    for r in (0, 17, 150, 299):
        np.testing.assert_allclose(O[0, r, 0], v[0, start_of[r]:r + 1, 0].mean(0), atol=1e-14)


def test_gqa_equals_mha_on_repeated_kv():
    """[P8] GQA/MQA == MHA on K/V repeated by repeat_interleave over heads
    (np.repeat along the head axis), the rule the transformers discussion
    states for repeat_kv."""
    q = rand(2, 9, 8, 4)
    k, v = rand(2, 11, 2, 4), rand(2, 11, 2, 4)
    kw = dict(scale=0.6, causal=True, window=(5, 1), softcap=4.0,
              alibi_slopes=np.linspace(0.1, 0.8, 8))
    O1, L1 = oracle.attention_fwd(q, k, v, **kw)
    O2, L2 = oracle.attention_fwd(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), **kw)
    np.testing.assert_allclose(O1, O2, atol=1e-15)
    np.testing.assert_allclose(L1, L2, atol=1e-15)


def test_noncausal_key_permutation_invariance():
    """[P9] Without position-dependent terms the result does not depend on
    the key order when K and V rows are permuted together."""
    q, k, v = rand(1, 6, 2, 5), rand(1, 13, 2, 5), rand(1, 13, 2, 5)
    perm = np.random.default_rng(3).permutation(13)
    O1, L1 = oracle.attention_fwd(q, k, v, scale=0.4, softcap=2.5)
    O2, L2 = oracle.attention_fwd(q, k[:, perm], v[:, perm], scale=0.4, softcap=2.5)
    np.testing.assert_allclose(O1, O2, atol=1e-14)
    np.testing.assert_allclose(L1, L2, atol=1e-14)


def test_alibi_zero_q_geometric_series():
    """[P10] Q = 0, causal, ALiBi slope a: row i weights key i - t by e^{-a t},
    t = 0..i, so LSE_i = log((1 - e^{-a (i+1)}) / (1 - e^{-a})) and O_i is the
    geometric-weighted mean of v_i, v_{i-1}, ..."""
    S, a = 40, 0.3
    q = np.zeros((1, S, 1, 3))
    k, v = rand(1, S, 1, 3), rand(1, S, 1, 3)
    O, L = oracle.attention_fwd(q, k, v, scale=1.0, causal=True, alibi_slopes=np.array([a]))
    for i in range(S):
        n = i + 1
        np.testing.assert_allclose(L[0, 0, i], math.log((1 - math.exp(-a * n)) / (1 - math.exp(-a))),
                                   rtol=1e-13)
        w = np.exp(-a * np.arange(n))
        expect = (w[:, None] * v[0, i::-1, 0][:n]).sum(0) / w.sum()
        np.testing.assert_allclose(O[0, i, 0], expect, atol=1e-14)


def test_alibi_sign_and_symmetry_noncausal():
    """ALiBi is a penalty (it lowers the LSE below the unbiased one) and,
    without a causal mask, Q = 0 gives symmetric weights e^{-a|i-j|}."""
    S, a = 9, 0.7
    q = np.zeros((1, S, 1, 2))
    k, v = rand(1, S, 1, 2), rand(1, S, 1, 2)
    _, L = oracle.attention_fwd(q, k, v, scale=1.0, alibi_slopes=np.array([a]))
    for i in range(S):
        z = sum(math.exp(-a * abs(i - j)) for j in range(S))
        np.testing.assert_allclose(L[0, 0, i], math.log(z), rtol=1e-14)
        assert L[0, 0, i] < math.log(S)


def test_alibi_per_batch_slopes_are_per_row_runs():
    """ALiBi slopes of shape (batch, nheads) ([FA] "Examples": alibi_slopes
    is (nheads,) or (batch_size, nheads)): batch row b uses row b of the
    table, so the result equals running each batch row alone with that 1-D
    row.  Forward and gradients, with rows that differ per batch and per
    head, and an [h, b] transposition must not pass."""
    rng = np.random.default_rng(21)
    B, Sq, Sk, Hq, Hkv, D = 3, 7, 9, 4, 2, 5
    q, k, v, do = (rng.standard_normal(s) for s in
                   [(B, Sq, Hq, D), (B, Sk, Hkv, D), (B, Sk, Hkv, D), (B, Sq, Hq, D)])
    slopes = rng.uniform(0.05, 1.5, (B, Hq))
    kw = dict(scale=0.6, causal=True, window=(5, 0))
    O, L = oracle.attention_fwd(q, k, v, alibi_slopes=slopes, **kw)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, alibi_slopes=slopes, **kw)
    for b in range(B):
        sl = slice(b, b + 1)
        Ob, Lb = oracle.attention_fwd(q[sl], k[sl], v[sl], alibi_slopes=slopes[b], **kw)
        np.testing.assert_allclose(O[sl], Ob, atol=1e-14)
        np.testing.assert_allclose(L[sl], Lb, rtol=1e-14)
        eq, ek, ev = oracle.attention_bwd(q[sl], k[sl], v[sl], do[sl], alibi_slopes=slopes[b], **kw)
        np.testing.assert_allclose(dq[sl], eq, atol=1e-14)
        np.testing.assert_allclose(dk[sl], ek, atol=1e-14)
        np.testing.assert_allclose(dv[sl], ev, atol=1e-14)
    # rows taken in another batch order give a different answer (the
    # comparison above can see a batch-index slip)
    Ox, _ = oracle.attention_fwd(q, k, v, alibi_slopes=slopes[::-1], **kw)
    assert np.abs(Ox - O).max() > 1e-3
    # decode takes the same table: batch row b of a (B, Hq) table
    Od, Ld = oracle.decode(q[:, -1:], k, v, np.array([9, 4, 7]), scale=0.6,
                           alibi_slopes=slopes)
    for b, n in enumerate((9, 4, 7)):
        ob, lb = oracle.attention_fwd(q[b:b + 1, -1:], k[b:b + 1, :n], v[b:b + 1, :n],
                                      scale=0.6, alibi_slopes=slopes[b])
        np.testing.assert_allclose(Od[b], ob[0], atol=1e-14)
        np.testing.assert_allclose(Ld[b], lb[0], rtol=1e-14)


def test_alibi_per_batch_brute_force_values():
    """Per-batch ALiBi against hand-countable values: Q = 0, causal, slope
    table a[b, h]: LSE of row i is the geometric series
    log((1 - e^{-a n}) / (1 - e^{-a})) with n = i + 1 and a = a[b, h]."""
    S = 12
    a = np.array([[0.2, 0.9], [1.3, 0.05]])
    q = np.zeros((2, S, 2, 3))
    k, v = rand(2, S, 1, 3), rand(2, S, 1, 3)
    _, L = oracle.attention_fwd(q, k, v, scale=1.0, causal=True, alibi_slopes=a)
    for b in range(2):
        for h in range(2):
            for i in range(S):
                n = i + 1
                expect = math.log((1 - math.exp(-a[b, h] * n)) / (1 - math.exp(-a[b, h])))
                assert abs(L[b, h, i] - expect) < 1e-13


def test_softcap_limits():
    """[P11] Softcap c: (a) Q = 0 is unaffected; (b) c -> infinity is no
    softcap; (c) tiny c squashes every score into (-c, c), so the output is the
    plain mean and LSE = log n within c; (d) saturated scores +-big map to +-c:
    with one key at +1000 and the rest at -1000 (c = 1) the weight of the
    first key is e / (e + (n-1)/e)."""
    q, k, v = rand(1, 5, 1, 4), rand(1, 8, 1, 4), rand(1, 8, 1, 4)
    O0, L0 = oracle.attention_fwd(q, k, v, scale=0.5)
    Ob, Lb = oracle.attention_fwd(q, k, v, scale=0.5, softcap=1e9)
    np.testing.assert_allclose(Ob, O0, atol=1e-12)
    np.testing.assert_allclose(Lb, L0, atol=1e-12)
    z = np.zeros_like(q)
    Oz, Lz = oracle.attention_fwd(z, k, v, scale=0.5, softcap=3.0)
    np.testing.assert_allclose(Lz, math.log(8), rtol=1e-14)
    Ot, Lt = oracle.attention_fwd(q, k, v, scale=0.5, softcap=1e-7)
    np.testing.assert_allclose(Ot[0, :, 0], np.broadcast_to(v[0, :, 0].mean(0), (5, 4)), atol=1e-6)
    np.testing.assert_allclose(Lt, math.log(8), atol=2e-7)
    # saturation
    qs = np.ones((1, 1, 1, 1))
    ks = np.array([1000.0] + [-1000.0] * 5).reshape(1, 6, 1, 1)
    vs = np.eye(6).reshape(1, 6, 1, 6)
    Os, Ls = oracle.attention_fwd(qs, ks, vs, scale=1.0, softcap=1.0)
    e = math.e
    np.testing.assert_allclose(Os[0, 0, 0, 0], e / (e + 5 / e), rtol=1e-14)
    np.testing.assert_allclose(Ls[0, 0, 0], math.log(e + 5 / e), rtol=1e-14)
    # the capped score stays strictly inside (-c, c): LSE < c + log(n)
    _, Lc = oracle.attention_fwd(q * 50, k, v, scale=1.0, softcap=2.0)
    assert np.all(Lc < 2.0 + math.log(8))


def test_fully_masked_rows():
    """A row with no allowed key (window entirely before the cache start)
    gives O = 0 and LSE = -inf."""
    q, k, v = rand(1, 6, 1, 3), rand(1, 3, 1, 3), rand(1, 3, 1, 3)
    # Sq > Sk, causal: rows i with i + (3 - 6) < 0 see nothing
    O, L = oracle.attention_fwd(q, k, v, scale=1.0, causal=True)
    assert np.all(np.isneginf(L[0, 0, :3])) and np.all(O[0, :3] == 0)
    assert np.all(np.isfinite(L[0, 0, 3:]))


def test_rows_api_matches_full():
    q, k, v = rand(1, 40, 4, 6), rand(1, 40, 2, 6), rand(1, 40, 2, 6)
    O, L = oracle.attention_fwd(q, k, v, scale=0.3, causal=True, window=(9, 0), row_chunk=7)
    rows = np.array([0, 5, 39, 22])
    o, l = oracle.attention_fwd_rows(q, k, v, 0, 3, rows, scale=0.3, causal=True, window=(9, 0))
    np.testing.assert_allclose(o, O[0, rows, 3], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l, L[0, 3, rows], rtol=1e-13)


# ---------------------------------------------------------------------------
# backward


def _loss(q, k, v, do, kw):
    O, _ = oracle.attention_fwd(q, k, v, **kw)
    return float((O * do).sum())


@pytest.mark.parametrize("kw", [
    dict(scale=0.7),
    dict(scale=0.7, causal=True),
    dict(scale=0.5, causal=True, window=(2, 0)),
    dict(scale=0.5, window=(1, 2), alibi_slopes=np.array([0.3, 0.6, 0.2, 0.9])),
    dict(scale=0.9, causal=True, softcap=1.3),
    dict(scale=0.8, causal=True, doc=True),
    dict(scale=0.6, causal=True, alibi2d=True),
])
def test_bwd_finite_differences(kw):
    """[P12] Central differences of L = sum(O * dO) in fp64 on a tiny GQA
    shape match the analytic gradients."""
    rng = np.random.default_rng(11)
    B, Sq, Sk, Hq, Hkv, D = 1, 6, 6, 4, 2, 3
    q, k, v, do = (rng.standard_normal(s) for s in
                   [(B, Sq, Hq, D), (B, Sk, Hkv, D), (B, Sk, Hkv, D), (B, Sq, Hq, D)])
    kw = dict(kw)
    if kw.pop("doc", False):
        doc = np.array([[0, 0, 1, 1, 1, 2]])
        kw.update(doc_q=doc, doc_k=doc)
    if kw.pop("alibi2d", False):
        # two batch rows with their own (B, Hq) slope rows
        B = 2
        q, k, v, do = (rng.standard_normal(s) for s in
                       [(B, Sq, Hq, D), (B, Sk, Hkv, D), (B, Sk, Hkv, D), (B, Sq, Hq, D)])
        kw["alibi_slopes"] = np.array([[0.3, 0.6, 0.2, 0.9], [1.1, 0.05, 0.7, 0.4]])
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, row_chunk=4, **kw)
    eps = 1e-6
    for x, gx in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            lp = _loss(q, k, v, do, kw)
            x[idx] = old - eps
            lm = _loss(q, k, v, do, kw)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(gx, num, rtol=1e-6, atol=1e-8)


def test_bwd_sum_identities():
    """[P13] sum_j dV[j, g] = sum_{h in g} sum_i dO_i over rows with a key.
    [P14] sum_j dK[j, g] = 0 without softcap (softmax Jacobian rows sum to
    zero; ALiBi has derivative 1 in the score), but not with softcap."""
    rng = np.random.default_rng(5)
    q, k, v, do = (rng.standard_normal(s) for s in
                   [(2, 10, 6, 4), (2, 12, 3, 4), (2, 12, 3, 4), (2, 10, 6, 4)])
    kw = dict(scale=0.5, causal=True, window=(4, 0), alibi_slopes=np.linspace(0.1, 1, 6))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, **kw)
    _, L = oracle.attention_fwd(q, k, v, **kw)
    has = np.isfinite(L)  # [B, Hq, Sq]
    for b in range(2):
        for g in range(3):
            expect = sum(do[b, has[b, h], h].sum(0) for h in (2 * g, 2 * g + 1))
            np.testing.assert_allclose(dv[b, :, g].sum(0), expect, atol=1e-12)
            np.testing.assert_allclose(dk[b, :, g].sum(0), 0.0, atol=1e-12)
    _, dk_c, _ = oracle.attention_bwd(q, k, v, do, softcap=1.0, **kw)
    assert np.abs(dk_c.sum(1)).max() > 1e-3


def test_bwd_gqa_equals_group_sum_of_mha():
    """[P15] GQA gradients of K/V are the sums over each query group of the
    MHA gradients computed on repeated K/V; dQ is unchanged."""
    rng = np.random.default_rng(6)
    q, k, v, do = (rng.standard_normal(s) for s in
                   [(1, 7, 8, 3), (1, 9, 2, 3), (1, 9, 2, 3), (1, 7, 8, 3)])
    kw = dict(scale=0.7, causal=True, softcap=2.0)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, **kw)
    dq2, dk2, dv2 = oracle.attention_bwd(q, np.repeat(k, 4, 2), np.repeat(v, 4, 2), do, **kw)
    np.testing.assert_allclose(dq, dq2, atol=1e-14)
    np.testing.assert_allclose(dk, dk2.reshape(1, 9, 2, 4, 3).sum(3), atol=1e-14)
    np.testing.assert_allclose(dv, dv2.reshape(1, 9, 2, 4, 3).sum(3), atol=1e-14)


def test_bwd_documents_are_independent():
    """[P16] With a document mask (causal inside each document, [GYM] packed
    sequences), the gradients of a packed sequence are the gradients of each
    document run on its own: the slices are concatenated and compared."""
    rng = np.random.default_rng(12)
    lens = inputs.doc_lengths(rng, 160, 10, 60)
    doc = inputs.doc_ids(lens)[None]
    S, Hq, Hkv, D = 160, 4, 2, 8
    q, k, v, do = (rng.standard_normal(s) for s in
                   [(1, S, Hq, D), (1, S, Hkv, D), (1, S, Hkv, D), (1, S, Hq, D)])
    kw = dict(scale=0.6, softcap=2.5)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, causal=True, doc_q=doc, doc_k=doc, **kw)
    s0 = 0
    for n in lens:
        sl = slice(s0, s0 + n)
        eq, ek, ev = oracle.attention_bwd(q[:, sl], k[:, sl], v[:, sl], do[:, sl], causal=True, **kw)
        np.testing.assert_allclose(dq[:, sl], eq, atol=1e-13)
        np.testing.assert_allclose(dk[:, sl], ek, atol=1e-13)
        np.testing.assert_allclose(dv[:, sl], ev, atol=1e-13)
        s0 += n
    assert s0 == S and len(lens) > 2


def test_bwd_delta_identity():
    """Delta_i = sum_j P_ij dP_ij equals <dO_i, O_i> (the form a kernel
    uses); checked through dQ of a case whose O is known."""
    rng = np.random.default_rng(8)
    q, k, v, do = (rng.standard_normal(s) for s in
                   [(1, 5, 1, 3), (1, 5, 1, 3), (1, 5, 1, 3), (1, 5, 1, 3)])
    O, L = oracle.attention_fwd(q, k, v, scale=0.5, causal=True)
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale=0.5, causal=True)
    # recompute dQ with Delta = <dO, O> by brute force loops
    for i in range(5):
        delta = float(do[0, i, 0] @ O[0, i, 0])
        acc = np.zeros(3)
        for j in range(i + 1):
            p = math.exp(0.5 * float(q[0, i, 0] @ k[0, j, 0]) - L[0, 0, i])
            dp = float(do[0, i, 0] @ v[0, j, 0])
            acc += 0.5 * p * (dp - delta) * k[0, j, 0]
        np.testing.assert_allclose(dq[0, i, 0], acc, atol=1e-13)


# ---------------------------------------------------------------------------
# decode


def test_decode_single_token_cache():
    """[P19] cache length 1: O = v_0 of that batch row."""
    q = rand(3, 1, 4, 8)
    kc, vc = rand(3, 16, 1, 8), rand(3, 16, 1, 8)
    O, L = oracle.decode(q, kc, vc, np.array([1, 1, 1]))
    for b in range(3):
        np.testing.assert_allclose(O[b, 0], np.broadcast_to(vc[b, 0, 0], (4, 8)), atol=1e-15)


def test_decode_equals_forward_over_prefix_and_split():
    """[P20] Split-K (any chunk length) then LSE-weighted combine equals the
    unsplit result to ~1e-15; [P21] MQA equals MHA on repeated K/V."""
    rng = np.random.default_rng(9)
    q = rng.standard_normal((4, 1, 8, 6))
    kc, vc = rng.standard_normal((4, 50, 1, 6)), rng.standard_normal((4, 50, 1, 6))
    lens = np.array([50, 1, 17, 33])
    O, L = oracle.decode(q, kc, vc, lens, scale=0.4)
    for split in (1, 7, 16, 64):
        Os, Ls = oracle.decode_split(q, kc, vc, lens, split, scale=0.4)
        np.testing.assert_allclose(Os, O, atol=2e-15)
        np.testing.assert_allclose(Ls, L, atol=2e-15)
    Om, Lm = oracle.decode(q, np.repeat(kc, 8, 2), np.repeat(vc, 8, 2), lens, scale=0.4)
    np.testing.assert_allclose(Om, O, atol=1e-15)
    # brute force on one batch row
    Ob, Lb = brute_fwd(q[2:3], kc[2:3, :17], vc[2:3, :17], 0.4)
    np.testing.assert_allclose(O[2:3], Ob, atol=1e-13)
    np.testing.assert_allclose(L[2:3], Lb, atol=1e-13)


def test_combine_partials_algebra():
    """Merging is exact for a two-way split computed by hand, ignores empty
    parts, and does not depend on the order of the parts."""
    rng = np.random.default_rng(10)
    u = rng.standard_normal(9)
    v = rng.standard_normal((9, 3))
    parts = [(0, 4), (4, 4), (4, 9)]  # the middle part is empty
    os_, ls = [], []
    for a, b in parts:
        if a == b:
            os_.append(np.zeros(3))
            ls.append(-np.inf)
            continue
        w = scipy.special.softmax(u[a:b])
        os_.append(w @ v[a:b])
        ls.append(scipy.special.logsumexp(u[a:b]))
    O, L = oracle.combine_partials(np.array(os_), np.array(ls))
    np.testing.assert_allclose(L, scipy.special.logsumexp(u), rtol=1e-15)
    np.testing.assert_allclose(O, scipy.special.softmax(u) @ v, atol=1e-15)
    O2, L2 = oracle.combine_partials(np.array(os_[::-1]), np.array(ls[::-1]))
    np.testing.assert_allclose(O2, O, atol=1e-15)
    Oe, Le = oracle.combine_partials(np.zeros((2, 3)), np.array([-np.inf, -np.inf]))
    assert np.isneginf(Le) and np.all(Oe == 0)


# ---------------------------------------------------------------------------
# block masks and unmasked fractions


def test_block_mask_causal_square():
    """[P16] Causal, square aligned tiles: diagonal PARTIAL, below FULL,
    above EMPTY.  At S = 2048 with 128 x 128 tiles that is 120 / 16 / 120."""
    bm = oracle.block_mask(1, 2048, 2048, 128, 128, causal=True)
    c = bm["cls"][0]
    n = 16
    expect = np.zeros((n, n), dtype=np.uint8)
    expect[np.tril_indices(n, -1)] = 2
    expect[np.diag_indices(n)] = 1
    np.testing.assert_array_equal(c, expect)
    assert [(c == x).sum() for x in (0, 1, 2)] == [120, 16, 120]


def _window_tiles_closed_form(S, left, bs):
    """Tile classes for causal + window (left, 0), square tiles of size bs,
    S a multiple of bs, left a multiple of bs: row block r has FULL tiles
    max(0, r - left/bs + 1) .. r - 1, PARTIAL tiles r and r - left/bs (if >= 0),
    EMPTY otherwise."""
    n = S // bs
    w = left // bs
    cls = np.zeros((n, n), dtype=np.uint8)
    for r in range(n):
        for c in range(max(0, r - w + 1), r):
            cls[r, c] = 2
        cls[r, r] = 1
        if r - w >= 0:
            cls[r, r - w] = 1
    return cls


def test_block_mask_window_closed_form():
    """[P17] Causal + window (4096, 0) at S = 16384, 128 x 128 tiles:
    12688 / 224 / 3472 empty / partial / full, matching the closed form
    (31 full + 2 partial tiles per row block once the window is saturated)."""
    bm = oracle.block_mask(1, 16384, 16384, 128, 128, causal=True, window=(4096, 0))
    c = bm["cls"][0]
    np.testing.assert_array_equal(c, _window_tiles_closed_form(16384, 4096, 128))
    assert [(c == x).sum() for x in (0, 1, 2)] == [12688, 224, 3472]


def test_block_mask_lists_and_ragged_edges():
    """CSR lists hold ascending indices of each class with a zero tail; the
    transposed lists are the same sets by column; a tile that crosses the end
    of the sequence is never FULL."""
    bm = oracle.block_mask(1, 100, 70, 32, 16, causal=False)
    c = bm["cls"][0]
    assert c.shape == (4, 5)
    assert np.all(c[:3, :4] == 2) and np.all(c[3] == 1) and np.all(c[:, 4] == 1)
    for name, val in (("partial", 1), ("full", 2)):
        for qb in range(4):
            hits = np.nonzero(c[qb] == val)[0]
            n = bm["kv_num_" + name][0, qb]
            assert n == len(hits)
            np.testing.assert_array_equal(bm["kv_idx_" + name][0, qb, :n], hits)
            assert np.all(bm["kv_idx_" + name][0, qb, n:] == 0)
        for kb in range(5):
            hits = np.nonzero(c[:, kb] == val)[0]
            n = bm["q_num_" + name][0, kb]
            np.testing.assert_array_equal(bm["q_idx_" + name][0, kb, :n], hits)
            assert np.all(bm["q_idx_" + name][0, kb, n:] == 0)


def test_block_mask_documents():
    """[P18] Document + causal mask: the allowed pairs total
    sum_docs L (L + 1) / 2, FULL tiles contain no disallowed pair, EMPTY tiles
    contain no allowed pair, and PARTIAL tiles contain both."""
    rng = np.random.default_rng(4)
    S, bs = 2048, 128
    lens = inputs.doc_lengths(rng, S, 100, 700)
    doc = inputs.doc_ids(lens)[None]
    assert oracle.allowed_pair_count(S, S, causal=True, doc_q=doc[0], doc_k=doc[0]) == \
        sum(n * (n + 1) // 2 for n in lens)
    bm = oracle.block_mask(1, S, S, bs, bs, causal=True, doc_q=doc, doc_k=doc)
    i = np.arange(S)
    ok = (doc[0][:, None] == doc[0][None, :]) & (i[None, :] <= i[:, None])
    for qb in range(S // bs):
        for kb in range(S // bs):
            t = ok[qb * bs:(qb + 1) * bs, kb * bs:(kb + 1) * bs]
            expect = 0 if not t.any() else (2 if t.all() else 1)
            assert bm["cls"][0, qb, kb] == expect


def test_unmasked_fractions():
    """[P22] causal: S (S + 1) / 2 pairs; [P23] causal + window (4096, 0) at
    S = 16384: sum_i (min(i, 4096) + 1) = 58,734,592 pairs."""
    assert oracle.allowed_pair_count(2048, 2048, causal=True) == 2048 * 2049 // 2
    n = oracle.allowed_pair_count(16384, 16384, causal=True, window=(4096, 0), row_chunk=2048)
    # rows i < 4096 see i + 1 keys, later rows see 4097
    assert n == 4096 * 4097 // 2 + (16384 - 4096) * 4097 == 58734592


@pytest.mark.parametrize("L", [0, 1, 5, 8, 9, 12])
def test_cache_length_predicate_counts(L):
    """The cache-length term of the predicate ([FA] "Examples",
    cache_seqlens: only the first L cached rows are attended): every row of
    a non-causal Sq x Sk problem sees exactly min(L, Sk) keys, namely keys
    0 .. min(L, Sk) - 1; with causal (bottom-right) row i sees
    min(L, i + Sk - Sq + 1) keys."""
    Sq, Sk = 4, 9
    ok = oracle.allowed_mask(np.arange(Sq), np.arange(Sk), Sq, Sk, kv_len=L)
    assert np.array_equal(ok.sum(1), np.full(Sq, min(L, Sk)))
    assert np.array_equal(np.nonzero(ok[0])[0], np.arange(min(L, Sk)))
    assert oracle.allowed_pair_count(Sq, Sk, kv_len=L) == Sq * min(L, Sk)
    okc = oracle.allowed_mask(np.arange(Sq), np.arange(Sk), Sq, Sk, causal=True, kv_len=L)
    for i in range(Sq):
        assert okc[i].sum() == max(0, min(L, i + Sk - Sq + 1))


def test_seeded_workload_side_data():
    """The packed-document and cache-length draws are reproducible (values
    produced by this generator, kept as a regression check of it)."""
    rng = np.random.default_rng(4)
    assert inputs.doc_lengths(rng, 8192) == [1558, 1946, 1836, 1172, 1680]
    assert inputs.doc_lengths(rng, 8192) == [2006, 1995, 400, 1069, 1344, 763, 615]
    lens = np.random.default_rng(5).integers(1024, 8192, size=32, endpoint=True)
    assert int(lens.sum()) == 138534


def test_f16_rounding_helpers():
    """IEEE half: 11 significant bits, ties to even, max 65504."""
    x = np.array([1.0, 1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, -2.5, 65504.0, 2.0 ** -24], dtype=np.float32)
    bits = inputs.f32_to_f16_bits(x)
    back = inputs.f16_bits_to_f64(bits)
    np.testing.assert_array_equal(back, [1.0, 1.0, 1.0 + 2.0 ** -9, -2.5, 65504.0, 2.0 ** -24])
    assert bits[0] == 0x3C00 and bits[3] == 0xC100


def test_bf16_rounding_helpers():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.5, 3.0e38, 1e-40], dtype=np.float32)
    bits = inputs.f32_to_bf16_bits(x)
    back = inputs.bf16_bits_to_f32(bits)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 1.5*2^-8 rounds up
    np.testing.assert_array_equal(back[:4], np.array([1.0, 1.0, 1.0078125, -2.5], dtype=np.float32))
    normal = np.abs(x) > 1e-37
    assert np.all(np.abs(back - x)[normal] <= np.abs(x)[normal] * 2.0 ** -8)


# ---------------------------------------------------------------------------
# several queries per sequence over a cache (chunked prefill, speculative
# decoding): [FA] "Examples" lets q of flash_attn_with_kvcache hold seqlen
# queries; with causal they are the last positions of the sequence.

def test_decode_multi_query_causal_rows_are_single_token_decodes():
    """[P22] Row t of a causal Sq-query decode over L keys equals the
    single-query decode of q_t over the first L - Sq + 1 + t keys (its own
    position); without causal every row sees all L keys.  Rows with no key
    (L < Sq) give O = 0, LSE = -inf."""
    rng = np.random.default_rng(31)
    B, Sq, Hq, Hkv, D, Smax = 4, 5, 6, 2, 8, 40
    q = rng.standard_normal((B, Sq, Hq, D))
    kc, vc = rng.standard_normal((B, Smax, Hkv, D)), rng.standard_normal((B, Smax, Hkv, D))
    lens = np.array([40, 5, 3, 17])
    O, L = oracle.decode(q, kc, vc, lens, scale=0.3, softcap=2.0, causal=True)
    On, Ln = oracle.decode(q, kc, vc, lens, scale=0.3, softcap=2.0)
    for t in range(Sq):
        own = np.maximum(lens - Sq + 1 + t, 0)
        O1, L1 = oracle.decode(q[:, t:t + 1], kc, vc, own, scale=0.3, softcap=2.0)
        np.testing.assert_allclose(O[:, t], O1[:, 0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(L[:, :, t], L1[:, :, 0], rtol=0, atol=1e-13)
        O2, L2 = oracle.decode(q[:, t:t + 1], kc, vc, lens, scale=0.3, softcap=2.0)
        np.testing.assert_allclose(On[:, t], O2[:, 0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(Ln[:, :, t], L2[:, :, 0], rtol=0, atol=1e-13)
    assert np.isneginf(L[2, :, :2]).all() and (O[2, :2] == 0).all()
    assert np.isfinite(L[2, :, 2:]).all()


def test_decode_multi_query_causal_brute_force():
    """[P23] Causal multi-query decode against pure-Python loops with exact
    sums (bottom-right causal predicate j <= i + L - Sq)."""
    rng = np.random.default_rng(32)
    B, Sq, Hq, Hkv, D, Smax = 2, 3, 4, 1, 5, 12
    q = rng.standard_normal((B, Sq, Hq, D))
    kc, vc = rng.standard_normal((B, Smax, Hkv, D)), rng.standard_normal((B, Smax, Hkv, D))
    lens = np.array([12, 7])
    O, L = oracle.decode(q, kc, vc, lens, scale=0.45, causal=True)
    for b in range(B):
        n = lens[b]
        Ob, Lb = brute_fwd(q[b:b + 1], kc[b:b + 1, :n], vc[b:b + 1, :n], 0.45, causal=True)
        np.testing.assert_allclose(O[b:b + 1], Ob, atol=1e-13)
        np.testing.assert_allclose(L[b:b + 1], Lb, atol=1e-13)


def test_decode_kvcache_speculative_append():
    """[P24] Appending S_new draft tokens and attending them causally equals a
    causal decode over the explicitly concatenated rows, and the last draft
    row equals an ordinary one-token decode over all rows."""
    rng = np.random.default_rng(33)
    B, S_new, Hq, Hkv, D, Smax = 3, 4, 4, 2, 6, 32
    q = rng.standard_normal((B, S_new, Hq, D))
    kc, vc = rng.standard_normal((B, Smax, Hkv, D)), rng.standard_normal((B, Smax, Hkv, D))
    kn, vn = rng.standard_normal((B, S_new, Hkv, D)), rng.standard_normal((B, S_new, Hkv, D))
    lens = np.array([0, 9, 28])
    O, L, _ = oracle.decode_kvcache(q, kc, vc, lens, k_new=kn, v_new=vn, scale=0.4, causal=True)
    cat_k, cat_v = np.zeros_like(kc), np.zeros_like(vc)
    for b in range(B):
        n = lens[b]
        cat_k[b, :n], cat_v[b, :n] = kc[b, :n], vc[b, :n]
        cat_k[b, n:n + S_new], cat_v[b, n:n + S_new] = kn[b], vn[b]
    for b in range(B):
        n = lens[b] + S_new
        Ob, Lb = brute_fwd(q[b:b + 1], cat_k[b:b + 1, :n], cat_v[b:b + 1, :n], 0.4, causal=True)
        np.testing.assert_allclose(O[b:b + 1], Ob, atol=1e-13)
        np.testing.assert_allclose(L[b:b + 1], Lb, atol=1e-13)
    O1, L1 = oracle.decode(q[:, -1:], cat_k, cat_v, lens + S_new, scale=0.4)
    np.testing.assert_allclose(O[:, -1], O1[:, 0], rtol=0, atol=1e-13)
