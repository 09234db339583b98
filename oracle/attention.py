"""fp64 reference definitions of exact attention (test infrastructure only).

Source tags ([TA], [FA], [HF], [GYM], [FX4]) are the web pages listed in
``oracle/__init__.py``.

Layouts follow the repository overview's problem statement for
``flash_attn_func`` ([FA], "Examples"): q is [B, Sq, Hq, D], k and v are
[B, Sk, Hkv, D], the output is [B, Sq, Hq, D].  The per-row log-sum-exp is
returned as [B, Hq, Sq] in natural-log units.

Definition computed, for batch b, query head h, query row i and key j, with
g = kv head of h and delta = Sk - Sq (the last query row is aligned with the
last key):

  s_ij = scale * <q_i, k_j>                        (scaled scores)
  t_ij = c * tanh(s_ij / c)  if softcap c > 0      (tanh softcap)
  u_ij = t_ij - slope_h * |i + delta - j|          (ALiBi bias, if given)
  allowed_ij = causal/window/document/length predicate
  LSE_i = log sum_{allowed j} exp(u_ij)            (-inf if nothing allowed)
  P_ij  = exp(u_ij - LSE_i) on allowed pairs, else 0
  O_i   = sum_j P_ij v_j                           (0 if nothing allowed)

[TA] "Key-Value Attention" gives the three steps (scores, softmax, weighted
sum of values); [FA] "Examples" says the softmax scale multiplies QK^T before
the softmax; [FX4] describes score modifications (ALiBi, softcapping) and mask
patterns (causal, sliding window) as pointwise hooks on that score.  Where
the pages are silent the readings used are: scale first, then softcap, then
the ALiBi bias; the ALiBi distance is |i + delta - j|; window bounds are
inclusive; causal and window are bottom-right aligned; a row with no allowed
key has O = 0 and LSE = -inf.

The row loops compute a few hundred rows at a time so the full Sq x Sk score
matrix is never held; for each row chunk the candidate keys are cut to the
range where the causal/window/length predicate can hold (pairs outside it
contribute exactly 0, and the tests check this against unrestricted brute
force).
"""

import numpy as np

_NEG_INF = -np.inf


def kv_head_of(h, Hq, Hkv):
    """Key/value head read by query head ``h``.

    [HF]: ``repeat_kv`` is documented as ``repeat_interleave`` over the head
    dimension with ``n_rep = Hq // Hkv`` copies of each kv head, so query head
    h sees kv head ``h // n_rep`` (grouped-query attention; Hkv == 1 is
    multi-query attention, [FA] "Examples").
    """
    if Hkv <= 0 or Hq % Hkv != 0:
        raise ValueError("Hq must be a positive multiple of Hkv")
    return h // (Hq // Hkv)


def allowed_mask(rows, cols, Sq, Sk, causal=False, window=(-1, -1),
                 doc_q=None, doc_k=None, kv_len=None):
    """Boolean matrix [len(rows), len(cols)]: may query ``i`` attend key ``j``.

    [GYM] defines the causal mask_mod as ``q_idx >= kv_idx``; [FA] "Examples"
    gives ``causal`` and ``window_size=(left, right)`` with -1 meaning no
    limit; [FX4] names causal and sliding-window masks as mask patterns.  With
    delta = Sk - Sq the conditions are

      causal:      j <= i + delta
      window left: j >= i + delta - left     (left >= 0)
      window right: j <= i + delta + right   (right >= 0)
      document:    doc_q[i] == doc_k[j]      (doc ids of one batch row)
      length:      j < kv_len                (valid prefix of a KV cache)

    and a pair is allowed when every given condition holds.
    """
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.asarray(cols, dtype=np.int64)[None, :]
    delta = Sk - Sq
    ok = (j >= 0) & (j < Sk) & (i >= 0) & (i < Sq)
    if causal:
        ok &= j <= i + delta
    left, right = window
    if left >= 0:
        ok &= j >= i + delta - left
    if right >= 0:
        ok &= j <= i + delta + right
    if doc_q is not None:
        dq = np.asarray(doc_q)[np.asarray(rows, dtype=np.int64)]
        dk = np.asarray(doc_k)[np.asarray(cols, dtype=np.int64)]
        ok &= dq[:, None] == dk[None, :]
    if kv_len is not None:
        ok &= j < kv_len
    return ok


def _key_range(rows, Sq, Sk, causal, window, kv_len):
    """Smallest [lo, hi) holding every key any of ``rows`` may attend.

    Keys outside it fail the causal/window/length predicate for every row of
    the chunk, so their terms are exactly 0."""
    delta = Sk - Sq
    lo, hi = 0, Sk
    rmin, rmax = int(np.min(rows)), int(np.max(rows))
    if causal:
        hi = min(hi, rmax + delta + 1)
    left, right = window
    if right >= 0:
        hi = min(hi, rmax + delta + right + 1)
    if left >= 0:
        lo = max(lo, rmin + delta - left)
    if kv_len is not None:
        hi = min(hi, int(kv_len))
    return lo, max(lo, hi)


def _slope(alibi_slopes, b, h):
    if alibi_slopes is None:
        return None
    a = np.asarray(alibi_slopes, dtype=np.float64)
    return float(a[h]) if a.ndim == 1 else float(a[b, h])


def _scores(q_rows, k_cols, rows, cols, Sq, Sk, scale, softcap, slope):
    """Steps 1-3 of the definition: scaled scores s and modified scores u."""
    s = scale * (q_rows @ k_cols.T)
    if softcap > 0:
        t = softcap * np.tanh(s / softcap)
    else:
        t = s
    if slope is not None:
        dist = np.abs(rows[:, None] + (Sk - Sq) - cols[None, :]).astype(np.float64)
        u = t - slope * dist
    else:
        u = t
    return s, u


def _probabilities(u, ok):
    """Softmax over the allowed entries of each row ([TA] "Key-Value
    Attention": the scores are turned into probabilities with a softmax).

    Returns P (zero on masked pairs and on rows with nothing allowed) and the
    row log-sum-exp (-inf on such rows).  The row maximum is subtracted
    before exponentiating, the usual stable form of the same quantity."""
    has = ok.any(axis=1)
    um = np.where(ok, u, _NEG_INF)
    m = np.where(has, um.max(axis=1), 0.0)
    e = np.where(ok, np.exp(np.where(ok, u, 0.0) - m[:, None]), 0.0)
    tot = e.sum(axis=1)
    safe = np.where(has, tot, 1.0)
    lse = np.where(has, m + np.log(safe), _NEG_INF)
    P = e / safe[:, None]
    return P, lse


def attention_fwd_rows(q, k, v, b, h, rows, scale=None, causal=False,
                       window=(-1, -1), alibi_slopes=None, softcap=0.0,
                       doc_q=None, doc_k=None, kv_len=None):
    """O [len(rows), D] and LSE [len(rows)] for query rows ``rows`` of
    batch ``b``, query head ``h`` (see the module docstring)."""
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    rows = np.asarray(rows, dtype=np.int64)
    g = kv_head_of(h, Hq, Hkv)
    lo, hi = _key_range(rows, Sq, Sk, causal, window, kv_len)
    cols = np.arange(lo, hi, dtype=np.int64)
    O = np.zeros((len(rows), v.shape[3]), dtype=np.float64)
    lse = np.full(len(rows), _NEG_INF)
    if len(cols) == 0:
        return O, lse
    q_rows = np.asarray(q[b, rows, h, :], dtype=np.float64)
    k_cols = np.asarray(k[b, lo:hi, g, :], dtype=np.float64)
    v_cols = np.asarray(v[b, lo:hi, g, :], dtype=np.float64)
    _, u = _scores(q_rows, k_cols, rows, cols, Sq, Sk, scale, softcap,
                   _slope(alibi_slopes, b, h))
    ok = allowed_mask(rows, cols, Sq, Sk, causal, window,
                      None if doc_q is None else doc_q[b],
                      None if doc_k is None else doc_k[b], kv_len)
    P, lse = _probabilities(u, ok)
    # [TA] "3. Weighted Sum of Values": each query's output is the
    # probability-weighted sum of the value vectors.
    O = P @ v_cols
    return O, lse


def attention_fwd(q, k, v, scale=None, causal=False, window=(-1, -1),
                  alibi_slopes=None, softcap=0.0, doc_q=None, doc_k=None,
                  kv_len=None, row_chunk=512):
    """Full forward: O [B, Sq, Hq, D] and LSE [B, Hq, Sq] (fp64)."""
    B, Sq, Hq, D = q.shape
    O = np.zeros((B, Sq, Hq, v.shape[3]), dtype=np.float64)
    LSE = np.full((B, Hq, Sq), _NEG_INF)
    for b in range(B):
        for h in range(Hq):
            for r0 in range(0, Sq, row_chunk):
                rows = np.arange(r0, min(Sq, r0 + row_chunk))
                o, l = attention_fwd_rows(q, k, v, b, h, rows, scale, causal,
                                          window, alibi_slopes, softcap,
                                          doc_q, doc_k, kv_len)
                O[b, rows, h, :] = o
                LSE[b, h, rows] = l
    return O, LSE


def attention_bwd(q, k, v, do, scale=None, causal=False, window=(-1, -1),
                  alibi_slopes=None, softcap=0.0, doc_q=None, doc_k=None,
                  row_chunk=512):
    """Gradients dQ, dK, dV of the scalar sum(O * dO), all fp64.

    Obtained by the chain rule through the definition in the module
    docstring ([FX4] says the backward reuses the forward's machinery; the
    steps below are the plain derivative):

      dV_j   = sum_i P_ij dO_i
      dP_ij  = <dO_i, v_j>
      Delta_i = sum_j P_ij dP_ij
      dU_ij  = P_ij (dP_ij - Delta_i)               (softmax Jacobian)
      dS_ij  = dU_ij * (1 - tanh(s_ij / c)^2)        (softcap c > 0; else dU)
      dQ_i   = scale * sum_j dS_ij k_j
      dK_j   = scale * sum_i dS_ij q_i

    The ALiBi bias does not depend on q, k or v.  dK and dV of a kv head sum
    the contributions of every query head that reads it (the gradient of
    repeat_interleave, [HF]).  Delta is formed as sum_j P dP here, not as
    <dO_i, O_i>; the two are equal.
    """
    B, Sq, Hq, D = q.shape
    _, Sk, Hkv, _ = k.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            slope = _slope(alibi_slopes, b, h)
            for r0 in range(0, Sq, row_chunk):
                rows = np.arange(r0, min(Sq, r0 + row_chunk))
                lo, hi = _key_range(rows, Sq, Sk, causal, window, None)
                if hi <= lo:
                    continue
                cols = np.arange(lo, hi)
                q_rows = np.asarray(q[b, rows, h, :], dtype=np.float64)
                do_rows = np.asarray(do[b, rows, h, :], dtype=np.float64)
                k_cols = np.asarray(k[b, lo:hi, g, :], dtype=np.float64)
                v_cols = np.asarray(v[b, lo:hi, g, :], dtype=np.float64)
                s, u = _scores(q_rows, k_cols, rows, cols, Sq, Sk, scale,
                               softcap, slope)
                ok = allowed_mask(rows, cols, Sq, Sk, causal, window,
                                  None if doc_q is None else doc_q[b],
                                  None if doc_k is None else doc_k[b])
                P, _ = _probabilities(u, ok)
                dv[b, lo:hi, g, :] += P.T @ do_rows
                dP = do_rows @ v_cols.T
                delta = (P * dP).sum(axis=1)
                dU = P * (dP - delta[:, None])
                if softcap > 0:
                    dS = dU * (1.0 - np.tanh(s / softcap) ** 2)
                else:
                    dS = dU
                dq[b, rows, h, :] = scale * (dS @ k_cols)
                dk[b, lo:hi, g, :] += scale * (dS.T @ q_rows)
    return dq, dk, dv


def decode(q, k_cache, v_cache, cache_seqlens, scale=None, softcap=0.0,
           alibi_slopes=None, window=(-1, -1), causal=False):
    """Attention of new queries over a KV cache ([FA] "Examples",
    ``flash_attn_with_kvcache``): q [B, Sq, Hq, D] attends to the first
    ``cache_seqlens[b]`` rows of k_cache/v_cache [B, Smax, Hkv, D] of its own
    batch row.  The queries are the last Sq positions (bottom-right aligned,
    the forward's convention for Sq != Sk), so with ``causal`` query t sees the
    first cache_seqlens[b] - Sq + 1 + t rows, and for Sq == 1 causal masking
    changes nothing.  This is the forward definition with
    Sk = cache_seqlens[b]; it is computed unsplit.

    Returns O [B, Sq, Hq, D] and LSE [B, Hq, Sq]."""
    B, Sq, Hq, D = q.shape
    O = np.zeros((B, Sq, Hq, v_cache.shape[3]), dtype=np.float64)
    LSE = np.full((B, Hq, Sq), _NEG_INF)
    for b in range(B):
        L = int(cache_seqlens[b])
        if L <= 0:
            continue
        slopes = alibi_slopes
        if slopes is not None and np.asarray(slopes).ndim == 2:
            slopes = np.asarray(slopes)[b:b + 1]
        o, l = attention_fwd(q[b:b + 1], k_cache[b:b + 1, :L],
                             v_cache[b:b + 1, :L], scale=scale,
                             causal=causal, window=window, softcap=softcap,
                             alibi_slopes=slopes)
        O[b] = o[0]
        LSE[b] = l[0]
    return O, LSE


def combine_partials(o_parts, lse_parts):
    """Merge attention results computed over disjoint key subsets.

    With partial results (O_s, LSE_s) over key sets K_s that partition the
    keys, the softmax over the union gives LSE = log sum_s exp(LSE_s) and
    O = sum_s exp(LSE_s - LSE) O_s: each partial output is an average under
    its own normaliser, reweighted by its share of the total.  This is the
    "intermediate results are stored ... build up the final result
    incrementally" step of [TA] "2. Online Softmax", applied to whole chunks.

    o_parts [n, ..., D], lse_parts [n, ...]; parts with LSE = -inf (empty key
    sets) get weight 0.  Returns (O [..., D], LSE [...])."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    has = np.isfinite(lse_parts)
    m = np.where(has, lse_parts, _NEG_INF).max(axis=0)
    any_ = np.isfinite(m)
    m_safe = np.where(any_, m, 0.0)
    w = np.where(has, np.exp(np.where(has, lse_parts, 0.0) - m_safe), 0.0)
    tot = w.sum(axis=0)
    safe = np.where(any_, tot, 1.0)
    lse = np.where(any_, m_safe + np.log(safe), _NEG_INF)
    O = (w[..., None] * o_parts).sum(axis=0) / safe[..., None]
    return O, lse


def decode_split(q, k_cache, v_cache, cache_seqlens, split_len, scale=None,
                 softcap=0.0):
    """Decode computed split-K style: each batch row's cache prefix is cut
    into consecutive chunks of ``split_len`` keys, each chunk is attended on
    its own (forward definition restricted to that chunk), and the chunk
    results are merged with ``combine_partials``.  Equal to ``decode`` up to
    rounding; used to check the merge algebra."""
    B, Sq, Hq, D = q.shape
    O = np.zeros((B, Sq, Hq, v_cache.shape[3]), dtype=np.float64)
    LSE = np.full((B, Hq, Sq), _NEG_INF)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    for b in range(B):
        L = int(cache_seqlens[b])
        parts_o, parts_l = [], []
        for j0 in range(0, L, split_len):
            j1 = min(L, j0 + split_len)
            o, l = attention_fwd(q[b:b + 1], k_cache[b:b + 1, j0:j1],
                                 v_cache[b:b + 1, j0:j1], scale=scale,
                                 softcap=softcap)
            parts_o.append(o[0])                 # [Sq, Hq, D]
            parts_l.append(l[0].T)               # [Sq, Hq]
        if parts_o:
            o, l = combine_partials(np.stack(parts_o), np.stack(parts_l))
            O[b] = o
            LSE[b] = l.T
    return O, LSE


EMPTY, PARTIAL, FULL = 0, 1, 2


def block_mask(B, Sq, Sk, block_m, block_n, causal=False, window=(-1, -1),
               doc_q=None, doc_k=None):
    """Block-sparse mask: classify every (block_m x block_n) tile.

    [GYM] builds a block mask from a mask_mod with ``create_block_mask`` and a
    block size; [FX4] describes block-sparse iteration in which tiles with no
    allowed pair are skipped.  A tile is EMPTY (0) when no pair in it is
    allowed, FULL (2) when it lies wholly inside [0, Sq) x [0, Sk) and every
    pair is allowed, PARTIAL (1) otherwise.  The predicate is evaluated on
    every pair by brute force.  The mask patterns here do not depend on the
    head, so one mask serves all heads.

    Returns a dict of int arrays:
      cls             uint8 [B, nQ, nK]
      kv_num_partial, kv_num_full   int32 [B, nQ]
      kv_idx_partial, kv_idx_full   int32 [B, nQ, nK]  ascending kv-block
                      indices of that class, unused tail 0
      q_num_partial, q_num_full     int32 [B, nK]
      q_idx_partial, q_idx_full     int32 [B, nK, nQ]  ascending q-block
                      indices (the transposed lists), unused tail 0
    """
    nQ = -(-Sq // block_m)
    nK = -(-Sk // block_n)
    cls = np.zeros((B, nQ, nK), dtype=np.uint8)
    cols = np.arange(Sk)
    for b in range(B):
        for qb in range(nQ):
            rows = np.arange(qb * block_m, min(Sq, (qb + 1) * block_m))
            ok = allowed_mask(rows, cols, Sq, Sk, causal, window,
                              None if doc_q is None else doc_q[b],
                              None if doc_k is None else doc_k[b])
            for kb in range(nK):
                tile = ok[:, kb * block_n:(kb + 1) * block_n]
                inside = tile.shape == (block_m, block_n)
                if not tile.any():
                    cls[b, qb, kb] = EMPTY
                elif inside and tile.all():
                    cls[b, qb, kb] = FULL
                else:
                    cls[b, qb, kb] = PARTIAL
    out = {"cls": cls}
    for name, c in (("partial", PARTIAL), ("full", FULL)):
        kv_num = np.zeros((B, nQ), dtype=np.int32)
        kv_idx = np.zeros((B, nQ, nK), dtype=np.int32)
        q_num = np.zeros((B, nK), dtype=np.int32)
        q_idx = np.zeros((B, nK, nQ), dtype=np.int32)
        for b in range(B):
            for qb in range(nQ):
                hits = np.nonzero(cls[b, qb] == c)[0]
                kv_num[b, qb] = len(hits)
                kv_idx[b, qb, :len(hits)] = hits
            for kb in range(nK):
                hits = np.nonzero(cls[b, :, kb] == c)[0]
                q_num[b, kb] = len(hits)
                q_idx[b, kb, :len(hits)] = hits
        out["kv_num_" + name] = kv_num
        out["kv_idx_" + name] = kv_idx
        out["q_num_" + name] = q_num
        out["q_idx_" + name] = q_idx
    return out


def allowed_pair_count(Sq, Sk, causal=False, window=(-1, -1), doc_q=None,
                       doc_k=None, kv_len=None, row_chunk=1024):
    """Number of allowed (i, j) pairs of one batch row, by brute force over
    the predicate (``doc_q``/``doc_k`` are that row's document ids)."""
    total = 0
    cols = np.arange(Sk)
    for r0 in range(0, Sq, row_chunk):
        rows = np.arange(r0, min(Sq, r0 + row_chunk))
        total += int(allowed_mask(rows, cols, Sq, Sk, causal, window,
                                  doc_q, doc_k, kv_len).sum())
    return total
