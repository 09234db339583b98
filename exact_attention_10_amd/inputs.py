"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random numbers and stores them; it holds none of the
attention arithmetic.  Every workload draws from
``numpy.random.default_rng(seed)`` (PCG64) in a fixed order: integer side
data first (document lengths, cache lengths), then q, k, v, then the output
gradient dO, each as float32 standard normals.  bf16 workloads round those
float32 draws to bfloat16 (round to nearest, ties to even) and keep the raw
16-bit patterns (fp16 workloads likewise round to IEEE half); both the GPU path and the fp64 CPU check consume exactly
those patterns.

The shapes are those of the pages' workloads: Llama-3.1-8B attention (32
query heads, 8 kv heads, head dim 128, sequence 2048) as trained in the
attention-gym FlexAttention memory report, a long-context sliding-window
variant of it, packed-document masking (FlexAttention document masks), and
a 128-query-head / 1-kv-head decode over a KV cache (the DeepSeek-style head
shape in the transformers attention_forward discussion).  No dataset is
involved.
"""

import numpy as np

# ---------------------------------------------------------------------------
# bf16 storage helpers (bit manipulation only)


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16, nearest-even; returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Exact widening of bfloat16 bit patterns to float32."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def f32_to_f16_bits(x):
    """Round float32 values to IEEE half, nearest-even (numpy's cast);
    returns uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f64(bits):
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------------------
# workloads


class Workload(dict):
    """Attribute-style dict: arrays plus the attention parameters."""

    __getattr__ = dict.__getitem__


def _normals(rng, shape, dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return f32_to_f16_bits(x)
    return x


def doc_lengths(rng, S, lo=256, hi=2048):
    """Packed-document lengths: integers uniform in [lo, hi] inclusive, drawn
    until they cover S; the last one is cut so the lengths sum to S."""
    out, total = [], 0
    while total < S:
        n = int(rng.integers(lo, hi, endpoint=True))
        out.append(n)
        total += n
    out[-1] -= total - S
    return out


def doc_ids(lengths):
    return np.repeat(np.arange(len(lengths), dtype=np.int32),
                     np.asarray(lengths, dtype=np.int64))


def random_case(seed, B, Sq, Sk, Hq, Hkv, D, dtype="bf16", grad=False,
                doc_len_range=None):
    """Generic seeded case (tests use it for small ragged shapes)."""
    rng = np.random.default_rng(seed)
    w = Workload(B=B, Sq=Sq, Sk=Sk, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype)
    if doc_len_range is not None:
        assert Sq == Sk
        lens = [doc_lengths(rng, Sq, *doc_len_range) for _ in range(B)]
        w["doc_lengths"] = lens
        w["doc"] = np.stack([doc_ids(l) for l in lens])
    w["q"] = _normals(rng, (B, Sq, Hq, D), dtype)
    w["k"] = _normals(rng, (B, Sk, Hkv, D), dtype)
    w["v"] = _normals(rng, (B, Sk, Hkv, D), dtype)
    if grad:
        w["do"] = _normals(rng, (B, Sq, Hq, D), dtype)
    return w


def tiny_dense():
    """B=1, Hq=Hkv=2, S=128, D=64, fp32, non-causal, seed 1."""
    w = random_case(1, 1, 128, 128, 2, 2, 64, dtype="f32")
    w.update(name="tiny_dense_fp32", scale=1.0 / 8.0, causal=False)
    return w


def llama8b_train():
    """Llama-3.1-8B-shaped training attention, forward and backward:
    B=1, Hq=32, Hkv=8, S=2048, D=128, bf16, causal, seed 2."""
    w = random_case(2, 1, 2048, 2048, 32, 8, 128, dtype="bf16", grad=True)
    w.update(name="llama8b_gqa_causal_s2048", scale=1.0 / np.sqrt(128.0),
             causal=True)
    return w


def long_local():
    """Long-context local attention: B=1, Hq=32, Hkv=8, S=16384, D=128,
    bf16, causal + window (4096, 0), seed 3.  Run A adds ALiBi with slopes
    2^(-8(h+1)/32); run B applies tanh softcap 50 to the scaled scores."""
    w = random_case(3, 1, 16384, 16384, 32, 8, 128, dtype="bf16")
    h = np.arange(32, dtype=np.float64)
    w.update(name="long_local_s16384_w4096", scale=1.0 / np.sqrt(128.0),
             causal=True, window=(4096, 0),
             alibi_slopes=np.exp2(-8.0 * (h + 1) / 32.0).astype(np.float32),
             softcap=50.0)
    return w


def doc_mask():
    """Packed-document block-sparse mask: B=2, Hq=Hkv=16, S=8192, D=64,
    bf16; document lengths uniform in [256, 2048]; mask = same document and
    causal; 128 x 128 blocks; seed 4."""
    w = random_case(4, 2, 8192, 8192, 16, 16, 64, dtype="bf16",
                    doc_len_range=(256, 2048))
    w.update(name="doc_mask_s8192", scale=1.0 / 8.0, causal=True,
             block=(128, 128))
    return w


def decode_mqa(seed=5, B=32, Hq=128, Smax=8192, D=128, lmin=1024, lmax=8192):
    """Decode over a KV cache, MQA: B=32, Hq=128, Hkv=1, one query per
    sequence, cache lengths uniform in [1024, 8192], D=128, bf16, seed 5."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(lmin, lmax, size=B, endpoint=True).astype(np.int32)
    w = Workload(B=B, Sq=1, Sk=Smax, Hq=Hq, Hkv=1, D=D, dtype="bf16",
                 cache_seqlens=lens)
    w["q"] = _normals(rng, (B, 1, Hq, D), "bf16")
    w["k"] = _normals(rng, (B, Smax, 1, D), "bf16")
    w["v"] = _normals(rng, (B, Smax, 1, D), "bf16")
    w.update(name="decode_mqa_b32_h128", scale=1.0 / np.sqrt(float(D)))
    return w


def to_pages(w, page_size, seed=17, spare_pages=5):
    """The same cache laid out as pages: every sequence's rows are scattered
    over a seeded random permutation of [num_pages, page_size, Hkv, D] pages
    (a few spare pages hold random junk).  Adds k_pages, v_pages and the
    int32 block_table [B, Smax / page_size] to a decode workload."""
    rng = np.random.default_rng(seed)
    k, v = w["k"], w["v"]
    B, Smax = k.shape[:2]
    assert Smax % page_size == 0
    nblk = Smax // page_size
    num_pages = B * nblk + spare_pages
    table = rng.permutation(num_pages)[: B * nblk].reshape(B, nblk).astype(np.int32)
    kp = _normals(rng, (num_pages, page_size) + k.shape[2:], "bf16")
    vp = _normals(rng, (num_pages, page_size) + v.shape[2:], "bf16")
    for b in range(B):
        kp[table[b]] = k[b].reshape((nblk, page_size) + k.shape[2:])
        vp[table[b]] = v[b].reshape((nblk, page_size) + v.shape[2:])
    w.update(k_pages=kp, v_pages=vp, block_table=table, page_size=page_size)
    return w


def new_tokens(w, s_new, seed=19):
    """Seeded new keys / values [B, s_new, Hkv, D] for an in-place append."""
    rng = np.random.default_rng(seed)
    shape = (w["k"].shape[0], s_new) + w["k"].shape[2:]
    w.update(k_new=_normals(rng, shape, "bf16"), v_new=_normals(rng, shape, "bf16"))
    return w


def as_f64(x, dtype):
    """The values a consumer of stored inputs sees, widened to fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f16":
        return f16_bits_to_f64(x)
    return np.asarray(x, dtype=np.float64)
