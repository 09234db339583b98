"""GPU parity of decode with several queries per sequence (chunked prefill,
speculative decoding: [FA] "Examples", flash_attn_with_kvcache with q of
seqlen > 1 and causal=True, bottom-right aligned) against the fp64 oracle,
through the C ABI via the ctypes binding."""

import numpy as np
import pytest

import oracle
from exact_attention_10_amd import inputs
from helpers import check_lse, check_o, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_10_amd import binding
    return binding


def dev16(x):
    return to_device(x, "bf16", torch)


def dev32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def host16(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def case(seed, B, Sq, Hq, Hkv, D, Smax, lens):
    rng = np.random.default_rng(seed)
    bits = lambda shape: inputs.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    return dict(q=bits((B, Sq, Hq, D)), k=bits((B, Smax, Hkv, D)), v=bits((B, Smax, Hkv, D)),
                lens=np.asarray(lens, dtype=np.int32))


def f64(x):
    return inputs.as_f64(x, "bf16")


CFGS = [
    # B, Sq, Hq, Hkv, D, Smax, lens, causal, softcap
    (4, 4, 32, 8, 128, 512, [512, 2, 100, 33], True, 0.0),      # 16 rows per kv head: one job
    (3, 3, 128, 1, 128, 1024, [1024, 700, 3], True, 4.0),       # 384 rows: 256- and 128-row jobs
    (2, 5, 16, 2, 64, 256, [256, 77], False, 0.0),              # non-causal: every row sees all keys
    (2, 2, 40, 1, 64, 256, [1, 200], True, 0.0),                # rows mix positions inside a job
    (2, 64, 8, 8, 128, 300, [300, 64], True, 0.0),              # a 64-query chunk
    (2, 4, 64, 1, 64, 256, [256, 130], True, 0.0),              # 256 rows: one wide job, D 64
    (3, 3, 64, 1, 128, 512, [512, 40, 3], False, 0.0),          # 192 rows: a wide job, two blocks idle
    (2, 8, 64, 2, 128, 640, [640, 300], True, 0.0),             # 512 rows per kv head: two wide jobs
]


@pytest.mark.parametrize("cfg", CFGS, ids=[str(i) for i in range(len(CFGS))])
def test_multi_query(b, cfg):
    B, Sq, Hq, Hkv, D, Smax, lens, causal, cap = cfg
    w = case(50 + Sq + Hq, B, Sq, Hq, Hkv, D, Smax, lens)
    O, L = oracle.decode(f64(w["q"]), f64(w["k"]), f64(w["v"]), w["lens"], scale=0.09, softcap=cap,
                         causal=causal)
    for splits in (0, 3, 1000):
        o, lse = b.attn_decode(dev16(w["q"]), dev16(w["k"]), dev16(w["v"]), dev32(w["lens"]),
                               softmax_scale=0.09, softcap=cap, causal=causal, num_splits=splits)
        torch.cuda.synchronize()
        check_o(to_f64(o), O, what="O(splits=%d)" % splits)
        check_lse(to_f64(lse), L)


@pytest.mark.parametrize("paged", [False, True])
def test_speculative_append(b, paged):
    """Four draft tokens: their keys/values are appended in place, then the
    four queries attend causally (each sees the cache and the drafts up to
    itself)."""
    B, S_new, Hq, Hkv, D, Smax = 4, 4, 32, 4, 128, 512
    w = case(61, B, S_new, Hq, Hkv, D, Smax, [0, 31, 300, 508])
    rng = np.random.default_rng(62)
    kn = inputs.f32_to_bf16_bits(rng.standard_normal((B, S_new, Hkv, D), dtype=np.float32))
    vn = inputs.f32_to_bf16_bits(rng.standard_normal((B, S_new, Hkv, D), dtype=np.float32))
    kw_o, kw_g = {}, {}
    kc, vc = w["k"], w["v"]
    if paged:
        pw = inputs.to_pages(dict(k=w["k"], v=w["v"], cache_seqlens=w["lens"]), 64)
        kc, vc = pw["k_pages"], pw["v_pages"]
        kw_o = dict(block_table=pw["block_table"], page_size=64)
        kw_g = dict(block_table=dev32(pw["block_table"]))
    O, L, (k_after, v_after) = oracle.decode_kvcache(f64(w["q"]), f64(kc), f64(vc), w["lens"],
                                                     k_new=f64(kn), v_new=f64(vn), scale=0.1,
                                                     causal=True, **kw_o)
    kd, vd = dev16(kc), dev16(vc)
    o, lse = b.attn_decode(dev16(w["q"]), kd, vd, dev32(w["lens"]), softmax_scale=0.1, causal=True,
                           k_new=dev16(kn), v_new=dev16(vn), **kw_g)
    torch.cuda.synchronize()
    check_o(to_f64(o), O)
    check_lse(to_f64(lse), L)
    np.testing.assert_array_equal(inputs.bf16_bits_to_f64(host16(kd)), k_after)
    np.testing.assert_array_equal(inputs.bf16_bits_to_f64(host16(vd)), v_after)


def test_speculative_mqa_b32_full(b):
    """The B=32, Hq=128 MQA decode workload (cache lengths U[1024, 8192],
    D=128) with four draft tokens appended to 256-row pages and attended
    causally: every output against the oracle."""
    w = inputs.decode_mqa()
    lens = w["cache_seqlens"] - 4  # the drafts fit the capacity
    rng = np.random.default_rng(63)
    q = inputs.f32_to_bf16_bits(rng.standard_normal((32, 4, 128, 128), dtype=np.float32))
    kn = inputs.f32_to_bf16_bits(rng.standard_normal((32, 4, 1, 128), dtype=np.float32))
    vn = inputs.f32_to_bf16_bits(rng.standard_normal((32, 4, 1, 128), dtype=np.float32))
    pw = inputs.to_pages(dict(k=w["k"], v=w["v"], cache_seqlens=lens), 256)
    O, L, _ = oracle.decode_kvcache(f64(q), f64(pw["k_pages"]), f64(pw["v_pages"]), lens,
                                    block_table=pw["block_table"], page_size=256, k_new=f64(kn),
                                    v_new=f64(vn), scale=w["scale"], causal=True)
    o, lse = b.attn_decode(dev16(q), dev16(pw["k_pages"]), dev16(pw["v_pages"]), dev32(lens),
                           softmax_scale=w["scale"], causal=True, block_table=dev32(pw["block_table"]),
                           k_new=dev16(kn), v_new=dev16(vn))
    torch.cuda.synchronize()
    check_o(to_f64(o), O)
    check_lse(to_f64(lse), L)


def test_multi_query_errors(b):
    w = case(70, 2, 3, 8, 2, 64, 128, [5, 6])
    q, k, lens = dev16(w["q"]), dev16(w["k"]), dev32(w["lens"])
    with pytest.raises(b.AttnError):  # more queries than cache rows
        b.attn_decode(dev16(np.zeros((2, 200, 8, 64), dtype=np.uint16)), k, k, lens)
    with pytest.raises(b.AttnError):  # window is not a decode option
        from exact_attention_10_amd import binding as bb
        p = bb._params(q, k, 64, None, True, (4, 0), None, 0.0, None)
        ws = torch.empty(bb.decode_workspace_size(q, k), dtype=torch.uint8, device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty((2, 8, 3), dtype=torch.float32, device="cuda")
        import ctypes
        bb._check(bb.library().attn_decode(ctypes.byref(p), bb._tensor(q), bb._tensor(k), bb._tensor(k),
                                           bb._ptr(lens), 0, bb._tensor(o), bb._ptr(lse), bb._ptr(ws),
                                           ws.numel(), bb._stream()))
