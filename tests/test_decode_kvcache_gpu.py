"""GPU parity of decode over a paged / batch-indexed KV cache with in-place
append ([FA] "Examples", flash_attn_with_kvcache: block_table,
cache_batch_idx, new k/v updating the cache in place) against the fp64
oracle, through the C ABI (attn_decode_kvcache) via the ctypes binding.
Outputs to the decode tolerances; the caches after the append bit-exact."""

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


def f64(w, name):
    return inputs.as_f64(w[name], "bf16")


def dev16(x):
    return to_device(x, "bf16", torch)


def dev32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def host16(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def gqa_case(seed, B, Hq, Hkv, D, Smax, lens):
    w = inputs.decode_mqa(seed=seed, B=B, Hq=Hq, Smax=Smax, D=D, lmin=1, lmax=Smax)
    if Hkv > 1:
        rng = np.random.default_rng(seed + 1)
        shape = (B, Smax, Hkv, D)
        w["k"] = inputs.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
        w["v"] = inputs.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    if lens is not None:
        w["cache_seqlens"] = np.asarray(lens, dtype=np.int32)
    return w


@pytest.mark.parametrize("cfg", [
    dict(B=4, Hq=128, Hkv=1, D=128, Smax=2048, page=256, lens=None),
    dict(B=3, Hq=16, Hkv=4, D=64, Smax=256, page=32, lens=[0, 1, 256]),
    dict(B=5, Hq=40, Hkv=8, D=128, Smax=512, page=64, lens=[33, 64, 65, 500, 511]),
])
def test_paged(b, cfg):
    w = gqa_case(31, cfg["B"], cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["Smax"], cfg["lens"])
    inputs.to_pages(w, cfg["page"])
    lens = w["cache_seqlens"]
    O, L, _ = oracle.decode_kvcache(f64(w, "q"), f64(w, "k_pages"), f64(w, "v_pages"), lens,
                                    block_table=w["block_table"], page_size=cfg["page"], scale=0.1)
    for splits in (0, 3, 1000):
        o, lse = b.attn_decode(dev16(w["q"]), dev16(w["k_pages"]), dev16(w["v_pages"]), dev32(lens),
                               softmax_scale=0.1, num_splits=splits, block_table=dev32(w["block_table"]))
        torch.cuda.synchronize()
        check_o(to_f64(o), O, what="O(splits=%d)" % splits)
        check_lse(to_f64(lse), L)


def test_paged_c5_full(b):
    """The B=32 Hq=128 MQA decode workload in 256-row pages."""
    w = inputs.to_pages(inputs.decode_mqa(), 256)
    lens = w["cache_seqlens"]
    O, L = oracle.decode(f64(w, "q"), f64(w, "k"), f64(w, "v"), lens, scale=w["scale"])
    o, lse = b.attn_decode(dev16(w["q"]), dev16(w["k_pages"]), dev16(w["v_pages"]), dev32(lens),
                           softmax_scale=w["scale"], block_table=dev32(w["block_table"]))
    torch.cuda.synchronize()
    check_o(to_f64(o), O)
    check_lse(to_f64(lse), L)


def test_cache_batch_idx(b):
    w = gqa_case(33, 4, 16, 2, 64, 128, [128, 5, 0, 77])
    rng = np.random.default_rng(34)
    extra = inputs.f32_to_bf16_bits(rng.standard_normal((3, 128, 2, 64), dtype=np.float32))
    kc = np.concatenate([w["k"], extra])
    vc = np.concatenate([w["v"], extra[::-1]])
    idx = np.array([5, 2, 0, 4], dtype=np.int32)
    lens = w["cache_seqlens"]
    O, L, _ = oracle.decode_kvcache(f64(w, "q"), inputs.as_f64(kc, "bf16"), inputs.as_f64(vc, "bf16"),
                                    lens, cache_batch_idx=idx, softcap=3.0, scale=0.2)
    o, lse = b.attn_decode(dev16(w["q"]), dev16(kc), dev16(vc), dev32(lens), softmax_scale=0.2,
                           softcap=3.0, cache_batch_idx=dev32(idx))
    torch.cuda.synchronize()
    check_o(to_f64(o), O)
    check_lse(to_f64(lse), L)


@pytest.mark.parametrize("paged,s_new", [(False, 1), (True, 1), (True, 5), (False, 3)])
def test_append(b, paged, s_new):
    w = gqa_case(35, 4, 32, 2, 128, 256, [0, 31, 100, 251 - 3])
    inputs.new_tokens(w, s_new)
    lens = w["cache_seqlens"]
    kw_o, kw_g = {}, {}
    if paged:
        inputs.to_pages(w, 64)
        kc, vc = w["k_pages"], w["v_pages"]
        kw_o = dict(block_table=w["block_table"], page_size=64)
        kw_g = dict(block_table=dev32(w["block_table"]))
    else:
        kc, vc = w["k"], w["v"]
    O, L, (k_after, v_after) = oracle.decode_kvcache(
        f64(w, "q"), inputs.as_f64(kc, "bf16"), inputs.as_f64(vc, "bf16"), lens,
        k_new=f64(w, "k_new"), v_new=f64(w, "v_new"), scale=0.1, **kw_o)
    kd, vd = dev16(kc), dev16(vc)
    o, lse = b.attn_decode(dev16(w["q"]), kd, vd, dev32(lens), softmax_scale=0.1,
                           k_new=dev16(w["k_new"]), v_new=dev16(w["v_new"]), **kw_g)
    torch.cuda.synchronize()
    check_o(to_f64(o), O)
    check_lse(to_f64(lse), L)
    # the caches were updated in place, bit for bit (the appended rows are copies)
    np.testing.assert_array_equal(inputs.bf16_bits_to_f64(host16(kd)), k_after)
    np.testing.assert_array_equal(inputs.bf16_bits_to_f64(host16(vd)), v_after)


def test_kvcache_errors(b):
    w = gqa_case(37, 2, 8, 1, 64, 128, [5, 6])
    inputs.to_pages(w, 64)
    q, lens = dev16(w["q"]), dev32(w["cache_seqlens"])
    with pytest.raises(b.AttnError):  # page size not a multiple of 32
        kp = dev16(w["k_pages"])[:, :48].contiguous()
        b.attn_decode(q, kp, kp, lens, block_table=dev32(w["block_table"]))
    with pytest.raises(b.AttnError):  # block_table with cache_batch_idx
        kp = dev16(w["k_pages"])
        b.attn_decode(q, kp, kp, lens, block_table=dev32(w["block_table"]),
                      cache_batch_idx=dev32([0, 1]))
