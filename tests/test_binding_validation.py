"""The Python binding rejects inconsistent arguments before anything reaches
the C ABI (CPU only: every check below fires before a device is touched).

The C ABI receives raw pointers and strides, so shapes, dtypes and devices
can only be checked here; a mismatch that got through would hand a kernel an
address outside a tensor.
"""

import pytest
import torch

binding = pytest.importorskip("exact_attention_10_amd.binding")

bf = torch.bfloat16


def qkv(B=2, Sq=8, Sk=8, Hq=4, Hkv=2, D=64, dtype=bf):
    return (torch.zeros(B, Sq, Hq, D, dtype=dtype), torch.zeros(B, Sk, Hkv, D, dtype=dtype),
            torch.zeros(B, Sk, Hkv, D, dtype=dtype))


def raises(fn, match):
    with pytest.raises(ValueError, match=match):
        fn()


def test_fwd_shape_checks():
    q, k, v = qkv()
    raises(lambda: binding.attn_fwd(q, k, v[:, :4]), "v must have shape")
    raises(lambda: binding.attn_fwd(q, k[..., :32], v[..., :32]), "k must be")
    raises(lambda: binding.attn_fwd(q, k[:1], v[:1]), "k must be")
    raises(lambda: binding.attn_fwd(q, k, v.float()), "v must be")
    raises(lambda: binding.attn_fwd(q[0], k, v), "4-d")
    raises(lambda: binding.attn_fwd(q, k, v, out=torch.zeros(2, 8, 4, 32, dtype=bf)), "out must have shape")
    raises(lambda: binding.attn_fwd(q, k, v, out=torch.zeros(2, 8, 4, 64)), "out must be")
    raises(lambda: binding.attn_fwd(q, k, v, lse=torch.zeros(2, 8, 4)), "lse must have shape")
    raises(lambda: binding.attn_fwd(q, k, v, lse=torch.zeros(2, 4, 8, dtype=torch.float64)), "lse must be")
    raises(lambda: binding.attn_fwd(q, k, v, lse=torch.zeros(2, 8, 4).transpose(1, 2)), "contiguous")


def test_alibi_shape_checks():
    q, k, v = qkv()
    raises(lambda: binding.attn_fwd(q, k, v, alibi_slopes=torch.zeros(3)), "alibi_slopes must be")
    raises(lambda: binding.attn_fwd(q, k, v, alibi_slopes=torch.zeros(4, 2)), "alibi_slopes must be")
    raises(lambda: binding.attn_fwd(q, k, v, alibi_slopes=torch.zeros(4, dtype=torch.float64)),
           "alibi_slopes must be")
    raises(lambda: binding.attn_fwd(q, k, v, alibi_slopes=torch.zeros(4, 2).t()), "contiguous")
    o, lse = q.clone(), torch.zeros(2, 4, 8)
    raises(lambda: binding.attn_bwd(q, k, v, o, o, lse, alibi_slopes=torch.zeros(2, 5)),
           "alibi_slopes must be")


def test_device_checks():
    q, k, v = qkv()
    # well-formed host tensors: refused because the library takes device pointers
    raises(lambda: binding.attn_fwd(q, k, v), "GPU tensor")
    o, lse = q.clone(), torch.zeros(2, 4, 8)
    raises(lambda: binding.attn_bwd(q, k, v, o, o, lse), "GPU tensor")


def test_bwd_shape_checks():
    q, k, v = qkv()
    o, lse = q.clone(), torch.zeros(2, 4, 8)
    raises(lambda: binding.attn_bwd(q, k, v, o[:, :4], o, lse), "out must have shape")
    raises(lambda: binding.attn_bwd(q, k, v, o, o.half(), lse), "dout must be")
    raises(lambda: binding.attn_bwd(q, k, v, o, o, None), "lse")
    raises(lambda: binding.attn_bwd(q, k, v, o, o, lse[:, :2]), "lse must have shape")
    raises(lambda: binding.attn_bwd(q, k, v, o, o, lse, dq=k.clone()), "dq must have shape")
    raises(lambda: binding.attn_bwd(q, k, v, o, o, lse, dk=q.clone()), "dk must have shape")
    raises(lambda: binding.attn_bwd(q, k, v, o, o, lse, dv=v.half()), "dv must be")
    raises(lambda: binding.attn_bwd(q, k, v, o, o, lse, workspace=torch.zeros(16)), "workspace must be")
    ws = torch.zeros(16, dtype=torch.uint8)
    raises(lambda: binding.attn_bwd_stage(1, q, k, v, o, o, lse, q.clone(), k.clone(), v[:1].clone(), ws),
           "dv must have shape")


def test_decode_shape_checks():
    B, Hq, Hkv, D, Smax = 3, 8, 1, 128, 64
    q = torch.zeros(B, 1, Hq, D, dtype=bf)
    kc = torch.zeros(B, Smax, Hkv, D, dtype=bf)
    vc = kc.clone()
    lens = torch.full((B,), 10, dtype=torch.int32)
    raises(lambda: binding.attn_decode(q, kc, vc, lens[:2]), "cache_seqlens must have shape")
    raises(lambda: binding.attn_decode(q, kc, vc, lens.long()), "cache_seqlens must be")
    raises(lambda: binding.attn_decode(q, kc, vc[:, :32], lens), "v_cache must have shape")
    raises(lambda: binding.attn_decode(q, kc[..., :64], vc[..., :64], lens), "head dim")
    raises(lambda: binding.attn_decode(q, kc[:2], vc[:2], lens), "batch rows")
    raises(lambda: binding.attn_decode(q, kc, vc, lens, block_table=torch.zeros(2, 4, dtype=torch.int32)),
           "block_table must have")
    raises(lambda: binding.attn_decode(q, kc, vc, lens, block_table=torch.zeros(3, 4)), "block_table must be")
    raises(lambda: binding.attn_decode(q, kc, vc, lens, cache_batch_idx=torch.zeros(2, dtype=torch.int32)),
           "cache_batch_idx must have shape")
    kn = torch.zeros(B, 2, Hkv, D, dtype=bf)
    raises(lambda: binding.attn_decode(q, kc, vc, lens, k_new=kn), "together")
    raises(lambda: binding.attn_decode(q, kc, vc, lens, k_new=kn, v_new=kn[:, :1]), "v_new must have shape")
    raises(lambda: binding.attn_decode(q, kc, vc, lens, k_new=kn[:, :, :, :64], v_new=kn[:, :, :, :64]),
           "k_new must be")
    raises(lambda: binding.attn_decode(q, kc, vc, lens, out=q[:, :, :4]), "out must have shape")
    raises(lambda: binding.attn_decode(q, kc, vc, lens, lse=torch.zeros(B, Hq, 2)), "lse must have shape")
    raises(lambda: binding.attn_decode(q, kc, vc, lens), "GPU tensor")


def test_block_mask_build_checks():
    d = torch.zeros(2, 256, dtype=torch.int32)
    raises(lambda: binding.block_mask_build(2, 256, 256, doc_q=d), "both")
    raises(lambda: binding.block_mask_build(2, 256, 256, doc_q=d[:1], doc_k=d), "doc_q must have shape")
    raises(lambda: binding.block_mask_build(2, 256, 256, doc_q=d, doc_k=d.long()), "doc_k must be")
    raises(lambda: binding.block_mask_build(2, 256, 256, doc_q=d, doc_k=d), "one GPU")
