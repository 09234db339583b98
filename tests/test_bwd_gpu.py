"""GPU parity of the backward (dQ, dK, dV from the saved LSE) against the
fp64 oracle's chain-rule gradients (through the C ABI via the ctypes binding)."""

import numpy as np
import pytest

import oracle
from exact_attention_10_amd import inputs
from helpers import GRAD_ATOL, check_o, f64, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_10_amd import binding
    return binding


def run_bwd(b, w, **kw):
    q, k, v, do = (to_device(w[n], "bf16", torch) for n in ("q", "k", "v", "do"))
    o, lse = b.attn_fwd(q, k, v, **kw)
    dq, dk, dv = b.attn_bwd(q, k, v, o, do, lse, **kw)
    torch.cuda.synchronize()
    return dq, dk, dv


def oracle_grads(w, kw, slopes=None):
    return oracle.attention_bwd(f64(w, "q"), f64(w, "k"), f64(w, "v"), f64(w, "do"),
                                scale=kw["softmax_scale"], causal=kw.get("causal", False),
                                window=kw.get("window", (-1, -1)), alibi_slopes=slopes,
                                softcap=kw.get("softcap", 0.0))


CASES = [
    # B, Sq, Sk, Hq, Hkv, D, options
    (1, 128, 128, 2, 2, 64, {}),
    (2, 200, 333, 4, 2, 64, {}),
    (1, 257, 257, 8, 2, 128, {"causal": True}),
    (1, 300, 190, 4, 1, 128, {"causal": True}),
    (1, 190, 300, 4, 4, 64, {"causal": True}),
    (1, 400, 400, 4, 2, 128, {"causal": True, "window": (100, 0)}),
    (1, 333, 333, 2, 1, 64, {"window": (70, 33)}),
    (1, 300, 300, 4, 2, 128, {"causal": True, "alibi": True}),
    (1, 300, 300, 4, 2, 128, {"causal": True, "softcap": 5.0}),
    (1, 280, 280, 4, 4, 64, {"causal": True, "softcap": 2.0, "alibi": True}),
    (1, 160, 160, 2, 1, 128, {"causal": True, "scale": -0.09}),
    (1, 256, 256, 2, 2, 128, {"window": (0, 0)}),        # each row sees only its own key
    # a single key: dV is the plain sum of the rows' dO, so few rows keep it
    # where bf16 output rounding (half a step) stays well below the bound
    (1, 9, 1, 2, 1, 128, {}),
    (1, 1, 700, 8, 1, 128, {}),                          # a single query
    (1, 97, 97, 4, 2, 64, {"causal": True}),             # one ragged tile in each direction
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_bwd_parity(b, case):
    _bwd_case(b, case)


@pytest.fixture
def gqa_schedule(b):
    """Sets attn_set_bwd_gqa_schedule for one test and restores automatic."""
    yield b.set_bwd_gqa_schedule
    b.set_bwd_gqa_schedule(0)


GQA_CASES = [c for c in CASES if c[3] > c[4]]


@pytest.mark.parametrize("mode", [1, 2])
@pytest.mark.parametrize("case", GQA_CASES, ids=[str(i) for i in range(len(GQA_CASES))])
def test_bwd_gqa_schedules(b, gqa_schedule, case, mode):
    """Both dK/dV schedules for grouped-query heads (per-head partials plus a
    group sum; the group's heads looped inside each workgroup) against the
    oracle, whichever the automatic choice would take."""
    gqa_schedule(mode)
    _bwd_case(b, case)


def _bwd_case(b, case):
    B, Sq, Sk, Hq, Hkv, D, opt = case
    w = inputs.random_case(300 + Sq + Sk + D, B, Sq, Sk, Hq, Hkv, D, dtype="bf16", grad=True)
    kw = dict(softmax_scale=opt.get("scale", 0.11 if D == 128 else 0.15),
              causal=opt.get("causal", False), window=opt.get("window", (-1, -1)),
              softcap=opt.get("softcap", 0.0))
    slopes = None
    if opt.get("alibi"):
        slopes = np.exp2(-8.0 * (np.arange(Hq) + 1) / Hq).astype(np.float32)
        kw["alibi_slopes"] = torch.from_numpy(slopes).cuda()
    dq, dk, dv = run_bwd(b, w, **kw)
    rq, rk, rv = oracle_grads(w, kw, slopes)
    check_o(to_f64(dq), rq, GRAD_ATOL, "dQ")
    check_o(to_f64(dk), rk, GRAD_ATOL, "dK")
    check_o(to_f64(dv), rv, GRAD_ATOL, "dV")


def test_bwd_llama8b_full(b):
    """B=1, Hq=32, Hkv=8, S=2048, D=128, causal: every gradient element against
    the oracle (dK/dV summed over each query group), and a second run
    bitwise identical (deterministic backward)."""
    w = inputs.llama8b_train()
    kw = dict(softmax_scale=w["scale"], causal=True)
    dq, dk, dv = run_bwd(b, w, **kw)
    rq, rk, rv = oracle_grads(w, kw)
    check_o(to_f64(dq), rq, GRAD_ATOL, "dQ")
    check_o(to_f64(dk), rk, GRAD_ATOL, "dK")
    check_o(to_f64(dv), rv, GRAD_ATOL, "dV")
    dq2, dk2, dv2 = run_bwd(b, w, **kw)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


def test_bwd_llama8b_group_loop(b, gqa_schedule):
    """The same workload with the G = 4 query heads of each kv head looped
    inside the dK/dV workgroups: every dK/dV element against the oracle, dQ
    unchanged bit for bit, and a second run bitwise identical."""
    w = inputs.llama8b_train()
    kw = dict(softmax_scale=w["scale"], causal=True)
    dq1, _, _ = run_bwd(b, w, **kw)
    gqa_schedule(2)
    dq, dk, dv = run_bwd(b, w, **kw)
    assert torch.equal(dq, dq1)
    _, rk, rv = oracle_grads(w, kw)
    check_o(to_f64(dk), rk, GRAD_ATOL, "dK")
    check_o(to_f64(dv), rv, GRAD_ATOL, "dV")
    dq2, dk2, dv2 = run_bwd(b, w, **kw)
    assert torch.equal(dk, dk2) and torch.equal(dv, dv2)


# ---------------------------------------------------------------------------
# Block-sparse backward ([GYM] create_block_mask; [FX4] block sparsity): the
# dK/dV kernel walks each key block's query-block lists, the dQ kernel each
# query block's key-block lists; partial tiles evaluate the predicate.

SPARSE_CASES = [
    # B, S, Hq, Hkv, D, block_n, causal, window, doc length range, options
    (2, 300, 4, 2, 64, 128, True, (-1, -1), (20, 90), {}),
    (1, 333, 2, 2, 128, 256, False, (-1, -1), (30, 200), {"softcap": 3.0}),
    (1, 257, 8, 2, 128, 128, True, (-1, -1), None, {}),
    (1, 400, 4, 1, 64, 128, True, (100, 0), None, {"alibi": True}),
    (2, 520, 4, 4, 128, 128, True, (-1, -1), (64, 300), {"scale": -0.08}),
]


@pytest.mark.parametrize("case", SPARSE_CASES, ids=[str(i) for i in range(len(SPARSE_CASES))])
def test_bwd_block_sparse(b, case):
    _sparse_case(b, case)


def test_bwd_block_sparse_group_loop(b, gqa_schedule):
    """A grouped-query block-sparse case with the heads looped in the dK/dV
    workgroups (the query-block lists are walked once per head)."""
    gqa_schedule(2)
    _sparse_case(b, (2, 300, 8, 2, 128, 128, True, (-1, -1), (20, 90), {"alibi": True}))


def _sparse_case(b, case):
    B, S, Hq, Hkv, D, bn, causal, window, doc_range, opt = case
    w = inputs.random_case(700 + S + D, B, S, S, Hq, Hkv, D, dtype="bf16", grad=True,
                           doc_len_range=doc_range)
    doc = w.get("doc")
    doc_t = torch.from_numpy(doc).cuda() if doc is not None else None
    m = b.block_mask_build(B, S, S, 128, bn, causal=causal, window=window, doc_q=doc_t, doc_k=doc_t)
    kw = dict(softmax_scale=opt.get("scale", 0.12), softcap=opt.get("softcap", 0.0), block_mask=m)
    slopes = None
    if opt.get("alibi"):
        slopes = np.exp2(-8.0 * (np.arange(Hq) + 1) / Hq).astype(np.float32)
        kw["alibi_slopes"] = torch.from_numpy(slopes).cuda()
    dq, dk, dv = run_bwd(b, w, **kw)
    rq, rk, rv = oracle.attention_bwd(f64(w, "q"), f64(w, "k"), f64(w, "v"), f64(w, "do"),
                                      scale=kw["softmax_scale"], causal=causal, window=window,
                                      alibi_slopes=slopes, softcap=kw["softcap"], doc_q=doc, doc_k=doc)
    check_o(to_f64(dq), rq, GRAD_ATOL, "dQ")
    check_o(to_f64(dk), rk, GRAD_ATOL, "dK")
    check_o(to_f64(dv), rv, GRAD_ATOL, "dV")


def test_bwd_doc_mask_s8192(b):
    """The packed-document workload (B=2, H=16, S=8192, D=64, causal within
    documents, 128x128 blocks) through the block-sparse backward.  Documents
    do not interact, so the oracle is run per document (the pinned
    per-document identity) on all 16 heads, and every gradient element is
    compared."""
    w = inputs.doc_mask()
    rng = np.random.default_rng(44)
    w["do"] = inputs.f32_to_bf16_bits(rng.standard_normal(w["q"].shape, dtype=np.float32))
    doc = torch.from_numpy(w["doc"]).cuda()
    m = b.block_mask_build(2, 8192, 8192, 128, 128, causal=True, doc_q=doc, doc_k=doc)
    dq, dk, dv = run_bwd(b, w, softmax_scale=w["scale"], block_mask=m)
    got = [to_f64(t) for t in (dq, dk, dv)]
    x = {n: f64(w, n) for n in ("q", "k", "v", "do")}
    for bb in range(2):
        s0 = 0
        for n in w["doc_lengths"][bb]:
            sl = slice(s0, s0 + n)
            ref = oracle.attention_bwd(x["q"][bb:bb + 1, sl], x["k"][bb:bb + 1, sl],
                                       x["v"][bb:bb + 1, sl], x["do"][bb:bb + 1, sl],
                                       scale=w["scale"], causal=True)
            for name, g, r in zip(("dQ", "dK", "dV"), got, ref):
                check_o(g[bb:bb + 1, sl], r, GRAD_ATOL, "%s b%d doc@%d" % (name, bb, s0))
            s0 += n
        assert s0 == 8192


@pytest.mark.parametrize("mode", [1, 2])
def test_bwd_alibi_per_batch_slopes(b, gqa_schedule, mode):
    """Backward with ALiBi slopes of shape (batch, nheads) ("FlashAttention:
    Fast and Memory-Efficient Exact Attention", "Examples"): every gradient
    element against the oracle with the same per-batch table, under both
    grouped-query dK/dV schedules (the slope is the per-head term the
    in-workgroup head loop must switch)."""
    gqa_schedule(mode)
    B, S, Hq, Hkv, D = 3, 300, 4, 2, 128
    w = inputs.random_case(71, B, S, S, Hq, Hkv, D, dtype="bf16", grad=True)
    slopes = np.random.default_rng(72).uniform(0.05, 1.0, (B, Hq)).astype(np.float32)
    kw = dict(softmax_scale=0.1, causal=True, window=(200, 0))
    dq, dk, dv = run_bwd(b, w, alibi_slopes=torch.from_numpy(slopes).cuda(), **kw)
    rq, rk, rv = oracle_grads(w, kw, slopes)
    check_o(to_f64(dq), rq, GRAD_ATOL, "dQ")
    check_o(to_f64(dk), rk, GRAD_ATOL, "dK")
    check_o(to_f64(dv), rv, GRAD_ATOL, "dV")


def test_bwd_block_sparse_errors(b):
    w = inputs.random_case(5, 1, 256, 256, 2, 2, 64, dtype="bf16", grad=True)
    q, k, v, do = (to_device(w[n], "bf16", torch) for n in ("q", "k", "v", "do"))
    m64 = b.block_mask_build(1, 256, 256, 128, 64, causal=True)
    o, lse = b.attn_fwd(q, k, v, block_mask=m64)
    with pytest.raises(b.AttnError):  # block_n = 64 is forward-only
        b.attn_bwd(q, k, v, o, do, lse, block_mask=m64)
    m = b.block_mask_build(1, 256, 256, 128, 128, causal=True)
    with pytest.raises(b.AttnError):  # the block mask carries the predicate
        b.attn_bwd(q, k, v, o, do, lse, causal=True, block_mask=m)


# ---------------------------------------------------------------------------
# deterministic=0 ([FA] deterministic flag): dQ accumulated by the dK/dV
# kernel with fp32 atomic adds (summation order not fixed), then scaled and
# rounded by a conversion pass.  Same gradients to the same tolerance.

def run_bwd_nd(b, w, bwd_kw, **kw):
    q, k, v, do = (to_device(w[n], "bf16", torch) for n in ("q", "k", "v", "do"))
    o, lse = b.attn_fwd(q, k, v, **kw)
    dq, dk, dv = b.attn_bwd(q, k, v, o, do, lse, deterministic=False, **kw, **bwd_kw)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("case", [CASES[i] for i in (1, 2, 3, 5, 7, 9, 10)],
                         ids=[str(i) for i in (1, 2, 3, 5, 7, 9, 10)])
def test_bwd_nondeterministic(b, case):
    B, Sq, Sk, Hq, Hkv, D, opt = case
    w = inputs.random_case(300 + Sq + Sk + D, B, Sq, Sk, Hq, Hkv, D, dtype="bf16", grad=True)
    kw = dict(softmax_scale=opt.get("scale", 0.11 if D == 128 else 0.15),
              causal=opt.get("causal", False), window=opt.get("window", (-1, -1)),
              softcap=opt.get("softcap", 0.0))
    slopes = None
    if opt.get("alibi"):
        slopes = np.exp2(-8.0 * (np.arange(Hq) + 1) / Hq).astype(np.float32)
        kw["alibi_slopes"] = torch.from_numpy(slopes).cuda()
    dq, dk, dv = run_bwd_nd(b, w, {}, **kw)
    rq, rk, rv = oracle_grads(w, kw, slopes)
    check_o(to_f64(dq), rq, GRAD_ATOL, "dQ")
    check_o(to_f64(dk), rk, GRAD_ATOL, "dK")
    check_o(to_f64(dv), rv, GRAD_ATOL, "dV")


def test_bwd_nondeterministic_block_sparse(b):
    w = inputs.random_case(77, 2, 300, 300, 4, 2, 128, dtype="bf16", grad=True, doc_len_range=(20, 90))
    doc_t = torch.from_numpy(w["doc"]).cuda()
    m = b.block_mask_build(2, 300, 300, 128, 128, causal=True, doc_q=doc_t, doc_k=doc_t)
    dq, dk, dv = run_bwd_nd(b, w, {}, softmax_scale=0.12, block_mask=m)
    rq, rk, rv = oracle.attention_bwd(f64(w, "q"), f64(w, "k"), f64(w, "v"), f64(w, "do"), scale=0.12,
                                      causal=True, doc_q=w["doc"], doc_k=w["doc"])
    check_o(to_f64(dq), rq, GRAD_ATOL, "dQ")
    check_o(to_f64(dk), rk, GRAD_ATOL, "dK")
    check_o(to_f64(dv), rv, GRAD_ATOL, "dV")


def test_bwd_nondeterministic_llama8b_full(b):
    """The B=1, Hq=32, Hkv=8, S=2048, D=128 causal workload with atomic dQ:
    every gradient element against the oracle, and dV and dQ against the
    deterministic schedule (whose dK/dV kernel at D = 128 forms dS from P
    handed between two waves in fp16, so its dK differs in rounding)."""
    w = inputs.llama8b_train()
    kw = dict(softmax_scale=w["scale"], causal=True)
    dq, dk, dv = run_bwd_nd(b, w, {}, **kw)
    rq, rk, rv = oracle_grads(w, kw)
    check_o(to_f64(dq), rq, GRAD_ATOL, "dQ")
    check_o(to_f64(dk), rk, GRAD_ATOL, "dK")
    check_o(to_f64(dv), rv, GRAD_ATOL, "dV")
    dq1, dk1, dv1 = run_bwd(b, w, **kw)
    assert torch.equal(dv, dv1)
    # dV comes from the same arithmetic in both schedules; dK of each is held
    # to the oracle above (its dS roundings differ, and dK sums cancelling
    # terms, so no tighter bound between the two holds by construction)
    assert float((dq.float() - dq1.float()).abs().max()) <= 1e-2


# ---------------------------------------------------------------------------
# Packed inputs and gradients ([FA] flash_attn_qkvpacked_func /
# flash_attn_kvpacked_func): the kernels read and write through strides, so
# packed tensors are used in place and the results are bitwise those of the
# separate tensors.

@pytest.mark.parametrize("D,causal", [(64, True), (128, False)])
def test_qkvpacked_fwd_bwd(b, D, causal):
    B, S, H = 2, 333, 4
    w = inputs.random_case(900 + D, B, S, S, H, H, D, dtype="bf16", grad=True)
    q, k, v, do = (to_device(w[n], "bf16", torch) for n in ("q", "k", "v", "do"))
    qkv = torch.stack([q, k, v], dim=2).contiguous()  # [B, S, 3, H, D]
    o_p, lse_p = b.attn_fwd_qkvpacked(qkv, softmax_scale=0.1, causal=causal)
    dqkv = b.attn_bwd_qkvpacked(qkv, o_p, do, lse_p, softmax_scale=0.1, causal=causal)
    o, lse = b.attn_fwd(q, k, v, softmax_scale=0.1, causal=causal)
    dq, dk, dv = b.attn_bwd(q, k, v, o, do, lse, softmax_scale=0.1, causal=causal)
    torch.cuda.synchronize()
    assert dqkv.shape == qkv.shape
    assert torch.equal(o_p, o) and torch.equal(lse_p, lse)
    assert torch.equal(dqkv[:, :, 0], dq) and torch.equal(dqkv[:, :, 1], dk) and torch.equal(dqkv[:, :, 2], dv)
    rq, rk, rv = oracle.attention_bwd(f64(w, "q"), f64(w, "k"), f64(w, "v"), f64(w, "do"), scale=0.1,
                                      causal=causal)
    check_o(to_f64(dqkv[:, :, 0]), rq, GRAD_ATOL, "dQ")
    check_o(to_f64(dqkv[:, :, 1]), rk, GRAD_ATOL, "dK")
    check_o(to_f64(dqkv[:, :, 2]), rv, GRAD_ATOL, "dV")


def test_kvpacked_gqa(b):
    B, S, Hq, Hkv, D = 1, 300, 8, 2, 128
    w = inputs.random_case(950, B, S, S, Hq, Hkv, D, dtype="bf16", grad=True)
    q, k, v, do = (to_device(w[n], "bf16", torch) for n in ("q", "k", "v", "do"))
    kv = torch.stack([k, v], dim=2).contiguous()  # [B, S, 2, Hkv, D]
    o, lse = b.attn_fwd_kvpacked(q, kv, softmax_scale=0.09, causal=True)
    dq, dkv = b.attn_bwd_kvpacked(q, kv, o, do, lse, softmax_scale=0.09, causal=True)
    dq2, dk2, dv2 = run_bwd(b, w, softmax_scale=0.09, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dkv[:, :, 0], dk2) and torch.equal(dkv[:, :, 1], dv2)
    rq, rk, rv = oracle.attention_bwd(f64(w, "q"), f64(w, "k"), f64(w, "v"), f64(w, "do"), scale=0.09,
                                      causal=True)
    check_o(to_f64(dkv[:, :, 0]), rk, GRAD_ATOL, "dK")
    check_o(to_f64(dkv[:, :, 1]), rv, GRAD_ATOL, "dV")


@pytest.mark.parametrize("deterministic", [True, False])
@pytest.mark.parametrize("case", [CASES[i] for i in (1, 3)], ids=["1", "3"])
def test_bwd_stages_equal_attn_bwd(b, case, deterministic):
    """attn_bwd_stage 0, 1, 2, 3 in order on one stream and workspace give
    exactly attn_bwd's gradients (either schedule; GQA and ragged shapes)."""
    B, Sq, Sk, Hq, Hkv, D, opt = case
    w = inputs.random_case(500 + Sq + D, B, Sq, Sk, Hq, Hkv, D, dtype="bf16", grad=True)
    kw = dict(softmax_scale=0.11, causal=opt.get("causal", False))
    q, k, v, do = (to_device(w[n], "bf16", torch) for n in ("q", "k", "v", "do"))
    o, lse = b.attn_fwd(q, k, v, **kw)
    ref = b.attn_bwd(q, k, v, o, do, lse, deterministic=deterministic, **kw)
    ws = torch.empty(b.bwd_workspace_size(q, k), dtype=torch.uint8, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    for st in range(4):
        b.attn_bwd_stage(st, q, k, v, o, do, lse, dq, dk, dv, ws, deterministic=deterministic, **kw)
    torch.cuda.synchronize()
    for x, y in zip((dq, dk, dv), ref):
        assert torch.equal(x, y)


def test_bwd_empty_inputs(b):
    """No keys: every row is empty (O = 0, LSE = -inf) and dQ is zero.  No
    queries: no row reaches any key, so dK and dV are zero."""
    q = torch.randn((1, 5, 4, 128), device="cuda").to(torch.bfloat16)
    k0 = torch.zeros((1, 0, 2, 128), dtype=torch.bfloat16, device="cuda")
    o, lse = b.attn_fwd(q, k0, k0)
    dq, dk, dv = b.attn_bwd(q, k0, k0, o, torch.randn_like(q), lse)
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and dk.numel() == 0 and dv.numel() == 0
    q0 = torch.zeros((1, 0, 4, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.randn((1, 70, 2, 128), device="cuda").to(torch.bfloat16)
    o0, lse0 = b.attn_fwd(q0, k, k, causal=True)
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(k, 7.0)
    _, dk, dv = b.attn_bwd(q0, k, k, o0, torch.zeros_like(q0), lse0, causal=True, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)
