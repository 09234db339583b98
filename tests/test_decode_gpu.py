"""GPU parity of split-K decode over a KV cache against the unsplit fp64
oracle (through the C ABI via the ctypes binding)."""

import numpy as np
import pytest

import oracle
from exact_attention_10_amd import inputs
from helpers import check_lse, check_o, f64, to_device, to_f64

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_attention_10_amd import binding
    return binding


def run_decode(b, w, **kw):
    q = to_device(w["q"], "bf16", torch)
    k = to_device(w["k"], "bf16", torch)
    v = to_device(w["v"], "bf16", torch)
    lens = torch.from_numpy(np.asarray(w["cache_seqlens"], dtype=np.int32)).cuda()
    o, lse = b.attn_decode(q, k, v, lens, **kw)
    torch.cuda.synchronize()
    return o, lse


def test_decode_mqa_full(b):
    """B=32, Hq=128, Hkv=1, D=128, cache lengths in [1024, 8192]: every
    output against the unsplit oracle, default split plan and an explicit one."""
    w = inputs.decode_mqa()
    O, L = oracle.decode(f64(w, "q"), f64(w, "k"), f64(w, "v"), w["cache_seqlens"],
                         scale=w["scale"])
    for splits in (0, 1, 3, 40, 5000):
        o, lse = run_decode(b, w, softmax_scale=w["scale"], num_splits=splits)
        check_o(to_f64(o), O, what="O(splits=%d)" % splits)
        check_lse(to_f64(lse), L)


@pytest.mark.parametrize("cfg", [
    dict(B=3, Hq=8, Hkv=2, D=64, Smax=500, lens=[1, 77, 500]),
    dict(B=2, Hq=256, Hkv=1, D=128, Smax=300, lens=[300, 129]),
    dict(B=4, Hq=16, Hkv=16, D=128, Smax=200, lens=[0, 64, 65, 199]),
    dict(B=2, Hq=40, Hkv=8, D=64, Smax=1000, lens=[999, 1000], softcap=3.0),
    dict(B=600, Hq=8, Hkv=8, D=64, Smax=40, lens="random"),
    dict(B=3, Hq=320, Hkv=1, D=128, Smax=100, lens=[100, 1, 33]),
    # more sequences than threads in a workgroup: the schedule scan runs in
    # several passes, and lengths past the LDS window are read from memory
    dict(B=700, Hq=8, Hkv=8, D=64, Smax=24, lens="random"),
])
def test_decode_ragged(b, cfg):
    """Ragged cache lengths (1, tile edges, empty caches), GQA groups that
    do not fill a 128-head job or span several, softcap, one workgroup over
    hundreds of sequences, more workgroups than key steps, more sequences than
    a workgroup has threads."""
    w = inputs.decode_mqa(seed=11, B=cfg["B"], Hq=cfg["Hq"], Smax=cfg["Smax"], D=cfg["D"],
                          lmin=1, lmax=cfg["Smax"])
    if cfg["Hkv"] > 1:
        rng = np.random.default_rng(12)
        shape = (cfg["B"], cfg["Smax"], cfg["Hkv"], cfg["D"])
        w["k"] = inputs.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
        w["v"] = inputs.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    if cfg["lens"] == "random":  # many short caches, some empty: one workgroup spans hundreds
        w["cache_seqlens"] = np.random.default_rng(13).integers(0, cfg["Smax"] + 1, cfg["B"]).astype(np.int32)
    else:
        w["cache_seqlens"] = np.array(cfg["lens"], dtype=np.int32)
    cap = cfg.get("softcap", 0.0)
    for splits in (0, 1, 7, 65536):
        o, lse = run_decode(b, w, softmax_scale=0.1, softcap=cap, num_splits=splits)
        O, L = oracle.decode(f64(w, "q"), f64(w, "k"), f64(w, "v"), w["cache_seqlens"],
                             scale=0.1, softcap=cap)
        check_o(to_f64(o), O)
        check_lse(to_f64(lse), L)


def test_decode_deterministic(b):
    w = inputs.decode_mqa()
    o1, l1 = run_decode(b, w, softmax_scale=w["scale"])
    o2, l2 = run_decode(b, w, softmax_scale=w["scale"])
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_status_length_out_of_range(b):
    """A cache length outside [0, Smax] is clamped on the device and reported
    in bit 1 of the workspace status word (which the kernels never clear);
    in-range lengths leave the word at 0.  Outputs follow the clamped
    lengths."""
    w = inputs.decode_mqa(seed=15, B=4, Hq=16, Smax=256, D=128, lmin=1, lmax=256)
    q, k, v = (to_device(w[n], "bf16", torch) for n in ("q", "k", "v"))
    ws = torch.zeros(b.decode_workspace_size(q, k), dtype=torch.uint8, device="cuda")
    lens = torch.tensor([10, 256, 3, 100], dtype=torch.int32, device="cuda")
    b.attn_decode(q, k, v, lens, softmax_scale=0.1, workspace=ws)
    assert b.decode_status(ws) == 0
    bad = np.array([-5, 300, 3, 100], dtype=np.int32)
    o, lse = b.attn_decode(q, k, v, torch.from_numpy(bad).cuda(), softmax_scale=0.1, workspace=ws)
    torch.cuda.synchronize()
    assert b.decode_status(ws) & 1
    O, L = oracle.decode(f64(w, "q"), f64(w, "k"), f64(w, "v"), np.clip(bad, 0, 256), scale=0.1)
    check_o(to_f64(o), O)
    check_lse(to_f64(lse), L)
    # sticky: a later clean call leaves the bit set until the caller clears it
    b.attn_decode(q, k, v, lens, softmax_scale=0.1, workspace=ws)
    assert b.decode_status(ws) & 1
    ws.zero_()
    b.attn_decode(q, k, v, lens, softmax_scale=0.1, workspace=ws)
    assert b.decode_status(ws) == 0


def test_decode_status_append_overflow(b):
    """With an in-place append of s_new rows, a length above Smax - s_new is
    clamped (the new rows then overwrite the last cached rows) and flagged."""
    B, Hq, Hkv, D, Smax, s_new = 2, 8, 1, 128, 64, 4
    w = inputs.decode_mqa(seed=16, B=B, Hq=Hq, Smax=Smax, D=D, lmin=1, lmax=Smax)
    q, k, v = (to_device(w[n], "bf16", torch) for n in ("q", "k", "v"))
    rng = np.random.default_rng(17)
    kn = torch.from_numpy(rng.standard_normal((B, s_new, Hkv, D), dtype=np.float32)).to(torch.bfloat16).cuda()
    vn = torch.from_numpy(rng.standard_normal((B, s_new, Hkv, D), dtype=np.float32)).to(torch.bfloat16).cuda()
    ws = torch.zeros(b.decode_workspace_size(q, k), dtype=torch.uint8, device="cuda")
    lens = torch.tensor([Smax - s_new, 7], dtype=torch.int32, device="cuda")
    b.attn_decode(q, k.clone(), v.clone(), lens, softmax_scale=0.1, k_new=kn, v_new=vn, workspace=ws)
    torch.cuda.synchronize()
    assert b.decode_status(ws) == 0
    lens = torch.tensor([Smax - s_new + 1, 7], dtype=torch.int32, device="cuda")
    b.attn_decode(q, k.clone(), v.clone(), lens, softmax_scale=0.1, k_new=kn, v_new=vn, workspace=ws)
    torch.cuda.synchronize()
    assert b.decode_status(ws) & 1


def test_decode_expired_wait_poisons_rows(b):
    """With the in-kernel wait bound at 0 (attn_debug_set_spin_limit) the
    decode ring's waits give up: the kernels still finish, bit 2 of the
    status word is set, the rows that may have read unsynchronised data are
    NaN in o and lse, and every other row is still correct.  The default
    bound gives a clean word and normal results again."""
    w = inputs.decode_mqa()
    q, k, v = (to_device(w[n], "bf16", torch) for n in ("q", "k", "v"))
    lens = torch.from_numpy(np.asarray(w["cache_seqlens"], dtype=np.int32)).cuda()
    ws = torch.zeros(b.decode_workspace_size(q, k), dtype=torch.uint8, device="cuda")
    try:
        b.set_spin_limit(0)
        o, lse = b.attn_decode(q, k, v, lens, softmax_scale=w["scale"], workspace=ws)
        torch.cuda.synchronize()
    finally:
        b.set_spin_limit(-1)
    assert b.decode_status(ws) & 2
    bad = torch.isnan(lse)  # [B, Hq, 1]
    assert bad.any()
    assert torch.equal(torch.isnan(o.float()).any(-1).permute(0, 2, 1), bad)
    O, L = oracle.decode(f64(w, "q"), f64(w, "k"), f64(w, "v"), w["cache_seqlens"], scale=w["scale"])
    good = (~bad).cpu().numpy()
    on = to_f64(o).transpose(0, 2, 1, 3)[good]
    check_o(on, O.transpose(0, 2, 1, 3)[good])
    check_lse(to_f64(lse)[good], L[good])
    ws.zero_()
    o2, l2 = b.attn_decode(q, k, v, lens, softmax_scale=w["scale"], workspace=ws)
    torch.cuda.synchronize()
    assert b.decode_status(ws) == 0
    check_o(to_f64(o2), O)
    check_lse(to_f64(l2), L)
