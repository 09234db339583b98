#!/usr/bin/env python3
"""Benchmark of the exact-attention hot path on one MI355X (gfx950).

A step is one forward and one backward pass over the Llama-3.1-8B-shaped
training attention (B=1, Hq=32, Hkv=8, S=2048, D=128, bf16, causal): attn_fwd,
then the four stages of attn_bwd.  Inputs are seeded synthetic N(0, 1) bf16
tensors resident in device memory before timing starts.  W untimed steps, then
K timed steps between two device synchronisations.  Throughput counts
4*D flops per allowed (query, key) pair and head for the forward and 2.5x that
for the backward (QK^T, PV; and QK^T, dO V^T, P^T dO, dS^T Q, dS K).

Besides the headline line the JSON carries:
  roofline      the dominant kernel's achieved rate against the bf16 MFMA
                peak, timed with HIP events around that kernel's own launches
                inside the timed steps;
  kernels       per-launch times and rates from a separate untimed pass with
                events around every launch (each event drains the queue, so
                these read a few microseconds high; the dominant kernel's
                entry is the timed-step value);
  extra         the other workloads: split-K decode over a KV cache (HBM
                GB/s, 8 rotating cache copies so the 256 MB last-level cache
                cannot hold the working set; contiguous and in 256-row pages
                through a random block table), long-context local attention
                with ALiBi / softcap, the packed-document block-sparse mask
                (device mask build and forward);
  cpu_baseline  the fp64 CPU oracle timed on this host's cores: one full step
                of the same workload (value) and every other workload
                (per_config), with the core count, CPU model and BLAS.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra]
                       [--no-cpu-baseline] [--copy-calibration]
"""

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

METRIC = ("attention fwd/bwd TFLOP/s and % bf16 MFMA peak; decode HBM GB/s (1 MI355X)")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
ROOT = os.path.dirname(os.path.abspath(__file__))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (256 MiB read, 256 MiB "
                         "written per launch), the reference for HBM byte counters")
    return ap.parse_args()


def copy_calibration():
    """A plain elementwise copy (dst = src * 1) of 256 MiB, five launches: the
    known-size kernel that scales the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 64 << 20  # fp32 elements = 256 MiB
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_launch": 4 * n,
                                           "bytes_written_per_launch": 4 * n, "launches": 5}}))


class Prepared:
    """ctypes argument tuples built once, so the timed loop only enqueues."""

    def __init__(self, fn, args):
        self.fn = fn
        self.args = args

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            from exact_attention_10_amd import binding
            raise binding.AttnError(st, binding.library().attn_last_error().decode())


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "exact_attention_10_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, src_hash, per_launch_units):
    """HBM bytes per launch from committed counter summaries, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or rec.get("source_hash") != src_hash:
        return None
    return rec["bytes_per_launch"]


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py measures one GPU; runs on %d GPUs are not part of this benchmark "
              "(the kernels shard by batch and kv head with no communication)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    sys.path.insert(0, ROOT)
    from exact_attention_10_amd import binding as b
    from exact_attention_10_amd import inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lib = b.library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---------------- headline workload: fwd + bwd, B1 Hq32 Hkv8 S2048 D128 causal
    w = inputs.llama8b_train()
    q, k, v, do = (to_dev(w[n]) for n in ("q", "k", "v", "do"))
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    p = b._params(q, k, D, w["scale"], True, (-1, -1), None, 0.0, None)
    ws_bytes = lib.attn_bwd_workspace_size(ctypes.byref(p))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    T = b._tensor
    fwd = Prepared(lib.attn_fwd, (ctypes.byref(p), T(q), T(k), T(v), T(o), b._ptr(lse), None,
                                  None, 0, stream))
    bwd_args = (ctypes.byref(p), T(q), T(k), T(v), T(o), T(do), b._ptr(lse), T(dq), T(dk), T(dv),
                1, b._ptr(ws), ws_bytes)
    stages = [Prepared(lib.attn_bwd_stage, bwd_args + (st, stream)) for st in range(4)]

    pairs = S * (S + 1) // 2
    fwd_flops = 4.0 * B * Hq * D * pairs
    bwd_flops = 2.5 * fwd_flops
    # attn_bwd_stage 0..3 of the deterministic schedule: dQ (with Delta and
    # lse2), dK/dV, group sum, and an empty last stage
    launches = [("fwd", fwd)] + list(zip(["bwd_dq", "bwd_dkdv", "bwd_group_sum", "bwd_stage3"], stages))
    # Contractions each kernel executes per allowed pair and head (recomputed
    # products included): forward QK^T, PV; dK/dV: QK^T, dO V^T, P^T dO,
    # dS^T Q; dQ: QK^T, dO V^T, dS K.  Of the backward's five counted
    # contractions (QK^T, dO V^T, P^T dO, dS^T Q, dS K) dK/dV is credited the
    # first four and dQ only dS K (its QK^T and dO V^T are recomputation).
    kernel_flops = {"fwd": fwd_flops, "bwd_dkdv": 2.0 * fwd_flops, "bwd_dq": 1.5 * fwd_flops}
    kernel_flops_counted = {"fwd": fwd_flops, "bwd_dkdv": 2.0 * fwd_flops, "bwd_dq": 0.5 * fwd_flops}
    src = {"fwd": ("fwd_bf16.hip", "common.h"), "bwd_dkdv": ("bwd_bf16.hip", "common.h"),
           "bwd_dq": ("bwd_bf16.hip", "common.h")}

    # A timing event costs a few microseconds of GPU time (the queue drains at
    # each one), so the timed steps carry events around the dominant kernel
    # only; the per-kernel breakdown comes from a separate pass with events
    # around every launch.
    dom_name = [None]

    def step(ev_all=None, ev_dom=None):
        for i, (n, fn) in enumerate(launches):
            if ev_all is not None:
                ev_all[i].record()
            if ev_dom is not None and n == dom_name[0]:
                ev_dom[0].record()
                fn()
                ev_dom[1].record()
            else:
                fn()
        if ev_all is not None:
            ev_all[len(launches)].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # breakdown pass (not timed)
    n_l = len(launches)
    bd = [[torch.cuda.Event(enable_timing=True) for _ in range(n_l + 1)] for _ in range(10)]
    for e in bd:
        step(ev_all=e)
    torch.cuda.synchronize()
    per_kernel_ms = {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in bd]))
                     for i, (n, _) in enumerate(launches)}
    dom = max(kernel_flops, key=lambda n: per_kernel_ms[n])
    dom_name[0] = dom

    # timed steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev_dom=evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    dom_ms = float(np.mean([a.elapsed_time(z) for a, z in evs]))
    value = (fwd_flops + bwd_flops) / (ms_per_step * 1e-3) / 1e12

    kernels = {}
    for n, ms in per_kernel_ms.items():
        if n == dom:
            ms = dom_ms  # measured inside the timed steps
        rec = {"ms": round(ms, 5)}
        if n in kernel_flops:
            rec["tflops_executed"] = round(kernel_flops[n] / (ms * 1e-3) / 1e12, 2)
            rec["tflops_counted"] = round(kernel_flops_counted[n] / (ms * 1e-3) / 1e12, 2)
        kernels[n] = rec
    bwd_ms = sum(kernels[n]["ms"] for n, _ in launches[1:])
    kernels["bwd_total"] = {"ms": round(bwd_ms, 5),
                            "tflops_counted": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 2)}

    achieved = kernel_flops[dom] / (dom_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": traffic_for(dom, source_hash(*src[dom]), 1)}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3.1-8b attention fwd+bwd: B=1 Hq=32 Hkv=8 S=2048 D=128 "
                               "causal bf16", "global_batch": B, "seq_len": S,
                   "parallelism": "none (1 GPU)"},
        "frac_of_bf16_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roofline,
        "kernels": kernels,
        # SHA-256 of the bf16 bytes of each seeded input as uploaded
        "inputs_sha256": {n: hashlib.sha256(np.ascontiguousarray(w[n]).tobytes()).hexdigest()
                          for n in ("q", "k", "v", "do")},
    }

    # the same backward with deterministic=0 (dQ by fp32 atomic adds in the
    # dK/dV kernel, then a scale-and-round pass): per-stage times
    nd_args = bwd_args[:10] + (0,) + bwd_args[11:]
    nd = [Prepared(lib.attn_bwd_stage, nd_args + (st, stream)) for st in range(4)]
    nd_ev = []
    for rep in range(7):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        for i, st in enumerate(nd):
            ev[i].record()
            st()
        ev[4].record()
        if rep >= 2:
            nd_ev.append(ev)
    torch.cuda.synchronize()
    nd_ms = [float(np.median([e[i].elapsed_time(e[i + 1]) for e in nd_ev])) for i in range(4)]
    out["bwd_deterministic0"] = {
        "stage_ms": dict(zip(["delta_and_zero", "dkdv_with_atomic_dq", "group_sum", "dq_convert"],
                             [round(x, 5) for x in nd_ms])),
        "total_ms": round(sum(nd_ms), 5),
        "deterministic1_total_ms": round(bwd_ms, 5)}

    del ws, dq, dk, dv
    if not args.no_extra:
        out["extra"] = extra_workloads(b, lib, inputs, torch, np, dev, to_dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, fwd_flops + bwd_flops)
    print(json.dumps(out), flush=True)


def timed(torch, np, fn, reps, warm=2):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(reps)]
    for s, e in evs:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    ts = [s.elapsed_time(e) for s, e in evs]
    return float(np.median(ts)), float(np.min(ts))


def timed_batch(torch, fn, n):
    """GPU time per call of n back-to-back calls between two events (the
    queue stays full, so per-call event overhead is not part of it)."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def graph_timed(torch, np, make_calls, reps=10):
    """GPU time per call of a short call sequence: the calls (built for the
    given stream) are captured once into a HIP graph and the graph is
    replayed; host launch overhead is not part of the figure.  Returns
    (ms per call, the eager and replayed outputs of the last call agree)."""
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        calls, out = make_calls(ctypes.c_void_p(st.cuda_stream))
        for c in calls:
            c()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=st):
        for c in calls:
            c()
    g.replay()
    torch.cuda.synchronize()
    same = bool(torch.equal(out, eager))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(st):
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * len(calls)), same


def extra_workloads(b, lib, inputs, torch, np, dev, to_dev):
    ex = {}
    # decode: B=32, Hq=128, Hkv=1, D=128, cache lengths in [1024, 8192]
    w = inputs.decode_mqa()
    lens = torch.from_numpy(w["cache_seqlens"]).to(dev)
    total = int(w["cache_seqlens"].sum())
    Bd, _, Hqd, Dd = w["q"].shape
    copies = []
    for _ in range(8):
        copies.append((to_dev(w["q"]), to_dev(w["k"]), to_dev(w["v"])))
    o = torch.empty_like(copies[0][0])
    lse = torch.empty((Bd, Hqd, 1), dtype=torch.float32, device=dev)
    ws = torch.empty(b.decode_workspace_size(copies[0][0], copies[0][1]), dtype=torch.uint8,
                     device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    calls = []
    for qq, kk, vv in copies:
        p = b._params(qq, kk, Dd, w["scale"], False, (-1, -1), None, 0.0, None)
        calls.append(Prepared(lib.attn_decode, (ctypes.byref(p), b._tensor(qq), b._tensor(kk),
                                                b._tensor(vv), b._ptr(lens), 0, b._tensor(o),
                                                b._ptr(lse), b._ptr(ws), ws.numel(), stream)))
        calls[-1].keep = p
    it = [0]

    def dec():
        calls[it[0] % 8]()
        it[0] += 1

    med, mn = timed(torch, np, dec, 40)

    def make_dec(st):
        cs = []
        for qq, kk, vv in copies:
            p = b._params(qq, kk, Dd, w["scale"], False, (-1, -1), None, 0.0, None)
            cs.append(Prepared(lib.attn_decode, (ctypes.byref(p), b._tensor(qq), b._tensor(kk),
                                                 b._tensor(vv), b._ptr(lens), 0, b._tensor(o),
                                                 b._ptr(lse), b._ptr(ws), ws.numel(), st)))
            cs[-1].keep = p
        return cs, o

    gms, gsame = graph_timed(torch, np, make_dec)
    algo_bytes = total * Dd * 2 * 2 + 2 * Bd * Hqd * Dd * 2 + Bd * Hqd * 4
    ex["decode_mqa_b32_h128"] = {
        "ms": round(gms, 5), "graph_replay_matches_eager": gsame,
        "ms_eager_launches": round(med, 5), "ms_eager_min": round(mn, 5),
        "hbm_gbs": round(algo_bytes / (gms * 1e-3) / 1e9, 1),
        "frac_of_hbm_peak": round(algo_bytes / (gms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "tflops": round(4.0 * Hqd * Dd * total / (gms * 1e-3) / 1e12, 2),
        "algorithmic_bytes": algo_bytes}
    del copies

    # the same decode over a paged cache (256-row pages, seeded random block table)
    inputs.to_pages(w, 256)
    table = torch.from_numpy(w["block_table"]).to(dev)
    pcopies = [(to_dev(w["q"]), to_dev(w["k_pages"]), to_dev(w["v_pages"])) for _ in range(8)]
    pcalls = []
    for qq, kk, vv in pcopies:
        p = b._params(qq, kk, Dd, w["scale"], False, (-1, -1), None, 0.0, None)
        p.Sk = w["block_table"].shape[1] * 256
        kv = b.attn_kvcache()
        kv.block_table = table.data_ptr()
        kv.max_blocks = w["block_table"].shape[1]
        kv.page_size = 256
        kv.num_pages = kk.shape[0]
        pcalls.append(Prepared(lib.attn_decode_kvcache,
                               (ctypes.byref(p), b._tensor(qq), b._tensor(kk), b._tensor(vv),
                                b._ptr(lens), ctypes.byref(kv), 0, b._tensor(o), b._ptr(lse),
                                b._ptr(ws), ws.numel(), stream)))
        pcalls[-1].keep = (p, kv)
    it[0] = 0

    def decp():
        pcalls[it[0] % 8]()
        it[0] += 1

    med, mn = timed(torch, np, decp, 40)

    def make_decp(st):
        cs = []
        for qq, kk, vv in pcopies:
            p = b._params(qq, kk, Dd, w["scale"], False, (-1, -1), None, 0.0, None)
            p.Sk = w["block_table"].shape[1] * 256
            kv = b.attn_kvcache()
            kv.block_table = table.data_ptr()
            kv.max_blocks = w["block_table"].shape[1]
            kv.page_size = 256
            kv.num_pages = kk.shape[0]
            cs.append(Prepared(lib.attn_decode_kvcache,
                               (ctypes.byref(p), b._tensor(qq), b._tensor(kk), b._tensor(vv),
                                b._ptr(lens), ctypes.byref(kv), 0, b._tensor(o), b._ptr(lse),
                                b._ptr(ws), ws.numel(), st)))
            cs[-1].keep = (p, kv)
        return cs, o

    gms, gsame = graph_timed(torch, np, make_decp)
    ex["decode_mqa_b32_h128_paged256"] = {
        "ms": round(gms, 5), "graph_replay_matches_eager": gsame,
        "ms_eager_launches": round(med, 5), "ms_eager_min": round(mn, 5),
        "hbm_gbs": round(algo_bytes / (gms * 1e-3) / 1e9, 1),
        "frac_of_hbm_peak": round(algo_bytes / (gms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}

    # speculative decoding on the same paged cache: 4 draft tokens per sequence
    # (seeded normals, seed 63) are appended in place and attend causally,
    # bottom-right aligned; Sq = 4, so 512 rows = 4 jobs per sequence
    Sd = 4
    rng = np.random.default_rng(63)
    lens_d = torch.from_numpy(w["cache_seqlens"] - Sd).to(dev)
    q4 = to_dev(inputs.f32_to_bf16_bits(rng.standard_normal((Bd, Sd, Hqd, Dd), dtype=np.float32)))
    kn = to_dev(inputs.f32_to_bf16_bits(rng.standard_normal((Bd, Sd, 1, Dd), dtype=np.float32)))
    vn = to_dev(inputs.f32_to_bf16_bits(rng.standard_normal((Bd, Sd, 1, Dd), dtype=np.float32)))
    o4 = torch.empty_like(q4)
    lse4 = torch.empty((Bd, Hqd, Sd), dtype=torch.float32, device=dev)

    def spec_params(kk):
        p = b._params(q4, kk, Dd, w["scale"], True, (-1, -1), None, 0.0, None)
        p.Sk = w["block_table"].shape[1] * 256
        kv = b.attn_kvcache()
        kv.block_table = table.data_ptr()
        kv.max_blocks = w["block_table"].shape[1]
        kv.page_size = 256
        kv.num_pages = kk.shape[0]
        kv.k_new, kv.v_new, kv.s_new = b._tensor(kn), b._tensor(vn), Sd
        return p, kv

    p4, _ = spec_params(pcopies[0][1])
    ws4 = torch.empty(lib.attn_decode_workspace_size(ctypes.byref(p4), 0), dtype=torch.uint8, device=dev)

    def make_spec(st):
        cs = []
        for _, kk, vv in pcopies:
            p, kv = spec_params(kk)
            cs.append(Prepared(lib.attn_decode_kvcache,
                               (ctypes.byref(p), b._tensor(q4), b._tensor(kk), b._tensor(vv),
                                b._ptr(lens_d), ctypes.byref(kv), 0, b._tensor(o4), b._ptr(lse4),
                                b._ptr(ws4), ws4.numel(), st)))
            cs[-1].keep = (p, kv)
        return cs, o4

    gms, gsame = graph_timed(torch, np, make_spec)
    seen = int(sum(Sd * int(n) - Sd * (Sd - 1) // 2 for n in w["cache_seqlens"]))
    spec_bytes = total * Dd * 2 * 2 + 2 * Bd * Sd * Hqd * Dd * 2 + Bd * Hqd * Sd * 4 + 4 * Bd * Sd * Dd * 2
    ex["specdecode_mqa_b32_h128_q4_paged256"] = {
        "ms": round(gms, 5), "graph_replay_matches_eager": gsame,
        "hbm_gbs": round(spec_bytes / (gms * 1e-3) / 1e9, 1),
        "frac_of_hbm_peak": round(spec_bytes / (gms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "tflops": round(4.0 * Hqd * Dd * seen / (gms * 1e-3) / 1e12, 2),
        "algorithmic_bytes": spec_bytes}
    del pcopies, o, ws, q4, kn, vn, o4, ws4

    # long-context local attention: S=16384, causal + window (4096, 0)
    w = inputs.long_local()
    q, k, v = to_dev(w["q"]), to_dev(w["k"]), to_dev(w["v"])
    oo = torch.empty_like(q)
    ll = torch.empty((1, 32, 16384), dtype=torch.float32, device=dev)
    slopes = torch.from_numpy(w["alibi_slopes"]).to(dev)
    pairs = 4096 * 4097 // 2 + (16384 - 4096) * 4097
    fl = 4.0 * 32 * 128 * pairs
    for name, kw in (("alibi", dict(alibi_slopes=slopes)), ("softcap50", dict(softcap=50.0))):
        med, _ = timed(torch, np, lambda: b.attn_fwd(q, k, v, softmax_scale=w["scale"], causal=True,
                                                     window=(4096, 0), out=oo, lse=ll, **kw), 5)
        ex["long_local_s16384_w4096_" + name] = {
            "ms": round(med, 4), "tflops": round(fl / (med * 1e-3) / 1e12, 2),
            "frac_of_bf16_peak": round(fl / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del q, k, v, oo, ll

    # packed-document block-sparse mask: B=2, H=16, S=8192, D=64
    w = inputs.doc_mask()
    q, k, v = to_dev(w["q"]), to_dev(w["k"]), to_dev(w["v"])
    doc = torch.from_numpy(w["doc"]).to(dev)
    m = b.block_mask_build(2, 8192, 8192, 128, 128, causal=True, doc_q=doc, doc_k=doc)
    # the build alone: the C call on a preallocated buffer
    desc = b.attn_mask_desc()
    desc.causal, desc.window_left, desc.window_right = 1, -1, -1
    desc.doc_q = desc.doc_k = doc.data_ptr()
    mout = b.attn_block_mask()
    nbytes = lib.attn_block_mask_bytes(2, 8192, 8192, 128, 128)
    mbuf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    build = Prepared(lib.block_mask_build, (ctypes.byref(desc), 2, 8192, 8192, 128, 128,
                                            b._ptr(mbuf), nbytes, ctypes.byref(mout),
                                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
    med_m, _ = timed(torch, np, build, 10)
    batch_m = timed_batch(torch, build, 50)
    same = all(torch.equal(x, y) for x, y in zip(m.arrays().values(),
                                                  b.BlockMask(mout, mbuf, doc, doc).arrays().values()))
    oo = torch.empty_like(q)
    ll = torch.empty((2, 16, 8192), dtype=torch.float32, device=dev)
    med, _ = timed(torch, np, lambda: b.attn_fwd(q, k, v, softmax_scale=w["scale"], block_mask=m,
                                                 out=oo, lse=ll), 10)
    pairs = sum(n * (n + 1) // 2 for lens_b in w["doc_lengths"] for n in lens_b)
    fl = 4.0 * 16 * 64 * pairs
    # block-sparse backward on the same mask (dO: seeded normals, seed 44)
    rng = np.random.default_rng(44)
    do = to_dev(inputs.f32_to_bf16_bits(rng.standard_normal(w["q"].shape, dtype=np.float32)))
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    pb = b._params(q, k, 64, w["scale"], False, (-1, -1), None, 0.0, m)
    wsb = torch.empty(lib.attn_bwd_workspace_size(ctypes.byref(pb)), dtype=torch.uint8, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    bwd_call = Prepared(lib.attn_bwd, (ctypes.byref(pb), b._tensor(q), b._tensor(k), b._tensor(v),
                                       b._tensor(oo), b._tensor(do), b._ptr(ll), b._tensor(gq),
                                       b._tensor(gk), b._tensor(gv), 1, b._ptr(wsb), wsb.numel(), stream))
    med_b, _ = timed(torch, np, bwd_call, 10)
    ex["doc_mask_s8192_d64"] = {"block_mask_build_ms": round(batch_m, 4),
                                "block_mask_build_single_call_ms": round(med_m, 4),
                                "block_mask_repeat_equal": same,
                                "fwd_ms": round(med, 4),
                                "tflops": round(fl / (med * 1e-3) / 1e12, 2),
                                "frac_of_bf16_peak": round(fl / (med * 1e-3) / 1e12 /
                                                           PEAK_BF16_TFLOPS, 4),
                                "bwd_ms": round(med_b, 4),
                                "bwd_tflops_counted": round(2.5 * fl / (med_b * 1e-3) / 1e12, 2)}
    return ex


def cpu_identity():
    """Host cores this process may use, the CPU model and numpy's BLAS."""
    cores = len(os.sched_getaffinity(0))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                blas = "%s %s" % (i.get("internal_api"), i.get("version"))
                break
    except Exception:
        pass
    return cores, model, blas


def cpu_baseline(w, step_flops):
    """The fp64 oracle (as it stands) on this host's cores, per workload: a
    thread pool over independent (batch, head-group[, row block]) units, one
    BLAS thread per worker (numpy releases the GIL inside BLAS and ufuncs).
    Every workload is run whole except the long-context one, which runs 8 of
    its 32 query heads per modifier (scaled by 4)."""
    import concurrent.futures
    sys.path.insert(0, ROOT)
    import numpy as np
    import oracle
    from exact_attention_10_amd import inputs
    cores, model, blas = cpu_identity()
    workers = max(1, min(cores, 16))
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1)
    except Exception:
        limit = None

    def run(units):
        t0 = time.perf_counter()
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(lambda f: f(), units))
        return time.perf_counter() - t0

    per = {}
    # tiny dense forward, fp32 inputs: B=1 Hq=Hkv=2 S=128 D=64
    t = inputs.tiny_dense()
    f = {n: inputs.as_f64(t[n], t["dtype"]) for n in ("q", "k", "v")}
    dt = run([lambda h=h: oracle.attention_fwd_rows(f["q"], f["k"], f["v"], 0, h, np.arange(128),
                                                     scale=t["scale"]) for h in range(2)])
    per["tiny_dense_fwd"] = {"seconds": round(dt, 4)}
    # the headline workload, forward and backward (units: kv-head groups)
    q, k, v, do = (inputs.as_f64(w[n], "bf16") for n in ("q", "k", "v", "do"))
    G = q.shape[2] // k.shape[2]
    grp = [(slice(G * g, G * g + G), slice(g, g + 1)) for g in range(k.shape[2])]
    dt_f = run([lambda hs=hs, ks=ks: oracle.attention_fwd(q[:, :, hs], k[:, :, ks], v[:, :, ks],
                                                           scale=w["scale"], causal=True)
                for hs, ks in grp])
    dt_b = run([lambda hs=hs, ks=ks: oracle.attention_bwd(q[:, :, hs], k[:, :, ks], v[:, :, ks],
                                                           do[:, :, hs], scale=w["scale"], causal=True)
                for hs, ks in grp])
    fwd_flops = step_flops / 3.5
    per["llama8b_fwd"] = {"seconds": round(dt_f, 3), "tflops": round(fwd_flops / dt_f / 1e12, 5)}
    per["llama8b_bwd"] = {"seconds": round(dt_b, 3), "tflops": round(2.5 * fwd_flops / dt_b / 1e12, 5)}
    # long-context local attention (8 of 32 heads, x4), ALiBi and softcap runs
    ll = inputs.long_local()
    q3, k3, v3 = (inputs.as_f64(ll[n], "bf16") for n in ("q", "k", "v"))
    pairs3 = 4096 * 4097 // 2 + (16384 - 4096) * 4097
    for name, kw in (("alibi", dict(alibi_slopes=ll["alibi_slopes"])), ("softcap50", dict(softcap=50.0))):
        units = [lambda h=h, r0=r0: oracle.attention_fwd_rows(q3, k3, v3, 0, h, np.arange(r0, r0 + 2048),
                                                               scale=ll["scale"], causal=True,
                                                               window=(4096, 0), **kw)
                 for h in range(0, 32, 4) for r0 in range(0, 16384, 2048)]
        dt = 4.0 * run(units)
        per["long_local_" + name + "_fwd"] = {"seconds": round(dt, 3),
                                              "tflops": round(4.0 * 32 * 128 * pairs3 / dt / 1e12, 5),
                                              "measured_heads": 8}
    del q3, k3, v3
    # packed-document mask forward (documents are independent: one unit per document)
    dm = inputs.doc_mask()
    q4, k4, v4 = (inputs.as_f64(dm[n], "bf16") for n in ("q", "k", "v"))
    units = []
    for bb in range(2):
        s0 = 0
        for n in dm["doc_lengths"][bb]:
            sl = slice(s0, s0 + n)
            units.append(lambda bb=bb, sl=sl: oracle.attention_fwd(q4[bb:bb + 1, sl], k4[bb:bb + 1, sl],
                                                                   v4[bb:bb + 1, sl], scale=dm["scale"],
                                                                   causal=True))
            s0 += n
    dt = run(units)
    pairs4 = sum(n * (n + 1) // 2 for lb in dm["doc_lengths"] for n in lb)
    per["doc_mask_fwd"] = {"seconds": round(dt, 3), "tflops": round(4.0 * 16 * 64 * pairs4 / dt / 1e12, 5)}
    del q4, k4, v4
    # MQA decode over the cache (one unit per sequence)
    dc = inputs.decode_mqa()
    q5, k5, v5 = (inputs.as_f64(dc[n], "bf16") for n in ("q", "k", "v"))
    lens = dc["cache_seqlens"]
    dt = run([lambda bb=bb: oracle.decode(q5[bb:bb + 1], k5[bb:bb + 1], v5[bb:bb + 1], lens[bb:bb + 1],
                                          scale=dc["scale"]) for bb in range(len(lens))])
    dec_bytes = int(lens.sum()) * 128 * 2 * 2 + 2 * 32 * 128 * 128 * 2 + 32 * 128 * 4
    per["decode_mqa"] = {"seconds": round(dt, 4), "gbs": round(dec_bytes / dt / 1e9, 3)}
    if limit is not None:
        limit.unregister() if hasattr(limit, "unregister") else None
    step_s = dt_f + dt_b
    return {"value": round(step_flops / step_s / 1e12, 5), "unit": "TFLOP/s", "cores": workers,
            "kind": "oracle", "seconds": round(step_s, 3), "cpu_model": model,
            "host_cores_available": cores, "blas": blas, "per_config": per,
            "sample": "value: one full fwd+bwd step of the B=1 Hq=32 Hkv=8 S=2048 D=128 causal "
                      "workload (fp64 numpy oracle, %d worker threads over kv-head groups, one BLAS "
                      "thread each); per_config: every workload whole except the 16K window one "
                      "(8 of 32 heads, scaled x4)" % workers}


if __name__ == "__main__":
    main()
