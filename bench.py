"""Benchmark of libdiffattn on one MI355X; prints one JSON line.

Headline (``value``): causal DiffAttn forward throughput in TFLOP/s on the
long-context workload B1 H16 N32768 d64 (V 128 wide), bf16, layer 12.  One step
is lambda + forward over that batch, with the inputs already resident in HBM.
FLOPs are counted as 12 d P per head (P = N(N+1)/2 causal pairs: two QK^T of
width d and two PV of width 2d), the work the exact blockwise algorithm executes.

Also reported in the same line:
  prefill - the same forward on the prefill workload B4 H8 N2048 d64 (bf16, layer 4,
            inputs scaled by 1/sqrt 2): kernel time, TFLOP/s and fraction of the peak.
  peaked  - the long-context forward on inputs 4x wider (N(0, 16)), whose rows often
            outgrow the fast pass's bound: time, ratio to normal inputs, rows flagged.
  decode  - one split-KV decode step, 64 sequences x 16 heads against caches of
            8192 tokens: HBM GB/s = (cache + query + output bytes) / step time.
  train   - forward (with saves) + backward on B8 H12 N4096 when the backward
            kernels are present: TFLOP/s under 12 d P + 20 d P per head.
  proj    - the projection GEMMs at the forward workload's shape (d_model = H 2d = 2048):
            the fused QKV projection (X [32768, 2048] x W [6144, 2048]^T, scattered into
            Q1/Q2/K1/K2/V) and the output projection (token-major Y [32768, 2048] x W_O^T),
            TFLOP/s at 2 M N K each against the bf16 peak, and the whole module step
            (projection, lambda, forward with token-major output, projection).
  ref_gemm - the box's best bf16 matrix-core rate through the vendor library (torch.matmul,
            8192^3), and the forward's rate as a fraction of it (a measured reference next to
            the nominal 2.5 PFLOP/s).
  copy    - a plain 2 GiB device-to-device copy: the HBM rate this machine reaches,
            and the kernel the HBM byte counters are calibrated on.
  roofline - for the dominant kernel (the forward), achieved TFLOP/s from HIP
            events around each forward launch in the timed region, against the
            bf16 dense MFMA peak of 2500 TFLOP/s; traffic = HBM bytes per launch
            from profiles/hbm_traffic.md when it was measured on the current source.
  cpu_baseline - the float64 oracle on the host cores (BLAS threads pinned to them), per
            workload on a bounded sample: whole heads (forward; forward and backward
            for training), whole decode sequences, the whole tiny workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--legs fwd,prefill,peaked,decode,train,proj,refgemm,copy]
                       [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DiffAttn fwd TFLOP/s + % bf16 MFMA peak; decode-step HBM GB/s"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def causal_pairs(n: int) -> int:
    return n * (n + 1) // 2


def fwd_flops(w) -> float:
    return 12.0 * w.head_dim * causal_pairs(w.seqlen) * w.batch * w.heads


def decode_bytes(w) -> int:
    bh = w.batch * w.heads
    cache = bh * w.seqlen * (w.head_dim * 2 + 2 * w.head_dim) * 2   # K1, K2, V bf16
    return cache + bh * 2 * w.head_dim * 2 + bh * 2 * w.head_dim * 2  # + q1, q2 + out


def time_steps(step, steps: int, warmup: int, inner_events=None):
    """Runs warmup + timed steps; returns (ms per step, list of inner kernel ms)."""
    import torch
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    inner = []
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(steps)] if inner_events else [None] * steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        step(pairs[i])
    stop.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    ms = start.elapsed_time(stop) / steps
    if inner_events:
        inner = [a.elapsed_time(b) for a, b in pairs]
    return ms, wall, inner


def leg_forward(steps, warmup, number=3):
    import torch
    from differential_attention_causal_amd import diffattn as da
    from differential_attention_causal_amd import synth
    w = synth.WORKLOADS[number]
    x = synth.make_inputs(w, "cuda:0")
    out = torch.empty_like(x["v"])
    p = da.problem(w.batch, w.heads, w.seqlen, w.head_dim, da.BF16)
    ws = torch.empty(da.workspace_bytes(da.OP_FWD, p), dtype=torch.uint8, device="cuda:0")
    torch.cuda.synchronize()

    def step(ev):
        st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
        if ev:
            ev[0].record()
        da.forward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st, out=out, workspace=ws)
        if ev:
            ev[1].record()

    ms, wall, inner = time_steps(step, steps, warmup, inner_events=True)
    fl = fwd_flops(w)
    kern_ms = sum(inner) / len(inner)
    achieved = fl / (kern_ms * 1e-3) / 1e12
    srt = sorted(inner)
    return w, {
        "ms_per_step": ms, "wall_ms_per_step": wall, "tflops": fl / (ms * 1e-3) / 1e12,
        "fwd_kernel_ms": kern_ms, "fwd_kernel_ms_median": srt[len(srt) // 2],
        "fwd_kernel_ms_min": srt[0], "flops_per_launch": fl,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": traffic_from_profiles("fwd_bf16_kernel<false, 2>", "fwd_bf16.hip", w.name)},
        "formula_tflops_8dP": fl * 8.0 / 12.0 / (ms * 1e-3) / 1e12,
    }


def leg_peaked(steps, warmup):
    """The long-context forward shape with Q, K and V drawn 4x wider (N(0, 16)): scores
    spread so far that many rows outgrow the fast pass's bound and are recomputed by the
    fixup pass. Reports the forward time, its ratio to the normal-input forward and the
    fraction of rows flagged."""
    import torch
    from differential_attention_causal_amd import diffattn as da
    from differential_attention_causal_amd import synth
    w = synth.custom("fwd", 1, 16, 32768, 64, 12, "bf16", scale=4.0, number=3)
    x = synth.make_inputs(w, "cuda:0")
    out = torch.empty_like(x["v"])
    p = da.problem(w.batch, w.heads, w.seqlen, w.head_dim, da.BF16)
    ws = torch.zeros(da.workspace_bytes(da.OP_FWD, p), dtype=torch.uint8, device="cuda:0")
    st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
    torch.cuda.synchronize()

    def step(ev):
        if ev:
            ev[0].record()
        da.forward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st, out=out, workspace=ws)
        if ev:
            ev[1].record()

    _, _, inner = time_steps(step, max(2, steps // 5), max(1, warmup // 5), inner_events=True)
    words = ws.view(torch.int32)
    flagged = int(sum(bin(int(v) & 0xffffffff).count("1") for v in words.cpu().tolist()))
    kern_ms = sum(inner) / len(inner)
    return {"workload": "long-context bf16 forward B1 H16 N32768 d64, inputs N(0, 16)",
            "fwd_kernel_ms": kern_ms, "tflops": fwd_flops(w) / (kern_ms * 1e-3) / 1e12,
            "rows_flagged": flagged, "rows": w.batch * w.heads * w.seqlen,
            "frac_rows_flagged": flagged / (w.batch * w.heads * w.seqlen)}


def leg_decode(steps, warmup):
    import torch
    from differential_attention_causal_amd import diffattn as da
    from differential_attention_causal_amd import synth
    w = synth.WORKLOADS[4]
    x = synth.make_inputs(w, "cuda:0")
    out = torch.empty(w.batch, w.heads, w.dv, dtype=torch.bfloat16, device="cuda:0")
    p = da.problem(w.batch, w.heads, w.seqlen, w.head_dim, da.BF16)
    ws = torch.empty(da.workspace_bytes(da.OP_DECODE, p), dtype=torch.uint8, device="cuda:0")
    torch.cuda.synchronize()

    def step(ev):
        st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
        if ev:
            ev[0].record()
        da.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st, out=out, workspace=ws)
        if ev:
            ev[1].record()

    ms, wall, inner = time_steps(step, steps, warmup, inner_events=True)
    nb = decode_bytes(w)
    kern_ms = sum(inner) / len(inner)
    gbs = nb / (kern_ms * 1e-3) / 1e9

    # The write half of a serving step: append one token per sequence to the caches
    # (each call starts from caches one row short of full, so every call writes).
    new = {k: x[k][:, :, 0].contiguous() for k in ("k1", "k2", "v")}
    full = torch.full((w.batch,), w.seqlen - 1, dtype=torch.int32, device="cuda:0")
    cl = full.clone()

    def append_step(ev):
        cl.copy_(full)
        if ev:
            ev[0].record()
        da.cache_append(new["k1"], new["k2"], new["v"], x["k1"], x["k2"], x["v"], cl)
        if ev:
            ev[1].record()

    _, _, app = time_steps(append_step, steps, warmup, inner_events=True)
    app_ms = sum(app) / len(app)

    # Grouped-query variant: the 16 query heads share 4 cache heads (a quarter of the
    # cache bytes per step).
    hkv = 4
    kv = {k: x[k][:, :hkv].contiguous() for k in ("k1", "k2", "v")}
    torch.cuda.synchronize()

    def gqa_step(ev):
        st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
        if ev:
            ev[0].record()
        da.decode(x["q1"], x["q2"], kv["k1"], kv["k2"], kv["v"], st, out=out, workspace=ws)
        if ev:
            ev[1].record()

    _, _, gq = time_steps(gqa_step, steps, warmup, inner_events=True)
    gq_ms = sum(gq) / len(gq)
    bh = w.batch * w.heads
    gq_bytes = (w.batch * hkv * w.seqlen * 4 * w.head_dim * 2 + 2 * bh * w.head_dim * 2 +
                bh * 2 * w.head_dim * 2)
    del kv
    app_bytes = 2 * w.batch * w.heads * (4 * w.head_dim) * 2   # rows read + rows written
    return {
        "workload": w.name, "value": nb / (ms * 1e-3) / 1e9, "unit": "GB/s",
        "ms_per_step": ms, "decode_ms": kern_ms, "bytes_per_step": nb,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS,
                     "traffic": traffic_from_profiles("decode_mfma_kernel", "decode.hip", w.name)},
        "gqa": {"workload": f"{w.name}, 4 cache heads (groups of 4)", "decode_ms": gq_ms,
                "bytes_per_step": gq_bytes, "GB_s": gq_bytes / (gq_ms * 1e-3) / 1e9,
                "frac": gq_bytes / (gq_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                "speedup_vs_mha": kern_ms / gq_ms},
        "append": {"us_per_call": app_ms * 1e3, "bytes": app_bytes,
                   "GB_s": app_bytes / (app_ms * 1e-3) / 1e9, "bound": "launch latency"},
    }


def leg_train(steps, warmup):
    import torch
    from differential_attention_causal_amd import diffattn as da
    from differential_attention_causal_amd import synth
    w = synth.WORKLOADS[5]
    x = synth.make_inputs(w, "cuda:0")
    sv = da.alloc_saved(w.batch, w.heads, w.seqlen, w.head_dim, "cuda:0")
    out = torch.empty_like(x["v"])
    p = da.problem(w.batch, w.heads, w.seqlen, w.head_dim, da.BF16)
    ws = torch.empty(max(16, da.workspace_bytes(da.OP_BWD, p)), dtype=torch.uint8,
                     device="cuda:0")
    wsf = torch.empty(da.workspace_bytes(da.OP_FWD, p), dtype=torch.uint8, device="cuda:0")
    torch.cuda.synchronize()

    def step(ev):
        st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
        da.forward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st, out=out, saved=sv,
                   workspace=wsf)
        if ev:
            ev[0].record()
        da.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lq1"], x["lk1"], x["lq2"],
                    x["lk2"], st, sv, x["dout"], workspace=ws)
        if ev:
            ev[1].record()

    ms, wall, inner = time_steps(step, steps, warmup, inner_events=True)
    pairs = causal_pairs(w.seqlen) * w.batch * w.heads
    fl = (12.0 + 20.0) * w.head_dim * pairs
    bwd_ms = sum(inner) / len(inner)
    bwd_tf = 20.0 * w.head_dim * pairs / (bwd_ms * 1e-3) / 1e12
    return {
        "workload": w.name, "value": fl / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
        "ms_per_step": ms, "bwd_ms": bwd_ms, "bwd_tflops": bwd_tf,
        # The backward's matrix-core rate against the bf16 peak: 20 d P counts each
        # product once; the kernels execute 28 d P (the dQ pass recomputes the scores
        # and dP), which is the rate the matrix cores actually sustain.
        "bwd_roofline": {"bound": "mfma", "achieved": bwd_tf, "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": bwd_tf / PEAK_BF16_TFLOPS,
                         "executed_tflops_28dP": bwd_tf * 28.0 / 20.0},
    }


def leg_proj(steps, warmup):
    import torch
    from differential_attention_causal_amd import diffattn as da
    from differential_attention_causal_amd import synth
    w = synth.WORKLOADS[3]
    B, N, H, d = w.batch, w.seqlen, w.heads, w.head_dim
    dm = 2 * H * d
    x = synth.make_proj_inputs(B, N, H, d, dm, "cuda:0", seed=5)
    lv = synth.make_inputs(w, "cuda:0")     # the forward workload's lambda vectors
    qkv = da.qkv_proj(x["x"], x["w_qkv"], H, d)
    y = torch.empty(B, N, H, 2 * d, dtype=torch.bfloat16, device="cuda:0")
    out = torch.empty(B, N, dm, dtype=torch.bfloat16, device="cuda:0")
    p = da.problem(B, H, N, d, da.BF16)
    ws = torch.empty(da.workspace_bytes(da.OP_FWD, p), dtype=torch.uint8, device="cuda:0")
    torch.cuda.synchronize()
    res = {}
    for name, fn, fl in (
            ("qkv_proj", lambda: da.qkv_proj(x["x"], x["w_qkv"], H, d, out=qkv),
             2.0 * B * N * dm * 6 * H * d),
            ("out_proj", lambda: da.out_proj(x["attn"], x["w_o"], out=out),
             2.0 * B * N * dm * 2 * H * d)):
        def step(ev, fn=fn):
            if ev:
                ev[0].record()
            fn()
            if ev:
                ev[1].record()
        ms, wall, inner = time_steps(step, steps, warmup, inner_events=True)
        k_ms = sum(inner) / len(inner)
        tf = fl / (k_ms * 1e-3) / 1e12
        res[name] = {"us": k_ms * 1e3, "tflops": tf, "frac_bf16_peak": tf / PEAK_BF16_TFLOPS}

    def module(ev):
        q1, q2, k1, k2, v = da.qkv_proj(x["x"], x["w_qkv"], H, d, out=qkv)
        st = da.lambda_(lv["lq1"], lv["lk1"], lv["lq2"], lv["lk2"], w.layer)
        da.forward(q1, q2, k1, k2, v, st, out=y, workspace=ws, layout="bnh")
        da.out_proj(y, x["w_o"], out=out)

    ms, wall, _ = time_steps(module, max(1, steps // 2), warmup)
    res["shape"] = f"B{B} N{N} H{H} d{d} d_model {dm}"
    res["module_ms"] = ms
    return res


def leg_ref_gemm(steps, warmup):
    """The best bf16 matrix-core rate this box shows through the vendor library
    (torch.matmul -> hipBLASLt, 8192^3): a measured reference beside the nominal peak."""
    import torch
    n = 8192
    g = torch.Generator(device="cuda:0").manual_seed(7)
    a = torch.randn(n, n, generator=g, device="cuda:0").to(torch.bfloat16)
    b = torch.randn(n, n, generator=g, device="cuda:0").to(torch.bfloat16)
    c = torch.empty(n, n, dtype=torch.bfloat16, device="cuda:0")
    torch.cuda.synchronize()

    def step(ev):
        if ev:
            ev[0].record()
        torch.matmul(a, b, out=c)
        if ev:
            ev[1].record()

    _, _, inner = time_steps(step, max(5, steps // 4), warmup, inner_events=True)
    k_ms = sorted(inner)[len(inner) // 2]
    return {"shape": f"{n}^3 bf16 (torch.matmul, hipBLASLt)", "ms": k_ms,
            "tflops": 2.0 * n ** 3 / (k_ms * 1e-3) / 1e12}


def leg_copy(steps, warmup):
    """A plain 2 GiB device-to-device copy: the measured HBM reference, and the kernel the
    FETCH_SIZE / WRITE_SIZE counters are calibrated on."""
    import torch
    n = 1 << 30
    a = torch.ones(n, dtype=torch.bfloat16, device="cuda:0")
    b = torch.empty_like(a)
    torch.cuda.synchronize()

    def step(ev):
        if ev:
            ev[0].record()
        b.copy_(a)
        if ev:
            ev[1].record()

    ms, wall, inner = time_steps(step, steps, warmup, inner_events=True)
    kern_ms = sum(inner) / len(inner)
    return {"bytes_read": 2 * n, "bytes_written": 2 * n,
            "GB_s": 4 * n / (kern_ms * 1e-3) / 1e9, "copy_ms": kern_ms}


def source_hash(source: str) -> str:
    """sha256 prefix over a kernel's source file and the two headers every kernel includes."""
    import hashlib
    h = hashlib.sha256()
    for f in (source, "common.h", "launch.h"):
        h.update(open(os.path.join(ROOT, "differential_attention_causal_amd", "csrc", f),
                      "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, source: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from profiles/hbm_traffic.md, if that
    row was measured on the current source of the kernel (see source_hash); else None."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.md")
    src = os.path.join(ROOT, "differential_attention_causal_amd", "csrc", source)
    if not (os.path.exists(path) and os.path.exists(src)):
        return None
    sha = source_hash(source)
    for line in open(path):
        cells = [c.strip().strip("`") for c in line.strip().strip("|").split("|")]
        if len(cells) >= 6 and cells[0] == kernel and cells[1] == sha and cells[2] == workload:
            try:
                return float(cells[5].replace(",", ""))
            except ValueError:
                return None
    return None


def cpu_baseline():
    """The float64 oracle timed on the host cores, per workload, on bounded samples of the
    same seeded inputs the GPU legs use (drawn on the GPU, copied to the host):
      1 tiny fp32 forward   - the whole workload (oracle.forward);
      2 prefill forward     - whole heads with the blocked oracle.head_forward;
      3 long-context fwd    - one whole head (N = 32768) with oracle.head_forward;
      4 decode step         - whole sequences (16 heads each) with oracle.decode;
      5 training fwd + bwd  - whole heads with oracle.head_forward and head_backward.
    BLAS threads are pinned to the cores this process may run on. Rates use the GPU legs'
    conventions: 12 d P FLOP per head forward, 20 d P backward, and the cache, query and
    output bytes of a decode step; full_s scales the sample's time to the whole workload."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits
    from differential_attention_causal_amd import synth
    from oracle import diffattn_oracle as orc
    cores = len(os.sched_getaffinity(0))
    entries = []

    def add(e):
        entries.append(e)
        print(f"[bench] cpu_baseline config {e['config']}: {e['wall_s']:.1f} s", file=sys.stderr,
              flush=True)

    def host(t):
        return t.float().cpu().double().numpy()

    def lam(x, w):
        lv = {k: host(x[k]) for k in ("lq1", "lk1", "lq2", "lk2")}
        return orc.lambda_scalar(lv["lq1"], lv["lk1"], lv["lq2"], lv["lk2"], w.layer)

    def heads_forward(number, n_heads, backward=False):
        w = synth.WORKLOADS[number]
        x = synth.make_inputs(w, "cuda:0")
        torch.cuda.synchronize()
        ls = lam(x, w)
        pairs = w.head_dim * w.seqlen * (w.seqlen + 1) // 2     # d P per head
        t0 = time.perf_counter()
        done = 0
        for i in range(n_heads):
            b, hh = divmod(i, w.heads)
            h = {k: host(x[k][b, hh]) for k in x if k not in ("lq1", "lk1", "lq2", "lk2")}
            orc.head_forward(h["q1"], h["q2"], h["k1"], h["k2"], h["v"], ls["lambda"],
                             ls["lambda_init"])
            if backward:
                orc.head_backward(h["q1"], h["q2"], h["k1"], h["k2"], h["v"], h["dout"],
                                  ls["lambda"], ls["lambda_init"])
            done += 1
        el = time.perf_counter() - t0
        del x
        flop = (32.0 if backward else 12.0) * pairs * done
        nh = w.batch * w.heads
        return {"config": number, "workload": w.name, "sample": f"{done} of {nh} heads",
                "wall_s": el, "gflops": flop / el / 1e9, "full_s": el * nh / done,
                "flop_convention": "12 d P + 20 d P per head" if backward else "12 d P per head"}

    with threadpool_limits(limits=cores):
        # 1: the whole tiny workload
        w = synth.WORKLOADS[1]
        x = synth.make_inputs(w, "cuda:0")
        h = {k: host(v) for k, v in x.items()}
        ls = lam(x, w)
        t0 = time.perf_counter()
        orc.forward(h["q1"], h["q2"], h["k1"], h["k2"], h["v"], ls["lambda"], ls["lambda_init"])
        el = time.perf_counter() - t0
        flop = 12.0 * w.head_dim * w.seqlen * (w.seqlen + 1) / 2 * w.batch * w.heads
        add({"config": 1, "workload": w.name, "sample": "whole workload",
                        "wall_s": el, "gflops": flop / el / 1e9, "full_s": el,
                        "flop_convention": "12 d P per head"})
        add(heads_forward(2, 4))
        add(heads_forward(3, 1))
        # 4: whole sequences of the decode step
        w = synth.WORKLOADS[4]
        x = synth.make_inputs(w, "cuda:0")
        torch.cuda.synchronize()
        ls = lam(x, w)
        n_seq = 4
        t0 = time.perf_counter()
        for b in range(n_seq):
            sl = {k: host(x[k][b:b + 1]) for k in ("q1", "q2", "k1", "k2", "v")}
            orc.decode(sl["q1"], sl["q2"], sl["k1"], sl["k2"], sl["v"], None, ls["lambda"],
                       ls["lambda_init"])
        el = time.perf_counter() - t0
        del x
        by = decode_bytes(w) * n_seq / w.batch
        add({"config": 4, "workload": w.name,
                        "sample": f"{n_seq} of {w.batch} sequences (16 heads each)",
                        "wall_s": el, "gb_s": by / el / 1e9, "full_s": el * w.batch / n_seq,
                        "bytes_convention": "cache + query + output bytes"})
        add(heads_forward(5, 2, backward=True))
    head = next(e for e in entries if e["config"] == 3)
    return {"value": head["gflops"] / 1e3, "unit": "TFLOP/s", "cores": cores,
            "blas_threads": cores, "kind": "oracle",
            "sample": "float64 oracle, blocked head_forward over one whole head (N = 32768) "
                      "of the long-context workload; per_config has every workload",
            "per_config": entries}


def _progress(msg: str, t0: float) -> None:
    """One line on stderr as each leg ends (the JSON record stays the only stdout line)."""
    print(f"[bench] {msg} ({time.perf_counter() - t0:.1f} s)", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--legs", default="fwd,prefill,peaked,decode,train,proj,refgemm,copy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the forward and decode shard over (batch, "
              "head) with no exchange, so there is no multi-GPU path to time; run with "
              "--gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    legs = set(args.legs.split(","))
    t0 = time.perf_counter()
    w, fwd = leg_forward(args.steps, args.warmup)
    _progress("forward", t0)
    rec = {
        "metric": METRIC, "value": fwd["tflops"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": fwd["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded normal inputs, generated on the GPU)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads,
                   "seq_len": w.seqlen, "head_dim": w.head_dim, "v_width": w.dv,
                   "layer": w.layer, "flop_convention": "12 d P per head"},
        "pct_bf16_mfma_peak": 100.0 * fwd["tflops"] / PEAK_BF16_TFLOPS,
        "roofline": fwd["roofline"],
        "fwd_kernel_ms": fwd["fwd_kernel_ms"],
        "fwd_kernel_ms_median": fwd["fwd_kernel_ms_median"],
        "fwd_kernel_ms_min": fwd["fwd_kernel_ms_min"],
        "formula_tflops_8dP": fwd["formula_tflops_8dP"],
    }
    if "prefill" in legs:
        wp, pf = leg_forward(args.steps, args.warmup, number=2)
        rec["prefill"] = {"workload": wp.name, "fwd_kernel_ms": pf["fwd_kernel_ms"],
                          "tflops": pf["roofline"]["achieved"], "frac": pf["roofline"]["frac"]}
        _progress("prefill", t0)
    if "peaked" in legs:
        rec["peaked"] = leg_peaked(args.steps, args.warmup)
        rec["peaked"]["time_vs_normal_inputs"] = rec["peaked"]["fwd_kernel_ms"] / fwd["fwd_kernel_ms"]
        _progress("peaked", t0)
    if "decode" in legs:
        rec["decode"] = leg_decode(args.steps, args.warmup)
        _progress("decode", t0)
    if "train" in legs:
        rec["train"] = leg_train(max(1, args.steps // 2), args.warmup)
        _progress("train", t0)
    if "proj" in legs:
        rec["proj"] = leg_proj(args.steps, args.warmup)
        _progress("proj", t0)
    if "refgemm" in legs:
        rec["ref_gemm"] = leg_ref_gemm(args.steps, args.warmup)
        rec["ref_gemm"]["fwd_frac_of_it"] = fwd["roofline"]["achieved"] / rec["ref_gemm"]["tflops"]
        _progress("refgemm", t0)
    if "copy" in legs:
        rec["copy"] = leg_copy(args.steps, args.warmup)
        _progress("copy", t0)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline()
        _progress("cpu_baseline", t0)
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
