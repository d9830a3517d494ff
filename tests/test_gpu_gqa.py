"""Grouped-query attention (K1, K2, V shared by groups of consecutive query heads) on the
GPU: forward, decode and the QKV projection.

Every GQA call is checked against the float64 oracle at the bars of the MHA tests (bf16
outputs 2e-2 max-abs, float32 1e-5 normwise relative per head), and against the same
library call with every K/V head repeated for the query heads of its group: bitwise for
the forward (the same kernel reads the same values); for decode, where one workgroup
serves several query heads with 32-key rounds instead of 64, within 2^-7 of each output
(the float32 accumulation order differs, which can move a bf16 rounding by one unit).
"""
import numpy as np
import pytest
import torch

from differential_attention_causal_amd import diffattn as da
from differential_attention_causal_amd import synth
from oracle import diffattn_oracle as orc
from tests.helpers import DEV, draw, np64, normwise_rel

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
FP32_TOL = 1e-5


def _group(x, hkv):
    """K/V with hkv heads (the first hkv of the drawn ones) and their per-group repeat."""
    g = x["q1"].shape[1] // hkv
    kv = {k: x[k][:, :hkv].contiguous() for k in ("k1", "k2", "v")}
    rep = {k: torch.repeat_interleave(t, g, dim=1).contiguous() for k, t in kv.items()}
    return kv, rep


@pytest.mark.parametrize("dtype,B,H,hkv,N", [("bf16", 2, 4, 2, 300), ("bf16", 1, 8, 1, 257),
                                             ("bf16", 1, 6, 3, 64), ("fp32", 2, 4, 1, 50)])
def test_forward_grouped(dtype, B, H, hkv, N):
    d = 64 if dtype == "bf16" else 32
    w = synth.custom("fwd", B, H, N, d, 7, dtype, number=1600 + N + H)
    x, _ = draw(w)
    kv, rep = _group(x, hkv)
    st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
    y = da.forward(x["q1"], x["q2"], kv["k1"], kv["k2"], kv["v"], st)
    ym = da.forward(x["q1"], x["q2"], rep["k1"], rep["k2"], rep["v"], st)
    torch.cuda.synchronize()
    assert torch.equal(y, ym)
    ls = orc.lambda_scalar(*(np64(x[k]) for k in ("lq1", "lk1", "lq2", "lk2")), w.layer)
    ref = orc.forward(np64(x["q1"]), np64(x["q2"]), np64(kv["k1"]), np64(kv["k2"]),
                      np64(kv["v"]), ls["lambda"], ls["lambda_init"])
    if dtype == "bf16":
        assert np.max(np.abs(np64(y) - ref)) <= BF16_TOL
    else:
        assert np.all(normwise_rel(np64(y), ref, axes=(2, 3)) <= FP32_TOL)


# Groups of 2, 3, 4, 6, 8, 16 and 32 query heads (the matrix-core kernel's column counts,
# 32 being the most it takes), cache lengths that end inside a round, a length of 1,
# caches longer than one split, and a length just past a split boundary.
@pytest.mark.parametrize("B,H,hkv,L,lens", [(3, 4, 2, 700, [700, 1, 333]),
                                            (2, 8, 1, 1500, [1500, 1024]),
                                            (1, 16, 4, 4100, None),
                                            (1, 6, 2, 333, None),
                                            (2, 6, 1, 20000, [20000, 8193]),
                                            (2, 16, 1, 9000, [9000, 4500]),
                                            (1, 32, 1, 2000, None)])
def test_decode_grouped(B, H, hkv, L, lens):
    _decode_grouped_case(B, H, hkv, L, lens)


def _decode_grouped_case(B, H, hkv, L, lens):
    w = synth.custom("decode", B, H, L, 64, 8, "bf16", number=1700 + L + H)
    x, _ = draw(w)
    kv, rep = _group(x, hkv)
    st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
    cl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    y = da.decode(x["q1"], x["q2"], kv["k1"], kv["k2"], kv["v"], st, cache_len=cl)
    ym = da.decode(x["q1"], x["q2"], rep["k1"], rep["k2"], rep["v"], st, cache_len=cl)
    torch.cuda.synchronize()
    assert np.all(np.abs(np64(y) - np64(ym)) <= 2.0 ** -7 * np.maximum(np.abs(np64(ym)), 1.0))
    ls = orc.lambda_scalar(*(np64(x[k]) for k in ("lq1", "lk1", "lq2", "lk2")), w.layer)
    ref = orc.decode(np64(x["q1"]), np64(x["q2"]), np64(kv["k1"]), np64(kv["k2"]),
                     np64(kv["v"]), lens, ls["lambda"], ls["lambda_init"])
    assert np.max(np.abs(np64(y) - ref)) <= BF16_TOL


def test_decode_grouped_long_splits():
    """Enough groups for the longest splits (8192 keys) with caches of three splits, and
    cache lengths at and around the split and round boundaries."""
    B, H, hkv, L = 32, 16, 4, 16385
    lens = np.random.default_rng(1717).integers(1, L + 1, B)
    lens[:8] = [L, 8192, 8193, 1, 16384, 31, 32, 8191]
    _decode_grouped_case(B, H, hkv, L, [int(v) for v in lens])


def test_decode_grouped_serving_workload():
    """64 sequences x 16 query heads sharing 4 cache heads, cache length 8192: every
    output against the oracle, one sequence at a time."""
    w = synth.WORKLOADS[4]
    x = synth.make_inputs(w, DEV)
    kv, _ = _group(x, 4)
    st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
    y = da.decode(x["q1"], x["q2"], kv["k1"], kv["k2"], kv["v"], st)
    torch.cuda.synchronize()
    y = np64(y)
    ls = orc.lambda_scalar(*(np64(x[k]) for k in ("lq1", "lk1", "lq2", "lk2")), w.layer)
    for b in range(w.batch):
        s = slice(b, b + 1)
        ref = orc.decode(np64(x["q1"][s]), np64(x["q2"][s]), np64(kv["k1"][s]),
                         np64(kv["k2"][s]), np64(kv["v"][s]), None, ls["lambda"],
                         ls["lambda_init"])
        assert np.max(np.abs(y[s] - ref)) <= BF16_TOL, b


@pytest.mark.parametrize("B,N,H,hkv,dm", [(1, 300, 4, 2, 128), (2, 77, 8, 1, 256)])
def test_qkv_proj_grouped(B, N, H, hkv, dm):
    d = 64
    x = synth.make_proj_inputs(B, N, H, d, dm, DEV, seed=1800 + N)
    # the fused weight of a grouped layer: H 2d query rows, then Hkv 2d key and value rows
    wq = x["w_qkv"][:2 * d * H]
    wk = x["w_qkv"][2 * d * H:2 * d * (H + hkv)]
    wv = x["w_qkv"][4 * d * H:2 * d * (2 * H + hkv)]
    w = torch.cat([wq, wk, wv]).contiguous()
    out = da.qkv_proj(x["x"], w, H, d, kv_heads=hkv)
    torch.cuda.synchronize()
    xs, wn = np64(x["x"]), np64(w)
    ref = orc.qkv_proj(xs, wn, H, d, kv_heads=hkv)
    absd = orc.qkv_proj(np.abs(xs), np.abs(wn), H, d, kv_heads=hkv)
    for name, g, r, a in zip(("q1", "q2", "k1", "k2", "v"), out, ref, absd):
        assert tuple(g.shape) == r.shape, name
        bound = 2.0 * (np.abs(r) * 2.0 ** -9 + dm * 2.0 ** -24 * a) + 1e-30
        assert np.all(np.abs(np64(g) - r) <= bound), name


@pytest.mark.parametrize("B,H,hkv,N", [(1, 4, 2, 200), (2, 4, 1, 129), (1, 6, 3, 64),
                                      (1, 4, 2, 600)])
def test_backward_grouped(B, H, hkv, N):
    """dK and dV of a shared head collect the contributions of its query heads: against
    the oracle (normwise relative 5e-2 per tensor, as for MHA), and against the sum over
    each group of the MHA backward on repeated K/V."""
    from tests.test_gpu_backward import TOL, rel
    w = synth.custom("train", B, H, N, 64, 5, "bf16", number=1900 + N + H)
    x, _ = draw(w)
    kv, rep = _group(x, hkv)
    st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
    lv = (x["lq1"], x["lk1"], x["lq2"], x["lk2"])
    sv = da.alloc_saved(B, H, N, 64, DEV)
    da.forward(x["q1"], x["q2"], kv["k1"], kv["k2"], kv["v"], st, saved=sv)
    g = da.backward(x["q1"], x["q2"], kv["k1"], kv["k2"], kv["v"], *lv, st, sv, x["dout"])
    svm = da.alloc_saved(B, H, N, 64, DEV)
    da.forward(x["q1"], x["q2"], rep["k1"], rep["k2"], rep["v"], st, saved=svm)
    gm = da.backward(x["q1"], x["q2"], rep["k1"], rep["k2"], rep["v"], *lv, st, svm, x["dout"])
    torch.cuda.synchronize()
    ref = orc.backward(np64(x["q1"]), np64(x["q2"]), np64(kv["k1"]), np64(kv["k2"]),
                       np64(kv["v"]), np64(x["dout"]), *(np64(t) for t in lv), w.layer)
    scale = max(float(np.max(np.abs(ref["dv"]))), 1e-30)
    for k in ("dq1", "dq2", "dk1", "dk2", "dv", "d_attn"):
        assert tuple(g[k].shape) == ref[k].shape, k
        assert rel(np64(g[k]), ref[k], scale) <= TOL, k
    gsz = H // hkv
    for k in ("dk1", "dk2", "dv"):
        summed = np64(gm[k]).reshape(B, hkv, gsz, N, -1).sum(axis=2)
        assert rel(np64(g[k]), summed, scale) <= TOL, k
    for k in ("dq1", "dq2", "d_attn", "dlq1", "d_rms_weight"):
        assert rel(np64(g[k]), np64(gm[k]), 1.0) <= 1e-6, k   # same kernels, same inputs
