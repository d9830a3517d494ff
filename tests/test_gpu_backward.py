"""GPU parity of the backward pass against the float64 oracle's analytic gradients.

The oracle's gradients are themselves checked against central finite differences of its
forward (tests/test_oracle.py). Tolerance for bf16 gradients: 5e-2 relative, normwise per
tensor (max |x - ref| / max |ref|) over the compared (b, h) slices. dlambda and the four
lambda-vector gradients (scalar sums over every row of every head) are compared with the
oracle's within 5e-2 relative plus a rounding allowance derived in dlam_noise.
"""
import os

import numpy as np
import pytest
import torch

from differential_attention_causal_amd import diffattn as da
from differential_attention_causal_amd import synth
from oracle import diffattn_oracle as orc
from tests.helpers import DEV, draw, lambda_state_tensor, np64

pytestmark = pytest.mark.gpu

TOL = 5e-2


def rel(a, ref, scale):
    """Normwise relative error; a reference that is identically zero (dQ and dK when the
    only visible key is the row's own) must come out zero up to rounding, 1e-4 of the
    gradient scale, which maps to an error of 0 here and to inf otherwise."""
    if np.max(np.abs(ref)) == 0.0:
        return 0.0 if np.max(np.abs(a)) <= 1e-4 * scale else float("inf")
    return float(np.max(np.abs(a - ref)) / np.max(np.abs(ref)))


def run_train(x, w, weight=None):
    st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
    sv = da.alloc_saved(w.batch, w.heads, w.seqlen, w.head_dim, DEV)
    da.forward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st, rms_weight=weight, saved=sv)
    g = da.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lq1"], x["lk1"], x["lq2"],
                    x["lk2"], st, sv, x["dout"], rms_weight=weight)
    torch.cuda.synchronize()
    return g


def dlam_noise(h, layer, heads, weight=None):
    """Rounding allowance for dlambda: 2^-7 sqrt(sum (G O2)^2) over rows i >= 1 and
    channels, with G and O2 from the oracle.

    dlambda = -sum_i sum_c G_ic O2_ic sums terms of both signs that cancel, so a
    relative bound alone fails where the true sum happens to be small. The bf16
    forward rounds each attention weight to 8 bits before the products with V, an
    unbiased error of up to 2^-9 of the weight; O1 and O2 (hence G) then carry errors of
    that relative size with random signs, and each row's term G_i . O2_i errs by about
    2^-9 |G_i * O2_i|, independently across rows. Summed, the error of dlambda is about
    2^-9 sqrt(sum (G O2)^2); the allowance is four times that. Row 0 sees one key, its
    weight is exactly 1 and its O1 = O2 = V0 carry no such error, so it is left out."""
    st = orc.lambda_scalar(h["lq1"], h["lk1"], h["lq2"], h["lk2"], layer)
    ss = 0.0
    for b, hh in heads:
        w = None if weight is None else weight[hh]
        _, sv = orc.head_forward(h["q1"][b, hh], h["q2"][b, hh], h["k1"][b, hh],
                                 h["k2"][b, hh], h["v"][b, hh], st["lambda"],
                                 st["lambda_init"], weight=w, want_saved=True)
        e = orc.epilogue_backward(sv["o1"], sv["o2"], h["dout"][b, hh], st["lambda"],
                                  st["lambda_init"], weight=w)
        ss += float(np.sum((e["G"][1:] * sv["o2"][1:]) ** 2))
    return 2.0 ** -7 * ss ** 0.5


def gpu_dlam(g, lq1, lk1, layer_state):
    """dlambda as the library computed it, recovered from dlq1 = dlambda e^a lk1 at the
    largest |lk1| entry (float64 division of the float32 output)."""
    i = int(np.argmax(np.abs(lk1)))
    return float(np64(g["dlq1"])[i]) / (layer_state["exp_a"] * lk1[i])


def check_lambda_grads(g, dlam_ref, noise, h, layer):
    """dlambda and the four lambda-vector gradients against the oracle: |error| within
    5e-2 |dlambda| plus the rounding allowance of dlam_noise; each vector gradient
    dl = dlambda x (a fixed factor) within that bound times the factor, plus its float32
    rounding. Returns the relative error of dlambda."""
    st = orc.lambda_scalar(h["lq1"], h["lk1"], h["lq2"], h["lk2"], layer)
    tol = TOL * abs(dlam_ref) + noise
    dl = gpu_dlam(g, h["lq1"], h["lk1"], st)
    assert abs(dl - dlam_ref) <= tol, (dl, dlam_ref, tol)
    fac = {"dlq1": st["exp_a"] * h["lk1"], "dlk1": st["exp_a"] * h["lq1"],
           "dlq2": -st["exp_b"] * h["lk2"], "dlk2": -st["exp_b"] * h["lq2"]}
    for k, f in fac.items():
        ref = dlam_ref * f
        err = np.abs(np64(g[k]) - ref)
        assert np.all(err <= tol * np.abs(f) + 2.0 ** -23 * np.abs(ref) + 1e-30), k
    return abs(dl - dlam_ref) / max(abs(dlam_ref), 1e-300)


def compare(g, ref, heads, h=None, layer=None, weight=None):
    """Per-tensor normwise relative error <= TOL (see rel); with h, also dlambda and the
    lambda-vector gradients against the oracle's (check_lambda_grads)."""
    scale = max(np.max(np.abs(np.stack([ref["dv"][b, hh] for b, hh in heads]))), 1e-30)
    for k in ("dq1", "dq2", "dk1", "dk2", "dv", "d_attn"):
        a = np.stack([np64(g[k][b, hh]) for b, hh in heads])
        r = np.stack([ref[k][b, hh] for b, hh in heads])
        e = rel(a, r, scale)
        assert e <= TOL, (k, e)
    if h is None:
        return
    check_lambda_grads(g, ref["dlam"], dlam_noise(h, layer, heads, weight), h, layer)


def check_weight_grad(g, ref):
    """d_rms_weight [H, 2d] against the oracle's (summed over the whole batch): normwise
    relative error within the gradient tolerance."""
    e = rel(np64(g["d_rms_weight"]), ref["d_rms_weight"], 1.0)
    assert e <= TOL, ("d_rms_weight", e)


@pytest.mark.parametrize("b,hh,n", [(1, 1, 1), (1, 1, 32), (1, 2, 33), (2, 1, 64), (1, 2, 129),
                                    (1, 2, 200), (1, 1, 256), (1, 1, 257), (1, 1, 300),
                                    (1, 1, 513), (1, 2, 1000)])
def test_backward_small(b, hh, n):
    w = synth.custom("train", b, hh, n, 64, 6, "bf16", number=700 + n)
    x, h = draw(w)
    g = run_train(x, w)
    ref = orc.backward(h["q1"], h["q2"], h["k1"], h["k2"], h["v"], h["dout"], h["lq1"],
                       h["lk1"], h["lq2"], h["lk2"], w.layer)
    compare(g, ref, [(i, j) for i in range(b) for j in range(hh)], h, w.layer)
    check_weight_grad(g, ref)


def test_backward_rms_weight():
    w = synth.custom("train", 1, 2, 150, 64, 3, "bf16", number=720)
    x, h = draw(w)
    gen = torch.Generator(device=DEV).manual_seed(3)
    weight = 1.0 + 0.25 * torch.randn(2, 128, generator=gen, device=DEV)
    g = run_train(x, w, weight)
    ref = orc.backward(h["q1"], h["q2"], h["k1"], h["k2"], h["v"], h["dout"], h["lq1"],
                       h["lk1"], h["lq2"], h["lk2"], w.layer, weight=np64(weight))
    compare(g, ref, [(0, 0), (0, 1)], h, w.layer, np64(weight))
    check_weight_grad(g, ref)


@pytest.mark.parametrize("b,hh,n", [(2, 3, 100), (1, 2, 64)])
def test_backward_token_major_dout(b, hh, n):
    """dout given as [B, N, H, 2d] (layout "bnh") yields bitwise the gradients of the same
    dout given as [B, H, N, 2d]."""
    w = synth.custom("train", b, hh, n, 64, 4, "bf16", number=760 + n)
    x, h = draw(w)
    st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
    sv = da.alloc_saved(b, hh, n, 64, DEV)
    da.forward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st, saved=sv)
    args = (x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lq1"], x["lk1"], x["lq2"], x["lk2"],
            st, sv)
    ga = da.backward(*args, x["dout"])
    gb = da.backward(*args, x["dout"].transpose(1, 2).contiguous(), layout="bnh")
    torch.cuda.synchronize()
    for k in ga:
        assert torch.equal(ga[k], gb[k]), k


def test_backward_weight_grad_empty_is_zero():
    d = 64
    st = lambda_state_tensor(0.5, 0.2, DEV)
    z = torch.empty(2, 3, 0, d, dtype=torch.bfloat16, device=DEV)
    zv = torch.empty(2, 3, 0, 2 * d, dtype=torch.bfloat16, device=DEV)
    lv = [torch.randn(d, device=DEV) for _ in range(4)]
    sv = da.alloc_saved(2, 3, 0, d, DEV)
    g = da.backward(z, z, z, z, zv, *lv, st, sv, zv)
    torch.cuda.synchronize()
    assert g["d_rms_weight"].shape == (3, 2 * d)
    assert torch.count_nonzero(g["d_rms_weight"]).item() == 0


def test_backward_one_head_n32_slice():
    """One head, N = 32, d = 64: the slice on which the oracle's gradients are
    finite-difference checked."""
    w = synth.custom("train", 1, 1, 32, 64, 6, "bf16", number=730)
    x, h = draw(w)
    g = run_train(x, w)
    ref = orc.backward(h["q1"], h["q2"], h["k1"], h["k2"], h["v"], h["dout"], h["lq1"],
                       h["lk1"], h["lq2"], h["lk2"], w.layer)
    compare(g, ref, [(0, 0)], h, w.layer)


def _per_head_parallel(fn, items):
    """fn over items on a thread pool, one BLAS thread each (numpy releases the GIL in
    its products and exponentials), as many workers as this process may use cores."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with threadpool_limits(1):
        with ThreadPoolExecutor(workers) as ex:
            return list(ex.map(fn, items))


def test_backward_training_workload():
    """B8 H12 N4096 d64, layer 6.
    - every gradient tensor of every head against the oracle's full backward;
    - dlambda, the four lambda-vector gradients and the RMSNorm weight gradient, which
      sum over all 96 heads, against the oracle's forward and epilogue backward on every
      head;
    - the training saves (lse, O1, O2, rstd) of every head;
    - the library's cross-head reduction of dlambda against a float64 host sum of its
      own G (d_attn) times its own saved O2, over every row of every head."""
    w = synth.WORKLOADS[5]
    x = synth.make_inputs(w, DEV)
    st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
    sv = da.alloc_saved(w.batch, w.heads, w.seqlen, w.head_dim, DEV)
    da.forward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st, saved=sv)
    g = da.backward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], x["lq1"], x["lk1"], x["lq2"],
                    x["lk2"], st, sv, x["dout"])
    torch.cuda.synchronize()
    for k in ("dq1", "dq2", "dk1", "dk2", "dv", "d_attn"):
        assert torch.isfinite(g[k].float()).all().item(), k
    h = {k: np64(x[k]) for k in ("q1", "q2", "k1", "k2", "v", "dout", "lq1", "lk1", "lq2", "lk2")}
    ls = orc.lambda_scalar(h["lq1"], h["lk1"], h["lq2"], h["lk2"], w.layer)
    lam, li = ls["lambda"], ls["lambda_init"]

    # the library's own reduction: dlambda = -sum G O2 over its float32 G and saved O2
    da_h, o2_h = np64(g["d_attn"]), np64(sv["o2"])
    terms = da_h * o2_h
    own = -float(np.sum(terms))
    l1 = float(np.sum(np.abs(terms)))
    del terms
    dl = gpu_dlam(g, h["lq1"], h["lk1"], ls)
    assert abs(dl - own) <= 2e-6 * l1, (dl, own, l1)

    # the oracle on every head: forward with saves, then the epilogue backward; the
    # library's saves of each head are compared on the way
    heads = [(b, hh) for b in range(w.batch) for hh in range(w.heads)]
    svh = {k: np64(sv[k]) for k in ("lse1", "lse2", "o1", "rstd")}
    svh["o2"] = o2_h

    def head(bh):
        b, hh = bh
        _, s = orc.head_forward(h["q1"][b, hh], h["q2"][b, hh], h["k1"][b, hh], h["k2"][b, hh],
                                h["v"][b, hh], lam, li, want_saved=True)
        e = orc.epilogue_backward(s["o1"], s["o2"], h["dout"][b, hh], lam, li)
        save_err = {k: float(np.max(np.abs(svh[k][b, hh] - s[k])))
                    for k in ("lse1", "lse2", "o1", "o2")}
        save_err["rstd"] = float(np.max(np.abs(svh["rstd"][b, hh] / s["rstd"] - 1.0)))
        return e["dlam"], e["dw"], float(np.sum((e["G"][1:] * s["o2"][1:]) ** 2)), save_err
    res = _per_head_parallel(head, heads)
    for k, tol in (("lse1", 2e-3), ("lse2", 2e-3), ("o1", 2e-2), ("o2", 2e-2), ("rstd", 2e-2)):
        worst = max(r[3][k] for r in res)
        assert worst <= tol, (k, worst)
    dlam_ref = sum(r[0] for r in res)
    noise = 2.0 ** -7 * sum(r[2] for r in res) ** 0.5
    e = check_lambda_grads(g, dlam_ref, noise, h, w.layer)
    print(f"training workload: dlambda {dl:.6e}, oracle {dlam_ref:.6e}, relative error "
          f"{e:.2e}, allowance {noise:.3e}")
    dw_ref = np.zeros((w.heads, w.dv))
    for (b, hh), r in zip(heads, res):
        dw_ref[hh] += r[1]
    assert rel(np64(g["d_rms_weight"]), dw_ref, 1.0) <= TOL

    # every head: each gradient tensor against the oracle's full backward, normwise per
    # head (a zero reference, impossible here, would be measured against max |dV|)
    gh = {k: np64(g[k]) for k in ("dq1", "dq2", "dk1", "dk2", "dv")}
    gh["d_attn"] = da_h

    def grads(bh):
        b, hh = bh
        sl = {k: h[k][b, hh] for k in ("q1", "q2", "k1", "k2", "v", "dout")}
        ref = orc.head_backward(sl["q1"], sl["q2"], sl["k1"], sl["k2"], sl["v"], sl["dout"],
                                lam, li)
        scale = np.max(np.abs(ref["dv"]))
        return {k: rel(gh[k][b, hh], ref[k], scale)
                for k in ("dq1", "dq2", "dk1", "dk2", "dv", "d_attn")}
    per = _per_head_parallel(grads, heads)
    for k in ("dq1", "dq2", "dk1", "dk2", "dv", "d_attn"):
        worst = max(p[k] for p in per)
        assert worst <= TOL, (k, worst)


def test_backward_lambda_vectors_full_length():
    """Two heads at the full sequence length of the training workload: the lambda-vector
    gradients and the RMSNorm weight gradient sum over every row."""
    w = synth.custom("train", 1, 2, 4096, 64, 6, "bf16", number=740)
    x, h = draw(w)
    g = run_train(x, w)
    ref = orc.backward(h["q1"], h["q2"], h["k1"], h["k2"], h["v"], h["dout"], h["lq1"],
                       h["lk1"], h["lq2"], h["lk2"], w.layer)
    compare(g, ref, [(0, 0), (0, 1)], h, w.layer)
    check_weight_grad(g, ref)


def test_backward_deterministic():
    w = synth.custom("train", 2, 2, 333, 64, 4, "bf16", number=750)
    x, h = draw(w)
    g1 = run_train(x, w)
    g2 = run_train(x, w)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k


def test_backward_empty_batch_gives_zero_lambda_grads():
    d = 64
    st = lambda_state_tensor(0.5, 0.2, DEV)
    z = torch.empty(0, 2, 16, d, dtype=torch.bfloat16, device=DEV)
    zv = torch.empty(0, 2, 16, 2 * d, dtype=torch.bfloat16, device=DEV)
    lv = [torch.randn(d, device=DEV) for _ in range(4)]
    sv = da.alloc_saved(0, 2, 16, d, DEV)
    g = da.backward(z, z, z, z, zv, *lv, st, sv, zv)
    torch.cuda.synchronize()
    for k in ("dlq1", "dlk1", "dlq2", "dlk2"):
        assert torch.count_nonzero(g[k]).item() == 0
