"""GPU parity of the backward pass against the float64 oracle's analytic gradients.

The oracle's gradients are themselves checked against central finite differences of its
forward (tests/test_oracle.py). Tolerance for bf16 gradients: 5e-2 relative, normwise per
tensor (max |x - ref| / max |ref|) over the compared (b, h) slices.
"""
import numpy as np
import pytest
import torch

from differential_attention_causal_amd import diffattn as da
from differential_attention_causal_amd import synth
from oracle import diffattn_oracle as orc
from tests.helpers import DEV, draw, np64

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


def sum_abs_terms(h, layer, heads, weight=None):
    """sum over rows i and channels c of |G_ic O2_ic| from the oracle: the condition of the
    double sum dlambda = -sum_i sum_c G_ic O2_ic, against which its error is measured. The
    sum mixes signs and cancels heavily (|dlambda| is 1e-4 .. 1e-1 of it here), and for a
    row that sees one key D2 itself is the eps-sized remainder of two cancelling terms."""
    st = orc.lambda_scalar(h["lq1"], h["lk1"], h["lq2"], h["lk2"], layer)
    tot = 0.0
    for b, hh in heads:
        w = None if weight is None else weight[hh]
        _, sv = orc.head_forward(h["q1"][b, hh], h["q2"][b, hh], h["k1"][b, hh], h["k2"][b, hh],
                                 h["v"][b, hh], st["lambda"], st["lambda_init"], weight=w,
                                 want_saved=True)
        r = orc.head_backward(h["q1"][b, hh], h["q2"][b, hh], h["k1"][b, hh], h["k2"][b, hh],
                              h["v"][b, hh], h["dout"][b, hh], st["lambda"], st["lambda_init"],
                              weight=w)
        tot += float(np.sum(np.abs(r["d_attn"] * sv["o2"])))
    return tot


def compare(g, ref, heads, h=None, layer=None, weight=None):
    """Per-tensor normwise relative error <= TOL (see rel). dlambda is checked against the
    oracle within 1e-2 of sum |G O2| (see sum_abs_terms), and the four vector gradients
    against dlambda times their fixed factors."""
    scale = max(np.max(np.abs(np.stack([ref["dv"][b, hh] for b, hh in heads]))), 1e-30)
    for k in ("dq1", "dq2", "dk1", "dk2", "dv", "d_attn"):
        a = np.stack([np64(g[k][b, hh]) for b, hh in heads])
        r = np.stack([ref[k][b, hh] for b, hh in heads])
        e = rel(a, r, scale)
        assert e <= TOL, (k, e)
    if h is None:
        return
    st = orc.lambda_scalar(h["lq1"], h["lk1"], h["lq2"], h["lk2"], layer)
    # dlambda from the GPU's dlq1 (= dlambda e^a lk1) at its largest |lk1| component
    i = int(np.argmax(np.abs(h["lk1"])))
    dlam_gpu = float(np64(g["dlq1"])[i]) / (st["exp_a"] * h["lk1"][i])
    bound = 1e-2 * sum_abs_terms(h, layer, heads, weight)
    assert abs(dlam_gpu - ref["dlam"]) <= bound, (dlam_gpu, ref["dlam"], bound)
    fac = {"dlq1": st["exp_a"] * h["lk1"], "dlk1": st["exp_a"] * h["lq1"],
           "dlq2": -st["exp_b"] * h["lk2"], "dlk2": -st["exp_b"] * h["lq2"]}
    for k, f in fac.items():
        np.testing.assert_allclose(np64(g[k]), dlam_gpu * f, rtol=1e-5,
                                   atol=1e-6 * abs(dlam_gpu) * np.max(np.abs(f)))


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
    st = da.lambda_state_tensor(0.5, 0.2, DEV)
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


def test_backward_training_workload_sampled():
    """B8 H12 N4096 d64, layer 6: every gradient tensor on three sampled heads."""
    w = synth.WORKLOADS[5]
    x = synth.make_inputs(w, DEV)
    g = run_train(x, w)
    for k in ("dq1", "dq2", "dk1", "dk2", "dv", "d_attn"):
        assert torch.isfinite(g[k].float()).all().item(), k
    lv = {k: np64(x[k]) for k in ("lq1", "lk1", "lq2", "lk2")}
    st = orc.lambda_scalar(lv["lq1"], lv["lk1"], lv["lq2"], lv["lk2"], w.layer)
    for b, hh in [(0, 0), (3, 7), (7, 11)]:
        sl = {k: np64(x[k][b, hh]) for k in ("q1", "q2", "k1", "k2", "v", "dout")}
        ref = orc.head_backward(sl["q1"], sl["q2"], sl["k1"], sl["k2"], sl["v"], sl["dout"],
                                st["lambda"], st["lambda_init"])
        scale = np.max(np.abs(ref["dv"]))
        for k in ("dq1", "dq2", "dk1", "dk2", "dv", "d_attn"):
            assert rel(np64(g[k][b, hh]), ref[k], scale) <= TOL, (b, hh, k)


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
    st = da.lambda_state_tensor(0.5, 0.2, DEV)
    z = torch.empty(0, 2, 16, d, dtype=torch.bfloat16, device=DEV)
    zv = torch.empty(0, 2, 16, 2 * d, dtype=torch.bfloat16, device=DEV)
    lv = [torch.randn(d, device=DEV) for _ in range(4)]
    sv = da.alloc_saved(0, 2, 16, d, DEV)
    g = da.backward(z, z, z, z, zv, *lv, st, sv, zv)
    torch.cuda.synchronize()
    for k in ("dlq1", "dlk1", "dlq2", "dlk2"):
        assert torch.count_nonzero(g[k]).item() == 0
