"""GPU parity of the projection GEMMs (fused W_Q/W_K/W_V input projection with its
per-head scatter, and the W_O output projection) against the float64 oracle.

Both sides take the same bf16 inputs; the GEMMs accumulate in float32 and round each
output once to bf16. Bound per element: half a bf16 unit of the result (2^-9 |ref|)
plus float32 accumulation error (K 2^-24 times the sum of |x w|), doubled for margin.
"""
import numpy as np
import pytest
import torch

from differential_attention_causal_amd import diffattn as da
from differential_attention_causal_amd import synth
from oracle import diffattn_oracle as orc
from tests.helpers import DEV, np64

pytestmark = pytest.mark.gpu


def _bound(ref, absdot, k):
    return 2.0 * (np.abs(ref) * 2.0 ** -9 + k * 2.0 ** -24 * absdot) + 1e-30


def _check_qkv(x, w, H, d, got, rows=None):
    xs = np64(x) if rows is None else np64(x)[:, rows]
    wn = np64(w)
    ref = orc.qkv_proj(xs, wn, H, d)
    absd = orc.qkv_proj(np.abs(xs), np.abs(wn), H, d)
    for name, g, r, a in zip(("q1", "q2", "k1", "k2", "v"), got, ref, absd):
        gg = np64(g) if rows is None else np64(g[:, :, rows])
        err = np.abs(gg - r)
        assert np.all(err <= _bound(r, a, xs.shape[-1])), (name, float(err.max()))


@pytest.mark.parametrize("B,N,H,d,dm", [(1, 300, 2, 64, 128), (2, 77, 3, 64, 192),
                                       (1, 1, 1, 32, 64), (3, 257, 1, 64, 256),
                                       (1, 512, 4, 64, 512)])
def test_qkv_proj(B, N, H, d, dm):
    x = synth.make_proj_inputs(B, N, H, d, dm, DEV, seed=1000 + N + dm)
    out = da.qkv_proj(x["x"], x["w_qkv"], H, d)
    torch.cuda.synchronize()
    _check_qkv(x["x"], x["w_qkv"], H, d, out)


@pytest.mark.parametrize("B,N,H,d,dm", [(1, 300, 2, 64, 128), (2, 77, 3, 64, 320),
                                       (1, 1, 1, 32, 64), (1, 512, 4, 64, 512)])
def test_out_proj(B, N, H, d, dm):
    x = synth.make_proj_inputs(B, N, H, d, dm, DEV, seed=1100 + N + dm)
    y = da.out_proj(x["attn"], x["w_o"])
    torch.cuda.synchronize()
    a, w = np64(x["attn"]), np64(x["w_o"])
    ref = orc.out_proj(a, w)
    absd = orc.out_proj(np.abs(a), np.abs(w))
    err = np.abs(np64(y) - ref)
    assert np.all(err <= _bound(ref, absd, H * 2 * d)), float(err.max())


def test_qkv_proj_long_context_workload_sampled():
    """B1 N32768, H16 d64, d_model 2048: sampled tokens against the oracle."""
    B, N, H, d, dm = 1, 32768, 16, 64, 2048
    x = synth.make_proj_inputs(B, N, H, d, dm, DEV, seed=1200)
    out = da.qkv_proj(x["x"], x["w_qkv"], H, d)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 4097, 20000, N - 257, N - 1])
    _check_qkv(x["x"], x["w_qkv"], H, d, out, rows)


def test_out_proj_long_context_workload_sampled():
    B, N, H, d, dm = 1, 32768, 16, 64, 2048
    x = synth.make_proj_inputs(B, N, H, d, dm, DEV, seed=1201)
    y = da.out_proj(x["attn"], x["w_o"])
    torch.cuda.synchronize()
    rows = np.array([0, 255, 256, 9999, N - 1])
    a, w = np64(x["attn"])[:, rows], np64(x["w_o"])
    ref = orc.out_proj(a, w)
    absd = orc.out_proj(np.abs(a), np.abs(w))
    err = np.abs(np64(y)[:, rows] - ref)
    assert np.all(err <= _bound(ref, absd, H * 2 * d)), float(err.max())


def test_proj_empty_and_deterministic():
    x = synth.make_proj_inputs(0, 16, 2, 64, 128, DEV, seed=1300)
    q = da.qkv_proj(x["x"], x["w_qkv"], 2, 64)
    assert q[0].numel() == 0
    x = synth.make_proj_inputs(2, 100, 2, 64, 128, DEV, seed=1301)
    a = da.qkv_proj(x["x"], x["w_qkv"], 2, 64)
    b = da.qkv_proj(x["x"], x["w_qkv"], 2, 64)
    for s, t in zip(a, b):
        assert torch.equal(s, t)


def test_projection_attention_projection_chain():
    """X -> fused QKV projection -> DiffAttn (token-major output) -> W_O, all on the
    device, against the oracle's float64 chain on the same bf16 weights and X. Each stage
    rounds its output to bf16 on the device; the float64 chain does not, so the bound is
    the composition of the stage bars: 5e-2 max-abs on outputs of order one."""
    B, N, H, d, dm = 1, 200, 2, 64, 256
    x = synth.make_proj_inputs(B, N, H, d, dm, DEV, seed=1500)
    lv = synth.make_lambda_layers(1, d, DEV, seed=1501)
    lam = [lv[k][0].contiguous() for k in ("lq1", "lk1", "lq2", "lk2")]
    st = da.lambda_(*lam, 4)
    q1, q2, k1, k2, v = da.qkv_proj(x["x"], x["w_qkv"], H, d)
    y = da.forward(q1, q2, k1, k2, v, st, layout="bnh")
    out = da.out_proj(y, x["w_o"])
    torch.cuda.synchronize()
    ls = orc.lambda_scalar(*(np64(t) for t in lam), 4)
    rq = orc.qkv_proj(np64(x["x"]), np64(x["w_qkv"]), H, d)
    ry = orc.forward(*rq, ls["lambda"], ls["lambda_init"])
    ref = orc.out_proj(ry.transpose(0, 2, 1, 3), np64(x["w_o"]))
    err = np.abs(np64(out) - ref)
    assert float(err.max()) <= 5e-2, float(err.max())
