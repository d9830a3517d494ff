"""GPU parity of the split-KV decode step against the float64 oracle."""
import numpy as np
import pytest
import torch

from differential_attention_causal_amd import diffattn as da
from differential_attention_causal_amd import synth
from oracle import diffattn_oracle as orc
from tests.helpers import DEV, draw, lam_pair, np64

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


@pytest.mark.parametrize("b,hh,L,lens", [(1, 1, 1, None), (2, 2, 64, None), (3, 2, 300, [300, 1, 129]),
                                       (2, 3, 1000, [513, 999]), (4, 1, 4100, [4100, 4096, 257, 2])])
def test_decode_small(b, hh, L, lens):
    w = synth.custom("decode", b, hh, L, 64, 8, "bf16", number=600 + L)
    x, h = draw(w)
    st, ls = lam_pair(x, h, w.layer)
    cl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    y = da.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st, cache_len=cl)
    torch.cuda.synchronize()
    ref = orc.decode(h["q1"], h["q2"], h["k1"], h["k2"], h["v"], lens, ls["lambda"],
                     ls["lambda_init"])
    assert np.max(np.abs(np64(y) - ref)) <= BF16_TOL


def test_decode_matches_last_prefill_row():
    """Decode against a cache equals the last row of the forward over the same tokens."""
    w = synth.custom("fwd", 2, 2, 700, 64, 8, "bf16", number=620)
    x, h = draw(w)
    st, ls = lam_pair(x, h, w.layer)
    y = da.forward(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st)
    yd = da.decode(x["q1"][:, :, -1].contiguous(), x["q2"][:, :, -1].contiguous(), x["k1"],
                   x["k2"], x["v"], st)
    torch.cuda.synchronize()
    assert np.max(np.abs(np64(yd) - np64(y[:, :, -1]))) <= BF16_TOL
    ref = orc.forward_rows(h["q1"][1, 1], h["q2"][1, 1], h["k1"][1, 1], h["k2"][1, 1],
                           h["v"][1, 1], [699], ls["lambda"], ls["lambda_init"])
    assert np.max(np.abs(np64(yd[1, 1]) - ref[0])) <= BF16_TOL


def test_decode_workload_sampled():
    """64 sequences x 16 heads, cache length 8192, layer 8: 48 sampled (b, h) pairs."""
    w = synth.WORKLOADS[4]
    x = synth.make_inputs(w, DEV)
    st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
    y = da.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st)
    torch.cuda.synchronize()
    lv = {k: np64(x[k]) for k in ("lq1", "lk1", "lq2", "lk2")}
    ls = orc.lambda_scalar(lv["lq1"], lv["lk1"], lv["lq2"], lv["lk2"], w.layer)
    rng = np.random.default_rng(9)
    pairs = {(0, 0), (63, 15)} | {(int(b), int(hh)) for b, hh in
                                  zip(rng.integers(0, 64, 46), rng.integers(0, 16, 46))}
    for b, hh in sorted(pairs):
        sl = {k: np64(x[k][b:b + 1, hh:hh + 1]) for k in ("q1", "q2", "k1", "k2", "v")}
        ref = orc.decode(sl["q1"], sl["q2"], sl["k1"], sl["k2"], sl["v"], None, ls["lambda"],
                         ls["lambda_init"])
        assert np.max(np.abs(np64(y[b, hh]) - ref[0, 0])) <= BF16_TOL, (b, hh)
    assert torch.isfinite(y.float()).all().item()


def test_decode_cache_beyond_len_is_ignored_bitwise():
    w = synth.custom("decode", 2, 2, 900, 64, 3, "bf16", number=640)
    x, h = draw(w)
    st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
    cl = torch.tensor([611, 77], dtype=torch.int32, device=DEV)
    y0 = da.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st, cache_len=cl)
    k1 = x["k1"].clone(); v = x["v"].clone()
    k1[0, :, 611:] = 9.0
    v[1, :, 77:] = -4.0
    y1 = da.decode(x["q1"], x["q2"], k1, x["k2"], v, st, cache_len=cl)
    y2 = da.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st, cache_len=cl)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)
    assert torch.equal(y0, y2)  # deterministic


def test_decode_lengths_clamped():
    w = synth.custom("decode", 2, 1, 100, 64, 3, "bf16", number=650)
    x, h = draw(w)
    st, ls = lam_pair(x, h, w.layer)
    cl = torch.tensor([0, 5000], dtype=torch.int32, device=DEV)   # clamp to 1 and L
    y = da.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st, cache_len=cl)
    torch.cuda.synchronize()
    ref = orc.decode(h["q1"], h["q2"], h["k1"], h["k2"], h["v"], [1, 100], ls["lambda"],
                     ls["lambda_init"])
    assert np.max(np.abs(np64(y) - ref)) <= BF16_TOL
