"""The allocation-free decode entry point, diffattn_decode_noalloc, against
diffattn_decode (the same kernels with a caller workspace) and the float64 oracle.

Two calls in a row on the static scratch, the second on a smaller problem (fewer
sequences, heads and splits, grouped-query attention), so it runs on what the first
left in the scratch: each must equal the workspace entry point's output bitwise and be
within the bf16 bar (2e-2 max-abs) of the oracle.
"""
import numpy as np
import pytest
import torch

from differential_attention_causal_amd import diffattn as da
from differential_attention_causal_amd import synth
from oracle import diffattn_oracle as orc
from tests.helpers import DEV, draw, np64

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2


def _inputs(B, H, Hkv, L, lens, number):
    w = synth.custom("decode", B, H, L, 64, 8, "bf16", number=number)
    x, h = draw(w)
    if Hkv != H:           # the first Hkv heads of the drawn caches serve as shared heads
        for k in ("k1", "k2", "v"):
            x[k] = x[k][:, :Hkv].contiguous()
            h[k] = h[k][:, :Hkv]
    x["len"] = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return w, x, h


def test_noalloc_decode_two_calls_match_workspace_decode():
    cases = [(16, 16, 16, 8192, [8192, 1, 4097, 8191] * 4, 1700),
             (3, 4, 2, 700, [700, 1, 333], 1701)]
    data, ref_ws = [], []
    for B, H, Hkv, L, lens, num in cases:
        w, x, h = _inputs(B, H, Hkv, L, lens, num)
        st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
        ref_ws.append(da.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st,
                                cache_len=x["len"]))
        data.append((w, x, h, st, lens))
    torch.cuda.synchronize()
    outs = []
    for w, x, h, st, lens in data:            # back to back on the shared scratch
        outs.append(da.decode_noalloc(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st,
                                      cache_len=x["len"]))
    torch.cuda.synchronize()
    for (w, x, h, st, lens), y, yr in zip(data, outs, ref_ws):
        assert torch.equal(y, yr)
        ls = orc.lambda_scalar(h["lq1"], h["lk1"], h["lq2"], h["lk2"], w.layer)
        ref = orc.decode(h["q1"], h["q2"], h["k1"], h["k2"], h["v"], lens, ls["lambda"],
                         ls["lambda_init"])
        assert np.max(np.abs(np64(y) - ref)) <= BF16_TOL
