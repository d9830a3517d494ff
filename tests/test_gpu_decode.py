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
                                       (2, 3, 1000, [513, 999]), (4, 1, 4100, [4100, 4096, 257, 2]),
                                       (2, 1, 40000, [40000, 33001])])
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


def test_decode_workload():
    """64 sequences x 16 heads, cache length 8192, layer 8: every (b, h) output against
    the oracle (the cache reaches the host one sequence at a time)."""
    w = synth.WORKLOADS[4]
    x = synth.make_inputs(w, DEV)
    st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
    y = da.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st)
    torch.cuda.synchronize()
    assert torch.isfinite(y.float()).all().item()
    lv = {k: np64(x[k]) for k in ("lq1", "lk1", "lq2", "lk2")}
    ls = orc.lambda_scalar(lv["lq1"], lv["lk1"], lv["lq2"], lv["lk2"], w.layer)
    yh = np64(y)
    worst = 0.0
    for b in range(w.batch):
        sl = {k: np64(x[k][b:b + 1]) for k in ("q1", "q2", "k1", "k2", "v")}
        ref = orc.decode(sl["q1"], sl["q2"], sl["k1"], sl["k2"], sl["v"], None, ls["lambda"],
                         ls["lambda_init"])
        worst = max(worst, float(np.max(np.abs(yh[b] - ref[0]))))
    assert worst <= BF16_TOL, worst


def test_decode_maximum_cache_length():
    """Cache capacity 2^22 (the largest supported; 8192 splits of 512 keys for one sequence
    and head, so the merge reads its partials in many batches), full and ragged lengths."""
    n = 1 << 22
    w = synth.custom("decode", 2, 1, n, 64, 8, "bf16", number=660)
    x = synth.make_inputs(w, DEV)
    st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
    lens = [n, n - 1000]
    cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    y = da.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st, cache_len=cl)
    torch.cuda.synchronize()
    lv = {k: np64(x[k]) for k in ("lq1", "lk1", "lq2", "lk2")}
    ls = orc.lambda_scalar(lv["lq1"], lv["lk1"], lv["lq2"], lv["lk2"], w.layer)
    for b in range(2):
        sl = {k: np64(x[k][b:b + 1]) for k in ("q1", "q2", "k1", "k2", "v")}
        ref = orc.decode(sl["q1"], sl["q2"], sl["k1"], sl["k2"], sl["v"], [lens[b]],
                         ls["lambda"], ls["lambda_init"])
        assert np.max(np.abs(np64(y[b:b + 1]) - ref)) <= BF16_TOL, b


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


def _append_case(w, lens, seed):
    """Caches drawn for workload w, plus new rows from a second draw of the same shape."""
    x, h = draw(w)
    y, g = draw(w, seed=seed)
    new = {k: y[k][:, :, 0].contiguous() for k in ("k1", "k2", "v")}
    cl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return x, h, new, cl


def test_cache_append_bitwise():
    """Every byte of the caches and lengths after an append equals the oracle's copy:
    lengths 0, inside, last free row, full, negative."""
    w = synth.custom("decode", 5, 3, 40, 64, 3, "bf16", number=660)
    lens = [0, 7, 39, 40, -2]
    x, h, new, cl = _append_case(w, lens, seed=4660)
    k1, k2, v = x["k1"].clone(), x["k2"].clone(), x["v"].clone()
    da.cache_append(new["k1"], new["k2"], new["v"], k1, k2, v, cl)
    torch.cuda.synchronize()
    i16 = lambda t: t.cpu().view(torch.int16).numpy()      # the copy moves bit patterns
    r1, r2, rv, rl = orc.cache_append(i16(new["k1"]), i16(new["k2"]), i16(new["v"]),
                                      i16(x["k1"]), i16(x["k2"]), i16(x["v"]), lens)
    assert cl.cpu().tolist() == list(rl) == [1, 8, 40, 40, 1]
    for got, ref in ((k1, r1), (k2, r2), (v, rv)):
        assert np.array_equal(i16(got), ref)


def test_cache_append_then_decode():
    """Append then decode equals the oracle's decode over its own appended caches, and
    twice in a row keeps growing the sequences."""
    w = synth.custom("decode", 3, 2, 300, 64, 5, "bf16", number=670)
    lens = [120, 299, 1]
    x, h, new, cl = _append_case(w, lens, seed=4670)
    st, ls = lam_pair(x, h, w.layer)
    k1, k2, v = x["k1"].clone(), x["k2"].clone(), x["v"].clone()
    hk = [h["k1"], h["k2"], h["v"]]
    hl = lens
    for step in range(2):
        da.cache_append(new["k1"], new["k2"], new["v"], k1, k2, v, cl)
        y = da.decode(x["q1"], x["q2"], k1, k2, v, st, cache_len=cl)
        torch.cuda.synchronize()
        *hk, hl = orc.cache_append(np64(new["k1"]), np64(new["k2"]), np64(new["v"]), *hk, hl)
        assert cl.cpu().tolist() == list(hl)
        ref = orc.decode(h["q1"], h["q2"], *hk, hl, ls["lambda"], ls["lambda_init"])
        assert np.max(np.abs(np64(y) - ref)) <= BF16_TOL, step


def test_cache_append_decode_workload():
    """64 sequences x 16 heads, L = 8192, every cache one row from full: after the append
    every length is L and the new rows are in place (sampled), bitwise."""
    w = synth.WORKLOADS[4]
    x = synth.make_inputs(w, DEV)
    gen = torch.Generator(device=DEV).manual_seed(4680)
    new = {k: torch.randn(x[k][:, :, 0].shape, generator=gen, device=DEV).to(torch.bfloat16)
           for k in ("k1", "k2", "v")}
    cl = torch.full((w.batch,), w.seqlen - 1, dtype=torch.int32, device=DEV)
    before = x["k1"][5, 3, w.seqlen - 2].clone()
    da.cache_append(new["k1"], new["k2"], new["v"], x["k1"], x["k2"], x["v"], cl)
    torch.cuda.synchronize()
    assert (cl == w.seqlen).all().item()
    for b, hh in ((0, 0), (5, 3), (63, 15)):
        for k in ("k1", "k2", "v"):
            assert torch.equal(x[k][b, hh, w.seqlen - 1], new[k][b, hh]), (b, hh, k)
    assert torch.equal(x["k1"][5, 3, w.seqlen - 2], before)
