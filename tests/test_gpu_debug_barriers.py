"""Race check: the debug-barrier build (DIFFATTN_DEBUG_BARRIERS, a full workgroup barrier at
every step of the forward, backward and projection main loops) must give the same bits as
the normal build. A race between the wavefronts of a workgroup (an LDS slot refilled
while another wavefront still reads it, a read before the fill landed) depends on timing,
so the two builds would differ. Both libraries are the in-tree builds; the debug one is
libdiffattn_debug.so next to libdiffattn.so."""
import contextlib
import os

import pytest
import torch

from differential_attention_causal_amd import diffattn as da, synth

from tests.helpers import DEV

pytestmark = pytest.mark.gpu

DEBUG_LIB = os.path.join(os.path.dirname(da.LIB_PATH), "libdiffattn_debug.so")


@contextlib.contextmanager
def library(path):
    saved = (da._LIB, da.LIB_PATH)
    da._LIB, da.LIB_PATH = None, path
    try:
        yield da._lib()
    finally:
        da._LIB, da.LIB_PATH = saved


def both(fn):
    """fn() run on the normal build, then on the debug-barrier build."""
    if not os.path.exists(DEBUG_LIB):
        raise FileNotFoundError(f"{DEBUG_LIB} is not built (run __graft_entry__.build())")
    a = fn()
    torch.cuda.synchronize()
    with library(DEBUG_LIB):
        b = fn()
        torch.cuda.synchronize()
    return a, b


def same(a, b):
    """Bit-for-bit equality (compared as raw bytes, so -0.0 and 0.0 differ too)."""
    assert a.dtype == b.dtype and a.shape == b.shape
    assert torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("B,H,N,hkv", [(1, 2, 1000, None), (2, 4, 1537, 2)])
def test_forward_and_backward_bitwise_equal_to_debug_barrier_build(B, H, N, hkv):
    w = synth.custom("fwd", B, H, N, 64, 5, "bf16", number=4100 + N)
    x = synth.make_inputs(w, DEV)
    kv = {k: x[k] if hkv is None else x[k][:, :hkv].contiguous() for k in ("k1", "k2", "v")}
    gen = torch.Generator(device=DEV).manual_seed(4100 + N)
    dy = torch.randn(B, H, N, 128, device=DEV, generator=gen).to(torch.bfloat16)
    wgt = 1.0 + 0.1 * torch.randn(H, 128, device=DEV, generator=gen)

    def run():
        st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
        saved = da.alloc_saved(B, H, N, 64, DEV)
        y = da.forward(x["q1"], x["q2"], kv["k1"], kv["k2"], kv["v"], st, rms_weight=wgt,
                       saved=saved)
        g = da.backward(x["q1"], x["q2"], kv["k1"], kv["k2"], kv["v"], x["lq1"], x["lk1"],
                        x["lq2"], x["lk2"], st, saved, dy, rms_weight=wgt)
        return [y] + [saved[k] for k in sorted(saved)] + [g[k] for k in sorted(g)]

    a, b = both(run)
    assert len(a) == len(b)
    for u, v in zip(a, b):
        same(u, v)


def test_decode_bitwise_equal_to_debug_barrier_build():
    w = synth.custom("decode", 4, 8, 3000, 64, 7, "bf16", number=4300)
    x = synth.make_inputs(w, DEV)
    kv = {k: x[k][:, :2].contiguous() for k in ("k1", "k2", "v")}
    cl = torch.tensor([3000, 1, 2049, 777], dtype=torch.int32, device=DEV)

    def run():
        st = da.lambda_(x["lq1"], x["lk1"], x["lq2"], x["lk2"], w.layer)
        y1 = da.decode(x["q1"], x["q2"], x["k1"], x["k2"], x["v"], st, cache_len=cl)
        y2 = da.decode(x["q1"], x["q2"], kv["k1"], kv["k2"], kv["v"], st, cache_len=cl)
        return [y1, y2]

    a, b = both(run)
    for u, v in zip(a, b):
        same(u, v)


def test_projections_bitwise_equal_to_debug_barrier_build():
    B, N, H, dm = 1, 700, 4, 256
    xp = synth.make_proj_inputs(B, N, H, 64, dm, DEV, seed=4200)

    def run():
        q1, q2, k1, k2, v = da.qkv_proj(xp["x"], xp["w_qkv"], H, 64)
        y = da.out_proj(xp["attn"], xp["w_o"])
        return [q1, q2, k1, k2, v, y]

    a, b = both(run)
    for u, v in zip(a, b):
        same(u, v)
