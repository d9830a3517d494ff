"""C-ABI checks that need no GPU: the library loads, exports every declared symbol,
and rejects invalid arguments with a status code before any HIP call.

Every call here is invalid on purpose, so no kernel is ever launched; the fake
device addresses are never dereferenced.
"""
import ctypes
import os
import re

import pytest
import torch

from differential_attention_causal_amd import diffattn as da

# Host logic only. The calls below carry fake device addresses and are all invalid, so
# none may reach a kernel; on a machine with a GPU the module is skipped rather than
# trusting that with real hardware attached.
pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="host-only argument checks with fake addresses")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "diffattn.h")

A = 1 << 20  # fake 16-byte aligned addresses, spaced far apart
def addr(i):
    return ctypes.c_void_p(A * (i + 1))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(diffattn_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(da.EXPORTS)
    lib = da.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = da.lib()
    for s in range(6):
        assert lib.diffattn_status_string(s).decode().startswith("DIFFATTN_")
    assert lib.diffattn_last_hip_error() == 0


WS = addr(40)            # a fake workspace far from the other fake buffers


def fwd(p, ptrs=None, saved=None, ws=WS, ws_bytes=1 << 20):
    ptrs = ptrs or [addr(i) for i in range(8)]
    return da.lib().diffattn_fwd(ctypes.byref(p), *ptrs, saved, ws, ws_bytes, None)


def test_forward_argument_checks():
    bf = lambda **kw: da.problem(**{**dict(batch=1, heads=2, seqlen=64, head_dim=64,
                                           dtype_code=da.BF16), **kw})
    lib = da.lib()
    assert lib.diffattn_fwd(None, *[addr(i) for i in range(8)], None, None, 0, None) == da.E_ARG
    assert fwd(bf(batch=-1)) == da.E_ARG
    assert fwd(bf(seqlen=-5)) == da.E_ARG
    assert fwd(bf(head_dim=0)) == da.E_ARG
    assert fwd(bf(head_dim=128)) == da.E_UNSUPPORTED
    assert fwd(bf(head_dim=16)) == da.E_UNSUPPORTED
    assert fwd(da.problem(1, 2, 64, 48, da.FP32)) == da.E_UNSUPPORTED
    p = bf(); p.causal = 0
    assert fwd(p) == da.E_UNSUPPORTED
    p = bf(); p.rms_eps = -1.0
    assert fwd(p) == da.E_ARG
    p = bf(); p.rms_eps = float("nan")
    assert fwd(p) == da.E_ARG
    p = bf(); p.dtype = 7
    assert fwd(p) == da.E_ARG
    # null tensor pointers
    for i in range(7):
        ptrs = [addr(j) for j in range(8)]
        if i == 6:
            i = 7  # out (index 6 is the optional RMSNorm weight)
        ptrs[i] = None
        assert fwd(bf(), ptrs) == da.E_ARG
    # misaligned pointer
    ptrs = [addr(j) for j in range(8)]
    ptrs[2] = ctypes.c_void_p(A * 3 + 2)
    assert fwd(bf(), ptrs) == da.E_ARG
    # output overlapping an input
    ptrs = [addr(j) for j in range(8)]
    ptrs[7] = ctypes.c_void_p(A * 1 + 64)
    assert fwd(bf(), ptrs) == da.E_ARG
    # saved buffers with a null field
    sv = da.Saved(A * 20, A * 21, A * 22, None, A * 24)
    assert fwd(bf(), saved=ctypes.byref(sv)) == da.E_ARG
    # float32 with training saves is not implemented
    sv = da.Saved(A * 20, A * 21, A * 22, A * 23, A * 24)
    assert fwd(da.problem(1, 2, 64, 16, da.FP32), saved=ctypes.byref(sv)) == da.E_UNSUPPORTED
    # overflow of the element count
    assert fwd(bf(batch=1 << 40, heads=1 << 20)) == da.E_ARG
    # bf16 sequences beyond the kernels' 32-bit per-head buffer offsets
    assert fwd(bf(batch=1, heads=1, seqlen=(1 << 22) + 1)) == da.E_UNSUPPORTED
    # bf16 needs its workspace: missing, too small, misaligned, overlapping the output
    need = da.workspace_bytes(da.OP_FWD, bf())
    assert need == 2 * 1 * 32
    assert fwd(bf(), ws=None, ws_bytes=0) == da.E_WORKSPACE
    assert fwd(bf(), ws_bytes=need - 1) == da.E_WORKSPACE
    assert fwd(bf(), ws=ctypes.c_void_p(A * 41 + 8), ws_bytes=need) == da.E_ARG
    assert fwd(bf(), ws=addr(7), ws_bytes=need) == da.E_ARG
    # float32 needs none
    assert da.workspace_bytes(da.OP_FWD, da.problem(1, 2, 64, 16, da.FP32)) == 0


def test_empty_problems_are_noops():
    # nothing to compute: valid, no pointer needed, no HIP call
    nul = [None] * 8
    for kw in (dict(batch=0), dict(heads=0), dict(seqlen=0)):
        p = da.problem(**{**dict(batch=2, heads=2, seqlen=16, head_dim=64,
                                 dtype_code=da.BF16), **kw})
        assert fwd(p, nul) == da.OK
        assert da.workspace_bytes(da.OP_DECODE, p) == 0
        assert da.lib().diffattn_decode(ctypes.byref(p), *[None] * 9, None, 0, None) == da.OK


def test_lambda_argument_checks():
    lib = da.lib()
    ptr = [addr(i) for i in range(5)]
    assert lib.diffattn_lambda(0, 1, *ptr, None) == da.E_ARG
    assert lib.diffattn_lambda(2000, 1, *ptr, None) == da.E_ARG
    assert lib.diffattn_lambda(64, 0, *ptr, None) == da.E_ARG
    assert lib.diffattn_lambda(64, -3, *ptr, None) == da.E_ARG
    assert lib.diffattn_lambda(64, 1, None, *ptr[1:], None) == da.E_ARG
    assert lib.diffattn_lambda(64, 1, *ptr[:4], None, None) == da.E_ARG
    assert lib.diffattn_lambda(64, 1, *ptr[:4], ctypes.c_void_p(A * 9 + 4), None) == da.E_ARG
    # state overlapping a lambda vector
    assert lib.diffattn_lambda(64, 1, *ptr[:4], ctypes.c_void_p(A + 8), None) == da.E_ARG


def test_lambda_layers_argument_checks():
    lib = da.lib()
    ptr = [addr(i * 64) for i in range(5)]   # four [n, 64] vectors and the states
    call = lambda d, n, first, mode, init, p: lib.diffattn_lambda_layers(d, n, first, mode,
                                                                         init, *p, None)
    assert call(0, 4, 1, 0, 0.0, ptr) == da.E_ARG
    assert call(1025, 4, 1, 0, 0.0, ptr) == da.E_ARG
    assert call(64, -1, 1, 0, 0.0, ptr) == da.E_ARG
    assert call(64, 65536, 1, 0, 0.0, ptr) == da.E_ARG
    assert call(64, 4, 0, 0, 0.0, ptr) == da.E_ARG
    assert call(64, 4, 2 ** 31 - 2, 0, 0.0, ptr) == da.E_ARG      # last index past int32
    assert call(64, 4, 1, 2, 0.8, ptr) == da.E_ARG                # unknown mode
    for bad_init in (float("inf"), float("-inf"), float("nan")):
        assert call(64, 4, 1, 1, bad_init, ptr) == da.E_ARG
    # nothing to do: OK without touching any pointer; the schedule ignores lambda_init
    assert call(64, 0, 1, 0, float("nan"), [None] * 5) == da.OK
    assert call(64, 0, 1, 1, 0.8, [None] * 5) == da.OK
    bad = list(ptr); bad[2] = None
    assert call(64, 4, 1, 1, 0.8, bad) == da.E_ARG
    bad = list(ptr); bad[4] = ctypes.c_void_p(A * 4 * 64 + 4)   # states not 8-byte aligned
    assert call(64, 4, 1, 0, 0.0, bad) == da.E_ARG
    bad = list(ptr); bad[1] = ctypes.c_void_p(A * 64 + 2)   # vector not 4-byte aligned
    assert call(64, 4, 1, 0, 0.0, bad) == da.E_ARG
    # states overlapping the last row of the third vector array ([4, 64] float32 = 1 KiB)
    bad = list(ptr); bad[4] = ctypes.c_void_p(A * (2 * 64 + 1) + 1024 - 8)
    assert call(64, 4, 1, 0, 0.0, bad) == da.E_ARG


def test_rms_eps_must_be_finite():
    lib = da.lib()
    ptrs = [addr(i * 64) for i in range(9)]
    for eps in (float("nan"), float("inf"), -1e-6):
        p = da.problem(1, 1, 16, 64, da.BF16)
        p.rms_eps = eps
        assert lib.diffattn_fwd(ctypes.byref(p), *ptrs[:8], None, None, 0, None) == da.E_ARG
    # the same call with a valid eps gets past the problem checks (to the workspace check)
    p = da.problem(1, 1, 16, 64, da.BF16)
    assert lib.diffattn_fwd(ctypes.byref(p), *ptrs[:8], None, None, 0, None) == da.E_WORKSPACE


def test_decode_argument_checks():
    lib = da.lib()
    p = da.problem(64, 16, 8192, 64, da.BF16)
    need = da.workspace_bytes(da.OP_DECODE, p)
    assert need > 0
    ptrs = [addr(i * 64) for i in range(9)]   # q1 q2 k1 k2 v len lam w out
    ws = addr(64 * 40)
    call = lambda p, ptrs, ws, n: lib.diffattn_decode(ctypes.byref(p), *ptrs, ws, n, None)
    assert call(p, ptrs, None, need) == da.E_WORKSPACE
    assert call(p, ptrs, ws, need - 4) == da.E_WORKSPACE
    assert call(da.problem(64, 16, 8192, 64, da.FP32), ptrs, ws, need) == da.E_UNSUPPORTED
    assert call(da.problem(64, 16, 8192, 32, da.BF16), ptrs, ws, need) == da.E_UNSUPPORTED
    bad = list(ptrs); bad[0] = None
    assert call(p, bad, ws, need) == da.E_ARG
    bad = list(ptrs); bad[8] = ptrs[2]      # out aliases the K1 cache
    assert call(p, bad, ws, need) == da.E_ARG
    bad = list(ptrs); bad[5] = ctypes.c_void_p(A * 5 * 64 + 2)   # misaligned cache_len
    assert call(p, bad, ws, need) == da.E_ARG
    # caches beyond the kernel's 32-bit per-head buffer offsets
    long = da.problem(1, 1, (1 << 22) + 1, 64, da.BF16)
    assert call(long, ptrs, ws, need) == da.E_UNSUPPORTED


def test_decode_noalloc_argument_checks():
    """The allocation-free decode runs the same host checks as diffattn_decode, and
    rejects a problem whose partials exceed the static scratch before any HIP call."""
    lib = da.lib()
    ptrs = [addr(i * 64) for i in range(9)]   # q1 q2 k1 k2 v len lam w out
    call = lambda p, ptrs: lib.diffattn_decode_noalloc(ctypes.byref(p), *ptrs, None)
    big = da.problem(64, 16, 1 << 20, 64, da.BF16)
    assert da.workspace_bytes(da.OP_DECODE, big) > da.DECODE_SCRATCH_BYTES
    assert call(big, ptrs) == da.E_SCRATCH
    fits = da.problem(64, 16, 8192, 64, da.BF16)
    assert da.workspace_bytes(da.OP_DECODE, fits) <= da.DECODE_SCRATCH_BYTES
    assert call(da.problem(64, 16, 8192, 64, da.FP32), ptrs) == da.E_UNSUPPORTED
    bad = list(ptrs); bad[0] = None
    assert call(fits, bad) == da.E_ARG
    bad = list(ptrs); bad[8] = ptrs[2]      # out aliases the K1 cache
    assert call(fits, bad) == da.E_ARG
    assert call(da.problem(0, 16, 8192, 64, da.BF16), ptrs) == da.OK
    assert "scratch" in lib.diffattn_status_string(da.E_SCRATCH).decode()


def test_cache_append_argument_checks():
    lib = da.lib()
    p = da.problem(4, 2, 128, 64, da.BF16)
    ptrs = [addr(i * 64) for i in range(7)]   # k1n k2n vn k1c k2c vc len
    call = lambda p, ptrs: lib.diffattn_cache_append(ctypes.byref(p), *ptrs, None)
    assert call(da.problem(4, 2, 128, 64, da.FP32), ptrs) == da.E_UNSUPPORTED
    assert call(da.problem(4, 2, 128, 32, da.BF16), ptrs) == da.E_UNSUPPORTED
    assert call(da.problem(1, 1, (1 << 22) + 1, 64, da.BF16), ptrs) == da.E_UNSUPPORTED
    for i in range(7):
        bad = list(ptrs); bad[i] = None
        assert call(p, bad) == da.E_ARG, i
    bad = list(ptrs); bad[1] = ctypes.c_void_p(A * 65 + 8)      # misaligned row
    assert call(p, bad) == da.E_ARG
    bad = list(ptrs); bad[6] = ctypes.c_void_p(A * 64 * 7 + 2)  # misaligned cache_len
    assert call(p, bad) == da.E_ARG
    bad = list(ptrs); bad[2] = ptrs[5]                          # new V row inside the V cache
    assert call(p, bad) == da.E_ARG
    bad = list(ptrs); bad[4] = ptrs[3]                          # K2 cache aliases K1 cache
    assert call(p, bad) == da.E_ARG
    bad = list(ptrs); bad[6] = ctypes.c_void_p(A * 193 + 16)     # length inside the K1 cache
    assert call(p, bad) == da.E_ARG
    # nothing to append: valid, no pointer needed
    assert call(da.problem(0, 2, 128, 64, da.BF16), [None] * 7) == da.OK


def test_backward_argument_checks():
    lib = da.lib()
    p = da.problem(2, 2, 128, 64, da.BF16)
    need = da.workspace_bytes(da.OP_BWD, p)
    assert need > 0
    ptrs = [addr(i * 64) for i in range(27)]
    sv = da.Saved(*(A * 64 * (40 + i) for i in range(5)))
    def call(p, ptrs, saved, ws, n):
        args = ptrs[:11] + [saved] + ptrs[11:23]
        return lib.diffattn_bwd(ctypes.byref(p), *args, ws, n, None)
    ws = addr(64 * 60)
    assert call(p, ptrs, ctypes.byref(sv), None, need) == da.E_WORKSPACE
    assert call(p, ptrs, ctypes.byref(sv), ws, need - 1) == da.E_WORKSPACE
    assert call(p, ptrs, None, ws, need) == da.E_ARG
    assert call(da.problem(2, 2, 128, 16, da.BF16), ptrs, ctypes.byref(sv), ws, need) == \
        da.E_UNSUPPORTED
    bad = list(ptrs); bad[12] = ptrs[0]     # dq1 aliases q1
    assert call(p, bad, ctypes.byref(sv), ws, need) == da.E_ARG
    bad = list(ptrs); bad[5] = None         # lq1
    assert call(p, bad, ctypes.byref(sv), ws, need) == da.E_ARG
    long = da.problem(1, 1, (1 << 22) + 1, 64, da.BF16)
    assert call(long, ptrs, ctypes.byref(sv), ws, need) == da.E_UNSUPPORTED
    bad = list(ptrs); bad[22] = ptrs[5]     # d_rms_weight aliases lq1
    assert call(p, bad, ctypes.byref(sv), ws, need) == da.E_ARG
    bad = list(ptrs); bad[22] = ctypes.c_void_p(A * 64 * 30 + 2)   # misaligned
    assert call(p, bad, ctypes.byref(sv), ws, need) == da.E_ARG
    lay = da.problem(2, 2, 128, 64, da.BF16, layout=2)                # unknown layout
    assert call(lay, ptrs, ctypes.byref(sv), ws, need) == da.E_ARG


def test_workspace_queries():
    # forward: 8 words of row flags per block of 256 query rows
    assert da.workspace_bytes(da.OP_FWD, da.problem(4, 8, 2048, 64, da.BF16)) == 4 * 8 * 8 * 32
    assert da.workspace_bytes(da.OP_FWD, da.problem(1, 1, 257, 64, da.BF16)) == 2 * 32
    assert da.workspace_bytes(da.OP_FWD, da.problem(4, 8, 2048, 64, da.FP32)) == 0
    p = da.problem(64, 16, 8192, 64, da.BF16)
    # per (b, h, split): 2 maps x (m, l, 128 accumulators) float32
    n = da.workspace_bytes(da.OP_DECODE, p)
    assert n % (64 * 16 * 2 * 130 * 4) == 0
    bad = da.problem(-1, 1, 1, 64, da.BF16)
    assert da.workspace_bytes(da.OP_BWD, bad) == 0


def test_projection_argument_checks():
    lib = da.lib()
    ptr = [addr(i * 64) for i in range(7)]
    p = da.problem(1, 16, 1024, 64, da.BF16)
    qkv = lambda p, dm, ptrs: lib.diffattn_qkv_proj(ctypes.byref(p), dm, *ptrs, None)
    outp = lambda p, dm, ptrs: lib.diffattn_out_proj(ctypes.byref(p), dm, *ptrs, None)
    assert qkv(p, 100, ptr) == da.E_UNSUPPORTED            # d_model not a multiple of 64
    assert qkv(p, 32, ptr) == da.E_ARG
    assert qkv(p, 1 << 17, ptr) == da.E_ARG
    assert qkv(da.problem(1, 16, 1024, 64, da.FP32), 2048, ptr) == da.E_UNSUPPORTED
    assert qkv(da.problem(1, 16, 1024, 48, da.BF16), 2048, ptr) == da.E_UNSUPPORTED
    assert qkv(da.problem(0, 16, 1024, 64, da.BF16), 2048, [None] * 7) == da.OK
    bad = list(ptr); bad[3] = None
    assert qkv(p, 2048, bad) == da.E_ARG
    bad = list(ptr); bad[0] = ctypes.c_void_p(A + 8)      # x misaligned
    assert qkv(p, 2048, bad) == da.E_ARG
    bad = list(ptr); bad[6] = ptr[0]                      # v aliases x
    assert qkv(p, 2048, bad) == da.E_ARG
    bad = list(ptr); bad[3] = ptr[2]                      # q2 aliases q1
    assert qkv(p, 2048, bad) == da.E_ARG
    assert outp(p, 96, ptr[:3]) == da.E_UNSUPPORTED
    bad = [ptr[0], ptr[1], ptr[0]]                        # y aliases attn
    assert outp(p, 2048, bad) == da.E_ARG
    # more rows than the GEMM takes
    assert qkv(da.problem(1 << 16, 1, 1 << 15, 64, da.BF16), 2048, ptr) == da.E_UNSUPPORTED


def test_grouped_query_argument_checks():
    lib = da.lib()
    ptrs = [addr(i * 64) for i in range(10)]
    ws = addr(64 * 60)
    fwd = lambda p: lib.diffattn_fwd(ctypes.byref(p), *ptrs[:8], None, ws, 1 << 20, None)
    assert fwd(da.problem(1, 8, 64, 64, da.BF16, kv_heads=3)) == da.E_ARG    # 3 does not divide 8
    assert fwd(da.problem(1, 8, 64, 64, da.BF16, kv_heads=16)) == da.E_ARG   # more K/V than Q heads
    assert fwd(da.problem(1, 8, 64, 64, da.BF16, kv_heads=-1)) == da.E_ARG
    # the backward also validates the grouping
    p = da.problem(2, 4, 128, 64, da.BF16, kv_heads=3)
    sv = da.Saved(*(A * 64 * (40 + i) for i in range(5)))
    args = [addr(i * 64) for i in range(23)]
    st = lib.diffattn_bwd(ctypes.byref(p), *args[:11], ctypes.byref(sv), *args[11:23], ws,
                          1 << 30, None)
    assert st == da.E_ARG


def test_call_logging_with_diffattn_log(tmp_path):
    """DIFFATTN_LOG=1 writes one line per entry-point call, with the problem shape, to
    stderr (here for calls the argument checks reject, so no GPU is touched)."""
    import subprocess
    import sys
    code = (
        "import ctypes\n"
        "from differential_attention_causal_amd import diffattn as da\n"
        "lib = da.lib()\n"
        "p = da.problem(2, 3, 17, 64, da.BF16)\n"
        "r = lib.diffattn_fwd(ctypes.byref(p), *([None] * 10), 0, None)\n"
        "assert r == da.E_ARG, r\n"
        "r = lib.diffattn_lambda(64, 1, *([None] * 6))\n"
        "assert r == da.E_ARG, r\n")
    env = dict(os.environ, DIFFATTN_LOG="1", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       cwd=ROOT, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "[diffattn] diffattn_fwd B=2 H=3 N=17 d=64 kv_heads=0 dtype=1" in r.stderr, r.stderr
    assert "[diffattn] diffattn_lambda\n" in r.stderr, r.stderr
