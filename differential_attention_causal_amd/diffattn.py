"""ctypes binding of libdiffattn (argument marshalling only).

Every function here checks tensor placement and shapes, fills the C structs and
calls the C-ABI of ``include/diffattn.h`` on torch's current stream.  All
arithmetic happens in the library's HIP kernels; there is no fallback of any
kind: if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import struct
from typing import Dict, Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdiffattn.so")

OK, E_ARG, E_UNSUPPORTED, E_WORKSPACE, E_HIP, E_SCRATCH = 0, 1, 2, 3, 4, 5
DECODE_SCRATCH_BYTES = 32 << 20   # DIFFATTN_DECODE_SCRATCH_BYTES
FP32, BF16 = 0, 1
OP_FWD, OP_DECODE, OP_BWD = 0, 1, 2
LAYOUT_BHN, LAYOUT_BNH = 0, 1
_LAYOUTS = {"bhn": LAYOUT_BHN, "bnh": LAYOUT_BNH}

# Every symbol declared in include/diffattn.h.
EXPORTS = ("diffattn_lambda", "diffattn_lambda_layers", "diffattn_qkv_proj",
           "diffattn_out_proj", "diffattn_fwd", "diffattn_decode", "diffattn_decode_noalloc",
           "diffattn_cache_append",
           "diffattn_bwd", "diffattn_workspace_bytes", "diffattn_status_string",
           "diffattn_last_hip_error")


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("heads", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("head_dim", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("dtype", ctypes.c_int),
                ("out_layout", ctypes.c_int32), ("kv_heads", ctypes.c_int64)]


class Saved(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("lse1", "lse2", "o1", "o2", "rstd")]


LAMBDA_STATE_BYTES = 48  # 4 doubles + 4 floats
STATE_FMT = "<4d4f"   # diffattn_lambda_state: 4 doubles, 4 floats


class DiffAttnError(RuntimeError):
    def __init__(self, fn: str, status: int, hip: int = 0):
        self.status = status
        msg = _lib().diffattn_status_string(status).decode()
        if status == E_HIP:
            msg += f" (hipError_t {hip})"
        super().__init__(f"{fn}: {msg}")


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libdiffattn.so not built at {LIB_PATH}; run "
                              "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        lib.diffattn_status_string.restype = ctypes.c_char_p
        lib.diffattn_status_string.argtypes = [ctypes.c_int]
        lib.diffattn_last_hip_error.restype = ctypes.c_int
        lib.diffattn_last_hip_error.argtypes = []
        lib.diffattn_workspace_bytes.restype = ctypes.c_size_t
        lib.diffattn_workspace_bytes.argtypes = [ctypes.c_int, ctypes.POINTER(Problem)]
        lib.diffattn_lambda.restype = ctypes.c_int
        lib.diffattn_lambda.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P]
        lib.diffattn_lambda_layers.restype = ctypes.c_int
        lib.diffattn_lambda_layers.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_float, P, P, P, P, P,
                                               P]
        lib.diffattn_qkv_proj.restype = ctypes.c_int
        lib.diffattn_qkv_proj.argtypes = [ctypes.POINTER(Problem), ctypes.c_int64] + [P] * 8
        lib.diffattn_out_proj.restype = ctypes.c_int
        lib.diffattn_out_proj.argtypes = [ctypes.POINTER(Problem), ctypes.c_int64] + [P] * 4
        lib.diffattn_fwd.restype = ctypes.c_int
        lib.diffattn_fwd.argtypes = [ctypes.POINTER(Problem), P, P, P, P, P, P, P, P,
                                     ctypes.POINTER(Saved), P, ctypes.c_size_t, P]
        lib.diffattn_decode.restype = ctypes.c_int
        lib.diffattn_decode.argtypes = [ctypes.POINTER(Problem), P, P, P, P, P, P, P, P, P, P,
                                        ctypes.c_size_t, P]
        lib.diffattn_decode_noalloc.restype = ctypes.c_int
        lib.diffattn_decode_noalloc.argtypes = [ctypes.POINTER(Problem)] + [P] * 10
        lib.diffattn_cache_append.restype = ctypes.c_int
        lib.diffattn_cache_append.argtypes = [ctypes.POINTER(Problem), P, P, P, P, P, P, P, P]
        lib.diffattn_bwd.restype = ctypes.c_int
        lib.diffattn_bwd.argtypes = ([ctypes.POINTER(Problem)] + [P] * 11 +
                                     [ctypes.POINTER(Saved)] + [P] * 13 +
                                     [ctypes.c_size_t, P])
        _LIB = lib
    return _LIB


def lib():
    """The loaded ctypes library (raises ImportError if it was not built)."""
    return _lib()


def _check(fn: str, status: int):
    if status != OK:
        raise DiffAttnError(fn, status, _lib().diffattn_last_hip_error() if status == E_HIP else 0)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _nbytes(t) -> int:
    """Size in bytes of a workspace tensor (any dtype), 0 for None."""
    return 0 if t is None else t.numel() * t.element_size()


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FP32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need_cuda(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("libdiffattn tensors must live in GPU memory")
            if not t.is_contiguous():
                raise ValueError("libdiffattn tensors must be contiguous")


def problem(batch, heads, seqlen, head_dim, dtype_code, eps=1e-5, layout=LAYOUT_BHN,
            kv_heads=0) -> Problem:
    return Problem(int(batch), int(heads), int(seqlen), int(head_dim), 1, float(eps),
                   int(dtype_code), int(layout), int(kv_heads))


def _layout(name: str) -> int:
    if name not in _LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(_LAYOUTS)}")
    return _LAYOUTS[name]


def _y_shape(B, H, N, d, layout: int):
    return (B, N, H, 2 * d) if layout == LAYOUT_BNH else (B, H, N, 2 * d)


def workspace_bytes(op: int, p: Problem) -> int:
    return int(_lib().diffattn_workspace_bytes(op, ctypes.byref(p)))


# ------------------------------------------------------------------ lambda
def lambda_(lq1, lk1, lq2, lk2, layer: int) -> torch.Tensor:
    """Device lambda state (48 bytes, uint8 tensor) for one layer."""
    _need_cuda(lq1, lk1, lq2, lk2)
    for t in (lq1, lk1, lq2, lk2):
        if t.dtype != torch.float32 or t.dim() != 1 or t.numel() != lq1.numel():
            raise ValueError("lambda vectors must be float32 [d] of equal length")
    st = torch.empty(LAMBDA_STATE_BYTES, dtype=torch.uint8, device=lq1.device)
    _check("diffattn_lambda", _lib().diffattn_lambda(
        lq1.numel(), int(layer), _ptr(lq1), _ptr(lk1), _ptr(lq2), _ptr(lk2), _ptr(st),
        _stream(lq1.device)))
    return st


def lambda_layers(lq1s, lk1s, lq2s, lk2s, first_layer: int,
                  lambda_init: Optional[float] = None) -> torch.Tensor:
    """Device lambda states for layers first_layer .. first_layer + n - 1 (uint8 tensor
    [n, 48]); the vectors are float32 [n, d]. lambda_init None: the per-layer schedule;
    a number: that lambda_init for every layer."""
    _need_cuda(lq1s, lk1s, lq2s, lk2s)
    for t in (lq1s, lk1s, lq2s, lk2s):
        if (t.dtype != torch.float32 or t.dim() != 2 or t.shape != lq1s.shape
                or not t.is_contiguous()):
            raise ValueError("lambda vectors must be contiguous float32 [n_layers, d] of "
                             "equal shape")
    n, d = lq1s.shape
    st = torch.empty(n, LAMBDA_STATE_BYTES, dtype=torch.uint8, device=lq1s.device)
    fixed = 0 if lambda_init is None else 1
    init = 0.0 if lambda_init is None else float(lambda_init)
    _check("diffattn_lambda_layers", _lib().diffattn_lambda_layers(
        d, n, int(first_layer), fixed, init, _ptr(lq1s), _ptr(lk1s), _ptr(lq2s), _ptr(lk2s),
        _ptr(st), _stream(lq1s.device)))
    return st


def read_lambda_state(st: torch.Tensor) -> Dict[str, float]:
    raw = bytes(st.cpu().numpy().tobytes())
    v = struct.unpack(STATE_FMT, raw)
    return {"lambda": v[0], "lambda_init": v[1], "exp_a": v[2], "exp_b": v[3],
            "lambda_f32": v[4], "lambda_init_f32": v[5], "one_minus_init_f32": v[6]}


# ------------------------------------------------------------------ projections
def qkv_proj(x, w_qkv, heads: int, head_dim: int, out=None, kv_heads: Optional[int] = None):
    """X [B, N, d_model] (bf16) times the fused weight [(H + 2 Hkv) 2d, d_model] (W_Q, W_K,
    W_V rows; Hkv = kv_heads, default H). Returns (q1, q2 [B, H, N, d], k1, k2
    [B, Hkv, N, d], v [B, Hkv, N, 2d])."""
    _need_cuda(x, w_qkv)
    if x.dim() != 3 or x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError("x must be contiguous bfloat16 [B, N, d_model]")
    B, N, dm = x.shape
    H, d = int(heads), int(head_dim)
    Hkv = H if kv_heads is None else int(kv_heads)
    if (tuple(w_qkv.shape) != (2 * d * (H + 2 * Hkv), dm) or w_qkv.dtype != torch.bfloat16
            or not w_qkv.is_contiguous()):
        raise ValueError("w_qkv must be contiguous bfloat16 [(H + 2 Hkv) 2d, d_model]")
    if out is None:
        f = dict(dtype=torch.bfloat16, device=x.device)
        out = (torch.empty(B, H, N, d, **f), torch.empty(B, H, N, d, **f),
               torch.empty(B, Hkv, N, d, **f), torch.empty(B, Hkv, N, d, **f),
               torch.empty(B, Hkv, N, 2 * d, **f))
    p = problem(B, H, N, d, BF16, kv_heads=Hkv)
    _check("diffattn_qkv_proj", _lib().diffattn_qkv_proj(
        ctypes.byref(p), dm, _ptr(x), _ptr(w_qkv), *(_ptr(t) for t in out),
        _stream(x.device)))
    return out


def out_proj(attn, w_o, out=None):
    """attn [B, N, H, 2d] (the forward's token-major output, bf16) times W_O^T, W_O
    [d_model, H 2d]. Returns Y [B, N, d_model]."""
    _need_cuda(attn, w_o)
    if attn.dim() != 4 or attn.dtype != torch.bfloat16 or not attn.is_contiguous():
        raise ValueError("attn must be contiguous bfloat16 [B, N, H, 2d]")
    B, N, H, d2 = attn.shape
    if (w_o.dim() != 2 or w_o.shape[1] != H * d2 or w_o.dtype != torch.bfloat16
            or not w_o.is_contiguous()):
        raise ValueError("w_o must be contiguous bfloat16 [d_model, H 2d]")
    dm = w_o.shape[0]
    if out is None:
        out = torch.empty(B, N, dm, dtype=torch.bfloat16, device=attn.device)
    p = problem(B, H, N, d2 // 2, BF16)
    _check("diffattn_out_proj", _lib().diffattn_out_proj(
        ctypes.byref(p), dm, _ptr(attn), _ptr(w_o), _ptr(out), _stream(attn.device)))
    return out


# ------------------------------------------------------------------ forward
def alloc_saved(B, H, N, d, device) -> Dict[str, torch.Tensor]:
    f = dict(dtype=torch.float32, device=device)
    return {"lse1": torch.empty(B, H, N, **f), "lse2": torch.empty(B, H, N, **f),
            "o1": torch.empty(B, H, N, 2 * d, **f), "o2": torch.empty(B, H, N, 2 * d, **f),
            "rstd": torch.empty(B, H, N, **f)}


def _saved_struct(sv: Optional[Dict[str, torch.Tensor]]):
    if sv is None:
        return None
    return Saved(*(sv[k].data_ptr() for k in ("lse1", "lse2", "o1", "o2", "rstd")))


def forward(q1, q2, k1, k2, v, lam_state, rms_weight=None, eps: float = 1e-5,
            out: Optional[torch.Tensor] = None, saved: Optional[Dict[str, torch.Tensor]] = None,
            workspace: Optional[torch.Tensor] = None, layout: str = "bhn"):
    """Causal DiffAttn forward. Q/K [B,H,N,d], V [B,H,N,2d] (float32 or bfloat16).

    Returns Y [B,H,N,2d] (layout "bhn") or [B,N,H,2d] (layout "bnh", the heads of a
    token side by side, as the output projection takes them).  ``saved`` (from
    ``alloc_saved``) requests the training saves.  ``workspace``: a uint8 device tensor
    of at least ``workspace_bytes(OP_FWD, ...)`` bytes (allocated here when omitted).
    """
    lay = _layout(layout)
    _need_cuda(q1, q2, k1, k2, v, lam_state, rms_weight, out, workspace)
    B, H, N, d = q1.shape
    Hkv = k1.shape[1]     # fewer K/V heads than query heads: grouped-query attention
    if tuple(q2.shape) != (B, H, N, d) or q2.dtype != q1.dtype:
        raise ValueError("Q1, Q2 must share shape and dtype")
    for t in (k1, k2):
        if tuple(t.shape) != (B, Hkv, N, d) or t.dtype != q1.dtype:
            raise ValueError("K1, K2 must be [B, Hkv, N, d] of the queries' dtype")
    if tuple(v.shape) != (B, Hkv, N, 2 * d) or v.dtype != q1.dtype:
        raise ValueError("V must be [B, Hkv, N, 2d] of the same dtype")
    if out is None:
        out = torch.empty(_y_shape(B, H, N, d, lay), dtype=v.dtype, device=v.device)
    elif tuple(out.shape) != _y_shape(B, H, N, d, lay):
        raise ValueError("out does not match the layout")
    p = problem(B, H, N, d, _dtype_code(q1), eps, lay, kv_heads=Hkv)
    svs = _saved_struct(saved)
    need = workspace_bytes(OP_FWD, p)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q1.device)
    _check("diffattn_fwd", _lib().diffattn_fwd(
        ctypes.byref(p), _ptr(q1), _ptr(q2), _ptr(k1), _ptr(k2), _ptr(v), _ptr(lam_state),
        _ptr(rms_weight), _ptr(out), ctypes.byref(svs) if svs is not None else None,
        _ptr(workspace), _nbytes(workspace), _stream(q1.device)))
    return out


# ------------------------------------------------------------------ decode
def decode(q1, q2, k1c, k2c, vc, lam_state, cache_len=None, rms_weight=None, eps: float = 1e-5,
           out=None, workspace=None):
    """One decode step: q [B,H,d], caches [B,Hkv,L,d] / [B,Hkv,L,2d] (Hkv dividing H:
    grouped-query attention when Hkv < H), cache_len int32 [B]."""
    _need_cuda(q1, q2, k1c, k2c, vc, lam_state, cache_len, rms_weight, out, workspace)
    B, Hkv, L, d = k1c.shape
    H = q1.shape[1]
    if tuple(q1.shape) != (B, H, d) or tuple(q2.shape) != (B, H, d):
        raise ValueError("queries must be [B, H, d]")
    if tuple(k2c.shape) != (B, Hkv, L, d) or tuple(vc.shape) != (B, Hkv, L, 2 * d):
        raise ValueError("caches must be [B, Hkv, L, d] and [B, Hkv, L, 2d]")
    p = problem(B, H, L, d, _dtype_code(k1c), eps, kv_heads=Hkv)
    if out is None:
        out = torch.empty(B, H, 2 * d, dtype=vc.dtype, device=vc.device)
    need = workspace_bytes(OP_DECODE, p)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=vc.device)
    _check("diffattn_decode", _lib().diffattn_decode(
        ctypes.byref(p), _ptr(q1), _ptr(q2), _ptr(k1c), _ptr(k2c), _ptr(vc), _ptr(cache_len),
        _ptr(lam_state), _ptr(rms_weight), _ptr(out), _ptr(workspace), _nbytes(workspace),
        _stream(vc.device)))
    return out


def decode_noalloc(q1, q2, k1c, k2c, vc, lam_state, cache_len=None, rms_weight=None,
                   eps: float = 1e-5, out=None):
    """decode() through the allocation-free entry point: the split partials live in the
    library's static per-device scratch, so no workspace is passed (``out`` is still
    allocated here when omitted). Calls that overlap on one device race."""
    _need_cuda(q1, q2, k1c, k2c, vc, lam_state, cache_len, rms_weight, out)
    B, Hkv, L, d = k1c.shape
    H = q1.shape[1]
    if tuple(q1.shape) != (B, H, d) or tuple(q2.shape) != (B, H, d):
        raise ValueError("queries must be [B, H, d]")
    if tuple(k2c.shape) != (B, Hkv, L, d) or tuple(vc.shape) != (B, Hkv, L, 2 * d):
        raise ValueError("caches must be [B, Hkv, L, d] and [B, Hkv, L, 2d]")
    p = problem(B, H, L, d, _dtype_code(k1c), eps, kv_heads=Hkv)
    if out is None:
        out = torch.empty(B, H, 2 * d, dtype=vc.dtype, device=vc.device)
    _check("diffattn_decode_noalloc", _lib().diffattn_decode_noalloc(
        ctypes.byref(p), _ptr(q1), _ptr(q2), _ptr(k1c), _ptr(k2c), _ptr(vc), _ptr(cache_len),
        _ptr(lam_state), _ptr(rms_weight), _ptr(out), _stream(vc.device)))
    return out


# ------------------------------------------------------------------ cache append
def cache_append(k1_new, k2_new, v_new, k1c, k2c, vc, cache_len):
    """Appends one token per sequence in place: rows [B,H,d]/[B,H,2d] go to cache row
    cache_len[b] (if below L), and cache_len [B] int32 is incremented on the device."""
    _need_cuda(k1_new, k2_new, v_new, k1c, k2c, vc, cache_len)
    B, H, L, d = k1c.shape
    p = problem(B, H, L, d, _dtype_code(k1c))
    _check("diffattn_cache_append", _lib().diffattn_cache_append(
        ctypes.byref(p), _ptr(k1_new), _ptr(k2_new), _ptr(v_new), _ptr(k1c), _ptr(k2c),
        _ptr(vc), _ptr(cache_len), _stream(k1c.device)))


# ------------------------------------------------------------------ backward
def backward(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, lam_state, saved, dout, rms_weight=None,
             eps: float = 1e-5, workspace=None, layout: str = "bhn",
             weight_grad: bool = True):
    """Gradients of sum(Y * dout); returns a dict of device tensors. ``dout`` is in the
    forward's output layout; ``d_rms_weight`` [H, 2d] is included when weight_grad."""
    _need_cuda(q1, q2, k1, k2, v, lq1, lk1, lq2, lk2, lam_state, dout, rms_weight, workspace)
    B, H, N, d = q1.shape
    lay = _layout(layout)
    if tuple(dout.shape) != _y_shape(B, H, N, d, lay):
        raise ValueError("dout does not match the layout")
    Hkv = k1.shape[1]     # grouped-query attention when fewer than H
    p = problem(B, H, N, d, _dtype_code(q1), eps, lay, kv_heads=Hkv)
    g = {"dq1": torch.empty_like(q1), "dq2": torch.empty_like(q2), "dk1": torch.empty_like(k1),
         "dk2": torch.empty_like(k2), "dv": torch.empty_like(v),
         "d_attn": torch.empty(B, H, N, 2 * d, dtype=torch.float32, device=q1.device)}
    for k in ("dlq1", "dlk1", "dlq2", "dlk2"):
        g[k] = torch.empty(d, dtype=torch.float32, device=q1.device)
    if weight_grad:
        g["d_rms_weight"] = torch.empty(H, 2 * d, dtype=torch.float32, device=q1.device)
    need = workspace_bytes(OP_BWD, p)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q1.device)
    svs = _saved_struct(saved)
    _check("diffattn_bwd", _lib().diffattn_bwd(
        ctypes.byref(p), _ptr(q1), _ptr(q2), _ptr(k1), _ptr(k2), _ptr(v), _ptr(lq1), _ptr(lk1),
        _ptr(lq2), _ptr(lk2), _ptr(lam_state), _ptr(rms_weight),
        ctypes.byref(svs) if svs is not None else None, _ptr(dout),
        _ptr(g["dq1"]), _ptr(g["dq2"]), _ptr(g["dk1"]), _ptr(g["dk2"]), _ptr(g["dv"]),
        _ptr(g["d_attn"]), _ptr(g["dlq1"]), _ptr(g["dlk1"]), _ptr(g["dlq2"]), _ptr(g["dlk2"]),
        _ptr(g.get("d_rms_weight")), _ptr(workspace), _nbytes(workspace), _stream(q1.device)))
    return g
