"""Float64 CPU oracle for causal differential attention (DiffAttn).

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain definition that the
HIP library is checked against.  Only the tests, the smoke check of the package
entry file and the CPU-baseline leg of the benchmark may import it; the library
and its Python binding never do, and this module imports nothing from them.

Every function takes numpy arrays (any float dtype; they are upcast exactly to
float64) and computes in float64.  Attention maps are materialised block by
block of query rows; nothing is fused or reordered beyond what the formulas
state.

Sources (page title, then section / equation):
  [HADA]   "Differential Transformer: Transformer que cancela ruido de atencao"
           (pt.news.hada.io), sections "Como a atencao diferencial funciona" and
           "Estrutura multi-head e arquitetura completa".
  [PRIOR]  "Differential Transformer: Canceling Context Noise with Differential
           Attention" (priorstack.com, Attention Mechanism tag page), section
           "Cancelling Context Noise Through Attention Map Subtraction".
  [INTOAI] "A Simple Principle From Noise-Cancelling Headphones Supercharges
           Transformers Like Never Before" (intoai.pub), sections "A Deeper Dive
           Into Attention Calculations" (causal mask) and "Differential Attention
           With Multiple Heads" (lambda shared per layer, per-head RMSNorm,
           scale by 1 - lambda_init).
  [BOOK]   "The Evolution of Transformer Attention" (open-bookmarks-2024.blogspot.com),
           section "Implementation and Future Prospects" (DiffAttn combined with
           grouped-query attention).
  [MLA]    "Multi-Head Latent Attention: Scaling LLM Serving Throughput via
           Low-Rank KV Compression" (priorstack.com, same tag page), section
           "The Memory Wall: Why the KV Cache Constrains LLM Serving" (the decode
           step reads the whole cache, which grows by one token per step).

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * 1/sqrt(d) uses d = width of one half (Q1, K1); V and the output are 2d wide.
  * the lambda vectors have length d.
  * RMSNorm over one head's 2d channels: x * (mean(x^2) + eps)^(-1/2) * w,
    eps added inside the root.
  * Y = (1 - lambda_init) * RMSNorm(O).
  * the backward pass is not printed on the pages; ``backward`` derives it by
    the chain rule from the forward definition.

Parity pins (tests/test_oracle.py): lambda_init closed form and limits, zero
lambda vectors, lambda = 0 against torch's float64 causal scaled-dot-product
attention, Q2 = Q1 and K2 = K1 giving (1 - lambda) times softmax attention,
rows of each map summing to one, row 0 attending only to V row 0, mask
perturbation invariance, RMSNorm against torch's rms_norm, a scalar brute-force
twin on tiny shapes, decode equal to the last prefill row, grouped-query
attention equal to the same computation with K/V repeated per head, append-then-decode
equal to the prefill row of the extended sequence, central finite
differences of the forward for every gradient, and, for the epilogue's own
backward, central differences in O1, in lambda with O1 and O2 held fixed, in the
scale of each O1 row and in the norm weight, plus equality of its dlambda with
the full backward's (computed there from the maps instead).
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np

DEFAULT_EPS = 1e-5


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# lambda
# --------------------------------------------------------------------------
def lambda_init(layer: int) -> float:
    """lambda_init = 0.8 - 0.6 * exp(-0.3 * (l - 1)) for layer index l >= 1.

    [HADA] "Como a atencao diferencial funciona", lambda_init equation.
    Evaluated left to right in float64: t = -0.3 * (l - 1); e = exp(t);
    0.8 - (0.6 * e), each step rounded once.
    """
    if int(layer) != layer or layer < 1:
        raise ValueError("layer index must be an integer >= 1")
    t = -0.3 * float(layer - 1)
    e = math.exp(t)
    return 0.8 - 0.6 * e


def lambda_scalar(lq1, lk1, lq2, lk2, layer: int,
                  fixed_init: Optional[float] = None) -> Dict[str, float]:
    """lambda = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init.

    [HADA] "Como a atencao diferencial funciona", lambda equation; [PRIOR],
    same formula.  One scalar per layer, shared by all heads ([INTOAI]
    "Differential Attention With Multiple Heads").

    The dot products are summed in index order in float64 (each product of
    two float32 values is exact in float64).  The result is returned in float64
    and rounded once to float32 (the value the kernels consume).

    fixed_init None: lambda_init follows the layer schedule; otherwise it is
    fixed_init for every layer (the pages also try one constant lambda_init,
    for example 0.8, in all layers: [HADA], the note after the lambda_init
    equation).
    """
    lq1, lk1, lq2, lk2 = (_f64(v).reshape(-1) for v in (lq1, lk1, lq2, lk2))
    if not (lq1.shape == lk1.shape == lq2.shape == lk2.shape):
        raise ValueError("lambda vectors must have equal length")
    a = 0.0
    for x, y in zip(lq1.tolist(), lk1.tolist()):
        a = a + x * y
    b = 0.0
    for x, y in zip(lq2.tolist(), lk2.tolist()):
        b = b + x * y
    ea = math.exp(a)
    eb = math.exp(b)
    li = lambda_init(layer) if fixed_init is None else float(fixed_init)
    lam = (ea - eb) + li
    return {
        "lambda": lam, "lambda_init": li, "exp_a": ea, "exp_b": eb,
        "lambda_f32": float(np.float32(lam)),
        "lambda_init_f32": float(np.float32(li)),
        "one_minus_init_f32": float(np.float32(1.0 - li)),
    }


def lambda_layers(lq1s, lk1s, lq2s, lk2s, first_layer: int,
                  fixed_init: Optional[float] = None) -> List[Dict[str, float]]:
    """lambda of n consecutive layers: row k of each [n, d] array belongs to
    layer first_layer + k, and each is lambda_scalar of that row ([HADA]: one
    lambda per layer, lambda_init from the layer index or fixed)."""
    rows = [_f64(v) for v in (lq1s, lk1s, lq2s, lk2s)]
    if rows[0].ndim != 2 or any(r.shape != rows[0].shape for r in rows):
        raise ValueError("lambda vectors must be [n_layers, d] of equal shape")
    return [lambda_scalar(rows[0][k], rows[1][k], rows[2][k], rows[3][k], first_layer + k,
                          fixed_init)
            for k in range(rows[0].shape[0])]


# --------------------------------------------------------------------------
# forward
# --------------------------------------------------------------------------
def causal_softmax(scores: np.ndarray, row_offset: int = 0) -> np.ndarray:
    """Row softmax with the causal mask M.

    scores[i, j] is query row (row_offset + i) against key j.  Entries with
    j > row_offset + i are masked ([INTOAI] "A Deeper Dive Into Attention
    Calculations": M is 0 where the query may see the key and -inf otherwise,
    so those probabilities are exactly 0).  Two passes: subtract the row
    maximum, exponentiate, divide by the row sum.
    """
    s = np.array(scores, dtype=np.float64, copy=True)
    n_rows, n_cols = s.shape
    rows = np.arange(n_rows)[:, None] + row_offset
    cols = np.arange(n_cols)[None, :]
    masked = cols > rows
    s[masked] = -np.inf
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    p[masked] = 0.0
    return p / p.sum(axis=1, keepdims=True)


def attention_maps(q1, k1, q2, k2):
    """A_k = causal_softmax(Q_k K_k^T / sqrt(d)) for one head, k = 1, 2.

    [HADA] / [PRIOR] DiffAttn equation; d is the width of Q1 and K1.
    """
    q1, k1, q2, k2 = (_f64(x) for x in (q1, k1, q2, k2))
    d = q1.shape[-1]
    s = 1.0 / math.sqrt(d)
    a1 = causal_softmax(s * (q1 @ k1.T))
    a2 = causal_softmax(s * (q2 @ k2.T))
    return a1, a2


def rms_norm_rows(o: np.ndarray, eps: float = DEFAULT_EPS, weight=None):
    """RMSNorm of each row over its full width: o * (mean(o^2) + eps)^(-1/2) * w.

    Per head, independently ([HADA] "Estrutura multi-head e arquitetura
    completa"; [INTOAI] "Differential Attention With Multiple Heads").
    Returns (normalised rows, rstd per row).
    """
    o = _f64(o)
    rstd = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    y = o * rstd
    if weight is not None:
        y = y * _f64(weight)
    return y, rstd[..., 0]


def head_forward(q1, q2, k1, k2, v, lam: float, lam_init: float,
                 eps: float = DEFAULT_EPS, weight=None, block: int = 1024,
                 want_saved: bool = False):
    """DiffAttn for one head over a causal sequence, then norm and scale.

    O = (A1 - lam * A2) V   ([HADA] / [PRIOR] DiffAttn equation, one product)
    Y = (1 - lam_init) * RMSNorm(O)   ([INTOAI] multi-head section)

    Query rows are processed in blocks of ``block`` rows against their causal
    key range [0, last row of the block].  With ``want_saved`` it also returns
    O1 = A1 V, O2 = A2 V, the log-sum-exp of each map's scaled scores, the
    pre-norm O and rstd (the quantities the backward pass needs).
    """
    q1, q2, k1, k2, v = (_f64(x) for x in (q1, q2, k1, k2, v))
    n, d = q1.shape
    dv = v.shape[-1]
    s = 1.0 / math.sqrt(d)
    o = np.empty((n, dv))
    saved = None
    if want_saved:
        saved = {"o1": np.empty((n, dv)), "o2": np.empty((n, dv)),
                 "lse1": np.empty(n), "lse2": np.empty(n)}
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        kend = r1                     # keys 0 .. r1-1 are the causal range
        s1 = s * (q1[r0:r1] @ k1[:kend].T)
        s2 = s * (q2[r0:r1] @ k2[:kend].T)
        a1 = causal_softmax(s1, row_offset=r0)
        a2 = causal_softmax(s2, row_offset=r0)
        o[r0:r1] = (a1 - lam * a2) @ v[:kend]
        if want_saved:
            saved["o1"][r0:r1] = a1 @ v[:kend]
            saved["o2"][r0:r1] = a2 @ v[:kend]
            for name, sc in (("lse1", s1), ("lse2", s2)):
                rows = np.arange(r1 - r0)[:, None] + r0
                cols = np.arange(kend)[None, :]
                sc = np.where(cols > rows, -np.inf, sc)
                m = sc.max(axis=1)
                saved[name][r0:r1] = m + np.log(np.exp(sc - m[:, None]).sum(axis=1))
    y, rstd = rms_norm_rows(o, eps, weight)
    y = (1.0 - lam_init) * y
    if want_saved:
        saved["o"] = o
        saved["rstd"] = rstd
        return y, saved
    return y


def forward(q1, q2, k1, k2, v, lam: float, lam_init: float, eps: float = DEFAULT_EPS,
            weight=None, block: int = 1024, want_saved: bool = False, heads=None):
    """Batched DiffAttn forward: tensors [B, H, N, d] and V [B, H, N, 2d].

    K1, K2 and V may have Hkv heads dividing H (grouped-query attention, named as
    a further speed-up for DiffAttn in [BOOK] "Implementation and Future
    Prospects"): query head h then uses K/V head h // (H / Hkv), the heads of a
    group being consecutive.
    ``weight`` is the per-channel RMSNorm weight, shape [H, 2d] or None (unit).
    ``heads`` optionally restricts the work to a list of (b, h) pairs; the
    other outputs are left as NaN.
    Returns Y [B, H, N, 2d] (float64), and the saved quantities when asked.
    """
    q1 = np.asarray(q1)
    B, H, N, _ = q1.shape
    dv = np.asarray(v).shape[-1]
    y = np.full((B, H, N, dv), np.nan)
    saved = None
    if want_saved:
        saved = {k: np.full((B, H, N, dv), np.nan) for k in ("o1", "o2", "o")}
        saved.update({k: np.full((B, H, N), np.nan) for k in ("lse1", "lse2", "rstd")})
    g = H // np.asarray(k1).shape[1]     # query heads per K/V head
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    for b, h in pairs:
        w = None if weight is None else np.asarray(weight)[h]
        kh = h // g
        r = head_forward(q1[b, h], q2[b, h], k1[b, kh], k2[b, kh], v[b, kh], lam, lam_init,
                         eps, w, block, want_saved)
        if want_saved:
            y[b, h], sv = r
            for k in saved:
                saved[k][b, h] = sv[k]
        else:
            y[b, h] = r
    return (y, saved) if want_saved else y


def forward_rows(q1, q2, k1, k2, v, rows, lam: float, lam_init: float,
                 eps: float = DEFAULT_EPS, weight=None):
    """DiffAttn output for selected query rows of one head only.

    Row i sees keys 0..i.  Used to check sampled outputs at sizes where the
    full oracle would take too long.  Same definition as ``head_forward``.
    """
    q1, q2, k1, k2, v = (_f64(x) for x in (q1, q2, k1, k2, v))
    d = q1.shape[-1]
    s = 1.0 / math.sqrt(d)
    out = []
    for i in rows:
        i = int(i)
        s1 = s * (k1[: i + 1] @ q1[i])
        s2 = s * (k2[: i + 1] @ q2[i])
        a1 = np.exp(s1 - s1.max())
        a1 /= a1.sum()
        a2 = np.exp(s2 - s2.max())
        a2 /= a2.sum()
        o = (a1 - lam * a2) @ v[: i + 1]
        y, _ = rms_norm_rows(o[None, :], eps, weight)
        out.append((1.0 - lam_init) * y[0])
    return np.stack(out) if out else np.zeros((0, v.shape[-1]))


def decode(q1, q2, k1c, k2c, vc, cache_len, lam: float, lam_init: float,
           eps: float = DEFAULT_EPS, weight=None):
    """One decode step: a single query per (b, h) against its cached keys.

    q1, q2 [B, H, d]; k1c, k2c [B, Hkv, L, d]; vc [B, Hkv, L, 2d] (query head
    h reads cache head h // (H / Hkv), as in ``forward``); cache_len [B] or
    None (= L).  The cache already holds the new token, so the query sits at
    position len - 1 and sees keys 0 .. len - 1 (the causal mask of the
    prefill, last row).  Returns Y [B, H, 2d].
    """
    q1 = np.asarray(q1)
    B, H, d = q1.shape
    L = np.asarray(k1c).shape[2]
    dv = np.asarray(vc).shape[-1]
    s = 1.0 / math.sqrt(d)
    y = np.empty((B, H, dv))
    g = H // np.asarray(k1c).shape[1]
    for b in range(B):
        n = L if cache_len is None else int(cache_len[b])
        for h in range(H):
            kh = h // g
            s1 = s * (_f64(k1c[b, kh, :n]) @ _f64(q1[b, h]))
            s2 = s * (_f64(k2c[b, kh, :n]) @ _f64(q2[b, h]))
            a1 = np.exp(s1 - s1.max())
            a1 /= a1.sum()
            a2 = np.exp(s2 - s2.max())
            a2 /= a2.sum()
            o = (a1 - lam * a2) @ _f64(vc[b, kh, :n])
            w = None if weight is None else np.asarray(weight)[h]
            yy, _ = rms_norm_rows(o[None, :], eps, w)
            y[b, h] = (1.0 - lam_init) * yy[0]
    return y


def cache_append(k1_new, k2_new, v_new, k1c, k2c, vc, cache_len):
    """One generated token appended to each sequence's cache: the write half of an
    autoregressive serving step, before the decode that reads the cache whole ([MLA],
    "The Memory Wall: Why the KV Cache Constrains LLM Serving": the cache grows by one
    token per generated token).

    For sequence b with n = max(cache_len[b], 0) < L, row n of every head receives
    k1_new[b, h], k2_new[b, h], v_new[b, h] and the length becomes n + 1; a full cache
    (n >= L) is left as it is.  Returns new arrays (k1c, k2c, vc, cache_len); the
    caches keep their dtype (the copy is exact).
    """
    k1c, k2c, vc = np.array(k1c), np.array(k2c), np.array(vc)
    lens = np.array(cache_len, dtype=np.int64)
    L = k1c.shape[2]
    for b in range(k1c.shape[0]):
        n = max(int(lens[b]), 0)
        if n >= L:
            continue
        k1c[b, :, n] = k1_new[b]
        k2c[b, :, n] = k2_new[b]
        vc[b, :, n] = v_new[b]
        lens[b] = n + 1
    return k1c, k2c, vc, lens


# --------------------------------------------------------------------------
# projections
# --------------------------------------------------------------------------
def qkv_proj(x, w_qkv, heads: int, head_dim: int, kv_heads=None):
    """The input projections: X times W_Q, W_K, W_V ([INTOAI] "Moving On To The
    Differential Transformer": Q and K are each split into two groups; "Differential
    Attention With Multiple Heads": two queries, two keys and a value per head).

    x [B, N, d_model]; w_qkv [(H + 2 Hkv) 2d, d_model] in the [out_features,
    in_features] layout, rows W_Q (H 2d), then W_K and W_V (Hkv 2d each; Hkv =
    kv_heads, default H: grouped-query attention when smaller). Reading (the
    pages fix no column order): row h 2d + j d + c of W_Q gives channel c of
    Q_(j+1) in head h, likewise for W_K, and row h 2d + c of W_V gives channel c
    of V in head h.
    Returns q1, q2 [B, H, N, d], k1, k2 [B, Hkv, N, d] and v [B, Hkv, N, 2d], in
    float64.
    """
    x, w = _f64(x), _f64(w_qkv)
    B, N, dm = x.shape
    H, d = heads, head_dim
    Hkv = H if kv_heads is None else kv_heads
    if w.shape != (2 * d * (H + 2 * Hkv), dm):
        raise ValueError("w_qkv must be [(H + 2 Hkv) 2d, d_model]")
    y = x @ w.T                                   # [B, N, (H + 2 Hkv) 2d]
    hd2, kd2 = 2 * H * d, 2 * Hkv * d
    q = y[..., :hd2].reshape(B, N, H, 2, d)
    k = y[..., hd2:hd2 + kd2].reshape(B, N, Hkv, 2, d)
    v = y[..., hd2 + kd2:].reshape(B, N, Hkv, 2 * d)
    per_head = lambda t: np.ascontiguousarray(t.transpose(0, 2, 1, 3))   # [B, H, N, *]
    return (per_head(q[..., 0, :]), per_head(q[..., 1, :]), per_head(k[..., 0, :]),
            per_head(k[..., 1, :]), per_head(v))


def out_proj(attn, w_o):
    """The output projection: the heads' outputs concatenated along channels, times
    W_O ([INTOAI] "Differential Attention With Multiple Heads"; [HADA] "Estrutura
    multi-head e arquitetura completa"). attn [B, N, H, 2d] (token-major, head h at
    channels h 2d .. h 2d + 2d - 1 of the concatenation); w_o [d_model, H 2d].
    Returns [B, N, d_model] in float64."""
    a = _f64(attn)
    B, N, H, d2 = a.shape
    return a.reshape(B, N, H * d2) @ _f64(w_o).T


# --------------------------------------------------------------------------
# backward (derived by the chain rule; the pages print no gradient formulas)
# --------------------------------------------------------------------------
def head_backward(q1, q2, k1, k2, v, dy, lam: float, lam_init: float,
                  eps: float = DEFAULT_EPS, weight=None):
    """Gradients of sum(Y * dY) for one head, with full N x N maps.

    Forward: A_k = causal_softmax(s Q_k K_k^T), O = (A1 - lam A2) V,
    Y = (1 - lam_init) * w * O * r with r = (mean(O^2) + eps)^(-1/2).

    Chain rule, with g = (1 - lam_init) * w * dY and n = width of O:
      G  = dL/dO = r * g - O * r^3 * rowsum(g * O) / n
      dV = (A1 - lam A2)^T G
      dA1 = G V^T,   dA2 = -lam G V^T
      dS_k = A_k * (dA_k - rowsum(A_k * dA_k))      (softmax Jacobian)
      dQ_k = s dS_k K_k,   dK_k = s dS_k^T Q_k
      dlam = -sum(A2 * (G V^T)) = -sum_i rowsum(G * O2)
      dw = (1 - lam_init) * sum over rows of dY * O * r   (the RMSNorm weight)
    Returns a dict with dq1, dq2, dk1, dk2, dv, d_attn (= G), dw and dlam.
    """
    q1, q2, k1, k2, v, dy = (_f64(x) for x in (q1, q2, k1, k2, v, dy))
    n, d = q1.shape
    dv_w = v.shape[-1]
    s = 1.0 / math.sqrt(d)
    a1, a2 = attention_maps(q1, k1, q2, k2)
    o = (a1 - lam * a2) @ v
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    w = np.ones(dv_w) if weight is None else _f64(weight)
    g = (1.0 - lam_init) * w * dy
    G = r * g - o * r ** 3 * np.sum(g * o, axis=-1, keepdims=True) / dv_w
    dv = (a1 - lam * a2).T @ G
    gv = G @ v.T
    da1 = gv
    da2 = -lam * gv
    ds1 = a1 * (da1 - np.sum(a1 * da1, axis=-1, keepdims=True))
    ds2 = a2 * (da2 - np.sum(a2 * da2, axis=-1, keepdims=True))
    return {
        "dq1": s * ds1 @ k1, "dk1": s * ds1.T @ q1,
        "dq2": s * ds2 @ k2, "dk2": s * ds2.T @ q2,
        "dv": dv, "d_attn": G, "dlam": float(-np.sum(a2 * gv)),
        "dw": (1.0 - lam_init) * np.sum(dy * o * r, axis=0),
    }


def epilogue_backward(o1, o2, dy, lam: float, lam_init: float, eps: float = DEFAULT_EPS,
                      weight=None):
    """Backward of the epilogue alone, rows of one head: the gradient at the RMSNorm input
    and the per-row terms the lambda and attention gradients use, from the two maps'
    outputs O1 = A1 V and O2 = A2 V and the upstream gradient dY.

    Forward of the epilogue ([HADA] DiffAttn equation, [INTOAI] "Differential Attention
    With Multiple Heads"): O = O1 - lam O2, r = (mean(O^2) + eps)^(-1/2),
    Y = (1 - lam_init) w O r.  Chain rule, with g = (1 - lam_init) w dY and n the width
    of O:
      G  = dL/dO = r g - O r^3 rowsum(g O) / n
      D1 = rowsum(G O1),  D2 = rowsum(G O2)
      dlam = -sum_i D2_i              (lam enters O only as -lam O2)
      dw = (1 - lam_init) sum over rows of dY O r
    Returns a dict with G, D1, D2 (per row), dlam and dw.
    """
    o1, o2, dy = _f64(o1), _f64(o2), _f64(dy)
    n = o1.shape[-1]
    o = o1 - lam * o2
    r = 1.0 / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)
    w = np.ones(n) if weight is None else _f64(weight)
    g = (1.0 - lam_init) * w * dy
    G = r * g - (r ** 3 / n) * o * np.sum(g * o, axis=-1, keepdims=True)
    d1 = np.sum(G * o1, axis=-1)
    d2 = np.sum(G * o2, axis=-1)
    return {"G": G, "D1": d1, "D2": d2, "dlam": float(-np.sum(d2)),
            "dw": (1.0 - lam_init) * np.sum(r * o * dy, axis=0)}


def backward(q1, q2, k1, k2, v, dy, lq1, lk1, lq2, lk2, layer: int,
             eps: float = DEFAULT_EPS, weight=None, heads=None):
    """Batched backward for tensors [B, H, N, *] and the four lambda vectors.

    dlam sums over every (b, h) (lambda is one scalar per layer).  The lambda
    vector gradients follow from lambda = exp(lq1.lk1) - exp(lq2.lk2) + init:
      dlq1 = dlam e^a lk1, dlk1 = dlam e^a lq1,
      dlq2 = -dlam e^b lk2, dlk2 = -dlam e^b lq2.
    lambda_init is a constant of the layer index and receives no gradient.
    d_rms_weight [H, 2d] sums each head's dw over the batch (the weight is one
    per head and channel).
    With grouped-query attention (K1, K2, V with Hkv < H heads, query head h
    reading K/V head h // (H / Hkv)) dk1, dk2 and dv of a K/V head sum the
    contributions of the query heads of its group.
    ``heads`` restricts the per-head tensors to the listed (b, h) pairs (the
    others stay NaN); dlam and the vector gradients then cover only those.
    """
    st = lambda_scalar(lq1, lk1, lq2, lk2, layer)
    lam, li = st["lambda"], st["lambda_init"]
    q1 = np.asarray(q1)
    B, H, N, d = q1.shape
    Hkv = np.asarray(k1).shape[1]
    g = H // Hkv
    dvw = np.asarray(v).shape[-1]
    out = {k: np.full((B, H, N, d), np.nan) for k in ("dq1", "dq2")}
    out.update({k: np.full((B, Hkv, N, d), np.nan) for k in ("dk1", "dk2")})
    out["dv"] = np.full((B, Hkv, N, dvw), np.nan)
    out["d_attn"] = np.full((B, H, N, dvw), np.nan)
    out["d_rms_weight"] = np.zeros((H, dvw))
    dlam = 0.0
    pairs = heads if heads is not None else [(b, h) for b in range(B) for h in range(H)]
    seen = set()       # K/V heads that already hold a contribution
    for b, h in pairs:
        w = None if weight is None else np.asarray(weight)[h]
        kh = h // g
        r = head_backward(q1[b, h], q2[b, h], k1[b, kh], k2[b, kh], v[b, kh], dy[b, h],
                          lam, li, eps, w)
        for k in ("dq1", "dq2", "d_attn"):
            out[k][b, h] = r[k]
        for k in ("dk1", "dk2", "dv"):
            if (b, kh) in seen:
                out[k][b, kh] = out[k][b, kh] + r[k]
            else:
                out[k][b, kh] = r[k]
        seen.add((b, kh))
        out["d_rms_weight"][h] += r["dw"]
        dlam += r["dlam"]
    lq1, lk1, lq2, lk2 = (_f64(x) for x in (lq1, lk1, lq2, lk2))
    out["dlam"] = dlam
    out["dlq1"] = dlam * st["exp_a"] * lk1
    out["dlk1"] = dlam * st["exp_a"] * lq1
    out["dlq2"] = -dlam * st["exp_b"] * lk2
    out["dlk2"] = -dlam * st["exp_b"] * lq2
    return out
