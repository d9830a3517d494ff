"""Pins of the float64 oracle against what the pages and mathematics fix.

None of these tests compares the oracle with itself.  Each check is chosen so
that a plausible mistake in the oracle (a dropped term, a wrong sign, a wrong
index or scale, a transposed operand) fails at least one of them; the last
test plants such mistakes in copies of the oracle and confirms that.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import diffattn_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


def rand(r, *shape, scale=1.0):
    return r.standard_normal(shape) * scale


def sdpa_causal(q, k, v):
    """torch's float64 CPU causal attention (scale 1/sqrt(q width))."""
    t = [torch.from_numpy(np.ascontiguousarray(x)).double() for x in (q, k, v)]
    return torch.nn.functional.scaled_dot_product_attention(
        t[0], t[1], t[2], is_causal=True).numpy()


# ---------------------------------------------------------------- lambda
def test_lambda_init_against_page_endpoints():
    g = json.load(open(os.path.join(GOLDEN, "lambda_init_endpoints.json")))
    assert abs(orc.lambda_init(1) - g["layer_1"]) < 1e-15
    assert abs(orc.lambda_init(200) - g["limit_deep_layers"]) < 1e-15
    vals = [orc.lambda_init(l) for l in range(1, 60)]
    assert all(b > a for a, b in zip(vals, vals[1:]))            # lower in early layers
    decay = math.exp(-0.3)
    for l in range(1, 40):                                        # gap to 0.8 shrinks by e^-0.3
        gap0 = g["limit_deep_layers"] - orc.lambda_init(l)
        gap1 = g["limit_deep_layers"] - orc.lambda_init(l + 1)
        assert abs(gap1 - decay * gap0) < 1e-15
    with pytest.raises(ValueError):
        orc.lambda_init(0)


def test_lambda_zero_vectors_is_lambda_init():
    z = np.zeros(16, np.float32)
    for l in (1, 4, 6, 8, 12):
        st = orc.lambda_scalar(z, z, z, z, l)
        assert st["lambda"] == orc.lambda_init(l)     # e^0 - e^0 = 0 exactly
        assert st["exp_a"] == 1.0 and st["exp_b"] == 1.0


def test_lambda_closed_form_logs():
    # lq1 . lk1 = ln 3 and lq2 . lk2 = ln 2 give lambda = 3 - 2 + lambda_init
    lq1 = np.zeros(8); lk1 = np.zeros(8); lq2 = np.zeros(8); lk2 = np.zeros(8)
    lq1[3] = 1.0; lk1[3] = math.log(3.0)
    lq2[5] = math.log(2.0); lk2[5] = 1.0
    st = orc.lambda_scalar(lq1, lk1, lq2, lk2, 1)
    assert abs(st["lambda"] - (1.0 + 0.2)) < 1e-14
    assert abs(st["exp_a"] - 3.0) < 1e-14 and abs(st["exp_b"] - 2.0) < 1e-14
    # the second pair enters with a minus sign and the first with a plus
    st2 = orc.lambda_scalar(lq2, lk2, lq1, lk1, 1)
    assert abs(st2["lambda"] - (-1.0 + 0.2)) < 1e-14
    # only the dot product matters: spreading it over indices changes nothing
    a = np.array([0.5, 0.25, -0.125, 0.0]); b = np.array([1.0, 2.0, 4.0, 3.0])
    st3 = orc.lambda_scalar(a, b, np.zeros(4), np.zeros(4), 2)
    assert abs(st3["exp_a"] - math.exp(0.5)) < 1e-15


def test_lambda_f32_rounding_once():
    r = rng(3)
    v = [rand(r, 64, scale=0.1).astype(np.float32) for _ in range(4)]
    st = orc.lambda_scalar(*v, 12)
    assert st["lambda_f32"] == float(np.float32(st["lambda"]))
    assert st["one_minus_init_f32"] == float(np.float32(1.0 - st["lambda_init"]))


# ---------------------------------------------------------------- forward
def test_rmsnorm_matches_torch():
    r = rng(1)
    x = rand(r, 7, 32)
    w = rand(r, 32)
    y, rstd = orc.rms_norm_rows(x, 1e-5, w)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (32,), torch.from_numpy(w), 1e-5)
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-13, atol=1e-14)
    # eps is added inside the root: a zero row stays zero and rstd = eps^-1/2
    y0, r0 = orc.rms_norm_rows(np.zeros((1, 8)), 1e-5)
    assert np.all(y0 == 0) and abs(r0[0] - 1e-5 ** -0.5) < 1e-9


@pytest.mark.parametrize("n,d", [(1, 4), (13, 8), (64, 16), (97, 32)])
def test_lambda_zero_is_causal_softmax_attention(n, d):
    r = rng(n * 100 + d)
    q1, k1, q2, k2 = (rand(r, 1, 1, n, d) for _ in range(4))
    v = rand(r, 1, 1, n, 2 * d)
    y, sv = orc.forward(q1, q2, k1, k2, v, 0.0, 0.3, want_saved=True, block=16)
    ref = sdpa_causal(q1, k1, v)
    np.testing.assert_allclose(sv["o"], ref, rtol=1e-12, atol=1e-13)
    yref = 0.7 * torch.nn.functional.rms_norm(torch.from_numpy(ref), (2 * d,), eps=1e-5).numpy()
    np.testing.assert_allclose(y, yref, rtol=1e-12, atol=1e-13)
    # the second map's own output is softmax attention of (Q2, K2)
    np.testing.assert_allclose(sv["o2"], sdpa_causal(q2, k2, v), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("lam", [0.2, 0.55, -0.3, 1.7])
def test_identical_maps_scale_softmax_attention(lam):
    r = rng(7)
    n, d = 50, 16
    q = rand(r, 1, 2, n, d)
    k = rand(r, 1, 2, n, d)
    v = rand(r, 1, 2, n, 2 * d)
    _, sv = orc.forward(q, q, k, k, v, lam, 0.5, want_saved=True, block=17)
    np.testing.assert_allclose(sv["o"], (1.0 - lam) * sdpa_causal(q, k, v), rtol=1e-11, atol=1e-12)


def test_identical_maps_lambda_one_is_zero():
    r = rng(8)
    q = rand(r, 2, 3, 33, 8); k = rand(r, 2, 3, 33, 8); v = rand(r, 2, 3, 33, 16)
    y = orc.forward(q, q, k, k, v, 1.0, 0.2)
    assert np.all(y == 0.0)


def test_rows_sum_to_one():
    r = rng(9)
    n, d = 40, 8
    q1, k1, q2, k2 = (rand(r, n, d) for _ in range(4))
    a1, a2 = orc.attention_maps(q1, k1, q2, k2)
    np.testing.assert_allclose(a1.sum(1), 1.0, atol=1e-14)
    np.testing.assert_allclose(a2.sum(1), 1.0, atol=1e-14)
    assert np.all(np.triu(a1, 1) == 0) and np.all(np.triu(a2, 1) == 0)
    # V = ones: every row of (A1 - lam A2) V equals 1 - lam
    lam = 0.37
    _, sv = orc.forward(q1[None, None], q2[None, None], k1[None, None], k2[None, None],
                        np.ones((1, 1, n, 2 * d)), lam, 0.1, want_saved=True)
    np.testing.assert_allclose(sv["o"], 1.0 - lam, atol=1e-14)


def test_row_zero_attends_only_to_v0():
    r = rng(10)
    n, d = 24, 16
    q1, k1, q2, k2 = (rand(r, 1, 1, n, d) for _ in range(4))
    v = rand(r, 1, 1, n, 2 * d)
    lam, li, eps = 0.61, 0.556, 1e-5
    y, sv = orc.forward(q1, q2, k1, k2, v, lam, li, eps=eps, want_saved=True)
    v0 = v[0, 0, 0]
    np.testing.assert_allclose(sv["o"][0, 0, 0], (1 - lam) * v0, rtol=1e-14)
    yexp = (1 - li) * (1 - lam) * v0 / math.sqrt((1 - lam) ** 2 * np.mean(v0 ** 2) + eps)
    np.testing.assert_allclose(y[0, 0, 0], yexp, rtol=1e-13)


def test_mask_perturbation_invariance():
    r = rng(11)
    n, d = 70, 16
    q1, q2, k1, k2 = (rand(r, 1, 1, n, d) for _ in range(4))
    v = rand(r, 1, 1, n, 2 * d)
    y0 = orc.forward(q1, q2, k1, k2, v, 0.4, 0.2, block=32)
    i0 = 41
    k1p, k2p, vp = k1.copy(), k2.copy(), v.copy()
    k1p[..., i0 + 1:, :] += 5.0
    k2p[..., i0 + 1:, :] -= 3.0
    vp[..., i0 + 1:, :] *= -7.0
    y1 = orc.forward(q1, q2, k1p, k2p, vp, 0.4, 0.2, block=32)
    assert np.array_equal(y0[..., : i0 + 1, :], y1[..., : i0 + 1, :])
    assert not np.allclose(y0[..., i0 + 1:, :], y1[..., i0 + 1:, :])


def brute_force(q1, q2, k1, k2, v, lam, li, eps):
    """Scalar loops over every element (one head)."""
    n, d = len(q1), len(q1[0])
    dv = len(v[0])
    s = 1.0 / math.sqrt(d)
    out = []
    for i in range(n):
        maps = []
        for q, k in ((q1, k1), (q2, k2)):
            sc = []
            for j in range(i + 1):
                acc = 0.0
                for t in range(d):
                    acc += q[i][t] * k[j][t]
                sc.append(acc * s)
            mx = max(sc)
            e = [math.exp(x - mx) for x in sc]
            tot = sum(e)
            maps.append([x / tot for x in e])
        o = []
        for c in range(dv):
            acc = 0.0
            for j in range(i + 1):
                acc += (maps[0][j] - lam * maps[1][j]) * v[j][c]
            o.append(acc)
        ms = sum(x * x for x in o) / dv
        rs = 1.0 / math.sqrt(ms + eps)
        out.append([(1.0 - li) * x * rs for x in o])
    return out


@pytest.mark.parametrize("n,d,lam", [(1, 2, 0.5), (5, 4, 0.2), (16, 8, 0.83), (11, 3, -0.4)])
def test_brute_force_twin(n, d, lam):
    r = rng(n + 31 * d)
    q1, q2, k1, k2 = (rand(r, n, d) for _ in range(4))
    v = rand(r, n, 2 * d)
    li = 0.666
    bf = np.array(brute_force(q1.tolist(), q2.tolist(), k1.tolist(), k2.tolist(), v.tolist(),
                              lam, li, 1e-5))
    y = orc.forward(q1[None, None], q2[None, None], k1[None, None], k2[None, None],
                    v[None, None], lam, li, block=4)[0, 0]
    np.testing.assert_allclose(y, bf, rtol=1e-12, atol=1e-12)
    rows = list(range(n))
    np.testing.assert_allclose(orc.forward_rows(q1, q2, k1, k2, v, rows, lam, li), bf,
                               rtol=1e-12, atol=1e-12)


def test_decode_equals_last_prefill_row():
    r = rng(12)
    B, H, L, d = 3, 2, 37, 16
    q1, q2, k1, k2 = (rand(r, B, H, L, d) for _ in range(4))
    v = rand(r, B, H, L, 2 * d)
    lam, li = 0.45, 0.72
    y = orc.forward(q1, q2, k1, k2, v, lam, li)
    lens = np.array([L, 1, 20])
    qd1 = np.stack([q1[b, :, lens[b] - 1] for b in range(B)])
    qd2 = np.stack([q2[b, :, lens[b] - 1] for b in range(B)])
    yd = orc.decode(qd1, qd2, k1, k2, v, lens, lam, li)
    for b in range(B):
        np.testing.assert_allclose(yd[b], y[b, :, lens[b] - 1], rtol=1e-12, atol=1e-13)
    yfull = orc.decode(q1[:, :, -1], q2[:, :, -1], k1, k2, v, None, lam, li)
    np.testing.assert_allclose(yfull, y[:, :, -1], rtol=1e-12, atol=1e-13)


def test_cache_append_then_decode_equals_prefill_row():
    """Appending token n to caches that hold tokens 0 .. n-1 (arbitrary values beyond)
    and decoding gives row n of the prefill over the extended sequence; a full cache and
    its length stay as they are, and a negative length counts as 0."""
    r = rng(21)
    B, H, L, d = 4, 2, 19, 8
    q1, q2, k1, k2 = (rand(r, B, H, L, d) for _ in range(4))
    v = rand(r, B, H, L, 2 * d)
    lam, li = 0.31, 0.6
    y = orc.forward(q1, q2, k1, k2, v, lam, li)
    lens = np.array([5, 0, L, -3])
    pos = np.array([5, 0, L - 1, 0])          # row each new token belongs to
    tok = lambda a: np.stack([a[b, :, pos[b]] for b in range(B)])
    junk = [rand(r, B, H, L, d), rand(r, B, H, L, d), rand(r, B, H, L, 2 * d)]
    caches = []
    for a, jk in zip((k1, k2, v), junk):
        c = jk.copy()
        for b in range(B):
            c[b, :, :max(lens[b], 0)] = a[b, :, :max(lens[b], 0)]
        caches.append(c)
    c1, c2, cv, nl = orc.cache_append(tok(k1), tok(k2), tok(v), *caches, lens)
    assert list(nl) == [6, 1, L, 1]
    np.testing.assert_array_equal(c1[2], caches[0][2])     # full: untouched
    yd = orc.decode(tok(q1), tok(q2), c1, c2, cv, nl, lam, li)
    for b in (0, 1, 3):
        np.testing.assert_allclose(yd[b], y[b, :, pos[b]], rtol=1e-12, atol=1e-13)


def test_saved_lse_is_log_normaliser():
    r = rng(13)
    n, d = 30, 8
    q1, q2, k1, k2 = (rand(r, n, d) for _ in range(4))
    v = rand(r, n, 2 * d)
    _, sv = orc.head_forward(q1, q2, k1, k2, v, 0.3, 0.2, want_saved=True, block=7)
    s = 1.0 / math.sqrt(d)
    for i in (0, 5, 29):
        ref = np.log(np.sum(np.exp(s * (k1[: i + 1] @ q1[i]))))
        assert abs(sv["lse1"][i] - ref) < 1e-12
    np.testing.assert_allclose(sv["o1"] - 0.3 * sv["o2"], sv["o"], atol=1e-13)


# ---------------------------------------------------------------- backward
def _loss(p, dy, layer, eps, weight):
    st = orc.lambda_scalar(p["lq1"], p["lk1"], p["lq2"], p["lk2"], layer)
    y = orc.forward(p["q1"], p["q2"], p["k1"], p["k2"], p["v"], st["lambda"],
                    st["lambda_init"], eps=eps, weight=weight)
    return float(np.sum(y * dy))


def _fd_check(n, d, B, H, layer, n_samples, seed, weight_on):
    r = rng(seed)
    p = {k: rand(r, B, H, n, d) for k in ("q1", "q2", "k1", "k2")}
    p["v"] = rand(r, B, H, n, 2 * d)
    for k in ("lq1", "lk1", "lq2", "lk2"):
        p[k] = rand(r, d, scale=0.1)
    dy = rand(r, B, H, n, 2 * d)
    weight = (1.0 + 0.3 * rand(r, H, 2 * d)) if weight_on else None
    eps = 1e-5
    g = orc.backward(p["q1"], p["q2"], p["k1"], p["k2"], p["v"], dy, p["lq1"], p["lk1"],
                     p["lq2"], p["lk2"], layer, eps=eps, weight=weight)
    h = 1e-6
    for name, gname in (("q1", "dq1"), ("q2", "dq2"), ("k1", "dk1"), ("k2", "dk2"),
                        ("v", "dv"), ("lq1", "dlq1"), ("lk1", "dlk1"), ("lq2", "dlq2"),
                        ("lk2", "dlk2")):
        x = p[name]
        flat = x.reshape(-1)
        idx = np.arange(flat.size) if flat.size <= n_samples else \
            r.choice(flat.size, n_samples, replace=False)
        fd = np.empty(len(idx))
        for t, i in enumerate(idx):
            old = flat[i]
            flat[i] = old + h
            lp = _loss(p, dy, layer, eps, weight)
            flat[i] = old - h
            lm = _loss(p, dy, layer, eps, weight)
            flat[i] = old
            fd[t] = (lp - lm) / (2 * h)
        an = g[gname].reshape(-1)[idx]
        scale = max(np.max(np.abs(an)), 1e-12)
        assert np.max(np.abs(an - fd)) / scale < 2e-6, name
    # the RMSNorm weight (one per head and channel), perturbed entry by entry
    if weight is not None:
        flat = weight.reshape(-1)
        idx = np.arange(flat.size) if flat.size <= n_samples else \
            r.choice(flat.size, n_samples, replace=False)
        fd = np.empty(len(idx))
        for t, i in enumerate(idx):
            old = flat[i]
            flat[i] = old + h
            lp = _loss(p, dy, layer, eps, weight)
            flat[i] = old - h
            lm = _loss(p, dy, layer, eps, weight)
            flat[i] = old
            fd[t] = (lp - lm) / (2 * h)
        an = g["d_rms_weight"].reshape(-1)[idx]
        assert np.max(np.abs(an - fd)) / max(np.max(np.abs(an)), 1e-12) < 2e-6, "weight"
    # gradient at the RMSNorm input: perturb O directly through the norm
    st = orc.lambda_scalar(p["lq1"], p["lk1"], p["lq2"], p["lk2"], layer)
    _, sv = orc.forward(p["q1"], p["q2"], p["k1"], p["k2"], p["v"], st["lambda"],
                        st["lambda_init"], eps=eps, weight=weight, want_saved=True)
    o = sv["o"]
    for (b, hh, i) in [(0, 0, 0), (B - 1, H - 1, n - 1), (0, H - 1, n // 2)]:
        w = None if weight is None else weight[hh]
        def f(row):
            y, _ = orc.rms_norm_rows(row[None], eps, w)
            return float(np.sum((1 - st["lambda_init"]) * y[0] * dy[b, hh, i]))
        row = o[b, hh, i].copy()
        fd = np.empty_like(row)
        for c in range(row.size):
            rp = row.copy(); rp[c] += h
            rm = row.copy(); rm[c] -= h
            fd[c] = (f(rp) - f(rm)) / (2 * h)
        np.testing.assert_allclose(g["d_attn"][b, hh, i], fd, rtol=2e-6,
                                   atol=2e-6 * np.max(np.abs(fd)))
    # dlam = -sum over (b, h, i) of rowsum(G * O2)
    assert abs(g["dlam"] + np.sum(g["d_attn"] * sv["o2"])) < 1e-9 * max(1, abs(g["dlam"]))


def test_backward_finite_differences_grouped():
    """Grouped-query attention: 4 query heads share 2 K/V heads, so dK and dV of a shared
    head collect both query heads' contributions; central differences of the grouped
    forward check every gradient entry."""
    r = rng(23)
    B, H, Hk, n, d = 1, 4, 2, 6, 4
    p = {k: rand(r, B, H, n, d) for k in ("q1", "q2")}
    p.update({k: rand(r, B, Hk, n, d) for k in ("k1", "k2")})
    p["v"] = rand(r, B, Hk, n, 2 * d)
    for k in ("lq1", "lk1", "lq2", "lk2"):
        p[k] = rand(r, d, scale=0.1)
    dy = rand(r, B, H, n, 2 * d)
    g = orc.backward(p["q1"], p["q2"], p["k1"], p["k2"], p["v"], dy, p["lq1"], p["lk1"],
                     p["lq2"], p["lk2"], 3)
    h = 1e-6
    for name in ("q1", "k1", "k2", "v", "lq2"):
        flat = p[name].reshape(-1)
        fd = np.empty(flat.size)
        for j in range(flat.size):
            old = flat[j]
            flat[j] = old + h
            lp = _loss(p, dy, 3, 1e-5, None)
            flat[j] = old - h
            lm = _loss(p, dy, 3, 1e-5, None)
            flat[j] = old
            fd[j] = (lp - lm) / (2 * h)
        an = g["d" + name].reshape(-1)
        assert np.max(np.abs(an - fd)) / max(np.max(np.abs(an)), 1e-12) < 2e-6, name


def test_backward_finite_differences_small_full():
    _fd_check(n=9, d=4, B=1, H=2, layer=3, n_samples=10 ** 9, seed=21, weight_on=True)


def test_backward_finite_differences_one_head_n32():
    # one head, N = 32, d = 64: the shape of a single head of the training workload
    _fd_check(n=32, d=64, B=1, H=1, layer=6, n_samples=96, seed=22, weight_on=False)


def _epilogue_fd_failures(m, r):
    """Central differences of the epilogue's loss sum((1 - lam_init) RMSNorm(O1 - lam O2)
    * dY), with the norm taken from torch (independent of the oracle), against
    m.epilogue_backward: G = dL/dO1, dlam with O1 and O2 held fixed, D1_i as the
    derivative in the scale of row i of O1, and the weight gradient. Also its dlam
    against the full backward's (formed there from the maps as -sum A2 (G V^T)).
    Returns the names of the checks that fail."""
    fails = []
    n, d2 = 6, 8
    o1, o2, dy = rand(r, n, d2), rand(r, n, d2), rand(r, n, d2)
    o2[2] *= 1e-3              # a row whose norm is closer to eps
    w = 1.0 + 0.3 * rand(r, d2)
    lam, li, eps = 0.45, 0.3, 1e-5
    e = m.epilogue_backward(o1, o2, dy, lam, li, eps, w)

    def loss(a1, a2, lm, wt):
        t = torch.from_numpy(np.ascontiguousarray(a1 - lm * a2))
        y = torch.nn.functional.rms_norm(t, (d2,), weight=torch.from_numpy(wt), eps=eps)
        return float(np.sum((1.0 - li) * y.numpy() * dy))
    h = 1e-6
    fd = np.empty((n, d2))
    for i in range(n):
        for c in range(d2):
            p_, q_ = o1.copy(), o1.copy()
            p_[i, c] += h; q_[i, c] -= h
            fd[i, c] = (loss(p_, o2, lam, w) - loss(q_, o2, lam, w)) / (2 * h)
    if np.max(np.abs(e["G"] - fd)) > 1e-6 * np.max(np.abs(fd)):
        fails.append("epilogue G")
    fdl = (loss(o1, o2, lam + h, w) - loss(o1, o2, lam - h, w)) / (2 * h)
    if abs(e["dlam"] - fdl) > 1e-6 * max(abs(fdl), 1e-9):
        fails.append("epilogue dlam")
    fd1 = np.empty(n)
    for i in range(n):
        p_, q_ = o1.copy(), o1.copy()
        p_[i] *= 1 + h; q_[i] *= 1 - h
        fd1[i] = (loss(p_, o2, lam, w) - loss(q_, o2, lam, w)) / (2 * h)
    if np.max(np.abs(e["D1"] - fd1)) > 1e-6 * np.max(np.abs(fd1)):
        fails.append("epilogue D1")
    fdw = np.empty(d2)
    for c in range(d2):
        p_, q_ = w.copy(), w.copy()
        p_[c] += h; q_[c] -= h
        fdw[c] = (loss(o1, o2, lam, p_) - loss(o1, o2, lam, q_)) / (2 * h)
    if np.max(np.abs(e["dw"] - fdw)) > 1e-6 * np.max(np.abs(fdw)):
        fails.append("epilogue dw")
    # the same dlam as the full backward, which forms it from the maps
    nn_, d = 9, 4
    q1, q2, k1, k2 = (rand(r, nn_, d) for _ in range(4))
    v, dyy = rand(r, nn_, 2 * d), rand(r, nn_, 2 * d)
    _, sv = m.head_forward(q1, q2, k1, k2, v, lam, li, want_saved=True)
    full = m.head_backward(q1, q2, k1, k2, v, dyy, lam, li)
    ep = m.epilogue_backward(sv["o1"], sv["o2"], dyy, lam, li)
    if abs(ep["dlam"] - full["dlam"]) > 1e-10 * max(abs(full["dlam"]), 1e-9):
        fails.append("epilogue dlam vs full backward")
    return fails


def test_epilogue_backward_pins():
    assert _epilogue_fd_failures(orc, rng(31)) == []


# ---------------------------------------------------------------- planted mistakes
def test_pins_catch_planted_mistakes(monkeypatch):
    """Copies of the oracle with one planted mistake each fail a pin above."""
    r = rng(40)
    n, d = 20, 8
    q1, q2, k1, k2 = (rand(r, 1, 1, n, d) for _ in range(4))
    v = rand(r, 1, 1, n, 2 * d)
    ref = sdpa_causal(q1, k1, v)

    def pins_hold():
        _, sv = orc.forward(q1, q2, k1, k2, v, 0.0, 0.3, want_saved=True)
        ok = np.allclose(sv["o"], ref, rtol=1e-10, atol=1e-11)
        _, sv2 = orc.forward(q1, q1, k1, k1, v, 0.4, 0.3, want_saved=True)
        ok &= np.allclose(sv2["o"], 0.6 * ref, rtol=1e-10, atol=1e-11)
        return bool(ok)

    assert pins_hold()
    good_softmax = orc.causal_softmax

    # 1. mask dropped
    monkeypatch.setattr(orc, "causal_softmax",
                        lambda s, row_offset=0: np.exp(s - s.max(1, keepdims=True)) /
                        np.exp(s - s.max(1, keepdims=True)).sum(1, keepdims=True))
    assert not pins_hold()
    monkeypatch.setattr(orc, "causal_softmax", good_softmax)
    # 2. mask off by one (query may not see itself)
    def shifted(s, row_offset=0):
        return good_softmax(s[:, :], row_offset=row_offset - 1) if s.shape[0] > 1 else good_softmax(s)
    monkeypatch.setattr(orc, "causal_softmax", shifted)
    assert not pins_hold()
    monkeypatch.setattr(orc, "causal_softmax", good_softmax)
    # 3. scale by 1/sqrt(2d) instead of 1/sqrt(d)
    good_sqrt = orc.math.sqrt
    monkeypatch.setattr(orc.math, "sqrt", lambda x: good_sqrt(2 * x))
    assert not pins_hold()
    monkeypatch.setattr(orc.math, "sqrt", good_sqrt)
    assert pins_hold()


# ---------------------------------------------------------------- planted mistakes in copies
def _planted_oracle(old, new):
    """A copy of the whole oracle module with one source substring replaced."""
    import inspect
    import types
    src = inspect.getsource(orc)
    assert src.count(old) == 1, old
    mod = types.ModuleType("planted_oracle")
    exec(compile(src.replace(old, new), "planted_oracle", "exec"), mod.__dict__)
    return mod


def _pin_failures(m):
    """Runs the independent pins against oracle module `m`; returns the names that fail."""
    fails = []
    golden = json.load(open(os.path.join(GOLDEN, "lambda_init_endpoints.json")))
    r = rng(77)
    # lambda_init at the page's endpoint, its limit, and the gap to it shrinking by e^-0.3
    if abs(m.lambda_init(1) - golden["layer_1"]) > 1e-15:
        fails.append("lambda_init(1)")
    if abs(m.lambda_init(200) - golden["limit_deep_layers"]) > 1e-15:
        fails.append("lambda_init limit")
    gaps = [golden["limit_deep_layers"] - m.lambda_init(l) for l in (3, 4)]
    if abs(gaps[1] - math.exp(-0.3) * gaps[0]) > 1e-15:
        fails.append("lambda_init decay")
    # lambda closed form: a = ln 2 (e^a = 2), b = 0 (e^b = 1) -> lambda = 1 + lambda_init
    d = 8
    lq1 = np.zeros(d); lk1 = np.zeros(d); lq1[0] = math.log(2.0); lk1[0] = 1.0
    st = m.lambda_scalar(lq1, lk1, np.zeros(d), np.zeros(d), 5)
    if abs(st["lambda"] - (1.0 + m.lambda_init(5))) > 1e-14:
        fails.append("lambda closed form")
    # one lambda_init for every layer: zero vectors give lambda = lambda_init at any layer,
    # and the closed form above gives 1 + lambda_init
    fixed = json.load(open(os.path.join(GOLDEN, "lambda_init_fixed.json")))
    li_fix = fixed["fixed_lambda_init_example"]
    for layer in (1, 9):
        z = np.zeros(d)
        if m.lambda_scalar(z, z, z, z, layer, fixed_init=li_fix)["lambda"] != li_fix:
            fails.append("fixed lambda_init")
    st = m.lambda_scalar(lq1, lk1, np.zeros(d), np.zeros(d), 5, fixed_init=li_fix)
    if abs(st["lambda"] - (1.0 + li_fix)) > 1e-14:
        fails.append("fixed lambda_init closed form")
    # many layers at once: row k is layer first + k (zero vectors: lambda = lambda_init,
    # 0.2 at layer 1 and the gap to 0.8 shrinking by e^-0.3 per layer)
    zs = np.zeros((3, d))
    lays = m.lambda_layers(zs, zs, zs, zs, 1)
    if abs(lays[0]["lambda"] - golden["layer_1"]) > 1e-15:
        fails.append("layers: first row")
    g0, g1 = (golden["limit_deep_layers"] - lays[k]["lambda"] for k in (0, 1))
    if abs(g1 - math.exp(-0.3) * g0) > 1e-15:
        fails.append("layers: row k is layer first + k")
    rows = rand(r, 4, 2, d)
    lays = m.lambda_layers(rows[0], rows[1], rows[2], rows[3], 4, fixed_init=li_fix)
    for k in range(2):
        ea = math.exp(float(np.dot(rows[0][k], rows[1][k])))
        eb = math.exp(float(np.dot(rows[2][k], rows[3][k])))
        if abs(lays[k]["lambda"] - (ea - eb + li_fix)) > 1e-12:
            fails.append("layers: row k uses vectors k")
    # forward: two-map composition of torch's causal attention, on one head
    n, d = 12, 4
    q1, q2, k1, k2 = (rand(r, 1, 1, n, d) for _ in range(4))
    v = rand(r, 1, 1, n, 2 * d)
    lam, li = 0.37, 0.25
    y, sv = m.forward(q1, q2, k1, k2, v, lam, li, want_saved=True)
    ref_o = sdpa_causal(q1, k1, v) - lam * sdpa_causal(q2, k2, v)
    if not np.allclose(sv["o"], ref_o, rtol=1e-10, atol=1e-12):
        fails.append("two-map composition")
    # RMSNorm and scale against torch's rms_norm, at a magnitude where eps matters
    t = torch.from_numpy(ref_o[0, 0]).double()
    ref_y = (1 - li) * torch.nn.functional.rms_norm(t, (2 * d,), eps=1e-5).numpy()
    if not np.allclose(y[0, 0], ref_y, rtol=1e-10, atol=1e-12):
        fails.append("norm and scale")
    small = 1e-3 * ref_o[0, 0]
    ys, _ = m.rms_norm_rows(small)
    ref_s = torch.nn.functional.rms_norm(torch.from_numpy(small), (2 * d,), eps=1e-5).numpy()
    if not np.allclose(ys, ref_s, rtol=1e-10, atol=1e-12):
        fails.append("rmsnorm eps")
    # row 0 closed form: Y[0] = (1 - li)(1 - lam) V0 / sqrt((1 - lam)^2 mean(V0^2) + eps)
    v0 = v[0, 0, 0]
    y0 = (1 - li) * (1 - lam) * v0 / math.sqrt((1 - lam) ** 2 * np.mean(v0 * v0) + 1e-5)
    if not np.allclose(y[0, 0, 0], y0, rtol=1e-12, atol=1e-14):
        fails.append("row 0")
    # lse is the log of the row normaliser
    s = 1.0 / math.sqrt(d)
    i = n - 1
    if abs(sv["lse2"][0, 0, i] - np.log(np.sum(np.exp(s * (k2[0, 0] @ q2[0, 0, i]))))) > 1e-12:
        fails.append("lse")
    # decode equals the last row of the prefill over the first len tokens
    ln = 7
    yd = m.decode(q1[:, :, ln - 1], q2[:, :, ln - 1], k1, k2, v, np.array([ln]), lam, li)
    yp = m.forward(q1[:, :, :ln], q2[:, :, :ln], k1[:, :, :ln], k2[:, :, :ln], v[:, :, :ln],
                   lam, li)
    if not np.allclose(yd[0, 0], yp[0, 0, ln - 1], rtol=1e-12, atol=1e-14):
        fails.append("decode")
    # append token ln - 1 to a cache holding tokens 0 .. ln - 2 (garbage beyond), then
    # decode: equal to the same prefill row; a full cache is left unchanged
    junk = lambda a: np.concatenate([a[:, :, :ln - 1], rand(r, *a[:, :, ln - 1:].shape)], 2)
    c1, c2, cv, lens = m.cache_append(k1[:, :, ln - 1], k2[:, :, ln - 1], v[:, :, ln - 1],
                                      junk(k1), junk(k2), junk(v), np.array([ln - 1]))
    ya = m.decode(q1[:, :, ln - 1], q2[:, :, ln - 1], c1, c2, cv, lens, lam, li)
    if lens[0] != ln or not np.allclose(ya[0, 0], yp[0, 0, ln - 1], rtol=1e-12, atol=1e-14):
        fails.append("append then decode")
    f1, _, _, flen = m.cache_append(k1[:, :, 0], k2[:, :, 0], v[:, :, 0], k1, k2, v,
                                    np.array([n]))
    if flen[0] != n or not np.array_equal(f1, k1):
        fails.append("append to a full cache")
    # backward: central finite differences of the module's own forward
    n, d, H = 5, 3, 2
    p = {k: rand(r, 1, H, n, d) for k in ("q1", "q2", "k1", "k2")}
    p["v"] = rand(r, 1, H, n, 2 * d)
    for k in ("lq1", "lk1", "lq2", "lk2"):
        p[k] = rand(r, d, scale=0.3)
    dy = rand(r, 1, H, n, 2 * d)
    g = m.backward(p["q1"], p["q2"], p["k1"], p["k2"], p["v"], dy, p["lq1"], p["lk1"],
                   p["lq2"], p["lk2"], 3)

    def loss():
        st = m.lambda_scalar(p["lq1"], p["lk1"], p["lq2"], p["lk2"], 3)
        return float(np.sum(m.forward(p["q1"], p["q2"], p["k1"], p["k2"], p["v"],
                                      st["lambda"], st["lambda_init"]) * dy))
    h = 1e-6
    for name in ("q1", "q2", "k1", "k2", "v", "lq1", "lk1", "lq2", "lk2"):
        flat = p[name].reshape(-1)
        fd = np.empty(flat.size)
        for j in range(flat.size):
            old = flat[j]
            flat[j] = old + h; lp = loss()
            flat[j] = old - h; lm = loss()
            flat[j] = old
            fd[j] = (lp - lm) / (2 * h)
        an = g["d" + name].reshape(-1)
        if np.max(np.abs(an - fd)) > 1e-5 * max(np.max(np.abs(fd)), 1e-9):
            fails.append("fd " + name)
    # grouped-query backward: dV of a K/V head shared by two query heads, by central
    # differences of the grouped forward
    pg = {k: rand(r, 1, 2, 4, 3) for k in ("q1", "q2")}
    pg.update({k: rand(r, 1, 1, 4, 3) for k in ("k1", "k2")})
    pg["v"] = rand(r, 1, 1, 4, 6)
    for k in ("lq1", "lk1", "lq2", "lk2"):
        pg[k] = p[k][:3].copy()
    dyg = rand(r, 1, 2, 4, 6)
    gg = m.backward(pg["q1"], pg["q2"], pg["k1"], pg["k2"], pg["v"], dyg, pg["lq1"],
                    pg["lk1"], pg["lq2"], pg["lk2"], 3)
    stg = m.lambda_scalar(pg["lq1"], pg["lk1"], pg["lq2"], pg["lk2"], 3)
    fv = pg["v"].reshape(-1)
    fdg = np.empty(fv.size)
    for j in range(fv.size):
        old = fv[j]
        fv[j] = old + h
        lp = float(np.sum(m.forward(pg["q1"], pg["q2"], pg["k1"], pg["k2"], pg["v"],
                                    stg["lambda"], stg["lambda_init"]) * dyg))
        fv[j] = old - h
        lm = float(np.sum(m.forward(pg["q1"], pg["q2"], pg["k1"], pg["k2"], pg["v"],
                                    stg["lambda"], stg["lambda_init"]) * dyg))
        fv[j] = old
        fdg[j] = (lp - lm) / (2 * h)
    if np.max(np.abs(gg["dv"].reshape(-1) - fdg)) > 1e-5 * max(np.max(np.abs(fdg)), 1e-9):
        fails.append("fd grouped dv")
    # the RMSNorm weight gradient, by central differences of the same loss
    wgt = 1.0 + 0.3 * rand(r, H, 2 * d)
    gw = m.backward(p["q1"], p["q2"], p["k1"], p["k2"], p["v"], dy, p["lq1"], p["lk1"],
                    p["lq2"], p["lk2"], 3, weight=wgt)["d_rms_weight"]
    st = m.lambda_scalar(p["lq1"], p["lk1"], p["lq2"], p["lk2"], 3)
    fdw = np.empty(wgt.size)
    for j in range(wgt.size):
        old = wgt.flat[j]
        wgt.flat[j] = old + h
        lp = float(np.sum(m.forward(p["q1"], p["q2"], p["k1"], p["k2"], p["v"], st["lambda"],
                                    st["lambda_init"], weight=wgt) * dy))
        wgt.flat[j] = old - h
        lm = float(np.sum(m.forward(p["q1"], p["q2"], p["k1"], p["k2"], p["v"], st["lambda"],
                                    st["lambda_init"], weight=wgt) * dy))
        wgt.flat[j] = old
        fdw[j] = (lp - lm) / (2 * h)
    if np.max(np.abs(gw.reshape(-1) - fdw)) > 1e-5 * max(np.max(np.abs(fdw)), 1e-9):
        fails.append("fd rms weight")
    fails += _epilogue_fd_failures(m, r)
    # projections. One-hot tokens: token t of the flattened batch is unit vector
    # e_(t mod d_model), so each output entry is one weight entry; the weight is coded
    # w[row, col] = row + 1000 col, which names the weight row that fed each output.
    B, N, H, d, dm = 2, 3, 2, 4, 8
    x = np.zeros((B, N, dm))
    for t in range(B * N):
        x.reshape(B * N, dm)[t, t % dm] = 1.0
    w = np.add.outer(np.arange(6 * H * d), 1000.0 * np.arange(dm))
    q1, q2, k1, k2, v = m.qkv_proj(x, w, H, d)
    hd2 = 2 * H * d
    ok = True
    for b in range(B):
        for i in range(N):
            col = 1000.0 * ((b * N + i) % dm)
            for hh in range(H):
                for c in range(d):
                    base = hh * 2 * d + c
                    ok &= q1[b, hh, i, c] == base + col and q2[b, hh, i, c] == base + d + col
                    ok &= k1[b, hh, i, c] == hd2 + base + col
                    ok &= k2[b, hh, i, c] == hd2 + base + d + col
                for c in range(2 * d):
                    ok &= v[b, hh, i, c] == 2 * hd2 + hh * 2 * d + c + col
    if not ok:
        fails.append("qkv projection placement")
    # grouped-query projection: H = 4 query heads, Hkv = 2 key/value heads
    Hq, Hk = 4, 2
    w = np.add.outer(np.arange(2 * d * (Hq + 2 * Hk)), 1000.0 * np.arange(dm))
    q1, q2, k1, k2, v = m.qkv_proj(x, w, Hq, d, kv_heads=Hk)
    qc, kc = 2 * Hq * d, 2 * Hk * d
    ok = q1.shape == (B, Hq, N, d) and k1.shape == (B, Hk, N, d) and v.shape == (B, Hk, N, 2 * d)
    for b in range(B):
        for i in range(N):
            col = 1000.0 * ((b * N + i) % dm)
            for hh in range(Hk):
                for c in range(d):
                    base = hh * 2 * d + c
                    ok &= k1[b, hh, i, c] == qc + base + col
                    ok &= k2[b, hh, i, c] == qc + base + d + col
                for c in range(2 * d):
                    ok &= v[b, hh, i, c] == qc + kc + hh * 2 * d + c + col
            ok &= q2[b, Hq - 1, i, 0] == (Hq - 1) * 2 * d + d + col
    if not ok:
        fails.append("grouped qkv projection placement")
    # grouped-query attention = the same computation with each K/V head repeated for the
    # query heads of its group (consecutive heads)
    n, dd, Hq, Hk = 7, 4, 4, 2
    q1, q2 = (rand(r, 1, Hq, n, dd) for _ in range(2))
    k1, k2 = (rand(r, 1, Hk, n, dd) for _ in range(2))
    v = rand(r, 1, Hk, n, 2 * dd)
    rep = lambda t: np.repeat(t, Hq // Hk, axis=1)
    yg = m.forward(q1, q2, k1, k2, v, 0.4, 0.3)
    ym = m.forward(q1, q2, rep(k1), rep(k2), rep(v), 0.4, 0.3)
    if not np.array_equal(yg, ym):
        fails.append("grouped forward")
    dg = m.decode(q1[:, :, -1], q2[:, :, -1], k1, k2, v, np.array([5]), 0.4, 0.3)
    dm_ = m.decode(q1[:, :, -1], q2[:, :, -1], rep(k1), rep(k2), rep(v), np.array([5]), 0.4, 0.3)
    if not np.array_equal(dg, dm_):
        fails.append("grouped decode")
    # output projection: brute-force sums over the concatenated channels
    attn = rand(r, B, N, H, 2 * d)
    wo = rand(r, 5, H * 2 * d)
    y = m.out_proj(attn, wo)
    for b, i, o in [(0, 0, 0), (1, 2, 4), (0, 1, 3)]:
        acc = 0.0
        for hh in range(H):
            for c in range(2 * d):
                acc += attn[b, i, hh, c] * wo[o, hh * 2 * d + c]
        if abs(y[b, i, o] - acc) > 1e-12:
            fails.append("out projection sum")
            break
    return fails


def test_pins_hold_on_the_oracle():
    assert _pin_failures(orc) == []


PLANTS = [
    ("lambda sign", "lam = (ea - eb) + li", "lam = (eb - ea) + li"),
    ("lambda_init form", "return 0.8 - 0.6 * e", "return 0.8 - 0.6 / e"),
    ("fixed lambda_init ignored",
     "li = lambda_init(layer) if fixed_init is None else float(fixed_init)",
     "li = lambda_init(layer)"),
    ("layers all use the first index", "rows[3][k], first_layer + k,", "rows[3][k], first_layer,"),
    ("layers read row 0 only", "lambda_scalar(rows[0][k], rows[1][k],", "lambda_scalar(rows[0][0], rows[1][0],"),
    ("DiffAttn sign", "o[r0:r1] = (a1 - lam * a2) @ v[:kend]",
     "o[r0:r1] = (a1 + lam * a2) @ v[:kend]"),
    ("second map uses K1", "s2 = s * (q2[r0:r1] @ k2[:kend].T)",
     "s2 = s * (q2[r0:r1] @ k1[:kend].T)"),
    ("transposed scores", "s1 = s * (q1[r0:r1] @ k1[:kend].T)",
     "s1 = s * (k1[:kend] @ q1[r0:r1].T)"),
    ("eps outside the root", "np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps)\n    y = o",
     "(np.sqrt(np.mean(o * o, axis=-1, keepdims=True)) + eps)\n    y = o"),
    ("scale by lambda_init", "    y = (1.0 - lam_init) * y\n    if want_saved:",
     "    y = lam_init * y\n    if want_saved:"),
    ("lse sign", "saved[name][r0:r1] = m + np.log(", "saved[name][r0:r1] = m - np.log("),
    ("decode length off by one", "n = L if cache_len is None else int(cache_len[b])",
     "n = L if cache_len is None else int(cache_len[b]) - 1"),
    ("append keeps the length", "        lens[b] = n + 1", "        lens[b] = n"),
    ("append writes V one row early", "vc[b, :, n] = v_new[b]", "vc[b, :, n - 1] = v_new[b]"),
    ("norm gradient sign", "G = r * g - o * r ** 3", "G = r * g + o * r ** 3"),
    ("dK transposed", '"dk1": s * ds1.T @ q1', '"dk1": s * ds1 @ q1'),
    ("dS2 uses A1", "ds2 = a2 * (da2 - np.sum(a2 * da2", "ds2 = a2 * (da2 - np.sum(a1 * da2"),
    ("dlq2 sign", 'out["dlq2"] = -dlam * st["exp_b"] * lk2', 'out["dlq2"] = dlam * st["exp_b"] * lk2'),
    ("rms weight gradient without r", '"dw": (1.0 - lam_init) * np.sum(dy * o * r, axis=0)',
     '"dw": (1.0 - lam_init) * np.sum(dy * o, axis=0)'),
    ("query halves swapped", "return (per_head(q[..., 0, :]), per_head(q[..., 1, :]),",
     "return (per_head(q[..., 1, :]), per_head(q[..., 0, :]),"),
    ("value block from the key rows", "v = y[..., hd2 + kd2:].reshape", "v = y[..., hd2:hd2 + kd2].reshape"),
    ("projection not transposed", "y = x @ w.T ", "y = x @ w.reshape(dm, -1) "),
    ("heads concatenated in reverse", "return a.reshape(B, N, H * d2) @",
     "return a[:, :, ::-1].reshape(B, N, H * d2) @"),
    ("grouped forward maps heads modulo", "        kh = h // g\n        r = head_forward(",
     "        kh = h % (H // g)\n        r = head_forward("),
    ("grouped decode maps heads modulo", "            kh = h // g\n            s1 = s *",
     "            kh = h % (H // g)\n            s1 = s *"),
    ("grouped keys: head and half swapped", "k = y[..., hd2:hd2 + kd2].reshape(B, N, Hkv, 2, d)",
     "k = y[..., hd2:hd2 + kd2].reshape(B, N, 2, Hkv, d).transpose(0, 1, 3, 2, 4)"),
    ("grouped dK keeps one head", "                out[k][b, kh] = out[k][b, kh] + r[k]",
     "                out[k][b, kh] = r[k]"),
    ("dlam sign", '"dlam": float(-np.sum(a2 * gv))', '"dlam": float(np.sum(a2 * gv))'),
    ("epilogue dlam sign", '"dlam": float(-np.sum(d2))', '"dlam": float(np.sum(d2))'),
    ("epilogue D2 from O1", "d2 = np.sum(G * o2, axis=-1)", "d2 = np.sum(G * o1, axis=-1)"),
    ("epilogue O with +lam", "    o = o1 - lam * o2\n", "    o = o1 + lam * o2\n"),
    ("epilogue norm term halved", "G = r * g - (r ** 3 / n) * o", "G = r * g - (r ** 3 / (2 * n)) * o"),
    ("epilogue weight gradient without the scale", '"dw": (1.0 - lam_init) * np.sum(r * o * dy',
     '"dw": np.sum(r * o * dy'),
]


@pytest.mark.parametrize("name,old,new", PLANTS, ids=[p[0] for p in PLANTS])
def test_planted_mistake_fails_a_pin(name, old, new):
    m = _planted_oracle(old, new)
    assert _pin_failures(m), name
