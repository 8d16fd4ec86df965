"""Pins of the CPU oracle's building blocks against facts the pages and the
mathematics fix (closed forms, invariants, library special cases, finite
differences).  CPU only."""
import numpy as np
import pytest
from scipy.special import logsumexp

import oracle as orc

EPS = 2.0 ** -23


def rng(seed=0):
    return np.random.Generator(np.random.PCG64(seed))


# ------------------------------------------------------------------ linear

def test_linear_matches_library_matmul():
    r = rng(1)
    x, W = r.standard_normal((13, 7)), r.standard_normal((5, 7))
    np.testing.assert_allclose(orc.linear(x, W), x @ W.T, rtol=1e-13, atol=1e-13)
    dy = r.standard_normal((13, 5))
    dx, dW = orc.linear_bwd(x, W, dy)
    np.testing.assert_allclose(dx, dy @ W, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dW, dy.T @ x, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ RMSNorm
# "nanochat 项目深度分析" §2.1 item 5: norm(x) = F.rms_norm over the last dim, no weight.

@pytest.mark.parametrize("scale", [1e-4, 0.02, 1.0, 300.0])
def test_rmsnorm_closed_form_rms(scale):
    x = rng(2).standard_normal((9, 64)) * scale
    y, rstd = orc.rmsnorm(x)
    m = (x ** 2).mean(-1)
    # mean(y^2) = m / (m + eps) exactly for y = x / sqrt(m + eps)
    np.testing.assert_allclose((y ** 2).mean(-1), m / (m + EPS), rtol=1e-13)
    np.testing.assert_allclose(rstd, 1.0 / np.sqrt(m + EPS), rtol=1e-14)


def test_rmsnorm_constant_row_and_scale_invariance():
    c = 0.37
    y, _ = orc.rmsnorm(np.full((1, 10), c))
    np.testing.assert_allclose(y, c / np.sqrt(c * c + EPS), rtol=1e-15)
    x = rng(3).standard_normal((4, 32))
    y1, _ = orc.rmsnorm(x)
    y2, _ = orc.rmsnorm(7.5 * x)
    np.testing.assert_allclose(y1, y2, rtol=1e-6)  # equal up to the epsilon's weight


def test_rmsnorm_backward_finite_difference():
    r = rng(4)
    x = r.standard_normal((3, 11)) * 0.1
    w = r.standard_normal((3, 11))          # loss = sum(w * y)
    y, rstd = orc.rmsnorm(x)
    dx = orc.rmsnorm_bwd(y, rstd, w)
    h = 1e-6
    fd = np.zeros_like(x)
    for idx in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[idx] += h
        xm[idx] -= h
        fd[idx] = ((orc.rmsnorm(xp)[0] * w).sum() - (orc.rmsnorm(xm)[0] * w).sum()) / (2 * h)
    np.testing.assert_allclose(dx, fd, rtol=1e-6, atol=1e-8)


# ------------------------------------------------------------------ RoPE
# "nanochat 项目深度分析" §2.1 item 1 and §5.3: split halves, y1 = x1 cos + x2 sin,
# y2 = -x1 sin + x2 cos.

def test_rope_position_zero_is_identity_bitwise():
    x = rng(5).standard_normal((2, 1, 3, 16))
    assert np.array_equal(orc.rope(x), x)


def test_rope_d2_is_textbook_rotation_by_minus_t():
    # D = 2: one pair, angle t * base^0 = t; the pages' signs make it the
    # rotation matrix [[cos t, sin t], [-sin t, cos t]], i.e. rotation by -t.
    T = 9
    x = rng(6).standard_normal((1, T, 1, 2))
    y = orc.rope(x)
    for t in range(T):
        R = np.array([[np.cos(t), np.sin(t)], [-np.sin(t), np.cos(t)]])
        np.testing.assert_allclose(y[0, t, 0], R @ x[0, t, 0], rtol=1e-14, atol=1e-15)


def test_rope_pair_norms_preserved_and_split_half_pairing():
    D = 16
    x = rng(7).standard_normal((2, 12, 3, D))
    y = orc.rope(x)
    h = D // 2
    np.testing.assert_allclose(y[..., :h] ** 2 + y[..., h:] ** 2, x[..., :h] ** 2 + x[..., h:] ** 2, rtol=1e-13)
    # an interleaved pairing (2i, 2i+1) would not preserve these sums
    assert not np.allclose(y[..., 0::2] ** 2 + y[..., 1::2] ** 2, x[..., 0::2] ** 2 + x[..., 1::2] ** 2)


def test_rope_frequencies():
    # unit vector on coordinate i of the first half: y_i = cos(phi), y_{i+D/2} = -sin(phi)
    D, T, base = 8, 50, 10000.0
    for i in range(D // 2):
        x = np.zeros((1, T, 1, D))
        x[..., i] = 1.0
        y = orc.rope(x, base=base)
        phi = np.unwrap(np.arctan2(-y[0, :, 0, i + D // 2], y[0, :, 0, i]))
        np.testing.assert_allclose(phi, np.arange(T) * base ** (-2.0 * i / D), rtol=1e-12, atol=1e-12)


def test_rope_relative_position_property():
    D = 32
    r = rng(8)
    qv, kv = r.standard_normal(D), r.standard_normal(D)
    T = 40
    Q = np.broadcast_to(qv, (1, T, 1, D)).copy()
    K = np.broadcast_to(kv, (1, T, 1, D)).copy()
    rq, rk = orc.rope(Q)[0, :, 0], orc.rope(K)[0, :, 0]
    for m, n, s in [(3, 1, 5), (10, 10, 7), (0, 20, 13)]:
        np.testing.assert_allclose(rq[m] @ rk[n], rq[m + s] @ rk[n + s], rtol=1e-10, atol=1e-12)


def test_rope_inverse_is_transpose():
    r = rng(9)
    x, g = r.standard_normal((2, 6, 2, 8)), r.standard_normal((2, 6, 2, 8))
    np.testing.assert_allclose(orc.rope(orc.rope(x), inverse=True), x, rtol=1e-13, atol=1e-14)
    # <R x, g> = <x, R^T g>: the inverse is the backward of the map
    np.testing.assert_allclose((orc.rope(x) * g).sum(), (x * orc.rope(g, inverse=True)).sum(), rtol=1e-13)


# ------------------------------------------------------------------ attention
# causal self-attention (devpress guide §4.1) with n_head / n_kv_head ("nanochat 项目深度分析" §2.1 item 6)

def qkv(B=2, T=9, H=4, Hkv=2, D=8, seed=10):
    r = rng(seed)
    return r.standard_normal((B, T, H, D)), r.standard_normal((B, T, Hkv, D)), r.standard_normal((B, T, Hkv, D))


def test_attention_future_invariance_bitwise():
    q, k, v = qkv()
    o, lse = orc.attention(q, k, v)
    t = 4
    k2, v2, q2 = k.copy(), v.copy(), q.copy()
    k2[:, t + 1:] += 3.0
    v2[:, t + 1:] -= 2.0
    q2[:, t + 1:] *= -1.0
    o2, lse2 = orc.attention(q2, k2, v2)
    assert np.array_equal(o[:, :t + 1], o2[:, :t + 1])
    assert np.array_equal(lse[:, :, :t + 1], lse2[:, :, :t + 1])


def test_attention_nan_poison_future_rows():
    q, k, v = qkv()
    o, _ = orc.attention(q, k, v)
    t = 3
    k2, v2 = k.copy(), v.copy()
    k2[:, t + 1:] = np.nan
    v2[:, t + 1:] = np.nan
    o2, _ = orc.attention(q, k2, v2)
    assert np.isfinite(o2[:, :t + 1]).all()
    assert np.array_equal(o[:, :t + 1], o2[:, :t + 1])


def test_attention_first_position_and_zero_query():
    q, k, v = qkv()
    o, _ = orc.attention(q, k, v)
    r = q.shape[2] // k.shape[2]
    for h in range(q.shape[2]):
        np.testing.assert_array_equal(o[:, 0, h], v[:, 0, h // r])
    o0, lse0 = orc.attention(np.zeros_like(q), k, v)
    T = q.shape[1]
    mean_v = np.cumsum(v, axis=1) / np.arange(1, T + 1)[None, :, None, None]
    for h in range(q.shape[2]):
        np.testing.assert_allclose(o0[:, :, h], mean_v[:, :, h // r], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse0, np.broadcast_to(np.log(np.arange(1, T + 1)), lse0.shape), rtol=1e-14)


def test_attention_rows_sum_to_one():
    q, k, v = qkv()
    o, _ = orc.attention(q, k, np.ones_like(v))
    np.testing.assert_allclose(o, 1.0, rtol=1e-14)


def test_attention_gqa_equals_mha_with_repeated_heads():
    q, k, v = qkv(H=6, Hkv=2)
    o, lse = orc.attention(q, k, v)
    krep, vrep = np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2)  # head h uses kv head h // 3
    o2, lse2 = orc.attention(q, krep, vrep)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_attention_lse_and_weights_match_library_softmax():
    q, k, v = qkv(B=1, T=6, H=2, Hkv=1, D=4)
    o, lse = orc.attention(q, k, v)
    D = q.shape[-1]
    for h in range(2):
        S = q[0, :, h] @ k[0, :, 0].T / np.sqrt(D)
        S = np.where(np.tril(np.ones_like(S)) > 0, S, -np.inf)
        np.testing.assert_allclose(lse[0, h], logsumexp(S, axis=1), rtol=1e-14)
        P = np.exp(S - logsumexp(S, axis=1, keepdims=True))
        np.testing.assert_allclose(o[0, :, h], P @ v[0, :, 0], rtol=1e-12, atol=1e-14)


def test_attention_backward_finite_difference():
    q, k, v = qkv(B=1, T=5, H=4, Hkv=2, D=4, seed=11)
    w = rng(12).standard_normal(q.shape)
    dq, dk, dv = orc.attention_bwd(q, k, v, w)
    h = 1e-6

    def L(q_, k_, v_):
        return (orc.attention(q_, k_, v_)[0] * w).sum()

    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            ap, am = arr.copy(), arr.copy()
            ap[idx] += h
            am[idx] -= h
            args_p = [ap if a is arr else a for a in (q, k, v)]
            args_m = [am if a is arr else a for a in (q, k, v)]
            fd[idx] = (L(*args_p) - L(*args_m)) / (2 * h)
        np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8)


# ------------------------------------------------------------------ cross-entropy

def test_cross_entropy_zero_logits_closed_form():
    V, N = 37, 6
    z = np.zeros((N, V))
    t = np.array([0, 5, 36, -1, 2, 2], dtype=np.int32)
    loss, lse, lr, valid = orc.cross_entropy(z, t)
    assert valid == 5
    np.testing.assert_allclose(loss, np.log(V), rtol=1e-15)
    dz = orc.cross_entropy_bwd(z, t, grad_scale=1.0)
    exp = np.full((N, V), 1.0 / V) / valid
    for n in range(N):
        if t[n] >= 0:
            exp[n, t[n]] -= 1.0 / valid
        else:
            exp[n] = 0.0
    np.testing.assert_allclose(dz, exp, rtol=1e-14, atol=1e-17)
    assert np.all(dz[3] == 0.0)


def test_cross_entropy_matches_library_logsumexp_and_fd():
    r = rng(13)
    z = r.standard_normal((5, 11)) * 3
    t = np.array([1, -1, 10, 0, 4], dtype=np.int32)
    loss, lse, lr, valid = orc.cross_entropy(z, t)
    np.testing.assert_allclose(lse, logsumexp(z, axis=1), rtol=1e-14)
    keep = t >= 0
    np.testing.assert_allclose(loss, np.mean(lse[keep] - z[keep, t[keep]]), rtol=1e-14)
    dz = orc.cross_entropy_bwd(z, t, grad_scale=0.5)
    np.testing.assert_allclose(dz.sum(1), 0.0, atol=1e-15)
    h = 1e-6
    fd = np.zeros_like(z)
    for idx in np.ndindex(z.shape):
        zp, zm = z.copy(), z.copy()
        zp[idx] += h
        zm[idx] -= h
        fd[idx] = 0.5 * (orc.cross_entropy(zp, t)[0] - orc.cross_entropy(zm, t)[0]) / (2 * h)
    np.testing.assert_allclose(dz, fd, rtol=1e-6, atol=1e-9)
