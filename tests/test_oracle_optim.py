"""Pins of the oracle's optimizer step (oracle/optim_oracle.c), CPU only.

- The Newton-Schulz iteration against its closed form: the iteration maps X = U S V^T to U p(S) V^T with the
  quintic p(s) = a s + b s^3 + c s^5, so five steps from G / ||G||_F give U p^5(S / ||G||_F) V^T, computed
  here from numpy's SVD.
- AdamW against torch.optim.AdamW in fp64 (a library routine of the same definition).
- The composed Muon step against torch.optim.Muon, whose Newton-Schulz runs in bf16: agreement to that
  routine's rounding, which is far tighter than what a wrong momentum form, lerp direction, aspect-ratio scale
  or weight-decay placement would leave.
- The packed step: each matrix goes through Muon with its own momentum buffer and aspect ratio, wte and
  lm_head through AdamW with their own learning rates, and nothing moves when gradients and state are zero.
"""
import numpy as np
import pytest
import torch

import oracle as orc

A, B, C = 3.4445, -4.7750, 2.0315


def quintic5(s):
    for _ in range(5):
        s = A * s + B * s ** 3 + C * s ** 5
    return s


def ns_closed_form(G):
    U, S, Vt = np.linalg.svd(G, full_matrices=False)
    return (U * quintic5(S / np.linalg.norm(G))) @ Vt


@pytest.mark.parametrize("shape", [(12, 20), (20, 12), (16, 16), (1, 9)])
def test_newton_schulz_equals_closed_form(shape):
    rng = np.random.default_rng(3)
    G = rng.standard_normal(shape)
    out = orc.newton_schulz(G)
    want = ns_closed_form(G)
    assert np.max(np.abs(out - want)) <= 1e-11 * np.max(np.abs(want))


def test_newton_schulz_spectrum_and_degenerate_input():
    # a chosen spectrum: output singular values are p^5(s / ||s||), all inside the iteration's band
    rng = np.random.default_rng(4)
    U, _ = np.linalg.qr(rng.standard_normal((24, 24)))
    V, _ = np.linalg.qr(rng.standard_normal((40, 40)))
    s = np.linspace(0.2, 1.0, 24)
    G = (U * s) @ V[:24]
    sv = np.linalg.svd(orc.newton_schulz(G), compute_uv=False)
    assert np.allclose(np.sort(sv), np.sort(quintic5(s / np.linalg.norm(s))), rtol=1e-10)
    assert sv.min() > 0.5 and sv.max() < 1.3
    # a zero matrix stays zero (the norm is clamped at eps, not divided by zero)
    assert np.array_equal(orc.newton_schulz(np.zeros((5, 7))), np.zeros((5, 7)))


def test_adamw_equals_torch():
    rng = np.random.default_rng(5)
    p0 = rng.standard_normal(50)
    grads = [rng.standard_normal(50) for _ in range(3)]
    lr, b1, b2, eps, wd = 0.2, 0.8, 0.95, 1e-10, 0.01
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.AdamW([tp], lr=lr, betas=(b1, b2), eps=eps, weight_decay=wd)
    p, m, v = p0.copy(), np.zeros(50), np.zeros(50)
    for t, g in enumerate(grads, 1):
        tp.grad = torch.tensor(g)
        opt.step()
        p, m, v = orc.adamw_update(p, g, m, v, t, lr, b1, b2, eps, wd)
        assert np.max(np.abs(p - tp.detach().numpy())) <= 1e-13 * np.max(np.abs(p))
    # first step from zero moments: the update is lr * g / (|g| + eps), i.e. lr * sign(g) here
    q, _, _ = orc.adamw_update(p0, grads[0], np.zeros(50), np.zeros(50), 1, lr, b1, b2, eps, 0.0)
    assert np.allclose(p0 - q, lr * np.sign(grads[0]), rtol=1e-8)


@pytest.mark.parametrize("shape", [(64, 48), (48, 128)])
def test_muon_step_agrees_with_torch(shape):
    rng = np.random.default_rng(6)
    p0 = rng.standard_normal(shape) * 0.02
    grads = [rng.standard_normal(shape) for _ in range(2)]
    lr, mu, wd = 0.02, 0.95, 0.1
    tp = torch.tensor(p0, dtype=torch.float64, requires_grad=True)
    opt = torch.optim.Muon([tp], lr=lr, momentum=mu, nesterov=True, weight_decay=wd)
    p, buf = p0.copy(), np.zeros(shape)
    for g in grads:
        prev = p.copy()
        tp.grad = torch.tensor(g)
        opt.step()
        p, buf = orc.muon_update(p, g, buf, lr, mu, True, wd)
        dt = tp.detach().numpy() - prev
        do = p - prev
        # torch's iteration runs in bf16: relative error of the update about 1e-2
        assert np.linalg.norm(do - dt) <= 3e-2 * np.linalg.norm(dt)
        tp.data = torch.tensor(p)     # continue both from the oracle's parameters


@pytest.mark.parametrize("shape,scale", [((64, 16), 2.0), ((16, 64), 1.0), ((32, 32), 1.0)])
def test_muon_aspect_ratio_scale(shape, scale):
    # momentum 0 without Nesterov makes the update the iterate of the gradient itself; from p = 0 with lr 1
    # the new parameter is -sqrt(max(1, rows / cols)) NS(g)
    g = np.random.default_rng(8).standard_normal(shape)
    p1, buf = orc.muon_update(np.zeros(shape), g, np.zeros(shape), 1.0, 0.0, False, 0.0)
    assert np.array_equal(buf, g)
    assert np.allclose(-p1, scale * orc.newton_schulz(g), rtol=1e-13, atol=1e-16)


def small_cfg():
    return orc.OracleConfig(2, 16, 2, 1, 8, 64, 37, 1, 4)


def test_packed_step_composition():
    cfg = small_cfg()
    P = orc.num_params(cfg)
    VC = 37 * 16
    rng = np.random.default_rng(7)
    params = rng.standard_normal(P) * 0.02
    grads = rng.standard_normal(P)
    state = rng.standard_normal(orc.optim_state_size(cfg)) ** 2       # moments and buffers from "earlier steps"
    assert state.size == P - 2 * VC + 4 * VC
    opt = orc.OptimConfig(weight_decay=0.05)
    newp, newst = orc.optim_step(cfg, params, grads, state, 3, opt)
    nmat = P - 2 * VC
    for l in range(cfg.n_layer):
        for w in range(6):
            off, r, c = orc.param_slice(cfg, l, w)
            sl = slice(off, off + r * c)
            bsl = slice(off - VC, off - VC + r * c)
            want_p, want_b = orc.muon_update(params[sl].reshape(r, c), grads[sl].reshape(r, c),
                                             state[bsl].reshape(r, c), opt.matrix_lr, opt.muon_momentum, True,
                                             opt.weight_decay)
            assert np.array_equal(newp[sl], want_p.ravel()) and np.array_equal(newst[bsl], want_b.ravel())
    for which, lr, base in ((0, opt.embedding_lr, nmat), (1, opt.unembedding_lr, nmat + 2 * VC)):
        off, r, c = orc.param_slice(cfg, -1, which)
        sl = slice(off, off + r * c)
        want = orc.adamw_update(params[sl], grads[sl], state[base:base + VC], state[base + VC:base + 2 * VC], 3, lr,
                                opt.adam_beta1, opt.adam_beta2, opt.adam_eps, opt.weight_decay)
        assert np.array_equal(newp[sl], want[0])
        assert np.array_equal(newst[base:base + VC], want[1]) and np.array_equal(newst[base + VC:base + 2 * VC],
                                                                                 want[2])
    # zero gradients and zero state, no weight decay: nothing moves
    z, zs = orc.optim_step(cfg, params, np.zeros(P), np.zeros(state.size), 1, orc.OptimConfig())
    assert np.array_equal(z, params) and not zs.any()
