"""Pins of the oracle's block variants (logit soft-cap, embedding norm), CPU only.

- Finite-difference gradients of every packed tensor with both variants on (central differences, odd shapes).
- Soft-cap: zero lm_head gives loss ln V for any cap (c tanh(0) = 0); a huge cap reproduces the uncapped model;
  every capped logit lies in (-c, c); the capped loss equals the cross-entropy (scipy logsumexp) of c tanh(z / c)
  computed from the oracle's own uncapped final-norm output.
- Embedding norm: the stream starts at unit RMS (m / (m + eps)); scaling wte by any a > 0 leaves the loss
  unchanged (exactly when eps = 0).
- The PyTorch fp64 autograd model with both variants, written from the formulas.
"""
import dataclasses

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

import oracle as orc
from test_oracle_model import FD_CFG, fd_inputs, torch_model_loss

VAR_CFG = dataclasses.replace(FD_CFG, logit_softcap=1.5, embed_norm=1)


def test_variant_gradients_match_central_finite_differences():
    cfg = VAR_CFG
    ids, tg, p = fd_inputs(cfg)
    _, g = orc.grad(cfg, ids, tg, p)
    r = np.random.Generator(np.random.PCG64(1))
    h = 1e-5
    for name, off, rows, cols in orc.tensor_names(cfg):
        n = rows * cols
        idx = off + r.choice(n, size=min(n, 16), replace=False)
        if name == "wte":
            idx = np.concatenate([idx, off + np.unique(ids)[:6] * cols + 5])
        fd = np.empty(len(idx))
        for j, i in enumerate(idx):
            pp, pm = p.copy(), p.copy()
            pp[i] += h
            pm[i] -= h
            fd[j] = (orc.forward(cfg, ids, tg, pp)[0] - orc.forward(cfg, ids, tg, pm)[0]) / (2 * h)
        err = np.max(np.abs(fd - g[idx])) / max(np.max(np.abs(g[off:off + n])), 1e-30)
        assert err < 1e-6, (name, err)


def test_softcap_special_cases_and_range():
    ids, tg, p = fd_inputs(FD_CFG)
    off, V, C = orc.param_slice(FD_CFG, -1, 1)
    z0 = p.copy()
    z0[off:off + V * C] = 0.0
    for cap in (0.7, 3.0):
        loss, _ = orc.forward(dataclasses.replace(FD_CFG, logit_softcap=cap), ids, tg, z0)
        assert abs(loss - np.log(V)) < 1e-13
    l_plain, a_plain = orc.forward(FD_CFG, ids, tg, p)
    l_huge, _ = orc.forward(dataclasses.replace(FD_CFG, logit_softcap=1e7), ids, tg, p)
    assert abs(l_huge - l_plain) < 1e-9 * abs(l_plain)
    # the capped loss is the cross-entropy of c tanh(z / c), z from the uncapped model's final-norm output
    cap = 1.5
    l_cap, a_cap = orc.forward(dataclasses.replace(FD_CFG, logit_softcap=cap), ids, tg, p)
    W = p[off:off + V * C].reshape(V, C)
    z = cap * np.tanh(a_plain["xf"] @ W.T / cap)
    assert np.all(np.abs(z) < cap)
    t = tg.reshape(-1)
    rows = (logsumexp(z, axis=1) - z[np.arange(t.size), np.maximum(t, 0)])[t >= 0]
    assert abs(l_cap - rows.mean()) < 1e-12 * abs(l_cap)


def test_embedding_norm_unit_rms_and_scale_invariance():
    cfg = dataclasses.replace(FD_CFG, embed_norm=1)
    ids, tg, p = fd_inputs(cfg)
    loss, acts = orc.forward(cfg, ids, tg, p)
    x0 = acts["x0"]
    m = np.mean(x0 ** 2, axis=1)
    np.testing.assert_allclose(np.mean(acts["x0n"] ** 2, axis=1), m / (m + cfg.norm_eps), rtol=1e-13)
    off, V, C = orc.param_slice(cfg, -1, 0)
    q = p.copy()
    q[off:off + V * C] *= 37.0
    loss2, _ = orc.forward(cfg, ids, tg, q)
    assert abs(loss2 - loss) < 1e-6 * abs(loss)          # eps / mean(x0^2) ~ 1e-6 breaks exact invariance
    c0 = dataclasses.replace(cfg, norm_eps=0.0)           # without eps the invariance is exact up to rounding
    assert abs(orc.forward(c0, ids, tg, q)[0] - orc.forward(c0, ids, tg, p)[0]) < 1e-13 * abs(loss)
    # without the norm the same scaling changes the model
    assert abs(orc.forward(FD_CFG, ids, tg, q)[0] - orc.forward(FD_CFG, ids, tg, p)[0]) > 1e-3


def test_variants_agree_with_torch_fp64_autograd():
    cfg = VAR_CFG
    ids, tg, p = fd_inputs(cfg)
    loss_t, g_t = torch_model_loss(cfg, ids, tg, p)
    loss_o, g_o = orc.grad(cfg, ids, tg, p)
    assert abs(loss_o - loss_t) <= 1e-12 * abs(loss_t)
    for name, off, r, c in orc.tensor_names(cfg):
        a, b = g_o[off:off + r * c], g_t[off:off + r * c]
        assert np.max(np.abs(a - b)) <= 1e-9 * max(np.max(np.abs(b)), 1e-30), name
