"""The C-ABI library loads, exports every function include/ncgpt.h declares,
and its host-side logic (parameter packing, shape validation, workspace plan)
agrees with the oracle's own packing.  No GPU and no kernel launches."""
import ctypes as ct
import os
import re

import pytest

import oracle as orc
from decoder_only_transformer_block_amd import ncgpt
from decoder_only_transformer_block_amd.inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "ncgpt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ncgpt_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    L = ncgpt.lib()
    names = declared_functions()
    assert len(names) >= 24
    for n in names:
        assert hasattr(L, n), n
    assert sorted(ncgpt.EXPORTS) == names


def ocfg(w):
    return orc.OracleConfig(w.n_layer, w.n_embd, w.n_head, w.n_kv_head, w.head_dim, w.mlp_dim, w.vocab_size,
                            w.batch, w.seq_len)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_packing_matches_oracle(name):
    w = WORKLOADS[name]
    cfg = ncgpt.Config.from_workload(w)
    oc = ocfg(w)
    assert ncgpt.num_params(cfg) == orc.num_params(oc)
    for layer, which in [(-1, 0), (-1, 1)] + [(l, k) for l in (0, w.n_layer - 1) for k in range(6)]:
        assert ncgpt.param_slice(cfg, layer, which) == orc.param_slice(oc, layer, which)
    with pytest.raises(ncgpt.NcgptError):
        ncgpt.param_slice(cfg, w.n_layer, 0)
    with pytest.raises(ncgpt.NcgptError):
        ncgpt.param_slice(cfg, -1, 2)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_optim_state_size_matches_oracle(name):
    w = WORKLOADS[name]
    assert ncgpt.optim_state_size(ncgpt.Config.from_workload(w)) == orc.optim_state_size(ocfg(w))


def create(cfg, dtype):
    ctx = ct.c_void_p()
    st = ncgpt.lib().ncgpt_create(ct.byref(cfg._c()), dtype, ct.byref(ctx))
    return st, ctx


def test_create_validates_shapes_and_plans_workspace():
    L = ncgpt.lib()
    base = ncgpt.Config.from_workload(WORKLOADS["small"])
    st, ctx = create(base, ncgpt.BF16)
    assert st == ncgpt.OK
    n = ct.c_size_t()
    assert L.ncgpt_workspace_size(ctx, ct.byref(n)) == ncgpt.OK
    w = WORKLOADS["small"]
    N = w.batch * w.seq_len
    # at least the saved bf16 activations of every layer plus the logits
    per_layer = N * (2 * w.n_embd + (w.n_head + 2 * w.n_kv_head) * w.head_dim + w.n_head * w.head_dim
                     + 2 * w.mlp_dim) * 2
    assert n.value >= w.n_layer * per_layer + N * w.vocab_size * 2
    # calls out of order are rejected on the host, before any device work
    assert L.ncgpt_forward(ctx, ct.c_void_p(16), ct.c_void_p(16)) == ncgpt.ESTATE
    assert b"bind" in L.ncgpt_last_error(ctx)
    assert L.ncgpt_loss(ctx, ct.c_void_p(16), ct.c_void_p(16)) == ncgpt.ESTATE
    assert L.ncgpt_backward(ctx, ct.c_void_p(16), 0, 1.0) == ncgpt.ESTATE
    assert b"bind" in L.ncgpt_last_error(ctx)   # an unbound context is refused before the order check
    L.ncgpt_destroy(ctx)

    bad = [
        (dict(head_dim=96), ncgpt.F32, ncgpt.EUNSUPPORTED),
        (dict(head_dim=64), ncgpt.BF16, ncgpt.EUNSUPPORTED),      # bf16 attention is built for D = 128
        (dict(head_dim=64), ncgpt.F16, ncgpt.EUNSUPPORTED),       # so is the fp16 one
        (dict(seq_len=192), ncgpt.F16, ncgpt.EUNSUPPORTED),
        (dict(n_kv_head=3, n_head=2), ncgpt.BF16, ncgpt.EUNSUPPORTED),
        (dict(n_embd=200), ncgpt.BF16, ncgpt.EUNSUPPORTED),
        (dict(vocab_size=8200), ncgpt.BF16, ncgpt.EUNSUPPORTED),
        (dict(vocab_size=65536 + 64), ncgpt.F32, ncgpt.EUNSUPPORTED),  # the embedding-gradient sort's limit
        (dict(seq_len=192), ncgpt.BF16, ncgpt.EUNSUPPORTED),
        (dict(batch=0), ncgpt.BF16, ncgpt.EINVAL),
        (dict(logit_softcap=-1.0), ncgpt.BF16, ncgpt.EINVAL),
        (dict(logit_softcap=float("inf")), ncgpt.F32, ncgpt.EINVAL),
        (dict(logit_softcap=float("nan")), ncgpt.F32, ncgpt.EINVAL),
        (dict(embed_norm=2), ncgpt.BF16, ncgpt.EINVAL),
    ]
    for kw, dt, want in bad:
        d = dict(base.__dict__)
        d.update(kw)
        st, ctx = create(ncgpt.Config(**d), dt)
        assert st == want, kw
        assert not ctx.value
    st, _ = create(base, 7)
    assert st == ncgpt.EINVAL
    st, ctx = create(base, ncgpt.F16)                                  # fp16 plans like bf16
    assert st == ncgpt.OK
    m16 = ct.c_size_t()
    assert L.ncgpt_workspace_size(ctx, ct.byref(m16)) == ncgpt.OK and m16.value > 0
    assert L.ncgpt_set_fp8(ctx, 1) == ncgpt.EUNSUPPORTED                # fp8 linears are bf16-only
    assert L.ncgpt_set_lm_head_mode(ctx, ncgpt.LOGITS_RECOMPUTED) == ncgpt.OK
    L.ncgpt_destroy(ctx)
    # the block variants: the embedding norm's rstd adds to the plan
    st, ctx = create(ncgpt.Config(**dict(base.__dict__, logit_softcap=15.0, embed_norm=1)), ncgpt.BF16)
    assert st == ncgpt.OK
    m = ct.c_size_t()
    assert L.ncgpt_workspace_size(ctx, ct.byref(m)) == ncgpt.OK
    assert m.value > n.value
    L.ncgpt_destroy(ctx)


def test_fp8_switch_validation():
    L = ncgpt.lib()
    st, ctx = create(ncgpt.Config.from_workload(WORKLOADS["tiny"]), ncgpt.F32)
    assert L.ncgpt_set_fp8(ctx, 1) == ncgpt.EUNSUPPORTED            # bf16 contexts only
    assert L.ncgpt_set_fp8(ctx, 0) == ncgpt.OK
    L.ncgpt_destroy(ctx)
    base = ncgpt.Config.from_workload(WORKLOADS["small"])
    st, ctx = create(base, ncgpt.BF16)
    assert L.ncgpt_set_fp8(ctx, 1) == ncgpt.OK
    assert L.ncgpt_set_fp8(ctx, 2) == ncgpt.EINVAL
    assert L.ncgpt_set_fp8(None, 1) == ncgpt.EINVAL
    L.ncgpt_destroy(ctx)
    st, ctx = create(ncgpt.Config(**dict(base.__dict__, n_embd=192, mlp_dim=768)), ncgpt.BF16)
    assert st == ncgpt.OK
    assert L.ncgpt_set_fp8(ctx, 1) == ncgpt.EUNSUPPORTED            # K = 192 is not a multiple of 128
    L.ncgpt_destroy(ctx)


def test_lm_head_mode_validation():
    L = ncgpt.lib()
    cfg = ncgpt.Config.from_workload(WORKLOADS["tiny"])
    st, ctx = create(cfg, ncgpt.F32)
    assert st == ncgpt.OK
    assert L.ncgpt_set_lm_head_mode(ctx, ncgpt.LOGITS_STORED) == ncgpt.OK
    assert L.ncgpt_set_lm_head_mode(ctx, ncgpt.LOGITS_RECOMPUTED) == ncgpt.EUNSUPPORTED  # bf16 only
    assert L.ncgpt_set_lm_head_mode(ctx, 2) == ncgpt.EINVAL
    L.ncgpt_destroy(ctx)
    st, ctx = create(ncgpt.Config.from_workload(WORKLOADS["small"]), ncgpt.BF16)
    assert L.ncgpt_set_lm_head_mode(ctx, ncgpt.LOGITS_RECOMPUTED) == ncgpt.OK
    assert L.ncgpt_set_lm_head_mode(None, 0) == ncgpt.EINVAL
    L.ncgpt_destroy(ctx)


def test_null_arguments_are_rejected():
    L = ncgpt.lib()
    assert L.ncgpt_num_params(None) == 0
    assert L.ncgpt_create(None, 0, None) == ncgpt.EINVAL
    assert L.ncgpt_check(None) == ncgpt.EINVAL
    L.ncgpt_destroy(None)
