"""ncgpt_bind_static: the step on the library's own per-GPU scratch array (no device allocation by the
library) gives exactly the results of the same step on a caller-allocated workspace (ncgpt_bind).  Two
calls in a row, the second with a smaller input, so the second runs on the array the first left dirty."""
import ctypes as ct

import numpy as np
import pytest
import torch

from decoder_only_transformer_block_amd import ncgpt
from decoder_only_transformer_block_amd.inputs import WORKLOADS
from gpu_util import make_inputs, say

pytestmark = pytest.mark.gpu


def step(w, dtype, static, ids, tg, params):
    cfg = ncgpt.Config.from_workload(w)
    m = ncgpt.Model(cfg, dtype, static_scratch=static)
    assert (m.workspace is None) == static
    assert m.workspace_bytes <= ncgpt.STATIC_SCRATCH_BYTES
    p = torch.from_numpy(params).cuda()
    g = torch.full_like(p, float("nan"))            # every gradient element must be written
    m.forward(torch.from_numpy(ids.reshape(-1)).cuda(), p)
    loss = m.loss(torch.from_numpy(tg.reshape(-1)).cuda())
    m.backward(g)
    m.check()
    lr = m.probe("loss_rows").cpu().numpy()
    out = loss.item(), g.cpu().numpy(), lr
    return m, out


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_static_scratch_matches_workspace(dtype):
    big = WORKLOADS["small"].with_(name="small_b2", batch=2)
    small = WORKLOADS["small"].with_(name="small_b1_t128", batch=1, seq_len=128)
    keep = []
    for w in (big, small):
        ids, tg, params = make_inputs(w)
        say(f"[gpu] {w.name} {dtype}: workspace step")
        m_ref, (l_ref, g_ref, lr_ref) = step(w, dtype, False, ids, tg, params)
        say(f"[gpu] {w.name} {dtype}: static-scratch step")
        m_st, (l_st, g_st, lr_st) = step(w, dtype, True, ids, tg, params)
        say(f"  loss workspace {l_ref:.7f} static {l_st:.7f}")
        assert np.isfinite(g_st).all()
        # same kernels in the same order on the same inputs: bitwise equal
        assert l_st == l_ref
        assert np.array_equal(g_st, g_ref)
        assert np.array_equal(lr_st, lr_ref)
        keep.append(m_st)
    # binding the second context took the array over: the first one's calls are refused until rebound
    first = keep[0]
    ids = torch.zeros(first.n_tokens, dtype=torch.int32, device="cuda")
    params = torch.zeros(first.n_params, dtype=torch.float32, device="cuda")
    with pytest.raises(ncgpt.NcgptError) as e:
        first.forward(ids, params)
    assert e.value.status == ncgpt.ESTATE


def test_static_scratch_rejects_oversized_workspace():
    w = WORKLOADS["small"]          # 8 x 256 tokens, vocab 8192: about 125 MiB in bf16
    cfg = ncgpt.Config.from_workload(w)
    ctx = ct.c_void_p()
    L = ncgpt.lib()
    assert L.ncgpt_create(ct.byref(cfg._c()), ncgpt.BF16, ct.byref(ctx)) == ncgpt.OK
    n = ct.c_size_t()
    L.ncgpt_workspace_size(ctx, ct.byref(n))
    assert n.value > ncgpt.STATIC_SCRATCH_BYTES
    assert L.ncgpt_bind_static(ctx, None) == ncgpt.ENOMEM
    msg = L.ncgpt_last_error(ctx).decode()
    assert str(n.value) in msg and str(ncgpt.STATIC_SCRATCH_BYTES) in msg
    assert L.ncgpt_forward(ctx, ct.c_void_p(16), ct.c_void_p(16)) == ncgpt.ESTATE   # nothing was bound
    L.ncgpt_destroy(ctx)
