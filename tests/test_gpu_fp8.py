"""GPU tests of the fp8 forward linears (ncgpt_set_fp8): E4M3 operands with per-row scales.

- The fp8 product itself, pinned exactly: the v heads of the qkv projection leave the GEMM unrotated and
  unnormalised, so they equal, up to fp32 summation order and the final bf16 rounding, a numpy emulation of the
  quantiser written from the OCP E4M3 definition (bias 7, 3 mantissa bits, subnormals down to 2^-9, round to
  nearest even): s = amax / 448 per row of the bf16 activation (the xn1 probe) and of the fp32 weight, and
  sum_k q_a q_b s_a s_b.  Bar max|g - o| / max|o| <= 4.5e-3 (the bf16 rounding of the output is up to 2^-8
  relative, measured 2.2-2.8e-3); the unquantised product is 3.6e-2 away, and a truncating rounding, a dropped
  or swapped scale or a wrong byte order lands at 1e-2 to 1e0.
- The whole step against the fp64 oracle (the unquantised model): the method has no fp8 reference, so the bars
  are tolerances.  E4M3 keeps 3 mantissa bits, a relative rounding error up to 2^-4 per operand, which leaves
  about 5 % noise in each product's output element; measured: activations within 0.10-0.17 (max relative), loss
  within 8.4e-4, per-tensor gradient cosine >= 0.962 at depth 12.  Bars: loss 5e-3, activations 0.3, gradient
  cosine 0.95.
- Both LM-head modes agree bit for bit (the recomputation reuses the loss's E4M3 rows); switching fp8 off gives
  the bf16 step bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle as orc
from decoder_only_transformer_block_amd import ncgpt
from decoder_only_transformer_block_amd.inputs import WORKLOADS, Workload
from gpu_util import GpuStep, cosine, make_inputs, maxrel, ocfg, say

GQA3 = Workload("gqa3", 2, 384, 3, 1, 128, 1536, 4160, 3, 128, "bf16", "zipf")
D12P = WORKLOADS["d12"].with_(name="d12_prefix256", batch=1, seq_len=256)


def e4m3(x):
    """Round float32 values (|x| <= 448) to the nearest OCP E4M3 value, ties to even."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    e = np.maximum(np.floor(np.log2(np.maximum(a, 2.0 ** -9))), -6.0)   # subnormals share exponent -6
    quantum = 2.0 ** (e - 3)
    return np.sign(x) * np.round(a / quantum) * quantum                 # numpy rounds half to even


def quant_rows(x):
    """Per-row quantisation as the kernel does it, in float32: inv = 448 / amax, q = E4M3(x inv), s = amax / 448."""
    x = np.asarray(x, np.float32)
    amax = np.max(np.abs(x), axis=1).astype(np.float32)
    inv = np.where(amax > 0, np.float32(448.0) / np.maximum(amax, np.float32(1e-38)), np.float32(0.0)).astype(np.float32)
    q = e4m3((x * inv[:, None]).astype(np.float32))
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    return q, s


def test_e4m3_rounding_reference():
    """CPU: the test-side E4M3 rounding against values the format fixes."""
    # values the format fixes: 448 (largest finite), ties to even (1.0625 -> 1, 17 -> 16), the smallest
    # subnormal 2^-9 and its half-way points
    got = e4m3([448.0, 1.0625, 1.1875, 17.0, 0.1, -3.3, 2.0 ** -9, 2.0 ** -10, 0.75 * 2.0 ** -9, 240.0])
    want = [448.0, 1.0, 1.25, 16.0, 0.1015625, -3.25, 2.0 ** -9, 0.0, 2.0 ** -9, 240.0]
    assert np.array_equal(got, want)


@pytest.mark.gpu
@pytest.mark.parametrize("name", ["small", "gqa3"])
def test_fp8_product_matches_e4m3_emulation(name):
    w = GQA3 if name == "gqa3" else WORKLOADS[name]
    ids, tg, params = make_inputs(w)
    s = GpuStep(w, "bf16", ids, params)
    s.m.set_fp8(True)
    loss, st = s.run(tg, backward=False)
    assert st == ncgpt.OK
    oc = ocfg(w)
    HD, KD, C = w.n_head * w.head_dim, w.n_kv_head * w.head_dim, w.n_embd
    for l in (0, w.n_layer - 1):
        xn1 = s.probe("xn1", l).reshape(-1, C).astype(np.float32)          # bf16 values, exact in fp32
        off, _, _ = orc.param_slice(oc, l, 2)                              # Wv [KD, C]
        wv = params[off:off + KD * C].reshape(KD, C)
        qa, sa = quant_rows(xn1)
        qb, sb = quant_rows(wv)
        want = (qa @ qb.T) * sa[:, None].astype(np.float64) * sb[None, :].astype(np.float64)
        got = s.probe("qkv", l).reshape(-1, HD + 2 * KD)[:, HD + KD:]
        e = np.max(np.abs(got - want)) / np.max(np.abs(want))
        # the same operands without the quantiser: far outside the bar
        plain = xn1.astype(np.float64) @ wv.T.astype(np.float64)
        e_plain = np.max(np.abs(got - plain)) / np.max(np.abs(plain))
        say(f"  layer {l}: fp8 product vs E4M3 emulation {e:.2e}, vs the unquantised product {e_plain:.2e}")
        assert e <= 4.5e-3, (l, e)
        assert e_plain > 5 * e


# small and depth 12 take the E4M3 rows of the norms from the norm kernel itself, gqa3 (n_embd 384) from the
# row quantiser; the last case adds the block variants (soft-cap 0.2 and the embedding norm)
CASES = [("small", WORKLOADS["small"], {}), ("gqa3", GQA3, {}), ("d12_prefix256", D12P, {}),
         ("small_variants", WORKLOADS["small"], dict(logit_softcap=0.2, embed_norm=1))]


@pytest.mark.gpu
@pytest.mark.parametrize("key,w,var", CASES, ids=[c[0] for c in CASES])
def test_fp8_step_close_to_oracle(key, w, var):
    ids, tg, params = make_inputs(w)
    say(f"[oracle] grad {w.name} {var}")
    lo, go = orc.grad(ocfg(w, **var), ids, tg, params)
    _, acts = orc.forward(ocfg(w, **var), ids, tg, params)
    s = GpuStep(w, "bf16", ids, params, **var)
    s.m.set_fp8(True)
    loss, st = s.run(tg)
    assert st == ncgpt.OK
    rel = abs(loss - lo) / abs(lo)
    say(f"  fp8 loss {loss:.6f} oracle {lo:.6f} rel {rel:.2e}")
    assert rel <= 5e-3
    for l in range(w.n_layer):
        for name in ("qkv", "y", "xn2", "act"):
            o = (acts["a"][l] ** 2 if name == "act" else acts[name][l]).reshape(-1)
            e = maxrel(s.probe(name, l), o)
            assert e <= 0.3, (name, l, e)
    cs = [(n, cosine(s.grads_np()[o:o + r * c], go[o:o + r * c])) for n, o, r, c in orc.tensor_names(ocfg(w))]
    say("  lowest gradient cosine " + " ".join(f"{n}={c:.4f}" for n, c in sorted(cs, key=lambda t: t[1])[:4]))
    assert min(c for _, c in cs) >= 0.95


@pytest.mark.gpu
def test_fp8_lm_head_modes_and_switch():
    w = WORKLOADS["small"]
    ids, tg, params = make_inputs(w)
    out = []
    for mode in (ncgpt.LOGITS_STORED, ncgpt.LOGITS_RECOMPUTED):
        s = GpuStep(w, "bf16", ids, params)
        s.m.set_fp8(True)
        s.m.set_lm_head_mode(mode)
        loss, st = s.run(tg)
        assert st == ncgpt.OK
        out.append((loss, s.probe("loss_rows"), s.grads_np()))
        del s
    assert out[0][0] == out[1][0] and np.array_equal(out[0][1], out[1][1]) and np.array_equal(out[0][2], out[1][2])
    # fp8 on, a step, fp8 off: the next step is the bf16 step bit for bit
    s = GpuStep(w, "bf16", ids, params)
    s.m.set_fp8(True)
    s.run(tg)
    s.m.set_fp8(False)
    l_off, _ = s.run(tg)
    g_off = s.grads_np()
    r = GpuStep(w, "bf16", ids, params)
    l_ref, _ = r.run(tg)
    assert l_off == l_ref and np.array_equal(g_off, r.grads_np())
    assert l_off != out[0][0]
