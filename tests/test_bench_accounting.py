"""The benchmark's FLOP accounting (the MFU numerator), pinned to independent figures.

Primary count: 6 FLOPs per matmul parameter per token (forward 2, backward 4; the LM head included,
the embedding gather excluded) plus the causal attention products, 6 L H D (T + 1) per token (the
forward's two products over the T(T+1)/2 causal pairs of a sequence, the backward's four).  The
alternate is the pages' own rule of thumb, FLOPs per token ~ 6 x N_params ("nanochat 项目深度分析"
§6.1, worked example 6 x 1.6e9 = 9.6e9)."""
import json
import os

import pytest

import bench
from decoder_only_transformer_block_amd.inputs import WORKLOADS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_depth12_count_by_hand():
    # per layer: qkv 768 x (6 + 2 x 6) x 128, out-proj 6 x 128 x 768, MLP 2 x 768 x 3072; lm_head 32768 x 768
    per_layer = 768 * 18 * 128 + 768 * 768 + 2 * 768 * 3072
    assert per_layer == 7_077_888
    n_mm = 12 * per_layer + 32768 * 768
    assert n_mm == 110_100_480
    attn = 6 * 12 * 6 * 128 * 2049
    assert bench.flops_per_token(WORKLOADS["d12"]) == 6 * n_mm + attn == 773_904_384


@pytest.mark.parametrize("name,mflops", [("tiny", 2.85), ("small", 31.46), ("d12", 773.90), ("d20", 2980.7),
                                          ("d24", 4681.1)])
def test_per_config_values(name, mflops):
    # the per-configuration table of the measurement plan (MFLOP per token, rounded as printed there)
    assert bench.flops_per_token(WORKLOADS[name]) / 1e6 == pytest.approx(mflops, abs=0.051)


def test_attention_term_counts_causal_pairs():
    # 6 L H D (T + 1) per token = 3 (fwd + bwd) x 2 D flops x L H x T (T + 1) / 2 pairs, over T tokens
    w = WORKLOADS["d20"]
    no_attn = w.with_(seq_len=0)
    per_token_attn = bench.flops_per_token(w) - bench.flops_per_token(no_attn) + 6 * w.n_layer * w.n_head * w.head_dim
    pairs = w.seq_len * (w.seq_len + 1) / 2
    assert per_token_attn * w.seq_len == pytest.approx(3 * 2 * 2 * w.head_dim * w.n_layer * w.n_head * pairs)


def test_pages_six_n_rule():
    g = json.load(open(os.path.join(GOLDEN, "flops_per_token.json")))
    assert bench.six_n_flops_per_token(g["params"]) == pytest.approx(g["flops_per_token"])
    # the same rule over the depth-12 model's 135.27 M parameters (embedding included): 811.6 MFLOP/token
    w = WORKLOADS["d12"]
    n_total = 2 * w.vocab_size * w.n_embd + w.n_layer * (
        w.n_embd * (w.n_head + 2 * w.n_kv_head) * w.head_dim + w.n_head * w.head_dim * w.n_embd
        + 2 * w.n_embd * w.mlp_dim)
    assert n_total == 135_266_304
    assert bench.six_n_flops_per_token(n_total) / 1e6 == pytest.approx(811.6, abs=0.05)


def test_mfu_definition():
    w = WORKLOADS["d12"]
    # 50.72 TFLOP per 65536-token step; at 40 % of 2516.6 TFLOP/s a step takes 50.4 ms
    step = bench.flops_per_token(w) * w.n_tokens
    assert step / 1e12 == pytest.approx(50.72, abs=0.01)
    assert bench.mfu(w, 50.4e-3) == pytest.approx(0.40, abs=0.001)


def test_clock_sampler_reads_the_starred_sclk_and_power(tmp_path):
    """The sampler takes the starred line of pp_dpm_sclk (a fixed level or the intermediate 'S:' state) and
    power1_input in microwatts, skips cards of other vendors, and rebases MFU to the observed clock."""
    import time
    other = tmp_path / "card0" / "device"
    other.mkdir(parents=True)
    (other / "vendor").write_text("0x10de\n")
    (other / "pp_dpm_sclk").write_text("0: 100Mhz *\n")
    dev = tmp_path / "card1" / "device"
    (dev / "hwmon" / "hwmon3").mkdir(parents=True)
    (dev / "vendor").write_text("0x1002\n")
    (dev / "pp_dpm_sclk").write_text("S: 2000Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    (dev / "hwmon" / "hwmon3" / "power1_input").write_text("1250000000\n")
    c = bench.ClockSampler(str(tmp_path))
    with c:
        time.sleep(0.15)
    out = c.summary(0.3)
    assert out["samples"] >= 2
    assert out["sclk_mhz_mean"] == 2000.0 and out["power_w_mean"] == 1250.0
    assert out["mfu_at_observed_clock"] == round(0.3 * 2400 / 2000, 4)
    assert bench.ClockSampler(str(tmp_path / "none")).summary(0.3) is None
