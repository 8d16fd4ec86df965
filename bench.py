"""Training-step throughput of the HIP path on one MI355X.

A step is one forward + loss + backward of the whole block stack over one
batch of synthetic tokens (inputs already resident in HBM).  Prints one JSON
line: tokens/s (whole job), ms/step, MFU against the bf16 dense MFMA peak,
the roofline position of the dominant kernel, and the CPU oracle's
throughput on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload d12] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA, 256 CUs at 2.4 GHz
PEAK_HBM_GBS = 8000.0
ROOT = os.path.dirname(os.path.abspath(__file__))
COPY_MIB = 256              # size of the calibration copy (see copy_calibration)
LOSS_SCALE = 2.0 ** 16      # the fp16 setting's gradient scale (grad_scale of the backward)


def flops_per_token(w):
    """Algorithmic FLOPs of one token's forward + backward: 6 per matmul
    parameter (lm_head included, the embedding gather excluded) plus the
    causal attention products, 6 * L * H * D * (T + 1)."""
    n_mm = w.n_layer * (w.n_embd * (w.n_head + 2 * w.n_kv_head) * w.head_dim + w.n_head * w.head_dim * w.n_embd
                        + 2 * w.n_embd * w.mlp_dim) + w.vocab_size * w.n_embd
    return 6 * n_mm + 6 * w.n_layer * w.n_head * w.head_dim * (w.seq_len + 1)


def six_n_flops_per_token(n_params):
    """The pages' rule of thumb, 6 x N_params FLOPs per token (all parameters, attention ignored); reported
    beside the primary count, not used for the MFU."""
    return 6.0 * n_params


def mfu(w, seconds_per_step):
    """Model FLOPs utilisation of one step of workload w against the bf16 dense MFMA peak."""
    return flops_per_token(w) * w.n_tokens / seconds_per_step / (PEAK_BF16_TFLOPS * 1e12)


def cpu_baseline(w):
    """The CPU oracle (fp64, OpenMP) timed on this host, forward + loss +
    backward: the whole step for workloads of at most 4096 tokens, otherwise
    one sequence of the workload's length (same model, batch 1)."""
    import oracle as orc
    from decoder_only_transformer_block_amd.inputs import init_params, split_stream, token_stream
    ws = w if w.n_tokens <= 4096 else w.with_(batch=1)
    cfg = orc.OracleConfig(ws.n_layer, ws.n_embd, ws.n_head, ws.n_kv_head, ws.head_dim, ws.mlp_dim, ws.vocab_size,
                           ws.batch, ws.seq_len)
    ids, tg = split_stream(token_stream(ws.vocab_size, ws.batch, ws.seq_len, ws.tokens, 1))
    params = init_params(orc.num_params(cfg), seed=0)
    orc.lib()
    t0 = time.perf_counter()
    orc.grad(cfg, ids, tg, params)
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    cores = min(cores, len(os.sched_getaffinity(0)))
    what = (f"the whole step, {ws.batch} x {ws.seq_len} tokens" if ws.batch == w.batch else
            f"1 sequence x {ws.seq_len} tokens (1/{w.batch} of a step)")
    return {"value": round(ws.n_tokens / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{w.name} model, {what}, forward+loss+backward in fp64, {dt:.2f} s"}


class ClockSampler:
    """Mean shader clock and board power over a timed region, read from the GPU's sysfs entries every 20 ms
    by a host thread: the current sclk is the starred line of pp_dpm_sclk, the power hwmon's power1_input
    (microwatts).  Reports None where the entries are absent."""

    def __init__(self, root="/sys/class/drm"):
        import glob
        self.sclk = self.power = None
        for d in sorted(glob.glob(os.path.join(root, "card*", "device"))):
            try:
                with open(os.path.join(d, "vendor")) as f:
                    if f.read().strip() != "0x1002":
                        continue
            except OSError:
                continue
            if os.path.exists(os.path.join(d, "pp_dpm_sclk")):
                self.sclk = os.path.join(d, "pp_dpm_sclk")
                pw = sorted(glob.glob(os.path.join(d, "hwmon", "hwmon*", "power1_input")))
                self.power = pw[0] if pw else None
                break
        self.mhz, self.watts = [], []

    def _read(self):
        try:
            with open(self.sclk) as f:
                for line in f:
                    if line.rstrip().endswith("*"):
                        self.mhz.append(float(line.split(":")[1].strip().split("Mhz")[0].split("MHz")[0]))
            if self.power:
                with open(self.power) as f:
                    self.watts.append(float(f.read()) / 1e6)
        except (OSError, ValueError, IndexError):
            pass

    def __enter__(self):
        import threading
        self._stop = threading.Event()

        def run():
            while not self._stop.wait(0.02):
                self._read()
        self._t = threading.Thread(target=run, daemon=True)
        if self.sclk:
            self._t.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.sclk:
            self._t.join()

    def summary(self, step_mfu):
        if not self.mhz:
            return None
        mhz = sum(self.mhz) / len(self.mhz)
        return {"sclk_mhz_mean": round(mhz, 1), "power_w_mean": round(sum(self.watts) / len(self.watts), 1)
                if self.watts else None, "samples": len(self.mhz),
                "mfu_at_observed_clock": round(step_mfu * 2400.0 / mhz, 4) if mhz > 0 else None}


def copy_calibration(dev):
    """One plain device-to-device copy of COPY_MIB MiB, outside every timed
    region.  Under rocprofv3 --pmc its FETCH_SIZE and WRITE_SIZE readings
    (known to be COPY_MIB MiB each) scale the same counters of the dominant
    kernel into bytes."""
    import torch
    src = torch.ones(COPY_MIB << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def measured_traffic(kernel, workload):
    """HBM-side bytes per launch of `kernel` from the committed rocprofv3
    counter summary profiles/traffic_<kernel>_<workload>.txt, or None when
    there is none or when the kernel's sources changed since it was taken
    (their sha256 is recorded in the summary)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        for src in kv["sources"].split():
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != kv["source_sha256"]:
            return None
        return {"bytes_per_launch": float(kv["traffic_bytes_per_launch"]),
                "fetch_bytes": float(kv["fetch_bytes_per_launch"]), "write_bytes": float(kv["write_bytes_per_launch"]),
                "fetch_factor": float(kv["fetch_factor"]), "write_factor": float(kv["write_factor"]),
                "summary": os.path.relpath(path, ROOT)}
    except (KeyError, ValueError, OSError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="d12")
    ap.add_argument("--dtype", default=None, choices=[None, "bf16", "f16", "f32"],
                    help="compute dtype (default: the workload's); f16 runs with a loss scale of 2^16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fp8", action="store_true",
                    help="forward linears on E4M3 operands with per-row scales (bf16 workloads)")
    ap.add_argument("--lm-head", choices=["stored", "recomputed"], default="stored",
                    help="where the backward's dz comes from: stored logits (default) or a second LM-head GEMM")
    ap.add_argument("--kernels", action="store_true", help="print the per-kernel table to stderr")
    ap.add_argument("--no-optim", action="store_true", help="skip timing the optimizer step")
    ap.add_argument("--no-decode", action="store_true", help="skip timing the KV-cache decode step")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from decoder_only_transformer_block_amd import ncgpt
    from decoder_only_transformer_block_amd.inputs import WORKLOADS, init_params, split_stream, token_stream

    w = WORKLOADS[args.workload]
    dtype = args.dtype or w.dtype
    cfg = ncgpt.Config.from_workload(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    m = ncgpt.Model(cfg, dtype)
    if args.lm_head == "recomputed":
        m.set_lm_head_mode(ncgpt.LOGITS_RECOMPUTED)
    if args.fp8:
        m.set_fp8(True)
    ids, tg = split_stream(token_stream(w.vocab_size, w.batch, w.seq_len, w.tokens, 1))
    ids_d = torch.from_numpy(ids.reshape(-1)).to(dev)
    tg_d = torch.from_numpy(tg.reshape(-1)).to(dev)
    params = torch.from_numpy(init_params(m.n_params, seed=0)).to(dev)
    grads = torch.zeros(m.n_params, dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    copy_calibration(dev)

    def step():
        m.forward(ids_d, params)
        m.loss(tg_d, loss)
        m.backward(grads, grad_scale=LOSS_SCALE if dtype == "f16" else 1.0)

    for _ in range(args.warmup):
        step()
    m.check()
    torch.cuda.synchronize()
    clock = ClockSampler()
    with clock:
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    m.check()
    ms = (t1 - t0) * 1e3 / args.steps
    tok_s = w.n_tokens / (ms / 1e3)
    fpt = flops_per_token(w)
    step_mfu = mfu(w, ms / 1e3)

    # second region of the same K steps with a HIP event pair around every launch
    m.timing(True)
    m.timing_reset()
    torch.cuda.synchronize()
    r0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    r1 = time.perf_counter()
    table = m.timing_read()
    m.timing(False)
    dom = max(table.items(), key=lambda kv: kv[1][1])
    name, (launches, tot_ms, fl, by) = dom
    avg_ms = tot_ms / launches
    if fl > 0:
        achieved = fl / launches / (avg_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "kernel": name, "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    else:
        achieved = by / launches / (avg_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "kernel": name, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    tr = measured_traffic(name, w.name)
    roof.update({"traffic": tr["bytes_per_launch"] if tr else None, "traffic_detail": tr,
                 "algorithmic_bytes_per_launch": by / launches if by else None, "avg_launch_ms": round(avg_ms, 4), "launches_per_step": launches // args.steps,
                 "share_of_step": round(tot_ms / sum(v[1] for v in table.values()), 4),
                 "region_ms_per_step": round((r1 - r0) * 1e3 / args.steps, 3)})
    if args.kernels:
        tot = sum(v[1] for v in table.values())
        print(f"{'kernel':44s} {'n/step':>6s} {'ms/step':>8s} {'share':>6s} {'TF/s':>7s} {'GB/s':>7s}", file=sys.stderr)
        for k, (n, t, f, b) in sorted(table.items(), key=lambda kv: -kv[1][1]):
            print(f"{k:44s} {n // args.steps:6d} {t / args.steps:8.3f} {t / tot:6.1%} "
                  f"{(f / (t / 1e3) / 1e12) if f else 0:7.1f} {(b / (t / 1e3) / 1e9) if b else 0:7.1f}",
                  file=sys.stderr)

    # the optimizer step (Muon + AdamW) that follows the gradients: timed on its own, not part of `value`
    optim = None
    if not args.no_optim:
        st = torch.zeros(ncgpt.optim_state_size(cfg), dtype=torch.float32, device=dev)
        p2 = params.clone()
        m.optim_step(p2, grads, st, 1)
        torch.cuda.synchronize()
        o0 = time.perf_counter()
        for t in range(2, 2 + args.steps):
            m.optim_step(p2, grads, st, t)
        torch.cuda.synchronize()
        o1 = time.perf_counter()
        m.timing(True)
        m.timing_reset()
        m.optim_step(p2, grads, st, 2 + args.steps)
        otab = m.timing_read()
        m.timing(False)
        m.check()
        gemm_fl = sum(v[2] for k, v in otab.items() if k.startswith("gemm"))
        gemm_ms = sum(v[1] for k, v in otab.items() if k.startswith("gemm"))
        optim = {"ms_per_step": round((o1 - o0) * 1e3 / args.steps, 3),
                 "newton_schulz_tflop": round(gemm_fl / 1e12, 3),
                 "newton_schulz_gemm_ms": round(gemm_ms, 3),
                 "newton_schulz_tflops": round(gemm_fl / (gemm_ms / 1e3) / 1e12, 1) if gemm_ms else None}
        if args.kernels:
            print("optimizer step:", file=sys.stderr)
            for k, (n, t_, f, b) in sorted(otab.items(), key=lambda kv: -kv[1][1]):
                print(f"  {k:44s} {n:6d} {t_:8.3f} {(f / (t_ / 1e3) / 1e12) if f else 0:7.1f} "
                      f"{(b / (t_ / 1e3) / 1e9) if b else 0:7.1f}", file=sys.stderr)

    # KV-cache decode at the end of the context: B sequences, one token each, against seq_len - 1 cached positions
    decode = None
    if not args.no_decode:
        cache = m.kv_cache()
        m.forward(ids_d, params)
        m.kv_fill(cache, w.seq_len - 1)
        tok = ids_d.view(w.batch, w.seq_len)[:, -1].contiguous()
        lg = torch.empty(w.batch * w.vocab_size, dtype=torch.float32, device=dev)
        m.decode_step(tok, params, cache, w.seq_len - 1, lg, recast=True)
        torch.cuda.synchronize()
        d0 = time.perf_counter()
        for _ in range(args.steps):
            m.decode_step(tok, params, cache, w.seq_len - 1, lg, recast=False)
        torch.cuda.synchronize()
        d1 = time.perf_counter()
        m.timing(True)
        m.timing_reset()
        m.decode_step(tok, params, cache, w.seq_len - 1, lg, recast=False)
        dtab = m.timing_read()
        m.timing(False)
        m.check()
        att = dtab.get("decode_attn")
        dms = (d1 - d0) * 1e3 / args.steps
        decode = {"ms_per_step": round(dms, 3), "tokens_per_s": round(w.batch / (dms / 1e3), 1),
                  "context": w.seq_len, "batch": w.batch,
                  "attention_ms": round(att[1], 3) if att else None,
                  "attention_gbs": round(att[3] / (att[1] / 1e3) / 1e9, 1) if att else None,
                  "kv_cache_bytes": m.kv_cache_bytes()}
        if args.kernels:
            print("decode step:", file=sys.stderr)
            for k, (n, t_, f, b) in sorted(dtab.items(), key=lambda kv: -kv[1][1]):
                print(f"  {k:44s} {n:6d} {t_:8.3f} {(f / (t_ / 1e3) / 1e12) if f else 0:7.1f} "
                      f"{(b / (t_ / 1e3) / 1e9) if b else 0:7.1f}", file=sys.stderr)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w)
    out = {
        "metric": "train tokens/sec + MFU (fwd+bwd step) on 1 MI355X, depth-12 GPT, T=2048",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8e4m3+bf16" if args.fp8 else "bf16") if dtype == "bf16" else dtype,
        "data": "synthetic",
        "mfu": round(step_mfu, 4),
        "gpu_clock": clock.summary(step_mfu),
        "flops_per_token": fpt,
        "config": {"workload": f"{w.name}: depth {w.n_layer}, n_embd {w.n_embd}, {w.n_head}x{w.head_dim} heads, "
                               f"{w.n_kv_head} kv heads, MLP {w.mlp_dim}, vocab {w.vocab_size}, "
                               f"{w.tokens} tokens", "global_batch": w.batch, "seq_len": w.seq_len,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "optimizer": optim,
        "decode": decode,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
