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


def flops_per_token(w):
    """Algorithmic FLOPs of one token's forward + backward: 6 per matmul
    parameter (lm_head included, the embedding gather excluded) plus the
    causal attention products, 6 * L * H * D * (T + 1)."""
    n_mm = w.n_layer * (w.n_embd * (w.n_head + 2 * w.n_kv_head) * w.head_dim + w.n_head * w.head_dim * w.n_embd
                        + 2 * w.n_embd * w.mlp_dim) + w.vocab_size * w.n_embd
    return 6.0 * n_mm + 6.0 * w.n_layer * w.n_head * w.head_dim * (w.seq_len + 1)


def cpu_baseline(w):
    """The CPU oracle (fp64, OpenMP) on one sequence of the workload's length
    (same model, same sequence length, batch 1): forward + loss + backward,
    timed on this host."""
    import oracle as orc
    from decoder_only_transformer_block_amd.inputs import init_params, split_stream, token_stream
    ws = w.with_(batch=1)
    cfg = orc.OracleConfig(ws.n_layer, ws.n_embd, ws.n_head, ws.n_kv_head, ws.head_dim, ws.mlp_dim, ws.vocab_size,
                           ws.batch, ws.seq_len)
    ids, tg = split_stream(token_stream(ws.vocab_size, 1, ws.seq_len, ws.tokens, 1))
    params = init_params(orc.num_params(cfg), seed=0)
    orc.lib()
    t0 = time.perf_counter()
    orc.grad(cfg, ids, tg, params)
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    cores = min(cores, len(os.sched_getaffinity(0)))
    return {"value": round(ws.seq_len / dt, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{w.name} model, 1 sequence x {ws.seq_len} tokens (1/{w.batch} of a step), "
                      f"forward+loss+backward in fp64, {dt:.1f} s"}


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
    ap.add_argument("--dtype", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernels", action="store_true", help="print the per-kernel table to stderr")
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
        m.backward(grads)

    for _ in range(args.warmup):
        step()
    m.check()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    m.check()
    ms = (t1 - t0) * 1e3 / args.steps
    tok_s = w.n_tokens / (ms / 1e3)
    fpt = flops_per_token(w)
    step_flops = fpt * w.n_tokens
    mfu = step_flops / (ms / 1e3) / (PEAK_BF16_TFLOPS * 1e12)

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
        "dtype": "bf16" if dtype == "bf16" else "f32",
        "data": "synthetic",
        "mfu": round(mfu, 4),
        "flops_per_token": fpt,
        "config": {"workload": f"{w.name}: depth {w.n_layer}, n_embd {w.n_embd}, {w.n_head}x{w.head_dim} heads, "
                               f"{w.n_kv_head} kv heads, MLP {w.mlp_dim}, vocab {w.vocab_size}, "
                               f"{w.tokens} tokens", "global_batch": w.batch, "seq_len": w.seq_len,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
