"""Seeded synthetic inputs and the workload shapes.

This module holds no arithmetic of the model: it only draws token streams and
initial weights, so both the HIP path's tests/benchmark and the CPU oracle's
tests feed identical inputs to the two sides.

Workloads (depth, width, heads, vocab, batch x sequence) are the depth-2 to
depth-24 GPT shapes this library is measured on.  Token streams stand in for
the pages' pretraining corpus (ClimbMix / FineWeb-EDU through a trained BPE,
devpress.csdn.net guide §3 and woshipm.com §四): only token frequency touches
the hot path (embedding-gradient collisions, loss values), so the small
shapes draw uniform ids and the full-size ones a truncated Zipf(1.1) over the
vocabulary.  Weights are i.i.d. N(0, 0.02) fp32, the master-weight dtype.
"""
from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    n_layer: int
    n_embd: int
    n_head: int
    n_kv_head: int
    head_dim: int
    mlp_dim: int
    vocab_size: int
    batch: int
    seq_len: int
    dtype: str          # "f32" or "bf16": the compute dtype
    tokens: str         # "uniform" or "zipf"

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    @property
    def n_tokens(self) -> int:
        return self.batch * self.seq_len


WORKLOADS = {
    "tiny": Workload("tiny", 2, 128, 2, 2, 64, 512, 512, 2, 64, "f32", "uniform"),
    "small": Workload("small", 4, 256, 2, 1, 128, 1024, 8192, 8, 256, "bf16", "uniform"),
    "d12": Workload("d12", 12, 768, 6, 6, 128, 3072, 32768, 32, 2048, "bf16", "zipf"),
    "d20": Workload("d20", 20, 1280, 10, 5, 128, 5120, 65536, 16, 2048, "bf16", "zipf"),
    "d24": Workload("d24", 24, 1536, 12, 4, 128, 6144, 65536, 8, 2048, "bf16", "zipf"),
}


def zipf_cdf(vocab_size: int, s: float = 1.1) -> np.ndarray:
    """CDF over ranks 1..V of p_r proportional to r^-s (float64)."""
    r = np.arange(1, vocab_size + 1, dtype=np.float64)
    p = r ** -s
    c = np.cumsum(p)
    return c / c[-1]


def token_stream(vocab_size: int, batch: int, seq_len: int, kind: str, seed: int) -> np.ndarray:
    """int32 [batch, seq_len + 1]: each row is one sequence of T+1 ids.

    kind "uniform": ids uniform in [0, V).  kind "zipf": id = rank - 1 drawn
    by inverse CDF of the truncated Zipf(1.1) law over the V ranks."""
    rng = np.random.Generator(np.random.PCG64(seed))
    shape = (batch, seq_len + 1)
    if kind == "uniform":
        return rng.integers(0, vocab_size, size=shape, dtype=np.int64).astype(np.int32)
    if kind == "zipf":
        u = rng.random(size=shape)
        ids = np.searchsorted(zipf_cdf(vocab_size), u, side="right")
        return np.minimum(ids, vocab_size - 1).astype(np.int32)
    raise ValueError(f"unknown token distribution {kind!r}")


def split_stream(stream: np.ndarray):
    """(inputs [B,T], targets [B,T]): targets are the inputs shifted by one."""
    return np.ascontiguousarray(stream[:, :-1]), np.ascontiguousarray(stream[:, 1:])


def init_params(n_params: int, seed: int = 0, std: float = 0.02) -> np.ndarray:
    """fp32 [P], i.i.d. N(0, std), in packing order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal(n_params, dtype=np.float32) * np.float32(std)


def workload_inputs(w: Workload, seed: int = 1):
    """(inputs, targets) int32 [B, T] for a workload."""
    return split_stream(token_stream(w.vocab_size, w.batch, w.seq_len, w.tokens, seed))
