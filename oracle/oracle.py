"""ctypes binding of oracle/liboracle.so -- TEST INFRASTRUCTURE, NOT PRODUCT CODE.

Plain fp64 CPU definition of one nanochat-style GPT training step.  What each
function computes, and which page passage it follows, is stated in
ncgpt_oracle.c.  Arrays are numpy; every floating-point output is float64.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this module.
"""
import ctypes as ct
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

WQ, WK, WV, WO, WFC, WPROJ = range(6)
LAYER_ACTS = ["xn1", "rstd1", "qkv", "rstdq", "rstdk", "y", "lse_att", "xmid", "xn2", "rstd2", "a", "xout"]


class _Cfg(ct.Structure):
    _fields_ = [(n, ct.c_int32) for n in ("n_layer", "n_embd", "n_head", "n_kv_head", "head_dim", "mlp_dim",
                                           "vocab_size", "batch", "seq_len")] + \
               [("rope_base", ct.c_double), ("norm_eps", ct.c_double), ("logit_softcap", ct.c_double),
                ("embed_norm", ct.c_int32)]


class _Layout(ct.Structure):
    _fields_ = [("x0", ct.c_int64), ("layer0", ct.c_int64), ("layer_stride", ct.c_int64),
                ("per_layer", ct.c_int64 * len(LAYER_ACTS)), ("xf", ct.c_int64), ("rstdf", ct.c_int64),
                ("lse", ct.c_int64), ("loss_rows", ct.c_int64), ("x0n", ct.c_int64), ("rstd0", ct.c_int64),
                ("total", ct.c_int64)]


class _Optim(ct.Structure):
    _fields_ = [("matrix_lr", ct.c_double), ("embedding_lr", ct.c_double), ("unembedding_lr", ct.c_double),
                ("muon_momentum", ct.c_double), ("muon_nesterov", ct.c_int32), ("ns_steps", ct.c_int32),
                ("ns_a", ct.c_double), ("ns_b", ct.c_double), ("ns_c", ct.c_double), ("ns_eps", ct.c_double),
                ("adam_beta1", ct.c_double), ("adam_beta2", ct.c_double), ("adam_eps", ct.c_double),
                ("weight_decay", ct.c_double)]


@dataclass(frozen=True)
class OptimConfig:
    """Hyper-parameters of the optimizer step.  Learning rates: "nanochat 项目深度分析" §2.2 / §4.2.  The
    Newton-Schulz constants and the momentum form: the published Muon description.  The AdamW moments'
    constants are not on the pages (PyTorch's AdamW defaults)."""
    matrix_lr: float = 0.02
    embedding_lr: float = 0.2
    unembedding_lr: float = 0.004
    muon_momentum: float = 0.95
    muon_nesterov: int = 1
    ns_steps: int = 5
    ns_a: float = 3.4445
    ns_b: float = -4.7750
    ns_c: float = 2.0315
    ns_eps: float = 1e-7
    adam_beta1: float = 0.9
    adam_beta2: float = 0.999
    adam_eps: float = 1e-8
    weight_decay: float = 0.0

    def _c(self):
        return _Optim(self.matrix_lr, self.embedding_lr, self.unembedding_lr, self.muon_momentum,
                      self.muon_nesterov, self.ns_steps, self.ns_a, self.ns_b, self.ns_c, self.ns_eps,
                      self.adam_beta1, self.adam_beta2, self.adam_eps, self.weight_decay)


@dataclass(frozen=True)
class OracleConfig:
    n_layer: int
    n_embd: int
    n_head: int
    n_kv_head: int
    head_dim: int
    mlp_dim: int
    vocab_size: int
    batch: int
    seq_len: int
    rope_base: float = 10000.0
    norm_eps: float = 2.0 ** -23
    logit_softcap: float = 0.0   # block variant: logits z -> c tanh(z / c) when c > 0
    embed_norm: int = 0          # block variant: RMSNorm right after the embedding

    def _c(self):
        return _Cfg(self.n_layer, self.n_embd, self.n_head, self.n_kv_head, self.head_dim, self.mlp_dim,
                    self.vocab_size, self.batch, self.seq_len, self.rope_base, self.norm_eps, self.logit_softcap,
                    self.embed_norm)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build()
        L = ct.CDLL(_LIB_PATH)
        P = ct.POINTER
        d, i32, i64 = P(ct.c_double), P(ct.c_int32), P(ct.c_int64)
        L.orc_num_params.argtypes = [P(_Cfg)]
        L.orc_num_params.restype = ct.c_int64
        L.orc_param_slice.argtypes = [P(_Cfg), ct.c_int, ct.c_int, i64, i64, i64]
        L.orc_acts_size.argtypes = [P(_Cfg)]
        L.orc_acts_size.restype = ct.c_int64
        L.orc_get_acts_layout.argtypes = [P(_Cfg), P(_Layout)]
        L.orc_linear_fwd.argtypes = [d, d, ct.c_int64, ct.c_int64, ct.c_int64, d]
        L.orc_linear_bwd.argtypes = [d, d, d, ct.c_int64, ct.c_int64, ct.c_int64, d, d, ct.c_int]
        L.orc_rmsnorm_fwd.argtypes = [d, ct.c_int64, ct.c_int64, ct.c_double, d, d]
        L.orc_rmsnorm_bwd.argtypes = [d, d, d, ct.c_int64, ct.c_int64, d, ct.c_int]
        L.orc_rope.argtypes = [d, ct.c_int64, ct.c_int64, ct.c_int64, ct.c_int64, ct.c_double, ct.c_int]
        L.orc_attention_fwd.argtypes = [d, d, d, ct.c_int64, ct.c_int64, ct.c_int64, ct.c_int64, ct.c_int64, d, d]
        L.orc_attention_bwd.argtypes = [d, d, d, d, ct.c_int64, ct.c_int64, ct.c_int64, ct.c_int64, ct.c_int64,
                                        d, d, d]
        L.orc_cross_entropy_fwd.argtypes = [d, i32, ct.c_int64, ct.c_int64, d, d, d]
        L.orc_cross_entropy_fwd.restype = ct.c_int64
        L.orc_cross_entropy_bwd.argtypes = [d, i32, ct.c_int64, ct.c_int64, ct.c_int64, ct.c_double, d]
        L.orc_forward.argtypes = [P(_Cfg), i32, i32, P(ct.c_float), d, d]
        L.orc_forward.restype = ct.c_int64
        L.orc_grad.argtypes = [P(_Cfg), i32, i32, P(ct.c_float), ct.c_double, d, d]
        L.orc_grad.restype = ct.c_int64
        L.orc_forward_f64.argtypes = [P(_Cfg), i32, i32, d, d, d]
        L.orc_forward_f64.restype = ct.c_int64
        L.orc_grad_f64.argtypes = [P(_Cfg), i32, i32, d, ct.c_double, d, d]
        L.orc_grad_f64.restype = ct.c_int64
        L.orc_newton_schulz.argtypes = [d, ct.c_int64, ct.c_int64, ct.c_int, ct.c_double, ct.c_double, ct.c_double,
                                        ct.c_double, d]
        L.orc_muon_update.argtypes = [d, d, d, ct.c_int64, ct.c_int64, ct.c_double, ct.c_double, ct.c_int,
                                      ct.c_double, ct.c_int, ct.c_double, ct.c_double, ct.c_double, ct.c_double]
        L.orc_adamw_update.argtypes = [d, d, d, d, ct.c_int64, ct.c_int64, ct.c_double, ct.c_double, ct.c_double,
                                       ct.c_double, ct.c_double]
        L.orc_optim_state_size.argtypes = [P(_Cfg)]
        L.orc_optim_state_size.restype = ct.c_int64
        L.orc_optim_step.argtypes = [P(_Cfg), d, d, d, ct.c_int64, P(_Optim)]
        _lib = L
    return _lib


def _f64(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(ct.POINTER(ct.c_double))


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(ct.POINTER(ct.c_int32))


def _out(shape):
    a = np.empty(shape, dtype=np.float64)
    return a, a.ctypes.data_as(ct.POINTER(ct.c_double))


# ---------------------------------------------------------------- packing

def num_params(cfg: OracleConfig) -> int:
    return int(lib().orc_num_params(ct.byref(cfg._c())))


def param_slice(cfg: OracleConfig, layer: int, which: int):
    """(offset, rows, cols) of a packed tensor.  layer=-1: which 0 = wte, 1 = lm_head."""
    o, r, c = ct.c_int64(), ct.c_int64(), ct.c_int64()
    if lib().orc_param_slice(ct.byref(cfg._c()), layer, which, ct.byref(o), ct.byref(r), ct.byref(c)) != 0:
        raise ValueError("bad tensor selector")
    return o.value, r.value, c.value


def tensor_names(cfg: OracleConfig):
    """[(name, offset, rows, cols)] for every packed tensor, in packing order."""
    out = [("wte",) + param_slice(cfg, -1, 0)]
    names = ["wq", "wk", "wv", "wo", "wfc", "wproj"]
    for l in range(cfg.n_layer):
        for w, nm in enumerate(names):
            out.append((f"h{l}.{nm}",) + param_slice(cfg, l, w))
    out.append(("lm_head",) + param_slice(cfg, -1, 1))
    return out


# ---------------------------------------------------------------- primitives

def linear(x, W):
    x, px = _f64(x)
    W, pw = _f64(W)
    rows, inn = x.shape
    out = W.shape[0]
    y, py = _out((rows, out))
    lib().orc_linear_fwd(px, pw, rows, inn, out, py)
    return y


def linear_bwd(x, W, dy):
    x, px = _f64(x)
    W, pw = _f64(W)
    dy, pd = _f64(dy)
    rows, inn = x.shape
    out = W.shape[0]
    dx, pdx = _out((rows, inn))
    dW, pdW = _out((out, inn))
    lib().orc_linear_bwd(px, pw, pd, rows, inn, out, pdx, pdW, 0)
    return dx, dW


def rmsnorm(x, eps=2.0 ** -23):
    x, px = _f64(x)
    n = x.shape[-1]
    rows = x.size // n
    y, py = _out(x.shape)
    r, pr = _out(x.shape[:-1])
    lib().orc_rmsnorm_fwd(px, rows, n, eps, py, pr)
    return y, r


def rmsnorm_bwd(y, rstd, dy):
    y, py = _f64(y)
    rstd, pr = _f64(rstd)
    dy, pd = _f64(dy)
    n = y.shape[-1]
    dx, pdx = _out(y.shape)
    lib().orc_rmsnorm_bwd(py, pr, pd, y.size // n, n, pdx, 0)
    return dx


def rope(x, base=10000.0, inverse=False):
    """x [B, T, nh, D]; returns a rotated copy."""
    x = np.array(x, dtype=np.float64, copy=True, order="C")
    B, T, nh, D = x.shape
    lib().orc_rope(x.ctypes.data_as(ct.POINTER(ct.c_double)), B, T, nh, D, base, 1 if inverse else 0)
    return x


def attention(q, k, v):
    """q [B,T,H,D], k/v [B,T,Hkv,D] -> (o [B,T,H,D], lse [B,H,T])."""
    q, pq = _f64(q)
    k, pk = _f64(k)
    v, pv = _f64(v)
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    o, po = _out(q.shape)
    lse, pl = _out((B, H, T))
    lib().orc_attention_fwd(pq, pk, pv, B, T, H, Hkv, D, po, pl)
    return o, lse


def attention_bwd(q, k, v, do):
    q, pq = _f64(q)
    k, pk = _f64(k)
    v, pv = _f64(v)
    do, pdo = _f64(do)
    B, T, H, D = q.shape
    Hkv = k.shape[2]
    dq, pdq = _out(q.shape)
    dk, pdk = _out(k.shape)
    dv, pdv = _out(v.shape)
    lib().orc_attention_bwd(pq, pk, pv, pdo, B, T, H, Hkv, D, pdq, pdk, pdv)
    return dq, dk, dv


def cross_entropy(z, targets):
    """-> (loss, lse [rows], loss_rows [rows], valid)."""
    z, pz = _f64(z)
    t, pt = _i32(targets)
    rows, V = z.shape
    lse, pl = _out(rows)
    lr, plr = _out(rows)
    loss = ct.c_double()
    valid = lib().orc_cross_entropy_fwd(pz, pt, rows, V, pl, plr, ct.byref(loss))
    return loss.value, lse, lr, int(valid)


def cross_entropy_bwd(z, targets, grad_scale=1.0):
    z, pz = _f64(z)
    t, pt = _i32(targets)
    rows, V = z.shape
    valid = int((t >= 0).sum())
    dz, pd = _out(z.shape)
    lib().orc_cross_entropy_bwd(pz, pt, rows, V, valid, grad_scale, pd)
    return dz


# ---------------------------------------------------------------- whole model

def _params(params):
    """fp32 master weights go to the fp32 entry points (widened exactly inside);
    float64 arrays go to the fp64 ones (used by the finite-difference pins)."""
    if np.asarray(params).dtype == np.float64:
        p = np.ascontiguousarray(params)
        return p, p.ctypes.data_as(ct.POINTER(ct.c_double)), True
    p = np.ascontiguousarray(params, dtype=np.float32)
    return p, p.ctypes.data_as(ct.POINTER(ct.c_float)), False


def acts_layout(cfg: OracleConfig):
    lay = _Layout()
    lib().orc_get_acts_layout(ct.byref(cfg._c()), ct.byref(lay))
    return lay


def forward(cfg: OracleConfig, ids, targets, params):
    """Forward + loss (params fp32, or float64 for the fp64 entry).  Returns (loss, acts) where acts is a dict of float64
    arrays: x0, per-layer lists (see LAYER_ACTS), xf, rstdf, lse, loss_rows."""
    ids, pi = _i32(np.asarray(ids).reshape(-1))
    targets, pt = _i32(np.asarray(targets).reshape(-1))
    p, pp, f64 = _params(params)
    if p.size != num_params(cfg):
        raise ValueError("params size mismatch")
    lay = acts_layout(cfg)
    buf, pb = _out(lay.total)
    loss = ct.c_double()
    fn = lib().orc_forward_f64 if f64 else lib().orc_forward
    valid = fn(ct.byref(cfg._c()), pi, pt, pp, pb, ct.byref(loss))
    if valid < 0:
        raise ValueError("oracle rejected the inputs (bad config or token id)")
    N = cfg.batch * cfg.seq_len
    C, H, Hkv, D, F = cfg.n_embd, cfg.n_head, cfg.n_kv_head, cfg.head_dim, cfg.mlp_dim
    shapes = {"xn1": (N, C), "rstd1": (N,), "qkv": (N, (H + 2 * Hkv) * D), "rstdq": (N, H), "rstdk": (N, Hkv),
              "y": (N, H * D), "lse_att": (cfg.batch, H, cfg.seq_len), "xmid": (N, C), "xn2": (N, C),
              "rstd2": (N,), "a": (N, F), "xout": (N, C)}
    acts = {"x0": buf[lay.x0:lay.x0 + N * C].reshape(N, C), "valid": int(valid)}
    for name in LAYER_ACTS:
        acts[name] = []
    for l in range(cfg.n_layer):
        base = lay.layer0 + l * lay.layer_stride
        for i, name in enumerate(LAYER_ACTS):
            sz = int(np.prod(shapes[name]))
            o = base + lay.per_layer[i]
            acts[name].append(buf[o:o + sz].reshape(shapes[name]))
    acts["xf"] = buf[lay.xf:lay.xf + N * C].reshape(N, C)
    acts["rstdf"] = buf[lay.rstdf:lay.rstdf + N]
    acts["lse"] = buf[lay.lse:lay.lse + N]
    acts["loss_rows"] = buf[lay.loss_rows:lay.loss_rows + N]
    acts["x0n"] = buf[lay.x0n:lay.x0n + N * C].reshape(N, C)
    return loss.value, acts


def grad(cfg: OracleConfig, ids, targets, params, grad_scale=1.0):
    """(loss, grads float64 [P]) with grads = grad_scale * d loss / d params."""
    ids, pi = _i32(np.asarray(ids).reshape(-1))
    targets, pt = _i32(np.asarray(targets).reshape(-1))
    p, pp, f64 = _params(params)
    P = num_params(cfg)
    if p.size != P:
        raise ValueError("params size mismatch")
    g, pg = _out(P)
    loss = ct.c_double()
    fn = lib().orc_grad_f64 if f64 else lib().orc_grad
    valid = fn(ct.byref(cfg._c()), pi, pt, pp, grad_scale, pg, ct.byref(loss))
    if valid < 0:
        raise ValueError("oracle rejected the inputs (bad config or token id)")
    return loss.value, g


# ---------------------------------------------------------------- optimizer step

def newton_schulz(G, steps=5, a=3.4445, b=-4.7750, c=2.0315, eps=1e-7):
    G, pg = _f64(G)
    rows, cols = G.shape
    out, po = _out((rows, cols))
    lib().orc_newton_schulz(pg, rows, cols, steps, a, b, c, eps, po)
    return out


def muon_update(p, g, buf, lr, momentum=0.95, nesterov=True, wd=0.0, steps=5, a=3.4445, b=-4.7750, c=2.0315,
                eps=1e-7):
    """Returns (new p, new buf); inputs are not modified."""
    p = np.array(p, dtype=np.float64, order="C")
    buf = np.array(buf, dtype=np.float64, order="C")
    g, pg = _f64(g)
    rows, cols = p.shape
    lib().orc_muon_update(p.ctypes.data_as(ct.POINTER(ct.c_double)), pg, buf.ctypes.data_as(ct.POINTER(ct.c_double)),
                          rows, cols, lr, momentum, int(nesterov), wd, steps, a, b, c, eps)
    return p, buf


def adamw_update(p, g, m, v, t, lr, b1=0.9, b2=0.999, eps=1e-8, wd=0.0):
    """Returns (new p, new m, new v)."""
    p = np.array(p, dtype=np.float64).ravel()
    m = np.array(m, dtype=np.float64).ravel()
    v = np.array(v, dtype=np.float64).ravel()
    g, pg = _f64(np.ravel(g))
    D = ct.POINTER(ct.c_double)
    lib().orc_adamw_update(p.ctypes.data_as(D), pg, m.ctypes.data_as(D), v.ctypes.data_as(D), p.size, t, lr, b1, b2,
                           eps, wd)
    return p, m, v


def optim_state_size(cfg: OracleConfig) -> int:
    return int(lib().orc_optim_state_size(ct.byref(cfg._c())))


def optim_step(cfg: OracleConfig, params, grads, state, t, opt: OptimConfig = OptimConfig()):
    """One optimizer step over packed parameters.  Returns (new params, new state) as float64."""
    p = np.array(params, dtype=np.float64)
    st = np.array(state, dtype=np.float64)
    g, pg = _f64(grads)
    D = ct.POINTER(ct.c_double)
    lib().orc_optim_step(ct.byref(cfg._c()), p.ctypes.data_as(D), pg, st.ctypes.data_as(D), t, ct.byref(opt._c()))
    return p, st


# ---------------------------------------------------------------- decode

def last_logits(cfg: OracleConfig, ids, params):
    """Next-token logits at the last position of each sequence of ids [B, t]: the causal forward over the
    whole prefix (a KV-cache decode step must equal it), then the final-norm row times lm_head^T (a numpy
    matmul).  float64 [B, V]."""
    ids = np.asarray(ids)
    B, t = ids.shape
    c = OracleConfig(cfg.n_layer, cfg.n_embd, cfg.n_head, cfg.n_kv_head, cfg.head_dim, cfg.mlp_dim, cfg.vocab_size,
                     B, t, cfg.rope_base, cfg.norm_eps, cfg.logit_softcap, cfg.embed_norm)
    _, acts = forward(c, ids, ids, params)
    xf = acts["xf"].reshape(B, t, cfg.n_embd)[:, -1]
    off, r, k = param_slice(c, -1, 1)
    W = np.asarray(params, dtype=np.float64)[off:off + r * k].reshape(r, k)
    z = xf @ W.T
    return cfg.logit_softcap * np.tanh(z / cfg.logit_softcap) if cfg.logit_softcap > 0 else z
