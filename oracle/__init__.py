"""fp64 CPU oracle for the gated delta rule (Kimi Delta Attention).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``gated_delta_rule_08_amd``) never imports it, and the two share no code: the
oracle is the plain sequential recurrence in ``kda_oracle.c`` (see the header
of that file for the passages of the pages each step follows), built with gcc.

Every function here takes numpy arrays, upcasts them to float64 (bf16 -> fp64
and fp32 -> fp64 are exact) and calls the C recurrence.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")

MODE_DELTA = 0       # gated delta rule (KDA / GDN / DeltaNet)
MODE_ADDITIVE = 1    # delta term disabled: gated linear attention

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.kda_oracle_run.argtypes = [ctypes.c_int] * 5 + [ctypes.POINTER(ctypes.c_int32)] + \
            [dp] * 8 + [ctypes.c_int]
        lib.kda_oracle_run.restype = ctypes.c_int
        lib.kda_oracle_bwd.argtypes = [ctypes.c_int] * 5 + [ctypes.POINTER(ctypes.c_int32)] + \
            [dp] * 14 + [ctypes.c_int]
        lib.kda_oracle_bwd.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    try:
        import torch  # tests hand over torch CPU tensors as well
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def run(q, k, v, g, beta, cu_seqlens=None, s0=None, mode: int = MODE_DELTA,
        nthreads: int | None = None):
    """Sequential recurrence over packed sequences.

    q, k, g: [T, H, dk]; v: [T, H, dv]; beta: [T, H]; cu_seqlens: [N+1] int
    (default: one sequence of length T); s0: [N, H, dk, dv] or None (zero state).
    Returns (o [T, H, dv], s_final [N, H, dk, dv]) as float64 arrays.
    """
    lib = _load()
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (T, H, dk) and g.shape == (T, H, dk)
    assert v.shape == (T, H, dv) and beta.shape == (T, H)
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int32)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    N = len(cu) - 1
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    s0 = _f64(s0)
    if s0 is not None:
        assert s0.shape == (N, H, dk, dv)
    o = np.zeros((T, H, dv), dtype=np.float64)
    sf = np.zeros((N, H, dk, dv), dtype=np.float64)
    if nthreads is None:
        nthreads = min(16, os.cpu_count() or 1)
    rc = lib.kda_oracle_run(int(mode), H, dk, dv, N,
                            cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
                            _ptr(o), _ptr(sf), int(nthreads))
    if rc != 0:
        raise RuntimeError("kda_oracle_run failed")
    return o, sf


def run_bwd(q, k, v, g, beta, d_o, cu_seqlens=None, s0=None, ds_final=None,
            mode: int = MODE_DELTA, nthreads: int | None = None):
    """Gradients of a scalar loss through the recurrence (reverse-mode, token by
    token; the derivation is in the header of ``kda_oracle.c``).

    d_o: dL/do [T, H, dv]; ds_final: dL/dS_final [N, H, dk, dv] or None (zero).
    Returns a dict of float64 arrays: dq, dk, dg [T, H, dk], dv [T, H, dv],
    dbeta [T, H], ds0 [N, H, dk, dv] (dL/dS0).
    """
    lib = _load()
    q, k, v, g, beta, d_o = map(_f64, (q, k, v, g, beta, d_o))
    T, H, dk = q.shape
    dv = v.shape[2]
    assert k.shape == (T, H, dk) and g.shape == (T, H, dk)
    assert v.shape == (T, H, dv) and beta.shape == (T, H) and d_o.shape == (T, H, dv)
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int32)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    N = len(cu) - 1
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    s0, ds_final = _f64(s0), _f64(ds_final)
    for a in (s0, ds_final):
        if a is not None:
            assert a.shape == (N, H, dk, dv)
    out = dict(dq=np.zeros((T, H, dk)), dk=np.zeros((T, H, dk)), dv=np.zeros((T, H, dv)),
               dg=np.zeros((T, H, dk)), dbeta=np.zeros((T, H)), ds0=np.zeros((N, H, dk, dv)))
    if nthreads is None:
        nthreads = min(16, os.cpu_count() or 1)
    rc = lib.kda_oracle_bwd(int(mode), H, dk, dv, N,
                            cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
                            _ptr(d_o), _ptr(ds_final), _ptr(out["dq"]), _ptr(out["dk"]),
                            _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]),
                            _ptr(out["ds0"]), int(nthreads))
    if rc != 0:
        raise RuntimeError("kda_oracle_bwd failed")
    return out


def decode(q, k, v, g, beta, s):
    """One token per sequence against the given states.

    q, k, g: [B, H, dk]; v: [B, H, dv]; beta: [B, H]; s: [B, H, dk, dv].
    Returns (o [B, H, dv], s_new [B, H, dk, dv]) in float64.  A decode step is
    the recurrence run for one token with the state as the incoming state.
    """
    q, k, v, g, beta, s = map(_f64, (q, k, v, g, beta, s))
    B = q.shape[0]
    cu = np.arange(B + 1, dtype=np.int32)
    return run(q, k, v, g, beta, cu_seqlens=cu, s0=s)


def prepare_inputs(q_raw, k_raw, gate_logits=None, beta_logits=None, gate_min=-np.inf,
                   gate="channel"):
    """Input preparation from the raw projections, in float64.

    q = normalize(silu(q_raw)), k = normalize(silu(k_raw)) over the key
    dimension of each (token, head) (heqinghuang "From GPT2 to Kimi3,
    Explained", section 09: unit-length queries and keys, F.normalize after
    SiLU; normalize divides by max(norm, 1e-12)); beta = sigmoid(beta logit)
    (same section: write strength in (0, 1)); alpha = sigmoid(gate logit) per
    key channel (engineermaxxing "From GPT-2 to Kimi K3", ch. 06b) and
    g = log(alpha), floored at gate_min (dev.to "From GPT-2 to Kimi K3",
    block 5: the decay parameterisation is bounded for bf16 stability; the
    pages give no value, so the floor is an argument, -inf = none).

    q_raw, k_raw: [..., dk].  gate_logits: [..., dk] (gate="channel"), [...]
    (gate="scalar", broadcast over dk) or None (gate="none": g = 0).
    beta_logits: [...] or None (beta = 1, for the additive mode).
    Returns (q, k, g, beta) in float64, g of shape [..., dk].
    """
    q_raw, k_raw = _f64(q_raw), _f64(k_raw)

    def silu(x):
        return x / (1.0 + np.exp(-x))

    def normalize(x):
        n = np.sqrt((x * x).sum(axis=-1, keepdims=True))
        return x / np.maximum(n, 1e-12)

    def log_sigmoid(x):
        # log(1 / (1 + e^-x)) = min(x, 0) - log1p(e^-|x|): no overflow for any x
        return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))

    q = normalize(silu(q_raw))
    k = normalize(silu(k_raw))
    dk = q.shape[-1]
    if gate == "none":
        g = np.zeros(q.shape)
    else:
        a = _f64(gate_logits)
        if gate == "scalar":
            a = np.repeat(a[..., None], dk, axis=-1)
        g = np.maximum(log_sigmoid(a), gate_min)
    if beta_logits is None:
        beta = np.ones(q.shape[:-1])
    else:
        beta = 1.0 / (1.0 + np.exp(-_f64(beta_logits)))
    return q, k, g, beta


def prepare_inputs_bwd(q_raw, k_raw, gate_logits, beta_logits, gate_min, gate, dq, dk, dg, dbeta):
    """Gradients through prepare_inputs (float64): the chain rule of its four maps.

    dq, dk: dL/dq, dL/dk [..., dk] of the prepared q, k; dg: dL/dg of the
    per-channel log-decay [..., dk] (for gate="scalar" the gate is broadcast, so
    its logit's gradient sums over the channels; unused for gate="none");
    dbeta: dL/dbeta [...] (unused when beta_logits is None).
    normalize(x) = x / max(|x|, 1e-12): d/dx = (I - y y^T) / |x| above the floor,
    I / 1e-12 below it; silu'(z) = s (1 + z (1 - s)) with s = sigmoid(z);
    d log sigmoid(a) / da = sigmoid(-a), zero where the floor gate_min is taken
    (log sigmoid(a) < gate_min); d sigmoid(b) / db = s (1 - s).
    Returns (dq_raw, dk_raw, dgate_logits or None, dbeta_logits or None).
    """
    def sig(x):
        return 1.0 / (1.0 + np.exp(-x))

    def silu_grad(z):
        s_ = sig(z)
        return s_ * (1.0 + z * (1.0 - s_))

    def norm_silu_bwd(z, dy):
        z, dy = _f64(z), _f64(dy)
        x = z * sig(z)
        n = np.sqrt((x * x).sum(axis=-1, keepdims=True))
        above = n > 1e-12
        nn = np.maximum(n, 1e-12)
        y = x / nn
        dx = np.where(above, (dy - y * (y * dy).sum(axis=-1, keepdims=True)) / nn, dy / nn)
        return dx * silu_grad(z)

    dq_raw = norm_silu_bwd(q_raw, dq)
    dk_raw = norm_silu_bwd(k_raw, dk)
    dgl = None
    if gate != "none":
        a = _f64(gate_logits)
        ls = np.minimum(a, 0.0) - np.log1p(np.exp(-np.abs(a)))
        pas = np.where(ls >= gate_min, sig(-a), 0.0)
        dg = _f64(dg)
        dgl = pas * (dg.sum(axis=-1) if gate == "scalar" else dg)
    dbl = None
    if beta_logits is not None:
        s_ = sig(_f64(beta_logits))
        dbl = _f64(dbeta) * s_ * (1.0 - s_)
    return dq_raw, dk_raw, dgl, dbl

