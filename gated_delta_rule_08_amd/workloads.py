"""Seeded synthetic workloads for the gated delta rule.

This module holds the configurations the library is tested and measured on and
the seeded input generators that serve both the GPU path and the CPU oracle.
It contains none of the method's arithmetic: it only draws random numbers and
shapes them (L2-normalised keys/queries, sigmoid write strengths, log-sigmoid
gates), the way the layer in front of the memory would.

Value recipe (the same for every configuration unless noted):
  q, k ~ N(0, 1), L2-normalised per (token, head) over the key dimension;
  v ~ N(0, 1);
  beta = sigmoid(N(0, 1)), one per (token, head);
  g = log alpha = log sigmoid(x), x ~ N(mu, 1) per (token, head, channel),
      mu = 3 (mu = 4 for the long-context prefill, i.e. slower decay);
  S0 ~ 0.02 * N(0, 1) where a configuration asks for an initial state.
Draw order from numpy's PCG64 with seed = 1000 + configuration index:
sequence lengths (varlen only) -> q -> k -> v -> beta logits -> alpha logits
-> S0.  Arithmetic is float32; q, k, v are then rounded to bf16 (round to
nearest even) for bf16 workloads and kept as float32 values, which are exactly
representable in the I/O dtype.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass(frozen=True)
class Config:
    index: int
    name: str
    kind: str            # "prefill" or "decode"
    num_heads: int
    dk: int
    dv: int
    io_dtype: str        # "fp32" or "bf16"
    chunk: int = 64
    batch: int = 1       # prefill: number of equal-length sequences; decode: batch
    seq_len: int = 0     # prefill: tokens per sequence (fixed-length configs)
    varlen: tuple | None = None   # (num_seqs, min_len, max_len) for packed batches
    alpha_mu: float = 3.0
    with_s0: bool = False
    scalar_gate_heads: tuple = ()  # heads whose gate is one scalar broadcast over dk

    @property
    def description(self) -> str:
        return self.name


CONFIGS = {
    0: Config(0, "tiny_fp32_B1_H2_T64_d16_C16", "prefill", 2, 16, 16, "fp32", chunk=16,
              batch=1, seq_len=64),
    1: Config(1, "prefill_bf16_B1_H16_T4096_d128_C64", "prefill", 16, 128, 128, "bf16",
              chunk=64, batch=1, seq_len=4096),
    2: Config(2, "decode_bf16_B256_H32_d128", "decode", 32, 128, 128, "bf16", batch=256,
              with_s0=True),
    3: Config(3, "prefill_long_bf16_B2_H32_T65536_d128_C64", "prefill", 32, 128, 128, "bf16",
              chunk=64, batch=2, seq_len=65536, alpha_mu=4.0),
    4: Config(4, "varlen_bf16_N64_len128-8192_H16_d128_C64_kda8_gdn8", "prefill", 16, 128, 128,
              "bf16", chunk=64, varlen=(64, 128, 8192), with_s0=True,
              scalar_gate_heads=tuple(range(8, 16))),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    out = rounded.view(np.float32).copy()
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.float32(np.nan)
    return out


def _l2_normalise(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-12))).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _log_sigmoid(x: np.ndarray) -> np.ndarray:
    # log sigmoid(x) = -softplus(-x), computed without overflow
    return (-np.logaddexp(np.float32(0.0), -x)).astype(np.float32)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def seq_lengths(cfg: Config, rng: np.random.Generator | None = None) -> np.ndarray:
    """Per-sequence lengths of a configuration (drawn first for packed batches)."""
    if cfg.varlen is not None:
        if rng is None:
            rng = np.random.Generator(np.random.PCG64(1000 + cfg.index))
        n, lo, hi = cfg.varlen
        return rng.integers(lo, hi + 1, size=n, dtype=np.int64).astype(np.int32)
    return np.full(cfg.batch, cfg.seq_len, dtype=np.int32)


def make_inputs(cfg: Config | int, seed: int | None = None) -> dict:
    """Draw every input of a configuration.

    Prefill returns q, k, g [T, H, dk], v [T, H, dv], beta [T, H], cu_seqlens
    [N+1] (int32) and s0 [N, H, dk, dv] or None.  Decode returns q, k, g
    [B, H, dk], v [B, H, dv], beta [B, H] and the resident states s0
    [B, H, dk, dv].  All float arrays are float32.
    """
    if isinstance(cfg, int):
        cfg = CONFIGS[cfg]
    rng = np.random.Generator(np.random.PCG64(1000 + cfg.index if seed is None else seed))
    H, dk, dv = cfg.num_heads, cfg.dk, cfg.dv
    if cfg.kind == "decode":
        T = cfg.batch
        cu = None
        N = cfg.batch
    else:
        lens = seq_lengths(cfg, rng)
        cu = np.zeros(len(lens) + 1, dtype=np.int32)
        np.cumsum(lens, out=cu[1:])
        T = int(cu[-1])
        N = len(lens)
    q = _l2_normalise(_normal(rng, (T, H, dk)))
    k = _l2_normalise(_normal(rng, (T, H, dk)))
    v = _normal(rng, (T, H, dv))
    if cfg.io_dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    beta = _sigmoid(_normal(rng, (T, H)))
    x = _normal(rng, (T, H, dk))
    x += np.float32(cfg.alpha_mu)
    g = _log_sigmoid(x)
    del x
    for h in cfg.scalar_gate_heads:
        g[:, h, :] = g[:, h, :1]   # one scalar per (token, head), broadcast over channels
    s0 = None
    if cfg.with_s0 or cfg.kind == "decode":
        s0 = (np.float32(0.02) * _normal(rng, (N, H, dk, dv))).astype(np.float32)
    out = dict(q=q, k=k, v=v, g=g, beta=beta, s0=s0, config=cfg)
    if cu is not None:
        out["cu_seqlens"] = cu
    return out


def random_problem(rng: np.random.Generator, T: int, H: int, dk: int, dv: int,
                   alpha_mu: float = 3.0, io_dtype: str = "fp32", unit_keys: bool = True,
                   g_scale: float = 1.0):
    """A small ad-hoc problem with the recipe above (used for edge cases)."""
    q = _normal(rng, (T, H, dk))
    k = _normal(rng, (T, H, dk))
    if unit_keys:
        q, k = _l2_normalise(q), _l2_normalise(k)
    v = _normal(rng, (T, H, dv))
    if io_dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    beta = _sigmoid(_normal(rng, (T, H)))
    x = _normal(rng, (T, H, dk)) * np.float32(g_scale) + np.float32(alpha_mu)
    g = _log_sigmoid(x)
    return dict(q=q, k=k, v=v, g=g, beta=beta)
