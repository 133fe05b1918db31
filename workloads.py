"""Seeded synthetic inputs for the delta-rule / Kalman-Delta scans.

This module only draws numbers: it holds none of the recurrence's arithmetic.
Both sides of every parity check (the HIP library and the fp64 oracle) take
their inputs from here, so they see bit-identical values.

Recipe (all draws from numpy's PCG64, float32 unless stated):
  * q, k, v ~ N(0, 1); k is L2-normalised over d_k in float32 (the state path
    assumes unit keys: "A Hippocampus for Linear Attention", sec. 3.4); q too
    when ``normalize_q`` is set (the tiny fp32 check).
  * For bf16 workloads q, k, v are then rounded to bfloat16 (round to nearest
    even); the arrays returned here hold those rounded values in float32, which
    is exact, and ``bf16_bits`` gives the raw 16-bit patterns.
  * alpha = exp(-softplus(x) * 0.1), beta = sigmoid(y), r = softplus(z) with
    x, y, z ~ N(0, 1), computed in float64 and stored as float32.
  * Draw order inside one generator: q, k, v, x, y, z.

Named workloads (shapes are [B, H, L, d]):
  tiny     B=1,  H=1,  L=64,    d=16,  fp32, q and k normalised, beta ~ U(0,1), alpha = 1
  gated    B=4,  H=16, L=4096,  d=128, bf16, chunk 64
  kdn_diag gated + r per token, diagonal covariance prior 1.0, sigma^2 = 1
  long     B=1,  H=32, L=65536, d=128, bf16, chunk 64
  decode   B=256, H=32, d=128, fp32, 512 single-token steps, top-64 cache
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "WORKLOADS", "bf16_round", "bf16_bits", "scan_inputs", "named_scan_inputs",
    "decode_step_inputs", "DECODE_SEED",
]

DECODE_SEED = 5000

WORKLOADS = {
    "tiny": dict(B=1, H=1, L=64, dk=16, dv=16, dtype="f32", chunk=16, seed=1000,
                 normalize_q=True, alpha="one", beta="uniform", with_r=False),
    "gated": dict(B=4, H=16, L=4096, dk=128, dv=128, dtype="bf16", chunk=64, seed=2000,
                  normalize_q=False, alpha="gated", beta="sigmoid", with_r=False),
    "kdn_diag": dict(B=4, H=16, L=4096, dk=128, dv=128, dtype="bf16", chunk=64, seed=3000,
                     normalize_q=False, alpha="gated", beta="sigmoid", with_r=True,
                     cov_init=1.0, q_noise_var=1.0),
    "long": dict(B=1, H=32, L=65536, dk=128, dv=128, dtype="bf16", chunk=64, seed=4000,
                 normalize_q=False, alpha="gated", beta="sigmoid", with_r=False),
    "decode": dict(B=256, H=32, dk=128, dv=128, steps=512, w=64, dtype="f32"),
}


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    out = rounded.view(np.float32).copy()
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.float32("nan")
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bfloat16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not bfloat16-representable; call bf16_round first")
    return (u >> 16).astype(np.uint16)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def scan_inputs(B: int, H: int, L: int, dk: int, dv: int, seed, dtype: str = "bf16",
                normalize_q: bool = False, alpha: str = "gated", beta: str = "sigmoid",
                with_r: bool = False) -> dict:
    """Draw one scan workload. Returns float32 arrays q, k, v ([B,H,L,d]) and
    alpha, beta, r ([B,H,L]; r is None unless ``with_r``)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.standard_normal((B, H, L, dk), dtype=np.float32)
    k = rng.standard_normal((B, H, L, dk), dtype=np.float32)
    v = rng.standard_normal((B, H, L, dv), dtype=np.float32)
    k = _unit_rows(k)
    if normalize_q:
        q = _unit_rows(q)
    if dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    elif dtype != "f32":
        raise ValueError(dtype)
    x = rng.standard_normal((B, H, L))
    y = rng.standard_normal((B, H, L))
    z = rng.standard_normal((B, H, L))
    if alpha == "gated":
        a = np.exp(-_softplus(x) * 0.1).astype(np.float32)
    elif alpha == "one":
        a = np.ones((B, H, L), np.float32)
    else:
        raise ValueError(alpha)
    if beta == "sigmoid":
        b = (1.0 / (1.0 + np.exp(-y))).astype(np.float32)
    elif beta == "uniform":
        b = rng.random((B, H, L)).astype(np.float32)
    else:
        raise ValueError(beta)
    r = _softplus(z).astype(np.float32) if with_r else None
    return dict(q=q, k=k, v=v, alpha=a, beta=b, r=r)


def named_scan_inputs(name: str, **override) -> dict:
    """Inputs for one of the named scan workloads (optionally with smaller shapes)."""
    cfg = dict(WORKLOADS[name])
    cfg.update(override)
    return scan_inputs(cfg["B"], cfg["H"], cfg["L"], cfg["dk"], cfg["dv"], cfg["seed"],
                       dtype=cfg["dtype"], normalize_q=cfg["normalize_q"], alpha=cfg["alpha"],
                       beta=cfg["beta"], with_r=cfg["with_r"])


def decode_step_inputs(step: int, B: int, H: int, dk: int, dv: int,
                       seed: int = DECODE_SEED) -> dict:
    """Per-step decode inputs from generator PCG64([seed, step]): fp32 q, k (unit), v
    ([B,H,d]) and alpha, beta ([B,H]) with the gated workload's distributions."""
    rng = np.random.Generator(np.random.PCG64([seed, step]))
    q = rng.standard_normal((B, H, dk), dtype=np.float32)
    k = _unit_rows(rng.standard_normal((B, H, dk), dtype=np.float32))
    v = rng.standard_normal((B, H, dv), dtype=np.float32)
    x = rng.standard_normal((B, H))
    y = rng.standard_normal((B, H))
    a = np.exp(-_softplus(x) * 0.1).astype(np.float32)
    b = (1.0 / (1.0 + np.exp(-y))).astype(np.float32)
    return dict(q=q, k=k, v=v, alpha=a, beta=b)
