"""Seeded synthetic inputs for the mHC seam block.

This module is the only code that the oracle side and the GPU side share.  It
draws random numbers and rounds them to bf16; it holds none of the method's
arithmetic (no projection, gate, Sinkhorn, collapse or norm).  Gate inputs for
the post stage are therefore returned as raw logits; callers turn them into
gates with the oracle (tests) or with the library's own pre stage (benchmark).

Recipe (numpy ``default_rng(seed)``, PCG64): draw in float32 in the order x,
fn, bias, pre_in, norm_weight, outlier rows; round each float32 once to bf16,
nearest-even.  Outlier tokens are scaled x100 before that single rounding.
Shapes: n = 4 residual streams, hidden C = 5120, K = 4C, 24 logits.
"""
from __future__ import annotations

import math

import numpy as np

NS = 4
HIDDEN = 5120
NLOG = 24


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (inputs are finite)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    out = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (out >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, std=1.0, chunk=1 << 24):
    """float32 normal draws, generated in chunks to bound temporary memory."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return out.reshape(shape)


def seam_weights(seed: int, K: int):
    """fn [K,24] ~ N(0, 0.02), bias [24] ~ N(0, 0.1), alpha = 1 (float32)."""
    rng = np.random.default_rng(seed)
    fn = _normal(rng, (K, NLOG), 0.02)
    bias = _normal(rng, (NLOG,), 0.1)
    alpha = np.ones(3, dtype=np.float32)
    return fn, bias, alpha


def pre_inputs(T: int, seed: int = 0, C: int = HIDDEN, delayed: bool = False,
               norm: bool = False, outlier_frac: float = 0.0):
    """Inputs of a pre seam (configs: T=8 no norm; T=128 delayed+norm; T=16384
    delayed+norm with 1% outlier rows).  Returns a dict of numpy arrays; x and
    norm_weight are bf16 bit patterns (uint16)."""
    K = NS * C
    rng = np.random.default_rng(seed)
    x32 = _normal(rng, (T, NS, C))
    fn = _normal(rng, (K, NLOG), 0.02)
    bias = _normal(rng, (NLOG,), 0.1)
    alpha = np.ones(3, dtype=np.float32)
    pre_in = rng.uniform(0.0, 1.0, size=(T, NS)).astype(np.float32) if delayed else None
    w = f32_to_bf16_bits(1.0 + _normal(rng, (C,), 0.1)) if norm else None
    outliers = np.zeros(0, dtype=np.int64)
    if outlier_frac > 0 and T > 0:
        n_out = int(math.ceil(outlier_frac * T))
        outliers = np.sort(rng.choice(T, size=n_out, replace=False))
        x32[outliers] *= np.float32(100.0)
    x = f32_to_bf16_bits(x32)
    del x32
    return dict(x=x, fn=fn, bias=bias, alpha=alpha, pre_in=pre_in, norm_weight=w,
                outliers=outliers, eps=1e-6, iters=20)


def post_inputs(T: int, seed: int = 3, C: int = HIDDEN):
    """Inputs of a post seam: y [T,C] and x [T,4,C] ~ N(0,1) bf16; raw gate
    logits: post_logit [T,4] ~ N(0,1) (post = 2*sigmoid) and comb_logit [T,4,4]
    ~ N(0,1) (comb = Sinkhorn of exp)."""
    rng = np.random.default_rng(seed)
    y = f32_to_bf16_bits(_normal(rng, (T, C)))
    x = f32_to_bf16_bits(_normal(rng, (T, NS, C)))
    post_logit = rng.standard_normal((T, NS), dtype=np.float32)
    comb_logit = rng.standard_normal((T, NS, NS), dtype=np.float32)
    return dict(y=y, x=x, post_logit=post_logit, comb_logit=comb_logit)


def entry_inputs(T: int, seed: int = 999, C: int = HIDDEN, norm: bool = True):
    """Model-entry seam: h [T,C] ~ N(0,1) bf16, fn_e [C,24] ~ N(0,0.02), bias, alpha,
    norm_weight = 1 + N(0, 0.1)."""
    rng = np.random.default_rng(seed)
    h = f32_to_bf16_bits(_normal(rng, (T, C)))
    fn = _normal(rng, (C, NLOG), 0.02)
    bias = _normal(rng, (NLOG,), 0.1)
    alpha = np.ones(3, dtype=np.float32)
    w = f32_to_bf16_bits(1.0 + _normal(rng, (C,), 0.1)) if norm else None
    return dict(h=h, fn=fn, bias=bias, alpha=alpha, norm_weight=w, eps=1e-6, iters=20)


def sweep_seam_weights(k: int, C: int = HIDDEN, norm: bool = True):
    """Weights of seam k of the 80-seam sweep: seed 1000 + k."""
    rng = np.random.default_rng(1000 + k)
    fn = _normal(rng, (NS * C, NLOG), 0.02)
    bias = _normal(rng, (NLOG,), 0.1)
    alpha = np.ones(3, dtype=np.float32)
    w = f32_to_bf16_bits(1.0 + _normal(rng, (C,), 0.1)) if norm else None
    return dict(fn=fn, bias=bias, alpha=alpha, norm_weight=w)
