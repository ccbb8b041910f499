"""Oracle for the weight-bound dense stack in front of the head: RMSNorm -> gate/up -> SiLU*mul
-> down -> residual, all projections int8 per-block-32 absmax.  TEST INFRASTRUCTURE ONLY.

Pages: the tuning-stack page's byte model (decode is bound by the bytes every forward
reads) and its axis-4 micro-optimisations (fused RMSNorm and SwiGLU); the pipelined-engine
page's quantization section (linear per-block-32 int8).  The pages do not define the block
further; readings (weightless RMSNorm, eps 1e-6, residual add, fp16 activations between the
projections, final weightless RMSNorm before the head) keep the 36-layer stack finite.

Parity pins: rmsnorm against closed forms (constant rows, scale invariance), silu against
special values, the projections against exact rational brute force on tiny shapes.
"""
from __future__ import annotations

import numpy as np

from .verify import dequantize

EPS = 1e-6


def rmsnorm_fp16(x: np.ndarray, eps: float = EPS) -> np.ndarray:
    """fp16(x / sqrt(mean(x^2) + eps)) per row, computed in fp64, no learned gain."""
    x = np.asarray(x).astype(np.float64)
    r = np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return (x / r).astype(np.float16)


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x) in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def linear_q8b32(q: np.ndarray, scale: np.ndarray, x16: np.ndarray) -> np.ndarray:
    """y[s, n] = sum_k x[s, k] * Wd[n, k] in fp64 (same contraction as the head)."""
    wd = dequantize(q, scale)
    x = np.atleast_2d(np.asarray(x16).astype(np.float64))
    return np.stack([wd @ x[s] for s in range(x.shape[0])])


def mlp_block(x16: np.ndarray, layer, eps: float = EPS, return_parts: bool = False):
    """One block: n = rmsnorm(x); m = fp16(silu(n Wg^T) * (n Wu^T)); x' = fp16(x + m Wd^T).

    ``layer`` = ((qg, sg), (qu, su), (qd, sd)).
    """
    (qg, sg), (qu, su), (qd, sd) = layer
    n = rmsnorm_fp16(x16, eps)
    g = linear_q8b32(qg, sg, n)
    u = linear_q8b32(qu, su, n)
    m = (silu(g) * u).astype(np.float16)
    y = linear_q8b32(qd, sd, m)
    xn = (np.asarray(x16).astype(np.float64) + y).astype(np.float16)
    if return_parts:
        return xn, {"n": n, "g": g, "u": u, "m": m, "y": y}
    return xn


def stack_forward(x16: np.ndarray, layers, eps: float = EPS) -> np.ndarray:
    """All blocks in order, then the final weightless RMSNorm: the head's fp16 input rows."""
    x = np.asarray(x16, dtype=np.float16)
    for layer in layers:
        x = mlp_block(x, layer, eps)
    return rmsnorm_fp16(x, eps)
