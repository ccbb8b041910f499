"""Seeded synthetic inputs for the greedy verify round.

This module produces the bytes that both the CPU oracle and the HIP path consume:
quantized heads, hidden rows, token contexts and forced drafts.  It holds no step of
the verify method itself (no dequantization, no matmul, no argmax, no acceptance, no
drafting).  The one piece of arithmetic here, turning an fp32 weight draw into int8 codes
with per-block-32 fp16 absmax scales, is input preparation: on the pages it happens once,
offline, when the model bundle is exported ("Quantization on the GPU delegate" on the
pipelined-engine page: linear per-block-32 int8, absmax symmetric for big-vocab heads).

Every generator is a pure function of its seed.  Large draws are split into fixed-size
row chunks, each with its own child ``SeedSequence``, so the bytes do not depend on the
number of worker threads.
"""
from __future__ import annotations

import hashlib
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

SEED_BASE = 20261202
BLOCK = 32                 # quantization block length along the hidden axis
ROWS_PER_CHUNK = 4096      # fixed chunking of weight draws (part of the seed recipe)
W_STD = 0.02               # head / projection weights are N(0, 0.02) before quantization


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# ----------------------------------------------------------------------------------------
# seeds
# ----------------------------------------------------------------------------------------
@dataclass(frozen=True)
class Streams:
    """Child seed sequences of one configuration, spawned in a fixed order."""
    weights: np.random.SeedSequence
    h_last: np.random.SeedSequence
    hidden: np.random.SeedSequence
    context: np.random.SeedSequence
    drafts: np.random.SeedSequence


def streams(config_id: int, seed_base: int = SEED_BASE) -> Streams:
    ss = np.random.SeedSequence(seed_base + int(config_id))
    w, hl, hd, ctx, dr = ss.spawn(5)
    return Streams(w, hl, hd, ctx, dr)


# ----------------------------------------------------------------------------------------
# quantized weights
# ----------------------------------------------------------------------------------------
def quantize_q8b32(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-block-32 absmax symmetric int8 quantization of fp32 rows ``w[R, H]``.

    scale = fp16(max|w| / 127) rounded to nearest-even; q = clamp(rint(w / scale), -127, 127)
    with half-to-even rounding, computed in fp64; an all-zero block gets scale 0 and q = 0.
    Returns ``q`` int8 ``[R, H]`` and ``scale`` fp16 ``[R, H/32]``.
    """
    w = np.asarray(w, dtype=np.float32)
    R, H = w.shape
    if H % BLOCK:
        raise ValueError(f"H={H} is not a multiple of {BLOCK}")
    blocks = w.reshape(R, H // BLOCK, BLOCK)
    m = np.abs(blocks).max(axis=2)
    s16 = (m.astype(np.float64) / 127.0).astype(np.float16)
    sf = s16.astype(np.float64)[..., None]
    safe = np.where(sf > 0, sf, 1.0)
    qf = np.where(sf > 0, np.rint(blocks.astype(np.float64) / safe), 0.0)
    q = np.clip(qf, -127, 127).astype(np.int8)
    return q.reshape(R, H), s16


def quantize_q4b32(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-block-32 absmax symmetric int4 quantization of fp32 rows ``w[R, H]``.

    scale = fp16(max|w| / 7) rounded to nearest-even; q = clamp(rint(w / scale), -7, 7) with
    half-to-even rounding, computed in fp64; an all-zero block gets scale 0 and q = 0.
    Packed 16 bytes per block, offset binary u = q + 8: byte i of block b holds element
    32b + i in its low nibble and element 32b + 16 + i in its high nibble.
    Returns ``packed`` uint8 ``[R, H/2]`` and ``scale`` fp16 ``[R, H/32]``.
    """
    w = np.asarray(w, dtype=np.float32)
    R, H = w.shape
    if H % BLOCK:
        raise ValueError(f"H={H} is not a multiple of {BLOCK}")
    blocks = w.reshape(R, H // BLOCK, BLOCK)
    m = np.abs(blocks).max(axis=2)
    s16 = (m.astype(np.float64) / 7.0).astype(np.float16)
    sf = s16.astype(np.float64)[..., None]
    safe = np.where(sf > 0, sf, 1.0)
    qf = np.where(sf > 0, np.rint(blocks.astype(np.float64) / safe), 0.0)
    u = (np.clip(qf, -7, 7) + 8).astype(np.uint8)                     # [R, H/32, 32], 1 .. 15
    packed = (u[:, :, :16] | (u[:, :, 16:] << 4)).astype(np.uint8)   # [R, H/32, 16]
    return packed.reshape(R, H // 2), s16


def quantized_head_q4(seq: np.random.SeedSequence, V: int, H: int,
                      std: float = W_STD, workers: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Draw fp32 N(0, std) weights ``[V, H]`` chunk by chunk (the same draws as
    ``quantized_head``) and quantize them to packed int4 (q4b32)."""
    if H % BLOCK:
        raise ValueError(f"H={H} is not a multiple of {BLOCK}")
    n_chunks = (V + ROWS_PER_CHUNK - 1) // ROWS_PER_CHUNK
    children = seq.spawn(n_chunks)
    q = np.empty((V, H // 2), dtype=np.uint8)
    s = np.empty((V, H // BLOCK), dtype=np.float16)

    def work(c: int) -> None:
        r0 = c * ROWS_PER_CHUNK
        r1 = min(V, r0 + ROWS_PER_CHUNK)
        rng = np.random.default_rng(children[c])
        w = rng.standard_normal((r1 - r0, H), dtype=np.float32) * np.float32(std)
        q[r0:r1], s[r0:r1] = quantize_q4b32(w)

    with ThreadPoolExecutor(workers or _workers()) as ex:
        list(ex.map(work, range(n_chunks)))
    return q, s


def quantized_head(seq: np.random.SeedSequence, V: int, H: int,
                   std: float = W_STD, workers: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Draw fp32 N(0, std) weights ``[V, H]`` chunk by chunk and quantize them (q8b32)."""
    if H % BLOCK:
        raise ValueError(f"H={H} is not a multiple of {BLOCK}")
    n_chunks = (V + ROWS_PER_CHUNK - 1) // ROWS_PER_CHUNK
    children = seq.spawn(n_chunks)
    q = np.empty((V, H), dtype=np.int8)
    s = np.empty((V, H // BLOCK), dtype=np.float16)

    def work(c: int) -> None:
        r0 = c * ROWS_PER_CHUNK
        r1 = min(V, r0 + ROWS_PER_CHUNK)
        rng = np.random.default_rng(children[c])
        w = rng.standard_normal((r1 - r0, H), dtype=np.float32) * np.float32(std)
        q[r0:r1], s[r0:r1] = quantize_q8b32(w)

    with ThreadPoolExecutor(workers or _workers()) as ex:
        list(ex.map(work, range(n_chunks)))
    return q, s


# ----------------------------------------------------------------------------------------
# hidden rows
# ----------------------------------------------------------------------------------------
def fp16_normal(seq_or_rng, shape) -> np.ndarray:
    """fp16(N(0,1)) draws: an fp32 standard normal rounded to nearest-even fp16."""
    rng = seq_or_rng if isinstance(seq_or_rng, np.random.Generator) else np.random.default_rng(seq_or_rng)
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


# ----------------------------------------------------------------------------------------
# token contexts
# ----------------------------------------------------------------------------------------
def uniform_context_with_span(rng: np.random.Generator, n: int, V: int,
                              span_len: int = 12, repeats: int = 16) -> tuple[np.ndarray, np.ndarray, list[int]]:
    """``n`` uniform ids in [0, V) with one uniform ``span_len`` span written at ``repeats``
    non-overlapping random offsets.  Returns (context, span, offsets)."""
    if repeats * span_len > n:
        raise ValueError("span repeats do not fit")
    ctx = rng.integers(0, V, size=n, dtype=np.int64).astype(np.int32)
    span = rng.integers(0, V, size=span_len, dtype=np.int64).astype(np.int32)
    # non-overlapping offsets: choose the gaps between the repeats
    free = n - repeats * span_len
    cuts = np.sort(rng.integers(0, free + 1, size=repeats))
    offsets = [int(cuts[i] + i * span_len) for i in range(repeats)]
    for o in offsets:
        ctx[o:o + span_len] = span
    return ctx, span, offsets


def zipf_ids(rng: np.random.Generator, count: int, V: int, a: float = 1.1) -> np.ndarray:
    """``count`` Zipf(a) ranks rejection-resampled to <= V, returned as ids rank-1."""
    out = np.empty(count, dtype=np.int64)
    filled = 0
    while filled < count:
        need = count - filled
        draw = rng.zipf(a, size=max(2 * need, 64))
        ok = draw[draw <= V]
        take = min(need, ok.size)
        out[filled:filled + take] = ok[:take]
        filled += take
    return (out - 1).astype(np.int32)


def zipf_context_with_copies(rng: np.random.Generator, n: int, V: int, copy_rate: float,
                             a: float = 1.1, span_min: int = 8, span_max: int = 32,
                             warmup: int = 64) -> tuple[np.ndarray, float]:
    """Build ``n`` ids left to right: while the copied fraction is below ``copy_rate`` (and at
    least ``warmup`` ids exist) copy a span of U{span_min..span_max} ids from a uniformly random
    earlier start, else append one Zipf(a) id.  Returns (context, realized copied fraction)."""
    ctx = np.empty(n, dtype=np.int32)
    length = 0
    copied = 0
    pool = zipf_ids(rng, n, V, a)
    pool_i = 0
    while length < n:
        if length >= warmup and copied < copy_rate * length:
            ell = int(rng.integers(span_min, span_max + 1))
            ell = min(ell, n - length, length)
            start = int(rng.integers(0, length - ell + 1))
            ctx[length:length + ell] = ctx[start:start + ell]
            length += ell
            copied += ell
        else:
            if pool_i >= pool.size:
                pool = zipf_ids(rng, n, V, a)
                pool_i = 0
            ctx[length] = pool[pool_i]
            pool_i += 1
            length += 1
    return ctx, copied / n


# ----------------------------------------------------------------------------------------
# forced drafts (every accept length exercised)
# ----------------------------------------------------------------------------------------
def forced_drafts(rng: np.random.Generator, argmax_rows: np.ndarray, K: int, V: int,
                  j: int | None = None) -> tuple[np.ndarray, int]:
    """Drafts d_1..d_K that equal the given argmax rows for the first ``j`` positions and then
    miss: d_i = a[i-1] for i <= j, d_{j+1} = (a[j] + 1 + r) mod V with r in [0, V-2], the rest
    uniform in [0, V).  ``argmax_rows`` holds a[0..K]; ``j`` ~ U{0..K} unless given."""
    a = np.asarray(argmax_rows, dtype=np.int64)
    if a.shape[0] != K + 1:
        raise ValueError("argmax_rows must hold K+1 entries")
    if j is None:
        j = int(rng.integers(0, K + 1))
    d = rng.integers(0, V, size=K, dtype=np.int64)
    d[:j] = a[:j]
    if j < K:
        r = int(rng.integers(0, V - 1))
        d[j] = (a[j] + 1 + r) % V
    return d.astype(np.int32), j


# ----------------------------------------------------------------------------------------
# token-dependent synthetic "models" (hidden row as a function of the token prefix)
# ----------------------------------------------------------------------------------------
class MarkovHidden:
    """h(prefix) = E[last token] with ``E`` a seeded fp16 N(0,1) table ``[V, H]``."""

    def __init__(self, seq_or_rng, V: int, H: int):
        self.table = fp16_normal(seq_or_rng, (V, H))

    def __call__(self, prefix) -> np.ndarray:
        return self.table[int(prefix[-1])]


class HashHidden:
    """h(prefix) = fp16(N(0,1)) seeded by a hash of the whole prefix."""

    def __init__(self, salt: int, H: int):
        self.salt = int(salt)
        self.H = H

    def __call__(self, prefix) -> np.ndarray:
        b = np.asarray(prefix, dtype=np.int32).tobytes()
        digest = hashlib.blake2b(b, digest_size=8, key=self.salt.to_bytes(8, "little")).digest()
        rng = np.random.default_rng(int.from_bytes(digest, "little"))
        return rng.standard_normal(self.H, dtype=np.float32).astype(np.float16)


class ScriptHidden:
    """A stand-in target whose greedy continuation is a fixed script ``T`` (ids): the hidden
    row at position p (the row after a prefix of p + 1 ids) is sign(q[T[p + 1]]) as fp16, the
    sign pattern of the head's own code row of the scripted id.  That row's logit on its own
    id sums |code| x scale over the whole hidden axis, every other id's logit is a signed random
    walk, so the argmax is the scripted id by a wide margin, and greedy decoding of the script
    reproduces it.  Rows depend only on the position; rows after a rejected draft are never
    used by an accept, so this is a valid target for speculative decoding.  With T built like
    the contexts (Zipf ids and copied spans), the n-gram drafter's acceptance rate lies
    strictly between 0 and 1.

    ``rows()`` gives all rows [len(T) - 1, H]: row p belongs to position p."""

    def __init__(self, q: np.ndarray, script: np.ndarray):
        self.q = q
        self.script = np.asarray(script, dtype=np.int64)

    def rows(self) -> np.ndarray:
        return np.sign(self.q[self.script[1:]]).astype(np.float16)

    def __call__(self, prefix) -> np.ndarray:
        return np.sign(self.q[self.script[len(prefix)]]).astype(np.float16)
