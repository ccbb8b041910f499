"""Oracle for one greedy verify round: dequantize -> fp64 logits -> argmax -> accept -> propose.

TEST INFRASTRUCTURE ONLY (see the package docstring).  numpy, fp64, no blocking or fusion
beyond what each definition states.

Parity pins (tests/test_oracle_*.py): dequantize+logits against exact rational brute force
and the unit-vector special case; argmax against a brute-force loop and constructed ties;
accept exhaustively over all match masks and against the closed-form E(alpha, K) of the
C-value speedup model; propose_scan against the independent hashtable ``NgramIndex`` and
constructed streams; the round driver against sequential greedy decoding (losslessness)
and the worked accounting of the feasibility page's implementation status.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
PAD = -1


# ----------------------------------------------------------------------------------------
# dequantize + logits
# ----------------------------------------------------------------------------------------
def dequantize(q: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """fp64 weights from int8 codes and per-block-32 fp16 scales.

    Pipelined-engine page, "Quantization on the GPU delegate": the head is linear
    per-block-32 int8 with symmetric absmax scaling, so a weight is its code times the scale
    of its 32-wide block along the hidden axis.  Exact in fp64 (8-bit code x 11-bit scale).
    """
    q = np.asarray(q)
    scale = np.asarray(scale)
    R, H = q.shape
    if H % BLOCK or scale.shape != (R, H // BLOCK):
        raise ValueError("scale must be [rows, H/32]")
    s = np.repeat(scale.astype(np.float64), BLOCK, axis=1)
    return q.astype(np.float64) * s


def dequantize_q4b32(packed: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """fp64 weights from packed int4 codes and per-block-32 fp16 scales.

    Pipelined-engine page, "Quantization on the GPU delegate" (int4 linear per-block-32,
    the class it ships) and "Numerics gating" (QAT q4_0 weights are trained for the
    per-block-32 absmax grid): a weight is its signed 4-bit code times the scale of its
    32-wide block.  Storage: 16 bytes per block; byte i holds element i (low nibble) and
    element i + 16 (high nibble) as offset binary, code = nibble - 8.
    """
    packed = np.asarray(packed, dtype=np.uint8)
    scale = np.asarray(scale)
    R, half = packed.shape
    H = 2 * half
    if H % BLOCK or scale.shape != (R, H // BLOCK):
        raise ValueError("packed must be [rows, H/2] and scale [rows, H/32]")
    by = packed.reshape(R, H // BLOCK, 16).astype(np.int64)
    lo = (by & 0xF) - 8                                   # elements 0 .. 15 of each block
    hi = (by >> 4) - 8                                    # elements 16 .. 31
    codes = np.concatenate([lo, hi], axis=2).reshape(R, H)
    return codes.astype(np.float64) * np.repeat(scale.astype(np.float64), BLOCK, axis=1)


def head_logits_q4b32(packed: np.ndarray, scale: np.ndarray, hidden: np.ndarray, chunk: int = 8192) -> np.ndarray:
    """All-position logits of an int4 per-block-32 head (see ``head_logits``)."""
    h = np.asarray(hidden).astype(np.float64)
    if h.ndim == 1:
        h = h[None, :]
    V = packed.shape[0]
    out = np.empty((h.shape[0], V), dtype=np.float64)
    for r0 in range(0, V, chunk):
        r1 = min(V, r0 + chunk)
        wd = dequantize_q4b32(packed[r0:r1], scale[r0:r1])
        for s in range(h.shape[0]):
            out[s, r0:r1] = wd @ h[s]
    return out


def head_logits(q: np.ndarray, scale: np.ndarray, hidden: np.ndarray, chunk: int = 8192) -> np.ndarray:
    """All-position logits L[s, v] = sum_k hidden[s, k] * Wd[v, k], in fp64.

    Feasibility page, C1 substrate map and the delta: a verify forward yields logits for
    every position of the window; hybrid verify-design page, verify graph: the static
    S=K+1 window carries all-position logits.  Here only the head matmul is modelled.
    The vocabulary is processed in row chunks only to bound memory; each row s is a
    matrix-vector product, so its value does not depend on how many rows are verified.
    """
    h = np.asarray(hidden).astype(np.float64)
    if h.ndim == 1:
        h = h[None, :]
    V = q.shape[0]
    out = np.empty((h.shape[0], V), dtype=np.float64)
    for r0 in range(0, V, chunk):
        r1 = min(V, r0 + chunk)
        wd = dequantize(q[r0:r1], scale[r0:r1])
        for s in range(h.shape[0]):
            out[s, r0:r1] = wd @ h[s]
    return out


# ----------------------------------------------------------------------------------------
# argmax
# ----------------------------------------------------------------------------------------
def argmax_lowest(L: np.ndarray) -> np.ndarray:
    """Per-position greedy token: the largest logit, the lowest vocabulary index on ties.

    Feasibility page, the delta: a batched argmax sampler reduces [K, vocab] to K ids.  The
    pages do not say how ties break; the lowest index is taken (numpy's first maximum).
    -0.0 and +0.0 compare equal.
    """
    L = np.atleast_2d(L)
    return np.argmax(L, axis=1).astype(np.int64)


def top2_gap(L: np.ndarray) -> np.ndarray:
    """top1 - top2 logit per row (0 when the maximum is attained twice; +inf for a single
    candidate, which has no runner-up to tie with)."""
    L = np.atleast_2d(L)
    if L.shape[1] < 2:
        return np.full(L.shape[0], np.inf)
    part = np.partition(L, L.shape[1] - 2, axis=1)
    return part[:, -1] - part[:, -2]


def admissible_sets(L: np.ndarray, tol: float = 1e-3) -> list[np.ndarray]:
    """Ids whose logit is within ``tol`` of the row maximum.

    Pipelined-engine page, numerics gating: a top-1 flip where the oracle's top-2 margin is
    below a floor is a knife-edge tie, not a failure.  With the 1e-3 floor a compared
    implementation may return any id of this set on a row whose gap is below 1e-3.
    """
    L = np.atleast_2d(L)
    mx = L.max(axis=1, keepdims=True)
    return [np.nonzero(row >= m - tol)[0] for row, m in zip(L, mx[:, 0])]


# ----------------------------------------------------------------------------------------
# accept (greedy, fused a0, correction/bonus unified)
# ----------------------------------------------------------------------------------------
def accept_length(argmax_rows, drafts) -> int:
    """Number of accepted drafts j.

    Feasibility page, the delta and the control-logic proof: draft d_i is accepted iff it
    equals the greedy token predicted for its position and every earlier draft was
    accepted.  With the fused window [a0, d_1..d_K], row i-1 predicts d_i, so
    j = max{i : d_m == argmax_rows[m-1] for all m <= i}.  A pad (-1) never matches.
    """
    a = [int(x) for x in argmax_rows]
    d = [int(x) for x in drafts]
    if len(a) != len(d) + 1:
        raise ValueError("argmax_rows must have K+1 entries for K drafts")
    j = 0
    while j < len(d) and d[j] != PAD and d[j] == a[j]:
        j += 1
    return j


def accept(argmax_rows, drafts) -> tuple[int, list[int]]:
    """(j, tokens to append): the accepted drafts d_1..d_j, then argmax_rows[j].

    Hybrid verify-design page, hybrid state discipline: the row after the last accepted
    token is the next round's pending token (the correction when a draft missed, the bonus
    when all K were accepted).  Feasibility page, implementation status: each round commits
    what was accepted and advances; tokens per round = 1 + j.
    """
    j = accept_length(argmax_rows, drafts)
    return j, [int(x) for x in drafts[:j]] + [int(argmax_rows[j])]


# ----------------------------------------------------------------------------------------
# n-gram prompt-lookup drafter
# ----------------------------------------------------------------------------------------
def _continuation(tokens, e: int, K: int) -> list[int]:
    L = len(tokens)
    cont = [int(t) for t in tokens[e + 1:min(e + K, L - 1) + 1]]
    return cont + [PAD] * (K - len(cont))


def propose_scan(tokens, n_max: int, K: int) -> tuple[list[int], int, int]:
    """Drafts from the most recent earlier occurrence of the stream's last n ids.

    Feasibility page, the delta: the n-gram drafter looks the last m tokens of the
    prompt+generated stream up and proposes the most recent continuation; the handoff's
    knobs give the order (PB_NG) and the draft length (PB_K).  Hybrid verify-design page,
    harness lessons: the stream ends in the pending token a0, so drafts continue past it.

    Readings: n runs n_max, n_max-1, ..., 1 and the first n with a match wins; the match
    end e ranges over [n-1, len-2] (a non-empty continuation exists, overlap with the
    suffix allowed) and the largest e wins; drafts are tokens[e+1 .. min(e+K, len-1)],
    padded with -1 to K.  Returns (drafts, n_valid, n_used) with n_used = 0 for no match.
    Brute-force scan, O(len * n_max).
    """
    tokens = [int(t) for t in tokens]
    L = len(tokens)
    for n in range(min(n_max, L - 1), 0, -1):
        suffix = tokens[L - n:]
        for e in range(L - 2, n - 2, -1):
            if tokens[e - n + 1:e + 1] == suffix:
                d = _continuation(tokens, e, K)
                return d, sum(1 for x in d if x != PAD), n
    return [PAD] * K, 0, 0


class NgramIndex:
    """Hashtable form of the same drafter: n-gram -> most recent end position.

    An independent implementation of ``propose_scan`` (the feasibility page describes the
    drafter as a host hashtable over the stream); the two must agree.  Insertions are
    incremental: only end positions e <= len-2 are ever visible to a query.
    """

    def __init__(self, n_max: int):
        self.n_max = n_max
        self.tables = [dict() for _ in range(n_max + 1)]
        self.indexed = 0          # end positions [0, indexed) have been inserted

    def propose(self, tokens, K: int) -> tuple[list[int], int, int]:
        tokens = [int(t) for t in tokens]
        L = len(tokens)
        while self.indexed <= L - 2:
            e = self.indexed
            for n in range(1, self.n_max + 1):
                if e - n + 1 >= 0:
                    self.tables[n][tuple(tokens[e - n + 1:e + 1])] = e
            self.indexed += 1
        for n in range(min(self.n_max, L - 1), 0, -1):
            e = self.tables[n].get(tuple(tokens[L - n:]))
            if e is not None:
                d = _continuation(tokens, e, K)
                return d, sum(1 for x in d if x != PAD), n
        return [PAD] * K, 0, 0


# ----------------------------------------------------------------------------------------
# speedup model
# ----------------------------------------------------------------------------------------
def expected_tokens_per_round(alpha: float, K: int) -> float:
    """E(alpha, K): expected committed tokens per verify round when each draft is accepted
    independently with probability alpha (accepted drafts plus one bonus/correction).
    Feasibility page, C-value speedup model (closed form; alpha = 1 gives K + 1)."""
    if alpha == 1.0:
        return float(K + 1)
    return (1.0 - alpha ** (K + 1)) / (1.0 - alpha)


# ----------------------------------------------------------------------------------------
# round and decoding drivers
# ----------------------------------------------------------------------------------------
def verify_round(q, scale, hidden_rows, drafts):
    """One fused round given the window's hidden rows: logits, argmax, accept.

    Returns (logits [S, V] fp64, argmax [S], j, appended tokens)."""
    L = head_logits(q, scale, hidden_rows)
    a = argmax_lowest(L)
    j, app = accept(a, drafts)
    return L, a, j, app


def greedy_decode(context, hidden_fn, argmax_fn, n_new: int) -> list[int]:
    """Plain greedy decoding: each step feeds the stream and appends the argmax of the row
    at its last position.  ``hidden_fn(prefix)`` gives that row, ``argmax_fn(rows)`` the
    per-row greedy ids."""
    toks = [int(t) for t in context]
    for _ in range(n_new):
        toks.append(int(argmax_fn(np.stack([hidden_fn(toks)]))[0]))
    return toks


def spec_decode(context, hidden_fn, argmax_fn, n_new: int, K: int, n_max: int,
                drafter=None, stats: dict | None = None, gate_after: int = 0) -> list[int]:
    """Greedy speculative decoding with the fused S=K+1 window.

    a0 bootstrap (hybrid verify-design page, hybrid state discipline and status: one probe
    forward of the context's last row gives the always-correct anchor); then per round:
    propose past a0, one verify of [a0, d_1..d_K] (pads feed token 0), accept, commit
    1 + j tokens.  ``drafter(tokens, K)`` overrides the n-gram drafter.  Stops once at least
    ``n_new`` tokens beyond the context are committed; returns exactly that many.

    ``gate_after`` > 0: the hit-rate gate of the feasibility page ("SHIPPED" note: the app
    drops the drafter after a number of zero-accept rounds).  Reading: once ``gate_after``
    consecutive rounds have accepted no draft, the drafter is dropped for the rest of the
    sequence and every later window holds only pads.  The committed stream is unchanged.
    """
    toks = [int(t) for t in context]
    target = len(toks) + n_new
    toks.append(int(argmax_fn(np.stack([hidden_fn(toks)]))[0]))       # a0
    forwards = 1
    index = NgramIndex(n_max)
    js = []
    zero_run = 0
    gated_at = None
    while len(toks) < target:
        if gated_at is not None:
            drafts = [PAD] * K
        elif drafter is None:
            drafts, _, _ = index.propose(toks, K)
        else:
            drafts = [int(x) for x in drafter(toks, K)]
        window = [toks[-1]] + [d if d != PAD else 0 for d in drafts]
        rows = np.stack([hidden_fn(toks[:-1] + window[:i + 1]) for i in range(K + 1)])
        a = argmax_fn(rows)
        forwards += 1
        j, app = accept(a, drafts)
        js.append(j)
        toks.extend(app)
        zero_run = zero_run + 1 if j == 0 else 0
        if gate_after > 0 and gated_at is None and zero_run >= gate_after:
            gated_at = len(js)
    if stats is not None:
        stats["forwards"] = forwards
        stats["accepted"] = js
        stats["gated_after_round"] = gated_at
    return toks[:target]
