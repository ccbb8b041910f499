"""Oracle for lossless sampling verify (temperature > 0).  TEST INFRASTRUCTURE ONLY.

Feasibility page ("Stream C - Speculative decoding"), the deferred list: to stay lossless
when sampling at a temperature above zero, the verify step has to work on the target's
probabilities and redraw a rejected position from the residual distribution; an argmax
comparison is only right for greedy decoding.  The pages name the method and stop there.
The steps below are the standard speculative-sampling rule (Leviathan, Kalman and Matias,
"Fast Inference from Transformers via Speculative Decoding", ICML 2023; Chen et al.,
"Accelerating Large Language Model Decoding with Speculative Sampling", 2023), written for a
drafter that proposes one token per position (a point mass q = e_d, as the n-gram drafter
does):

    p_s = softmax(L_s / T)                    target distribution at window row s
    draft d_{s+1} is kept with probability min(1, p_s(d) / q(d)) = p_s(d)
    at the first rejected draft, row s's token is drawn from max(0, p_s - q), renormalised
    if all K drafts are kept, one more token is drawn from p_K.

A pad (-1) has no mass under p, so it is always rejected and its residual is p itself.

Random numbers.  Both sides must draw the same ones, and the noise of a whole [S, V] window
cannot be passed in, so both implement one counter-based generator from its published
definition: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy
as 1, 2, 3", SC'11), key = the caller's 64-bit seed (low word first).  A round that starts
at stream length P0 (window row s predicts the token at position P0 + s) uses
    noise of (row s, token v):   counter (v, P0, s // 4, 0), output word s % 4
    accept test of d_{s+1}:      counter (0, P0, s // 4, 1), output word s % 4
and a 32-bit word w becomes the uniform (floor(w / 2^9) + 1/2) / 2^23 in (0, 1), exact in
fp32.  P0 grows every round, so no counter is used for two committed decisions.  Draws
from a distribution use the Gumbel-max form: the sample is the argmax over the support of
log r_v - log(-log u_v) (lowest id on ties), which has law r (E. J. Gumbel, 1954).

Parity pins (tests/test_oracle_sampling.py): the generator against the published
known-answer vectors and, through the same code at 64-bit width, against numpy's
Philox4x64-10; Gumbel-max frequencies against the distribution (chi-square); the decoding
driver against plain autoregressive sampling in law (chi-square over the first tokens of a
Markov stand-in model) and token for token when no draft is offered; the temperature -> 0
limit against greedy speculative decoding.
"""
from __future__ import annotations

import numpy as np

from .verify import NgramIndex, PAD

# Philox constants (the SC'11 paper): multipliers and Weyl key increments per word width.
_PHILOX = {
    32: dict(m=(0xD2511F53, 0xCD9E8D57), w=(0x9E3779B9, 0xBB67AE85)),
    64: dict(m=(0xD2E7470EE14C6C93, 0xCA5A826395121157), w=(0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B)),
}


def philox4(counter, key, width: int = 32, rounds: int = 10):
    """Philox4xW-R block function: four W-bit counter words and two key words -> four words.

    One round: the products of words 0 and 2 with the two multipliers give (hi, lo) halves;
    the new words are (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key gains its Weyl
    increments between rounds.  Python integers (exact), elementwise over equal-length
    sequences of counters (each counter a 4-tuple); returns a list of 4-tuples.
    """
    cst = _PHILOX[width]
    mask = (1 << width) - 1
    out = []
    for c, k in zip(counter, key):
        c0, c1, c2, c3 = (int(x) & mask for x in c)
        k0, k1 = (int(x) & mask for x in k)
        for r in range(rounds):
            if r:
                k0 = (k0 + cst["w"][0]) & mask
                k1 = (k1 + cst["w"][1]) & mask
            p0 = cst["m"][0] * c0
            p1 = cst["m"][1] * c2
            c0, c1, c2, c3 = ((p1 >> width) ^ c1 ^ k0) & mask, p1 & mask, ((p0 >> width) ^ c3 ^ k1) & mask, p0 & mask
        out.append((c0, c1, c2, c3))
    return out


def philox4x32_np(c0, c1, c2, c3, k0: int, k1: int, rounds: int = 10):
    """Philox4x32-10 over numpy arrays of counter words (uint32 arithmetic carried in uint64);
    the same rounds as ``philox4``, vectorised for whole [S, V] noise planes."""
    m0, m1 = (np.uint64(x) for x in _PHILOX[32]["m"])
    w0, w1 = _PHILOX[32]["w"]
    lo = np.uint64(0xFFFFFFFF)
    c = [np.asarray(x, dtype=np.uint64) & lo for x in (c0, c1, c2, c3)]
    c = np.broadcast_arrays(*c)
    c = [x.copy() for x in c]
    k0 &= 0xFFFFFFFF
    k1 &= 0xFFFFFFFF
    for r in range(rounds):
        if r:
            k0 = (k0 + w0) & 0xFFFFFFFF
            k1 = (k1 + w1) & 0xFFFFFFFF
        p0 = m0 * c[0]
        p1 = m1 * c[2]
        c = [((p1 >> np.uint64(32)) ^ c[1] ^ np.uint64(k0)) & lo, p1 & lo,
             ((p0 >> np.uint64(32)) ^ c[3] ^ np.uint64(k1)) & lo, p0 & lo]
    return c


def uniform01(word) -> np.ndarray:
    """A 32-bit word -> (floor(w / 2^9) + 1/2) / 2^23, strictly inside (0, 1)."""
    w = np.asarray(word, dtype=np.uint64)
    return ((w >> np.uint64(9)).astype(np.float64) + 0.5) / float(1 << 23)


def _seed_key(seed: int):
    seed = int(seed) & ((1 << 64) - 1)
    return seed & 0xFFFFFFFF, seed >> 32


def noise_uniforms(seed: int, P0: int, S: int, V: int) -> np.ndarray:
    """Uniforms [S, V] for the Gumbel noise of a round starting at stream length P0."""
    k0, k1 = _seed_key(seed)
    out = np.empty((S, V), dtype=np.float64)
    v = np.arange(V, dtype=np.uint64)
    for s in range(S):
        words = philox4x32_np(v, P0, s // 4, 0, k0, k1)
        out[s] = uniform01(words[s % 4])
    return out


def accept_uniforms(seed: int, P0: int, K: int) -> np.ndarray:
    """Uniforms [K]: entry s decides draft d_{s+1} against window row s."""
    k0, k1 = _seed_key(seed)
    out = np.empty(K, dtype=np.float64)
    for s in range(K):
        words = philox4x32_np(0, P0, s // 4, 1, k0, k1)
        out[s] = uniform01(words[s % 4])
    return out


# ----------------------------------------------------------------------------------------
# distributions and draws
# ----------------------------------------------------------------------------------------
def probabilities(L: np.ndarray, T: float) -> tuple[np.ndarray, np.ndarray]:
    """p = softmax(L / T) per row in fp64, and the log-normaliser lse = log sum exp(L / T)."""
    z = np.atleast_2d(np.asarray(L, dtype=np.float64)) / float(T)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    tot = e.sum(axis=1, keepdims=True)
    return e / tot, (m + np.log(tot))[:, 0]


def residual(p: np.ndarray, d: int) -> np.ndarray:
    """max(0, p - q) renormalised, q the point mass at draft d (a pad has no mass: r = p).
    When p is itself the point mass at d the residual is empty and zeros are returned."""
    p = np.asarray(p, dtype=np.float64)
    q = np.zeros_like(p)
    if 0 <= d < p.shape[0]:
        q[d] = 1.0
    r = np.maximum(0.0, p - q)
    tot = r.sum()
    return r / tot if tot > 0 else r


def gumbel_sample(dist: np.ndarray, u: np.ndarray) -> int:
    """Draw from ``dist`` with uniforms ``u`` (one per id): argmax over the support of
    log dist_v - log(-log u_v), lowest id on ties; -1 for an empty support."""
    dist = np.asarray(dist, dtype=np.float64)
    support = dist > 0
    if not support.any():
        return -1
    key = np.full(dist.shape, -np.inf)
    key[support] = np.log(dist[support]) - np.log(-np.log(u[support]))
    return int(np.flatnonzero(key == key.max())[0])


def sampling_verify(L: np.ndarray, drafts, T: float, seed: int, P0: int) -> dict:
    """One sampling-verify round over the window's logits L [S = K+1, V].

    Returns the accepted length j, the appended tokens d_1..d_j, y_j, and, for parity of
    every window row: ``p_draft[s]`` = p_s(d_{s+1}) (0 for pads), ``u_accept[s]``,
    ``sample[s]`` = the residual draw of row s against d_{s+1} (row K: a draw from p_K) and
    ``lse[s]``.
    """
    L = np.atleast_2d(np.asarray(L, dtype=np.float64))
    S, V = L.shape
    K = S - 1
    drafts = [int(d) for d in drafts]
    if len(drafts) != K:
        raise ValueError("need K = S - 1 drafts")
    p, lse = probabilities(L, T)
    un = noise_uniforms(seed, P0, S, V)
    ua = accept_uniforms(seed, P0, K)
    p_draft = np.array([p[s, d] if 0 <= d < V else 0.0 for s, d in enumerate(drafts)])
    sample = [gumbel_sample(residual(p[s], drafts[s]), un[s]) for s in range(K)]
    sample.append(gumbel_sample(p[K], un[K]))
    j = 0
    while j < K and ua[j] < min(1.0, p_draft[j]):
        j += 1
    return dict(j=j, appended=drafts[:j] + [sample[j]], p_draft=p_draft, u_accept=ua,
                sample=np.array(sample), lse=lse, accepted=[bool(ua[s] < p_draft[s]) for s in range(K)])


# ----------------------------------------------------------------------------------------
# decoding drivers
# ----------------------------------------------------------------------------------------
def sample_decode(context, logits_fn, n_new: int, T: float, seed: int) -> list[int]:
    """Plain autoregressive sampling: the token at position P is drawn from
    softmax(L / T) of the row at the stream's last position, with the noise of a one-row
    round starting at P.  ``logits_fn(prefix)`` gives that row's logits [V]."""
    toks = [int(t) for t in context]
    for _ in range(n_new):
        L = np.asarray(logits_fn(toks), dtype=np.float64)[None, :]
        p, _ = probabilities(L, T)
        toks.append(gumbel_sample(p[0], noise_uniforms(seed, len(toks), 1, L.shape[1])[0]))
    return toks


def spec_sample_decode(context, logits_fn, n_new: int, K: int, n_max: int, T: float, seed: int,
                       drafter=None, stats: dict | None = None) -> list[int]:
    """Speculative sampling with the fused S = K+1 window, the n-gram drafter by default.

    The anchor a0 is drawn from the context's last row as a one-row round (the sampling
    counterpart of the greedy bootstrap); each round then drafts past the anchor, verifies
    [a0, d_1..d_K] (pads feed token 0), keeps j drafts and appends the residual or bonus
    draw.  Returns exactly ``n_new`` tokens beyond the context.
    """
    toks = [int(t) for t in context]
    target = len(toks) + n_new
    toks = sample_decode(toks, logits_fn, 1, T, seed)                  # a0
    index = NgramIndex(n_max)
    js = []
    while len(toks) < target:
        if drafter is None:
            drafts, _, _ = index.propose(toks, K)
        else:
            drafts = [int(x) for x in drafter(toks, K)]
        window = [toks[-1]] + [d if d != PAD else 0 for d in drafts]
        L = np.stack([np.asarray(logits_fn(toks[:-1] + window[:i + 1]), dtype=np.float64) for i in range(K + 1)])
        r = sampling_verify(L, drafts, T, seed, len(toks))
        js.append(r["j"])
        toks.extend(r["appended"])
    if stats is not None:
        stats["accepted"] = js
    return toks[:target]
