"""Pins for the oracle's accept and n-gram drafter.

accept: exhaustive over every match mask, the invariants the fused scheme implies, and the
closed-form E(alpha, K) and the printed speedup table of the feasibility page's C-value model.
propose: the brute-force scan against the independent hashtable index, hand-derived streams,
and the planted-span construction of the tiny configuration.
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle.verify import PAD
from weight_bound_verify_amd import synth


# ---------------------------------------------------------------- accept
@pytest.mark.parametrize("K", range(0, 9))
def test_accept_exhaustive_masks(K):
    rng = np.random.default_rng(K)
    for mask in itertools.product([0, 1], repeat=K):
        a = rng.integers(0, 50, size=K + 1)
        d = [int(a[i]) if mask[i] else int(a[i]) + 1 + int(rng.integers(0, 10)) for i in range(K)]
        lead = 0
        while lead < K and mask[lead]:
            lead += 1
        j, app = oracle.accept(a, d)
        assert j == lead
        assert app == d[:j] + [int(a[j])]
        assert len(app) == 1 + j


def test_accept_invariants():
    a = [5, 9, 2, 7, 7]
    assert oracle.accept_length(a, a[:4]) == 4                # drafts == argmaxes -> j = K
    assert oracle.accept_length(a, [6, 9, 2, 7]) == 0         # d1 differs -> j = 0
    assert oracle.accept_length(a, [5, 9, PAD, PAD]) == 2     # pads never match
    j, app = oracle.accept(a, a[:4])
    assert app == [5, 9, 2, 7, 7]                             # bonus = last row
    with pytest.raises(ValueError):
        oracle.accept_length([1, 2], [1, 2])


def test_expected_tokens_closed_form_edges():
    assert oracle.expected_tokens_per_round(0.0, 8) == 1.0
    assert oracle.expected_tokens_per_round(1.0, 8) == 9.0
    for K in (1, 4, 8):
        for al in (0.3, 0.7):
            assert oracle.expected_tokens_per_round(al, K) == pytest.approx(sum(al ** i for i in range(K + 1)))


def test_printed_speedup_table(golden):
    g = golden("speedup_model.json")
    K = g["K_max"]
    for cv, row in g["speedup"].items():
        for al, want in zip(g["alpha"], row):
            best = max(oracle.expected_tokens_per_round(al, k) for k in range(1, K + 1)) / float(cv)
            assert round(best, 2) == pytest.approx(want, abs=1e-9), (cv, al)


@pytest.mark.parametrize("alpha,K", [(0.5, 8), (0.8, 4), (0.9, 8)])
def test_accept_statistics_match_closed_form(alpha, K):
    rng = np.random.default_rng(int(alpha * 100) + K)
    n = 40000
    tot = 0
    for _ in range(n):
        a = rng.integers(0, 1000, size=K + 1)
        hit = rng.random(K) < alpha
        d = [int(a[i]) if hit[i] else int(a[i]) + 1 for i in range(K)]
        tot += 1 + oracle.accept_length(a, d)
    mean = tot / n
    want = oracle.expected_tokens_per_round(alpha, K)
    assert abs(mean - want) < 0.05 * want


# ---------------------------------------------------------------- propose
def test_propose_hand_cases():
    # ... 1 2 3 4 5 ... 1 2 3 : last trigram seen ending at index 2 -> continuation 4 5 ...
    toks = [1, 2, 3, 4, 5, 6, 9, 1, 2, 3]
    assert oracle.propose_scan(toks, 3, 4) == ([4, 5, 6, 9], 4, 3)
    # continuation truncated at the stream end and padded
    assert oracle.propose_scan([7, 8, 7, 8], 3, 4) == ([7, 8, PAD, PAD], 2, 2)
    # most recent occurrence wins
    toks = [1, 2, 10, 1, 2, 20, 1, 2]
    assert oracle.propose_scan(toks, 2, 1) == ([20], 1, 2)
    # fall back to n = 1 when no bigram repeats
    toks = [4, 5, 6, 3, 6]
    assert oracle.propose_scan(toks, 3, 2) == ([3, 6], 2, 1)
    # nothing repeats: all pads
    assert oracle.propose_scan([1, 2, 3], 3, 3) == ([PAD] * 3, 0, 0)
    # overlap with the suffix is allowed: run of equal ids
    assert oracle.propose_scan([5, 5, 5, 5], 3, 2) == ([5, PAD], 1, 3)
    # single token stream and empty-ish inputs
    assert oracle.propose_scan([3], 3, 2) == ([PAD, PAD], 0, 0)


def test_propose_scan_agrees_with_hashtable_incrementally():
    rng = np.random.default_rng(0)
    for case in range(300):
        V = int(rng.integers(2, 12))
        n_max = int(rng.integers(1, 5))
        K = int(rng.integers(1, 10))
        toks = list(rng.integers(0, V, size=int(rng.integers(1, 6))))
        idx = oracle.NgramIndex(n_max)
        for _ in range(12):
            assert idx.propose(toks, K) == oracle.propose_scan(toks, n_max, K)
            toks += list(rng.integers(0, V, size=int(rng.integers(1, 4))))


def test_propose_planted_span_tiny_config_recipe():
    rng = np.random.default_rng(synth.streams(0).context)
    ctx, span, offsets = synth.uniform_context_with_span(rng, 512, 8192, 12, 16)
    # a stream that ends inside a planted span continues with the rest of the span
    for cut in (3, 6, 9):
        toks = list(ctx[:offsets[-1] + cut])
        d, nv, nu = oracle.propose_scan(toks, 3, 8)
        rest = list(span[cut:cut + 8])
        assert d[:len(rest)] == rest and nu == 3


def test_ngram_index_never_sees_the_query_suffix():
    idx = oracle.NgramIndex(3)
    assert idx.propose([1, 2, 3], 2) == ([PAD, PAD], 0, 0)
    assert idx.propose([1, 2, 3, 1, 2, 3], 2) == ([1, 2], 2, 3)
