"""Pins for the sampling-verify oracle (oracle/sampling.py): the counter-based generator
against published known answers and numpy's own Philox, Gumbel-max draws against their law,
and the decoding driver against plain autoregressive sampling (in law, and token for token
when no draft is offered) and against greedy speculative decoding in the T -> 0 limit."""
import json
import os

import numpy as np
import pytest
from scipy.stats import chi2

import oracle
from oracle import sampling as smp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_philox4x32_known_answers():
    with open(os.path.join(GOLDEN, "philox4x32_kat.json")) as f:
        kat = json.load(f)
    for vec in kat["vectors"]:
        c = tuple(int(x, 16) for x in vec["counter"])
        k = tuple(int(x, 16) for x in vec["key"])
        want = tuple(int(x, 16) for x in vec["out"])
        assert smp.philox4([c], [k], 32)[0] == want
        got = smp.philox4x32_np(*c, k[0], k[1])
        assert tuple(int(w) for w in got) == want


def test_philox_block_function_matches_numpy_philox4x64():
    """The same block function at 64-bit width is numpy's Philox4x64-10 (numpy advances the
    counter by one before each block)."""
    rng = np.random.default_rng(5)
    for _ in range(20):
        c = [int(x) for x in rng.integers(0, 2 ** 63, size=4, dtype=np.uint64)]
        k = [int(x) for x in rng.integers(0, 2 ** 63, size=2, dtype=np.uint64)]
        bg = np.random.Philox(counter=np.array(c, dtype=np.uint64), key=np.array(k, dtype=np.uint64))
        raw = [int(x) for x in bg.random_raw(4)]
        assert list(smp.philox4([(c[0] + 1, c[1], c[2], c[3])], [k], 64)[0]) == raw


def test_vectorised_philox_equals_scalar_rounds():
    rng = np.random.default_rng(6)
    c = rng.integers(0, 2 ** 32, size=(4, 50), dtype=np.uint64)
    k0, k1 = 0x12345678, 0x9abcdef0
    vec = smp.philox4x32_np(c[0], c[1], c[2], c[3], k0, k1)
    for i in range(50):
        want = smp.philox4([tuple(int(x) for x in c[:, i])], [(k0, k1)], 32)[0]
        assert tuple(int(w[i]) for w in vec) == want


def test_uniform01_range_exact_and_uniform():
    w = np.array([0, 511, 512, 2 ** 32 - 1], dtype=np.uint64)
    u = smp.uniform01(w)
    assert u[0] == u[1] == 0.5 / 2 ** 23 and u[2] == 1.5 / 2 ** 23 and u[3] == 1 - 0.5 / 2 ** 23
    assert np.all(u.astype(np.float32).astype(np.float64) == u)          # exact in fp32
    x = smp.noise_uniforms(3, 100, 9, 20000)
    assert 0 < x.min() and x.max() < 1
    assert abs(x.mean() - 0.5) < 0.003 and abs(x.var() - 1 / 12) < 0.002
    # rows of one round and rows of different rounds are not the same draws
    assert not np.array_equal(x[0], x[4]) and not np.array_equal(x[0], smp.noise_uniforms(3, 101, 1, 20000)[0])


def _chi2_pvalue(counts, probs):
    n = counts.sum()
    exp = probs * n
    keep = exp >= 5
    c = np.append(counts[keep], counts[~keep].sum())
    e = np.append(exp[keep], exp[~keep].sum())
    if e[-1] == 0:
        c, e = c[:-1], e[:-1]
    stat = ((c - e) ** 2 / e).sum()
    return chi2.sf(stat, len(c) - 1)


def test_gumbel_max_draws_have_the_distribution_as_law():
    dist = np.array([0.05, 0.0, 0.3, 0.15, 0.45, 0.05])
    counts = np.zeros(6)
    for P in range(20000):
        counts[smp.gumbel_sample(dist, smp.noise_uniforms(11, P, 1, 6)[0])] += 1
    assert counts[1] == 0
    assert _chi2_pvalue(counts, dist) > 1e-3


def test_residual_special_cases():
    p = np.array([0.2, 0.5, 0.3])
    r = smp.residual(p, 1)
    assert r[1] == 0 and np.isclose(r.sum(), 1) and np.allclose(r[[0, 2]], p[[0, 2]] / 0.5)
    assert np.array_equal(smp.residual(p, -1), p)                       # pad: nothing removed
    assert smp.gumbel_sample(smp.residual(np.array([0.0, 1.0, 0.0]), 1), np.full(3, 0.5)) == -1
    # a draw from the residual never returns the rejected draft
    for P in range(200):
        assert smp.gumbel_sample(r, smp.noise_uniforms(2, P, 1, 3)[0]) != 1


def test_accept_probability_is_p_of_the_draft_on_its_own_row():
    rng = np.random.default_rng(8)
    L = rng.standard_normal((5, 7))
    drafts = [3, 1, -1, 6]
    r = smp.sampling_verify(L, drafts, 0.8, 99, 40)
    p, lse = smp.probabilities(L, 0.8)
    assert np.allclose(lse, np.log(np.exp(L / 0.8).sum(axis=1)))
    assert r["p_draft"][0] == p[0, 3] and r["p_draft"][1] == p[1, 1] and r["p_draft"][2] == 0 and r["p_draft"][3] == p[3, 6]
    j = r["j"]
    assert all(r["u_accept"][s] < r["p_draft"][s] for s in range(j))
    assert j == 4 or r["u_accept"][j] >= r["p_draft"][j]
    assert r["appended"] == drafts[:j] + [int(r["sample"][j])]
    assert j <= 2                                                        # the pad always stops it


class Markov:
    """Stand-in target model whose logits depend on the last token only."""

    def __init__(self, V, seed, scale=1.5):
        self.table = np.random.default_rng(seed).standard_normal((V, V)) * scale
        self.V = V

    def __call__(self, prefix):
        return self.table[prefix[-1]]

    def probs(self, T):
        return smp.probabilities(self.table, T)[0]


def _law_counts(model, T, K, drafter, n_seeds, n_new=3, ctx=(0, 1, 2, 0, 1), dec=smp.spec_sample_decode):
    V = model.V
    counts = np.zeros(V ** n_new)
    for seed in range(n_seeds):
        if dec is smp.sample_decode:
            out = dec(list(ctx), model, n_new, T, seed)
        else:
            out = dec(list(ctx), model, n_new, K, 2, T, seed, drafter=drafter)
        cell = 0
        for t in out[len(ctx):]:
            cell = cell * V + t
        counts[cell] += 1
    return counts


def _exact_law(model, T, n_new=3, last=1):
    P = model.probs(T)
    V = model.V
    law = np.zeros(V ** n_new)
    for cell in range(V ** n_new):
        toks = [(cell // V ** (n_new - 1 - i)) % V for i in range(n_new)]
        pr, prev = 1.0, last
        for t in toks:
            pr *= P[prev, t]
            prev = t
        law[cell] = pr
    return law


def _greedy_chain_drafter(model, miss_every=3):
    """Proposes the model's greedy continuation, with every third position replaced by a
    wrong id, so rounds see both kept and rejected drafts."""
    def drafter(toks, K):
        out, t = [], toks[-1]
        for i in range(K):
            t = int(np.argmax(model.table[t]))
            out.append(t if (len(toks) + i) % miss_every else (t + 1) % model.V)
        return out
    return drafter


@pytest.mark.parametrize("T", [1.0, 0.6])
def test_speculative_sampling_has_the_target_law(T):
    """Lossless in law: the first three tokens of speculative sampling follow the target's
    own autoregressive law exactly (chi-square over all V^3 outcomes)."""
    model = Markov(4, 21)
    stats = {}
    counts = _law_counts(model, T, 3, _greedy_chain_drafter(model), 3000)
    assert _chi2_pvalue(counts, _exact_law(model, T)) > 1e-3
    # drafts are kept in some rounds and rejected in others
    smp.spec_sample_decode([0, 1, 2, 0, 1], model, 12, 3, 2, T, 7, drafter=_greedy_chain_drafter(model), stats=stats)
    assert max(stats["accepted"]) > 0 and min(stats["accepted"]) < 3


def test_plain_sampling_has_the_target_law():
    model = Markov(4, 21)
    counts = _law_counts(model, 1.0, 0, None, 3000, dec=smp.sample_decode)
    assert _chi2_pvalue(counts, _exact_law(model, 1.0)) > 1e-3


def test_no_drafts_equals_plain_sampling_token_for_token():
    model = Markov(50, 3)
    for seed in range(20):
        ctx = list(np.random.default_rng(seed).integers(0, 50, 8))
        pads = lambda toks, K: [-1] * K
        assert (smp.spec_sample_decode(ctx, model, 15, 4, 3, 0.9, seed, drafter=pads)
                == smp.sample_decode(ctx, model, 15, 0.9, seed))


def test_zero_temperature_limit_is_greedy_speculative_decoding():
    """T -> 0: p becomes the point mass at the argmax, a draft is kept iff it is the argmax
    and every draw is the argmax, so the stream is greedy speculative decoding's."""
    rng = np.random.default_rng(4)
    for case in range(30):
        V = int(rng.integers(5, 40))
        model = Markov(V, 100 + case, scale=1.0)
        ctx = [int(x) for x in rng.integers(0, V, 12)]
        K = int(rng.integers(1, 6))
        greedy = oracle.spec_decode(ctx, lambda p: model(p), lambda rows: np.argmax(rows, axis=1), 20, K, 3)
        samp = smp.spec_sample_decode(ctx, model, 20, K, 3, 1e-6, case)
        assert samp == greedy
