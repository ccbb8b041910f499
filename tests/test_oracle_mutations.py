"""Planted mistakes: each mutant is a copy of an oracle step with one plausible error (a
dropped term, a wrong index, a flipped tie rule), and each must fail the pin that guards
that step.  The mistakes live here, on the CPU, never in the product path."""
from fractions import Fraction

import numpy as np

import oracle
from oracle.verify import PAD
from weight_bound_verify_amd import synth


def _exact_row(q, s, h):
    return [float(sum(Fraction(float(s[v, k // 32])) * int(q[v, k]) * Fraction(float(h[k]))
                      for k in range(q.shape[1]))) for v in range(q.shape[0])]


def test_dequant_with_wrong_block_scale_is_caught():
    def mutant(q, scale):                           # scale index off by one block
        sh = np.roll(scale.astype(np.float64), 1, axis=1)
        return q.astype(np.float64) * np.repeat(sh, 32, axis=1)
    rng = np.random.default_rng(0)
    q, s = synth.quantize_q8b32(rng.standard_normal((8, 64), dtype=np.float32) * np.float32(0.02))
    h = synth.fp16_normal(rng, 64)
    ex = _exact_row(q, s, h)
    good = oracle.dequantize(q, s) @ h.astype(np.float64)
    bad = mutant(q, s) @ h.astype(np.float64)
    assert np.allclose(good, ex, rtol=0, atol=1e-12)
    assert not np.allclose(bad, ex, rtol=0, atol=1e-6)


def test_highest_index_tie_rule_is_caught():
    L = np.array([[0.0, 2.0, 1.0, 2.0]])
    mutant = lambda L: L.shape[1] - 1 - np.argmax(L[:, ::-1], axis=1)
    assert oracle.argmax_lowest(L)[0] == 1 and mutant(L)[0] == 3


def test_accept_off_by_one_is_caught():
    def mutant(a, d):                               # compares d_i with the row of d_i itself
        j = 0
        while j < len(d) and d[j] == a[j + 1]:
            j += 1
        return j
    a = [3, 4, 5, 6]
    d = [3, 4, 5]
    assert oracle.accept_length(a, d) == 3 and mutant(a, d) != 3


def test_oldest_occurrence_drafter_is_caught():
    def mutant(tokens, n_max, K):                   # scans from the oldest match
        L = len(tokens)
        for n in range(min(n_max, L - 1), 0, -1):
            for e in range(n - 1, L - 1):
                if tokens[e - n + 1:e + 1] == tokens[L - n:]:
                    c = tokens[e + 1:min(e + K, L - 1) + 1]
                    return c + [PAD] * (K - len(c))
        return [PAD] * K
    toks = [1, 2, 10, 1, 2, 20, 1, 2]
    assert oracle.propose_scan(toks, 2, 1)[0] == [20] and mutant(toks, 2, 1) == [10]


def test_rmsnorm_without_mean_is_caught():
    x = np.full((1, 64), 3.0, dtype=np.float16)
    mutant = lambda x: (x / np.sqrt(np.sum(x.astype(np.float64) ** 2) + 1e-6)).astype(np.float16)
    assert (oracle.rmsnorm_fp16(x, 0.0) == 1).all() and not (mutant(x) == 1).all()


def test_int4_nibble_order_swap_is_caught():
    def mutant(packed, scale):                      # high nibble read as the first 16 elements
        by = np.asarray(packed).reshape(packed.shape[0], -1, 16).astype(np.int64)
        codes = np.concatenate([(by >> 4) - 8, (by & 15) - 8], axis=2).reshape(packed.shape[0], -1)
        return codes * np.repeat(scale.astype(np.float64), 32, axis=1)
    codes = np.array([((k * 5) % 15) - 7 for k in range(32)], dtype=np.int64)
    p, s = synth.quantize_q4b32((codes.astype(np.float32) * np.float32(0.5))[None])
    assert np.array_equal(oracle.dequantize_q4b32(p, s)[0], codes * 0.5)
    assert not np.array_equal(mutant(p, s)[0], codes * 0.5)


def test_int4_missing_offset_is_caught():
    mutant = lambda packed, scale: np.repeat(scale.astype(np.float64), 32, axis=1) * np.concatenate(
        [np.asarray(packed).reshape(1, -1, 16) & 15, np.asarray(packed).reshape(1, -1, 16) >> 4], axis=2).reshape(1, -1)
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 3] = 1.0
    p, s = synth.quantize_q4b32(w)
    e = np.zeros(32)
    e[3] = 1.0
    assert oracle.dequantize_q4b32(p, s)[0] @ e == float(s[0, 0]) * 7
    assert mutant(p, s)[0] @ e != float(s[0, 0]) * 7


def _sampling_law_pvalue():
    """The law pin of speculative sampling (chi-square over the first three tokens)."""
    from tests.test_oracle_sampling import Markov, _chi2_pvalue, _exact_law, _greedy_chain_drafter, _law_counts
    model = Markov(4, 21)
    counts = _law_counts(model, 1.0, 3, _greedy_chain_drafter(model), 3000)
    return _chi2_pvalue(counts, _exact_law(model, 1.0))


def test_residual_that_keeps_the_rejected_draft_is_caught(monkeypatch):
    from oracle import sampling as smp
    monkeypatch.setattr(smp, "residual", lambda p, d: np.asarray(p, dtype=np.float64))   # redraw from p itself
    assert _sampling_law_pvalue() < 1e-6


def test_accept_test_on_the_wrong_row_is_caught(monkeypatch):
    from oracle import sampling as smp
    orig = smp.sampling_verify

    def mutant(L, drafts, T, seed, P0):             # d_{s+1} tested against row s+1, not row s
        r = orig(L, drafts, T, seed, P0)
        p, _ = smp.probabilities(L, T)
        K = len(drafts)
        pd = np.array([p[s + 1, d] if 0 <= d < p.shape[1] else 0.0 for s, d in enumerate(drafts)])
        j = 0
        while j < K and r["u_accept"][j] < pd[j]:
            j += 1
        r["j"], r["appended"] = j, list(drafts[:j]) + [int(r["sample"][j])]
        return r
    monkeypatch.setattr(smp, "sampling_verify", mutant)
    assert _sampling_law_pvalue() < 1e-6


def test_tree_walk_that_ignores_the_parent_link_is_caught():
    from tests.test_oracle_tree import _brute_force_accept, _random_tree

    def mutant(a, parents, drafts):             # moves to any later node with the right token
        K = len(parents)
        c, path = 0, []
        while True:
            nxt = next((i for i in range(c + 1, K + 1) if drafts[i - 1] != PAD and drafts[i - 1] == a[c]), None)
            if nxt is None:
                break
            path.append(nxt)
            c = nxt
        return len(path), [drafts[i - 1] for i in path] + [a[c]]
    rng = np.random.default_rng(0)
    caught = False
    for _ in range(300):
        K = int(rng.integers(2, 16))
        parents, drafts = _random_tree(rng, K, 3)
        a = [int(x) for x in rng.integers(0, 3, size=K + 1)]
        good = _brute_force_accept(a, parents, drafts)
        assert oracle.tree_accept(a, parents, drafts)[:2] == good
        caught |= mutant(a, parents, drafts) != good
    assert caught


def test_stack_forward_mutants_are_caught():
    """Three plausible composition mistakes in the stack driver (the last block dropped, the
    blocks run in reverse, the final norm left out), each caught by the hand-built stack of
    tests/test_oracle_stack.py (coordinate 2 reached only by A then B; the final norm of e_0 is
    5.65625)."""
    from test_oracle_stack import _mover
    A, B = _mover(0, 1), _mover(1, 2)
    x = np.zeros((1, 32), np.float16)
    x[0, 0] = 1

    def drop_last(x16, layers, eps):
        for layer in layers[:-1]:
            x16 = oracle.mlp_block(x16, layer, eps)
        return oracle.rmsnorm_fp16(x16, eps)

    def reversed_order(x16, layers, eps):
        for layer in layers[::-1]:
            x16 = oracle.mlp_block(x16, layer, eps)
        return oracle.rmsnorm_fp16(x16, eps)

    def no_final_norm(x16, layers, eps):
        for layer in layers:
            x16 = oracle.mlp_block(x16, layer, eps)
        return x16

    assert oracle.stack_forward(x, [A, B], eps=0.0)[0, 2] > 0
    assert drop_last(x, [A, B], 0.0)[0, 2] == 0
    assert reversed_order(x, [A, B], 0.0)[0, 2] == 0
    assert oracle.stack_forward(x, [B], eps=0.0)[0, 0] == 5.65625
    assert no_final_norm(x, [B], 0.0)[0, 0] != 5.65625
