"""Pins for the tree-verify oracle (oracle/tree.py): the walk against brute force over all
paths and against the linear accept on chains, the drafter against the linear drafter and
trie invariants, a hand-built example, and tree speculative decoding against plain greedy
decoding (lossless) on stand-in models whose rows depend on the whole path."""
import hashlib

import numpy as np
import pytest

import oracle
from oracle import tree as tr
from oracle.verify import PAD


def _random_tree(rng, K, V):
    """Random tree with distinct sibling tokens (pads allowed as leaves)."""
    parents, drafts = [], []
    kids = {0: set()}
    for i in range(1, K + 1):
        p = int(rng.integers(0, i))
        free = [t for t in range(V) if t not in kids[p]]
        if rng.random() < 0.1 or not free:
            parents.append(0)
            drafts.append(PAD)
            kids[i] = set()
            continue
        t = int(free[int(rng.integers(0, len(free)))])
        kids[p].add(t)
        kids[i] = set()
        parents.append(p)
        drafts.append(t)
    return parents, drafts


def _brute_force_accept(a, parents, drafts):
    K = len(parents)
    best, best_depth = 0, 0
    for i in range(1, K + 1):                  # the deepest node whose whole path matches
        node, ok, depth = i, True, 0
        while node != 0:
            p = parents[node - 1]
            if drafts[node - 1] == PAD or drafts[node - 1] != a[p]:
                ok = False
                break
            node, depth = p, depth + 1
        if ok and depth > best_depth:
            best, best_depth = i, depth
    path = []
    node = best
    while node != 0:
        path.append(node)
        node = parents[node - 1]
    path = path[::-1]
    end = best
    return len(path), [drafts[i - 1] for i in path] + [a[end]]


def test_tree_accept_matches_brute_force():
    rng = np.random.default_rng(0)
    for case in range(3000):
        K = int(rng.integers(1, 16))
        V = int(rng.integers(2, 6))           # few ids: many matching paths
        parents, drafts = _random_tree(rng, K, V)
        a = rng.integers(0, V, size=K + 1)
        j, app, path = tr.tree_accept(a, parents, drafts)
        bj, bapp = _brute_force_accept(list(a), parents, drafts)
        assert (j, app) == (bj, bapp), (case, parents, drafts, list(a))
        assert len(path) == j


def test_chain_tree_is_the_linear_accept():
    rng = np.random.default_rng(1)
    for _ in range(2000):
        K = int(rng.integers(1, 16))
        a = rng.integers(0, 4, size=K + 1)
        d = [int(x) if rng.random() > 0.1 else PAD for x in rng.integers(0, 4, size=K)]
        chain = list(range(K))                 # node i+1 hangs under node i
        j, app, _ = tr.tree_accept(a, chain, d)
        assert (j, app) == oracle.accept(a, d)


def test_one_branch_drafter_is_the_linear_drafter():
    rng = np.random.default_rng(2)
    for _ in range(400):
        n = int(rng.integers(1, 120))
        toks = [int(x) for x in rng.integers(0, int(rng.integers(2, 12)), size=n)]
        K = int(rng.integers(1, 16))
        nm = int(rng.integers(1, 5))
        parents, drafts, used, real = tr.propose_tree(toks, nm, K, 1, K)
        d_lin, nvalid, nused = oracle.propose_scan(toks, nm, K)
        assert drafts == list(d_lin) and used == nused and real == nvalid
        assert parents == list(range(K))[:real] + [0] * (K - real)


def test_drafter_trie_invariants():
    rng = np.random.default_rng(3)
    for _ in range(600):
        n = int(rng.integers(2, 200))
        toks = [int(x) for x in rng.integers(0, int(rng.integers(2, 10)), size=n)]
        K = int(rng.integers(1, 16))
        B = int(rng.integers(1, 5))
        D = int(rng.integers(1, K + 1))
        parents, drafts, used, real = tr.propose_tree(toks, 3, K, B, D)
        assert len(parents) == len(drafts) == K
        assert all(d == PAD for d in drafts[real:]) and all(p == 0 for p in parents[real:])
        sib = set()
        for i in range(real):
            assert 0 <= parents[i] <= i and drafts[i] != PAD          # parent precedes the node
            assert (parents[i], drafts[i]) not in sib                 # distinct sibling tokens
            sib.add((parents[i], drafts[i]))
            assert len(tr.path_tokens(parents, drafts, i + 1)) <= D
        # every ranked continuation's prefix is a path while the node budget lasts
        for (_, e) in tr._ranked_matches(toks, 3)[:B]:
            cont = toks[e + 1: min(e + 1 + D, n)]
            node = 0
            for t in cont:
                nxt = [i + 1 for i in range(real) if parents[i] == node and drafts[i] == t]
                if not nxt:
                    assert real == K                                 # only a full budget stops it
                    break
                node = nxt[0]


def test_hand_built_tree():
    # suffix (1, 2) occurs ending at positions 6 and 2; continuations 4 7 1 2 and 3 9 1 2
    toks = [5, 1, 2, 3, 9, 1, 2, 4, 7, 1, 2]
    parents, drafts, used, real = tr.propose_tree(toks, 2, 6, 2, 4)
    assert used == 2 and real == 6
    assert drafts == [4, 7, 1, 2, 3, 9]
    assert parents == [0, 1, 2, 3, 0, 5]
    # greedy rows that follow the second branch: 3 then 9, then a miss
    a = [3, 0, 0, 0, 0, 9, 8]
    assert tr.tree_accept(a, parents, drafts)[:2] == (2, [3, 9, 8])
    # both branches share no prefix; a third branch (1, 2) ending at 1 would merge nowhere
    p3, d3, _, r3 = tr.propose_tree(toks + [9, 1, 2], 2, 15, 3, 3)
    assert r3 == len(d3) - d3.count(PAD)


class PathHash:
    """Stand-in whose row depends on the whole stream (a hash of the prefix)."""

    def __init__(self, V, H, seed):
        self.V, self.H, self.seed = V, H, seed
        self.W = np.random.default_rng(seed).standard_normal((V, H))

    def hidden(self, prefix):
        h = hashlib.sha256(bytes(str((self.seed, prefix[-3:], len(prefix) % 5)), "ascii")).digest()
        return np.random.default_rng(int.from_bytes(h[:8], "little")).standard_normal(self.H)

    def argmax(self, rows):
        return oracle.argmax_lowest(rows @ self.W.T)


@pytest.mark.parametrize("B,D", [(1, 8), (2, 4), (3, 3), (4, 6), (4, 2)])
def test_tree_speculative_decoding_is_lossless(B, D):
    rng = np.random.default_rng(10 + B * 7 + D)
    for case in range(60):
        V = int(rng.integers(3, 9))
        m = PathHash(V, 6, case)
        ctx = [int(x) for x in rng.integers(0, V, size=int(rng.integers(1, 40)))]
        K = int(rng.integers(max(1, D), 16))
        stats = {}
        out = tr.tree_spec_decode(ctx, m.hidden, m.argmax, 30, K, 3, B, D, stats=stats)
        assert out == oracle.greedy_decode(ctx, m.hidden, m.argmax, 30)


def test_one_branch_tree_decoding_equals_linear_decoding_round_by_round():
    rng = np.random.default_rng(20)
    for case in range(40):
        V = int(rng.integers(3, 9))
        m = PathHash(V, 6, 100 + case)
        ctx = [int(x) for x in rng.integers(0, V, size=30)]
        K = int(rng.integers(1, 12))
        s_lin, s_tree = {}, {}
        a = oracle.spec_decode(ctx, m.hidden, m.argmax, 40, K, 3, stats=s_lin)
        b = tr.tree_spec_decode(ctx, m.hidden, m.argmax, 40, K, 3, 1, K, stats=s_tree)
        assert a == b and s_lin["accepted"] == s_tree["accepted"]


def test_wider_trees_accept_at_least_as_often_on_repetitive_text():
    """More branches never shorten the accepted path when the extra branches only add nodes
    (same first branch, larger node budget)."""
    rng = np.random.default_rng(30)
    gain = 0
    for case in range(100):
        V = 4
        m = PathHash(V, 6, 500 + case)
        ctx = [int(x) for x in rng.integers(0, V, size=60)]
        s1, s4 = {}, {}
        tr.tree_spec_decode(ctx, m.hidden, m.argmax, 30, 15, 3, 1, 5, stats=s1)
        tr.tree_spec_decode(ctx, m.hidden, m.argmax, 30, 15, 3, 3, 5, stats=s4)
        gain += sum(s4["accepted"]) / len(s4["accepted"]) - sum(s1["accepted"]) / len(s1["accepted"])
    assert gain > 0
