"""Oracle for greedy tree verify.  TEST INFRASTRUCTURE ONLY.

Feasibility page ("Stream C - Speculative decoding"), the deferred list and the EAGLE-3 + tree
handoff: a drafter proposes a TREE of candidate continuations, verify runs one forward over all
tree nodes under a tree attention mask, and the linear accept loop becomes a walk down the
tree.  The pages stop there; the readings below are the plainest ones that keep the linear
chain as the special case (a one-branch tree is the linear window).

Tree.  Node 0 is the anchor a0 (the pending token); draft nodes 1..K each have a parent index
p(i) < i and a token t(i) (a pad is -1, a leaf that never matches).  Window row i is the
model's row after the path root -> i, so S = K + 1 rows as in the linear window.

Accept (greedy).  From node c = 0: let a = argmax of row c; move to the child of c whose token
is a (lowest node index if several); repeat until no child matches.  The tokens of the path's
nodes and the final a are committed: j = path length drafts plus one correction/bonus token.

Drafter.  The linear n-gram drafter ranks earlier end positions e of the stream's suffix by
(match length l(e) up to n_max, then recency e) and continues the best one.  The tree drafter
takes the ``branches`` best-ranked positions with l(e) > 0, truncates each continuation to
``depth`` tokens (and at the stream's end), and inserts them into a prefix tree in rank order,
reusing a node when its token already hangs under the same parent, creating nodes in order
until K exist; remaining draft slots are pads hung under the root.  One branch of depth K is
the linear drafter.

Parity pins (tests/test_oracle_tree.py): accept against brute force over all root-to-node
paths; a chain tree against the linear accept; the drafter with one branch against
propose_scan and its trie against invariants (parents first, distinct sibling tokens, every
inserted prefix present); tree speculative decoding against plain greedy decoding (lossless)
on stand-in models whose rows depend on the whole path.
"""
from __future__ import annotations

import numpy as np

from .verify import PAD


def tree_accept(argmax_rows, parents, drafts):
    """Greedy walk.  ``argmax_rows`` [K+1], ``parents`` / ``drafts`` [K] describe nodes 1..K.
    Returns (j, appended tokens, path of node indices excluding the root)."""
    a = [int(x) for x in argmax_rows]
    K = len(a) - 1
    parents = [int(p) for p in parents]
    drafts = [int(d) for d in drafts]
    if len(parents) != K or len(drafts) != K:
        raise ValueError("need K parents and K drafts")
    c, path = 0, []
    while True:
        nxt = None
        for i in range(1, K + 1):                     # lowest node index first
            if parents[i - 1] == c and drafts[i - 1] != PAD and drafts[i - 1] == a[c]:
                nxt = i
                break
        if nxt is None:
            break
        path.append(nxt)
        c = nxt
    return len(path), [drafts[i - 1] for i in path] + [a[c]], path


def _ranked_matches(tokens, n_max: int):
    """End positions e <= len-2 with l(e) > 0, best first by (l(e), e)."""
    toks = [int(t) for t in tokens]
    n = len(toks)
    out = []
    for e in range(n - 1):
        l = 0
        while l < n_max and e - l >= 0 and toks[e - l] == toks[n - 1 - l]:
            l += 1
        if l > 0:
            out.append((l, e))
    out.sort(reverse=True)
    return out


def propose_tree(tokens, n_max: int, K: int, branches: int, depth: int):
    """Tree drafts: (parents [K], drafts [K], n used = l of the best match or 0, real nodes)."""
    toks = [int(t) for t in tokens]
    n = len(toks)
    ranked = _ranked_matches(toks, n_max)[:branches]
    parents, drafts = [], []
    children = {0: {}}                                   # node -> {token: child node}
    for (_, e) in ranked:
        cont = toks[e + 1: min(e + 1 + depth, n)]
        node = 0
        for t in cont:
            if t in children[node]:
                node = children[node][t]
                continue
            if len(drafts) >= K:
                break
            drafts.append(t)
            parents.append(node)
            new = len(drafts)
            children[node][t] = new
            children[new] = {}
            node = new
    real = len(drafts)
    while len(drafts) < K:
        drafts.append(PAD)
        parents.append(0)
    return parents, drafts, (ranked[0][0] if ranked else 0), real


def path_tokens(parents, drafts, i: int):
    """Tokens of the path root -> node i (excluding the root), pads fed as token 0."""
    out = []
    while i != 0:
        d = drafts[i - 1]
        out.append(d if d != PAD else 0)
        i = parents[i - 1]
    return out[::-1]


def tree_spec_decode(context, hidden_fn, argmax_fn, n_new: int, K: int, n_max: int, branches: int, depth: int,
                     drafter=None, stats: dict | None = None) -> list[int]:
    """Greedy speculative decoding with tree drafts and the tree walk.

    The anchor bootstrap and the stopping rule follow ``spec_decode``; row i of a round's
    window is ``hidden_fn`` of the stream followed by the path root -> i (the tree attention
    mask: a node sees its ancestors only).  ``drafter(tokens, K)`` may replace the n-gram tree
    drafter and returns (parents, drafts).
    """
    toks = [int(t) for t in context]
    target = len(toks) + n_new
    toks.append(int(argmax_fn(np.stack([hidden_fn(toks)]))[0]))       # a0
    js = []
    while len(toks) < target:
        if drafter is None:
            parents, drafts, _, _ = propose_tree(toks, n_max, K, branches, depth)
        else:
            parents, drafts = drafter(toks, K)
        rows = np.stack([hidden_fn(toks + path_tokens(parents, drafts, i)) for i in range(K + 1)])
        a = argmax_fn(rows)
        j, app, _ = tree_accept(a, parents, drafts)
        js.append(j)
        toks.extend(app)
    if stats is not None:
        stats["accepted"] = js
    return toks[:target]
