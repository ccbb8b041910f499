"""GPU parity of tree verify (specverify_propose_tree / _accept_tree / _round_tree) against the
CPU oracle (oracle/tree.py): the drafter and the walk bit-exactly, the fused round against the
separate calls, a device-resident tree decoding loop against plain greedy decoding, and one
branch against the linear round."""
import numpy as np
import pytest
import torch

import oracle
from oracle import tree as tr
from weight_bound_verify_amd import specverify as sv
from weight_bound_verify_amd import synth

from gpu_util import check_argmax, dev, say, to_dev
from test_oracle_tree import _random_tree

pytestmark = pytest.mark.gpu


def _state(n):
    st = sv.new_state(dev())
    st[sv.STATE_LEN] = n
    return st


@pytest.mark.parametrize("n,vocab,nmax,K,B,D", [
    (1, 5, 3, 8, 2, 4), (2, 2, 3, 4, 4, 4), (40, 3, 3, 15, 4, 5), (300, 6, 3, 15, 3, 15),
    (300, 4, 2, 8, 1, 8), (513, 10, 4, 12, 4, 3), (4096, 50, 3, 15, 4, 6), (16000, 8, 3, 15, 2, 7),
    (20000, 5, 3, 10, 4, 10), (33000, 7, 3, 12, 3, 6),   # the last is longer than the LDS copy: global memory
])
def test_propose_tree_matches_oracle(n, vocab, nmax, K, B, D):
    rng = np.random.default_rng(n + K + B)
    for case in range(4):
        toks = rng.integers(0, vocab, size=n).astype(np.int32)
        tokens = to_dev(np.concatenate([toks, np.zeros(8, dtype=np.int32)]))
        state = _state(n)
        parents = torch.full((K,), -9, dtype=torch.int32, device=dev())
        drafts = torch.full((K,), -9, dtype=torch.int32, device=dev())
        sv.propose_tree(tokens, state, parents, drafts, nmax, B, D)
        torch.cuda.synchronize()
        p_ref, d_ref, used, real = tr.propose_tree(list(toks), nmax, K, B, D)
        assert parents.cpu().tolist() == p_ref and drafts.cpu().tolist() == d_ref, (case, n)
        st = state.cpu().numpy()
        assert st[sv.STATE_NVALID] == real and st[sv.STATE_NUSED] == used


@pytest.mark.parametrize("filler", [(1 << 27) - 3001, (1 << 27) + 5])
def test_propose_tree_long_stream_equals_its_live_part(filler):
    """A stream of 2^27 ids or more (the drafter's 64-bit key merge; shorter streams pack the
    (length, end) keys into 32 bits) and one just below: `filler` copies of an id the rest never
    uses, then a 3000-id Zipf context.  No n-gram that reaches into the filler matches the
    suffix, and match lengths and their order do not depend on where the context starts, so the
    tree equals the oracle's tree over the context alone."""
    V, nmax, K, B, D = 64, 3, 15, 4, 6
    ctx = synth.zipf_context_with_copies(np.random.default_rng(filler & 0xffff), 3000, V, 0.3)[0].astype(np.int32)
    say(f"propose_tree over {filler} filler ids + 3000")
    n = filler + ctx.size
    toks = np.full(n + 8, V + 1, dtype=np.int32)
    toks[filler:n] = ctx
    tokens = to_dev(toks)
    del toks
    state = _state(n)
    parents = torch.full((K,), -9, dtype=torch.int32, device=dev())
    drafts = torch.full((K,), -9, dtype=torch.int32, device=dev())
    sv.propose_tree(tokens, state, parents, drafts, nmax, B, D)
    torch.cuda.synchronize()
    p_ref, d_ref, used, real = tr.propose_tree(list(ctx), nmax, K, B, D)
    assert real > 0
    assert parents.cpu().tolist() == p_ref and drafts.cpu().tolist() == d_ref
    st = state.cpu().numpy()
    assert st[sv.STATE_NVALID] == real and st[sv.STATE_NUSED] == used
    del tokens
    torch.cuda.empty_cache()


def test_propose_tree_one_branch_is_the_linear_drafter():
    rng = np.random.default_rng(3)
    for case in range(20):
        n = int(rng.integers(2, 3000))
        toks = rng.integers(0, int(rng.integers(2, 30)), size=n).astype(np.int32)
        K = int(rng.integers(1, 16))
        tokens = to_dev(toks)
        st_a, st_b = _state(n), _state(n)
        parents = torch.empty(K, dtype=torch.int32, device=dev())
        d_tree = torch.empty(K, dtype=torch.int32, device=dev())
        d_lin = torch.empty(K, dtype=torch.int32, device=dev())
        sv.propose_tree(tokens, st_a, parents, d_tree, 3, 1, K)
        sv.propose(tokens, st_b, d_lin, 3)
        torch.cuda.synchronize()
        assert torch.equal(d_tree, d_lin) and torch.equal(st_a, st_b)
        real = int(st_a[sv.STATE_NVALID])
        assert parents.cpu().tolist() == list(range(real)) + [0] * (K - real)


def test_accept_tree_matches_oracle_random():
    rng = np.random.default_rng(4)
    for case in range(300):
        K = int(rng.integers(1, 16))
        V = int(rng.integers(2, 6))
        parents, drafts = _random_tree(rng, K, V)
        a = rng.integers(0, V, size=K + 1).astype(np.int32)
        len0 = int(rng.integers(1, 50))
        buf = np.full(len0 + K + 1 + 4, -5, dtype=np.int32)
        tokens = to_dev(buf)
        state = _state(len0)
        sv.accept_tree(to_dev(a), to_dev(np.array(parents, dtype=np.int32)),
                       to_dev(np.array(drafts, dtype=np.int32)), tokens, state)
        torch.cuda.synchronize()
        j, app, _ = tr.tree_accept(a, parents, drafts)
        out = tokens.cpu().numpy()
        st = state.cpu().numpy()
        assert st[sv.STATE_LEN] == len0 + 1 + j and st[sv.STATE_J] == j, case
        assert list(out[len0:len0 + j + 1]) == app, case
        assert np.all(out[len0 + j + 1:] == -5) and np.all(out[:len0] == -5)


def test_accept_tree_ignores_parents_that_do_not_precede_their_node():
    # node 2 names itself as parent, node 3 names node 4: neither can be walked to
    parents = [0, 2, 4, 3]
    drafts = [7, 8, 9, 6]
    a = np.array([7, 8, 9, 6, 1], dtype=np.int32)
    tokens = to_dev(np.zeros(16, dtype=np.int32))
    state = _state(2)
    sv.accept_tree(to_dev(a), to_dev(np.array(parents, dtype=np.int32)), to_dev(np.array(drafts, dtype=np.int32)),
                   tokens, state)
    torch.cuda.synchronize()
    assert int(state[sv.STATE_LEN]) == 4 and tokens[2:4].cpu().tolist() == [7, 8]


def test_accept_tree_capacity_overflow_writes_nothing():
    tokens = to_dev(np.full(8, -5, dtype=np.int32))
    state = _state(4)
    sv.accept_tree(to_dev(np.zeros(5, dtype=np.int32)), to_dev(np.zeros(4, dtype=np.int32)),
                   to_dev(np.zeros(4, dtype=np.int32)), tokens, state)
    torch.cuda.synchronize()
    assert int(state[sv.STATE_LEN]) == 4 and int(state[sv.STATE_FLAGS]) & sv.FLAG_CAPACITY
    assert tokens.cpu().tolist() == [-5] * 8


@pytest.mark.parametrize("ctx_len", [600, 32755, 40000])
def test_round_tree_equals_separate_calls(ctx_len):
    """The fused tree round against the separate calls, for streams below the tail's LDS copy
    (32768 ids), growing across it within the rounds, and above it (global memory)."""
    V, H, K, B, D = 5000, 1024, 8, 3, 4
    S = K + 1
    say(f"round_tree vs separate calls, context {ctx_len}")
    rng = np.random.default_rng(12)
    q, s = synth.quantized_head(np.random.SeedSequence(5), V, H)
    wq, ws = to_dev(q), to_dev(s)
    ctx = synth.zipf_context_with_copies(np.random.default_rng(3), ctx_len, V, 0.3)[0].astype(np.int32)
    cap = ctx_len + 1400
    work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())

    def fresh():
        t = torch.zeros(cap, dtype=torch.int32, device=dev())
        t[:len(ctx)] = to_dev(ctx)
        st = _state(len(ctx))
        p = torch.empty(K, dtype=torch.int32, device=dev())
        d = torch.empty(K, dtype=torch.int32, device=dev())
        sv.propose_tree(t, st, p, d, 3, B, D)
        return t, st, p, d

    ta, sa, pa, da = fresh()
    tb, sb, pb, db = fresh()
    am_a = torch.empty(S, dtype=torch.int32, device=dev())
    am_b = torch.empty(S, dtype=torch.int32, device=dev())
    for r in range(30):
        # rows favour the drafted tokens now and then so that some paths are accepted
        hidden = to_dev(synth.fp16_normal(rng, (S, H)))
        sv.round_tree(wq, ws, hidden, pa, da, ta, sa, pa, da, am_a, work, 3, B, D)
        sv.verify(wq, ws, hidden, am_b, work)
        sv.accept_tree(am_b, pb, db, tb, sb)
        sv.propose_tree(tb, sb, pb, db, 3, B, D)
        torch.cuda.synchronize()
        assert torch.equal(am_a, am_b) and torch.equal(sa, sb), r
        assert torch.equal(pa, pb) and torch.equal(da, db) and torch.equal(ta, tb), r
    assert int(sa[sv.STATE_ROUNDS]) == 30


def _device_tree_loop(q, s, table, ctx, n_new, K, B, D, linear=False):
    """Greedy tree decoding on the device: window rows gathered from the token-indexed table
    (the Markov stand-in: a node's row depends on its own token, which a tree attention mask
    preserves), one fused round per step, no host synchronisation inside a round."""
    V, H = q.shape
    S = K + 1
    cap = len(ctx) + n_new + 2 * S
    buf = np.zeros(cap, dtype=np.int32)
    buf[:len(ctx)] = ctx
    tokens = to_dev(buf)
    state = _state(len(ctx))
    wq, ws, tab = to_dev(q), to_dev(s), to_dev(table)
    work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    a0 = torch.empty(1, dtype=torch.int32, device=dev())
    argmax = torch.empty(S, dtype=torch.int32, device=dev())
    parents = torch.empty(K, dtype=torch.int32, device=dev())
    drafts = torch.empty(K, dtype=torch.int32, device=dev())
    window = torch.empty((S, H), dtype=torch.float16, device=dev())
    h_last = torch.empty((1, H), dtype=torch.float16, device=dev())
    sv.gather_window(tokens, state, drafts[:0], tab, h_last)
    sv.verify(wq, ws, h_last, a0, sv.workspace(sv.verify_workspace_bytes(V, H, 1), dev()))
    sv.accept(a0, None, tokens, state)                                  # anchor bootstrap
    if linear:
        sv.propose(tokens, state, drafts, 3)
    else:
        sv.propose_tree(tokens, state, parents, drafts, 3, B, D)
    rounds = 0
    while True:
        torch.cuda.synchronize()
        if int(state[sv.STATE_LEN]) >= len(ctx) + n_new:
            break
        sv.gather_window(tokens, state, drafts, tab, window)
        if linear:
            sv.round(wq, ws, window, drafts, tokens, state, drafts, argmax, work, 3)
        else:
            sv.round_tree(wq, ws, window, parents, drafts, tokens, state, parents, drafts, argmax, work, 3, B, D)
        rounds += 1
    torch.cuda.synchronize()
    n = int(state[sv.STATE_LEN])
    return tokens[:n].cpu().tolist(), state.cpu().numpy(), rounds


@pytest.mark.parametrize("V,H,K,B,D", [(4096, 512, 8, 2, 4), (2048, 256, 15, 4, 5), (512, 128, 6, 3, 2)])
def test_device_tree_loop_equals_greedy(V, H, K, B, D):
    say(f"tree loop V={V} H={H} K={K} B={B} D={D}")
    rng = np.random.default_rng(V + K + B)
    q, s = synth.quantized_head(np.random.SeedSequence(V), V, H)
    model = synth.MarkovHidden(rng, V, H)
    ctx, _, _ = synth.uniform_context_with_span(rng, 512, V, 12, 16)
    n_new = 200
    got, stv, rounds = _device_tree_loop(q, s, model.table, ctx, n_new, K, B, D)
    memo = {}

    def logits_after(t):
        if t not in memo:
            memo[t] = oracle.head_logits(q, s, model.table[t][None])
        return memo[t]

    ref = list(ctx)
    while len(ref) < len(got):
        ref.append(int(oracle.argmax_lowest(logits_after(ref[-1]))[0]))
    for p in range(len(ctx), len(got)):
        if got[p] != ref[p]:
            L = logits_after(got[p - 1])
            assert oracle.top2_gap(L)[0] < 1e-3 and got[p] in oracle.admissible_sets(L)[0], p
            break
    assert stv[sv.STATE_FLAGS] == 0
    say(f"  rounds {rounds}, tokens/round {(len(got) - len(ctx)) / max(rounds, 1):.2f}")
    assert rounds < n_new


def test_one_branch_tree_loop_equals_linear_loop():
    V, H, K = 2048, 256, 8
    rng = np.random.default_rng(7)
    q, s = synth.quantized_head(np.random.SeedSequence(9), V, H)
    model = synth.MarkovHidden(rng, V, H)
    ctx, _, _ = synth.uniform_context_with_span(rng, 400, V, 10, 12)
    a = _device_tree_loop(q, s, model.table, ctx, 150, K, 1, K)
    b = _device_tree_loop(q, s, model.table, ctx, 150, K, 1, K, linear=True)
    assert a[0] == b[0] and a[2] == b[2]
    assert np.array_equal(a[1][sv.STATE_HIST:sv.STATE_HIST + K + 1], b[1][sv.STATE_HIST:sv.STATE_HIST + K + 1])


def test_tree_rounds_replay_from_a_graph():
    """Tree rounds (gather the node rows, round_tree) captured once in a HIP graph and replayed
    three times continue the stream exactly like the same rounds run eagerly."""
    V, H, K, B, D, R = 2048, 256, 8, 3, 4, 6
    S = K + 1
    rng = np.random.default_rng(31)
    q, s = synth.quantized_head(np.random.SeedSequence(33), V, H)
    table = synth.MarkovHidden(rng, V, H).table
    ctx, _, _ = synth.uniform_context_with_span(rng, 300, V, 10, 8)
    cap = len(ctx) + 1 + 3 * R * S + 8

    class TreeLoop:
        def __init__(self):
            buf = np.zeros(cap, dtype=np.int32)
            buf[:len(ctx)] = ctx
            self.tokens = to_dev(buf)
            self.state = _state(len(ctx))
            self.wq, self.ws, self.tab = to_dev(q), to_dev(s), to_dev(table)
            self.work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
            self.argmax = torch.empty(S, dtype=torch.int32, device=dev())
            self.parents = torch.empty(K, dtype=torch.int32, device=dev())
            self.drafts = torch.empty(K, dtype=torch.int32, device=dev())
            self.window = torch.empty((S, H), dtype=torch.float16, device=dev())
            h_last = torch.empty((1, H), dtype=torch.float16, device=dev())
            a0 = torch.empty(1, dtype=torch.int32, device=dev())
            sv.gather_window(self.tokens, self.state, self.drafts[:0], self.tab, h_last)
            sv.verify(self.wq, self.ws, h_last, a0, sv.workspace(sv.verify_workspace_bytes(V, H, 1), dev()))
            sv.accept(a0, None, self.tokens, self.state)
            sv.propose_tree(self.tokens, self.state, self.parents, self.drafts, 3, B, D)

        def run(self, n):
            for _ in range(n):
                sv.gather_window(self.tokens, self.state, self.drafts, self.tab, self.window)
                sv.round_tree(self.wq, self.ws, self.window, self.parents, self.drafts, self.tokens, self.state,
                              self.parents, self.drafts, self.argmax, self.work, 3, B, D)

    eager = TreeLoop()
    eager.run(3 * R)
    torch.cuda.synchronize()
    g = TreeLoop()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            g.run(R)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for _ in range(3):
        graph.replay()
        torch.cuda.synchronize()
        _ = (g.state[sv.STATE_LEN] + 1).item()          # eager work between replays
    assert torch.equal(g.tokens, eager.tokens) and torch.equal(g.state, eager.state)
    assert torch.equal(g.parents, eager.parents) and torch.equal(g.drafts, eager.drafts)


def test_tree_rounds_hit_rate_gate():
    """gate_after = 2 with rows that never take a draft: the gate fires after the second round
    and every later tree is pads, even when the stream's end would give the drafter a match."""
    V, H, K, B, D = 3000, 256, 8, 3, 4
    S = K + 1
    rng = np.random.default_rng(51)
    q, s = synth.quantized_head(np.random.SeedSequence(52), V, H)
    wq, ws = to_dev(q), to_dev(s)
    ctx = np.tile(np.arange(1, 40, dtype=np.int32), 10)            # repetitive: the branches share one path
    tokens = torch.zeros(len(ctx) + 64, dtype=torch.int32, device=dev())
    tokens[:len(ctx)] = to_dev(ctx)
    state = _state(len(ctx))
    state[sv.STATE_GATE_AFTER] = 2
    parents = torch.empty(K, dtype=torch.int32, device=dev())
    drafts = torch.empty(K, dtype=torch.int32, device=dev())
    argmax = torch.empty(S, dtype=torch.int32, device=dev())
    work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    sv.propose_tree(tokens, state, parents, drafts, 3, B, D)
    torch.cuda.synchronize()
    assert drafts.cpu().tolist() == [1, 2, 3, 4, -1, -1, -1, -1]
    hidden = to_dev(synth.fp16_normal(rng, (S, H)))
    for r in range(4):
        sv.round_tree(wq, ws, hidden, parents, drafts, tokens, state, parents, drafts, argmax, work, 3, B, D)
        torch.cuda.synchronize()
        if int(state[sv.STATE_J]) != 0:
            pytest.skip("a draft happened to match the synthetic rows")
    st = state.cpu().numpy()
    assert st[sv.STATE_GATED] == 2 and st[sv.STATE_ZERO_RUN] == 4 and st[sv.STATE_ROUNDS] == 4
    assert drafts.cpu().tolist() == [-1] * K and parents.cpu().tolist() == [0] * K
    # end the stream in a token the context repeats: gated, the drafter still emits pads ...
    n = int(st[sv.STATE_LEN])
    tokens[n - 1] = int(ctx[-1])
    sv.propose_tree(tokens, state, parents, drafts, 3, B, D)
    torch.cuda.synchronize()
    assert drafts.cpu().tolist() == [-1] * K
    # ... and with the gate cleared it proposes again
    state[sv.STATE_GATED] = 0
    sv.propose_tree(tokens, state, parents, drafts, 3, B, D)
    torch.cuda.synchronize()
    assert (drafts.cpu().numpy() >= 0).any()


def test_round_tree_full_35b_head_shape():
    """One tree round at the full 35B-A3B-shaped head (V = 248320, H = 2048), 8 nodes from the
    3 best matches at depth 4, in the launch configuration the bench uses: the argmax rows
    against the oracle's logits (near-tie rule), then the walk (rows steered down a real
    path), the committed stream and the next tree bit-exactly against the oracle applied to
    the GPU's argmax rows."""
    V, H, K, B, D = 248320, 2048, 8, 3, 4
    S = K + 1
    say(f"round_tree full V={V} H={H} K={K} B={B} D={D}")
    q, s = synth.quantized_head(synth.streams(2).weights, V, H)
    ctx = synth.zipf_context_with_copies(np.random.default_rng(35), 4096, V, 0.3)[0].astype(np.int32)
    parents0, drafts0, _, real = tr.propose_tree(ctx, 3, K, B, D)
    assert real == K and sum(p == 0 for p in parents0) >= 2       # a full tree that branches at the root
    # row c steers the argmax to the token of node c's highest-index child (a leaf: a random
    # id): fp16(50 x the dequantised weight row) wins by a wide margin, so the walk leaves the
    # first branch and goes down to a leaf
    rng = np.random.default_rng(31)

    def steer(tok):
        d = (q[tok].astype(np.float64).reshape(-1, 32) * s[tok].astype(np.float64)[:, None]).reshape(-1)
        return (50.0 * d).astype(np.float16)

    rows = []
    for c in range(S):
        kids = [i for i in range(1, K + 1) if parents0[i - 1] == c and drafts0[i - 1] != -1]
        rows.append(steer(drafts0[kids[-1] - 1] if kids else int(rng.integers(0, V))))
    hidden = np.stack(rows)
    cap = len(ctx) + 64
    tokens = torch.zeros(cap, dtype=torch.int32, device=dev())
    tokens[:len(ctx)] = to_dev(ctx)
    state = _state(len(ctx))
    parents = torch.empty(K, dtype=torch.int32, device=dev())
    drafts = torch.empty(K, dtype=torch.int32, device=dev())
    sv.propose_tree(tokens, state, parents, drafts, 3, B, D)
    torch.cuda.synchronize()
    assert parents.cpu().tolist() == list(parents0) and drafts.cpu().tolist() == list(drafts0)
    argmax = torch.empty(S, dtype=torch.int32, device=dev())
    work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    sv.round_tree(to_dev(q), to_dev(s), to_dev(hidden), parents, drafts, tokens, state, parents, drafts, argmax,
                  work, 3, B, D)
    torch.cuda.synchronize()
    a_gpu = argmax.cpu().numpy()
    L = oracle.head_logits(q, s, hidden)
    check_argmax(a_gpu, L)
    j, app, path = tr.tree_accept(a_gpu, parents0, drafts0)
    assert j >= 2 and path[0] != 1
    st = state.cpu().numpy()
    assert st[sv.STATE_J] == j and st[sv.STATE_LEN] == len(ctx) + 1 + j
    stream = list(ctx) + app
    assert tokens[:len(stream)].cpu().tolist() == stream
    p1, d1, _, _ = tr.propose_tree(stream, 3, K, B, D)
    assert parents.cpu().tolist() == list(p1) and drafts.cpu().tolist() == list(d1)


def test_generate_tree_equals_round_by_round():
    """specverify_generate_tree over R rounds leaves the stream, the state word and the next
    tree bit-identical to R calls of gather_window + round_tree (the loop the greedy-equality
    test above checks against plain greedy decoding)."""
    V, H, K, B, D, R = 4096, 512, 8, 3, 4, 150
    S = K + 1
    rng = np.random.default_rng(81)
    q, s = synth.quantized_head(np.random.SeedSequence(82), V, H)
    model = synth.MarkovHidden(rng, V, H)
    ctx, _, _ = synth.uniform_context_with_span(rng, 512, V, 12, 16)
    wq, ws, tab = to_dev(q), to_dev(s), to_dev(model.table)
    cap = len(ctx) + R * S + 8

    def fresh():
        t = torch.zeros(cap, dtype=torch.int32, device=dev())
        t[:len(ctx)] = to_dev(ctx)
        st = _state(len(ctx))
        h_last = torch.empty((1, H), dtype=torch.float16, device=dev())
        a0 = torch.empty(1, dtype=torch.int32, device=dev())
        sv.gather_window(t, st, torch.empty(0, dtype=torch.int32, device=dev()), tab, h_last)
        sv.verify(wq, ws, h_last, a0, sv.workspace(sv.verify_workspace_bytes(V, H, 1), dev()))
        sv.accept(a0, None, t, st)
        p = torch.empty(K, dtype=torch.int32, device=dev())
        d = torch.empty(K, dtype=torch.int32, device=dev())
        sv.propose_tree(t, st, p, d, 3, B, D)
        return t, st, p, d

    work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    window = torch.empty((S, H), dtype=torch.float16, device=dev())
    argmax = torch.empty(S, dtype=torch.int32, device=dev())
    ta, sa, pa, da = fresh()
    sv.generate_tree(wq, ws, tab, ta, sa, pa, da, window, argmax, work, R, 3, B, D)
    tb, sb, pb, db = fresh()
    for _ in range(R):
        sv.gather_window(tb, sb, db, tab, window)
        sv.round_tree(wq, ws, window, pb, db, tb, sb, pb, db, argmax, work, 3, B, D)
    torch.cuda.synchronize()
    assert int(sa[sv.STATE_ROUNDS]) == R and int(sa[sv.STATE_FLAGS]) == 0
    assert torch.equal(sa, sb) and torch.equal(ta, tb) and torch.equal(pa, pb) and torch.equal(da, db)
    assert int(sa[sv.STATE_SUMJ]) > 0                              # the tree drafter took drafts
