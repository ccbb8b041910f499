"""GPU parity of the device-resident generation loop (specverify_generate: gather the window
from a token-indexed stand-in model, verify, accept, draft, R rounds with no host sync) and of
the hit-rate gate, against the oracle's speculative decoding driver and plain greedy decoding."""
import numpy as np
import pytest
import torch

import oracle
from weight_bound_verify_amd import specverify as sv
from weight_bound_verify_amd import synth

from gpu_util import dev, say, to_dev

pytestmark = pytest.mark.gpu


class Loop:
    """Device buffers of one generation: anchor bootstrap and first drafts done on creation."""

    def __init__(self, q, s, table, ctx, K, n_max, gate_after, cap):
        V, H = q.shape
        self.K, self.n_max = K, n_max
        buf = np.zeros(cap, dtype=np.int32)
        buf[:len(ctx)] = ctx
        self.tokens = to_dev(buf)
        self.state = sv.new_state(dev())
        self.state[sv.STATE_LEN] = len(ctx)
        self.state[sv.STATE_GATE_AFTER] = gate_after
        self.wq, self.ws, self.table = to_dev(q), to_dev(s), to_dev(table)
        self.work = sv.workspace(sv.verify_workspace_bytes(V, H, K + 1), dev())
        self.drafts = torch.empty(K, dtype=torch.int32, device=dev())
        self.window = torch.empty((K + 1, H), dtype=torch.float16, device=dev())
        self.argmax = torch.empty(K + 1, dtype=torch.int32, device=dev())
        a0 = torch.empty(1, dtype=torch.int32, device=dev())
        w0 = torch.empty((1, H), dtype=torch.float16, device=dev())
        sv.gather_window(self.tokens, self.state, self.drafts[:0], self.table, w0)      # anchor row only
        sv.verify(self.wq, self.ws, w0, a0, sv.workspace(sv.verify_workspace_bytes(V, H, 1), dev()))
        sv.accept(a0, None, self.tokens, self.state)
        sv.propose(self.tokens, self.state, self.drafts, n_max)

    def run(self, rounds):
        sv.generate(self.wq, self.ws, self.table, self.tokens, self.state, self.drafts, self.window, self.argmax,
                    self.work, rounds, self.n_max)

    def result(self):
        torch.cuda.synchronize()
        st = self.state.cpu().numpy().copy()
        return self.tokens[:st[sv.STATE_LEN]].cpu().tolist(), st


def _oracle(q, s, table, ctx, K, n_max, gate_after, n_tokens):
    memo = {}

    def argmax_fn(rows):
        out = []
        for r in rows:
            key = r.tobytes()
            if key not in memo:
                memo[key] = int(oracle.argmax_lowest(oracle.head_logits(q, s, r[None]))[0])
            out.append(memo[key])
        return np.array(out)

    model = lambda prefix: table[int(prefix[-1])]
    st = {}
    toks = oracle.spec_decode(list(ctx), model, argmax_fn, n_tokens, K, n_max, stats=st, gate_after=gate_after)
    return toks, st


def _tied(q, s, table, got, ctx):
    """Every position where the device stream left greedy decoding must be a near tie."""
    for p in range(len(ctx), len(got)):
        L = oracle.head_logits(q, s, table[got[p - 1]][None])
        if got[p] != int(oracle.argmax_lowest(L)[0]):
            assert oracle.top2_gap(L)[0] < 1e-3 and got[p] in oracle.admissible_sets(L)[0], p
            return p
    return None


@pytest.mark.parametrize("V,H,K,n_max,gate", [(8192, 512, 8, 3, 0), (2048, 256, 4, 2, 0), (512, 128, 16, 3, 2),
                                              (3000, 1024, 8, 3, 1), (777, 2048, 3, 1, 3)])
def test_generate_equals_oracle_spec_decode(V, H, K, n_max, gate):
    say(f"generate V={V} H={H} K={K} n={n_max} gate={gate}")
    rng = np.random.default_rng(V + 7 * K)
    q, s = synth.quantized_head(np.random.SeedSequence(V + H), V, H)
    table = synth.MarkovHidden(rng, V, H).table
    ctx, _, _ = synth.uniform_context_with_span(rng, 300, V, 12, 8)
    R = 60
    loop = Loop(q, s, table, ctx, K, n_max, gate, cap=len(ctx) + 1 + R * (K + 1) + 8)
    loop.run(R)
    got, st = loop.result()
    assert st[sv.STATE_FLAGS] == 0 and st[sv.STATE_ROUNDS] == R
    ref, ost = _oracle(q, s, table, ctx, K, n_max, gate, len(got) - len(ctx) + R * (K + 1))
    if _tied(q, s, table, got, ctx) is None:
        # identical greedy ids: the stream, every round's j and the gate round match exactly
        assert got == ref[:len(got)]
        js = ost["accepted"][:R]
        assert [int(st[sv.STATE_HIST + j]) for j in range(K + 1)] == [js.count(j) for j in range(K + 1)]
        assert st[sv.STATE_SUMJ] == sum(js)
        g = ost["gated_after_round"]
        assert st[sv.STATE_GATED] == (g if g is not None and g <= R else 0)
    say(f"  rounds {R}, tokens {len(got) - len(ctx)}, sum j {st[sv.STATE_SUMJ]}, gated at {st[sv.STATE_GATED]}")


def test_gate_drops_the_drafter_and_stays_lossless():
    """A context with no repeats and a gate of 1: the first zero-accept round drops the
    drafter; every later round commits exactly one token and drafts only pads."""
    rng = np.random.default_rng(3)
    V, H, K = 4096, 256, 8
    q, s = synth.quantized_head(np.random.SeedSequence(44), V, H)
    table = synth.MarkovHidden(rng, V, H).table
    ctx = rng.permutation(V)[:200].astype(np.int32)
    R = 30
    loop = Loop(q, s, table, ctx, K, 3, 1, cap=len(ctx) + 1 + R * (K + 1) + 8)
    loop.run(R)
    got, st = loop.result()
    assert st[sv.STATE_GATED] >= 1
    assert (loop.drafts.cpu().numpy() == -1).all() and st[sv.STATE_NVALID] == 0
    gated = int(st[sv.STATE_GATED])
    assert st[sv.STATE_HIST] >= R - gated + 1           # every round from the gating one on accepts nothing
    if _tied(q, s, table, got, ctx) is None:
        ref, ost = _oracle(q, s, table, ctx, K, 3, 1, len(got) - len(ctx))
        assert got == ref[:len(got)]
        assert ost["gated_after_round"] == gated


def test_graph_replay_equals_eager_rounds():
    """R rounds captured once in a HIP graph and replayed three times (eager work and a
    synchronisation between replays) continue the stream exactly like 3R eager rounds."""
    rng = np.random.default_rng(11)
    V, H, K, R = 2048, 512, 8, 10
    q, s = synth.quantized_head(np.random.SeedSequence(5), V, H)
    table = synth.MarkovHidden(rng, V, H).table
    ctx, _, _ = synth.uniform_context_with_span(rng, 256, V, 12, 8)
    cap = len(ctx) + 1 + 3 * R * (K + 1) + 8
    eager = Loop(q, s, table, ctx, K, 3, 0, cap)
    eager.run(3 * R)
    want, st_e = eager.result()

    g = Loop(q, s, table, ctx, K, 3, 0, cap)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        tokens0 = g.tokens.clone()
        state0 = g.state.clone()
        drafts0 = g.drafts.clone()
        with torch.cuda.graph(graph, stream=side):
            g.run(R)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    # capture does not execute: restore nothing was changed, then replay
    assert torch.equal(g.tokens, tokens0) and torch.equal(g.state, state0) and torch.equal(g.drafts, drafts0)
    for _ in range(3):
        graph.replay()
        torch.cuda.synchronize()
        _ = (g.state[sv.STATE_LEN] + 1).item()          # eager work between replays
    got, st_g = g.result()
    assert got == want
    assert np.array_equal(st_g, st_e)


@pytest.mark.parametrize("V,H,K,n_max", [(5000, 512, 8, 3), (30000, 1024, 4, 3), (2048, 256, 16, 2)])
def test_script_target_rounds_equal_oracle_spec_decode(V, H, K, n_max):
    """The stand-in target whose greedy continuation is a fixed script (Zipf ids with 30% copied
    spans; the window row at position p is the sign pattern of the scripted id's code row), run
    round after round on the device (specverify_gather_positions picks the window from the
    state word, then the fused round), against oracle.spec_decode with the same target: identical committed streams,
    accept length per round and histogram; greedy decoding of the target reproduces the script;
    the acceptance rate lies strictly between 0 and 1."""
    say(f"script target V={V} H={H} K={K} n={n_max}")
    S = K + 1
    rng = np.random.default_rng(V + K)
    q, s = synth.quantized_head(np.random.SeedSequence(V + H), V, H)
    ctx_len, rounds = 600, 120
    script, _ = synth.zipf_context_with_copies(rng, ctx_len + rounds * S + 2 * S, V, 0.3)
    model = synth.ScriptHidden(q, script)
    rows = to_dev(model.rows())
    cap = len(script)
    buf = np.zeros(cap, np.int32)
    buf[:ctx_len] = script[:ctx_len]
    tokens, state = to_dev(buf), sv.new_state(dev())
    state[sv.STATE_LEN] = ctx_len
    wq, ws = to_dev(q), to_dev(s)
    work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    a0 = torch.empty(1, dtype=torch.int32, device=dev())
    sv.verify(wq, ws, rows[ctx_len - 1:ctx_len].clone(), a0, sv.workspace(sv.verify_workspace_bytes(V, H, 1), dev()))
    sv.accept(a0, None, tokens, state)
    drafts = torch.empty(K, dtype=torch.int32, device=dev())
    sv.propose(tokens, state, drafts, n_max)
    window = torch.empty((S, H), dtype=torch.float16, device=dev())
    am = torch.empty(S, dtype=torch.int32, device=dev())
    js = []
    for _ in range(rounds):
        sv.gather_positions(state, cap, rows, window)
        sv.round(wq, ws, window, drafts, tokens, state, drafts, am, work, n_max)
        js.append(state[sv.STATE_J].clone())
    torch.cuda.synchronize()
    st = state.cpu().numpy()
    assert st[sv.STATE_FLAGS] == 0 and st[sv.STATE_ROUNDS] == rounds
    n = int(st[sv.STATE_LEN])
    got = tokens[:n].cpu().tolist()
    assert got == script[:n].tolist(), "greedy decoding of the script target is the script"

    def argmax_fn(rws):
        return oracle.argmax_lowest(oracle.head_logits(q, s, rws))

    stats = {}
    ref = oracle.spec_decode(script[:ctx_len].tolist(), model, argmax_fn, n - ctx_len, K, n_max, stats=stats)
    assert got == ref
    j_dev = [int(j) for j in torch.stack(js).cpu().tolist()]
    assert j_dev == stats["accepted"][:rounds]
    hist = np.bincount(j_dev, minlength=K + 1)
    assert hist.tolist() == st[sv.STATE_HIST:sv.STATE_HIST + K + 1].tolist()
    alpha = sum(j_dev) / (sum(j_dev) + int(hist[:K].sum()))
    assert 0.0 < alpha < 1.0, alpha


def test_gather_positions_rows_and_out_of_range():
    """window[i] = rows[len - 1 + i]; a position past the rows or a bad length writes a zero row
    and sets the capacity flag."""
    rows = to_dev(synth.fp16_normal(np.random.default_rng(5), (40, 256)))
    win = torch.full((5, 256), float("nan"), dtype=torch.float16, device=dev())
    st = sv.new_state(dev())
    st[sv.STATE_LEN] = 10
    sv.gather_positions(st, 100, rows, win)
    torch.cuda.synchronize()
    assert torch.equal(win, rows[9:14]) and int(st[sv.STATE_FLAGS]) == 0
    st[sv.STATE_LEN] = 38                                  # positions 37 .. 41: the last two are past the rows
    sv.gather_positions(st, 100, rows, win)
    torch.cuda.synchronize()
    assert torch.equal(win[:3], rows[37:40]) and not win[3:].any()
    assert int(st[sv.STATE_FLAGS]) == sv.FLAG_CAPACITY
    st[sv.STATE_FLAGS] = 0
    st[sv.STATE_LEN] = 101                                 # longer than the token buffer
    sv.gather_positions(st, 100, rows, win)
    torch.cuda.synchronize()
    assert not win.any() and int(st[sv.STATE_FLAGS]) == sv.FLAG_CAPACITY
