"""GPU parity of sampling verify (specverify_verify_sample / _accept_sample / _round_sample)
against the CPU oracle (oracle/sampling.py), plus the law of the device's draws.

Comparison rule.  The oracle works in fp64 on exact logits; the device in fp32.  A row's draw
must equal the oracle's unless the oracle's two best residual keys lie within the keys'
tolerance (logit tolerance / T plus the noise's fp32 error), and then it must be one of the
keys within that tolerance of the best.  A draft's keep/reject decision must equal the
oracle's unless |u - p(d)| is within p's tolerance.  Accept and propose are then compared
exactly against the oracle applied to the device's own draws and decisions."""
import numpy as np
import pytest
import torch
from scipy.stats import chi2

import oracle
from oracle import sampling as smp
from weight_bound_verify_amd import specverify as sv
from weight_bound_verify_amd import synth

from gpu_util import TOL, check_logits, dev, head, say, to_dev

pytestmark = pytest.mark.gpu

NOISE_TOL = 1e-4        # fp32 -log(-log u) against fp64, absolute


def _keys(L, drafts, T, seed, P0):
    """Oracle residual keys [S, V]: log r_s(v) - log(-log u_s(v)), -inf off the support."""
    S, V = L.shape
    p, _ = smp.probabilities(L, T)
    un = smp.noise_uniforms(seed, P0, S, V)
    keys = np.full((S, V), -np.inf)
    for s in range(S):
        d = drafts[s] if s < S - 1 else -1
        r = smp.residual(p[s], d)
        sup = r > 0
        keys[s, sup] = np.log(r[sup]) - np.log(-np.log(un[s, sup]))
    return keys


def _key_tol(L, T):
    floor = np.sqrt(np.mean(L * L, axis=1))
    return 2 * TOL * np.maximum(np.abs(L).max(axis=1), floor) / T + NOISE_TOL


def check_draws(sample, L, drafts, T, seed, P0):
    keys = _keys(L, drafts, T, seed, P0)
    tol = _key_tol(L, T)
    ambiguous = 0
    for s in range(L.shape[0]):
        order = np.argsort(-keys[s], kind="stable")
        best = int(order[0])
        if sample[s] == best:
            continue
        gap = keys[s, best] - keys[s, order[1]]
        assert gap < tol[s] and keys[s, sample[s]] >= keys[s, best] - tol[s], \
            f"row {s}: device draw {sample[s]} oracle {best} gap {gap:.3g} tol {tol[s]:.3g}"
        ambiguous += 1
    return ambiguous


def _setup(V, H, S, seed, P0, match=0.5):
    q, s = head(V * 13 + H + S, V, H)
    rng = np.random.default_rng(seed)
    hidden = synth.fp16_normal(rng, (S, H))
    L = oracle.head_logits(q, s, hidden)
    # drafts: the row's argmax with probability `match` (so p(d) is large), else a random id
    # or a pad
    greedy = oracle.argmax_lowest(L)
    drafts = []
    for i in range(S - 1):
        x = rng.random()
        drafts.append(int(greedy[i]) if x < match else (-1 if x > 0.9 else int(rng.integers(0, V))))
    return q, s, hidden, L, drafts


def gpu_verify_sample(q, s, hidden, drafts, T, seed, P0, logits=True):
    V, H = q.shape
    S = hidden.shape[0]
    state = sv.new_state(dev())
    state[sv.STATE_LEN] = P0
    dr = to_dev(np.array(drafts + [0], dtype=np.int32))
    sample = torch.full((S,), -7, dtype=torch.int32, device=dev())
    lse = torch.full((S,), float("nan"), dtype=torch.float32, device=dev())
    zd = torch.full((S,), float("nan"), dtype=torch.float32, device=dev())
    lg = torch.full((S, V), float("nan"), dtype=torch.float32, device=dev()) if logits else None
    work = sv.workspace(sv.sample_workspace_bytes(V, H, S), dev())
    sv.verify_sample(to_dev(q), to_dev(s), to_dev(hidden), dr, T, seed, state, sample, lse, zd, work, lg)
    torch.cuda.synchronize()
    return (sample.cpu().numpy(), lse.cpu().numpy().astype(np.float64), zd.cpu().numpy().astype(np.float64),
            lg.cpu().numpy().astype(np.float64) if logits else None)


SHAPES = [
    (1000, 256, 1, 1.0), (3000, 512, 9, 0.7), (8192 + 37, 2048, 9, 1.0), (2048, 1024, 16, 0.5),
    (4099, 320, 5, 1.3), (300, 16384, 4, 0.9),      # the last splits the hidden axis (combine pass)
]


@pytest.mark.parametrize("V,H,S,T", SHAPES)
def test_verify_sample_matches_oracle(V, H, S, T):
    say(f"verify_sample V={V} H={H} S={S} T={T}")
    seed, P0 = (V * 7919 + S) | (1 << 40), 1234 + S
    q, s, hidden, L, drafts = _setup(V, H, S, 3, P0)
    sample, lse, zd, lg = gpu_verify_sample(q, s, hidden, drafts, T, seed, P0)
    check_logits(lg, L)
    _, lse_o = smp.probabilities(L, T)
    ltol = _key_tol(L, T)
    assert np.all(np.abs(lse - lse_o) <= ltol), (lse, lse_o)
    for r, d in enumerate(drafts):
        if 0 <= d < V:
            assert abs(zd[r] - L[r, d] / T) <= ltol[r]
    amb = check_draws(sample, L, drafts, T, seed, P0)
    say(f"  ambiguous draws {amb}")


def test_accept_sample_matches_oracle_decisions():
    """Many windows: the device's keep/reject decisions and appended tokens against the oracle
    applied to the device's own draws."""
    V, H, S, T = 3000, 512, 9, 0.1        # a peaked target: p(argmax) is large, so drafts are kept
    rng = np.random.default_rng(11)
    q, s = head(77, V, H)
    wq, ws = to_dev(q), to_dev(s)
    K = S - 1
    work = sv.workspace(sv.sample_workspace_bytes(V, H, S), dev())
    kept_total = rejected_total = 0
    for case in range(24):
        seed = int(rng.integers(0, 2 ** 63))
        P0 = int(rng.integers(20, 900))
        hidden = synth.fp16_normal(rng, (S, H))
        L = oracle.head_logits(q, s, hidden)
        greedy = oracle.argmax_lowest(L)
        drafts = [int(greedy[i]) if rng.random() < 0.7 else int(rng.integers(0, V)) for i in range(K)]
        stream = rng.integers(0, V, size=P0).astype(np.int32)
        tokens = torch.zeros(P0 + 64, dtype=torch.int32, device=dev())
        tokens[:P0] = to_dev(stream)
        state = sv.new_state(dev())
        state[sv.STATE_LEN] = P0
        dr = to_dev(np.array(drafts, dtype=np.int32))
        sample = torch.empty(S, dtype=torch.int32, device=dev())
        lse = torch.empty(S, dtype=torch.float32, device=dev())
        zd = torch.empty(S, dtype=torch.float32, device=dev())
        sv.verify_sample(wq, ws, to_dev(hidden), dr, T, seed, state, sample, lse, zd, work)
        sv.accept_sample(sample, lse, zd, dr, V, seed, tokens, state)
        torch.cuda.synchronize()
        smp_d = sample.cpu().numpy()
        check_draws(smp_d, L, drafts, T, seed, P0)
        p, lse_o = smp.probabilities(L, T)
        u = smp.accept_uniforms(seed, P0, K)
        ltol = _key_tol(L, T)
        st = state.cpu().numpy()
        j = int(st[sv.STATE_J])
        for i in range(j + 1 if j < K else K):
            pd = p[i, drafts[i]]
            want = u[i] < pd
            got = i < j
            if want != got:
                assert abs(u[i] - pd) <= 2.5 * ltol[i] * pd + 1e-6, f"case {case} row {i}: u {u[i]} p {pd}"
        out = tokens.cpu().numpy()
        assert st[sv.STATE_LEN] == P0 + 1 + j
        assert list(out[P0:P0 + j + 1]) == drafts[:j] + [int(smp_d[j])]
        assert np.array_equal(out[:P0], stream)
        kept_total += j
        rejected_total += j < K
    assert kept_total > 0 and rejected_total > 0


@pytest.mark.parametrize("ctx_len", [600, 32755, 40000])
def test_round_sample_equals_separate_calls(ctx_len):
    """The fused sampling round against the separate calls, for streams below the round tail's
    LDS copy (32768 ids), growing across it within the rounds, and above it (the tail's
    global-memory path)."""
    V, H, K, T = 5000, 1024, 8, 0.9
    S = K + 1
    say(f"round_sample vs separate calls, context {ctx_len}")
    rng = np.random.default_rng(12)
    q, s = head(5, V, H)
    wq, ws = to_dev(q), to_dev(s)
    ctx = synth.zipf_context_with_copies(np.random.default_rng(3), ctx_len, V, 0.3)[0].astype(np.int32)
    cap = ctx_len + 1400
    work = sv.workspace(sv.sample_workspace_bytes(V, H, S), dev())

    def fresh():
        t = torch.zeros(cap, dtype=torch.int32, device=dev())
        t[:len(ctx)] = to_dev(ctx)
        st = sv.new_state(dev())
        st[sv.STATE_LEN] = len(ctx)
        d = torch.empty(K, dtype=torch.int32, device=dev())
        sv.propose(t, st, d, 3)
        return t, st, d

    ta, sa, da = fresh()
    tb, sb, db = fresh()
    samp_a = torch.empty(S, dtype=torch.int32, device=dev())
    lse_a = torch.empty(S, dtype=torch.float32, device=dev())
    samp_b, lse_b = torch.empty_like(samp_a), torch.empty_like(lse_a)
    zd_b = torch.empty(S, dtype=torch.float32, device=dev())
    for r in range(30):
        hidden = to_dev(synth.fp16_normal(rng, (S, H)))
        seed = 1000 + r
        sv.round_sample(wq, ws, hidden, da, T, seed, ta, sa, da, work, 3, samp_a, lse_a)
        sv.verify_sample(wq, ws, hidden, db, T, seed, sb, samp_b, lse_b, zd_b, work)
        sv.accept_sample(samp_b, lse_b, zd_b, db, V, seed, tb, sb)
        sv.propose(tb, sb, db, 3)
        torch.cuda.synchronize()
        assert torch.equal(samp_a, samp_b) and torch.equal(lse_a, lse_b), r
        assert torch.equal(sa, sb) and torch.equal(da, db), r
        assert torch.equal(ta, tb), r
    assert int(sa[sv.STATE_ROUNDS]) == 30


def test_zero_temperature_limit_is_the_greedy_round():
    """T -> 0: the sampling round commits exactly what the greedy round commits wherever the
    top-2 logit gap is far above the noise scale times T."""
    V, H, K = 4000, 512, 8
    S = K + 1
    T = 1e-6
    rng = np.random.default_rng(13)
    q, s = head(6, V, H)
    wq, ws = to_dev(q), to_dev(s)
    ws_g = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    ws_s = sv.workspace(sv.sample_workspace_bytes(V, H, S), dev())
    checked = 0
    for r in range(20):
        hidden = synth.fp16_normal(rng, (S, H))
        L = oracle.head_logits(q, s, hidden)
        if oracle.top2_gap(L).min() < 1e-4:
            continue
        greedy = oracle.argmax_lowest(L)
        j_forced = int(rng.integers(0, K + 1))
        drafts = [int(greedy[i]) if i < j_forced else int((greedy[i] + 1) % V) for i in range(K)]
        res = []
        for sampling in (False, True):
            t = torch.zeros(256, dtype=torch.int32, device=dev())
            st = sv.new_state(dev())
            st[sv.STATE_LEN] = 100
            din = to_dev(np.array(drafts, dtype=np.int32))
            dout = torch.empty(K, dtype=torch.int32, device=dev())
            if sampling:
                sv.round_sample(wq, ws, to_dev(hidden), din, T, 99 + r, t, st, dout, ws_s)
            else:
                am = torch.empty(S, dtype=torch.int32, device=dev())
                sv.round(wq, ws, to_dev(hidden), din, t, st, dout, am, ws_g)
            torch.cuda.synchronize()
            res.append((t.cpu().numpy().copy(), st.cpu().numpy().copy()))
        assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
        assert res[1][1][sv.STATE_J] == j_forced
        checked += 1
    assert checked >= 10


def test_device_draws_follow_softmax():
    """Law of the device's draws (independent of the oracle's generator): over many rounds
    (each with its own start position) the bonus row's draws are distributed as softmax(L/T)."""
    V, H, T = 24, 64, 1.0
    q, s = head(8, V, H)
    rng = np.random.default_rng(14)
    hidden = synth.fp16_normal(rng, (1, H)) * np.float16(4.0)
    L = oracle.head_logits(q, s, hidden.astype(np.float16))
    p, _ = smp.probabilities(L, T)
    wq, ws, hd = to_dev(q), to_dev(s), to_dev(hidden.astype(np.float16))
    work = sv.workspace(sv.sample_workspace_bytes(V, H, 1), dev())
    n = 4000
    state = sv.new_state(dev())
    draws = torch.empty((n,), dtype=torch.int32, device=dev())
    lse = torch.empty(1, dtype=torch.float32, device=dev())
    zd = torch.empty(1, dtype=torch.float32, device=dev())
    for i in range(n):
        state[sv.STATE_LEN] = 10 + i
        sv.verify_sample(wq, ws, hd, None, T, 5, state, draws[i:i + 1], lse, zd, work)
    torch.cuda.synchronize()
    counts = np.bincount(draws.cpu().numpy(), minlength=V).astype(np.float64)
    exp = p[0] * n
    keep = exp >= 5
    c = np.append(counts[keep], counts[~keep].sum())
    e = np.append(exp[keep], exp[~keep].sum())
    stat = ((c - e) ** 2 / np.maximum(e, 1e-12)).sum()
    assert chi2.sf(stat, len(c) - 1) > 1e-3, (counts, exp)


@pytest.mark.parametrize("V,H", [(248320, 2048)])
def test_verify_sample_full_35b_head_shape(V, H):
    """The 35B-A3B-shaped head at full size, in the launch configuration the bench uses."""
    S, T = 9, 0.7
    say(f"verify_sample full V={V} H={H}")
    seed, P0 = 0x1234_5678_9ABC, 4096
    q, s = synth.quantized_head(synth.streams(2).weights, V, H)
    rng = np.random.default_rng(21)
    hidden = synth.fp16_normal(rng, (S, H))
    L = oracle.head_logits(q, s, hidden)
    greedy = oracle.argmax_lowest(L)
    drafts = [int(greedy[i]) if i % 3 else int(rng.integers(0, V)) for i in range(S - 1)]
    sample, lse, zd, _ = gpu_verify_sample(q, s, hidden, drafts, T, seed, P0, logits=False)
    _, lse_o = smp.probabilities(L, T)
    assert np.all(np.abs(lse - lse_o) <= _key_tol(L, T))
    check_draws(sample, L, drafts, T, seed, P0)


def test_sampling_rounds_replay_from_a_graph():
    """Sampling rounds captured once in a HIP graph and replayed three times continue the
    stream exactly like the same rounds run eagerly (the draws depend only on the seed and the
    stream position, both on the device)."""
    V, H, K, T, R = 3000, 512, 6, 0.3, 6
    S = K + 1
    rng = np.random.default_rng(41)
    q, s = head(43, V, H)
    hid = [to_dev(synth.fp16_normal(rng, (S, H))) for _ in range(R)]
    ctx = synth.zipf_context_with_copies(np.random.default_rng(4), 400, V, 0.3)[0].astype(np.int32)
    cap = len(ctx) + 3 * R * S + 8

    class SampleLoop:
        def __init__(self):
            self.tokens = torch.zeros(cap, dtype=torch.int32, device=dev())
            self.tokens[:len(ctx)] = to_dev(ctx)
            self.state = sv.new_state(dev())
            self.state[sv.STATE_LEN] = len(ctx)
            self.wq, self.ws = to_dev(q), to_dev(s)
            self.work = sv.workspace(sv.sample_workspace_bytes(V, H, S), dev())
            self.drafts = torch.empty(K, dtype=torch.int32, device=dev())
            sv.propose(self.tokens, self.state, self.drafts, 3)

        def run(self):
            for r in range(R):
                sv.round_sample(self.wq, self.ws, hid[r], self.drafts, T, 77, self.tokens, self.state, self.drafts,
                                self.work)

    eager = SampleLoop()
    for _ in range(3):
        eager.run()
    torch.cuda.synchronize()
    g = SampleLoop()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            g.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for _ in range(3):
        graph.replay()
        torch.cuda.synchronize()
        _ = (g.state[sv.STATE_LEN] + 1).item()
    assert torch.equal(g.tokens, eager.tokens) and torch.equal(g.state, eager.state)
    assert torch.equal(g.drafts, eager.drafts)


def test_sampling_rounds_hit_rate_gate():
    """gate_after = 2 with a flat target (no draft is kept at T = 1 over 3000 ids): the gate
    fires after the second round and the drafter then proposes only pads, even when the
    stream's end would give it a match."""
    V, H, K, T = 3000, 256, 8, 1.0
    S = K + 1
    rng = np.random.default_rng(61)
    q, s = head(62, V, H)
    wq, ws = to_dev(q), to_dev(s)
    ctx = np.tile(np.arange(1, 40, dtype=np.int32), 10)
    tokens = torch.zeros(len(ctx) + 64, dtype=torch.int32, device=dev())
    tokens[:len(ctx)] = to_dev(ctx)
    state = sv.new_state(dev())
    state[sv.STATE_LEN] = len(ctx)
    state[sv.STATE_GATE_AFTER] = 2
    drafts = torch.empty(K, dtype=torch.int32, device=dev())
    work = sv.workspace(sv.sample_workspace_bytes(V, H, S), dev())
    sv.propose(tokens, state, drafts, 3)
    torch.cuda.synchronize()
    assert (drafts.cpu().numpy() >= 0).all()
    hidden = to_dev(synth.fp16_normal(rng, (S, H)))
    for r in range(4):
        sv.round_sample(wq, ws, hidden, drafts, T, 5 + r, tokens, state, drafts, work)
        torch.cuda.synchronize()
        if int(state[sv.STATE_J]) != 0:
            pytest.skip("a draft happened to be kept")
    st = state.cpu().numpy()
    assert st[sv.STATE_GATED] == 2 and st[sv.STATE_ZERO_RUN] == 4 and st[sv.STATE_ROUNDS] == 4
    assert drafts.cpu().tolist() == [-1] * K
    n = int(st[sv.STATE_LEN])
    tokens[n - 1] = int(ctx[-1])
    sv.propose(tokens, state, drafts, 3)
    torch.cuda.synchronize()
    assert drafts.cpu().tolist() == [-1] * K
    state[sv.STATE_GATED] = 0
    sv.propose(tokens, state, drafts, 3)
    torch.cuda.synchronize()
    assert (drafts.cpu().numpy() >= 0).any()


def test_round_sample_full_35b_head_shape():
    """One sampling round at the full 35B-A3B-shaped head (V = 248320, H = 2048, K = 8,
    T = 0.7) in the launch configuration the bench uses.  Rows 0..4 are steered onto drafts
    1..5 (kept), row 5 onto a token other than draft 6 (rejected; the residual draw is that
    token): the draws against the oracle's Gumbel keys, the keep decisions against the oracle's
    accept uniforms, then the committed stream and the next drafts bit-exactly."""
    V, H, K, T = 248320, 2048, 8, 0.7
    S = K + 1
    say(f"round_sample full V={V} H={H} K={K} T={T}")
    q, s = synth.quantized_head(synth.streams(2).weights, V, H)
    rng = np.random.default_rng(71)
    ctx = synth.zipf_context_with_copies(np.random.default_rng(72), 4096, V, 0.3)[0].astype(np.int32)
    P0 = len(ctx)
    seed = 0x5EED_0F_5A3B

    def steer(tok):
        d = (q[tok].astype(np.float64).reshape(-1, 32) * s[tok].astype(np.float64)[:, None]).reshape(-1)
        return (50.0 * d).astype(np.float16)

    drafts = [int(x) for x in rng.choice(V, size=K, replace=False)]
    other = int(ctx[1000]) if int(ctx[1000]) != drafts[5] else int(ctx[1001])   # in the context: the
    # drafter then finds the committed stream's last id earlier and proposes real drafts
    rows = [steer(drafts[i]) for i in range(5)] + [steer(other)]
    rows += list(synth.fp16_normal(rng, (S - 6, H)))
    hidden = np.stack(rows)
    cap = P0 + 64
    tokens = torch.zeros(cap, dtype=torch.int32, device=dev())
    tokens[:P0] = to_dev(ctx)
    state = sv.new_state(dev())
    state[sv.STATE_LEN] = P0
    d_in = to_dev(np.array(drafts, dtype=np.int32))
    d_out = torch.empty(K, dtype=torch.int32, device=dev())
    sample = torch.empty(S, dtype=torch.int32, device=dev())
    lse = torch.empty(S, dtype=torch.float32, device=dev())
    work = sv.workspace(sv.sample_workspace_bytes(V, H, S), dev())
    sv.round_sample(to_dev(q), to_dev(s), to_dev(hidden), d_in, T, seed, tokens, state, d_out, work, 3, sample, lse)
    torch.cuda.synchronize()
    L = oracle.head_logits(q, s, hidden)
    smp_d = sample.cpu().numpy()
    check_draws(smp_d, L, drafts, T, seed, P0)
    p, _ = smp.probabilities(L, T)
    u = smp.accept_uniforms(seed, P0, K)
    st = state.cpu().numpy()
    j = int(st[sv.STATE_J])
    assert j == 5 and all(u[i] < p[i, drafts[i]] for i in range(5)) and not u[5] < p[5, drafts[5]]
    assert int(smp_d[5]) == other
    stream = list(ctx) + drafts[:5] + [other]
    assert st[sv.STATE_LEN] == len(stream) and tokens[:len(stream)].cpu().tolist() == stream
    nxt = oracle.propose_scan(stream, 3, K)[0]
    assert d_out.cpu().tolist() == list(nxt) and max(nxt) >= 0


def test_generate_sample_equals_round_by_round():
    """specverify_generate_sample over R rounds (one seed: the noise is keyed by the stream
    position) leaves the stream, the state word and the next drafts bit-identical to R calls
    of gather_window + round_sample with the same seed."""
    V, H, K, T, R = 3000, 512, 6, 0.3, 25
    S = K + 1
    rng = np.random.default_rng(91)
    q, s = head(92, V, H)
    model = synth.MarkovHidden(rng, V, H)
    ctx, _, _ = synth.uniform_context_with_span(rng, 400, V, 12, 16)
    wq, ws, tab = to_dev(q), to_dev(s), to_dev(model.table)
    cap = len(ctx) + R * S + 8
    seed = 0xC0FFEE

    def fresh():
        t = torch.zeros(cap, dtype=torch.int32, device=dev())
        t[:len(ctx)] = to_dev(ctx)
        st = sv.new_state(dev())
        st[sv.STATE_LEN] = len(ctx)
        d = torch.empty(K, dtype=torch.int32, device=dev())
        sv.propose(t, st, d, 3)
        return t, st, d

    work = sv.workspace(sv.sample_workspace_bytes(V, H, S), dev())
    window = torch.empty((S, H), dtype=torch.float16, device=dev())
    ta, sa, da = fresh()
    sv.generate_sample(wq, ws, tab, ta, sa, da, window, work, R, T, seed)
    tb, sb, db = fresh()
    for _ in range(R):
        sv.gather_window(tb, sb, db, tab, window)
        sv.round_sample(wq, ws, window, db, T, seed, tb, sb, db, work)
    torch.cuda.synchronize()
    assert int(sa[sv.STATE_ROUNDS]) == R and int(sa[sv.STATE_FLAGS]) == 0
    assert torch.equal(sa, sb) and torch.equal(ta, tb) and torch.equal(da, db)
