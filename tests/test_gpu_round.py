"""GPU parity of specverify_propose / specverify_accept and of whole device-resident rounds."""
import numpy as np
import pytest
import torch

import oracle
from weight_bound_verify_amd import specverify as sv
from weight_bound_verify_amd import synth

from gpu_util import check_argmax, dev, say, to_dev

pytestmark = pytest.mark.gpu


def _state(length):
    st = sv.new_state(dev())
    st[sv.STATE_LEN] = length
    return st


def test_accept_matches_oracle_random():
    rng = np.random.default_rng(0)
    for case in range(300):
        K = int(rng.integers(0, 64))
        a = rng.integers(0, 50, size=K + 1).astype(np.int32)
        j_true = int(rng.integers(0, K + 1))
        d = rng.integers(-1, 50, size=K).astype(np.int32)
        d[:j_true] = a[:j_true]
        length = int(rng.integers(1, 100))
        cap = length + K + 1 + int(rng.integers(0, 5))
        toks0 = rng.integers(0, 50, size=cap).astype(np.int32)
        tokens = to_dev(toks0)
        state = _state(length)
        dd = to_dev(d) if K > 0 else torch.empty(1, dtype=torch.int32, device=dev())
        sv.accept(to_dev(a), dd[:K] if K > 0 else dd, tokens, state)
        torch.cuda.synchronize()
        j, app = oracle.accept(a, d)
        got = tokens.cpu().numpy()
        stv = state.cpu().numpy()
        assert stv[sv.STATE_LEN] == length + 1 + j and stv[sv.STATE_J] == j, case
        assert list(got[length:length + 1 + j]) == app
        assert np.array_equal(got[:length], toks0[:length]) and np.array_equal(got[length + 1 + j:], toks0[length + 1 + j:])
        if K > 0:
            assert stv[sv.STATE_ROUNDS] == 1 and stv[sv.STATE_SUMJ] == j and stv[sv.STATE_HIST + j] == 1
            assert stv[sv.STATE_ZERO_RUN] == (1 if j == 0 else 0) and stv[sv.STATE_GATED] == 0
        else:                   # the anchor bootstrap commits a0 and is not a round
            assert stv[sv.STATE_ROUNDS] == 0 and stv[sv.STATE_HIST] == 0 and stv[sv.STATE_ZERO_RUN] == 0


def test_accept_capacity_overflow_writes_nothing():
    tokens = to_dev(np.arange(10, dtype=np.int32))
    state = _state(5)
    a = to_dev(np.array([1, 2, 3, 4, 5], dtype=np.int32))
    d = to_dev(np.array([1, 2, 3, 4], dtype=np.int32))
    sv.accept(a, d, tokens, state)            # 5 + 4 + 1 = 10 <= 10: fits
    sv.accept(a, d, tokens, state)            # len 10: overflow
    torch.cuda.synchronize()
    stv = state.cpu().numpy()
    assert stv[sv.STATE_LEN] == 10 and stv[sv.STATE_FLAGS] & sv.FLAG_CAPACITY
    assert tokens.cpu().tolist() == [0, 1, 2, 3, 4, 1, 2, 3, 4, 5]


def test_accept_k0_is_the_anchor_bootstrap():
    tokens = to_dev(np.zeros(8, dtype=np.int32))
    state = _state(3)
    sv.accept(to_dev(np.array([42], dtype=np.int32)), None, tokens, state)
    torch.cuda.synchronize()
    assert int(state[sv.STATE_LEN]) == 4 and int(tokens[3]) == 42


@pytest.mark.parametrize("length,V,n_max,K", [
    (0, 5, 3, 4), (1, 5, 3, 4), (2, 2, 3, 8), (50, 3, 3, 8), (513, 30, 3, 8), (4096, 200, 3, 8),
    (8200, 6, 8, 63), (20000, 1000, 3, 16), (16384, 4, 1, 1), (9000, 8000, 5, 33),
])
def test_propose_matches_oracle(length, V, n_max, K):
    rng = np.random.default_rng(length + V)
    toks = rng.integers(0, V, size=length).astype(np.int32)
    cap = length + 70
    buf = np.zeros(cap, dtype=np.int32)
    buf[:length] = toks
    tokens = to_dev(buf)
    state = _state(length)
    drafts = torch.full((K,), -5, dtype=torch.int32, device=dev())
    sv.propose(tokens, state, drafts, n_max)
    torch.cuda.synchronize()
    d, nv, nu = oracle.propose_scan(list(toks), n_max, K)
    assert drafts.cpu().tolist() == d
    assert int(state[sv.STATE_NVALID]) == nv and int(state[sv.STATE_NUSED]) == nu


def test_propose_zipf_contexts_many_suffixes():
    rng = np.random.default_rng(7)
    ctx, frac = synth.zipf_context_with_copies(rng, 4096, 151936, 0.3)
    assert 0.25 < frac < 0.35
    idx = oracle.NgramIndex(3)
    buf = np.zeros(4200, dtype=np.int32)
    buf[:4096] = ctx
    tokens = to_dev(buf)
    for cut in list(range(10, 4096, 97)) + [4096]:
        state = _state(cut)
        drafts = torch.empty(8, dtype=torch.int32, device=dev())
        sv.propose(tokens, state, drafts, 3)
        torch.cuda.synchronize()
        assert drafts.cpu().tolist() == idx.propose(list(ctx[:cut]), 8)[0], cut


def test_propose_corrupt_length_sets_flag_and_pads():
    tokens = to_dev(np.arange(16, dtype=np.int32))
    state = _state(17)                                # len > cap
    drafts = torch.zeros(4, dtype=torch.int32, device=dev())
    sv.propose(tokens, state, drafts, 3)
    torch.cuda.synchronize()
    assert drafts.cpu().tolist() == [-1] * 4 and int(state[sv.STATE_FLAGS]) & sv.FLAG_CAPACITY


def _device_spec_loop(q, s, table, ctx, n_new, K, n_max):
    """Greedy spec decoding with every step on the device: the hidden row of a window
    position is the Markov table row of its token (the stand-in model), gathered on the
    device, so no host synchronisation happens inside the loop."""
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
    drafts = torch.empty(K, dtype=torch.int32, device=dev())
    last = (state[0:1] - 1).long()
    sv.verify(wq, ws, tab.index_select(0, tokens.index_select(0, last).long()).contiguous(), a0,
              sv.workspace(sv.verify_workspace_bytes(V, H, 1), dev()))
    sv.accept(a0, None, tokens, state)                                  # anchor bootstrap
    rounds = 0
    while True:
        torch.cuda.synchronize()
        if int(state[sv.STATE_LEN]) >= len(ctx) + n_new:
            break
        sv.propose(tokens, state, drafts, n_max)
        window = torch.cat([tokens.index_select(0, (state[0:1] - 1).long()), drafts.clamp(min=0)])
        hidden = tab.index_select(0, window.long()).contiguous()
        sv.verify(wq, ws, hidden, argmax, work)
        sv.accept(argmax, drafts, tokens, state)
        rounds += 1
    torch.cuda.synchronize()
    n = int(state[sv.STATE_LEN])
    return tokens[:n].cpu().tolist(), state.cpu().numpy(), rounds


@pytest.mark.parametrize("V,H,K,n_max", [(8192, 512, 8, 3), (2048, 256, 4, 2), (512, 128, 16, 3)])
def test_device_spec_loop_equals_greedy(V, H, K, n_max):
    say(f"device loop V={V} H={H} K={K}")
    rng = np.random.default_rng(V + K)
    q, s = synth.quantized_head(np.random.SeedSequence(V), V, H)
    model = synth.MarkovHidden(rng, V, H)
    ctx, _, _ = synth.uniform_context_with_span(rng, 512, V, 12, 16)
    n_new = 200
    got, stv, rounds = _device_spec_loop(q, s, model.table, ctx, n_new, K, n_max)
    # oracle greedy reference with the same head and stand-in model (next-token logits of a
    # token depend only on that token, so they are memoised)
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
            # allowed only where the oracle's top-2 gap is below 1e-3 and the id is admissible
            L = logits_after(got[p - 1])
            assert oracle.top2_gap(L)[0] < 1e-3 and got[p] in oracle.admissible_sets(L)[0], p
            break
    assert stv[sv.STATE_FLAGS] == 0
    assert stv[sv.STATE_SUMJ] == sum(j * stv[sv.STATE_HIST + j] for j in range(K + 1))
    say(f"  rounds {rounds}, tokens/round {(len(got) - len(ctx)) / max(rounds, 1):.2f}")
    assert rounds < n_new                           # drafts are accepted on the cycling stand-in


def test_forced_drafts_full_35b_head_every_accept_length():
    V, H, K = 248320, 2048, 8
    S = K + 1
    st = synth.streams(2)
    q, s = synth.quantized_head(st.weights, V, H)
    rng_h = np.random.default_rng(st.hidden)
    rng_d = np.random.default_rng(st.drafts)
    wq, ws = to_dev(q), to_dev(s)
    work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    seen = set()
    for r in range(K + 1):
        hidden = synth.fp16_normal(rng_h, (S, H))
        L = oracle.head_logits(q, s, hidden)
        a_ref = oracle.argmax_lowest(L)
        d, j_forced = synth.forced_drafts(rng_d, a_ref, K, V, j=r)
        tokens = to_dev(np.zeros(64, dtype=np.int32))
        state = _state(1)
        argmax = torch.empty(S, dtype=torch.int32, device=dev())
        sv.verify(wq, ws, to_dev(hidden), argmax, work)
        sv.accept(argmax, to_dev(d), tokens, state)
        torch.cuda.synchronize()
        a = argmax.cpu().numpy()
        check_argmax(a, L)
        j, app = oracle.accept(a, d)
        if np.array_equal(a, a_ref):
            assert j == j_forced
        assert int(state[sv.STATE_LEN]) == 2 + j and tokens[1:2 + j].cpu().tolist() == app
        seen.add(j)
    assert seen == set(range(K + 1))
