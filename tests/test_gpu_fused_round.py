"""specverify_round (verify -> accept -> next drafts, fused into the matmul's last workgroup
when the hidden axis is not split) against the three separate entry points and the oracle."""
import numpy as np
import pytest
import torch

import oracle
from weight_bound_verify_amd import specverify as sv
from weight_bound_verify_amd import synth

from gpu_util import check_argmax, dev, say, to_dev

pytestmark = pytest.mark.gpu


def _setup(V, H, K, ctx_len, seed, cap_extra=200):
    rng = np.random.default_rng(seed)
    q, s = synth.quantized_head(np.random.SeedSequence(seed), V, H)
    ctx, _ = synth.zipf_context_with_copies(rng, ctx_len, V, 0.3)
    hidden = synth.fp16_normal(rng, (6, K + 1, H))
    return q, s, ctx, hidden, ctx_len + cap_extra


def _state_tokens(ctx, cap):
    buf = np.zeros(cap, dtype=np.int32)
    buf[:len(ctx)] = ctx
    st = sv.new_state(dev())
    st[sv.STATE_LEN] = len(ctx)
    return to_dev(buf), st


@pytest.mark.parametrize("V,H,K,alias", [(30000, 2048, 8, True), (30000, 2048, 8, False), (5000, 512, 16, True),
                                         (777, 8192, 4, True), (3000, 16384, 8, False), (20000, 1024, 3, True),
                                         (30000, 2048, 40, True), (6000, 512, 63, False)])
def test_round_equals_separate_calls(V, H, K, alias):
    """Every round: the fused round equals the three separate entry points bit for bit, its
    argmax equals the oracle's (near-tie rule), the ids it commits equal oracle.accept on the
    GPU's argmax and the drafts it verified, and the next drafts equal oracle.propose_scan on
    the committed stream."""
    say(f"round V={V} H={H} K={K} alias={alias}")
    S = K + 1
    q, s, ctx, hidden, cap = _setup(V, H, K, 700, V + H + K)
    wq, ws, hd = to_dev(q), to_dev(s), to_dev(hidden)
    # reference: separate entry points
    t_ref, st_ref = _state_tokens(ctx, cap)
    d_ref = torch.empty(K, dtype=torch.int32, device=dev())
    a_ref = torch.empty(S, dtype=torch.int32, device=dev())
    w_ref = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    # fused
    t_f, st_f = _state_tokens(ctx, cap)
    d_f = torch.empty(K, dtype=torch.int32, device=dev())
    d_f2 = torch.empty(K, dtype=torch.int32, device=dev())
    a_f = torch.empty(S, dtype=torch.int32, device=dev())
    w_f = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    sv.propose(t_ref, st_ref, d_ref)
    sv.propose(t_f, st_f, d_f)
    torch.cuda.synchronize()
    stream = list(ctx)
    drafts = d_f.cpu().tolist()
    assert drafts == list(oracle.propose_scan(stream, 3, K)[0])
    for r in range(len(hidden)):
        sv.verify(wq, ws, hd[r], a_ref, w_ref)
        sv.accept(a_ref, d_ref, t_ref, st_ref)
        sv.propose(t_ref, st_ref, d_ref)
        if alias:
            sv.round(wq, ws, hd[r], d_f, t_f, st_f, d_f, a_f, w_f)
        else:
            src, dst = (d_f, d_f2) if r % 2 == 0 else (d_f2, d_f)
            sv.round(wq, ws, hd[r], src, t_f, st_f, dst, a_f, w_f)
        torch.cuda.synchronize()
        assert torch.equal(a_f, a_ref), r
        cur = d_f if (alias or r % 2 == 1) else d_f2
        assert torch.equal(cur, d_ref), r
        assert torch.equal(st_f, st_ref) and torch.equal(t_f, t_ref), r
        # the oracle: argmax of this window, accept on the GPU's argmax, drafts on the stream
        a_gpu = a_f.cpu().numpy()
        check_argmax(a_gpu, oracle.head_logits(q, s, hidden[r]))
        j, app = oracle.accept(a_gpu, drafts)
        stream += app
        n = int(st_f[sv.STATE_LEN])
        assert n == len(stream) and t_f[:n].cpu().tolist() == stream, r
        assert int(st_f[sv.STATE_J]) == j, r
        drafts = cur.cpu().tolist()
        d_or, nv, nu = oracle.propose_scan(stream, 3, K)
        assert drafts == list(d_or), r
        assert int(st_f[sv.STATE_NVALID]) == nv and int(st_f[sv.STATE_NUSED]) == nu, r
    assert int(st_f[sv.STATE_ROUNDS]) == len(hidden)


def test_round_full_c3_shape_forced_drafts_every_j():
    """The fused round at the 35B-A3B-shaped head (V=248320, H=2048, K=8) with drafts forced to
    match the oracle's first j greedy ids, j = 0 .. K, each once: the committed ids equal
    oracle.accept on the GPU's argmax, j is the forced one (unless a near tie moved an id), and
    the next drafts equal oracle.propose_scan on the committed stream."""
    V, H, K = 248320, 2048, 8
    S = K + 1
    say("round full C3 shape, forced drafts j = 0..8")
    rng = np.random.default_rng(31)
    q, s = synth.quantized_head(np.random.SeedSequence(31), V, H)
    ctx, _ = synth.zipf_context_with_copies(rng, 4096, V, 0.3)
    wq, ws = to_dev(q), to_dev(s)
    t, st = _state_tokens(ctx, 4096 + 20 * S)
    d = torch.empty(K, dtype=torch.int32, device=dev())
    a = torch.empty(S, dtype=torch.int32, device=dev())
    work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    stream = list(ctx)
    seen = set()
    hidden_all = synth.fp16_normal(rng, (K + 1, S, H))
    L_all = oracle.head_logits(q, s, hidden_all.reshape((K + 1) * S, H)).reshape(K + 1, S, V)
    for j_forced in range(K + 1):
        hidden, L = hidden_all[j_forced], L_all[j_forced]
        fd, _ = synth.forced_drafts(rng, oracle.argmax_lowest(L), K, V, j=j_forced)
        din = to_dev(fd)
        sv.round(wq, ws, to_dev(hidden), din, t, st, d, a, work)
        torch.cuda.synchronize()
        a_gpu = a.cpu().numpy()
        exempt = check_argmax(a_gpu, L)
        j, app = oracle.accept(a_gpu, fd.tolist())
        if exempt == 0:
            assert j == j_forced
        seen.add(j)
        stream += app
        n = int(st[sv.STATE_LEN])
        assert n == len(stream) and t[:n].cpu().tolist() == stream, j_forced
        assert int(st[sv.STATE_J]) == j
        assert d.cpu().tolist() == list(oracle.propose_scan(stream, 3, K)[0]), j_forced
    assert seen == set(range(K + 1))
    assert int(st[sv.STATE_FLAGS]) == 0


def test_round_argmax_matches_oracle_and_workspace_is_shared_across_window_sizes():
    V, H, K = 50000, 2048, 8
    S = K + 1
    q, s, ctx, hidden, cap = _setup(V, H, K, 300, 3)
    wq, ws = to_dev(q), to_dev(s)
    work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    t, st = _state_tokens(ctx, cap)
    d = torch.empty(K, dtype=torch.int32, device=dev())
    am = torch.empty(S, dtype=torch.int32, device=dev())
    sv.propose(t, st, d)
    for r in range(3):
        # interleave plain verify calls (S = 1 and S = K+1) on the same workspace
        a1 = torch.empty(1, dtype=torch.int32, device=dev())
        sv.verify(wq, ws, to_dev(hidden[r][:1]), a1, work)
        sv.round(wq, ws, to_dev(hidden[r]), d, t, st, d, am, work)
        torch.cuda.synchronize()
        L = oracle.head_logits(q, s, hidden[r])
        check_argmax(am.cpu().numpy(), L)
        assert int(a1[0]) == int(am[0]) or oracle.top2_gap(L)[0] < 1e-3


@pytest.mark.parametrize("ctx_len", [16380, 32755, 40000])
def test_round_long_streams_equal_separate_calls(ctx_len):
    """Streams around the round tail's LDS copy (32768 ids): below it, growing across it
    within the rounds, and above it (the tail's global-memory path).  The fused round against
    the separate calls, and the last drafts against the oracle's drafter."""
    V, H, K = 5000, 512, 8
    S = K + 1
    say(f"round long stream {ctx_len}")
    rng = np.random.default_rng(ctx_len)
    q, s = synth.quantized_head(np.random.SeedSequence(ctx_len), V, H)
    ctx, _ = synth.zipf_context_with_copies(rng, ctx_len, V, 0.3)
    wq, ws = to_dev(q), to_dev(s)
    cap = ctx_len + 400
    t_ref, st_ref = _state_tokens(ctx, cap)
    t_f, st_f = _state_tokens(ctx, cap)
    d_ref = torch.empty(K, dtype=torch.int32, device=dev())
    d_f = torch.empty(K, dtype=torch.int32, device=dev())
    a_ref = torch.empty(S, dtype=torch.int32, device=dev())
    a_f = torch.empty(S, dtype=torch.int32, device=dev())
    work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    sv.propose(t_ref, st_ref, d_ref)
    sv.propose(t_f, st_f, d_f)
    for r in range(25):
        hd = to_dev(synth.fp16_normal(rng, (S, H)))
        sv.verify(wq, ws, hd, a_ref, work)
        sv.accept(a_ref, d_ref, t_ref, st_ref)
        sv.propose(t_ref, st_ref, d_ref)
        sv.round(wq, ws, hd, d_f, t_f, st_f, d_f, a_f, work)
        torch.cuda.synchronize()
        assert torch.equal(a_f, a_ref) and torch.equal(d_f, d_ref), r
        assert torch.equal(st_f, st_ref) and torch.equal(t_f, t_ref), r
    n = int(st_f[sv.STATE_LEN])
    assert n >= ctx_len + 25 and int(st_f[sv.STATE_FLAGS]) == 0
    assert d_f.cpu().tolist() == list(oracle.propose_scan(t_f[:n].cpu().tolist(), 3, K)[0])
