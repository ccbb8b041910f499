"""A window row whose logits are all NaN (e.g. an fp16 activation that overflowed upstream)
has no argmax: verify reports -1 for it (the int8 and int4 heads), and every accept step refuses
to commit -1 (sticky argmax flag, no token, no round recorded), the fused sampling round
included.  Rows past the first rejected draft do not matter."""
import numpy as np
import pytest
import torch

import oracle
from weight_bound_verify_amd import specverify as sv
from weight_bound_verify_amd import synth

from gpu_util import check_argmax, dev, say, to_dev

pytestmark = pytest.mark.gpu

NAN16 = np.uint16(0x7E00).view(np.float16)


def _state(length):
    st = sv.new_state(dev())
    st[sv.STATE_LEN] = length
    return st


@pytest.mark.parametrize("V,H", [(5000, 512), (3000, 16384)])       # unsplit, and the split-sum path
def test_verify_nan_row_has_no_argmax(V, H):
    say(f"nan row verify V={V} H={H}")
    rng = np.random.default_rng(V + H)
    q, s = synth.quantized_head(np.random.SeedSequence(V), V, H)
    hidden = synth.fp16_normal(rng, (5, H))
    hidden[3] = NAN16
    am = torch.full((5,), 7, dtype=torch.int32, device=dev())
    sv.verify(to_dev(q), to_dev(s), to_dev(hidden), am, sv.workspace(sv.verify_workspace_bytes(V, H, 5), dev()))
    torch.cuda.synchronize()
    a = am.cpu().numpy()
    assert a[3] == -1
    ok = [0, 1, 2, 4]
    check_argmax(a[ok], oracle.head_logits(q, s, hidden[ok]))


def test_round_with_nan_row_at_j_commits_nothing():
    """Drafts match rows 0 and 1, row 2 is NaN: the id to commit (argmax of row 2) is missing,
    so the round writes nothing and sets the flag; the drafter still drafts the same stream.
    With the NaN row after the first miss the round commits as usual."""
    V, H, K = 5000, 512, 4
    S = K + 1
    rng = np.random.default_rng(3)
    q, s = synth.quantized_head(np.random.SeedSequence(3), V, H)
    wq, ws = to_dev(q), to_dev(s)
    ctx = rng.integers(0, V, size=300).astype(np.int32)
    work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    for nan_row, j_forced, expect_flag in [(2, 2, True), (4, 1, False), (0, 0, True)]:
        say(f"nan row {nan_row}, forced j {j_forced}")
        hidden = synth.fp16_normal(rng, (S, H))
        L = oracle.head_logits(q, s, hidden)
        d, _ = synth.forced_drafts(rng, oracle.argmax_lowest(L), K, V, j=j_forced)
        hidden[nan_row] = NAN16
        buf = np.zeros(400, np.int32)
        buf[:300] = ctx
        tokens, st = to_dev(buf), _state(300)
        d_out = torch.empty(K, dtype=torch.int32, device=dev())
        am = torch.empty(S, dtype=torch.int32, device=dev())
        sv.round(wq, ws, to_dev(hidden), to_dev(d), tokens, st, d_out, am, work)
        torch.cuda.synchronize()
        stv, a = st.cpu().numpy(), am.cpu().numpy()
        assert a[nan_row] == -1
        ok = [r for r in range(S) if r != nan_row]
        assert check_argmax(a[ok], L[ok]) == 0, "a near tie moved a forced row; pick another seed"
        if expect_flag:
            assert stv[sv.STATE_FLAGS] == sv.FLAG_ARGMAX
            assert stv[sv.STATE_LEN] == 300 and stv[sv.STATE_ROUNDS] == 0
            assert np.array_equal(tokens.cpu().numpy(), buf)
            assert d_out.cpu().tolist() == list(oracle.propose_scan(list(ctx), 3, K)[0])
        else:
            assert stv[sv.STATE_FLAGS] == 0
            j, app = oracle.accept(a, d.tolist())
            assert j == j_forced and stv[sv.STATE_LEN] == 301 + j
            assert tokens[300:301 + j].cpu().tolist() == app


def test_standalone_accepts_refuse_a_missing_id():
    K = 3
    buf = np.arange(20, dtype=np.int32)
    d = to_dev(np.array([5, 6, 7], np.int32))
    # greedy: j = 2 (rows 0, 1 match), argmax[2] = -1
    tokens, st = to_dev(buf), _state(10)
    sv.accept(to_dev(np.array([5, 6, -1, 9], np.int32)), d, tokens, st)
    # tree: the chain 0 -> 1 -> 2 matches twice, the last node's argmax is -1
    t_tree, st_tree = to_dev(buf), _state(10)
    sv.accept_tree(to_dev(np.array([5, 6, -1, 9], np.int32)), to_dev(np.array([0, 1, 2], np.int32)), d,
                   t_tree, st_tree)
    # sampling: every draft rejected (zd = -inf) and row 0 drew nothing
    t_s, st_s = to_dev(buf), _state(10)
    neg = torch.full((K + 1,), float("-inf"), dtype=torch.float32, device=dev())
    sv.accept_sample(to_dev(np.array([-1, 1, 2, 3], np.int32)), torch.zeros(K + 1, device=dev()), neg, d, 100,
                     12345, t_s, st_s)
    torch.cuda.synchronize()
    for t, st in [(tokens, st), (t_tree, st_tree), (t_s, st_s)]:
        stv = st.cpu().numpy()
        assert stv[sv.STATE_FLAGS] == sv.FLAG_ARGMAX and stv[sv.STATE_LEN] == 10 and stv[sv.STATE_ROUNDS] == 0
        assert np.array_equal(t.cpu().numpy(), buf)


def test_verify_q4_nan_row_has_no_argmax():
    """The int4 head: the NaN row reports -1, the other rows match the oracle."""
    V, H = 3001, 1024
    rng = np.random.default_rng(11)
    p, s = synth.quantized_head_q4(np.random.SeedSequence(11), V, H)
    hidden = synth.fp16_normal(rng, (6, H))
    hidden[2] = NAN16
    am = torch.full((6,), 7, dtype=torch.int32, device=dev())
    sv.verify_q4(to_dev(p), to_dev(s), to_dev(hidden), am, sv.workspace(sv.verify_workspace_bytes(V, H, 6), dev()))
    torch.cuda.synchronize()
    a = am.cpu().numpy()
    assert a[2] == -1
    ok = [0, 1, 3, 4, 5]
    check_argmax(a[ok], oracle.head_logits_q4b32(p, s, hidden[ok]))


def test_round_sample_nan_first_row_commits_nothing():
    """Sampling verify with window row 0 all NaN: its keep test cannot pass and its draw is
    missing, so the fused round commits nothing, records no round and sets the flag."""
    V, H, K = 4000, 512, 4
    S = K + 1
    rng = np.random.default_rng(12)
    q, s = synth.quantized_head(np.random.SeedSequence(12), V, H)
    hidden = synth.fp16_normal(rng, (S, H))
    hidden[0] = NAN16
    buf = np.zeros(400, np.int32)
    buf[:300] = rng.integers(0, V, size=300)
    tokens, st = to_dev(buf), _state(300)
    d_in = to_dev(rng.integers(0, V, size=K).astype(np.int32))
    d_out = torch.empty(K, dtype=torch.int32, device=dev())
    work = sv.workspace(sv.sample_workspace_bytes(V, H, S), dev())
    sv.round_sample(to_dev(q), to_dev(s), to_dev(hidden), d_in, 0.7, 2026, tokens, st, d_out, work)
    torch.cuda.synchronize()
    stv = st.cpu().numpy()
    assert stv[sv.STATE_FLAGS] == sv.FLAG_ARGMAX and stv[sv.STATE_LEN] == 300 and stv[sv.STATE_ROUNDS] == 0
    assert np.array_equal(tokens.cpu().numpy(), buf)
