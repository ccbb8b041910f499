"""GPU parity of the int4 per-block-32 head (specverify_verify_q4b32 / _round_q4b32) against the
CPU oracle: logits within 1e-3 relative (row-rms floor), argmax exact except at oracle top-2
gaps below 1e-3, and the fused round equal to verify -> accept -> propose."""
import numpy as np
import pytest
import torch

import oracle
from weight_bound_verify_amd import specverify as sv
from weight_bound_verify_amd import synth

from gpu_util import check_argmax, check_logits, dev, say, to_dev

pytestmark = pytest.mark.gpu


def _gpu_verify_q4(p, s, hidden, want_logits=True):
    V = p.shape[0]
    S = hidden.shape[0]
    am = torch.full((S,), -7, dtype=torch.int32, device=dev())
    lg = torch.full((S, V), float("nan"), dtype=torch.float32, device=dev()) if want_logits else None
    work = sv.workspace(sv.verify_workspace_bytes(V, 2 * p.shape[1], S), dev())
    sv.verify_q4(to_dev(p), to_dev(s), to_dev(hidden), am, work, lg)
    torch.cuda.synchronize()
    return am.cpu().numpy(), (lg.cpu().numpy().astype(np.float64) if want_logits else None)


@pytest.mark.parametrize("V,H,S", [(1, 256, 1), (17, 256, 9), (1000, 512, 9), (4099, 2048, 16), (777, 2560, 5),
                                   (33, 2048, 9), (16, 4096, 3),
                                   (3000, 4096, 9), (513, 5120, 2), (70000, 1024, 3)])
def test_verify_q4_matches_oracle(V, H, S):
    say(f"verify q4 V={V} H={H} S={S}")
    p, s = synth.quantized_head_q4(np.random.SeedSequence(V * 5 + H + S), V, H)
    hidden = synth.fp16_normal(np.random.default_rng(S + 3), (S, H))
    a, lg = _gpu_verify_q4(p, s, hidden)
    L = oracle.head_logits_q4b32(p, s, hidden)
    worst = check_logits(lg, L)
    check_argmax(a, L)
    a2, _ = _gpu_verify_q4(p, s, hidden, want_logits=False)
    assert np.array_equal(a, a2)
    say(f"  max rel err {worst:.2e}")


def test_verify_q4_exact_on_integer_inputs():
    """Unit scales and small integer hidden values: every partial sum is an exact fp32 integer."""
    rng = np.random.default_rng(0)
    V, H, S = 2000, 512, 9
    u = rng.integers(1, 16, size=(V, H)).astype(np.uint8)
    p = np.zeros((V, H // 2), dtype=np.uint8)
    for b in range(H // 32):
        p[:, 16 * b:16 * b + 16] = u[:, 32 * b:32 * b + 16] | (u[:, 32 * b + 16:32 * b + 32] << 4)
    s = np.ones((V, H // 32), dtype=np.float16)
    hidden = rng.integers(-3, 4, size=(S, H)).astype(np.float16)
    a, lg = _gpu_verify_q4(p, s, hidden)
    L = oracle.head_logits_q4b32(p, s, hidden)
    assert np.array_equal(lg, L)
    assert np.array_equal(a, oracle.argmax_lowest(L))


def test_verify_q4_full_35b_head_shape():
    V, H, S = 248320, 2048, 9
    st = synth.streams(2)
    p, s = synth.quantized_head_q4(st.weights, V, H)
    hidden = synth.fp16_normal(np.random.default_rng(st.hidden), (S, H))
    a, lg = _gpu_verify_q4(p, s, hidden)
    L = oracle.head_logits_q4b32(p, s, hidden)
    check_logits(lg, L)
    check_argmax(a, L)


@pytest.mark.parametrize("V,H,K", [(5000, 1024, 8), (2000, 512, 15), (300, 2560, 1)])
def test_round_q4_equals_separate_calls(V, H, K):
    rng = np.random.default_rng(V + K)
    p, s = synth.quantized_head_q4(np.random.SeedSequence(V), V, H)
    ctx, _, _ = synth.uniform_context_with_span(rng, 400, V, 12, 8)
    hidden = synth.fp16_normal(rng, (K + 1, H))
    S = K + 1
    cap = len(ctx) + 4 * S
    outs = []
    for fused in (False, True):
        buf = np.zeros(cap, dtype=np.int32)
        buf[:len(ctx)] = ctx
        tokens, state = to_dev(buf), sv.new_state(dev())
        state[sv.STATE_LEN] = len(ctx)
        drafts = torch.empty(K, dtype=torch.int32, device=dev())
        nxt = torch.empty(K, dtype=torch.int32, device=dev())
        argmax = torch.empty(S, dtype=torch.int32, device=dev())
        work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
        wq, ws, hd = to_dev(p), to_dev(s), to_dev(hidden)
        sv.propose(tokens, state, drafts, 3)
        if fused:
            sv.round_q4(wq, ws, hd, drafts, tokens, state, nxt, argmax, work)
        else:
            sv.verify_q4(wq, ws, hd, argmax, work)
            sv.accept(argmax, drafts, tokens, state)
            sv.propose(tokens, state, nxt, 3)
        torch.cuda.synchronize()
        outs.append((tokens.cpu().numpy(), state.cpu().numpy(), nxt.cpu().numpy(), argmax.cpu().numpy()))
    for x, y in zip(outs[0], outs[1]):
        assert np.array_equal(x, y)
    L = oracle.head_logits_q4b32(p, s, hidden)
    check_argmax(outs[1][3], L)
