"""specverify_round_noalloc (the round with the library's static scratch, no workspace, no
allocation) against specverify_round with a caller workspace, through the C ABI: two calls in
a row on fresh state, the second with a smaller input, every output bit for bit; a shape
whose scratch would not fit is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import oracle
from weight_bound_verify_amd import specverify as sv
from weight_bound_verify_amd import synth

from gpu_util import check_argmax, dev, say, to_dev

pytestmark = pytest.mark.gpu


def _inputs(V, H, K, seed):
    rng = np.random.default_rng(seed)
    q, s = synth.quantized_head(np.random.SeedSequence(seed), V, H)
    ctx, _ = synth.zipf_context_with_copies(rng, 2000, V, 0.3)
    hidden = synth.fp16_normal(rng, (K + 1, H))
    return q, s, ctx, hidden


def _one_round(fn, wq, ws, hd, ctx, K, V, with_ws):
    S = K + 1
    cap = len(ctx) + 4 * S
    buf = np.zeros(cap, np.int32)
    buf[:len(ctx)] = ctx
    tokens = to_dev(buf)
    st = sv.new_state(dev())
    st[sv.STATE_LEN] = len(ctx)
    d_in = torch.empty(K, dtype=torch.int32, device=dev())
    sv.propose(tokens, st, d_in)
    d_out = torch.full((K,), -9, dtype=torch.int32, device=dev())
    am = torch.full((S,), -9, dtype=torch.int32, device=dev())
    lg = torch.full((S, V), float("nan"), dtype=torch.float32, device=dev())
    if with_ws:
        fn(wq, ws, hd, d_in, tokens, st, d_out, am, sv.workspace(sv.verify_workspace_bytes(V, wq.shape[1], S), dev()),
           logits=lg)
    else:
        fn(wq, ws, hd, d_in, tokens, st, d_out, am, logits=lg)
    torch.cuda.synchronize()
    return dict(tokens=tokens.cpu().numpy(), state=st.cpu().numpy(), d_in=d_in.cpu().numpy(),
                d_out=d_out.cpu().numpy(), argmax=am.cpu().numpy(), logits=lg.cpu().numpy())


@pytest.mark.parametrize("order", ["large_then_small", "small_after_large_twice"])
def test_noalloc_round_equals_round(order):
    # the 35B-A3B-shaped head, then smaller ones (the last one splits its hidden axis across
    # workgroups, with the split sums in the static scratch too)
    shapes = [(248320, 2048, 8, 41), (30000, 1024, 3, 42), (3000, 16384, 8, 44)]
    if order == "small_after_large_twice":
        shapes = [shapes[0], shapes[0], shapes[2], shapes[1]]
    for V, H, K, seed in shapes:
        say(f"noalloc round V={V} H={H} K={K}")
        q, s, ctx, hidden = _inputs(V, H, K, seed)
        wq, ws, hd = to_dev(q), to_dev(s), to_dev(hidden)
        ref = _one_round(sv.round, wq, ws, hd, ctx, K, V, True)
        got = _one_round(sv.round_noalloc, wq, ws, hd, ctx, K, V, False)
        for k in ("tokens", "state", "d_in", "d_out", "argmax"):
            assert np.array_equal(got[k], ref[k]), k
        assert np.array_equal(got["logits"].view(np.uint32), ref["logits"].view(np.uint32))
        if V * H <= 50_000_000:
            check_argmax(got["argmax"], oracle.head_logits(q, s, hidden))
        del wq, ws


def test_noalloc_round_refuses_a_split_hidden_axis():
    V, H, K = 30000, 16384, 8
    assert sv.verify_workspace_bytes(V, H, K + 1) > 8 * 64 * 4096
    q, s, ctx, hidden = _inputs(V, H, K, 43)
    tokens = to_dev(np.zeros(4000, np.int32))
    st = sv.new_state(dev())
    st[sv.STATE_LEN] = 100
    d = torch.zeros(K, dtype=torch.int32, device=dev())
    am = torch.zeros(K + 1, dtype=torch.int32, device=dev())
    with pytest.raises(sv.SpecVerifyError) as e:
        sv.round_noalloc(to_dev(q), to_dev(s), to_dev(hidden), d, tokens, st, d, am)
    assert e.value.status == 2 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert int(st[sv.STATE_LEN]) == 100 and int(st[sv.STATE_ROUNDS]) == 0
