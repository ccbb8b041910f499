"""End-to-end pins of the oracle round driver.

The feasibility page's control-logic proof checks the fused greedy scheme against plain
greedy decoding on thousands of random cases with hash and Markov stand-in models; the same
property pins the oracle's propose/verify/accept composition here (>= 3000 cases).  The
worked accounting of its implementation status (96 tokens, K = 4, every draft accepted)
pins tokens per round = 1 + j and the forward count.
"""
import numpy as np
import pytest

import oracle
from weight_bound_verify_amd import synth


def _head(rng, V, H):
    q, s = synth.quantize_q8b32(rng.standard_normal((V, H), dtype=np.float32) * np.float32(0.02))
    return lambda rows: oracle.argmax_lowest(oracle.head_logits(q, s, rows))


def _cases(n_cases, seed):
    rng = np.random.default_rng(seed)
    for c in range(n_cases):
        V = int(rng.integers(3, 40))
        H = 32 * int(rng.integers(1, 3))
        K = int(rng.choice([1, 2, 3, 4, 8, 16]))
        n_max = int(rng.integers(1, 4))
        ctx = list(rng.integers(0, V, size=int(rng.integers(1, 24))))
        n_new = int(rng.integers(1, 40))
        argmax_fn = _head(rng, V, H)
        if c % 2 == 0:
            hidden_fn = synth.MarkovHidden(rng, V, H)
        else:
            hidden_fn = synth.HashHidden(int(rng.integers(0, 2**62)), H)
        yield ctx, hidden_fn, argmax_fn, n_new, K, n_max


def test_spec_decode_is_token_identical_to_greedy_3000_cases():
    n = 0
    accepted = 0
    for ctx, hidden_fn, argmax_fn, n_new, K, n_max in _cases(3000, 1234):
        st = {}
        ref = oracle.greedy_decode(ctx, hidden_fn, argmax_fn, n_new)
        got = oracle.spec_decode(ctx, hidden_fn, argmax_fn, n_new, K, n_max, stats=st)
        assert got == ref
        assert all(0 <= j <= K for j in st["accepted"])
        accepted += sum(st["accepted"])
        n += 1
    assert n == 3000
    assert accepted > 0          # the Markov stand-in cycles, so drafts do get accepted


def test_perfect_drafter_accepts_every_draft_and_worked_accounting(golden):
    g = golden("worked_accounting.json")
    rng = np.random.default_rng(77)
    V, H = 64, 64
    argmax_fn = _head(rng, V, H)
    hidden_fn = synth.HashHidden(99, H)
    ctx = list(rng.integers(0, V, size=10))
    ref = oracle.greedy_decode(ctx, hidden_fn, argmax_fn, g["gen"] + g["K"] + 1)

    def perfect(toks, K):        # the model's own future greedy tokens, past the anchor
        return ref[len(toks):len(toks) + K]

    st = {}
    got = oracle.spec_decode(ctx, hidden_fn, argmax_fn, g["gen"], g["K"], g["ngram"], drafter=perfect, stats=st)
    assert got == ref[:len(ctx) + g["gen"]]
    assert all(j == g["K"] for j in st["accepted"])
    assert np.mean(st["accepted"]) == pytest.approx(g["accepted_per_round"])
    assert st["forwards"] == g["forwards"]


def test_drafter_must_continue_past_the_anchor():
    # proposing continuations of the stream *without* a0 re-proposes a0 and accepts nothing
    rng = np.random.default_rng(5)
    V, H = 2048, 32
    argmax_fn = _head(rng, V, H)
    hidden_fn = synth.HashHidden(3, H)
    ctx = list(rng.integers(0, V, size=8))
    ref = oracle.greedy_decode(ctx, hidden_fn, argmax_fn, 60)

    def off_by_one(toks, K):
        return ref[len(toks) - 1:len(toks) - 1 + K]

    st = {}
    got = oracle.spec_decode(ctx, hidden_fn, argmax_fn, 40, 4, 3, drafter=off_by_one, stats=st)
    assert got == ref[:len(ctx) + 40]
    # a draft can only be accepted where the greedy stream repeats a token back to back
    repeats = sum(1 for i in range(len(ctx), len(ref) - 1) if ref[i] == ref[i + 1])
    assert sum(st["accepted"]) <= repeats == 0


def test_verify_window_equals_sequential_single_row_argmaxes():
    rng = np.random.default_rng(8)
    q, s = synth.quantize_q8b32(rng.standard_normal((500, 128), dtype=np.float32) * np.float32(0.02))
    h = synth.fp16_normal(rng, (9, 128))
    a = oracle.argmax_lowest(oracle.head_logits(q, s, h))
    seq = [int(oracle.argmax_lowest(oracle.head_logits(q, s, h[i:i + 1]))[0]) for i in range(9)]
    assert list(a) == seq


def test_hit_rate_gate_is_lossless_and_drops_the_drafter():
    """Gating never changes the committed stream (it equals greedy decoding), and once it
    fires every later round commits exactly one token (feasibility page, SHIPPED note)."""
    n_gated = 0
    for c, (ctx, hidden_fn, argmax_fn, n_new, K, n_max) in enumerate(_cases(400, 4321)):
        g = 1 + c % 4
        st = {}
        ref = oracle.greedy_decode(ctx, hidden_fn, argmax_fn, n_new)
        got = oracle.spec_decode(ctx, hidden_fn, argmax_fn, n_new, K, n_max, stats=st, gate_after=g)
        assert got == ref
        js, at = st["accepted"], st["gated_after_round"]
        if at is not None:
            n_gated += 1
            assert js[at - g:at] == [0] * g                 # the g zero-accept rounds that fired it
            assert all(j == 0 for j in js[at:])             # pads are never accepted
            # no earlier run of g zero-accept rounds
            run = 0
            for j in js[:at - 1]:
                run = run + 1 if j == 0 else 0
                assert run < g
    assert n_gated > 50


def test_gate_with_never_hitting_and_always_hitting_drafters():
    rng = np.random.default_rng(9)
    V, H, K = 32, 64, 4
    argmax_fn = _head(rng, V, H)
    hidden_fn = synth.HashHidden(5, H)
    ctx = list(rng.integers(0, V, size=12))
    n_new = 40
    ref = oracle.greedy_decode(ctx, hidden_fn, argmax_fn, n_new + K + 1)
    # a drafter that is always wrong (greedy id + 1): the gate fires after exactly g rounds
    # and every round, gated or not, commits one token
    st = {}
    wrong = lambda toks, k: [(ref[len(toks)] + 1) % V] + [0] * (k - 1)
    got = oracle.spec_decode(ctx, hidden_fn, argmax_fn, n_new, K, 3, drafter=wrong, stats=st, gate_after=3)
    assert got == ref[:len(ctx) + n_new]
    # the a0 bootstrap commits the first new token, each round one more
    assert st["gated_after_round"] == 3 and len(st["accepted"]) == n_new - 1 and sum(st["accepted"]) == 0
    # a perfect drafter never gates: every round commits K + 1 tokens
    st = {}
    perfect = lambda toks, k: ref[len(toks):len(toks) + k]
    got = oracle.spec_decode(ctx, hidden_fn, argmax_fn, n_new, K, 3, drafter=perfect, stats=st, gate_after=1)
    assert got == ref[:len(ctx) + n_new]
    assert st["gated_after_round"] is None and set(st["accepted"]) == {K}


def test_script_target_greedy_decoding_reproduces_the_script():
    """The script stand-in (row at position p = sign pattern of the scripted id's code row):
    plain greedy decoding and speculative decoding with the n-gram drafter both reproduce the
    script, and the drafter's acceptance rate lies strictly between 0 and 1 (the script copies
    30% of its spans, as the contexts do)."""
    V, H, K = 3000, 256, 8
    q, s = synth.quantized_head(np.random.SeedSequence(77), V, H)
    script, _ = synth.zipf_context_with_copies(np.random.default_rng(78), 1200, V, 0.3)
    model = synth.ScriptHidden(q, script)
    argmax_fn = lambda rows: oracle.argmax_lowest(oracle.head_logits(q, s, rows))
    ctx = script[:400].tolist()
    assert oracle.greedy_decode(ctx, model, argmax_fn, 200) == script[:600].tolist()
    st = {}
    assert oracle.spec_decode(ctx, model, argmax_fn, 700, K, 3, stats=st) == script[:1100].tolist()
    js = np.array(st["accepted"])
    alpha = js.sum() / (js.sum() + (js < K).sum())
    assert 0.0 < alpha < 1.0
    assert np.array_equal(model.rows()[399], model(script[:400]))
