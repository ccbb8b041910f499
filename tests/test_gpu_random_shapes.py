"""Seeded random shapes against the CPU oracle.

The fixed-shape tests pick the launch configurations by hand; here the (V, H, S) cases are
drawn once from fixed seeds, so that shapes nobody chose reach every configuration branch:
window sizes 1 .. 64 (one, two and four MFMA tiles, the 17th-row and split paths), every hidden
size that is a multiple of 32 up to 8192 for the int8 head (fast and generic kernels, one or
several hidden-axis splits), the int4 head's supported widths, and vocabularies whose last
16-row tile is ragged.  Each case meets the fixed-shape tests' bar: logits within 1e-3 of the
oracle's (relative, with the row RMS as floor), argmax equal except below a 1e-3 top-2 gap.  A
large-vocabulary sweep (65536 .. 300000 rows, H <= 2048, S = 1 .. 17) reaches the heads that take
their items in one contiguous range per die.  A sampling-verify sweep draws (V, H, S, T) and
checks draws and log-sum-exp as the fixed-shape sampling tests do.  A fused-round sweep draws
(V, H, K, n-gram order, context length) and checks the committed ids and next drafts of three
rounds exactly against oracle.accept and oracle.propose_scan; a tree-round sweep does the same
for tree verify (K nodes, B branches, depth D) against oracle.tree, and a dense-stack sweep
checks random block shapes block by block."""
import numpy as np
import pytest
import torch

import oracle
from oracle import sampling as smp
from oracle import tree as tr
from weight_bound_verify_amd import specverify as sv
from weight_bound_verify_amd import synth

from gpu_util import check_argmax, check_logits, dev, gpu_verify, say, to_dev

pytestmark = pytest.mark.gpu

ELEMS = 6_000_000          # at most V * H weights per case, so the oracle finishes in about a second


def _cases(seed, n, widths, smax):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        H = int(rng.choice(widths))
        S = int(rng.integers(1, smax + 1))
        V = int(rng.integers(1, min(20000, ELEMS // H) + 1))
        out.append((V, H, S))
    return out


INT8_CASES = _cases(20261203, 40, np.arange(32, 8193, 32), 64)
# the int4 head's widths: 8 blocks per wave at 1, 2, 4, 5, 6, 8, 10, 12, 14 or 16 waves, or
# 16 blocks per wave at 4 .. 12 waves
INT4_WIDTHS = [256, 512, 1024, 1280, 1536, 2048, 2560, 3072, 3584, 4096, 5120, 6144]
INT4_CASES = _cases(20261204, 16, INT4_WIDTHS, 16)


@pytest.mark.parametrize("V,H,S", INT8_CASES)
def test_verify_random_shape(V, H, S):
    say(f"verify random V={V} H={H} S={S}")
    q, s = synth.quantized_head(np.random.SeedSequence(V * 31 + H * 7 + S), V, H)
    hidden = synth.fp16_normal(np.random.default_rng(V + S), (S, H))
    a, lg = gpu_verify(q, s, hidden)
    L = oracle.head_logits(q, s, hidden)
    check_logits(lg, L)
    check_argmax(a, L)
    # the timed path (no logits written) takes the same decisions
    a2, _ = gpu_verify(q, s, hidden, want_logits=False)
    assert np.array_equal(a, a2)


def _large_vocab_cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        H = int(32 * rng.integers(1, 65))
        out.append((int(rng.integers(65536, min(300000, 200_000_000 // H) + 1)), H, int(rng.integers(1, 18))))
    return out


@pytest.mark.parametrize("V,H,S", _large_vocab_cases(20261209, 8))
def test_verify_large_vocab_random_shape(V, H, S):
    """Vocabularies of 65536 rows or more at hidden sizes up to 2048, where the one-tile argmax
    head takes its items in one contiguous range per die whenever every workgroup gets at
    least 8 items: every logit and argmax row against the oracle, and the timed path (no
    logits) agrees."""
    say(f"verify large vocab V={V} H={H} S={S}")
    q, s = synth.quantized_head(np.random.SeedSequence(V * 3 + H + S), V, H)
    hidden = synth.fp16_normal(np.random.default_rng(V + H + S), (S, H))
    a, lg = gpu_verify(q, s, hidden)
    L = oracle.head_logits(q, s, hidden)
    check_logits(lg, L)
    check_argmax(a, L)
    a2, _ = gpu_verify(q, s, hidden, want_logits=False)
    assert np.array_equal(a, a2)


@pytest.mark.parametrize("V,H,S", INT4_CASES)
def test_verify_q4_random_shape(V, H, S):
    say(f"verify q4 random V={V} H={H} S={S}")
    p, s = synth.quantized_head_q4(np.random.SeedSequence(V * 29 + H * 5 + S), V, H)
    hidden = synth.fp16_normal(np.random.default_rng(V + 2 * S), (S, H))
    am = torch.full((S,), -7, dtype=torch.int32, device=dev())
    lg = torch.full((S, V), float("nan"), dtype=torch.float32, device=dev())
    work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    sv.verify_q4(to_dev(p), to_dev(s), to_dev(hidden), am, work, lg)
    torch.cuda.synchronize()
    L = oracle.head_logits_q4b32(p, s, hidden)
    check_logits(lg.cpu().numpy().astype(np.float64), L)
    check_argmax(am.cpu().numpy(), L)


def _sample_cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        H = int(32 * rng.integers(1, 257))
        V = int(rng.integers(2, min(20000, ELEMS // H) + 1))
        out.append((V, H, int(rng.integers(1, 17)), round(float(rng.uniform(0.3, 1.5)), 3)))
    return out


@pytest.mark.parametrize("V,H,S,T", _sample_cases(20261208, 12))
def test_verify_sample_random_shape(V, H, S, T):
    """Sampling verify (its own epilogue and launch shapes) at random shapes, on the rule of the
    fixed-shape sampling tests: logits, log-sum-exp and draft logits within tolerance, every
    draw the oracle's unless its two best residual keys are within the keys' tolerance."""
    from test_gpu_sample import _key_tol, _setup, check_draws, gpu_verify_sample
    say(f"verify_sample random V={V} H={H} S={S} T={T}")
    seed, P0 = (V * 104729 + H + S) | (1 << 41), 77 + H
    q, s, hidden, L, drafts = _setup(V, H, S, V + H, P0)
    sample, lse, zd, lg = gpu_verify_sample(q, s, hidden, drafts, T, seed, P0)
    check_logits(lg, L)
    _, lse_o = smp.probabilities(L, T)
    ltol = _key_tol(L, T)
    assert np.all(np.abs(lse - lse_o) <= ltol), (lse, lse_o)
    for r, d in enumerate(drafts):
        if 0 <= d < V:
            assert abs(zd[r] - L[r, d] / T) <= ltol[r]
    check_draws(sample, L, drafts, T, seed, P0)


def _round_cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        H = int(32 * rng.integers(1, 129))
        K = int(rng.integers(1, 64))
        V = int(rng.integers(2, min(20000, ELEMS // H) + 1))
        out.append((V, H, K, int(rng.integers(1, 9)), int(rng.integers(0, 3000))))
    return out


@pytest.mark.parametrize("V,H,K,n,ctx_len", _round_cases(20261205, 12) + [(2000, 512, 8, 3, 0)])
def test_round_random_shape(V, H, K, n, ctx_len):
    """Three fused rounds from a Zipf context with copied spans, and once from an empty stream
    (no drafts, so the first round commits only the argmax of its first window row)."""
    say(f"round random V={V} H={H} K={K} n={n} ctx={ctx_len}")
    S = K + 1
    rng = np.random.default_rng(V + H + K + n + ctx_len)
    q, s = synth.quantized_head(np.random.SeedSequence(V + 3 * H), V, H)
    ctx = synth.zipf_context_with_copies(rng, ctx_len, V, 0.3)[0] if ctx_len else np.zeros(0, np.int32)
    hidden = synth.fp16_normal(rng, (3, S, H))
    cap = ctx_len + 3 * S + 8
    buf = np.zeros(cap, dtype=np.int32)
    buf[:ctx_len] = ctx
    tokens = to_dev(buf)
    state = sv.new_state(dev())
    state[sv.STATE_LEN] = ctx_len
    drafts = torch.empty(K, dtype=torch.int32, device=dev())
    argmax = torch.empty(S, dtype=torch.int32, device=dev())
    work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    wq, ws = to_dev(q), to_dev(s)
    sv.propose(tokens, state, drafts, n)
    torch.cuda.synchronize()
    stream = [int(t) for t in ctx]
    d = drafts.cpu().tolist()
    assert d == list(oracle.propose_scan(stream, n, K)[0])
    for r in range(3):
        sv.round(wq, ws, to_dev(hidden[r]), drafts, tokens, state, drafts, argmax, work, n)
        torch.cuda.synchronize()
        a_gpu = argmax.cpu().numpy()
        check_argmax(a_gpu, oracle.head_logits(q, s, hidden[r]))
        _, app = oracle.accept(a_gpu, d)
        stream += app
        m = int(state[sv.STATE_LEN])
        assert m == len(stream) and tokens[:m].cpu().tolist() == stream, r
        d = drafts.cpu().tolist()
        assert d == list(oracle.propose_scan(stream, n, K)[0]), r
    assert int(state[sv.STATE_FLAGS]) == 0


def _tree_cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        H = int(32 * rng.integers(1, 129))
        V = int(rng.choice([int(rng.integers(2, 40)), int(rng.integers(40, min(20000, ELEMS // H) + 1))]))
        K = int(rng.integers(1, 16))
        out.append((V, H, K, int(rng.integers(1, 5)), int(rng.integers(1, K + 1)), int(rng.integers(1, 9)),
                    int(rng.integers(1, 3000))))
    return out


@pytest.mark.parametrize("V,H,K,B,D,n,ctx_len", _tree_cases(20261206, 10))
def test_round_tree_random_shape(V, H, K, B, D, n, ctx_len):
    """Three fused tree rounds (K nodes from the B best matches D deep, n-gram order n): the
    argmax rows against the oracle's logits (near-tie rule), then the walk, the committed stream
    and the next tree exactly against oracle.tree applied to the GPU's argmax rows.  Small
    vocabularies make accepted paths common."""
    say(f"round_tree random V={V} H={H} K={K} B={B} D={D} n={n} ctx={ctx_len}")
    S = K + 1
    rng = np.random.default_rng(V + H + K + B + D + n + ctx_len)
    q, s = synth.quantized_head(np.random.SeedSequence(V + 5 * H), V, H)
    ctx = synth.zipf_context_with_copies(rng, ctx_len, V, 0.3)[0]
    hidden = synth.fp16_normal(rng, (3, S, H))
    cap = ctx_len + 3 * S + 8
    buf = np.zeros(cap, dtype=np.int32)
    buf[:ctx_len] = ctx
    tokens = to_dev(buf)
    state = sv.new_state(dev())
    state[sv.STATE_LEN] = ctx_len
    parents = torch.empty(K, dtype=torch.int32, device=dev())
    drafts = torch.empty(K, dtype=torch.int32, device=dev())
    argmax = torch.empty(S, dtype=torch.int32, device=dev())
    work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    wq, ws = to_dev(q), to_dev(s)
    sv.propose_tree(tokens, state, parents, drafts, n, B, D)
    torch.cuda.synchronize()
    stream = [int(t) for t in ctx]
    p0, d0, _, _ = tr.propose_tree(stream, n, K, B, D)
    assert parents.cpu().tolist() == list(p0) and drafts.cpu().tolist() == list(d0)
    for r in range(3):
        sv.round_tree(wq, ws, to_dev(hidden[r]), parents, drafts, tokens, state, parents, drafts, argmax, work,
                      n, B, D)
        torch.cuda.synchronize()
        a_gpu = argmax.cpu().numpy()
        check_argmax(a_gpu, oracle.head_logits(q, s, hidden[r]))
        j, app, _ = tr.tree_accept(a_gpu, p0, d0)
        stream += app
        m = int(state[sv.STATE_LEN])
        assert m == len(stream) and tokens[:m].cpu().tolist() == stream and int(state[sv.STATE_J]) == j, r
        p0, d0, _, _ = tr.propose_tree(stream, n, K, B, D)
        assert parents.cpu().tolist() == list(p0) and drafts.cpu().tolist() == list(d0), r
    assert int(state[sv.STATE_FLAGS]) == 0


def _stack_cases(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        H = int(512 * rng.integers(1, 9))
        F = int(512 * rng.integers(1, 13))
        if H * F > 8 * 1024 * 1024:
            continue
        out.append((H, F, int(rng.integers(1, 17)), int(rng.integers(1, 4))))
    return out


@pytest.mark.parametrize("H,F,S,L", _stack_cases(20261207, 10))
def test_stack_random_shape(H, F, S, L):
    """The dense stack at random block shapes (hidden and inner sizes multiples of 512, S = 1..16,
    1..3 blocks): every block of the multi-block call equals a single-block call on its input,
    and each single-block call meets the teacher-forced oracle bounds of the fixed-shape stack
    tests at both stages."""
    from test_gpu_stack_fused import _check_block, _run, _stacked
    say(f"stack random H={H} F={F} S={S} L={L}")
    rng = np.random.default_rng(H + 7 * F + S + L)
    layers, mats = _stacked(rng, L, H, F)
    x = (synth.fp16_normal(rng, (S, H)).astype(np.float32) * 3).astype(np.float16)
    _, xl, nrm = _run(mats, x, L)
    prev = x
    for li in range(L):
        _, xl1, nrm1, m_gpu, ss = _run([m[li:li + 1] for m in mats], prev, 1, want_ws=True)
        assert np.array_equal(xl1[0], xl[li]), f"block {li}: differs from a single-block call"
        _check_block(prev, layers[li], xl1[0], nrm1, m_gpu, ss)
        prev = xl[li]
    assert np.array_equal(nrm, nrm1)
