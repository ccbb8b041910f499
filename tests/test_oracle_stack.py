"""Pins for the stack oracle: RMSNorm closed forms, SiLU special values, projections
against exact rational arithmetic, and the composition order of one block."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from weight_bound_verify_amd import synth


def test_rmsnorm_closed_forms():
    x = np.full((2, 64), 3.0, dtype=np.float16)
    x[1] *= -1
    y = oracle.rmsnorm_fp16(x, eps=0.0)
    assert (y[0] == 1).all() and (y[1] == -1).all()
    rng = np.random.default_rng(0)
    v = synth.fp16_normal(rng, (3, 256))
    a = oracle.rmsnorm_fp16(v, eps=0.0).astype(np.float64)
    assert np.sqrt(np.mean(a * a, axis=1)) == pytest.approx(np.ones(3), abs=2e-3)
    # scale invariance (powers of two keep fp16 inputs exact)
    b = oracle.rmsnorm_fp16((v.astype(np.float64) * 4).astype(np.float16), eps=0.0)
    assert np.array_equal(a.astype(np.float16), b)


def test_rmsnorm_eps_on_zero_row():
    y = oracle.rmsnorm_fp16(np.zeros((1, 32), np.float16))
    assert not y.any()


def test_silu_special_values():
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(40.0) == pytest.approx(40.0)
    assert oracle.silu(-40.0) == pytest.approx(0.0, abs=1e-15)
    assert oracle.silu(1.0) == pytest.approx(1.0 / (1.0 + np.exp(-1.0)))


def test_linear_matches_exact_rational():
    rng = np.random.default_rng(4)
    q, s = synth.quantize_q8b32(rng.standard_normal((6, 64), dtype=np.float32) * np.float32(0.02))
    x = synth.fp16_normal(rng, (2, 64))
    y = oracle.linear_q8b32(q, s, x)
    for si in range(2):
        for n in range(6):
            ex = sum(Fraction(float(s[n, k // 32])) * int(q[n, k]) * Fraction(float(x[si, k])) for k in range(64))
            assert abs(y[si, n] - float(ex)) <= 1e-12 * max(1.0, abs(float(ex)))


def test_mlp_block_composition_by_hand():
    # gate/up/down chosen so every intermediate is known: unit scales, single codes
    H, F = 32, 32
    qg = np.zeros((F, H), np.int8); qu = np.zeros((F, H), np.int8); qd = np.zeros((H, F), np.int8)
    qg[0, 0] = 1; qu[0, 0] = 2; qd[3, 0] = 1
    one = lambda r: np.ones((r, 1), np.float16)
    x = np.zeros((1, H), np.float16); x[0, 0] = 1
    layer = ((qg, one(F)), (qu, one(F)), (qd, one(H)))
    xn, parts = oracle.mlp_block(x, layer, eps=0.0, return_parts=True)
    n0 = np.sqrt(32.0)                                  # rmsnorm of e_0
    assert float(parts["n"][0, 0]) == pytest.approx(n0, rel=1e-3)
    m0 = float(oracle.silu(float(parts["n"][0, 0])) * 2 * float(parts["n"][0, 0]))
    assert float(parts["m"][0, 0]) == pytest.approx(m0, rel=1e-3)
    assert float(xn[0, 3]) == pytest.approx(m0, rel=1e-3)
    assert float(xn[0, 0]) == 1.0


def test_stack_forward_stays_finite_with_residual_and_norm():
    rng = np.random.default_rng(1)
    H, F = 64, 128
    layers = []
    for _ in range(6):
        mk = lambda r, c: synth.quantize_q8b32(rng.standard_normal((r, c), dtype=np.float32) * np.float32(0.02))
        layers.append((mk(F, H), mk(F, H), mk(H, F)))
    x = synth.fp16_normal(rng, (3, H))
    out = oracle.stack_forward(x, layers)
    assert np.isfinite(out.astype(np.float64)).all()
    assert np.sqrt(np.mean(out.astype(np.float64) ** 2, axis=1)) == pytest.approx(np.ones(3), abs=5e-3)


def _mover(src, dst, up_scale=1.0 / 16):
    """A 32-wide block whose gate and up rows read only coordinate `src` (codes 1, unit gate
    scale, up scale `up_scale`) and whose down projection writes m[0] to coordinate `dst`: on
    an input with x[src] = 0 it is the identity (silu(0) = 0)."""
    H = F = 32
    qg = np.zeros((F, H), np.int8); qu = np.zeros((F, H), np.int8); qd = np.zeros((H, F), np.int8)
    qg[0, src] = 1
    qu[0, src] = 1
    qd[dst, 0] = 1
    ones = np.ones((F, 1), np.float16)
    return ((qg, ones), (qu, np.full((F, 1), up_scale, np.float16)), (qd, np.ones((H, 1), np.float16)))


def test_stack_forward_layer_order_drop_repeat_and_final_norm():
    """Hand-built stack on x = e_0 (H = 32, eps = 0): A moves coordinate 0 into 1, B moves 1 into
    2, so B alone is the identity and only A-then-B reaches coordinate 2.  The final weightless
    norm of e_0 is fp16(sqrt(32)) = 5.65625 at coordinate 0.  A dropped, repeated or reordered
    layer, or a missing final norm, changes a known entry."""
    A, B = _mover(0, 1), _mover(1, 2)
    x = np.zeros((1, 32), np.float16)
    x[0, 0] = 1
    run = lambda layers: oracle.stack_forward(x, layers, eps=0.0)[0].astype(np.float64)
    out_b = run([B])
    assert out_b[0] == 5.65625 and not out_b[1:].any()          # identity block, then the final norm
    assert np.array_equal(run([]), out_b)                         # no block: the final norm alone
    out_a, out_ab, out_ba, out_aa = run([A]), run([A, B]), run([B, A]), run([A, A])
    assert out_a[1] > 0 and out_a[2] == 0 and not out_a[3:].any()
    assert np.array_equal(out_ba, out_a)                          # B first sees x[1] = 0
    assert out_ab[2] > 0 and out_ab[1] > 0                        # A first feeds B
    assert not np.array_equal(out_ab, out_ba)
    # a repeated A moves coordinate 0 into 1 twice: a larger share at coordinate 1
    assert out_aa[1] / out_aa[0] > out_a[1] / out_a[0]
    # every output row has unit rms (the final norm), up to fp16 rounding
    for o in (out_a, out_ab, out_aa):
        assert np.sqrt(np.mean(o * o)) == pytest.approx(1.0, abs=2e-3)
    # three layers: A, B, then a mover of 2 into 3 reaches coordinate 3 only in that order
    C = _mover(2, 3)
    assert run([A, B, C])[3] > 0 and run([A, C, B])[3] == 0 and run([C, A, B])[3] == 0
