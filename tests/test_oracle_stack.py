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
