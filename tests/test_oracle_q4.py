"""Pins for the int4 per-block-32 head: the quantizer (input bytes) against the invariants of
absmax symmetric rounding and a hand-packed block, the oracle's int4 dequantize / logits
against exact rational arithmetic, a unit-vector special case and the nibble layout."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from weight_bound_verify_amd import synth


def test_q4_quantizer_invariants():
    q, s = synth.quantized_head_q4(np.random.SeedSequence(7), 500, 256)
    assert q.dtype == np.uint8 and q.shape == (500, 128) and s.shape == (500, 8)
    lo, hi = q & 0xF, q >> 4
    u = np.concatenate([lo.reshape(500, 8, 16), hi.reshape(500, 8, 16)], axis=2)
    assert u.min() >= 1 and u.max() <= 15                 # offset binary of -7 .. 7
    codes = u.astype(np.int64) - 8
    # with an RNE fp16 scale, max|w| / scale lies within 2^-11 of 7: every nonzero block
    # reaches exactly +-7 and the clamp never fires
    assert (np.abs(codes).max(axis=2) == 7).all()


def test_q4_reconstruction_bound_and_same_draws_as_int8():
    rng = np.random.default_rng(4)
    w = rng.standard_normal((40, 96), dtype=np.float32) * np.float32(0.02)
    p, s = synth.quantize_q4b32(w)
    wd = oracle.dequantize_q4b32(p, s)
    sf = np.repeat(s.astype(np.float64), 32, axis=1)
    assert (np.abs(w.astype(np.float64) - wd) <= sf / 2 + 1e-18).all()
    # the int4 head draws the same fp32 weights as the int8 one: both reconstruct them
    q8, s8 = synth.quantized_head(np.random.SeedSequence(3), 300, 64)
    q4, s4 = synth.quantized_head_q4(np.random.SeedSequence(3), 300, 64)
    w8 = oracle.dequantize(q8, s8)
    w4 = oracle.dequantize_q4b32(q4, s4)
    bound = np.repeat(s4.astype(np.float64), 32, axis=1) / 2 + np.repeat(s8.astype(np.float64), 32, axis=1) / 2
    assert (np.abs(w8 - w4) <= bound + 1e-18).all()


def test_q4_hand_packed_block_layout():
    """Byte i of a block: element i in the low nibble, element i + 16 in the high one."""
    codes = np.array([((k * 5) % 15) - 7 for k in range(32)], dtype=np.int64)      # -7 .. 7, all distinct mod 15
    u = codes + 8
    packed = np.array([[u[i] | (u[16 + i] << 4) for i in range(16)]], dtype=np.uint8)
    scale = np.array([[0.5]], dtype=np.float16)
    wd = oracle.dequantize_q4b32(packed, scale)
    assert np.array_equal(wd[0], codes * 0.5)
    # and the quantizer packs exactly so
    p, s = synth.quantize_q4b32((codes.astype(np.float32) * np.float32(0.5))[None])
    assert np.array_equal(p, packed) and s[0, 0] == np.float16(0.5)


def test_q4_all_zero_block():
    w = np.zeros((2, 64), dtype=np.float32)
    w[1, 40] = 3.0
    p, s = synth.quantize_q4b32(w)
    assert s[0, 0] == 0 and s[0, 1] == 0 and s[1, 0] == 0
    assert (oracle.dequantize_q4b32(p, s)[0] == 0).all()
    assert oracle.dequantize_q4b32(p, s)[1, 40] == float(np.float16(3.0 / 7)) * 7


@pytest.mark.parametrize("V,H,S", [(5, 32, 1), (17, 64, 3), (33, 128, 9)])
def test_q4_logits_match_exact_rational(V, H, S):
    rng = np.random.default_rng(V * H + S)
    p, s = synth.quantize_q4b32(rng.standard_normal((V, H), dtype=np.float32) * np.float32(0.05))
    x = synth.fp16_normal(rng, (S, H))
    L = oracle.head_logits_q4b32(p, s, x)
    for r in range(S):
        for v in range(V):
            acc = Fraction(0)
            for b in range(H // 32):
                sc = Fraction(float(s[v, b]))
                for i in range(16):
                    byte = int(p[v, 16 * b + i])
                    for k, code in ((32 * b + i, (byte & 15) - 8), (32 * b + 16 + i, (byte >> 4) - 8)):
                        acc += sc * code * Fraction(float(x[r, k]))
            assert abs(float(acc) - L[r, v]) <= 1e-12 * max(1.0, abs(float(acc)))


def test_q4_unit_vector_reads_a_code_column():
    rng = np.random.default_rng(2)
    V, H = 50, 96
    u = rng.integers(1, 16, size=(V, H)).astype(np.uint8)
    packed = np.zeros((V, H // 2), dtype=np.uint8)
    for b in range(H // 32):
        packed[:, 16 * b:16 * b + 16] = u[:, 32 * b:32 * b + 16] | (u[:, 32 * b + 16:32 * b + 32] << 4)
    s = np.ones((V, H // 32), dtype=np.float16)
    for k in (0, 15, 16, 31, 47, 95):
        e = np.zeros((1, H), dtype=np.float16)
        e[0, k] = 1
        assert np.array_equal(oracle.head_logits_q4b32(packed, s, e)[0], u[:, k].astype(np.float64) - 8)
