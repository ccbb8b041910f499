"""Pins for the quantized inputs and the oracle's dequantize / logits / argmax.

Nothing here compares the oracle with itself: the quantizer is checked against invariants
that absmax symmetric rounding implies, the logits against exact rational arithmetic and a
unit-vector special case, the argmax against a plain loop and constructed ties.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from weight_bound_verify_amd import synth


# ---------------------------------------------------------------- quantizer (input bytes)
def test_quantizer_invariants_on_seeded_head():
    q, s = synth.quantized_head(np.random.SeedSequence(7), 1000, 256)
    assert q.dtype == np.int8 and s.dtype == np.float16
    assert s.shape == (1000, 8)
    qb = q.reshape(1000, 8, 32).astype(np.int64)
    assert np.abs(qb).max() <= 127
    # absmax with an RNE fp16 scale: max|w|/scale lies within 2^-11 of 127, so every
    # nonzero block reaches exactly +-127 and the clamp never fires
    nz = s.astype(np.float64) > 0
    assert nz.all()
    assert (np.abs(qb).max(axis=2) == 127).all()


def test_quantizer_reconstruction_bound():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((64, 128), dtype=np.float32) * np.float32(0.02))
    q, s = synth.quantize_q8b32(w)
    sf = np.repeat(s.astype(np.float64), 32, axis=1)
    err = np.abs(w.astype(np.float64) - q.astype(np.float64) * sf)
    assert (err <= sf / 2 + 1e-18).all()


def test_quantizer_hand_blocks():
    w = np.zeros((3, 32), dtype=np.float32)
    w[0, 5] = 0.5
    w[0, 6] = -0.5
    w[1, :] = -0.25           # constant block -> all codes -127
    # row 2 stays all-zero -> scale 0, codes 0
    q, s = synth.quantize_q8b32(w)
    assert q[0, 5] == 127 and q[0, 6] == -127 and np.count_nonzero(q[0]) == 2
    assert (q[1] == -127).all()
    assert s[2, 0] == 0 and not q[2].any()
    assert s[0, 0] == np.float16(0.5 / 127)


def test_quantized_head_independent_of_thread_count():
    a = synth.quantized_head(np.random.SeedSequence(11), 9000, 64, workers=1)
    b = synth.quantized_head(np.random.SeedSequence(11), 9000, 64, workers=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------- dequantize + logits
def _exact_logits(q, s, h):
    V, H = q.shape
    out = []
    for row in h:
        hr = [Fraction(float(x)) for x in row]
        lr = []
        for v in range(V):
            tot = Fraction(0)
            for b in range(H // 32):
                blk = sum(int(q[v, k]) * hr[k] for k in range(32 * b, 32 * b + 32))
                tot += Fraction(float(s[v, b])) * blk
            lr.append(tot)
        out.append(lr)
    return out


@pytest.mark.parametrize("V,H,S", [(5, 32, 1), (13, 64, 3), (16, 128, 2)])
def test_logits_match_exact_rational(V, H, S):
    rng = np.random.default_rng(V * 100 + H + S)
    q, s = synth.quantize_q8b32(rng.standard_normal((V, H), dtype=np.float32) * np.float32(0.02))
    h = synth.fp16_normal(rng, (S, H))
    L = oracle.head_logits(q, s, h, chunk=4)
    ex = _exact_logits(q, s, h)
    scale = max(abs(float(x)) for r in ex for x in r)
    for si in range(S):
        for v in range(V):
            assert abs(L[si, v] - float(ex[si][v])) <= 1e-12 * scale


def test_logits_unit_vector_reads_a_code_column():
    rng = np.random.default_rng(5)
    q = rng.integers(-127, 128, size=(40, 96)).astype(np.int8)
    s = np.ones((40, 3), dtype=np.float16)
    for k in (0, 31, 32, 95):
        h = np.zeros((1, 96), dtype=np.float16)
        h[0, k] = 1
        L = oracle.head_logits(q, s, h, chunk=7)
        assert np.array_equal(L[0], q[:, k].astype(np.float64))


def test_logits_scale_is_per_row_and_per_block():
    q = np.ones((2, 64), dtype=np.int8)
    s = np.array([[1, 2], [4, 8]], dtype=np.float16)
    h = np.ones((1, 64), dtype=np.float16)
    L = oracle.head_logits(q, s, h)
    assert L[0, 0] == 32 * 1 + 32 * 2 and L[0, 1] == 32 * 4 + 32 * 8


def test_logits_rows_independent_of_window_size():
    rng = np.random.default_rng(9)
    q, s = synth.quantize_q8b32(rng.standard_normal((300, 64), dtype=np.float32) * np.float32(0.02))
    h = synth.fp16_normal(rng, (9, 64))
    full = oracle.head_logits(q, s, h, chunk=64)
    for i in range(9):
        assert np.array_equal(full[i], oracle.head_logits(q, s, h[i:i + 1], chunk=64)[0])


def test_dequantize_rejects_bad_scale_shape():
    with pytest.raises(ValueError):
        oracle.dequantize(np.zeros((2, 64), np.int8), np.zeros((2, 3), np.float16))


# ---------------------------------------------------------------- argmax
def test_argmax_matches_loop_and_breaks_ties_low():
    rng = np.random.default_rng(1)
    L = rng.standard_normal((6, 50))
    L[2, 7] = L[2, 30] = L[2].max() + 1.0      # exact tie -> lowest index
    L[4, :] = 0.0
    L[4, 11] = -0.0                             # -0 == +0: still index 0
    got = oracle.argmax_lowest(L)
    for r in range(6):
        best = 0
        for v in range(1, 50):
            if L[r, v] > L[r, best]:
                best = v
        assert got[r] == best
    assert got[2] == 7 and got[4] == 0


def test_argmax_tie_from_duplicated_head_rows():
    rng = np.random.default_rng(2)
    q, s = synth.quantize_q8b32(rng.standard_normal((20, 64), dtype=np.float32) * np.float32(0.02))
    h = synth.fp16_normal(rng, (4, 64))
    a0 = oracle.argmax_lowest(oracle.head_logits(q, s, h))
    q2 = np.concatenate([q, q])
    s2 = np.concatenate([s, s])
    a1 = oracle.argmax_lowest(oracle.head_logits(q2, s2, h))
    assert np.array_equal(a0, a1)              # the copy in rows 20..39 never wins


def test_top2_gap_and_admissible_set():
    L = np.array([[1.0, 3.0, 2.9995, -1.0], [0.0, 0.0, -5.0, -5.0]])
    gap = oracle.top2_gap(L)
    assert gap[0] == pytest.approx(0.0005) and gap[1] == 0.0
    adm = oracle.admissible_sets(L, 1e-3)
    assert list(adm[0]) == [1, 2] and list(adm[1]) == [0, 1]
    assert oracle.top2_gap(np.array([[0.5], [-2.0]])).tolist() == [np.inf, np.inf]
