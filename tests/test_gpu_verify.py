"""GPU parity of specverify_verify (q8b32 head matmul + fused argmax) against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from weight_bound_verify_amd import specverify as sv
from weight_bound_verify_amd import synth

from gpu_util import check_argmax, check_logits, dev, gpu_verify, head, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("V,H,S", [
    (1, 32, 1), (15, 32, 2), (17, 64, 9), (1000, 256, 9), (1000, 256, 16), (1000, 256, 17),
    (333, 2048, 33), (100, 96, 64), (8192, 512, 9), (4099, 320, 5), (70000, 64, 3), (777, 5120, 2),
    # 17 rows: one MFMA tile plus the 17th row's dot products (H = 512, 1024, 2048, 2560, 4096)
    (3001, 512, 17), (1000, 1024, 17), (5003, 2048, 17), (2000, 2560, 17), (1500, 4096, 17),
    # one rolling register set, each with a ragged last tile: the argmax head at H = 2560, and
    # the 17-row head at H = 5120 (8 of each wave's 20 blocks of window rows held in LDS)
    (4099, 2560, 9), (2500, 5120, 17),
    # more than 32 rows in two passes of the two-tile kernel (rows 0 .. 31, then the rest), each
    # writing whole dot products, at the hidden sizes a two-tile shape covers unsplit
    (5000, 512, 40), (3001, 1024, 64), (2000, 1280, 33), (4099, 2048, 48),
])
def test_verify_matches_oracle(V, H, S):
    say(f"verify V={V} H={H} S={S}")
    q, s = head(V * 7 + H + S, V, H)
    hidden = synth.fp16_normal(np.random.default_rng(S), (S, H))
    a, lg = gpu_verify(q, s, hidden)
    L = oracle.head_logits(q, s, hidden)
    worst = check_logits(lg, L)
    check_argmax(a, L)
    say(f"  max rel err {worst:.2e}")


def test_verify_exact_on_integer_inputs():
    # unit scales and small integer hidden values: every partial sum is an exact fp32 integer
    rng = np.random.default_rng(0)
    V, H, S = 3000, 512, 9
    q = rng.integers(-127, 128, size=(V, H)).astype(np.int8)
    s = np.ones((V, H // 32), dtype=np.float16)
    hidden = rng.integers(-3, 4, size=(S, H)).astype(np.float16)
    a, lg = gpu_verify(q, s, hidden)
    L = oracle.head_logits(q, s, hidden)
    assert np.array_equal(lg, L)
    assert np.array_equal(a, oracle.argmax_lowest(L))


def test_verify_ties_take_lowest_index():
    rng = np.random.default_rng(1)
    V, H, S = 2000, 256, 9
    q, s = head(5, V, H)
    q[1500] = q[123]          # duplicated rows: exact ties
    s[1500] = s[123]
    hidden = synth.fp16_normal(rng, (S, H))
    hidden[3] = 0             # all-zero row: every logit is 0 -> id 0
    hidden[0] = np.sign(q[123]).astype(np.float16)     # rows 123 and 1500 tie for the maximum
    L = oracle.head_logits(q, s, hidden)
    assert L[0].argmax() == 123 and L[0, 1500] == L[0, 123]
    a, _ = gpu_verify(q, s, hidden)
    assert a[0] == 123 and a[3] == 0
    check_argmax(a, L)


def test_verify_without_logits_same_argmax():
    q, s = head(9, 5000, 1024)
    hidden = synth.fp16_normal(np.random.default_rng(2), (9, 1024))
    a1, _ = gpu_verify(q, s, hidden, want_logits=True)
    a2, _ = gpu_verify(q, s, hidden, want_logits=False)
    assert np.array_equal(a1, a2)


def test_verify_deterministic_and_window_size_invariant():
    V, H = 20000, 2048
    q, s = head(11, V, H)
    hidden = synth.fp16_normal(np.random.default_rng(3), (16, H))
    wq, ws = to_dev(q), to_dev(s)
    a16, l16 = gpu_verify(q, s, hidden, wq=wq, ws=ws)
    a16b, l16b = gpu_verify(q, s, hidden, wq=wq, ws=ws)
    assert np.array_equal(l16, l16b) and np.array_equal(a16, a16b)
    for S in (1, 9):
        aS, lS = gpu_verify(q, s, hidden[:S], wq=wq, ws=ws)
        assert np.array_equal(lS, l16[:S]), f"S={S} rows differ bitwise from S=16"
        assert np.array_equal(aS, a16[:S])


@pytest.mark.parametrize("nw,grid", [(4, 0), (8, 1), (16, 7), (0, 4096), (8, 300)])
def test_verify_launch_shapes_agree(nw, grid):
    V, H, S = 6000, 2560, 9
    q, s = head(13, V, H)
    hidden = synth.fp16_normal(np.random.default_rng(4), (S, H))
    L = oracle.head_logits(q, s, hidden)
    try:
        sv.set_tuning(nw, grid)
        a, lg = gpu_verify(q, s, hidden)
    finally:
        sv.set_tuning(0, 0)
    check_logits(lg, L)
    check_argmax(a, L)


@pytest.mark.parametrize("V,S,groups", [(70001, 9, 0), (70031, 17, 0), (70031, 1, 64), (70001, 16, 333),
                                        (65573, 9, 104), (65573, 9, 100)])
def test_verify_per_die_item_ranges(V, S, groups):
    """Heads over 2 KB rows with at least 8 items per workgroup take their items in one
    contiguous range per die: item counts that 8 divides and that it does not (4376, 4377, 4099),
    a last tile of one row, the 17-row window, and grids capped at 64, 104 and 333 workgroups
    (8, 13 and 40 per die).  A cap of 100 leaves a grid of 100, which cannot be rounded up to a
    multiple of 8 within the cap, so that launch keeps the interleaved order.  Every logit
    (pre-filled with NaN) and every argmax row against the oracle."""
    H = 2048
    say(f"per-die item ranges V={V} S={S} groups={groups}")
    q, s = head(V + S, V, H)
    hidden = synth.fp16_normal(np.random.default_rng(V + S + groups), (S, H))
    try:
        sv.set_tuning(0, groups)
        a, lg = gpu_verify(q, s, hidden)
        a2, _ = gpu_verify(q, s, hidden, want_logits=False)
    finally:
        sv.set_tuning(0, 0)
    L = oracle.head_logits(q, s, hidden)
    check_logits(lg, L)
    check_argmax(a, L)
    assert np.array_equal(a, a2)


def test_verify_split_hidden_axis_path():
    # S = 40 (three M tiles of 16) with H = 16384: the hidden axis is split across workgroups
    V, H, S = 900, 16384, 40
    assert sv.verify_workspace_bytes(V, H, S) > 8 * S * 4096
    q, s = head(17, V, H)
    hidden = synth.fp16_normal(np.random.default_rng(5), (S, H))
    a, lg = gpu_verify(q, s, hidden)
    L = oracle.head_logits(q, s, hidden)
    check_logits(lg, L)
    check_argmax(a, L)


@pytest.mark.parametrize("S", [9, 17])
def test_verify_full_35b_head_shape(S):
    V, H = 248320, 2048
    say(f"full head V={V} H={H} S={S}")
    st = synth.streams(2)
    q, s = synth.quantized_head(st.weights, V, H)
    hidden = synth.fp16_normal(st.hidden, (S, H))
    a, lg = gpu_verify(q, s, hidden)
    L = oracle.head_logits(q, s, hidden)
    check_logits(lg, L)
    ex = check_argmax(a, L)
    say(f"  argmax rows exempt by the 1e-3 gap rule: {ex}")


@pytest.mark.parametrize("V,H", [(151936, 2560), (151936, 4096)])
def test_verify_full_151936_vocab_heads(V, H):
    """The Qwen3-4B-shaped head (H = 2560: 8 blocks x 10 waves) and the dense stack's head
    (H = 4096: 16 x 8) at full size and S = 9, in the launch configuration the bench uses."""
    S = 9
    say(f"full head V={V} H={H} S={S}")
    st = synth.streams(1 if H == 2560 else 4)
    q, s = synth.quantized_head(st.weights, V, H)
    hidden = synth.fp16_normal(st.hidden, (S, H))
    a, lg = gpu_verify(q, s, hidden)
    L = oracle.head_logits(q, s, hidden)
    check_logits(lg, L)
    check_argmax(a, L)


@pytest.mark.parametrize("S", [2, 9, 17])
def test_verify_full_large_hidden_shape(S):
    """248320 x 5120 at every window size of that workload, in the launch configuration the
    bench uses (S = 17: the one-tile kernel with the 17th row's dot products and 8 of each
    wave's 20 blocks of window rows in LDS); the oracle computes every logit in fp64."""
    V, H = 248320, 5120
    say(f"full head V={V} H={H} S={S}")
    st = synth.streams(3)
    q, s = synth.quantized_head(st.weights, V, H)
    hidden = synth.fp16_normal(st.hidden, (S, H))
    a, lg = gpu_verify(q, s, hidden)
    L = oracle.head_logits(q, s, hidden)
    check_logits(lg, L)
    check_argmax(a, L)


@pytest.mark.parametrize("V,H,S", [(1000, 512, 9), (4099, 2048, 9), (777, 4096, 16), (70000, 2048, 1), (5000, 5120, 9),
                                   (33, 512, 3)])
def test_verify_ring_kernel_matches_oracle(V, H, S):
    """The chunked ring kernel for the head (selected through the tuning switch)."""
    say(f"verify ring kernel V={V} H={H} S={S}")
    q, s = head(V * 3 + H + S, V, H)
    hidden = synth.fp16_normal(np.random.default_rng(S + 1), (S, H))
    try:
        sv.set_tuning(0, 0, 0, 2)
        a, lg = gpu_verify(q, s, hidden)
        a2, _ = gpu_verify(q, s, hidden, want_logits=False)
    finally:
        sv.set_tuning(0, 0, 0, 0)
    L = oracle.head_logits(q, s, hidden)
    check_logits(lg, L)
    check_argmax(a, L)
    assert np.array_equal(a, a2)


@pytest.mark.parametrize("H", [2048, 5120])
def test_verify_17_rows_both_kernels_agree(H):
    """A 17-row window through the one-tile-plus-dot-products kernel and through two 16-row
    tiles: the same argmax wherever the top-2 gap is clear of the tolerance."""
    V, S = 9000, 17
    q, s = head(17, V, H)
    hidden = synth.fp16_normal(np.random.default_rng(17), (S, H))
    L = oracle.head_logits(q, s, hidden)
    a1, l1 = gpu_verify(q, s, hidden)
    sv.set_tuning(0, 0, 0, 3)
    try:
        a2, l2 = gpu_verify(q, s, hidden)
    finally:
        sv.set_tuning(0, 0, 0, 0)
    check_logits(l1, L)
    check_logits(l2, L)
    check_argmax(a1, L)
    check_argmax(a2, L)


@pytest.mark.parametrize("V,H,S", [(20000, 2048, 9), (900, 16384, 40), (20000, 2048, 40)])
def test_timing_hook_brackets_exactly_one_matmul(V, H, S):
    """specverify_profile_next_matmul attaches the caller's events to the next matmul's dispatch
    (through the combine pass when the hidden axis is split, the second shape; across both
    passes of a window of more than 32 rows, the third): both events
    complete with a positive duration, the results are those of an untimed call, and the hook
    is consumed, so the next call runs untimed."""
    q, s = head(23, V, H)
    hidden = to_dev(synth.fp16_normal(np.random.default_rng(9), (S, H)))
    wq, ws = to_dev(q), to_dev(s)
    work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    a0 = torch.empty(S, dtype=torch.int32, device=dev())
    a1 = torch.empty(S, dtype=torch.int32, device=dev())
    a2 = torch.empty(S, dtype=torch.int32, device=dev())
    sv.verify(wq, ws, hidden, a0, work)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sv.profile_next_matmul(e0, e1)
    sv.verify(wq, ws, hidden, a1, work)
    sv.verify(wq, ws, hidden, a2, work)                  # the hook is spent: untimed
    torch.cuda.synchronize()
    assert e0.query() and e1.query()
    assert e0.elapsed_time(e1) > 0.0
    assert torch.equal(a0, a1) and torch.equal(a0, a2)
