"""GPU parity of specverify_stack (the whole dense stack in two chunked launches per block, its
RMSNorm carried as per-tile sum-of-squares partials) against the CPU oracle.

A single-block call is checked teacher-forced at both of its stages against oracle.mlp_block:
m = silu(g)*u (read back from the workspace) against the oracle's m from the same input, then
the block output against x + m_gpu Wd^T.  A multi-block call is checked by exact equality: every
block output it writes to x_layers must equal, bit for bit, a single-block call on that block's
input (the previous output), because both compute the same sums in the same order (the norm
partials of a caller's input are summed in the order the down epilogue uses).  So every block of
a multi-block call meets the single-block bound.  The dense-stack workload itself (36 blocks of
4096 -> 12288 -> 4096 at S = 9, then the 151936-row head) is checked this way in full."""
import numpy as np
import pytest
import torch

import oracle
from weight_bound_verify_amd import specverify as sv
from weight_bound_verify_amd import synth

from gpu_util import check_argmax, check_logits, dev, gpu_verify, say, to_dev

pytestmark = pytest.mark.gpu


def _check_f16(got16, ref64, slack=1e-4):
    """fp16 outputs: within one fp16 rounding step of the fp64 value plus slack * row rms."""
    got = got16.astype(np.float64)
    ulp = np.spacing(np.abs(ref64.astype(np.float16))).astype(np.float64)
    rms = np.sqrt(np.mean(ref64 * ref64, axis=-1, keepdims=True))
    err = np.abs(got - ref64)
    bad = np.argwhere(~(err <= ulp + slack * rms))
    assert bad.size == 0, f"{len(bad)} outputs outside, first {bad[:3].tolist()} err {err[tuple(bad[0])]}"


def _m_bound(x16, parts, layer, eps=1e-6):
    """Largest |m_gpu - m| the rounding of the normalised row can cause: where x / rms lies
    within fp32 noise (4e-7 relative) of an fp16 rounding midpoint the library may round n to
    the other neighbour (its 1/rms is fp32); each such element moves g and u by at most one
    n ulp times the weights, and m = silu(g) u moves by |silu'(g)| |u| dg + |silu(g)| du
    (|silu'| <= 1.1)."""
    xx = x16.astype(np.float64)
    t = xx / np.sqrt(np.mean(xx * xx, axis=-1, keepdims=True) + eps)
    n16 = t.astype(np.float16).astype(np.float64)
    ulp_n = np.spacing(np.abs(t.astype(np.float16))).astype(np.float64)
    amb = np.abs(np.abs(t - n16) - ulp_n / 2) <= 4e-7 * np.abs(t) + 1e-12
    dn = np.where(amb, ulp_n, 0.0)                                   # [S][H]
    (qg, sg), (qu, su), _ = layer
    dg = dn @ np.abs(oracle.dequantize(qg, sg)).T                    # [S][F]
    du = dn @ np.abs(oracle.dequantize(qu, su)).T
    g, u = parts["g"], parts["u"]
    return 1.1 * np.abs(u) * dg + np.abs(oracle.silu(g)) * du


def _stacked(rng, L, H, F):
    def w(r, c):
        return synth.quantize_q8b32(rng.standard_normal((r, c), dtype=np.float32) * np.float32(synth.W_STD))
    layers = [(w(F, H), w(F, H), w(H, F)) for _ in range(L)]
    cat = lambda i, j: np.stack([lay[i][j] for lay in layers])
    return layers, [cat(0, 0), cat(0, 1), cat(1, 0), cat(1, 1), cat(2, 0), cat(2, 1)]


def _run(mats, x, L, eps=1e-6, layers_out=True, want_ws=False):
    S, H = x.shape
    F = mats[0].shape[1]
    dm = [to_dev(m) for m in mats]
    xd = to_dev(x)
    xl = torch.full((L, S, H), float("nan"), dtype=torch.float16, device=dev()) if layers_out else None
    nrm = torch.full((S, H), float("nan"), dtype=torch.float16, device=dev())
    ws = sv.workspace(sv.stack_forward_workspace_bytes(H, F, S), dev())
    sv.stack(*dm, xd, nrm, ws, eps, x_layers=xl)
    torch.cuda.synchronize()
    out = (xd.cpu().numpy(), (xl.cpu().numpy() if layers_out else None), nrm.cpu().numpy())
    if not want_ws:
        return out
    # workspace layout: m = silu(g)*u [S][F] fp16, then the sum-of-squares partials [S][H/16] fp32,
    # each part 256-byte aligned
    w = ws.cpu().numpy()
    m = w[:2 * S * F].view(np.float16).reshape(S, F)
    off = (2 * S * F + 255) // 256 * 256
    ss = w[off:off + 4 * S * (H // 16)].view(np.float32).reshape(S, H // 16)
    return out + (m, ss)


SHAPES = [
    (512, 1024, 9, 3),      # 4 waves, one chunk (held window rows)
    (1024, 1536, 16, 2),    # gate/up 8 waves x 1 chunk; down 12 waves x 1 chunk
    (2048, 512, 1, 2),
    (512, 2048, 5, 2),
    (4096, 12288, 9, 1),    # the dense-stack workload's block shape
    (2560, 1536, 9, 2),     # 10 waves x 2 held chunks (gate/up); 12 waves (down)
    (3584, 2560, 16, 1),    # 14 waves; down 10 waves
]


def _check_block(x, layer, xl0, nrm, m_gpu, ss, eps=1e-6):
    """One block from input x, teacher-forced at both stages: the GPU's m = silu(g)*u within one
    fp16 rounding of the oracle's m from the same input (the norm and both projections of
    gate/up; plus the effect of normalised elements whose fp16 rounding fp32 cannot decide),
    the block output within one rounding of x + m_gpu Wd^T (the down projection, residual and
    store), the down epilogue's sum-of-squares partials and the final norm."""
    S, H = x.shape
    _, parts = oracle.mlp_block(x, layer, eps=eps, return_parts=True)
    ref_m = oracle.silu(parts["g"]) * parts["u"]
    ulp = np.spacing(np.abs(ref_m.astype(np.float16))).astype(np.float64)
    rms = np.sqrt(np.mean(ref_m * ref_m, axis=-1, keepdims=True))
    err = np.abs(m_gpu.astype(np.float64) - ref_m)
    bad = np.argwhere(~(err <= ulp + 1e-5 * rms + _m_bound(x, parts, layer, eps)))
    assert bad.size == 0, f"m: {len(bad)} outside, first {bad[:3].tolist()} err {err[tuple(bad[0])]}"
    _check_f16(xl0, x.astype(np.float64) + oracle.linear_q8b32(*layer[2], m_gpu), slack=1e-5)
    out = xl0.astype(np.float64)
    # the down epilogue's per-16-column sums of squares of the stored fp16 outputs
    ref_ss = (out.reshape(S, H // 16, 16) ** 2).sum(-1)
    assert np.allclose(ss, ref_ss, rtol=1e-5, atol=0), "sum-of-squares partials"
    _check_f16(nrm, out / np.sqrt(np.mean(out * out, axis=1, keepdims=True) + eps), slack=1e-5)


SPLITS = {(512, 1024, 9, 3): 2, (1024, 1536, 16, 2): 3, (512, 2048, 5, 2): 4, (4096, 12288, 9, 1): 8,
          (2560, 1536, 9, 2): 3, (3584, 2560, 16, 1): 5}


@pytest.mark.parametrize("H,F,S,L,split", [(*sh, "unsplit") for sh in SHAPES] +
                         [(*sh, "split") for sh in SHAPES if sh in SPLITS])
def test_stack_block_by_block_teacher_forced(H, F, S, L, split):
    """Each block on its own (L = 1 per call), checked at both stages against the oracle, with
    the down projection unsplit (the automatic choice) and, where a held-row shape splits it,
    with its hidden axis split across workgroups (2 .. 8 slices, each shape's own count)."""
    split = SPLITS[(H, F, S, L)] if split == "split" else 0
    say(f"stack block by block H={H} F={F} S={S} L={L} split={split}")
    rng = np.random.default_rng(H + 3 * F + S + L)
    layers, mats = _stacked(rng, L, H, F)
    x = (synth.fp16_normal(rng, (S, H)).astype(np.float32) * 3).astype(np.float16)
    sv.set_tuning(0, 0, 0, 0, split)
    try:
        base = (2 * S * F + 255) // 256 * 256 + (4 * S * (H // 16) + 255) // 256 * 256
        assert (sv.stack_forward_workspace_bytes(H, F, S) > base) == (split > 1), "split not applied"
        for li in range(L):
            one = [m[li:li + 1] for m in mats]
            _, xl, nrm, m_gpu, ss = _run(one, x, 1, want_ws=True)
            _check_block(x, layers[li], xl[0], nrm, m_gpu, ss)
            x = xl[0]
    finally:
        sv.set_tuning(0, 0, 0, 0, 0)


@pytest.mark.parametrize("ks", [2, 3, 4, 6, 8])
def test_stack_down_split_counts(ks):
    """The dense-stack block shape (4096 -> 12288 -> 4096, S = 9) with its down projection
    split 2 .. 8 ways where a shape exists (3, 4, 6, 8; 2 falls back to unsplit): two blocks,
    each teacher-forced against the oracle; the second block's norm comes from the fold's
    sum-of-squares partials, and the tile counters the first launch left must be zero again."""
    H, F, S, L = 4096, 12288, 9, 2
    say(f"stack down split ks={ks}")
    rng = np.random.default_rng(77 + ks)
    layers, mats = _stacked(rng, L, H, F)
    x = (synth.fp16_normal(rng, (S, H)).astype(np.float32) * 3).astype(np.float16)
    sv.set_tuning(0, 0, 0, 0, ks)
    try:
        _, xl, nrm = _run(mats, x, L)
        # the counters after a call: zero (the workspace's last 256-byte-aligned part when split)
        ws = sv.workspace(sv.stack_forward_workspace_bytes(H, F, S), dev())
        ws.fill_(0x5A)
        sv.stack(*[to_dev(m) for m in mats], to_dev(x), to_dev(np.zeros((S, H), np.float16)), ws, 1e-6,
                 x_layers=to_dev(np.zeros((L, S, H), np.float16)))
        torch.cuda.synchronize()
        al = lambda b: (b + 255) // 256 * 256
        base = al(2 * S * F) + al(4 * S * (H // 16))
        tiles = H // 16
        if ws.numel() > base:
            cnt = ws.cpu().numpy()[-al(4 * tiles):][:4 * tiles].view(np.uint32)
            assert (cnt == 0).all(), "tile counters not left at zero"
        prev = x
        for li in range(L):
            _, xl1, nrm1, m_gpu, ss = _run([m[li:li + 1] for m in mats], prev, 1, want_ws=True)
            assert np.array_equal(xl1[0], xl[li]), f"block {li}: multi-block output differs"
            _check_block(prev, layers[li], xl1[0], nrm1, m_gpu, ss)
            prev = xl[li]
        assert np.array_equal(nrm, nrm1)
    finally:
        sv.set_tuning(0, 0, 0, 0, 0)


@pytest.mark.parametrize("H,F,S,L", [sh for sh in SHAPES if sh[3] > 1])
def test_stack_equals_chained_single_blocks(H, F, S, L):
    """The multi-block call (each block's norm from the previous down epilogue's partials) writes
    the same bits as L single-block calls chained on its own outputs, each of which is checked
    against the oracle as above; its final norm equals the last single-block call's."""
    say(f"stack H={H} F={F} S={S} L={L}")
    rng = np.random.default_rng(H + 3 * F + S + L)
    layers, mats = _stacked(rng, L, H, F)
    x = (synth.fp16_normal(rng, (S, H)).astype(np.float32) * 3).astype(np.float16)
    x_out, xl, nrm = _run(mats, x, L)
    assert np.array_equal(x_out, x), "x must be left unchanged when x_layers is given"
    prev = x
    for li in range(L):
        one = [m[li:li + 1] for m in mats]
        _, xl1, nrm1, m_gpu, ss = _run(one, prev, 1, want_ws=True)
        assert np.array_equal(xl1[0], xl[li]), f"block {li}: multi-block output differs from a single-block call"
        _check_block(prev, layers[li], xl1[0], nrm1, m_gpu, ss)
        prev = xl[li]
    assert np.array_equal(nrm, nrm1), "final norm differs from the last single-block call's"


def test_stack_in_place_is_bit_identical_to_layer_outputs():
    rng = np.random.default_rng(5)
    H, F, S, L = 1024, 2048, 9, 4
    _, mats = _stacked(rng, L, H, F)
    x = synth.fp16_normal(rng, (S, H))
    _, xl, n1 = _run(mats, x, L)
    x_in_place, _, n2 = _run(mats, x, L, layers_out=False)
    assert np.array_equal(x_in_place, xl[L - 1])
    assert np.array_equal(n1, n2)


def test_stack_depth_variants_bit_identical():
    """The pipeline depth changes only when loads are issued, never the arithmetic order."""
    rng = np.random.default_rng(6)
    H, F, S, L = 2048, 4096, 9, 2
    _, mats = _stacked(rng, L, H, F)
    x = synth.fp16_normal(rng, (S, H))
    try:
        outs = []
        for nw, depth in [(8, 2), (8, 4), (4, 2), (4, 4)]:
            sv.set_tuning(nw, 0, depth)
            _, xl, nrm = _run(mats, x, L)
            outs.append((nw, xl, nrm))
    finally:
        sv.set_tuning(0, 0, 0)
    for (nw0, a, na), (nw1, b, nb) in zip(outs, outs[1:]):
        if nw0 == nw1:
            assert np.array_equal(a, b) and np.array_equal(na, nb)


def test_stack_eps_and_zero_rows():
    """An all-zero window row stays zero through the blocks (rmsnorm of 0 is 0 with eps > 0);
    every block equals a single-block call on its input and meets the oracle bound at eps = 1e-3."""
    rng = np.random.default_rng(8)
    H, F, S, L = 512, 1024, 4, 2
    layers, mats = _stacked(rng, L, H, F)
    x = synth.fp16_normal(rng, (S, H))
    x[2] = 0
    _, xl, nrm = _run(mats, x, L, eps=1e-3)
    assert (xl[:, 2] == 0).all() and (nrm[2] == 0).all()
    prev = x
    for li in range(L):
        _, xl1, nrm1, m_gpu, ss = _run([m[li:li + 1] for m in mats], prev, 1, eps=1e-3, want_ws=True)
        assert np.array_equal(xl1[0], xl[li])
        _check_block(prev, layers[li], xl1[0], nrm1, m_gpu, ss, eps=1e-3)
        prev = xl[li]


def test_stack_timing_hook_times_the_first_gate_up():
    """specverify_profile_next_matmul before specverify_stack attaches the events to block 0's
    gate/up launch: both complete with a positive duration shorter than the whole call, and
    every output is bit-identical to an untimed call."""
    rng = np.random.default_rng(15)
    H, F, S, L = 1024, 2048, 9, 4
    _, mats = _stacked(rng, L, H, F)
    x = synth.fp16_normal(rng, (S, H))
    ref = _run(mats, x, L)
    dm = [to_dev(m) for m in mats]
    xd = to_dev(x)
    xl = torch.empty((L, S, H), dtype=torch.float16, device=dev())
    nrm = torch.empty((S, H), dtype=torch.float16, device=dev())
    ws = sv.workspace(sv.stack_forward_workspace_bytes(H, F, S), dev())
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sv.profile_next_matmul(e0, e1)
    a.record()
    sv.stack(*dm, xd, nrm, ws, 1e-6, x_layers=xl)
    b.record()
    torch.cuda.synchronize()
    t_gu, t_all = e0.elapsed_time(e1), a.elapsed_time(b)
    assert 0.0 < t_gu < t_all
    assert np.array_equal(xl.cpu().numpy(), ref[1]) and np.array_equal(nrm.cpu().numpy(), ref[2])


# ---------------------------------------------------------------------------------------------
# The dense-stack workload in full: 36 blocks of 4096 -> 12288 -> 4096 at S = 9 through one
# specverify_stack call (the call the dense-stack bench times), then the 151936 x 4096 head.
# Layer l's three matrices are seeded row rotations of three drawn base matrices (distinct
# layers with the drawn value distribution, built on the device in seconds), so a dropped,
# repeated or reordered block changes the outputs.
# ---------------------------------------------------------------------------------------------
C5_H, C5_F, C5_S, C5_L, C5_V = 4096, 12288, 9, 36, 151936


def _c5_layer(base, shifts, li):
    """Layer li's ((qg, sg), (qu, su), (qd, sd)) on the host: base matrix m rotated by shifts[li, m] rows."""
    return tuple((np.roll(q, int(shifts[li, m]), axis=0), np.roll(s, int(shifts[li, m]), axis=0))
                 for m, (q, s) in enumerate(base))


@pytest.fixture(scope="module")
def c5_stack():
    H, F, S, L = C5_H, C5_F, C5_S, C5_L
    say("C5 stack: drawing the base matrices")
    rng = np.random.default_rng(20261206)
    base = [synth.quantized_head(np.random.SeedSequence(20261206 + i), r, c)
            for i, (r, c) in enumerate([(F, H), (F, H), (H, F)])]
    shifts = np.stack([rng.integers(1, n, size=L) for n in (F, F, H)], axis=1)     # [L][3]
    mats = []
    for m, (q, s) in enumerate(base):
        qd, sd = to_dev(q), to_dev(s)
        Q = torch.empty((L,) + q.shape, dtype=torch.int8, device=dev())
        Sc = torch.empty((L,) + s.shape, dtype=torch.float16, device=dev())
        for li in range(L):
            Q[li].copy_(torch.roll(qd, int(shifts[li, m]), 0))
            Sc[li].copy_(torch.roll(sd, int(shifts[li, m]), 0))
        mats += [Q, Sc]
        del qd, sd
    x = synth.fp16_normal(rng, (S, H))
    xd = to_dev(x)
    xl = torch.full((L, S, H), float("nan"), dtype=torch.float16, device=dev())
    nrm = torch.full((S, H), float("nan"), dtype=torch.float16, device=dev())
    ws = sv.workspace(sv.stack_forward_workspace_bytes(H, F, S), dev())
    say("C5 stack: the 36-block call")
    sv.stack(*mats, xd, nrm, ws, 1e-6, x_layers=xl)
    torch.cuda.synchronize()
    xl_h, nrm_h = xl.cpu().numpy(), nrm.cpu().numpy()
    say("C5 stack: 36 single-block calls on the call's own block inputs")
    singles, equal = [], []
    xl1 = torch.empty((1, S, H), dtype=torch.float16, device=dev())
    nrm1 = torch.empty((S, H), dtype=torch.float16, device=dev())
    for li in range(L):
        prev = xd if li == 0 else xl[li - 1]
        sv.stack(*[m[li:li + 1] for m in mats], prev.clone(), nrm1, ws, 1e-6, x_layers=xl1)
        torch.cuda.synchronize()
        w = ws.cpu().numpy()
        m_gpu = w[:2 * S * F].view(np.float16).reshape(S, F).copy()
        off = (2 * S * F + 255) // 256 * 256
        ss = w[off:off + 4 * S * (H // 16)].view(np.float32).reshape(S, H // 16).copy()
        singles.append((xl1[0].cpu().numpy(), nrm1.cpu().numpy(), m_gpu, ss))
        equal.append(bool(torch.equal(xl1[0], xl[li])))
    del mats
    torch.cuda.empty_cache()
    return dict(base=base, shifts=shifts, x=x, xl=xl_h, nrm=nrm_h, singles=singles, equal=equal,
                nrm_last_equal=bool(np.array_equal(singles[-1][1], nrm_h)))


def test_c5_stack_equals_chained_single_blocks(c5_stack):
    """Every block output of the 36-block call equals a single-block call on its input, and the
    call's norm_out equals the last single-block call's."""
    bad = [li for li, ok in enumerate(c5_stack["equal"]) if not ok]
    assert not bad, f"blocks {bad} differ from single-block calls"
    assert c5_stack["nrm_last_equal"]


@pytest.mark.parametrize("lo", range(0, C5_L, 6))
def test_c5_stack_blocks_against_oracle(c5_stack, lo):
    """Blocks lo .. lo+5 of the 36-block call, teacher-forced against oracle.mlp_block."""
    for li in range(lo, min(lo + 6, C5_L)):
        say(f"C5 block {li}")
        x_in = c5_stack["x"] if li == 0 else c5_stack["xl"][li - 1]
        xl0, nrm1, m_gpu, ss = c5_stack["singles"][li]
        _check_block(x_in, _c5_layer(c5_stack["base"], c5_stack["shifts"], li), xl0, nrm1, m_gpu, ss)


def test_c5_head_after_the_stack(c5_stack):
    """The 151936 x 4096 head on the stack's norm_out: argmax against the oracle's on the same
    rows (near-tie rule) and logits within the tolerance."""
    say("C5 head")
    q, s = synth.quantized_head(np.random.SeedSequence(20261207), C5_V, C5_H)
    nrm = c5_stack["nrm"]
    a_gpu, lg = gpu_verify(q, s, nrm)
    L = oracle.head_logits(q, s, nrm)
    check_argmax(a_gpu, L)
    check_logits(lg, L)
