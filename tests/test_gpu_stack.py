"""GPU parity of the dense stack entry points (rmsnorm, gate/up + SiLU*mul, down + residual)
against the CPU oracle, teacher-forced: each GPU op and its oracle twin consume the same fp16
input, and fp16 outputs may differ by one fp16 rounding step plus the fp32 accumulation error."""
import numpy as np
import pytest
import torch

import oracle
from weight_bound_verify_amd import specverify as sv
from weight_bound_verify_amd import synth

from gpu_util import check_argmax, dev, say, to_dev

pytestmark = pytest.mark.gpu


def _check_f16(got16, ref64, slack=1e-4):
    got = got16.astype(np.float64)
    ref16 = ref64.astype(np.float16)
    ulp = np.spacing(np.abs(ref16)).astype(np.float64)
    rms = np.sqrt(np.mean(ref64 * ref64, axis=-1, keepdims=True))
    err = np.abs(got - ref64)
    bound = ulp + slack * rms
    bad = np.argwhere(~(err <= bound))
    assert bad.size == 0, f"{len(bad)} outputs outside, first {bad[:3].tolist()} err {err[tuple(bad[0])]} bound {bound[tuple(bad[0])]}"
    return int(np.count_nonzero(got16 != ref16))


def _w(rng, r, c):
    return synth.quantize_q8b32(rng.standard_normal((r, c), dtype=np.float32) * np.float32(synth.W_STD))


def _gpu_gateup(g, u, x):
    N, K = g[0].shape
    m = torch.empty((x.shape[0], N), dtype=torch.float16, device=dev())
    nb = sv.stack_workspace_bytes(N, K, x.shape[0], True)
    sv.gateup_silu(to_dev(g[0]), to_dev(g[1]), to_dev(u[0]), to_dev(u[1]), to_dev(x), m,
                   sv.workspace(nb, dev()) if nb else None)
    torch.cuda.synchronize()
    return m.cpu().numpy()


def _gpu_linear(w, x, residual):
    N, K = w[0].shape
    y = torch.empty((x.shape[0], N), dtype=torch.float16, device=dev())
    nb = sv.stack_workspace_bytes(N, K, x.shape[0], False)
    sv.linear(to_dev(w[0]), to_dev(w[1]), to_dev(x), y, None if residual is None else to_dev(residual),
              sv.workspace(nb, dev()) if nb else None)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("S,H", [(9, 4096), (1, 32), (16, 5120), (3, 96), (2, 12288), (1, 65536)])
def test_rmsnorm(S, H):
    x = (synth.fp16_normal(np.random.default_rng(H), (S, H)).astype(np.float32) * 7).astype(np.float16)
    y = torch.empty((S, H), dtype=torch.float16, device=dev())
    sv.rmsnorm(to_dev(x), y, 1e-6)
    torch.cuda.synchronize()
    xx = x.astype(np.float64)
    ref = xx / np.sqrt(np.mean(xx * xx, axis=1, keepdims=True) + 1e-6)
    assert np.array_equal(oracle.rmsnorm_fp16(x), ref.astype(np.float16))
    _check_f16(y.cpu().numpy(), ref, slack=1e-5)


@pytest.mark.parametrize("N,K,S", [(12288, 4096, 9), (100, 64, 2), (1000, 256, 16)])
def test_gateup_silu(N, K, S):
    say(f"gate/up N={N} K={K} S={S}")
    rng = np.random.default_rng(N + K)
    g, u = _w(rng, N, K), _w(rng, N, K)
    x = oracle.rmsnorm_fp16(synth.fp16_normal(rng, (S, K)))
    m = _gpu_gateup(g, u, x)
    ref = oracle.silu(oracle.linear_q8b32(*g, x)) * oracle.linear_q8b32(*u, x)
    flips = _check_f16(m, ref)
    say(f"  outputs differing from the oracle's fp16 rounding: {flips} of {m.size}")


@pytest.mark.parametrize("N,K,S,res", [(4096, 12288, 9, True), (4096, 12288, 9, False), (77, 96, 5, True),
                                       (300, 65536, 2, True)])
def test_linear_residual(N, K, S, res):
    say(f"linear N={N} K={K} S={S} residual={res}")
    rng = np.random.default_rng(N + K + S)
    w = _w(rng, N, K)
    x = synth.fp16_normal(rng, (S, K))
    r = (synth.fp16_normal(rng, (S, N)).astype(np.float32) * 4).astype(np.float16) if res else None
    y = _gpu_linear(w, x, r)
    ref = oracle.linear_q8b32(*w, x)
    if res:
        ref = ref + r.astype(np.float64)
    _check_f16(y, ref)


def test_rmsnorm_in_place():
    x = (synth.fp16_normal(np.random.default_rng(8), (5, 9216)).astype(np.float32) * 3).astype(np.float16)
    buf = to_dev(x)
    sv.rmsnorm(buf, buf, 1e-6)
    torch.cuda.synchronize()
    xx = x.astype(np.float64)
    _check_f16(buf.cpu().numpy(), xx / np.sqrt(np.mean(xx * xx, axis=1, keepdims=True) + 1e-6), slack=1e-5)


@pytest.mark.parametrize("N,K,S,res", [(4096, 12288, 9, True), (4096, 12288, 16, True), (77, 96, 5, True),
                                       (300, 65536, 2, True), (5000, 1024, 3, True), (9000, 12288, 4, False),
                                       (1, 32, 1, True)])
def test_linear_residual_rmsnorm(N, K, S, res):
    """End of one block plus the next block's input norm, in one call."""
    say(f"linear+residual+rmsnorm N={N} K={K} S={S} residual={res}")
    rng = np.random.default_rng(N * 7 + K + S)
    w = _w(rng, N, K)
    x = synth.fp16_normal(rng, (S, K))
    r = (synth.fp16_normal(rng, (S, N)).astype(np.float32) * 4).astype(np.float16) if res else None
    y = torch.empty((S, N), dtype=torch.float16, device=dev())
    n = torch.empty((S, N), dtype=torch.float16, device=dev())
    nb = sv.stack_workspace_bytes(N, K, S, False)
    sv.linear_residual_rmsnorm(to_dev(w[0]), to_dev(w[1]), to_dev(x), y, n, None if r is None else to_dev(r),
                               1e-6, sv.workspace(nb, dev()) if nb else None)
    torch.cuda.synchronize()
    ref = oracle.linear_q8b32(*w, x)
    if res:
        ref = ref + r.astype(np.float64)
    y16 = y.cpu().numpy()
    _check_f16(y16, ref)
    # the norm of the library's own fp16 y (teacher-forced)
    yy = y16.astype(np.float64)
    _check_f16(n.cpu().numpy(), yy / np.sqrt(np.mean(yy * yy, axis=1, keepdims=True) + 1e-6), slack=1e-5)


def test_linear_output_may_alias_residual():
    rng = np.random.default_rng(3)
    w = _w(rng, 512, 256)
    x = synth.fp16_normal(rng, (9, 256))
    r = synth.fp16_normal(rng, (9, 512))
    buf = to_dev(r)
    sv.linear(to_dev(w[0]), to_dev(w[1]), to_dev(x), buf, buf)
    torch.cuda.synchronize()
    _check_f16(buf.cpu().numpy(), oracle.linear_q8b32(*w, x) + r.astype(np.float64))


def test_small_stack_end_to_end_teacher_forced():
    rng = np.random.default_rng(11)
    L_, H, F, V, S = 6, 512, 1536, 5000, 9
    layers = [(_w(rng, F, H), _w(rng, F, H), _w(rng, H, F)) for _ in range(L_)]
    hq, hs = _w(rng, V, H)
    x = synth.fp16_normal(rng, (S, H))
    xd = to_dev(x)
    n = torch.empty_like(xd)
    m = torch.empty((S, F), dtype=torch.float16, device=dev())
    gw = sv.workspace(sv.stack_workspace_bytes(F, H, S, True), dev())
    dw = sv.workspace(sv.stack_workspace_bytes(H, F, S, False), dev())
    sv.rmsnorm(xd, n)
    for li, (g, u, d) in enumerate(layers):
        x_in = xd.cpu().numpy()
        n_in = n.cpu().numpy()
        xx = x_in.astype(np.float64)
        _check_f16(n_in, xx / np.sqrt(np.mean(xx * xx, axis=1, keepdims=True) + 1e-6), slack=1e-5)
        sv.gateup_silu(to_dev(g[0]), to_dev(g[1]), to_dev(u[0]), to_dev(u[1]), n, m, gw)
        if li % 2:
            sv.linear(to_dev(d[0]), to_dev(d[1]), m, xd, xd, dw)
            sv.rmsnorm(xd, n)
        else:       # the fused end-of-block call; y aliases the residual stream
            sv.linear_residual_rmsnorm(to_dev(d[0]), to_dev(d[1]), m, xd, n, xd, 1e-6, dw)
        torch.cuda.synchronize()
        # oracle block on the GPU's own layer input
        ref_x, parts = oracle.mlp_block(x_in, (g, u, d), return_parts=True)
        ref_full = x_in.astype(np.float64) + oracle.linear_q8b32(*d, m.cpu().numpy())
        _check_f16(xd.cpu().numpy(), ref_full)
    am = torch.empty(S, dtype=torch.int32, device=dev())
    lg = torch.empty((S, V), dtype=torch.float32, device=dev())
    sv.verify(to_dev(hq), to_dev(hs), n, am, sv.workspace(sv.verify_workspace_bytes(V, H, S), dev()), lg)
    torch.cuda.synchronize()
    L = oracle.head_logits(hq, hs, n.cpu().numpy())
    check_argmax(am.cpu().numpy(), L)
