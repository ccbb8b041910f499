"""Shared helpers of the GPU parity tests (comparison rules against the CPU oracle)."""
import numpy as np
import torch

import oracle
from weight_bound_verify_amd import specverify as sv
from weight_bound_verify_amd import synth

TOL = 1e-3     # logits: |gpu - ref| <= TOL * max(|ref|, rms(ref row)); argmax exempt below a TOL gap


def dev():
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev())


def head(seed, V, H):
    q, s = synth.quantized_head(np.random.SeedSequence(seed), V, H)
    return q, s


def gpu_verify(q, s, hidden, want_logits=True, wq=None, ws=None):
    V, H = q.shape
    S = hidden.shape[0]
    wq = to_dev(q) if wq is None else wq
    ws = to_dev(s) if ws is None else ws
    hd = to_dev(hidden)
    am = torch.full((S,), -7, dtype=torch.int32, device=dev())
    lg = torch.full((S, V), float("nan"), dtype=torch.float32, device=dev()) if want_logits else None
    work = sv.workspace(sv.verify_workspace_bytes(V, H, S), dev())
    sv.verify(wq, ws, hd, am, work, lg)
    torch.cuda.synchronize()
    return am.cpu().numpy(), (lg.cpu().numpy().astype(np.float64) if want_logits else None)


def check_logits(lg, L, tol=TOL):
    floor = np.sqrt(np.mean(L * L, axis=1, keepdims=True))
    err = np.abs(lg - L)
    bound = tol * np.maximum(np.abs(L), floor)
    bad = np.argwhere(~(err <= bound))
    assert bad.size == 0, f"{len(bad)} logits outside tolerance, first {bad[:3].tolist()} err {err[tuple(bad[0])]}"
    return float((err / np.maximum(np.abs(L), floor)).max())


def check_argmax(a_gpu, L, tol=TOL):
    a_ref = oracle.argmax_lowest(L)
    gap = oracle.top2_gap(L)
    adm = oracle.admissible_sets(L, tol)
    exempt = 0
    for r in range(L.shape[0]):
        if a_gpu[r] == a_ref[r]:
            continue
        assert gap[r] < tol and a_gpu[r] in adm[r], f"row {r}: gpu {a_gpu[r]} oracle {a_ref[r]} gap {gap[r]}"
        exempt += 1
    return exempt
