"""The C-ABI library loads, exports every function include/specverify.h declares, and rejects
bad arguments on the host before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

from weight_bound_verify_amd import specverify as sv

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "specverify.h")

P = ctypes.c_void_p
NULL = None
A16 = P(0x10000)          # aligned fake addresses: never dereferenced on the host
A2 = P(0x10002)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(specverify_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return sv.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 10
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(sv.EXPORTS)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for macro, val in [("SV_MAX_S", sv.SV_MAX_S), ("SV_MAX_NGRAM", sv.SV_MAX_NGRAM), ("SV_BLOCK", sv.SV_BLOCK),
                       ("SV_STATE_WORDS", sv.STATE_WORDS), ("SV_STATE_LEN", sv.STATE_LEN),
                       ("SV_STATE_FLAGS", sv.STATE_FLAGS), ("SV_STATE_HIST", sv.STATE_HIST),
                       ("SV_STATE_GATE_AFTER", sv.STATE_GATE_AFTER), ("SV_STATE_ZERO_RUN", sv.STATE_ZERO_RUN),
                       ("SV_STATE_GATED", sv.STATE_GATED), ("SV_FLAG_TOKEN", sv.FLAG_TOKEN),
                       ("SV_FLAG_CAPACITY", sv.FLAG_CAPACITY), ("SV_FLAG_ARGMAX", sv.FLAG_ARGMAX)]:
        assert re.search(rf"#define {macro} {val}\b", text), macro


def test_status_strings(lib):
    assert lib.specverify_status_string(0) == b"ok"
    assert lib.specverify_status_string(4) == b"workspace too small"
    assert lib.specverify_status_string(99) == b"unknown status"


def test_verify_argument_errors(lib):
    ws = sv.load().specverify_verify_workspace_bytes(1000, 256, 9)
    assert ws > 0
    call = lib.specverify_verify
    assert call(NULL, A16, 1000, 256, A16, 9, A16, NULL, A16, ws, NULL) == 1
    assert call(A16, A16, 1000, 250, A16, 9, A16, NULL, A16, ws, NULL) == 2     # H % 32
    assert call(A16, A16, 0, 256, A16, 9, A16, NULL, A16, ws, NULL) == 2        # V
    assert call(A16, A16, 1000, 256, A16, 65, A16, NULL, A16, ws, NULL) == 2    # S > 64
    assert call(A16, A16, 1000, 256, A16, 0, A16, NULL, A16, ws, NULL) == 2     # S = 0
    assert call(A2, A16, 1000, 256, A16, 9, A16, NULL, A16, ws, NULL) == 3      # wq alignment
    assert call(A16, A16, 1000, 256, A2, 9, A16, NULL, A16, ws, NULL) == 3      # hidden alignment
    assert call(A16, A2, 1000, 256, A16, 9, A16, NULL, A16, ws, NULL) == 3      # scale alignment
    assert call(A16, A16, 1000, 256, A16, 9, A16, NULL, A16, ws - 1, NULL) == 4
    assert b"workspace" in lib.specverify_last_error()
    assert lib.specverify_verify_workspace_bytes(1000, 250, 9) == 0


def test_accept_and_propose_argument_errors(lib):
    assert lib.specverify_accept(NULL, A16, 8, A16, 100, A16, NULL) == 1
    assert lib.specverify_accept(A16, NULL, 8, A16, 100, A16, NULL) == 1        # drafts needed for K > 0
    assert lib.specverify_accept(A16, A16, 64, A16, 100, A16, NULL) == 2
    assert lib.specverify_accept(A16, A16, -1, A16, 100, A16, NULL) == 2
    assert lib.specverify_accept(A16, A16, 8, A16, 0, A16, NULL) == 5
    assert lib.specverify_accept(A2, A16, 8, A16, 100, A16, NULL) == 3
    assert lib.specverify_propose(A16, 100, A16, 0, 8, A16, NULL) == 2          # ngram order
    assert lib.specverify_propose(A16, 100, A16, 9, 8, A16, NULL) == 2
    assert lib.specverify_propose(A16, 100, A16, 3, 0, A16, NULL) == 2          # K
    assert lib.specverify_propose(NULL, 100, A16, 3, 8, A16, NULL) == 1


def test_stack_argument_errors(lib):
    assert lib.specverify_rmsnorm(A16, 9, 100, ctypes.c_float(1e-6), A16, NULL) == 2
    assert lib.specverify_rmsnorm(A16, 9, 256, ctypes.c_float(-1.0), A16, NULL) == 2
    assert lib.specverify_linear_q8b32(A16, A16, 64, 256, A16, 17, NULL, A16, NULL, 0, NULL) == 2  # S <= 16
    assert lib.specverify_gateup_silu_q8b32(A16, A16, NULL, A16, 64, 256, A16, 9, A16, NULL, 0, NULL) == 1
    need = lib.specverify_stack_workspace_bytes(64, 65536, 9, 1)
    assert need > 0                                     # very long inputs split the hidden axis
    assert lib.specverify_gateup_silu_q8b32(A16, A16, A16, A16, 64, 65536, A16, 9, A16, NULL, 0, NULL) == 4
    fused = lib.specverify_linear_residual_rmsnorm_q8b32
    fused.argtypes = [P, P, ctypes.c_int32, ctypes.c_int32, P, ctypes.c_int32, P, P, ctypes.c_float, P, P,
                      ctypes.c_size_t, P]
    A16b, A16c = P(0x20000), P(0x30000)
    assert fused(A16, A16, 64, 256, A16, 9, A16b, A16b, 1e-6, NULL, NULL, 0, NULL) == 1        # norm_out
    assert fused(A16, A16, 64, 256, A16, 9, A16b, A16b, 1e-6, A16b, NULL, 0, NULL) == 2        # aliases y
    assert fused(A16, A16, 64, 256, A16, 9, A16b, A16b, -1.0, A16c, NULL, 0, NULL) == 2        # eps
    assert fused(A16, A16, 64, 256, A16, 17, A16b, A16b, 1e-6, A16c, NULL, 0, NULL) == 2       # S <= 16
    need = lib.specverify_stack_workspace_bytes(64, 65536, 9, 0)
    assert need > 0
    assert fused(A16, A16, 64, 65536, A16, 9, A16b, A16b, 1e-6, A16c, NULL, 0, NULL) == 4


def test_whole_stack_argument_errors(lib):
    f = lib.specverify_stack
    ws = lib.specverify_stack_forward_workspace_bytes(4096, 12288, 9)
    assert ws == 2 * 9 * 12288 + 4 * 9 * 256          # m [S][F] fp16 + sum-of-squares partials [S][H/16]
    # a down projection split 8 ways (a tuning choice) adds fp32 slice sums [8][S][H] and one
    # counter per 16-row tile
    try:
        lib.specverify_set_tuning(0, 0, 0, 0, 8)
        assert lib.specverify_stack_forward_workspace_bytes(4096, 12288, 9) == ws + 4 * 8 * 9 * 4096 + 4 * 256
    finally:
        lib.specverify_set_tuning(0, 0, 0, 0, 0)
    assert lib.specverify_stack_forward_workspace_bytes(4096, 12288, 17) == 0
    assert lib.specverify_stack_forward_workspace_bytes(4000, 12288, 9) == 0
    B, C, D = P(0x20000), P(0x40000), P(0x60000)
    ok = [A16, A16, A16, A16, A16, A16, 2, 4096, 12288, B, 9, ctypes.c_float(1e-6), NULL, C, D, ws, NULL]
    def call(**kw):
        args = list(ok)
        for k, v in kw.items():
            args[int(k[1:])] = v
        return f(*args)
    assert call(a0=NULL) == 1                           # weights
    assert call(a13=NULL) == 1                          # norm_out
    assert call(a6=0) == 2                              # L
    assert call(a10=17) == 2                            # S
    assert call(a7=4000) == 2                           # H not a multiple of 512
    assert call(a11=ctypes.c_float(-1.0)) == 2          # eps
    assert call(a13=B) == 2                             # norm_out overlaps x
    assert call(a9=A2) == 3                             # x alignment
    assert call(a15=ws - 1) == 4                        # workspace
    assert b"workspace" in lib.specverify_last_error()


def test_every_documented_stack_shape_has_a_launch_configuration(lib):
    """H and F multiples of 512 with H*F < 2^31 are documented as supported: each must get a
    configuration (a non-zero workspace answer) for every S it allows."""
    sizes = [512, 1024, 1536, 2048, 2560, 3072, 3584, 4096, 5120, 6144, 8192, 12288, 14336, 65536]
    for H in sizes:
        for F in sizes:
            for S in (1, 9, 16):
                got = lib.specverify_stack_forward_workspace_bytes(H, F, S)
                assert (got > 0) == (H * F < 2 ** 31), (H, F, S)


def test_generate_and_gather_argument_errors(lib):
    ws = lib.specverify_verify_workspace_bytes(1000, 256, 9)
    g = lib.specverify_generate
    ok = [A16, A16, 1000, 256, A16, 8, 5, A16, 100, A16, 3, A16, A16, A16, A16, ws, NULL]
    def call(**kw):
        args = list(ok)
        for k, v in kw.items():
            args[int(k[1:])] = v
        return g(*args)
    assert call(a4=NULL) == 1                           # table
    assert call(a5=0) == 2                              # K
    assert call(a6=-1) == 2                             # rounds
    assert call(a10=0) == 2                             # n-gram order
    assert call(a4=A2) == 3                             # table alignment
    assert call(a15=ws - 1) == 4                        # workspace
    gw = lib.specverify_gather_window
    assert gw(A16, 100, A16, A16, 8, NULL, 1000, 256, A16, NULL) == 1
    assert gw(A16, 100, A16, NULL, 0, A16, 1000, 256, A16, NULL) != 1      # drafts optional at K = 0
    assert gw(A16, 100, A16, A16, 64, A16, 1000, 256, A16, NULL) == 2
    assert gw(A16, 100, A16, A16, 8, A16, 1000, 250, A16, NULL) == 2
    assert gw(A16, 100, A16, A16, 8, A16, 1000, 256, A2, NULL) == 3


def test_int4_head_argument_errors(lib):
    ws = lib.specverify_verify_workspace_bytes(1000, 2048, 9)
    f = lib.specverify_verify_q4b32
    assert f(NULL, A16, 1000, 2048, A16, 9, A16, NULL, A16, ws, NULL) == 1
    assert f(A16, A16, 1000, 2000, A16, 9, A16, NULL, A16, ws, NULL) == 2      # H not a multiple of 256
    assert f(A16, A16, 1000, 2048, A16, 17, A16, NULL, A16, ws, NULL) == 2     # S <= 16
    assert f(A2, A16, 1000, 2048, A16, 9, A16, NULL, A16, ws, NULL) == 3
    assert f(A16, A16, 1000, 2048, A16, 9, A16, NULL, A16, 100, NULL) == 4
    r = lib.specverify_round_q4b32
    assert r(A16, A16, 1000, 2048, A16, 16, A16, A16, 100, A16, 3, A16, A16, NULL, A16, ws, NULL) == 2  # K <= 15
    assert r(A16, A16, 1000, 2048, A16, 8, NULL, A16, 100, A16, 3, A16, A16, NULL, A16, ws, NULL) == 1


def test_sampling_argument_errors(lib):
    ws = lib.specverify_sample_workspace_bytes(1000, 256, 9)
    assert ws > lib.specverify_verify_workspace_bytes(1000, 256, 9)
    assert lib.specverify_sample_workspace_bytes(1000, 256, 17) == 0            # S <= 16
    v = lib.specverify_verify_sample
    assert v(A16, A16, 1000, 256, A16, 9, A16, 0.8, 1, NULL, A16, A16, A16, NULL, A16, ws, NULL) == 1   # state
    assert v(A16, A16, 1000, 256, A16, 9, NULL, 0.8, 1, A16, A16, A16, A16, NULL, A16, ws, NULL) == 1   # drafts
    assert v(A16, A16, 1000, 256, A16, 17, A16, 0.8, 1, A16, A16, A16, A16, NULL, A16, ws, NULL) == 2   # S
    for bad_t in (0.0, -1.0, float("inf"), float("nan"), 1e-45):
        assert v(A16, A16, 1000, 256, A16, 9, A16, bad_t, 1, A16, A16, A16, A16, NULL, A16, ws, NULL) == 2
    assert b"temperature" in lib.specverify_last_error()
    assert v(A16, A16, 1000, 256, A16, 9, A16, 0.8, 1, A16, A2, A16, A16, NULL, A16, ws, NULL) == 3     # sample
    assert v(A16, A16, 1000, 256, A16, 9, A16, 0.8, 1, A16, A16, A16, A16, NULL, A16, ws - 1, NULL) == 4
    a = lib.specverify_accept_sample
    assert a(A16, A16, A16, NULL, 8, 1000, 1, A16, 100, A16, NULL) == 1         # drafts with K > 0
    assert a(A16, A16, A16, A16, 16, 1000, 1, A16, 100, A16, NULL) == 2         # K <= 15
    assert a(A16, A16, A16, A16, 8, 0, 1, A16, 100, A16, NULL) == 2             # V
    assert a(A16, A16, A16, A16, 8, 1000, 1, A16, 0, A16, NULL) == 5            # cap
    r = lib.specverify_round_sample
    assert r(A16, A16, 1000, 256, A16, 16, A16, 0.8, 1, A16, 100, A16, 3, A16, NULL, NULL, A16, ws, NULL) == 2
    assert r(A16, A16, 1000, 256, A16, 8, NULL, 0.8, 1, A16, 100, A16, 3, A16, NULL, NULL, A16, ws, NULL) == 1
    assert r(A16, A16, 1000, 256, A16, 8, A16, 0.8, 1, A16, 100, A16, 9, A16, NULL, NULL, A16, ws, NULL) == 2
    assert r(A16, A16, 1000, 256, A16, 8, A16, 0.8, 1, A16, 100, A16, 3, A16, NULL, NULL, A16, ws - 1, NULL) == 4


def test_tree_argument_errors(lib):
    pt = lib.specverify_propose_tree
    assert pt(NULL, 100, A16, 3, 8, 2, 4, A16, A16, NULL) == 1
    assert pt(A16, 100, A16, 3, 16, 2, 4, A16, A16, NULL) == 2              # K <= 15
    assert pt(A16, 100, A16, 3, 8, 5, 4, A16, A16, NULL) == 2               # branches <= 4
    assert pt(A16, 100, A16, 3, 8, 2, 9, A16, A16, NULL) == 2               # depth <= K
    assert pt(A16, 100, A16, 3, 8, 2, 0, A16, A16, NULL) == 2               # depth >= 1
    assert pt(A16, 100, A16, 9, 8, 2, 4, A16, A16, NULL) == 2               # ngram_max
    assert pt(A16, 0, A16, 3, 8, 2, 4, A16, A16, NULL) == 5                 # cap
    assert pt(A16, 100, A16, 3, 8, 2, 4, A2, A16, NULL) == 3
    at = lib.specverify_accept_tree
    assert at(A16, NULL, A16, 8, A16, 100, A16, NULL) == 1
    assert at(A16, A16, A16, 0, A16, 100, A16, NULL) == 2
    assert at(A16, A16, A16, 16, A16, 100, A16, NULL) == 2
    rt = lib.specverify_round_tree
    ws = lib.specverify_verify_workspace_bytes(1000, 256, 9)
    assert rt(A16, A16, 1000, 256, A16, 8, NULL, A16, A16, 100, A16, 3, 2, 4, A16, A16, A16, NULL, A16, ws, NULL) == 1
    assert rt(A16, A16, 1000, 256, A16, 16, A16, A16, A16, 100, A16, 3, 2, 4, A16, A16, A16, NULL, A16, ws, NULL) == 2
    assert rt(A16, A16, 1000, 250, A16, 8, A16, A16, A16, 100, A16, 3, 2, 4, A16, A16, A16, NULL, A16, ws, NULL) == 2
    assert rt(A16, A16, 1000, 256, A16, 8, A16, A16, A16, 100, A16, 3, 2, 4, A16, A16, A16, NULL, A16, 8, NULL) == 4


def test_generation_loop_argument_errors(lib):
    """The sampling and tree generation loops check their arguments before touching the
    device: every case below returns its status without a GPU (a valid call fails only at the
    device query here)."""
    gs = lib.specverify_generate_sample
    ws = lib.specverify_sample_workspace_bytes(1000, 256, 9)
    ok = (A16, A16, 1000, 256, A16, 8, 3, 0.8, 1, A16, 100, A16, 3, A16, A16, A16, ws, NULL)

    def with_(args, i, v):
        a = list(args)
        a[i] = v
        return a
    assert gs(*ok) in (6, 7)                                              # no device
    assert gs(*with_(ok, 4, NULL)) == 1                                   # table
    assert gs(*with_(ok, 14, NULL)) == 1                                  # window
    assert gs(*with_(ok, 5, 16)) == 2                                     # K <= 15
    assert gs(*with_(ok, 6, -1)) == 2                                     # rounds >= 0
    assert gs(*with_(ok, 7, 0.0)) == 2                                    # temperature > 0
    assert gs(*with_(ok, 4, A2)) == 3                                     # table alignment
    assert gs(*with_(ok, 16, ws - 1)) == 4                                # workspace
    assert gs(*with_(ok, 10, 0)) == 5                                     # cap
    gt = lib.specverify_generate_tree
    wt = lib.specverify_verify_workspace_bytes(1000, 256, 9)
    ok = (A16, A16, 1000, 256, A16, 8, 3, A16, 100, A16, 3, 2, 4, A16, A16, A16, A16, A16, wt, NULL)
    assert gt(*ok) in (6, 7)
    assert gt(*with_(ok, 4, NULL)) == 1                                   # table
    assert gt(*with_(ok, 13, NULL)) == 1                                  # parents
    assert gt(*with_(ok, 5, 0)) == 2                                      # K >= 1
    assert gt(*with_(ok, 11, 5)) == 2                                     # branches <= 4
    assert gt(*with_(ok, 12, 9)) == 2                                     # depth <= K
    assert gt(*with_(ok, 6, -2)) == 2                                     # rounds >= 0
    assert gt(*with_(ok, 15, A2)) == 3                                    # window alignment
    assert gt(*with_(ok, 18, 8)) == 4                                     # workspace
    assert gt(*with_(ok, 8, 0)) == 5                                      # cap


def test_missing_library_raises(monkeypatch, tmp_path):
    monkeypatch.setattr(sv, "_lib", None)
    monkeypatch.setattr(sv, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="missing"):
        sv.load()


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: any other count exits with status 2 and says so, before
    touching torch or the library."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2 and "one GPU" in res.stderr and res.stdout == ""


def test_bench_workload_overrides():
    """--K, --ngram, --seed and --logits: the workload's K and name follow an override; the
    decode step and the 16-row window limit of the sampling, tree, int4 and stack paths refuse
    one; a nonzero seed moves every seeded stream while seed 0 keeps the workload's own;
    --logits is refused where no round call writes logits."""
    import importlib.util
    import types
    import numpy as np
    from weight_bound_verify_amd import synth
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    args = lambda config, K=None, ngram=3, seed=0, logits=False: types.SimpleNamespace(
        config=config, K=K, ngram=ngram, seed=seed, logits=logits)

    wl = bench.configure_workload(args("c3", K=16, ngram=2))
    assert wl["K"] == 16 and wl["ngram"] == 2 and "K=16 S=17" in wl["name"] and "K=8" not in wl["name"]
    assert bench.WORKLOADS["c3"]["K"] == 8                         # the table itself is untouched
    for cfg in ("c1", "c2", "c3", "c3q4", "c3tree", "c4s17", "c5"):
        bench.configure_workload(args(cfg, logits=True))           # these write logits when asked
    wl = bench.configure_workload(args("c3tree", K=12))
    assert "12 tree nodes (S=13)" in wl["name"]
    for bad in (args("c4s1", K=2), args("c3samp", K=16), args("c3tree", K=16), args("c3q4", K=16),
                args("c5", K=16), args("c3", K=64),
                args("c3", K=0), args("c3", ngram=0), args("c3", ngram=9), args("c3", seed=-1),
                args("c3samp", logits=True), args("c3gen", logits=True), args("c4s1", logits=True)):
        with pytest.raises(SystemExit):
            bench.configure_workload(bad)

    def first_words(wl):
        return words(bench._streams(wl, synth))

    def words(st):
        return [np.random.default_rng(getattr(st, f)).integers(0, 2 ** 32, 2).tolist()
                for f in ("weights", "h_last", "hidden", "context", "drafts")]
    same = first_words(bench.configure_workload(args("c3")))
    assert same == words(synth.streams(2))
    moved = first_words(bench.configure_workload(args("c3", seed=1)))
    assert all(a != b for a, b in zip(same, moved))
    other = first_words(bench.configure_workload(args("c2", seed=1)))       # config 1, seed 1
    assert all(a != b for a, b in zip(moved, other))


def test_round_noalloc_refuses_scratch_beyond_its_static_array(lib):
    """A split hidden axis over a large vocabulary needs more than the 2 MiB library-held
    scratch: refused on the host (SV_ERR_SHAPE) before any HIP call, with the sizes in the
    message; argument errors come first as for specverify_round."""
    call = lib.specverify_round_noalloc
    assert call(A16, A16, 30000, 16384, A16, 8, A16, A16, 100, A16, 3, A16, A16, NULL, NULL) == 2
    msg = lib.specverify_last_error().decode()
    assert "4614912" in msg and "2097152" in msg
    assert call(NULL, A16, 1000, 256, A16, 8, A16, A16, 100, A16, 3, A16, A16, NULL, NULL) == 1
    assert call(A16, A16, 1000, 256, A16, 0, A16, A16, 100, A16, 3, A16, A16, NULL, NULL) == 2      # K
    assert call(A16, A16, 1000, 256, A16, 8, A16, A16, 100, A16, 9, A16, A16, NULL, NULL) == 2      # ngram
    assert call(A16, A16, 1000, 256, A16, 8, A16, A16, 100, A16, 3, A16, A2, NULL, NULL) == 3       # argmax


def test_gather_positions_argument_errors(lib):
    call = lib.specverify_gather_positions
    assert call(NULL, 10, A16, 40, 256, 4, A16, NULL) == 1
    assert call(A16, 10, A16, 40, 250, 4, A16, NULL) == 2          # H % 32
    assert call(A16, 10, A16, 0, 256, 4, A16, NULL) == 2            # no rows
    assert call(A16, 10, A16, 40, 256, 64, A16, NULL) == 2          # K
    assert call(A16, 0, A16, 40, 256, 4, A16, NULL) == 5            # cap
    assert call(A16, 10, A2, 40, 256, 4, A16, NULL) == 3            # rows alignment
