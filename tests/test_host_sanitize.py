"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

1. The round tails' LDS scans (scan_best_lds, scan_top_lds) run on the host, thread by
   simulated thread, over streams held in arrays of exactly the readable length the kernels
   guarantee: AddressSanitizer stops any read outside it (the regression test for the read
   below the LDS array that faulted the tree drafter's scan), and the results must equal the
   oracle's ranking of end positions (oracle.tree._ranked_matches), also on streams whose ids
   are negative or INT_MIN (ids are never range-checked).  The global-memory drafter's chunk
   and halo arithmetic (chunk_window, chunk_key) runs the same way at chunk sizes 1 .. 8192,
   each chunk staged into an array of exactly kHalo + chunk ids.
2. The library's host code (argument validation, launch-shape selection, workspace sizing)
   built with both sanitizers runs the C-ABI tests of test_abi_cpu.py.

Device code is built as usual; each -fsanitize flag applies to the host pass only."""
import os
import subprocess
import sys

import numpy as np
import pytest

from oracle.tree import _ranked_matches

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
INT_MIN = -(1 << 31)


def _asan_runtime():
    out = subprocess.run([os.path.join(os.path.dirname(HIPCC), "amdclang++"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True).stdout.strip()
    if not out or not os.path.exists(out):
        pytest.skip("no AddressSanitizer runtime in this toolchain")
    return out


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


@pytest.fixture(scope="module")
def scan_harness(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    exe = str(tmp_path_factory.mktemp("scan") / "scan_check")
    src = os.path.join(ROOT, "tests", "host_scan_check.cpp")
    res = subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17", *HOST_SAN, src, "-o", exe],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    return exe


def _streams(rng):
    cases = []
    for n in list(range(0, 21)) + [31, 32, 33, 34, 35, 63, 64, 65, 66, 67, 255, 256, 257, 1000, 4097, 32768]:
        for vocab in (3, 50):
            ids = rng.integers(0, vocab, size=n).astype(np.int64)
            if n > 4 and rng.random() < 0.5:                     # ids the library never range-checks
                ids[rng.integers(0, n, size=max(1, n // 5))] = rng.choice([-1, INT_MIN, 2**31 - 1])
            cases.append(ids)
    # suffixes made only of INT_MIN and -1: the value a pre-stream position once held
    cases += [np.array([INT_MIN] * k, np.int64) for k in range(1, 10)]
    cases += [np.array([-1] * k, np.int64) for k in range(1, 10)]
    cases.append(np.array([INT_MIN, 5, INT_MIN, INT_MIN], np.int64))
    return cases


def test_lds_scans_stay_in_bounds_and_match_the_oracle(scan_harness):
    rng = np.random.default_rng(11)
    lines, expect = [], []
    streams = _streams(rng)
    runs = [(ids, nmax, nt) for ids in streams for nmax in (1, 3, 4, 5, 8) for nt in (1, 7, 64, 1024)
            if len(ids) < 5000 or (nmax in (3, 8) and nt == 1024)]
    lines.append(str(len(runs)))
    for ids, nmax, nt in runs:
        lines.append(f"{len(ids)} {nmax} {nt}")
        lines.append(" ".join(str(int(x)) for x in ids))
        ranked = _ranked_matches(ids.tolist(), nmax)
        best = ranked[0] if ranked else (0, 0)
        top = (ranked + [(0, 0)] * 4)[:4]
        expect.append((best, top))
    res = subprocess.run([scan_harness], input="\n".join(lines) + "\n", capture_output=True, text=True,
                         env=_env(), timeout=600)
    assert res.returncode == 0, res.stderr[-4000:]
    out = res.stdout.strip().splitlines()
    assert len(out) == len(runs)
    for (ids, nmax, nt), line, (best, top) in zip(runs, out, expect):
        v = [int(x) for x in line.split()]
        got_best, got_top = (v[0], v[1]), [(v[2 + 2 * i], v[3 + 2 * i]) for i in range(4)]
        assert got_best == tuple(best), (len(ids), nmax, nt, got_best, best)
        assert got_top == [tuple(t) for t in top], (len(ids), nmax, nt, got_top, top)
        # the global-memory drafter's chunked scan at chunk sizes 1, 2, 3, 5, 8, 17, 64, 8192
        chunked = [(v[10 + 2 * i], v[11 + 2 * i]) for i in range(8)]
        assert all(c == tuple(best) for c in chunked), (len(ids), nmax, nt, chunked, best)


@pytest.fixture(scope="module")
def asan_lib(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not found")
    sys.path.insert(0, ROOT)
    from weight_bound_verify_amd import build
    out = str(tmp_path_factory.mktemp("asan") / "libspecverify_asan.so")
    build.build(extra=HOST_SAN, out=out)
    return out


def test_abi_checks_under_sanitizers(asan_lib):
    """test_abi_cpu.py against the instrumented library, in a child process with the sanitizer
    runtime preloaded; a sanitizer report aborts the child."""
    code = ("import sys, pytest\n"
            "from weight_bound_verify_amd import specverify as sv\n"
            f"sv.LIB_PATH = {asan_lib!r}\n"
            "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', 'tests/test_abi_cpu.py']))\n")
    env = _env()
    env["LD_PRELOAD"] = _asan_runtime()
    env["PYTHONPATH"] = ROOT + os.pathsep + os.path.join(ROOT, "tests")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, env=env,
                         timeout=900)
    assert res.returncode == 0, (res.stdout[-3000:], res.stderr[-3000:])
    assert " passed" in res.stdout
