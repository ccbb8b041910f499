"""Build libspecverify.so in-tree for gfx950 (``python -m weight_bound_verify_amd.build``).

Each ``csrc/*.hip`` file is compiled to an object of its own, in parallel, then the objects
are linked into one shared library.  ``build(extra=..., out=...)`` builds a variant with extra
hipcc flags into another file (the CPU tests build an instrumented copy of the host code this
way); the product library is always ``libspecverify.so``.
"""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libspecverify.so")
OBJ_DIR = os.path.join(HERE, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-fp32 instructions are disabled for all device code (the compiler otherwise forms
# v_pk_* fp32 ops from scalar float code); hipcc's host pass warns about the unknown
# feature, which is harmless.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def _noise(res) -> list[str]:
    return [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln and ln.strip()]


def _compile(src: str, obj: str, extra: list[str]) -> tuple[int, list[str]]:
    res = subprocess.run([HIPCC, *FLAGS, *extra, "-c", src, "-o", obj], capture_output=True, text=True)
    return res.returncode, _noise(res)


def build(verbose: bool = False, extra: list[str] | None = None, out: str | None = None,
          jobs: int | None = None) -> str:
    out = out or LIB
    extra = list(extra or [])
    tag = "rel" if not extra else "x" + hashlib.sha1(" ".join(extra).encode()).hexdigest()[:8]
    os.makedirs(OBJ_DIR, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJ_DIR, f"{os.path.splitext(os.path.basename(s))[0]}.{tag}.o") for s in srcs]
    jobs = jobs or max(1, min(len(srcs), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda so: _compile(so[0], so[1], extra), zip(srcs, objs)))
    msgs = [m for _, ms in results for m in ms]
    if any(rc != 0 for rc, _ in results):
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    tmp = out + ".tmp"
    res = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *extra, *objs, "-o", tmp],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + "\n".join(_noise(res)))
    msgs += _noise(res)
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
