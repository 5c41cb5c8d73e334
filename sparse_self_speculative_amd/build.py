"""Build libsspec.so (gfx950) in-tree with hipcc.

python -m sparse_self_speculative_amd.build

The kernel instances of the eight GQA group sizes live in eight translation
units (csrc/kernels.hip with -DSSPEC_G=1..8) compiled in parallel with the
host code (csrc/sspec.hip), the KV-cache maintenance kernels
(csrc/kvcache.hip), the KV offload engine (csrc/offload.hip) and the batch
scheduler (csrc/sched.hip); the objects are linked into one shared library.
Extra hipcc flags (development only, e.g. -DSSPEC_ONLY_G=4 or -DSSPEC_TRACE=1)
can be passed in the SSPEC_EXTRA_FLAGS environment variable, and
SSPEC_BUILD_OUT names another output library (the binding loads it when
SSPEC_LIB points at it).
"""

from __future__ import annotations

import os
import shlex
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libsspec.so")
BUILD_DIR = os.path.join(HERE, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # keep hipcc from forming packed fp32 instructions on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]


def _filtered(res) -> list[str]:
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    return [ln for ln in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in ln]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    extra = shlex.split(os.environ.get("SSPEC_EXTRA_FLAGS", ""))
    out = os.path.abspath(os.environ.get("SSPEC_BUILD_OUT", OUT))
    # one object directory per output library, so builds of different
    # libraries (other flags) never mix their objects
    build_dir = BUILD_DIR if out == OUT else os.path.join(BUILD_DIR, out.strip("/").replace("/", "_") + ".d")
    os.makedirs(build_dir, exist_ok=True)
    jobs = [([*HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, "sspec.hip")], os.path.join(build_dir, "host.o")),
            ([*HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, "kvcache.hip")], os.path.join(build_dir, "kvcache.o")),
            ([*HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, "offload.hip")], os.path.join(build_dir, "offload.o")),
            ([*HIPCC_FLAGS, *extra, "-c", os.path.join(CSRC, "sched.hip")], os.path.join(build_dir, "sched.o"))]
    for g in range(1, 9):
        jobs.append(([*HIPCC_FLAGS, *extra, f"-DSSPEC_G={g}", "-c", os.path.join(CSRC, "kernels.hip")],
                     os.path.join(build_dir, f"kernels_g{g}.o")))

    def compile_one(job):
        args, obj = job
        cmd = [hipcc, *args, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        return cmd, subprocess.run(cmd, capture_output=True, text=True)

    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(compile_one, jobs))
    failed = False
    for cmd, res in results:
        msgs = _filtered(res)
        if res.returncode != 0:
            failed = True
            sys.stderr.write(" ".join(cmd) + "\n" + "\n".join(msgs) + "\n")
        elif verbose and msgs:
            print("\n".join(msgs))
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = out + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *[obj for _, obj in jobs]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + "\n".join(_filtered(res)) + "\n")
        raise RuntimeError(f"link failed with exit code {res.returncode}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
