"""Build libmla.so (the gfx950 kernels and their C ABI) and its checked twin in place with hipcc.

    python -m paged_mla_latent_amd.build            # both libraries
    python -m paged_mla_latent_amd.build --release  # libmla.so only

Object files go to paged_mla_latent_amd/_build/ (_build_checked/), the libraries to
paged_mla_latent_amd/libmla.so and libmla_checked.so; the measurement helper of bench.py (a
streaming-read reference kernel, include/mla_bench.h) to libmla_bench.so.  The checked build compiles the same
sources with -DMLA_CHECKED: its kernels test the decode preconditions (block ids inside the
pool, lengths inside the block table) before forming any address.  Every call recompiles.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libmla.so")
CHECKED_LIB_PATH = os.path.join(HERE, "libmla_checked.so")
SOURCES = ["mla_api.hip", "decode.hip", "decode_wide.hip", "merge.hip", "cache_write.hip", "gather.hip"]
BENCH_LIB_PATH = os.path.join(HERE, "libmla_bench.so")
BENCH_SOURCE = "bench_read.hip"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden",
    # Keep the compiler from forming packed fp32 arithmetic (v_pk_*_f32).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def _run(cmd: list[str]) -> str:
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in proc.stdout.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"command failed ({proc.returncode}): {' '.join(cmd)}\n{out}")
    return out


def _jobs(checked: bool):
    build_dir = os.path.join(HERE, "_build_checked" if checked else "_build")
    os.makedirs(build_dir, exist_ok=True)
    objs = [os.path.join(build_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    extra = ["-DMLA_CHECKED=1"] if checked else []
    cmds = [[HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(SOURCES, objs)]
    return objs, cmds


def _link(objs: list[str], path: str) -> None:
    tmp = path + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, path)


def build(verbose: bool = False, checked: bool = True) -> str:
    """Compile every source for gfx950 and link libmla.so (and, with checked=True, also
    libmla_checked.so); returns the release library's path."""
    variants = [False, True] if checked else [False]
    plans = {v: _jobs(v) for v in variants}
    cmds = [c for v in variants for c in plans[v][1]]
    bench_obj = os.path.join(HERE, "_build", os.path.splitext(BENCH_SOURCE)[0] + ".o")
    cmds.append([HIPCC, *COMMON, "-c", os.path.join(CSRC, BENCH_SOURCE), "-o", bench_obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(cmds))) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    for v in variants:
        _link(plans[v][0], CHECKED_LIB_PATH if v else LIB_PATH)
    _link([bench_obj], BENCH_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, checked="--release" not in sys.argv))
