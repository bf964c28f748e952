"""Build libkvq.so (the HIP library behind include/kvq.h) in-tree for gfx950, and libkvq_probe.so (the
streaming-read probe the benchmark measures the HBM read ceiling with; not part of the cache's ABI).

Each translation unit is compiled by hipcc in parallel, then linked into a shared library that sits
next to this file. Flags:
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed fp32 instructions are generated.
* ``-fhip-fp32-correctly-rounded-divide-sqrt`` and, for the append kernels, ``-ffp-contract=off``: the
  quantizer's fp32 division and rounding are plain IEEE operations, bit-identical to a CPU evaluation.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
PROBE_LIB = os.path.join(HERE, "libkvq_probe.so")
BUILD = os.path.join(HERE, "_build")

COMMON = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fhip-fp32-correctly-rounded-divide-sqrt", "-Wno-unused-command-line-argument"]

UNITS = [
    ("kvq_host.cpp", ["-ffp-contract=off"]),
    ("kvq_append.hip", ["-ffp-contract=off"]),
    ("kvq_decode.hip", ["-ffp-contract=fast"]),
    ("kvq_gather.hip", ["-ffp-contract=fast"]),
    ("kvq_scratch.hip", ["-ffp-contract=off"]),
    ("kvq_index.hip", ["-ffp-contract=off"]),
    ("kvq_mq.hip", ["-ffp-contract=fast"]),
    ("kvq_mq_var.hip", ["-ffp-contract=fast"]),
    ("kvq_mq_pair.hip", ["-ffp-contract=fast"]),
    ("kvq_mq_pair_kv.hip", ["-ffp-contract=fast"]),
]
PROBE_UNITS = [("kvq_probe.hip", [])]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the kvq HIP library cannot be built")


def _up_to_date(src: str, obj: str) -> bool:
    if not os.path.exists(obj):
        return False
    t = os.path.getmtime(obj)
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".h")]
    deps.append(os.path.join(os.path.dirname(HERE), "include", "kvq.h"))
    return all(os.path.getmtime(d) <= t for d in deps)


def _compile(src: str, extra, incremental: bool = False) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    if incremental and _up_to_date(src, obj):
        return obj
    cmd = [_hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = True, incremental: bool = False) -> str:
    """Compile every unit (incremental=True: only units older than their source or a header) and link."""
    os.makedirs(BUILD, exist_ok=True)
    units = UNITS + PROBE_UNITS
    with cf.ThreadPoolExecutor(max_workers=len(units)) as ex:
        objs = list(ex.map(lambda u: _compile(*u, incremental=incremental), units))
    _link(objs[:len(UNITS)], LIB)
    _link(objs[len(UNITS):], PROBE_LIB)
    if verbose:
        print(f"[kvq] built {LIB} and {PROBE_LIB}", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(incremental="--incremental" in sys.argv)
