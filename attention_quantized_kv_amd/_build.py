"""Compile libkvq.so (HIP for gfx950) in-tree with hipcc: every source to an
object in parallel, then one link."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
OBJ = os.path.join(HERE, "_build")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function",
    # packed fp32 VALU ops stay off: hipcc emits them from plain float code otherwise
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
]
_NOISE = "is not a recognized feature for this target"


def sources() -> list[str]:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd: list[str]) -> tuple[int, str]:
    res = subprocess.run(cmd, capture_output=True, text=True)
    return res.returncode, "\n".join(l for l in (res.stdout + res.stderr).splitlines() if _NOISE not in l)


def build(verbose: bool = False, extra: list[str] | None = None, jobs: int | None = None) -> str:
    """Compile every HIP source into attention_quantized_kv_amd/libkvq.so."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sources()
    objs = [os.path.join(OBJ, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[HIPCC, *FLAGS, *(extra or []), "-c", "-o", o, s] for s, o in zip(srcs, objs)]
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_run, cmds))
    for cmd, (rc, msgs) in zip(cmds, results):
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            raise RuntimeError(f"hipcc failed ({rc}) on {cmd[-1]}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs)
    tmp = LIB + ".tmp"
    rc, msgs = _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    if rc != 0:
        raise RuntimeError(f"link failed ({rc}):\n{msgs}")
    os.replace(tmp, LIB)
    build_probe(extra)
    return LIB


PROBE_SRC = os.path.join(HERE, "probe", "read_probe.hip")
PROBE_LIB = os.path.join(HERE, "libkvq_probe.so")


def build_probe(extra: list[str] | None = None) -> str:
    """The plain HBM read kernel bench.py compares the decode kernels with
    (measurement only; not part of libkvq)."""
    tmp = PROBE_LIB + ".tmp"
    rc, msgs = _run([HIPCC, *FLAGS, *(extra or []), "-shared", "-o", tmp, PROBE_SRC])
    if rc != 0:
        raise RuntimeError(f"hipcc failed ({rc}) on {PROBE_SRC}:\n{msgs}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose=False))
