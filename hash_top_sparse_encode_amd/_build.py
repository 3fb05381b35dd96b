"""Build libhata.so in-tree with hipcc for gfx950 (MI355X / CDNA4)."""
from __future__ import annotations

import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libhata.so")
# The same library with the decode step's phase timestamps compiled in
# (HATA_PHASE_TRACE; hata_phase_trace), for the per-phase breakdown of a step.
TRACE_LIB_PATH = os.path.join(PKG, "libhata_trace.so")

SOURCES = ["api.cpp", "encode_exact.hip", "encode_rows.hip", "decode.hip", "decode_r32.hip",
           "decode_r64.hip", "decode_r128.hip", "decode_r256.hip", "recall.hip", "bits.hip",
           "train.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 ops stay disabled (the compiler emits them from plain float
# code otherwise).
COMMON_FLAGS = [
    "-x", "hip", "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _compile(src: str, trace: bool = False) -> str:
    name = src.rsplit(".", 1)[0] + (".trace.o" if trace else ".o")
    obj = os.path.join(BUILD_DIR, name)
    flags = [*COMMON_FLAGS, "-DHATA_PHASE_TRACE"] if trace else COMMON_FLAGS
    cmd = [HIPCC, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, path: str) -> None:
    tmp = path + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, path)


def build() -> str:
    """Compile every HIP source and link libhata.so and libhata_trace.so
    (always recompiles)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    traced = [s for s in SOURCES if s.startswith("decode")]
    jobs = [(s, False) for s in SOURCES] + [(s, True) for s in traced]
    with ThreadPoolExecutor(8) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    plain = objs[:len(SOURCES)]
    trace_of = dict(zip(traced, objs[len(SOURCES):]))
    _link(plain, LIB_PATH)
    _link([trace_of.get(s, o) for s, o in zip(SOURCES, plain)], TRACE_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
