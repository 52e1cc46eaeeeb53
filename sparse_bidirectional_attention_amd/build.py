"""Build libsdattn.so (gfx950) in-tree with hipcc.

    python -m sparse_bidirectional_attention_amd.build

compiles every .hip source of csrc/ for gfx950 and the plain C++ host sources,
and links them into sparse_bidirectional_attention_amd/libsdattn.so.  It also
builds libsdattn_fake.so (tests/host): the schedule driver and the argument
checks linked against a recording fake backend, for CPU-only tests, and
libsdattn_probe.so (csrc/probe): an MFMA-only throughput probe the bench
uses to measure the power-limited MFMA ceiling.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsdattn.so")
FAKE_SRC = os.path.join(ROOT, "tests", "host", "fake_backend.cpp")
FAKE_LIB = os.path.join(ROOT, "tests", "host", "libsdattn_fake.so")
PROBE_SRC = os.path.join(CSRC, "probe", "mfma_ceiling.hip")
PROBE_LIB = os.path.join(PKG, "libsdattn_probe.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 VALU ops stay disabled for every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in arch VGPRs: the softmax rescales O with VALU ops,
    # which cannot address AGPRs (the default form copies O every tile)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument", "-fvisibility=hidden",
]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wextra", "-Wno-unused-parameter"]

HIP_SOURCES = ["api.hip", "block_plan.hip", "flash_bf16.hip", "flash_f32.hip", "losa.hip", "mask_overlap.hip", "noalloc.hip",
               "select_blocks.hip", "select_columns.hip", "select_exact.hip"]
CXX_SOURCES = ["host_common.cpp", "schedule.cpp"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs_list = []
    objs = []
    for s in HIP_SOURCES:
        o = os.path.join(BUILD, s.replace(".hip", ".o"))
        objs.append(o)
        jobs_list.append([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
    for s in CXX_SOURCES:
        o = os.path.join(BUILD, s.replace(".cpp", ".o"))
        objs.append(o)
        jobs_list.append(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, s), "-o", o])
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs_list))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    build_fake(verbose)
    build_probe(verbose)
    return LIB


def build_fake(verbose: bool = False) -> str:
    """CPU-only library: argument checks + schedule driver + fake backend."""
    srcs = [os.path.join(CSRC, s) for s in CXX_SOURCES] + [FAKE_SRC]
    tmp = FAKE_LIB + ".tmp"
    _run(["g++", *CXX_FLAGS, "-shared", "-I", CSRC, "-o", tmp, *srcs], verbose)
    os.replace(tmp, FAKE_LIB)
    return FAKE_LIB


def build_probe(verbose: bool = False) -> str:
    """The MFMA-only throughput probe (measurement aid, its own library),
    built with the compiler's default accumulator registers (not forced into
    arch VGPRs: the probe has no VALU work that reads them)."""
    tmp = PROBE_LIB + ".tmp"
    flags = [f for f in HIP_FLAGS if f not in ("-mllvm", "-amdgpu-mfma-vgpr-form")]
    _run([HIPCC, *flags, "-shared", "-o", tmp, PROBE_SRC], verbose)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
