"""Build libkvq.so (and the libkvq_probe.so measurement aid) in-tree for gfx950 with hipcc.

Run ``python -m rotated_int2_kv_centering_amd.build`` (or call ``build()``).
The libraries are written next to this file; every call recompiles.
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
LIB = os.path.join(HERE, "libkvq.so")
SOURCES = ["kvq_api.cpp", "kvq_append.hip", "kvq_decode.hip", "kvq_decode_g8.hip", "kvq_decode_g16.hip",
           "kvq_eval.hip", "kvq_noalloc.hip"]
# measurement aid (HBM read-rate probe), a library of its own outside the decode path
PROBE_LIB = os.path.join(HERE, "libkvq_probe.so")
PROBE_SOURCES = ["hbm_probe.hip"]
ARCH = "gfx950"

# hipcc flags: no fast-math (the quantizer needs IEEE fp32 division and
# round-to-nearest-even); packed fp32 instructions disabled in device code;
# MFMA accumulators in VGPRs (the online-softmax rescale works on them with
# VALU ops, which cannot read AGPRs).
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libkvq)")


def _run(cmd, verbose: bool):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature; that warning is harmless
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l]
    if proc.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def _link(sources, lib: str, verbose: bool) -> str:
    """Compile every source to an object (in parallel), then link the shared library."""
    obj_dir = os.path.join(HERE, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    objs = [os.path.join(obj_dir, os.path.splitext(s)[0] + ".o") for s in sources]
    jobs = [[hipcc(), *HIP_FLAGS, *inc, "-c", os.path.join(CSRC, s), "-o", o] for s, o in zip(sources, objs)]
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1, 8)) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    out_tmp = lib + ".tmp"
    _run([hipcc(), *HIP_FLAGS, "-shared", *objs, "-o", out_tmp], verbose)
    os.replace(out_tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile every source, link libkvq.so and libkvq_probe.so; returns libkvq.so's path."""
    _link(PROBE_SOURCES, PROBE_LIB, verbose)
    return _link(SOURCES, LIB, verbose)


# A host-sanitized variant for the CPU checks of the C ABI: the host-only source
# (argument validation, sizes, workspace layout) is compiled with g++ under
# AddressSanitizer and UndefinedBehaviorSanitizer and linked with the device
# objects of the last build(); load it with gcc's libasan preloaded.  It is a
# test artefact, never loaded by the package.
HOST_SOURCES = ["kvq_api.cpp"]
SANITIZED_LIB = os.path.join(HERE, "_build", "libkvq_hostsan.so")
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-fno-sanitize-recover=undefined"]


def build_host_sanitized(verbose: bool = False) -> str:
    """Link _build/libkvq_hostsan.so: sanitized host objects plus build()'s device objects."""
    obj_dir = os.path.join(HERE, "_build")
    dev_objs = [os.path.join(obj_dir, os.path.splitext(s)[0] + ".o") for s in SOURCES if s not in HOST_SOURCES]
    if not all(os.path.exists(o) for o in dev_objs):
        build(verbose)
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    host_objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(obj_dir, os.path.splitext(src)[0] + ".hostsan.o")
        _run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", *SAN_FLAGS, "-D__HIP_PLATFORM_AMD__", "-I",
              os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
              os.path.join(CSRC, src), "-o", obj], verbose)
        host_objs.append(obj)
    _run(["g++", "-shared", *SAN_FLAGS, *host_objs, *dev_objs, "-L", os.path.join(rocm, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", SANITIZED_LIB], verbose)
    return SANITIZED_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
