"""Build the gfx950 shared libraries in-tree with hipcc.

    python -m mla_latent_kv_02_amd.build

produces mla_latent_kv_02_amd/libmla.so (the MLA decode library behind
include/mla.h), workloads/libmla_synth.so (the device side of the seeded
input generator) and workloads/libmla_probe.so (the bench's HBM streaming
probes).  Every call recompiles.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmla.so")
SYNTH_SRC = os.path.join(ROOT, "workloads", "synth_fill.hip")
SYNTH_LIB = os.path.join(ROOT, "workloads", "libmla_synth.so")
PROBE_SRC = os.path.join(ROOT, "workloads", "stream_probe.hip")
PROBE_LIB = os.path.join(ROOT, "workloads", "libmla_probe.so")

ARCH = "gfx950"
# No packed-fp32 instructions anywhere.
DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-source extra flags: MFMA accumulators of built-in MFMAs in the VGPR form
# (the decode kernel pins its large accumulator to AGPRs itself).
EXTRA_FLAGS = {"proj_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
               "decode_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
               "prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}

SOURCES = ["mla_api.cpp", "decode_mfma.hip", "decode_generic.hip", "combine.hip",
           "absorb.hip", "out_proj.hip", "cache_append.hip", "proj_mfma.hip", "tail_mfma.hip",
           "block_pool.cpp", "gemm_nt.hip", "prefill.hip"]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 4, lib_path: str = LIB, host_flags=(), synth: bool = True) -> None:
    """Compile libmla.so (to ``lib_path``) and, with ``synth``, libmla_synth.so
    and libmla_probe.so.
    ``host_flags`` go to the host side of every compile and the link (each one
    behind -Xarch_host, e.g. sanitizers for a host-checking build)."""
    hipcc = _hipcc()
    host = [x for f in host_flags for x in ("-Xarch_host", f)]
    with tempfile.TemporaryDirectory(prefix="mla_build_") as tmp:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            _run([hipcc, *DEVICE_FLAGS, *EXTRA_FLAGS.get(src, []), *host, *lang, "-I", CSRC,
                  "-I", os.path.join(ROOT, "include"),
                  "-c", os.path.join(CSRC, src), "-o", obj])
            return obj
        with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
            objs = list(ex.map(compile_one, SOURCES))
        tmp_lib = lib_path + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *host, "-o", tmp_lib, *objs])
        os.replace(tmp_lib, lib_path)
        if not synth:
            return
        synth_obj = os.path.join(tmp, "synth.o")
        _run([hipcc, *DEVICE_FLAGS, "-c", SYNTH_SRC, "-o", synth_obj])
        tmp_synth = SYNTH_LIB + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_synth, synth_obj])
        os.replace(tmp_synth, SYNTH_LIB)
        probe_obj = os.path.join(tmp, "probe.o")
        _run([hipcc, *DEVICE_FLAGS, "-c", PROBE_SRC, "-o", probe_obj])
        tmp_probe = PROBE_LIB + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp_probe, probe_obj])
        os.replace(tmp_probe, PROBE_LIB)
    if verbose:
        print(f"built {LIB}, {SYNTH_LIB} and {PROBE_LIB}")


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
