"""Code generation of the decode kernel: no register spills in its stage loops.

The decode kernel holds its output accumulator in all 256 AGPRs and the query
operand in about 144 VGPRs, so a change that adds a few live registers to the
stage loop makes the compiler spill there, and every scratch access in the
loop is a vector-memory operation that also waits for the stage loads in
flight: the kernel then runs several times slower with unchanged results.
This test compiles decode_mfma.hip for gfx950 with the library's flags (no
GPU needed), finds the stage loops in the assembly (innermost loops that hold
the MFMAs of a whole stage) and checks that those of the bf16 kernels, and the
buffer-load (contiguous and paged) ones of the fp8 kernels, have no scratch
access.  (The fp8 generic-layout loop does spill; that path only runs for
paged caches whose block size is not a multiple of 32 tokens or whose blocks
lie 4 GiB or more apart.)
"""
import os
import re
import shutil
import subprocess

import pytest

from mla_latent_kv_02_amd import build as mla_build

SRC = os.path.join(mla_build.CSRC, "decode_mfma.hip")
LAYOUTS = {0: "contiguous", 1: "paged", 2: "generic"}


def _loops(body):
    """(start, end) line ranges of the backward branches in one function."""
    labels = {}
    for i, l in enumerate(body):
        m = re.match(r"^(\.LBB\S+):", l)
        if m:
            labels[m.group(1)] = i
    out = []
    for i, l in enumerate(body):
        m = re.search(r"s_c?branch\w*\s+(\.LBB\S+)\s*$", l)
        if m and labels.get(m.group(1), i + 1) < i:
            out.append((labels[m.group(1)], i))
    return out


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("no hipcc")
    out = str(tmp_path_factory.mktemp("asm") / "decode_mfma.s")
    cmd = [hipcc, *mla_build.DEVICE_FLAGS, *mla_build.EXTRA_FLAGS["decode_mfma.hip"], "-I", mla_build.CSRC,
           "-I", os.path.join(mla_build.ROOT, "include"), "--cuda-device-only", "-S", SRC, "-o", out]
    cmd = [c for c in cmd if c != "-fPIC"]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-3000:]
    return open(out).read().split("\n")


def _kernels(lines):
    ks = {}
    for i, l in enumerate(lines):
        m = re.match(r"^(_ZN3mla12_GLOBAL__N_118decode_mfma_kernelILi(\d)ELb(\d)EEEvNS0_10DecodeArgsE):", l)
        if m:
            end = next(j for j in range(i, len(lines)) if lines[j].startswith(".Lfunc_end"))
            ks[(int(m.group(2)), m.group(3) == "1")] = lines[i:end]
    return ks


def _stage_loops(body):
    """Innermost loops with the MFMAs of at least one stage."""
    loops = []
    for j, i in set(_loops(body)):
        seg = body[j:i + 1]
        if sum("v_mfma" in x for x in seg) < 150:
            continue
        loops.append((j, i, seg))
    inner = [(j, i, seg) for (j, i, seg) in loops
             if not any(j <= j2 and i2 <= i and (j2, i2) != (j, i) for (j2, i2, _) in loops)]
    return inner


def test_decode_kernels_call_nothing(asm):
    """Everything is inlined into the six kernels: a call from a kernel whose
    accumulator lives in AGPRs saves and restores registers around it (an
    outlined segment body once made the paged kernel five times slower)."""
    funcs = [m.group(1) for l in asm for m in [re.search(r"\.type\s+(\S+),@function", l)] if m]
    assert len(funcs) == 6 and all("decode_mfma_kernelILi" in f and not f.startswith("_ZZ") for f in funcs), funcs
    assert not any("s_swappc" in l or "s_setpc" in l for l in asm)


def test_decode_stage_loops_do_not_spill(asm):
    ks = _kernels(asm)
    assert set(ks) == {(l, f) for l in (0, 1, 2) for f in (False, True)}, sorted(ks)
    report = []
    for (layout, fp8), body in sorted(ks.items()):
        loops = _stage_loops(body)
        assert loops, (layout, fp8)
        for j, i, seg in loops:
            scratch = sum("scratch_" in x for x in seg)
            buffered = any("buffer_load" in x and " lds" in x for x in seg)
            report.append(f"{LAYOUTS[layout]} {'fp8' if fp8 else 'bf16'} loop@{j}: scratch {scratch}, "
                          f"{'buffer' if buffered else 'global'} loads")
            if not fp8 or buffered:
                assert scratch == 0, report[-1]
    # the contiguous and paged kernels of both dtypes have their buffer-load stage loops
    for key in ((0, False), (1, False), (0, True), (1, True)):
        assert any(any("buffer_load" in x for x in seg) for _, _, seg in _stage_loops(ks[key])), key
    print("\n".join(report))
