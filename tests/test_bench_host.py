"""Host-side pieces of bench.py that need no GPU: the prefill line's CPU
baseline (the oracle on a bounded sample) reports FLOPs by the same
definition as the GPU line, counted here independently for a tiny workload;
the streaming-probe library loads and checks its sizes."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_prefill_cpu_baseline_flop_accounting(monkeypatch):
    w = W.custom(name="pf_tiny", seed=5, batch=1, n_q=1, n_h=4, d_c=64, d_rope=16, d_nope=32, d_v=32,
                 dtype="f32", ctx=40)
    ticks = iter(np.arange(0, 1000) * 1e-6)   # every oracle call "takes" 1 us
    monkeypatch.setattr(bench.time, "perf_counter", lambda: float(next(ticks)))
    r = bench.prefill_cpu_baseline(w, ctx=40, n_q=24, min_seconds=100.0, q_sample=8, head_group=2)
    # all 4 heads run (2 groups of 2), 1 us each
    assert r["seconds"] == 0.0   # 2 us in all, reported in ms resolution
    assert "4 of 4 heads" in r["sample"] and "last 8 query tokens" in r["sample"]
    pos = np.arange(40 - 8, 40)
    flops = 4 * (40 * 2 * 64 * (32 + 32) + int((pos + 1).sum()) * 2 * (32 + 16 + 32))
    assert abs(r["value"] - flops / 2e-6 / 1e12) <= 1e-6   # 0.7488 TFLOP/s
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s"


def test_stream_probe_library_exports_its_probes():
    """The bench's HBM streaming probes load without a GPU and reject bad
    sizes on the host (a non-multiple of 16 bytes, a block count the 256
    workgroups cannot split into whole stages)."""
    import ctypes
    import bench
    if not os.path.exists(bench.PROBE_LIB):
        pytest.skip("libmla_probe.so not built")
    lib = ctypes.CDLL(bench.PROBE_LIB)
    lib.probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p]
    lib.probe_stream_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p]
    assert lib.probe_stream_read(16, 100, 0, 16, None) == 1
    assert lib.probe_stream_read(None, 1024, 0, 16, None) == 1
    assert lib.probe_stream_rows(16, 16, 100, 1, 16, None) == 1     # 200 stages over 256 workgroups
    assert lib.probe_stream_rows(16, 16, 0, 1, 16, None) == 1
