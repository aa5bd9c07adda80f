"""Benchmark of one MLA decode step (weight absorption, latent cache) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload v3_paged]

A step is the whole hot path over one batch: append the step's own latents to
the cache and absorb the query through W_UK (+ query RoPE) in one launch
(mla_append_absorb_q, unless --separate-append), decode attention over
the latent cache split into token-balanced work units, log-sum-exp combine of
the partials, and the W_UV up-projection (the last two as one pass over the
partials, mla_combine_out_proj, unless --separate-tail).  Inputs are seeded synthetic
DeepSeek-V3-shaped tensors already resident in HBM when timing starts.

Timing: every timed rep (a step, or in a second pass a step with events
around mla_decode) runs right after an untimed flush that reads and writes
1 GiB, so no rep finds the cache, weights or queries in L2 or the 256 MB
memory-side cache, and the GPU stays busy between reps (the clock cannot
idle-recover).  Each rep has its own HIP event pair on the launch stream.

Prints one JSON line: algorithmic GB/s of the step (value, from the mean
step time), decode tokens/s, median and minimum step and kernel times, the
roofline of the dominant kernel (mla_decode), and the fp64 CPU oracle timed
on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20,
                    help="untimed steps first (at least --warmup-seconds of them)")
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="time floor of the warm-up: steps continue until both --warmup steps and this many "
                         "seconds have run")
    ap.add_argument("--kernel-reps", type=int, default=20,
                    help="minimum number of mla_decode launches timed for the roofline (at least --steps)")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="MiB read and written by the untimed flush before every timed rep (0 = no flush)")
    ap.add_argument("--flush-kind", choices=("rw+read", "rw"), default="rw+read",
                    help="rw+read: write the flush buffer, then read another one so the caches end clean; rw: only "
                         "the read-write pass (its dirty lines are written back inside the next rep)")
    ap.add_argument("--workload", default="v3_paged",
                    help="v3_paged (default: the largest single-GPU workload, B=128 ragged contexts, paged), "
                         "v3_b64, v3_split, v3_b1, tiny_fp32")
    ap.add_argument("--prefill", choices=("prompt4k", "chunk1k"), default=None,
                    help="time mla_prefill instead of the decode step: a 4096-token prompt (B=1), or 1024-token "
                         "chunks after 7168 cached tokens (B=4)")
    ap.add_argument("--cache", choices=("native", "fp8"), default="native",
                    help="cache storage: the workload's own dtype, or fp8 e4m3 with per-128-channel scales")
    ap.add_argument("--num-splits", type=int, default=0, help="0 = library default for the batch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="replay the timed steps from a HIP graph captured once (eager launches are as fast "
                         "or faster on these kernels, so they are the default)")
    ap.add_argument("--separate-append", action="store_true",
                    help="append the step's rows with mla_cache_append, then mla_absorb_q (two launches)")
    ap.add_argument("--separate-tail", action="store_true",
                    help="mla_combine then mla_out_proj instead of mla_combine_out_proj")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain fp32 copy kernel (dst = -src) over this many MiB, 5 times: the "
                         "calibration run for the HBM byte counters")
    ap.add_argument("--stream-probe-mib", type=int, default=0,
                    help="only measure plain HBM streaming over buffers of this many MiB: torch's sum (read only) "
                         "and neg (read + write), 20 reps each with HIP events, after the same flush as the bench; "
                         "the practical ceiling the decode rates are set against")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="minimum oracle time in the CPU sample")
    ap.add_argument("--folds", action="store_true",
                    help="instead of the step bench: the weight folds' per-step products (layer output through "
                         "W_comb = W_UV W_O vs through W_UV then W_O; q_lat through W_KQ = W_UQ W_UK^T) at the "
                         "workload's batch, d_model 7168, d_q 1536")
    ap.add_argument("--session", action="store_true",
                    help="instead of the step bench: multi-step decode (DecodeSession) over a paged cache that "
                         "grows by n_q tokens per sequence per step, blocks from the library's block pool; "
                         "the workload's contexts are the prompts")
    return ap.parse_args()


def algorithmic_bytes(w, ctx):
    """Bytes the method itself must move (no partials, padding or re-reads)."""
    eb = 2 if w.dtype == "bf16" else 4
    B, nq = w.batch, w.n_q
    cache = int(ctx.sum()) * w.cache_row_bytes
    q_in = B * nq * w.n_h * (w.d_nope + w.d_rope) * eb
    q_abs = B * nq * w.n_h * (w.d_c + w.d_rope) * eb
    wts = w.n_h * w.d_c * (w.d_nope + w.d_v) * eb
    out = B * nq * w.n_h * w.d_v * 4
    append = B * nq * (w.row * eb + w.cache_row_bytes)   # new raw rows in, cache rows out
    u_lse = B * nq * w.n_h * (w.d_c + 1) * 4
    return {"step": cache + q_in + wts + out + append, "decode": cache + q_abs + u_lse, "cache": cache}


def decode_flops(w, ctx, pos):
    """2 * rows * (d_c + d_rope + d_c) per visible (query, cached token) pair."""
    import numpy as np
    visible = np.minimum(pos + 1, ctx[:, None]).sum()
    return int(visible) * w.n_h * 2 * (2 * w.d_c + w.d_rope)


def host_cpu():
    """Threads the oracle uses and what they run on: the cores this process may
    run on (sched_getaffinity), capped by OMP_NUM_THREADS when the host sets a
    CPU share that way, and the model name from /proc/cpuinfo."""
    affinity = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(affinity, int(cap)) if cap.isdigit() and int(cap) > 0 else affinity
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return threads, affinity, model


def blas_threads(n):
    """Context manager that runs the BLAS / OpenMP pools with n threads."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=n)
    except Exception:   # threadpoolctl missing: the pools keep their defaults
        import contextlib
        return contextlib.nullcontext()


def cpu_baseline(w, min_seconds=10.0, head_group=16):
    """The fp64 oracle timed on a bounded sample of the same workload.

    Sequences are taken shortest and longest first, then in index order; each
    sequence is decoded for all its query tokens, one group of heads at a time,
    until the oracle has run for at least ``min_seconds`` (one group of 16
    heads is a few seconds at most).  Only the oracle calls are timed, not
    the generation of the synthetic rows.  GB/s = cache bytes the sample
    attended (each sequence's rows times the fraction of heads done) / time.
    """
    import numpy as np
    import oracle
    import workloads as W
    cores, affinity, model = host_cpu()
    with blas_threads(cores):
        return _cpu_baseline(w, min_seconds, head_group, cores, affinity, model)


def _cpu_baseline(w, min_seconds, head_group, cores, affinity, model):
    import numpy as np
    import oracle
    import workloads as W
    ctx = W.context_lengths(w)
    order = [int(np.argmin(ctx)), int(np.argmax(ctx))] + list(range(w.batch))
    order = list(dict.fromkeys(order))
    wt, q = W.weights(w), W.queries(w)
    pos = W.positions(w, ctx)
    fp8 = w.cache_dtype == "fp8"
    spent, sample_bytes, head_rows, done = 0.0, 0.0, 0, []
    for b in order:
        rows = W.cache_rows(w, b, 0, int(ctx[b]))
        c_kv = rows["c_kv"]
        if fp8:   # the oracle's quantisation of the sequence, timed with its decode
            t0 = time.perf_counter()
            c_kv = oracle.fp8_dequantize_latent(*oracle.fp8_quantize_latent(c_kv))
            spent += time.perf_counter() - t0
        heads_done = 0
        for h0 in range(0, w.n_h, head_group):
            heads = list(range(h0, min(h0 + head_group, w.n_h)))
            t0 = time.perf_counter()
            oracle.decode_sequence(q["q_nope"][b], q["q_rope"][b], pos[b], c_kv, rows["k_rope_raw"],
                                   wt["w_uk"], wt["w_uv"], w.sm_scale, w.rope_base, heads=heads)
            spent += time.perf_counter() - t0
            heads_done += len(heads)
            if spent >= min_seconds:
                break
        sample_bytes += int(ctx[b]) * w.cache_row_bytes * heads_done / w.n_h
        head_rows += heads_done * w.n_q
        done.append(f"{b}(ctx {int(ctx[b])}, {heads_done} heads)")
        if spent >= min_seconds:
            break
    return {"value": round(sample_bytes / spent / 1e9, 6), "unit": "GB/s", "cores": int(cores), "kind": "oracle",
            "affinity_cores": int(affinity), "cpu_model": model,
            "sample": f"sequences {', '.join(done)} of {w.name}, all {w.n_q} query token(s), heads in groups of "
                      f"{head_group}; {'fp8 quantise + dequantise, ' if fp8 else ''}fp64 reconstruct-then-attend; "
                      f"GB/s = attended cache bytes x heads done/"
                      f"{w.n_h} / oracle time",
            "seconds": round(spent, 3),
            "head_rows_per_s": round(head_rows / spent, 3)}


# the decode kernel and the device header with its work plan (which sets the
# partials it writes)
DECODE_SOURCES = tuple(os.path.join(os.path.dirname(os.path.abspath(__file__)), "mla_latent_kv_02_amd", "csrc", f)
                       for f in ("decode_mfma.hip", "mla_device.h"))
PROFILES = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles")


def measured_traffic(workload):
    """HBM bytes per decode launch from the committed counter summaries.

    A summary under profiles/ carries a line ``traffic-record: {json}`` with the
    workload, the sha256 of the decode kernel's sources (DECODE_SOURCES, in
    that order, concatenated) when the counters were taken, and the calibrated
    FETCH_SIZE + WRITE_SIZE bytes per launch.  The figure is returned only
    while the sources are unchanged; otherwise None.
    """
    import hashlib
    try:
        h = hashlib.sha256()
        for path in DECODE_SOURCES:
            with open(path, "rb") as f:
                h.update(f.read())
        sha = h.hexdigest()
        names = sorted(os.listdir(PROFILES))
    except OSError:
        return None
    for name in names:
        if not name.endswith((".md", ".txt")):
            continue
        with open(os.path.join(PROFILES, name)) as f:
            for line in f:
                if not line.startswith("traffic-record:"):
                    continue
                rec = json.loads(line.split(":", 1)[1])
                if rec.get("workload") == workload and rec.get("source_sha256") == sha:
                    return int(rec["fetch_bytes"] + rec["write_bytes"])
    return None


def copy_probe(mib):
    """A plain elementwise copy of known size, for scaling the byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"copy probe: 5 x {mib} MiB read + {mib} MiB written")


PROBE_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "workloads", "libmla_probe.so")


def stream_probe(mib, flush_mib, reps=20):
    """Plain HBM streaming rates over `mib` MiB, each rep timed with its own
    events after the bench's flush; prints one JSON line:
      read, copy: torch.sum (reads only) and torch.neg into a second buffer
        (reads + writes);
      hip_read, hip_read_nt: 16-byte loads, 8 in flight per lane, over 256
        workgroups of 4 waves, plain and non-temporal (workloads/stream_probe.hip);
      rows_paged_nt: the decode kernel's stage loads (36 KiB stages of
        1152-byte rows, 4-slot LDS ring, two barriers a stage) over 64-row
        blocks in a seeded random order, non-temporal, with no work between."""
    import ctypes
    import numpy as np
    import torch
    n = mib * (1 << 20) // 4
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (n,), dtype=torch.int32, device="cuda").view(torch.float32)
    dst = torch.empty_like(src)
    acc = torch.zeros((), dtype=torch.float32, device="cuda")
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    flush = make_flush(flush_mib)
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                                      ctypes.c_void_p]
    lib.probe_stream_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    n_blocks = (n * 4 // 73728) // 128 * 128          # 64-row blocks of 1152 bytes, 2 stages each over 256 WGs
    order = torch.from_numpy(np.random.default_rng(7).permutation(n_blocks).astype(np.int32)).cuda()

    def call(status):
        if status != 0:
            raise RuntimeError(f"stream probe launch failed ({status})")
    out = {"probe": "hbm_stream", "mib": mib, "reps": reps, "flush_mib_per_rep": flush_mib}
    for name, fn, nbytes in (
            ("read", lambda: torch.sum(src, (0,), out=acc), n * 4),
            ("copy", lambda: torch.neg(src, out=dst), n * 8),
            ("hip_read", lambda: call(lib.probe_stream_read(src.data_ptr(), n * 4, 0, sink.data_ptr(), stream)), n * 4),
            ("hip_read_nt", lambda: call(lib.probe_stream_read(src.data_ptr(), n * 4, 1, sink.data_ptr(), stream)),
             n * 4),
            ("rows_paged_nt", lambda: call(lib.probe_stream_rows(src.data_ptr(), order.data_ptr(), n_blocks, 1,
                                                                 sink.data_ptr(), stream)), n_blocks * 73728)):
        ts = []
        for r in range(reps + 3):
            flush()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            if r >= 3:
                ts.append(e0.elapsed_time(e1) * 1e-3)
        rates = np.array([nbytes / t / 1e9 for t in ts])
        out[name + "_gbs"] = {"median": round(float(np.median(rates)), 1), "min": round(float(rates.min()), 1),
                              "max": round(float(rates.max()), 1), "bytes_per_rep": nbytes}
    print(json.dumps(out), flush=True)


def rows_stream_rate(flush, mib=2048, reps=10):
    """The decode kernel's own load schedule at memory speed: median GB/s of
    probe_stream_rows (36 KiB stages of 1152-byte rows over randomly ordered
    64-row blocks, non-temporal, no work between) over `mib` MiB of random
    data, each rep after the bench's flush.  The practical rate the decode's
    counter traffic is set against."""
    import ctypes
    import numpy as np
    import torch
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.probe_stream_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p]
    n_blocks = (mib * (1 << 20) // 73728) // 128 * 128
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (n_blocks * 73728 // 4,), dtype=torch.int32, device="cuda")
    order = torch.from_numpy(np.random.default_rng(7).permutation(n_blocks).astype(np.int32)).cuda()
    sink = torch.zeros(256, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rates = []
    for r in range(reps + 2):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        if lib.probe_stream_rows(src.data_ptr(), order.data_ptr(), n_blocks, 1, sink.data_ptr(), stream) != 0:
            raise RuntimeError("stream probe launch failed")
        e1.record()
        torch.cuda.synchronize()
        if r >= 2:
            rates.append(n_blocks * 73728 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src
    return float(np.median(rates))


def make_flush(mib, kind="rw+read"):
    """An untimed flush of the GPU caches before a timed rep.

    "rw": one elementwise kernel that reads and writes ``mib`` MiB (4x the
    256 MB memory-side cache for the default 1 GiB): afterwards L2 and that
    cache hold nothing of the rep's inputs, but they hold dirty lines whose
    write-back then lands inside the timed rep.  "rw+read" (default): the
    same, then a reduction that only reads another ``mib`` MiB, which writes
    the dirty lines back before the rep and leaves the caches clean."""
    import torch
    if mib <= 0:
        return lambda: None
    n = mib * (1 << 20) // 4
    buf = torch.zeros(n, dtype=torch.float32, device="cuda")
    if kind == "rw":
        return lambda: buf.add_(1.0)
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    acc = torch.zeros((), dtype=torch.float32, device="cuda")

    def flush():
        buf.add_(1.0)
        torch.sum(src, (0,), out=acc)
    return flush


def folds_bench(args):
    """Time the per-step products of the weight folds against their bytes."""
    import numpy as np
    import torch
    import mla_latent_kv_02_amd as mla
    import workloads as W
    from workloads.device import dims_of, to_device

    w = W.get(args.workload)
    if w.dtype != "bf16":
        sys.exit("--folds runs the bf16 V3-shaped workloads")
    d_model, d_q = 7168, 1536
    dims = dims_of(w)
    M = w.batch * w.n_q
    g = torch.Generator(device="cuda").manual_seed(w.seed)
    rnd = lambda *shape, scale=1.0: (torch.randn(shape, generator=g, device="cuda") * scale)
    w_uv = to_device(W.weights(w)["w_uv"], "bf16", "cuda")
    w_uk = to_device(W.weights(w)["w_uk"], "bf16", "cuda")
    w_o = rnd(d_model, w.n_h, w.d_v, scale=(w.n_h * w.d_v) ** -0.5).to(torch.bfloat16)
    w_uq = rnd(d_q, w.n_h, w.d_nope, scale=d_q ** -0.5).to(torch.bfloat16)
    u = rnd(w.batch, w.n_q, w.n_h, w.d_c)
    o = torch.empty((w.batch, w.n_q, w.n_h, w.d_v), device="cuda")
    y = torch.empty((w.batch, w.n_q, d_model), device="cuda")
    c_q = rnd(w.batch, w.n_q, d_q).to(torch.bfloat16)
    q_nope = rnd(w.batch, w.n_q, w.n_h, w.d_nope).to(torch.bfloat16)
    q_rope = rnd(w.batch, w.n_q, w.n_h, w.d_rope).to(torch.bfloat16)
    pos = torch.zeros((w.batch, w.n_q), dtype=torch.int32, device="cuda")
    q_lat = torch.empty((w.batch, w.n_q, w.n_h, w.d_c), dtype=torch.bfloat16, device="cuda")
    q_pe = torch.empty((w.batch, w.n_q, w.n_h, w.d_rope), dtype=torch.bfloat16, device="cuda")
    w_comb = torch.empty((d_model, w.n_h, w.d_c), dtype=torch.bfloat16, device="cuda")
    w_kq = torch.empty((w.n_h, w.d_c, d_q), dtype=torch.bfloat16, device="cuda")
    mla.mla_fold_out(dims, w_uv, w_o, w_comb)
    mla.mla_fold_q(dims, w_uq, w_uk, w_kq)

    def timed(fn, reps=50):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3    # us

    nb = lambda t: t.numel() * t.element_size()
    rows = []
    def row(name, fn, nbytes):
        us = timed(fn)
        rows.append({"product": name, "us": round(us, 2), "bytes": int(nbytes),
                     "GBps": round(nbytes / (us * 1e-6) / 1e9, 1), "frac_of_8TBps": round(nbytes / (us * 1e-6) / 8e12, 3)})
        log(f"{name}: {us:.1f} us, {nbytes / 1e6:.1f} MB")
    row("output unfolded: mla_out_proj (u W_UV) + mla_o_proj (o W_O)",
        lambda: (mla.mla_out_proj(dims, u, w_uv, o), mla.mla_o_proj(dims, o, w_o, y)),
        nb(u) + nb(w_uv) + 2 * nb(o) + nb(w_o) + nb(y))
    row("output folded: mla_out_proj_folded (u W_comb)", lambda: mla.mla_out_proj_folded(dims, u, w_comb, y),
        nb(u) + nb(w_comb) + nb(y))
    row("query absorbed: mla_absorb_q (q_nope -> q_lat; c_q W_UQ is outside the library)",
        lambda: mla.mla_absorb_q(dims, q_nope, q_rope, pos, w_uk, q_lat, q_pe),
        nb(q_nope) + nb(q_rope) + nb(w_uk) + nb(q_lat) + nb(q_pe))
    row("query folded: mla_absorb_q_folded (c_q W_KQ)",
        lambda: mla.mla_absorb_q_folded(dims, c_q, q_rope, pos, w_kq, q_lat, q_pe),
        nb(c_q) + nb(q_rope) + nb(w_kq) + nb(q_lat) + nb(q_pe))
    result = {"metric": "MLA weight folds: per-step products, time and HBM GB/s (DeepSeek-V3 shapes)",
              "value": rows[1]["us"], "unit": "us (folded output product)", "higher_is_better": False,
              "n_gpus": 1, "dtype": "bf16", "data": "synthetic (seeded N(0,1/fan_in) weights)",
              "config": {"workload": f"{w.name} batch: {M} query rows, d_model {d_model}, d_q {d_q}"},
              "products": rows}
    print(json.dumps(result), flush=True)


def session_bench(args):
    """Multi-step decode over a growing paged cache: prefill the workload's
    contexts through DecodeSession.append, then time --steps steps (after
    --warmup) of DecodeSession.step, each appending n_q new rows per sequence."""
    import numpy as np
    import torch
    import workloads as W
    from mla_latent_kv_02_amd.plan import default_num_splits
    from mla_latent_kv_02_amd.step import DecodeSession
    from workloads.device import dims_of, to_device

    w = W.get(args.workload)
    if w.dtype != "bf16":
        sys.exit("--session runs the bf16 V3-shaped workloads")
    bs = w.block_size or 64
    ctx = W.context_lengths(w)
    grow = (args.warmup + args.steps + 1) * w.n_q
    need = (ctx.astype(np.int64) + grow + bs - 1) // bs
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    num_splits = args.num_splits or default_num_splits(int(ctx.sum()), w.n_q, w.n_h)
    sess = DecodeSession(dims_of(w), w.batch, w.n_q, num_splits, tdt, n_blocks=int(need.sum()), block_size=bs,
                         max_blocks=int(need.max()))
    log(f"session on {w.name}: prefill {int(ctx.sum())} tokens in blocks of {bs}")
    t0 = time.perf_counter()
    seq_all = np.repeat(np.arange(w.batch, dtype=np.int32), ctx)
    tok_all = np.concatenate([np.arange(c, dtype=np.int32) for c in ctx])
    table = torch.from_numpy(W.normal_table_bf16_bits().view(np.int16)).cuda() if w.dtype == "bf16" else None
    chunk = 1 << 20
    for s0 in range(0, len(seq_all), chunk):
        sq, tk = seq_all[s0:s0 + chunk], tok_all[s0:s0 + chunk]
        raw = torch.empty((len(sq), w.row), dtype=tdt, device="cuda")
        sd, td = torch.from_numpy(sq).cuda(), torch.from_numpy(tk).cuda()
        W.fill_cache_rows_device(w, sd.data_ptr(), td.data_ptr(), len(sq), table.data_ptr(), raw.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
        sess.append(sq, tk, raw[:, :w.d_c], raw[:, w.d_c:])
        del raw
    log(f"prefilled in {time.perf_counter() - t0:.1f} s")
    wt, q = W.weights(w), W.queries(w)
    w_uk, w_uv = to_device(wt["w_uk"], w.dtype, "cuda"), to_device(wt["w_uv"], w.dtype, "cuda")
    q_nope, q_rope = to_device(q["q_nope"], w.dtype, "cuda"), to_device(q["q_rope"], w.dtype, "cuda")
    g = torch.Generator(device="cuda").manual_seed(w.seed)
    new = torch.randn((w.batch, w.n_q, w.row), generator=g, device="cuda").to(tdt)
    c_new, r_new = new[..., :w.d_c], new[..., w.d_c:]
    c_new, r_new = c_new.contiguous(), r_new.contiguous()
    for _ in range(args.warmup):
        sess.step(c_new, r_new, q_nope, q_rope, w_uk, w_uv)
    torch.cuda.synchronize()
    ctx0 = sess.ctx.astype(np.int64).copy()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        sess.step(c_new, r_new, q_nope, q_rope, w_uk, w_uv)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # cache rows attended over the timed steps (query j of a step sees ctx + j + 1 rows)
    attended = sum(int(((ctx0 + k * w.n_q)[:, None] + np.arange(1, w.n_q + 1)[None, :]).sum())
                   for k in range(1, args.steps + 1))
    row_bytes = w.row * (2 if w.dtype == "bf16" else 4)
    result = {
        "metric": "MLA multi-step decode over a growing paged cache: decode tokens/s (DeepSeek-V3 shapes)",
        "value": round(w.batch * w.n_q / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded Philox N(0,1) prompt latents, N(0,1) new rows and queries)",
        "config": {"workload": f"{w.name} as prompts, +{w.n_q} token(s) per sequence per step",
                   "batch": w.batch, "n_q": w.n_q, "block_size": bs, "num_splits": num_splits,
                   "prompt_tokens": int(ctx.sum()), "blocks": int(need.sum())},
        "cache_GBps_attended": round(attended / args.steps * row_bytes / (ms * 1e-3) / 1e9, 2),
    }
    print(json.dumps(result), flush=True)


PREFILL_WORKLOADS = {"prompt4k": (1, 4096, 4096), "chunk1k": (4, 8192, 1024)}   # B, ctx, n_q


def prefill_cpu_baseline(w, ctx, n_q, min_seconds=10.0, q_sample=256, head_group=16):
    """The fp64 oracle on a bounded sample of a prefill workload: sequence 0,
    its last ``q_sample`` query tokens (each sees ~ctx cached tokens, the
    costliest rows), heads in groups of ``head_group`` until the oracle has run
    for ``min_seconds``.  The oracle rebuilds K and V of the heads it runs
    (ctx tokens) and attends; the sample's FLOPs follow the GPU line's
    definition (reconstruction of those heads' ctx tokens + attention of the
    sampled rows), so TFLOP/s is comparable.  Queries are seeded normal draws
    (timing only)."""
    cores, affinity, model = host_cpu()
    with blas_threads(cores):
        r = _prefill_cpu_baseline(w, ctx, n_q, min_seconds, q_sample, head_group)
    r.update({"cores": int(cores), "affinity_cores": int(affinity), "cpu_model": model})
    return r


def _prefill_cpu_baseline(w, ctx, n_q, min_seconds, q_sample, head_group):
    import numpy as np
    import oracle
    import workloads as W
    rng = np.random.default_rng(73)
    nq = min(q_sample, n_q)
    q_nope = rng.standard_normal((nq, w.n_h, w.d_nope))
    q_rope = rng.standard_normal((nq, w.n_h, w.d_rope))
    pos = np.arange(ctx - nq, ctx)
    wt = W.weights(w)
    rows = W.cache_rows(w, 0, 0, ctx)
    spent, heads_done, flops = 0.0, 0, 0.0
    for h0 in range(0, w.n_h, head_group):
        heads = list(range(h0, min(h0 + head_group, w.n_h)))
        t0 = time.perf_counter()
        oracle.decode_sequence(q_nope, q_rope, pos, rows["c_kv"], rows["k_rope_raw"], wt["w_uk"], wt["w_uv"],
                               w.sm_scale, w.rope_base, heads=heads)
        spent += time.perf_counter() - t0
        heads_done += len(heads)
        flops += len(heads) * (ctx * 2 * w.d_c * (w.d_nope + w.d_v)
                               + int((pos + 1).sum()) * 2 * (w.d_nope + w.d_rope + w.d_v))
        if spent >= min_seconds:
            break
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "kind": "oracle",
            "sample": f"sequence 0 of {w.name} (ctx {ctx}), its last {nq} query tokens, {heads_done} of {w.n_h} "
                      f"heads in groups of {head_group}; fp64 rebuild of those heads' K/V then causal attention; "
                      f"FLOPs as in the GPU line",
            "seconds": round(spent, 3)}


def prefill_bench(args):
    """mla_prefill at V3 shapes: the cache holds ctx rows per sequence, the last
    n_q of them are queries (positions ctx - n_q .. ctx - 1).  Cache rows come
    from the seeded device generator, queries from a seeded device normal draw.
    FLOPs = attention 2 (d_nope + d_rope + d_v) per (query, visible token, head)
    + reconstruction 2 d_c (d_nope + d_v) per (cached token, head)."""
    import torch
    import mla_latent_kv_02_amd as mla
    import workloads as W
    from workloads.device import stage
    B, ctx, n_q = PREFILL_WORKLOADS[args.prefill]
    w = W.custom(name=f"v3_prefill_{args.prefill}", seed=71, batch=B, n_q=1, ctx=ctx,
                 description=f"DeepSeek-V3 shapes, B={B}, ctx {ctx}, the last {n_q} tokens prefilled")
    log(f"staging {w.name}")
    st = stage(w)
    d = st["dims"]
    g = torch.Generator(device="cuda").manual_seed(72)
    bf = torch.bfloat16
    q_nope = torch.randn((B, n_q, w.n_h, w.d_nope), generator=g, device="cuda").to(bf)
    q_rope = torch.randn((B, n_q, w.n_h, w.d_rope), generator=g, device="cuda").to(bf)
    positions = torch.arange(ctx - n_q, ctx, dtype=torch.int32, device="cuda").repeat(B, 1).contiguous()
    w_kv = torch.empty((w.n_h, w.d_nope + w.d_v, w.d_c), dtype=bf, device="cuda")
    mla.mla_prefill_weights(d, st["w_uk"], st["w_uv"], w_kv)
    ws = torch.empty((mla.mla_prefill_workspace_bytes(d, B, ctx) // 2,), dtype=bf, device="cuda")
    q_pe = torch.empty((B, n_q, w.n_h, w.d_rope), dtype=bf, device="cuda")
    out = torch.empty((B, n_q, w.n_h, w.d_v), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, n_q, w.n_h), dtype=torch.float32, device="cuda")

    def run():
        mla.mla_prefill(d, ctx, q_nope, q_rope, positions, st["cache"], w_kv, ws, q_pe, out, lse)

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        run()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    visible = B * sum(p + 1 for p in range(ctx - n_q, ctx))
    f_attn = visible * w.n_h * 2 * (w.d_nope + w.d_rope + w.d_v)
    f_rec = B * ctx * w.n_h * 2 * w.d_c * (w.d_nope + w.d_v)
    tflops = (f_attn + f_rec) / (ms * 1e-3) / 1e12
    log(f"prefill {ms * 1e3:.1f} us; attention {f_attn / 1e9:.1f} GFLOP + reconstruction {f_rec / 1e9:.1f} GFLOP")
    print(json.dumps({
        "metric": "MLA prefill TFLOP/s (DeepSeek-V3 shapes)", "value": round(tflops, 2), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Philox N(0,1) cache latents, seeded device N(0,1) queries, N(0,1/d_c) weights)",
        "config": {"workload": w.name, "description": w.description, "batch": B, "ctx": ctx, "n_q": n_q,
                   "n_h": w.n_h, "d_c": w.d_c, "d_rope": w.d_rope, "d_nope": w.d_nope, "d_v": w.d_v},
        "tokens_per_s": round(B * n_q / (ms * 1e-3), 1),
        "flops_per_call": {"attention": f_attn, "reconstruction": f_rec},
        "roofline": {"kernel": "mla_prefill (reconstruct_gemm_kernel + prefill_attn_kernel)", "bound": "mfma",
                     "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFS, 4), "traffic": None},
        "cpu_baseline": None if args.no_cpu_baseline else prefill_cpu_baseline(w, ctx, n_q, args.cpu_seconds)}),
        flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); multi-GPU sharding of this "
              f"path is a design note, not a measured configuration.", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.stream_probe_mib:
        stream_probe(args.stream_probe_mib, args.flush_mib)
        return
    if args.session:
        session_bench(args)
        return
    if args.folds:
        folds_bench(args)
        return
    if args.prefill:
        prefill_bench(args)
        return
    import numpy as np
    import torch
    import mla_latent_kv_02_amd as mla
    import workloads as W
    from mla_latent_kv_02_amd.plan import default_num_splits
    from mla_latent_kv_02_amd.step import DecodeStep
    from workloads.device import stage

    w = W.get(args.workload)
    if args.cache == "fp8":
        w = W.with_fp8_cache(w)
    log(f"staging {w.name}: {w.description}")
    t0 = time.perf_counter()
    st = stage(w)
    log(f"staged in {time.perf_counter() - t0:.1f} s")
    ctx, pos = st["ctx_host"], st["positions_host"]
    num_splits = args.num_splits or default_num_splits(int(ctx.sum()), w.n_q, w.n_h)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    step = DecodeStep(st["dims"], w.batch, w.n_q, num_splits, tdt)

    # the step's own latents: the last n_q rows of every sequence (raw, before rotation)
    seq_ids = np.repeat(np.arange(w.batch, dtype=np.int32), w.n_q)
    tok = pos.reshape(-1).astype(np.int32)
    raw = torch.empty((len(seq_ids), w.row), dtype=tdt, device="cuda")
    if w.dtype == "bf16":
        table = torch.from_numpy(W.normal_table_bf16_bits().view(np.int16)).cuda()
        sd, td = torch.from_numpy(seq_ids).cuda(), torch.from_numpy(tok).cuda()
        W.fill_cache_rows_device(w, sd.data_ptr(), td.data_ptr(), len(seq_ids), table.data_ptr(), raw.data_ptr(),
                                 torch.cuda.current_stream().cuda_stream)
    else:
        rows = [W.cache_rows(w, int(b), int(t), int(t) + 1) for b, t in zip(seq_ids, tok)]
        raw.copy_(torch.from_numpy(np.concatenate([np.concatenate([r["c_kv"], r["k_rope_raw"]], 1) for r in rows])))
        sd, td = torch.from_numpy(seq_ids).cuda(), torch.from_numpy(tok).cuda()
    new_tokens = (sd, td, raw[:, :w.d_c], raw[:, w.d_c:])

    stream = torch.cuda.current_stream()
    d = st["dims"]
    # combine + up-projection as one pass over the partials where it is compiled
    fused_tail = w.dtype == "bf16" and w.d_c == 512 and w.d_v == 128 and not args.separate_tail

    def run_step(ev=None):
        if args.separate_append:
            mla.mla_cache_append(d, st["cache"], *new_tokens)
            mla.mla_absorb_q(d, st["q_nope"], st["q_rope"], st["positions"], st["w_uk"], step.q_lat, step.q_pe)
        else:
            mla.mla_append_absorb_q(d, st["cache"], *new_tokens, st["q_nope"], st["q_rope"], st["positions"],
                                    st["w_uk"], step.q_lat, step.q_pe)
        if ev is not None:
            ev[0].record(stream)
        mla.mla_decode(d, step.q_lat, step.q_pe, st["cache"], st["positions"], num_splits, step.u_part,
                       step.lse_part)
        if ev is not None:
            ev[1].record(stream)
        if fused_tail:
            mla.mla_combine_out_proj(d, st["cache"].ctx_lens, num_splits, step.u_part, step.lse_part, st["w_uv"],
                                     step.out, step.lse)
        else:
            mla.mla_combine(d, st["cache"].ctx_lens, num_splits, step.u_part, step.lse_part, step.u, step.lse)
            mla.mla_out_proj(d, step.u, st["w_uv"], step.out)

    flush = make_flush(args.flush_mib, args.flush_kind)
    log(f"num_splits={num_splits}; warmup >= {args.warmup} steps and >= {args.warmup_seconds} s")
    warm_steps, warm_t0 = 0, time.perf_counter()
    while warm_steps < args.warmup or time.perf_counter() - warm_t0 < args.warmup_seconds:
        flush()
        run_step()
        warm_steps += 1
        if warm_steps % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warm_s = time.perf_counter() - warm_t0
    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_step()
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
    # (1) the step: K reps, each right after an untimed flush, each with its own
    # event pair on the launch stream
    log(f"timing {args.steps} steps" + (" (graph replays)" if graph is not None else ""))
    step_ms = []
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for e0, e1 in evs:
        flush()
        e0.record(stream)
        if graph is not None:
            graph.replay()
        else:
            run_step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    step_ms = [e0.elapsed_time(e1) for e0, e1 in evs]
    ms_step = sum(step_ms) / len(step_ms)
    # (2) the dominant kernel: max(K, --kernel-reps) more reps, each after a flush,
    # with an event pair right around mla_decode
    n_dec = max(args.steps, args.kernel_reps)
    dec_evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_dec)]
    for ev in dec_evs:
        flush()
        run_step(ev)
    torch.cuda.synchronize()
    dec_ms = [a.elapsed_time(b) for a, b in dec_evs]
    dec_avg = sum(dec_ms) / len(dec_ms)
    med = lambda v: sorted(v)[len(v) // 2] if len(v) % 2 else 0.5 * (sorted(v)[len(v) // 2 - 1] + sorted(v)[len(v) // 2])
    log(f"step mean {ms_step * 1e3:.1f} us, median {med(step_ms) * 1e3:.1f}, min {min(step_ms) * 1e3:.1f} "
        f"(wall incl. flushes {wall / args.steps * 1e6:.1f} us); decode kernel mean {dec_avg * 1e3:.1f} us, median "
        f"{med(dec_ms) * 1e3:.1f}, min {min(dec_ms) * 1e3:.1f} over {n_dec} launches")

    nbytes = algorithmic_bytes(w, ctx)
    flops = decode_flops(w, ctx, pos)
    value = nbytes["step"] / (ms_step * 1e-3) / 1e9
    achieved = nbytes["decode"] / (dec_avg * 1e-3) / 1e9
    tflops = flops / (dec_avg * 1e-3) / 1e12
    # the bound is whichever roofline takes longer at peak rates
    mfma_bound = flops / (MFMA_BF16_PEAK_TFS * 1e12) > nbytes["decode"] / (HBM_PEAK_GBS * 1e9)
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s",
                "frac": round(tflops / MFMA_BF16_PEAK_TFS, 4), "hbm_gbs": round(achieved, 2),
                "hbm_frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "mfma_tflops": round(tflops, 2),
                "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFS, 4)}
    result = {
        "metric": "MLA decode latent-cache GB/s + tokens/s (DeepSeek-V3 shapes), % of roofline",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic (seeded Philox N(0,1) latents/queries, "
        "N(0,1/d_c) weights)",
        "timing": {"step_us": {"mean": round(ms_step * 1e3, 2), "median": round(med(step_ms) * 1e3, 2),
                               "min": round(min(step_ms) * 1e3, 2), "reps": len(step_ms)},
                   "decode_us": {"mean": round(dec_avg * 1e3, 2), "median": round(med(dec_ms) * 1e3, 2),
                                 "min": round(min(dec_ms) * 1e3, 2), "reps": len(dec_ms)},
                   "flush_mib_per_rep": args.flush_mib, "flush_kind": args.flush_kind,
                   "warmup_steps_run": warm_steps,
                   "warmup_seconds_run": round(warm_s, 3),
                   "note": "one HIP event pair per rep on the launch stream; before every rep an untimed flush: "
                           "read+write flush_mib_per_rep MiB, then (rw+read) read another flush_mib_per_rep MiB "
                           "so no dirty line is left; value and ms_per_step use the mean"},
        "config": {"workload": w.name, "description": w.description, "fused_tail": fused_tail,
                   "fused_append": not args.separate_append,
                   "step_launch": "graph" if graph is not None else "eager", "batch": w.batch, "n_q": w.n_q,
                   "n_h": w.n_h, "d_c": w.d_c, "d_rope": w.d_rope, "d_nope": w.d_nope, "d_v": w.d_v,
                   "context_tokens": int(ctx.sum()), "block_size": w.block_size, "num_splits": num_splits,
                   "cache": w.cache_dtype, "cache_row_bytes": w.cache_row_bytes},
        "tokens_per_s": round(w.batch * w.n_q / (ms_step * 1e-3), 1),
        "kv_tokens_per_s": round(float(ctx.sum()) / (ms_step * 1e-3), 1),
        "step_bytes": nbytes["step"],
        "roofline": {"kernel": "mla_decode (decode_mfma_kernel)", **roof,
                     "traffic": measured_traffic(w.name), "bytes_per_launch": nbytes["decode"],
                     "flops_per_launch": flops, "avg_launch_us": round(dec_avg * 1e3, 3),
                     "median_launch_us": round(med(dec_ms) * 1e3, 3), "min_launch_us": round(min(dec_ms) * 1e3, 3),
                     "launches_timed": len(dec_ms)},
        "cpu_baseline": None,
    }
    # the chip's practical streaming rate for the decode's access pattern, measured here
    # (reported as null when the probe library is not built; the line stands without it)
    if os.path.exists(PROBE_LIB):
        rate = rows_stream_rate(flush)
        traffic = result["roofline"]["traffic"]
        result["roofline"]["practical"] = {
            "probe": "the decode's stage loads over randomly ordered 64-row blocks of 1152-byte rows, non-temporal, "
                     "no work between (workloads/stream_probe.hip), median GB/s after the flush",
            "gbs": round(rate, 1),
            "frac_algorithmic": round(achieved / rate, 4),
            "frac_traffic": round(traffic / (dec_avg * 1e-3) / 1e9 / rate, 4) if traffic else None}
        log(f"decode load schedule at memory speed: {rate:.0f} GB/s")
    else:
        result["roofline"]["practical"] = None
        log(f"{PROBE_LIB} is not built: no practical streaming rate")
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a CPU sample")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
