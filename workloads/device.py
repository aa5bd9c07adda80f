"""Device-side staging of a synthetic workload (torch tensors on the GPU).

Builds the inputs of one decode step for a Workload: weights, queries,
positions, context lengths and a filled latent cache (contiguous or paged).
Raw cache rows come from the same counter-based generator as the host
functions in ``workloads`` (device copy in synth_fill.hip); they are written
into the cache by the library's own ``mla_cache_append`` (which rotates the
positional keys).  Unused cache slots hold NaN so that a kernel that reads
outside the valid rows shows it.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import (Workload, block_table, context_lengths, fill_cache_rows_device, normal_table_bf16_bits,
               positions, queries, weights)


def _torch():
    import torch
    return torch


def to_device(x: np.ndarray, dtype: str, device):
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(device=device, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def dims_of(w: Workload):
    import mla_latent_kv_02_amd as mla
    return mla.Dims(w.n_h, w.d_c, w.d_rope, w.d_nope, w.d_v, w.sm_scale, w.rope_base)


def stage(w: Workload, device="cuda", chunk_tokens: int = 1 << 20, ctx: Optional[np.ndarray] = None,
          stream=None) -> dict:
    """All inputs of one decode step of ``w`` on ``device``; ``ctx`` overrides
    the context lengths (for small parity cases)."""
    torch = _torch()
    import mla_latent_kv_02_amd as mla
    dev = torch.device(device)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    ctx = context_lengths(w) if ctx is None else np.asarray(ctx, dtype=np.int32)
    pos = positions(w, ctx)
    wt = weights(w)
    q = queries(w)
    out = {
        "workload": w, "dims": dims_of(w), "ctx_host": ctx, "positions_host": pos,
        "w_uk": to_device(wt["w_uk"], w.dtype, dev), "w_uv": to_device(wt["w_uv"], w.dtype, dev),
        "q_nope": to_device(q["q_nope"], w.dtype, dev), "q_rope": to_device(q["q_rope"], w.dtype, dev),
        "positions": torch.from_numpy(pos).to(dev), "ctx_lens": torch.from_numpy(ctx).to(dev),
    }
    B, row = w.batch, w.row
    fp8 = w.cache_dtype == "fp8"

    def poisoned(shape):
        # unused slots hold NaN: bf16 / fp32 NaN, or 0xFF bytes for fp8 rows
        # (NaN codes, NaN bf16 key, NaN fp32 scales)
        if fp8:
            return torch.full(shape[:-1] + (w.cache_row_bytes,), 0xFF, dtype=torch.uint8, device=dev)
        return torch.full(shape, float("nan"), dtype=tdt, device=dev)

    if w.block_size:
        table, n_blocks = block_table(w, ctx)
        data = poisoned((n_blocks, w.block_size, row))
        tbl = torch.from_numpy(table).to(dev)
        cache = mla.LatentCache(data=data, ctx_lens=out["ctx_lens"], block_table=tbl, block_size=w.block_size)
        out["block_table_host"] = table
    else:
        s_max = int(ctx.max()) if len(ctx) else 1
        data = poisoned((B, max(s_max, 1), row))
        cache = mla.LatentCache(data=data, ctx_lens=out["ctx_lens"])
    out["cache"] = cache

    # token list (sequence, position) of every cached token, in chunks
    seq_all = np.repeat(np.arange(B, dtype=np.int32), ctx)
    tok_all = np.concatenate([np.arange(c, dtype=np.int32) for c in ctx]) if B else np.zeros(0, np.int32)
    dims = out["dims"]
    table_dev = None
    if w.dtype == "bf16":
        table_dev = torch.from_numpy(normal_table_bf16_bits().view(np.int16)).to(dev)
    if w.dtype != "bf16":
        chunk_tokens = max(len(seq_all), 1)     # host rows, whole batch at once (small cases)
    for s0 in range(0, len(seq_all), chunk_tokens):
        seq_c = torch.from_numpy(seq_all[s0:s0 + chunk_tokens]).to(dev)
        tok_c = torch.from_numpy(tok_all[s0:s0 + chunk_tokens]).to(dev)
        n = seq_c.shape[0]
        if w.dtype == "bf16":
            raw = torch.empty((n, row), dtype=torch.bfloat16, device=dev)
            st = torch.cuda.current_stream().cuda_stream if stream is None else stream
            fill_cache_rows_device(w, seq_c.data_ptr(), tok_c.data_ptr(), n, table_dev.data_ptr(),
                                   raw.data_ptr(), st)
        else:
            from . import cache_rows
            parts = []
            for b in range(B):
                r = cache_rows(w, b, 0, int(ctx[b]))
                parts.append(np.concatenate([r["c_kv"], r["k_rope_raw"]], axis=1))
            raw = torch.from_numpy(np.concatenate(parts, axis=0).astype(np.float32)).to(dev)
        mla.mla_cache_append(dims, cache, seq_c, tok_c, raw[:, :w.d_c], raw[:, w.d_c:], stream=stream)
        del raw
    torch.cuda.synchronize(dev)
    return out
