"""Host-side check of the values the library reads only on the device.

The C ABI checks shapes, dtypes and alignment on the host, but context
lengths, query positions, block ids and append targets live in device memory
and are the caller's contract: the kernels read them as they are.  This module
copies them to the host and checks them, so that a test or a debugging session
finds a breach as an exception that names it, before the launch.  It
synchronises and copies, so it is opt-in: the binding runs it before each
decode and append call when the environment variable MLA_CHECK_CONTRACT is
"1", and the functions below can be called directly.

What the contract is (MLA decode over a latent cache of a decoding batch):
  - 0 <= ctx_lens[b] <= the cache's capacity for one sequence
    (max_blocks * block_size for a paged cache, S_max for a contiguous one);
  - paged: every block that holds one of the first ctx_lens[b] tokens of
    sequence b has an id in [0, n_blocks);
  - decode step: query j of sequence b is the token at position
    ctx_lens[b] - n_q + j (the n_q new tokens are the last n_q of the context;
    a negative position sees no token);
  - append: seq_ids[k] in [0, B), 0 <= positions[k] < capacity, the target
    block reserved (id in [0, n_blocks)), and no two new tokens written to
    the same cache row.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np


class ContractError(ValueError):
    """A device-side argument breaks the library's contract."""


def _host(x) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x)


def capacity(block_size: int, max_blocks: int, s_max: int) -> int:
    """Tokens one sequence can hold: max_blocks * block_size when paged
    (block_size > 0), else s_max."""
    return block_size * max_blocks if block_size else s_max


def ctx_errors(ctx_lens, cap: int) -> List[str]:
    ctx = _host(ctx_lens).astype(np.int64)
    errs = []
    bad = np.nonzero((ctx < 0) | (ctx > cap))[0]
    for b in bad[:4]:
        errs.append(f"ctx_lens[{b}] = {ctx[b]} outside [0, {cap}]")
    if len(bad) > 4:
        errs.append(f"... {len(bad)} context lengths outside [0, {cap}]")
    return errs


def block_errors(ctx_lens, block_table, block_size: int, n_blocks: int) -> List[str]:
    """Every block covering tokens [0, ctx_lens[b]) of a sequence has an id in
    [0, n_blocks)."""
    ctx = _host(ctx_lens).astype(np.int64)
    table = _host(block_table).astype(np.int64)
    errs = []
    for b, c in enumerate(ctx):
        need = min(-(-max(int(c), 0) // block_size), table.shape[1])
        ids = table[b, :need]
        bad = np.nonzero((ids < 0) | (ids >= n_blocks))[0]
        if len(bad):
            k = int(bad[0])
            errs.append(f"sequence {b}: block {k} (tokens {k * block_size}..{(k + 1) * block_size - 1}) "
                        f"has id {ids[k]}, outside [0, {n_blocks})")
        if len(errs) >= 4:
            break
    return errs


def position_errors(ctx_lens, positions) -> List[str]:
    """positions[b][j] == ctx_lens[b] - n_q + j."""
    ctx = _host(ctx_lens).astype(np.int64)
    pos = _host(positions).astype(np.int64)
    if pos.ndim != 2 or pos.shape[0] != ctx.shape[0]:
        return [f"positions must be [B][n_q] with B = {ctx.shape[0]}, got {pos.shape}"]
    n_q = pos.shape[1]
    want = ctx[:, None] - n_q + np.arange(n_q)[None, :]
    bad = np.argwhere(pos != want)
    errs = [f"positions[{b}][{j}] = {pos[b, j]}, the decode step puts it at {want[b, j]}"
            for b, j in bad[:4]]
    if len(bad) > 4:
        errs.append(f"... {len(bad)} positions off")
    return errs


def append_errors(seq_ids, positions, B: int, cap: int, block_table=None, block_size: int = 0,
                  n_blocks: int = 0) -> List[str]:
    seq = _host(seq_ids).astype(np.int64)
    pos = _host(positions).astype(np.int64)
    errs = []
    bad = np.nonzero((seq < 0) | (seq >= B))[0]
    if len(bad):
        errs.append(f"seq_ids[{bad[0]}] = {seq[bad[0]]} outside [0, {B})")
        return errs
    bad = np.nonzero((pos < 0) | (pos >= cap))[0]
    if len(bad):
        errs.append(f"positions[{bad[0]}] = {pos[bad[0]]} outside [0, {cap})")
        return errs
    if block_size:
        table = _host(block_table).astype(np.int64)
        ids = table[seq, pos // block_size]
        bad = np.nonzero((ids < 0) | (ids >= n_blocks))[0]
        if len(bad):
            k = int(bad[0])
            errs.append(f"new token {k} (sequence {seq[k]}, position {pos[k]}) goes to block id {ids[k]}, "
                        f"outside [0, {n_blocks})")
            return errs
        rows = ids * block_size + pos % block_size
    else:
        rows = seq * cap + pos
    uniq, counts = np.unique(rows, return_counts=True)
    if len(uniq) != len(rows):
        r = uniq[np.argmax(counts)]
        ks = np.nonzero(rows == r)[0][:2]
        errs.append(f"new tokens {ks[0]} and {ks[1]} are written to the same cache row")
    return errs


def _cache_shape(cache):
    """(block_size, max_blocks, s_max, n_blocks, B_cap) of a LatentCache."""
    if cache.block_size:
        return cache.block_size, int(cache.block_table.shape[1]), 0, int(cache.data.shape[0]), \
            int(cache.block_table.shape[0])
    return 0, 0, int(cache.data.shape[1]), 0, int(cache.data.shape[0])


def decode_errors(cache, positions: Optional[object] = None) -> List[str]:
    """Breaches of the decode contract by a LatentCache (and the queries'
    positions, when given)."""
    bs, mb, s_max, n_blocks, _ = _cache_shape(cache)
    errs = ctx_errors(cache.ctx_lens, capacity(bs, mb, s_max))
    if bs and not errs:
        errs += block_errors(cache.ctx_lens, cache.block_table, bs, n_blocks)
    if positions is not None:
        errs += position_errors(cache.ctx_lens, positions)
    return errs


def cache_append_errors(cache, seq_ids, positions) -> List[str]:
    bs, mb, s_max, n_blocks, b_cap = _cache_shape(cache)
    B = int(cache.ctx_lens.shape[0]) if cache.block_size else min(b_cap, int(cache.ctx_lens.shape[0]))
    return append_errors(seq_ids, positions, B, capacity(bs, mb, s_max), cache.block_table, bs, n_blocks)


def _raise(fn: str, errs: List[str]) -> None:
    if errs:
        raise ContractError(f"{fn}: " + "; ".join(errs))


def check_decode(cache, positions=None, fn: str = "mla_decode") -> None:
    _raise(fn, decode_errors(cache, positions))


def check_cache_append(cache, seq_ids, positions, fn: str = "mla_cache_append") -> None:
    _raise(fn, cache_append_errors(cache, seq_ids, positions))


def check_ctx_lens(ctx_lens, fn: str = "mla_combine") -> None:
    _raise(fn, ctx_errors(ctx_lens, np.iinfo(np.int32).max))
