"""Seeded synthetic inputs for MLA decode (weights, queries, latent cache).

This module holds no attention arithmetic: it only draws numbers and lays
them out.  It serves both sides of the parity tests: the fp64 oracle (via
the host functions here) and the HIP library (via the same host arrays, or
via ``fill_cache_rows_device`` for the multi-gigabyte caches, which runs the
identical generator on the GPU).

Generator
---------
Every value comes from Philox4x32-10 (Salmon, Moraes, Dror, Shaw,
"Parallel Random Numbers: As Easy as 1, 2, 3", SC'11), a counter-based
generator: output = Philox(counter, key), no state.  Each call yields four
32-bit words = eight 16-bit lanes; lane ``u`` (0..65535) selects a
quantile of the standard normal from a fixed table,

    z(u) = Phi^{-1}((u + 1/2) / 65536),

so draws are N(0, 1) quantised to 65536 equiprobable levels (|z| <= 4.33).
Tables are kept in fp32 and in bf16 (round-to-nearest-even of the fp32
value).  Because the map from (counter, key) to a stored value is integer
arithmetic plus a table lookup, the host (numpy) and device (HIP)
implementations give bit-identical values.

Counter layout: element ``e`` of row ``r`` of sequence ``b`` of a stream
uses counter (e // 8, r, b, 0) and key (seed, stream); lane e % 8 is the
low (even) or high (odd) half of word (e % 8) // 2.  Flat tensors use
row = 0, b = 0 and counter word 0 = flat_index // 8 (tensors here have
fewer than 2**35 elements).

Workloads
---------
The five decode workloads at DeepSeek-V3 shapes (n_h=128, d_c=512,
d_rope=64, d_nope=d_v=128) plus a tiny fp32 case.  Per-token positions
follow the convention that the query tokens' own latents are already in the
cache: query j of n_q sits at position ctx - n_q + j.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from statistics import NormalDist
from typing import Optional

import numpy as np

# ----------------------------------------------------------------- streams
STREAM_W_UK = 1
STREAM_W_UV = 2
STREAM_W_UQ = 3
STREAM_HIDDEN = 4
STREAM_Q_NOPE = 5
STREAM_Q_ROPE = 6
STREAM_CACHE = 7  # raw cache rows: [c_kv (d_c) | k_rope before rotation (d_rope)]

_PHILOX_M0 = np.uint64(0xD2511F53)
_PHILOX_M1 = np.uint64(0xCD9E8D57)
_PHILOX_W0 = 0x9E3779B9
_PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32 with 10 rounds on arrays of counters; returns 4 uint32 arrays."""
    c0 = np.asarray(c0, dtype=np.uint64)
    c1 = np.asarray(c1, dtype=np.uint64)
    c2 = np.asarray(c2, dtype=np.uint64)
    c3 = np.asarray(c3, dtype=np.uint64)
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    c0, c1, c2, c3 = (x.copy() for x in (c0, c1, c2, c3))
    key0, key1 = k0 & 0xFFFFFFFF, k1 & 0xFFFFFFFF
    for rnd in range(10):
        if rnd:
            key0 = (key0 + _PHILOX_W0) & 0xFFFFFFFF
            key1 = (key1 + _PHILOX_W1) & 0xFFFFFFFF
        p0 = _PHILOX_M0 * c0
        p1 = _PHILOX_M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(key0), lo1,
                          hi0 ^ c3 ^ np.uint64(key1), lo0)
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bit pattern (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 (returned as fp32)."""
    return bf16_bits_to_f32(_f32_to_bf16_bits(x))


_TABLES = {}


def normal_table_f32() -> np.ndarray:
    if "f32" not in _TABLES:
        nd = NormalDist()
        z = np.array([nd.inv_cdf((k + 0.5) / 65536.0) for k in range(65536)], dtype=np.float64)
        _TABLES["f32"] = z.astype(np.float32)
    return _TABLES["f32"]


def normal_table_bf16_bits() -> np.ndarray:
    if "bf16" not in _TABLES:
        _TABLES["bf16"] = _f32_to_bf16_bits(normal_table_f32())
    return _TABLES["bf16"]


def _lanes(n_elems: int, row: np.ndarray, seq: np.ndarray, seed: int, stream: int) -> np.ndarray:
    """16-bit lanes for elements 0..n_elems-1 of each (row, seq) pair.

    ``row`` and ``seq`` are broadcast-compatible integer arrays; the result has
    shape row.shape + (n_elems,).
    """
    n_blk = (n_elems + 7) // 8
    row = np.asarray(row, dtype=np.uint64)[..., None]
    seq = np.asarray(seq, dtype=np.uint64)[..., None]
    blk = np.arange(n_blk, dtype=np.uint64)
    w = philox4x32_10(blk, row, seq, np.uint64(0), seed, stream)
    words = np.stack(w, axis=-1)  # [..., n_blk, 4]
    lo = (words & np.uint32(0xFFFF)).astype(np.uint16)
    hi = (words >> np.uint32(16)).astype(np.uint16)
    lanes = np.stack([lo, hi], axis=-1).reshape(words.shape[:-2] + (n_blk * 8,))
    return lanes[..., :n_elems]


def standard_normal_flat(n: int, seed: int, stream: int, dtype: str = "f32") -> np.ndarray:
    """n N(0,1) draws of a flat tensor (counter word 0 = index // 8)."""
    n_blk = (n + 7) // 8
    blk = np.arange(n_blk, dtype=np.uint64)
    w = philox4x32_10(blk & _MASK32, blk >> np.uint64(32), np.uint64(0), np.uint64(0), seed, stream)
    words = np.stack(w, axis=-1)
    lanes = np.stack([(words & np.uint32(0xFFFF)).astype(np.uint16),
                      (words >> np.uint32(16)).astype(np.uint16)], axis=-1).reshape(-1)[:n]
    return normal_table_f32()[lanes]


# --------------------------------------------------------------- workloads
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    n_q: int
    n_h: int
    d_c: int
    d_rope: int
    d_nope: int
    d_v: int
    dtype: str            # "f32" or "bf16": storage type of cache, queries, weights
    ctx: Optional[int]    # fixed context, or None for a ragged batch
    ctx_range: Optional[tuple] = None  # inclusive (lo, hi) for ragged batches
    block_size: int = 0   # 0 = contiguous cache, else tokens per paged block
    d_q: Optional[int] = None  # hidden size when queries come from h @ W_UQ
    rope_base: float = 10000.0
    description: str = ""
    cache: str = ""       # cache storage: "" = dtype; "fp8" = e4m3 codes with per-tile scales (bf16 inputs)

    @property
    def row(self) -> int:
        return self.d_c + self.d_rope

    @property
    def cache_dtype(self) -> str:
        return self.cache or self.dtype

    @property
    def cache_row_bytes(self) -> int:
        """Bytes of one cache row: fp8 rows are [d_c codes | d_rope bf16 | d_c/128 fp32 scales]."""
        if self.cache_dtype == "fp8":
            return self.d_c + 2 * self.d_rope + 4 * (self.d_c // 128)
        return self.row * (2 if self.dtype == "bf16" else 4)

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d_nope + self.d_rope))


WORKLOADS = {
    "tiny_fp32": Workload(
        "tiny_fp32", seed=1, batch=1, n_q=1, n_h=4, d_c=64, d_rope=16, d_nope=32, d_v=32,
        dtype="f32", ctx=256, d_q=64,
        description="tiny fp32 decode: B=1, n_h=4, d_c=64, d_rope=16, d_nope=d_v=32, ctx 256"),
    "v3_b1": Workload(
        "v3_b1", seed=2, batch=1, n_q=1, n_h=128, d_c=512, d_rope=64, d_nope=128, d_v=128,
        dtype="bf16", ctx=4096,
        description="DeepSeek-V3 shapes, B=1, ctx 4096, bf16 contiguous latent cache"),
    "v3_b64": Workload(
        "v3_b64", seed=3, batch=64, n_q=1, n_h=128, d_c=512, d_rope=64, d_nope=128, d_v=128,
        dtype="bf16", ctx=8192,
        description="DeepSeek-V3 shapes, B=64, ctx 8192 each, bf16 contiguous latent cache"),
    "v3_paged": Workload(
        "v3_paged", seed=4, batch=128, n_q=1, n_h=128, d_c=512, d_rope=64, d_nope=128, d_v=128,
        dtype="bf16", ctx=None, ctx_range=(1024, 32768), block_size=64,
        description="DeepSeek-V3 shapes, B=128, ctx ~ U{1024..32768}, paged cache, block 64"),
    "v3_split": Workload(
        "v3_split", seed=5, batch=4, n_q=2, n_h=128, d_c=512, d_rope=64, d_nope=128, d_v=128,
        dtype="bf16", ctx=131072,
        description="DeepSeek-V3 shapes, B=4, ctx 131072, 2 query tokens, split-KV"),
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def with_fp8_cache(w: Workload) -> Workload:
    """The same workload over an fp8 e4m3 latent cache (bf16 queries and weights)."""
    if w.dtype != "bf16":
        raise ValueError("fp8 caches go with bf16 queries and weights")
    return dataclasses.replace(w, name=w.name + "_fp8", cache="fp8",
                               description=w.description + ", fp8 e4m3 cache with per-128-channel scales")


def custom(**kw) -> Workload:
    """A workload with explicit fields (for small parity cases)."""
    base = dict(name="custom", seed=11, batch=1, n_q=1, n_h=128, d_c=512, d_rope=64,
                d_nope=128, d_v=128, dtype="bf16", ctx=256)
    base.update(kw)
    return Workload(**base)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    """Values as stored (fp32 array holding bf16-representable values for bf16)."""
    return round_to_bf16(x) if dtype == "bf16" else x.astype(np.float32)


def context_lengths(w: Workload) -> np.ndarray:
    if w.ctx is not None:
        return np.full(w.batch, w.ctx, dtype=np.int32)
    lo, hi = w.ctx_range
    rng = np.random.default_rng([w.seed, 0xC7])
    return rng.integers(lo, hi + 1, size=w.batch, dtype=np.int64).astype(np.int32)


def positions(w: Workload, ctx: Optional[np.ndarray] = None) -> np.ndarray:
    """[B][n_q] positions of the query tokens (their latents are the last n_q cached)."""
    ctx = context_lengths(w) if ctx is None else ctx
    return (ctx[:, None] - w.n_q + np.arange(w.n_q, dtype=np.int32)[None, :]).astype(np.int32)


def block_table(w: Workload, ctx: Optional[np.ndarray] = None):
    """(table [B][max_blocks] int32, n_blocks): sequences take consecutive
    entries of a seeded random permutation of the physical blocks; unused
    table entries are -1."""
    assert w.block_size > 0
    ctx = context_lengths(w) if ctx is None else ctx
    nb = (ctx.astype(np.int64) + w.block_size - 1) // w.block_size
    n_blocks = int(nb.sum())
    perm = np.random.default_rng([w.seed, 0xB7]).permutation(n_blocks).astype(np.int32)
    max_blocks = int(nb.max())
    table = np.full((w.batch, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(w.batch):
        table[b, :nb[b]] = perm[off:off + nb[b]]
        off += nb[b]
    return table, n_blocks


def weights(w: Workload) -> dict:
    """W_UK [n_h][d_c][d_nope] and W_UV [n_h][d_c][d_v], N(0, 1/d_c) (fan-in d_c)."""
    s = np.float32(1.0 / np.sqrt(w.d_c))
    wuk = standard_normal_flat(w.n_h * w.d_c * w.d_nope, w.seed, STREAM_W_UK) * s
    wuv = standard_normal_flat(w.n_h * w.d_c * w.d_v, w.seed, STREAM_W_UV) * s
    return {
        "w_uk": _store(wuk.reshape(w.n_h, w.d_c, w.d_nope), w.dtype),
        "w_uv": _store(wuv.reshape(w.n_h, w.d_c, w.d_v), w.dtype),
    }


def queries(w: Workload) -> dict:
    """q_nope [B][n_q][n_h][d_nope] and q_rope [B][n_q][n_h][d_rope] (before RoPE).

    With ``d_q`` set, the query is synthesised as h @ W_UQ with h ~ N(0,1) of
    width d_q and W_UQ ~ N(0, 1/d_q) of shape [d_q][n_h*(d_nope+d_rope)]; each
    head's slice is [q_nope | q_rope].  Otherwise both parts are N(0,1) draws.
    """
    B, nq, nh = w.batch, w.n_q, w.n_h
    if w.d_q:
        dh = w.d_nope + w.d_rope
        h = standard_normal_flat(B * nq * w.d_q, w.seed, STREAM_HIDDEN).astype(np.float64)
        wuq = standard_normal_flat(w.d_q * nh * dh, w.seed, STREAM_W_UQ).astype(np.float64)
        wuq *= 1.0 / np.sqrt(w.d_q)
        q = (h.reshape(B * nq, w.d_q) @ wuq.reshape(w.d_q, nh * dh)).reshape(B, nq, nh, dh)
        q = q.astype(np.float32)
        return {"q_nope": _store(q[..., :w.d_nope], w.dtype),
                "q_rope": _store(q[..., w.d_nope:], w.dtype)}
    qn = standard_normal_flat(B * nq * nh * w.d_nope, w.seed, STREAM_Q_NOPE)
    qr = standard_normal_flat(B * nq * nh * w.d_rope, w.seed, STREAM_Q_ROPE)
    return {"q_nope": _store(qn.reshape(B, nq, nh, w.d_nope), w.dtype),
            "q_rope": _store(qr.reshape(B, nq, nh, w.d_rope), w.dtype)}


def cache_rows(w: Workload, b: int, t0: int = 0, t1: Optional[int] = None) -> dict:
    """Raw cache rows of sequence b for tokens t0..t1-1 (host).

    Returns c_kv [n][d_c] and k_rope_raw [n][d_rope] (the positional key before
    its rotation), as stored values in fp32 arrays.
    """
    if t1 is None:
        t1 = int(context_lengths(w)[b])
    rows = np.arange(t0, t1, dtype=np.int64)
    lanes = _lanes(w.row, rows, np.int64(b), w.seed, STREAM_CACHE)
    if w.dtype == "bf16":
        vals = bf16_bits_to_f32(normal_table_bf16_bits()[lanes])
    else:
        vals = normal_table_f32()[lanes]
    return {"c_kv": vals[:, :w.d_c], "k_rope_raw": vals[:, w.d_c:]}


# ------------------------------------------------------- device generator
_SYNTH_LIB = None
_HERE = os.path.dirname(os.path.abspath(__file__))
SYNTH_LIB_PATH = os.path.join(_HERE, "libmla_synth.so")


def _synth_lib():
    global _SYNTH_LIB
    if _SYNTH_LIB is None:
        if not os.path.exists(SYNTH_LIB_PATH):
            raise RuntimeError(f"{SYNTH_LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(SYNTH_LIB_PATH)
        lib.synth_fill_cache_rows.restype = ctypes.c_int
        lib.synth_fill_cache_rows.argtypes = [
            ctypes.c_uint32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_void_p]
        lib.synth_error_name.restype = ctypes.c_char_p
        lib.synth_error_name.argtypes = [ctypes.c_int]
        _SYNTH_LIB = lib
    return _SYNTH_LIB


def fill_cache_rows_device(w: Workload, seq_ids_dev: int, tok_dev: int, n_tokens: int,
                           table_dev: int, out_dev: int, stream: int = 0) -> None:
    """Generate raw cache rows on the GPU for a token list.

    Token k of the list is token ``tok[k]`` of sequence ``seq_ids[k]``; its
    row of d_c + d_rope bf16 values (identical to ``cache_rows``) is written
    to out[k][:].  ``table_dev`` is the device copy of
    ``normal_table_bf16_bits()``.  Pointers are raw device addresses.
    """
    assert w.dtype == "bf16"
    rc = _synth_lib().synth_fill_cache_rows(
        ctypes.c_uint32(w.seed), ctypes.c_int32(STREAM_CACHE), ctypes.c_int32(w.row),
        ctypes.c_int32(n_tokens), ctypes.c_void_p(seq_ids_dev), ctypes.c_void_p(tok_dev),
        ctypes.c_void_p(table_dev), ctypes.c_void_p(out_dev), ctypes.c_void_p(stream))
    if rc == -1:
        raise ValueError("synth_fill_cache_rows: invalid argument")
    if rc != 0:
        name = _synth_lib().synth_error_name(rc).decode()
        raise RuntimeError(f"synth_fill_cache_rows: launch failed with {name} ({rc})")
