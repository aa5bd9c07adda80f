"""ctypes binding of libmla.so (include/mla.h): argument marshalling only.

Every function takes torch device tensors, checks that their shapes, dtypes
and placement match the C declaration, and passes raw device pointers and the
current HIP stream to the library.  No step of the computation runs here.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree build; MLA_LIBRARY names another build of the same ABI (for
# comparing kernel variants).  Either way the HIP library is required.
LIB_PATH = os.environ.get("MLA_LIBRARY") or os.path.join(HERE, "libmla.so")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_HIP, MLA_ERR_OUT_OF_BLOCKS, MLA_ERR_TOO_LARGE = 0, 1, 2, 3, 4, 5
NOALLOC_SCRATCH_BYTES = 128 << 20     # MLA_NOALLOC_SCRATCH_BYTES
F32, BF16, FP8_E4M3 = 0, 1, 2

EXPORTED = ("mla_absorb_q", "mla_decode", "mla_combine", "mla_out_proj", "mla_combine_out_proj",
            "mla_cache_append", "mla_append_absorb_q", "mla_num_partials", "mla_cache_row_bytes",
            "mla_status_string", "mla_version", "mla_last_hip_error", "mla_hip_error_name",
            "mla_decode_out_noalloc",
            "mla_block_pool_bytes", "mla_block_pool_init", "mla_block_pool_reserve", "mla_block_pool_reserve_all",
            "mla_block_pool_release", "mla_fold_out", "mla_out_proj_folded", "mla_o_proj", "mla_fold_q",
            "mla_absorb_q_folded", "mla_prefill_weights", "mla_prefill_workspace_bytes", "mla_prefill",
            "mla_block_pool_table", "mla_block_pool_free_count")


class MlaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


class _Dims(ctypes.Structure):
    _fields_ = [("n_h", ctypes.c_int32), ("d_c", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("d_nope", ctypes.c_int32), ("d_v", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("rope_base", ctypes.c_float)]


class _Cache(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("data", ctypes.c_void_p), ("seq_stride", ctypes.c_int64),
                ("block_size", ctypes.c_int32), ("block_table", ctypes.c_void_p),
                ("max_blocks", ctypes.c_int32), ("ctx_lens", ctypes.c_void_p)]


_LIB = None


def load_library(path: str = LIB_PATH):
    """Load libmla.so; raises if it has not been built (there is no fallback)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -m mla_latent_kv_02_amd.build` "
                           "(the HIP library is required; there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    P, I32, I64, V = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    DP, CP = ctypes.POINTER(_Dims), ctypes.POINTER(_Cache)
    sig = {
        "mla_absorb_q": [DP, I32, I32, ctypes.c_int, P, P, P, P, P, P, V],
        "mla_decode": [DP, I32, I32, P, P, CP, P, I32, P, P, V],
        "mla_combine": [DP, I32, I32, P, I32, P, P, P, P, V],
        "mla_out_proj": [DP, I32, I32, P, ctypes.c_int, P, P, V],
        "mla_combine_out_proj": [DP, I32, I32, P, I32, P, P, ctypes.c_int, P, P, P, V],
        "mla_decode_out_noalloc": [DP, I32, I32, P, P, CP, P, I32, ctypes.c_int, P, P, P, V],
        "mla_cache_append": [DP, CP, I32, P, P, P, I64, P, I64, V],
        "mla_append_absorb_q": [DP, CP, I32, P, P, P, I64, P, I64, I32, I32, ctypes.c_int, P, P, P, P, P, P, V],
        "mla_fold_out": [DP, I32, P, P, P, V],
        "mla_out_proj_folded": [DP, I32, I32, I32, P, P, P, V],
        "mla_o_proj": [DP, I32, I32, I32, P, P, P, V],
        "mla_fold_q": [DP, I32, P, P, P, V],
        "mla_absorb_q_folded": [DP, I32, I32, I32, P, P, P, P, P, P, V],
        "mla_prefill_weights": [DP, P, P, P, V],
        "mla_prefill": [DP, I32, I32, I32, P, P, P, CP, P, P, I64, P, P, P, V],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    for name, args in (("mla_block_pool_init", [P, I64, I32, I32, I32, I32]),
                       ("mla_block_pool_reserve", [P, I32, I32]), ("mla_block_pool_reserve_all", [P, P]),
                       ("mla_block_pool_release", [P, I32])):
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.mla_block_pool_bytes.argtypes = [I32, I32, I32]
    lib.mla_block_pool_bytes.restype = ctypes.c_int64
    lib.mla_block_pool_table.argtypes = [P]
    lib.mla_block_pool_table.restype = ctypes.POINTER(ctypes.c_int32)
    lib.mla_block_pool_free_count.argtypes = [P]
    lib.mla_block_pool_free_count.restype = ctypes.c_int32
    lib.mla_num_partials.argtypes = [I32, I32]
    lib.mla_num_partials.restype = ctypes.c_int64
    lib.mla_prefill_workspace_bytes.argtypes = [DP, I32, I32]
    lib.mla_prefill_workspace_bytes.restype = ctypes.c_int64
    lib.mla_cache_row_bytes.argtypes = [DP, ctypes.c_int]
    lib.mla_cache_row_bytes.restype = ctypes.c_int64
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_version.restype = ctypes.c_char_p
    lib.mla_last_hip_error.restype = ctypes.c_int32
    lib.mla_hip_error_name.argtypes = [ctypes.c_int32]
    lib.mla_hip_error_name.restype = ctypes.c_char_p
    _LIB = lib
    return lib


@dataclasses.dataclass(frozen=True)
class Dims:
    n_h: int
    d_c: int
    d_rope: int
    d_nope: int
    d_v: int
    sm_scale: float = 0.0      # 0 -> 1/sqrt(d_nope + d_rope)
    rope_base: float = 0.0     # 0 -> 10000

    def _c(self) -> _Dims:
        return _Dims(self.n_h, self.d_c, self.d_rope, self.d_nope, self.d_v, self.sm_scale, self.rope_base)


@dataclasses.dataclass
class LatentCache:
    """Device latent cache: ``data`` is [B][S_max][row] (contiguous) or
    [n_blocks][block_size][row] (paged, with ``block_table`` [B][max_blocks]);
    ``ctx_lens`` [B] int32.  fp32 / bf16 rows hold d_c + d_rope elements; a
    uint8 ``data`` tensor is an fp8 e4m3 cache whose rows are
    mla_cache_row_bytes(dims, FP8_E4M3) bytes (codes | bf16 key | fp32 scales)."""
    data: "torch.Tensor"
    ctx_lens: "torch.Tensor"
    block_table: Optional["torch.Tensor"] = None
    block_size: int = 0

    @property
    def fp8(self) -> bool:
        return self.data.dtype == _torch().uint8

    @property
    def query_dtype(self):
        """dtype of the queries, new rows and q_lat / q_pe that go with this cache."""
        return _torch().bfloat16 if self.fp8 else self.data.dtype

    def row_width(self, dims: "Dims") -> int:
        """Last dimension ``data`` must have for ``dims``."""
        if self.fp8:
            return mla_cache_row_bytes(dims, FP8_E4M3)
        return dims.d_c + dims.d_rope

    def _c(self) -> _Cache:
        _dev(self.data, "cache.data")
        _dev(self.ctx_lens, "cache.ctx_lens", _torch().int32)
        if self.block_size:
            if self.block_table is None:
                raise ValueError("paged cache needs block_table")
            _dev(self.block_table, "cache.block_table", _torch().int32)
            if self.data.dim() != 3 or self.data.shape[1] != self.block_size:
                raise ValueError("paged cache data must be [n_blocks][block_size][row]")
            return _Cache(_cache_dtype(self.data), self.data.data_ptr(), 0, self.block_size,
                          self.block_table.data_ptr(), self.block_table.shape[1], self.ctx_lens.data_ptr())
        if self.data.dim() != 3:
            raise ValueError("contiguous cache data must be [B][S_max][row]")
        return _Cache(_cache_dtype(self.data), self.data.data_ptr(), self.data.stride(0), 0, None, 0,
                      self.ctx_lens.data_ptr())


def _torch():
    import torch
    return torch


def _dtype(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _cache_dtype(t) -> int:
    return FP8_E4M3 if t.dtype == _torch().uint8 else _dtype(t)


def mla_cache_row_bytes(dims: "Dims", dtype: int) -> int:
    """Bytes of one cache row (mla_cache_row_bytes); raises for an invalid pair."""
    d = dims._c()
    n = int(load_library().mla_cache_row_bytes(ctypes.byref(d), dtype))
    if n < 0:
        raise ValueError(f"no cache row of dtype {dtype} for {dims}")
    return n


def _dev(t, name, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _shape(t, name, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _contract(check: str, *args, fn: str) -> None:
    """With MLA_CHECK_CONTRACT=1, copy the device-side arguments the library
    trusts (context lengths, positions, block ids, append targets) to the host
    and check them before the call (contract.py); off by default."""
    if os.environ.get("MLA_CHECK_CONTRACT") != "1":
        return
    cuda = _torch().cuda
    if cuda.is_initialized() and cuda.is_current_stream_capturing():
        return      # no host copy inside a graph capture; the eager calls before it are checked
    from . import contract
    getattr(contract, check)(*args, fn=fn)


def _check(fn: str, status: int):
    if status != MLA_OK:
        lib = load_library()
        msg = lib.mla_status_string(status).decode()
        if status == MLA_ERR_HIP:   # name the HIP error behind it
            code = lib.mla_last_hip_error()
            msg += f": {lib.mla_hip_error_name(code).decode()} ({code})"
        raise MlaError(fn, status, msg)


def mla_num_partials(B: int, num_splits: int) -> int:
    return int(load_library().mla_num_partials(B, num_splits))


def _absorb_checks(dims: Dims, q_nope, q_rope, positions, w_uk, q_lat, q_pe):
    B, n_q = q_nope.shape[0], q_nope.shape[1]
    for t, n in ((q_nope, "q_nope"), (q_rope, "q_rope"), (w_uk, "w_uk"), (q_lat, "q_lat"), (q_pe, "q_pe")):
        _dev(t, n, q_nope.dtype)
    _dev(positions, "positions", _torch().int32)
    _shape(q_nope, "q_nope", (B, n_q, dims.n_h, dims.d_nope))
    _shape(q_rope, "q_rope", (B, n_q, dims.n_h, dims.d_rope))
    _shape(positions, "positions", (B, n_q))
    _shape(w_uk, "w_uk", (dims.n_h, dims.d_c, dims.d_nope))
    _shape(q_lat, "q_lat", (B, n_q, dims.n_h, dims.d_c))
    _shape(q_pe, "q_pe", (B, n_q, dims.n_h, dims.d_rope))
    return B, n_q


def mla_absorb_q(dims: Dims, q_nope, q_rope, positions, w_uk, q_lat, q_pe, stream=None) -> None:
    B, n_q = _absorb_checks(dims, q_nope, q_rope, positions, w_uk, q_lat, q_pe)
    dt = _dtype(q_nope)
    d = dims._c()
    _check("mla_absorb_q", load_library().mla_absorb_q(
        ctypes.byref(d), B, n_q, dt, q_nope.data_ptr(), q_rope.data_ptr(), positions.data_ptr(),
        w_uk.data_ptr(), q_lat.data_ptr(), q_pe.data_ptr(), _stream(stream)))


def mla_decode(dims: Dims, q_lat, q_pe, cache: LatentCache, positions, num_splits: int,
               u_part, lse_part, stream=None) -> None:
    B, n_q = q_lat.shape[0], q_lat.shape[1]
    torch = _torch()
    _dev(q_lat, "q_lat", cache.query_dtype)
    _dev(q_pe, "q_pe", cache.query_dtype)
    _dev(positions, "positions", torch.int32)
    _dev(u_part, "u_part", torch.float32)
    _dev(lse_part, "lse_part", torch.float32)
    _shape(q_lat, "q_lat", (B, n_q, dims.n_h, dims.d_c))
    _shape(q_pe, "q_pe", (B, n_q, dims.n_h, dims.d_rope))
    _shape(positions, "positions", (B, n_q))
    _shape(cache.ctx_lens, "cache.ctx_lens", (B,))
    if cache.data.shape[-1] != cache.row_width(dims):
        raise ValueError(f"cache rows must be {cache.row_width(dims)} wide")
    if cache.block_size == 0 and cache.data.shape[0] < B:
        raise ValueError("contiguous cache holds fewer sequences than B")
    slots = mla_num_partials(B, num_splits)
    _shape(u_part, "u_part", (slots, n_q, dims.n_h, dims.d_c))
    _shape(lse_part, "lse_part", (slots, n_q, dims.n_h, 2))
    d, c = dims._c(), cache._c()
    _contract("check_decode", cache, positions, fn="mla_decode")
    _check("mla_decode", load_library().mla_decode(
        ctypes.byref(d), B, n_q, q_lat.data_ptr(), q_pe.data_ptr(), ctypes.byref(c),
        positions.data_ptr(), num_splits, u_part.data_ptr(), lse_part.data_ptr(), _stream(stream)))


def mla_combine(dims: Dims, ctx_lens, num_splits: int, u_part, lse_part, u, lse=None, stream=None) -> None:
    torch = _torch()
    B, n_q = u.shape[0], u.shape[1]
    _dev(ctx_lens, "ctx_lens", torch.int32)
    for t, n in ((u_part, "u_part"), (lse_part, "lse_part"), (u, "u")):
        _dev(t, n, torch.float32)
    slots = mla_num_partials(B, num_splits)
    _shape(ctx_lens, "ctx_lens", (B,))
    _shape(u_part, "u_part", (slots, n_q, dims.n_h, dims.d_c))
    _shape(lse_part, "lse_part", (slots, n_q, dims.n_h, 2))
    _shape(u, "u", (B, n_q, dims.n_h, dims.d_c))
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        _shape(lse, "lse", (B, n_q, dims.n_h))
    d = dims._c()
    _contract("check_ctx_lens", ctx_lens, fn="mla_combine")
    _check("mla_combine", load_library().mla_combine(
        ctypes.byref(d), B, n_q, ctx_lens.data_ptr(), num_splits, u_part.data_ptr(), lse_part.data_ptr(),
        u.data_ptr(), None if lse is None else lse.data_ptr(), _stream(stream)))


def mla_out_proj(dims: Dims, u, w_uv, out, stream=None) -> None:
    torch = _torch()
    B, n_q = u.shape[0], u.shape[1]
    _dev(u, "u", torch.float32)
    _dev(w_uv, "w_uv")
    _dev(out, "out", torch.float32)
    _shape(u, "u", (B, n_q, dims.n_h, dims.d_c))
    _shape(w_uv, "w_uv", (dims.n_h, dims.d_c, dims.d_v))
    _shape(out, "out", (B, n_q, dims.n_h, dims.d_v))
    d = dims._c()
    _check("mla_out_proj", load_library().mla_out_proj(
        ctypes.byref(d), B, n_q, u.data_ptr(), _dtype(w_uv), w_uv.data_ptr(), out.data_ptr(), _stream(stream)))


def mla_combine_out_proj(dims: Dims, ctx_lens, num_splits: int, u_part, lse_part, w_uv, out, lse=None,
                         stream=None) -> None:
    torch = _torch()
    B, n_q = out.shape[0], out.shape[1]
    _dev(ctx_lens, "ctx_lens", torch.int32)
    for t, n in ((u_part, "u_part"), (lse_part, "lse_part"), (out, "out")):
        _dev(t, n, torch.float32)
    _dev(w_uv, "w_uv")
    slots = mla_num_partials(B, num_splits)
    _shape(ctx_lens, "ctx_lens", (B,))
    _shape(u_part, "u_part", (slots, n_q, dims.n_h, dims.d_c))
    _shape(lse_part, "lse_part", (slots, n_q, dims.n_h, 2))
    _shape(w_uv, "w_uv", (dims.n_h, dims.d_c, dims.d_v))
    _shape(out, "out", (B, n_q, dims.n_h, dims.d_v))
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        _shape(lse, "lse", (B, n_q, dims.n_h))
    d = dims._c()
    _contract("check_ctx_lens", ctx_lens, fn="mla_combine_out_proj")
    _check("mla_combine_out_proj", load_library().mla_combine_out_proj(
        ctypes.byref(d), B, n_q, ctx_lens.data_ptr(), num_splits, u_part.data_ptr(), lse_part.data_ptr(),
        _dtype(w_uv), w_uv.data_ptr(), out.data_ptr(), None if lse is None else lse.data_ptr(), _stream(stream)))


def mla_decode_out_noalloc(dims: Dims, q_lat, q_pe, cache: LatentCache, positions, num_splits: int, w_uv, out,
                           lse=None, stream=None) -> None:
    """mla_decode then mla_combine_out_proj with the partials in the
    library's own per-GPU scratch (no buffer of the caller's, no allocation)."""
    B, n_q = q_lat.shape[0], q_lat.shape[1]
    torch = _torch()
    _dev(q_lat, "q_lat", cache.query_dtype)
    _dev(q_pe, "q_pe", cache.query_dtype)
    _dev(positions, "positions", torch.int32)
    _dev(out, "out", torch.float32)
    _dev(w_uv, "w_uv")
    _shape(q_lat, "q_lat", (B, n_q, dims.n_h, dims.d_c))
    _shape(q_pe, "q_pe", (B, n_q, dims.n_h, dims.d_rope))
    _shape(positions, "positions", (B, n_q))
    _shape(cache.ctx_lens, "cache.ctx_lens", (B,))
    _shape(w_uv, "w_uv", (dims.n_h, dims.d_c, dims.d_v))
    _shape(out, "out", (B, n_q, dims.n_h, dims.d_v))
    if cache.data.shape[-1] != cache.row_width(dims):
        raise ValueError(f"cache rows must be {cache.row_width(dims)} wide")
    if cache.block_size == 0 and cache.data.shape[0] < B:
        raise ValueError("contiguous cache holds fewer sequences than B")
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        _shape(lse, "lse", (B, n_q, dims.n_h))
    d, c = dims._c(), cache._c()
    _contract("check_decode", cache, positions, fn="mla_decode_out_noalloc")
    _check("mla_decode_out_noalloc", load_library().mla_decode_out_noalloc(
        ctypes.byref(d), B, n_q, q_lat.data_ptr(), q_pe.data_ptr(), ctypes.byref(c), positions.data_ptr(),
        num_splits, _dtype(w_uv), w_uv.data_ptr(), out.data_ptr(), None if lse is None else lse.data_ptr(),
        _stream(stream)))


def mla_cache_append(dims: Dims, cache: LatentCache, seq_ids, positions, c_kv_new, k_rope_new,
                     stream=None) -> None:
    """c_kv_new [n][>= d_c] and k_rope_new [n][>= d_rope] (row strides taken from
    the tensors, so both may be column slices of one [n][d_c + d_rope] array)."""
    n = _append_checks(dims, cache, seq_ids, positions, c_kv_new, k_rope_new)
    d, c = dims._c(), cache._c()
    _contract("check_cache_append", cache, seq_ids, positions, fn="mla_cache_append")
    _check("mla_cache_append", load_library().mla_cache_append(
        ctypes.byref(d), ctypes.byref(c), n, seq_ids.data_ptr(), positions.data_ptr(),
        c_kv_new.data_ptr(), c_kv_new.stride(0), k_rope_new.data_ptr(), k_rope_new.stride(0),
        _stream(stream)))


def mla_append_absorb_q(dims: Dims, cache: LatentCache, seq_ids, new_positions, c_kv_new, k_rope_new,
                        q_nope, q_rope, positions, w_uk, q_lat, q_pe, stream=None) -> None:
    """mla_cache_append(cache, seq_ids, new_positions, c_kv_new, k_rope_new) then
    mla_absorb_q(q_nope, q_rope, positions, w_uk, q_lat, q_pe), in one launch
    where the library has the fused kernel."""
    n = _append_checks(dims, cache, seq_ids, new_positions, c_kv_new, k_rope_new)
    B, n_q = _absorb_checks(dims, q_nope, q_rope, positions, w_uk, q_lat, q_pe)
    d, c = dims._c(), cache._c()
    _contract("check_cache_append", cache, seq_ids, new_positions, fn="mla_append_absorb_q")
    _check("mla_append_absorb_q", load_library().mla_append_absorb_q(
        ctypes.byref(d), ctypes.byref(c), n, seq_ids.data_ptr(), new_positions.data_ptr(),
        c_kv_new.data_ptr(), c_kv_new.stride(0), k_rope_new.data_ptr(), k_rope_new.stride(0),
        B, n_q, _dtype(q_nope), q_nope.data_ptr(), q_rope.data_ptr(), positions.data_ptr(),
        w_uk.data_ptr(), q_lat.data_ptr(), q_pe.data_ptr(), _stream(stream)))


def _append_checks(dims: Dims, cache: LatentCache, seq_ids, positions, c_kv_new, k_rope_new) -> int:
    torch = _torch()
    n = seq_ids.shape[0]
    _dev(seq_ids, "seq_ids", torch.int32)
    _dev(positions, "positions", torch.int32)
    _shape(positions, "positions", (n,))
    for t, name in ((c_kv_new, "c_kv_new"), (k_rope_new, "k_rope_new")):
        if not t.is_cuda or t.dtype != cache.query_dtype or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name} must be a [n][width] device tensor of dtype {cache.query_dtype} "
                             "with unit column stride")
        if t.shape[0] != n:
            raise ValueError(f"{name} must have {n} rows")
    if c_kv_new.shape[1] != dims.d_c or k_rope_new.shape[1] != dims.d_rope:
        raise ValueError("c_kv_new / k_rope_new widths must be d_c / d_rope")
    return n


class BlockPool:
    """The library's block pool of a paged cache (mla_block_pool_*), in a host
    buffer this object owns.  ``table`` is a NumPy view of the pool's host
    block table [B][max_blocks] (-1 past a sequence's blocks)."""

    def __init__(self, n_blocks: int, block_size: int, B: int, max_blocks: int):
        import numpy as np
        lib = load_library()
        nbytes = lib.mla_block_pool_bytes(n_blocks, B, max_blocks)
        if nbytes < 0:
            raise ValueError("invalid block pool shape")
        self._buf = np.zeros((nbytes + 3) // 4, dtype=np.int32)
        self._ptr = self._buf.ctypes.data_as(ctypes.c_void_p)
        _check("mla_block_pool_init", lib.mla_block_pool_init(self._ptr, nbytes, n_blocks, block_size, B,
                                                              max_blocks))
        self.n_blocks, self.block_size, self.B, self.max_blocks = n_blocks, block_size, B, max_blocks
        self.table = np.ctypeslib.as_array(lib.mla_block_pool_table(self._ptr), shape=(B, max_blocks))

    def reserve(self, b: int, n_tokens: int) -> None:
        _check("mla_block_pool_reserve", load_library().mla_block_pool_reserve(self._ptr, b, n_tokens))

    def reserve_all(self, n_tokens) -> None:
        """n_tokens: int32 array of B entries (negative = leave that sequence)."""
        import numpy as np
        n = np.ascontiguousarray(n_tokens, dtype=np.int32)
        if n.shape != (self.B,):
            raise ValueError(f"n_tokens must have {self.B} entries")
        _check("mla_block_pool_reserve_all", load_library().mla_block_pool_reserve_all(
            self._ptr, n.ctypes.data_as(ctypes.c_void_p)))

    def release(self, b: int) -> None:
        _check("mla_block_pool_release", load_library().mla_block_pool_release(self._ptr, b))

    @property
    def free_count(self) -> int:
        return load_library().mla_block_pool_free_count(self._ptr)


# ---- weight folds (mla_fold_out / mla_out_proj_folded / mla_o_proj / mla_fold_q / mla_absorb_q_folded)

def _bf16_dev(t, name, shape):
    torch = _torch()
    _dev(t, name, torch.bfloat16)
    _shape(t, name, shape)


def mla_fold_out(dims: Dims, w_uv, w_o, w_comb, stream=None) -> None:
    """w_uv [n_h][d_c][d_v], w_o [d_model][n_h][d_v] -> w_comb [d_model][n_h][d_c] (all bf16)."""
    d_model = w_o.shape[0]
    _bf16_dev(w_uv, "w_uv", (dims.n_h, dims.d_c, dims.d_v))
    _bf16_dev(w_o, "w_o", (d_model, dims.n_h, dims.d_v))
    _bf16_dev(w_comb, "w_comb", (d_model, dims.n_h, dims.d_c))
    d = dims._c()
    _check("mla_fold_out", load_library().mla_fold_out(ctypes.byref(d), d_model, w_uv.data_ptr(), w_o.data_ptr(),
                                                       w_comb.data_ptr(), _stream(stream)))


def mla_out_proj_folded(dims: Dims, u, w_comb, y, stream=None) -> None:
    """u [B][n_q][n_h][d_c] fp32, w_comb [d_model][n_h][d_c] bf16 -> y [B][n_q][d_model] fp32."""
    torch = _torch()
    B, n_q, d_model = u.shape[0], u.shape[1], w_comb.shape[0]
    _dev(u, "u", torch.float32)
    _shape(u, "u", (B, n_q, dims.n_h, dims.d_c))
    _bf16_dev(w_comb, "w_comb", (d_model, dims.n_h, dims.d_c))
    _dev(y, "y", torch.float32)
    _shape(y, "y", (B, n_q, d_model))
    d = dims._c()
    _check("mla_out_proj_folded", load_library().mla_out_proj_folded(
        ctypes.byref(d), d_model, B, n_q, u.data_ptr(), w_comb.data_ptr(), y.data_ptr(), _stream(stream)))


def mla_o_proj(dims: Dims, o, w_o, y, stream=None) -> None:
    """o [B][n_q][n_h][d_v] fp32, w_o [d_model][n_h][d_v] bf16 -> y [B][n_q][d_model] fp32."""
    torch = _torch()
    B, n_q, d_model = o.shape[0], o.shape[1], w_o.shape[0]
    _dev(o, "o", torch.float32)
    _shape(o, "o", (B, n_q, dims.n_h, dims.d_v))
    _bf16_dev(w_o, "w_o", (d_model, dims.n_h, dims.d_v))
    _dev(y, "y", torch.float32)
    _shape(y, "y", (B, n_q, d_model))
    d = dims._c()
    _check("mla_o_proj", load_library().mla_o_proj(ctypes.byref(d), d_model, B, n_q, o.data_ptr(), w_o.data_ptr(),
                                                   y.data_ptr(), _stream(stream)))


def mla_fold_q(dims: Dims, w_uq, w_uk, w_kq, stream=None) -> None:
    """w_uq [d_q][n_h][d_nope], w_uk [n_h][d_c][d_nope] -> w_kq [n_h][d_c][d_q] (all bf16)."""
    d_q = w_uq.shape[0]
    _bf16_dev(w_uq, "w_uq", (d_q, dims.n_h, dims.d_nope))
    _bf16_dev(w_uk, "w_uk", (dims.n_h, dims.d_c, dims.d_nope))
    _bf16_dev(w_kq, "w_kq", (dims.n_h, dims.d_c, d_q))
    d = dims._c()
    _check("mla_fold_q", load_library().mla_fold_q(ctypes.byref(d), d_q, w_uq.data_ptr(), w_uk.data_ptr(),
                                                   w_kq.data_ptr(), _stream(stream)))


def mla_absorb_q_folded(dims: Dims, c_q, q_rope, positions, w_kq, q_lat, q_pe, stream=None) -> None:
    """c_q [B][n_q][d_q], w_kq [n_h][d_c][d_q] -> q_lat [B][n_q][n_h][d_c]; q_pe = RoPE(q_rope) (bf16)."""
    torch = _torch()
    B, n_q, d_q = c_q.shape
    _bf16_dev(c_q, "c_q", (B, n_q, d_q))
    _bf16_dev(q_rope, "q_rope", (B, n_q, dims.n_h, dims.d_rope))
    _dev(positions, "positions", torch.int32)
    _shape(positions, "positions", (B, n_q))
    _bf16_dev(w_kq, "w_kq", (dims.n_h, dims.d_c, d_q))
    _bf16_dev(q_lat, "q_lat", (B, n_q, dims.n_h, dims.d_c))
    _bf16_dev(q_pe, "q_pe", (B, n_q, dims.n_h, dims.d_rope))
    d = dims._c()
    _check("mla_absorb_q_folded", load_library().mla_absorb_q_folded(
        ctypes.byref(d), d_q, B, n_q, c_q.data_ptr(), q_rope.data_ptr(), positions.data_ptr(), w_kq.data_ptr(),
        q_lat.data_ptr(), q_pe.data_ptr(), _stream(stream)))


def mla_prefill_weights(dims: Dims, w_uk, w_uv, w_kv, stream=None) -> None:
    """w_kv [n_h][d_nope + d_v][d_c] bf16 from W_UK [n_h][d_c][d_nope] and W_UV [n_h][d_c][d_v]."""
    torch = _torch()
    for t, n in ((w_uk, "w_uk"), (w_uv, "w_uv"), (w_kv, "w_kv")):
        _dev(t, n, torch.bfloat16)
    _shape(w_uk, "w_uk", (dims.n_h, dims.d_c, dims.d_nope))
    _shape(w_uv, "w_uv", (dims.n_h, dims.d_c, dims.d_v))
    _shape(w_kv, "w_kv", (dims.n_h, dims.d_nope + dims.d_v, dims.d_c))
    d = dims._c()
    _check("mla_prefill_weights", load_library().mla_prefill_weights(
        ctypes.byref(d), w_uk.data_ptr(), w_uv.data_ptr(), w_kv.data_ptr(), _stream(stream)))


def mla_prefill_workspace_bytes(dims: Dims, B: int, max_ctx: int) -> int:
    d = dims._c()
    return int(load_library().mla_prefill_workspace_bytes(ctypes.byref(d), B, max_ctx))


def mla_prefill(dims: Dims, max_ctx: int, q_nope, q_rope, positions, cache: LatentCache, w_kv, workspace,
                q_pe, out, lse=None, stream=None) -> None:
    """Prefill of the last n_q cached tokens of each sequence (see mla.h).
    ``workspace`` is a device tensor of at least mla_prefill_workspace_bytes
    bytes; on return it holds kv [B][max_ctx][n_h][d_nope + d_v] bf16."""
    torch = _torch()
    B, n_q = q_nope.shape[0], q_nope.shape[1]
    for t, n in ((q_nope, "q_nope"), (q_rope, "q_rope"), (q_pe, "q_pe"), (w_kv, "w_kv")):
        _dev(t, n, torch.bfloat16)
    _dev(positions, "positions", torch.int32)
    _dev(out, "out", torch.float32)
    _dev(workspace, "workspace")
    _shape(q_nope, "q_nope", (B, n_q, dims.n_h, dims.d_nope))
    _shape(q_rope, "q_rope", (B, n_q, dims.n_h, dims.d_rope))
    _shape(q_pe, "q_pe", (B, n_q, dims.n_h, dims.d_rope))
    _shape(positions, "positions", (B, n_q))
    _shape(w_kv, "w_kv", (dims.n_h, dims.d_nope + dims.d_v, dims.d_c))
    _shape(out, "out", (B, n_q, dims.n_h, dims.d_v))
    _shape(cache.ctx_lens, "cache.ctx_lens", (B,))
    if lse is not None:
        _dev(lse, "lse", torch.float32)
        _shape(lse, "lse", (B, n_q, dims.n_h))
    if cache.data.shape[-1] != cache.row_width(dims):
        raise ValueError(f"cache rows must be {cache.row_width(dims)} wide")
    if cache.block_size == 0 and (cache.data.shape[0] < B or cache.data.shape[1] < max_ctx):
        raise ValueError("the contiguous cache must hold B sequences of max_ctx rows")
    d, c = dims._c(), cache._c()
    nbytes = workspace.numel() * workspace.element_size()
    _check("mla_prefill", load_library().mla_prefill(
        ctypes.byref(d), B, n_q, max_ctx, q_nope.data_ptr(), q_rope.data_ptr(), positions.data_ptr(),
        ctypes.byref(c), w_kv.data_ptr(), workspace.data_ptr(), nbytes, q_pe.data_ptr(), out.data_ptr(),
        None if lse is None else lse.data_ptr(), _stream(stream)))
