"""C-ABI checks that need no GPU: the library loads, exports every function
include/mla.h declares, and rejects bad arguments on the host (before any
HIP call, so these run on a machine without a GPU)."""
import ctypes
import os
import re

import pytest

import mla_latent_kv_02_amd as mla
from mla_latent_kv_02_amd import _binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        pytest.skip("libmla.so not built")
    return mla.load_library()


def test_header_declares_the_boundary():
    names = _declared()
    for fn in ("mla_absorb_q", "mla_decode", "mla_combine", "mla_out_proj", "mla_cache_append"):
        assert fn in names
    assert set(names) == set(bd.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings_and_version(lib):
    for code in range(6):
        assert lib.mla_status_string(code)
    assert b"unknown" in lib.mla_status_string(99)
    assert b"gfx950" in lib.mla_version()


def test_num_partials(lib):
    assert lib.mla_num_partials(64, 256) == 319
    assert lib.mla_num_partials(1, 1) == 1
    assert lib.mla_num_partials(0, 8) == 0
    assert lib.mla_num_partials(4, 0) == -1


V3 = bd._Dims(128, 512, 64, 128, 128, 0.0, 0.0)
FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: validation fails first


def _cache(**kw):
    c = dict(dtype=1, data=0x10000, seq_stride=576 * 16, block_size=0, block_table=None, max_blocks=0,
             ctx_lens=0x20000)
    c.update(kw)
    return bd._Cache(c["dtype"], c["data"], c["seq_stride"], c["block_size"], c["block_table"],
                     c["max_blocks"], c["ctx_lens"])


@pytest.mark.parametrize("dims", [
    None,
    bd._Dims(0, 512, 64, 128, 128, 0, 0),      # no heads
    bd._Dims(128, 500, 64, 128, 128, 0, 0),    # d_c not a multiple of 8
    bd._Dims(128, 512, 63, 128, 128, 0, 0),    # odd d_rope
    bd._Dims(128, 512, 64, 0, 128, 0, 0),      # d_nope = 0
    bd._Dims(128, 512, 64, 128, 128, -1.0, 0),  # negative scale
])
def test_decode_rejects_bad_dims(lib, dims):
    c = _cache()
    d = None if dims is None else ctypes.byref(dims)
    st = lib.mla_decode(d, 2, 1, FAKE, FAKE, ctypes.byref(c), FAKE, 4, FAKE, FAKE, None)
    assert st == bd.MLA_ERR_INVALID_ARG


def test_decode_rejects_bad_arguments(lib):
    c = _cache()
    ok_args = [ctypes.byref(V3), 2, 1, FAKE, FAKE, ctypes.byref(c), FAKE, 4, FAKE, FAKE, None]
    for idx, bad in ((1, -1), (2, 0), (3, None), (4, None), (6, None), (7, 0), (7, -3), (8, None), (9, None)):
        args = list(ok_args)
        args[idx] = bad
        assert lib.mla_decode(*args) == bd.MLA_ERR_INVALID_ARG, idx
    # cache descriptor problems
    for kw in (dict(data=None), dict(ctx_lens=None), dict(dtype=7), dict(block_size=-1),
               dict(block_size=64, block_table=None), dict(block_size=64, block_table=0x30000, max_blocks=0),
               dict(data=0x10008)):
        cc = _cache(**kw)
        args = list(ok_args)
        args[5] = ctypes.byref(cc)
        assert lib.mla_decode(*args) == bd.MLA_ERR_INVALID_ARG, kw
    args = list(ok_args)
    args[5] = None
    assert lib.mla_decode(*args) == bd.MLA_ERR_INVALID_ARG


def test_zero_batch_is_a_no_op(lib):
    c = _cache()
    assert lib.mla_decode(ctypes.byref(V3), 0, 1, None, None, ctypes.byref(c), None, 4, None, None, None) == 0
    assert lib.mla_absorb_q(ctypes.byref(V3), 0, 1, 1, None, None, None, None, None, None, None) == 0
    assert lib.mla_combine(ctypes.byref(V3), 0, 1, None, 4, None, None, None, None, None) == 0
    assert lib.mla_out_proj(ctypes.byref(V3), 0, 1, None, 1, None, None, None) == 0


def test_other_entry_points_reject_bad_arguments(lib):
    d = ctypes.byref(V3)
    assert lib.mla_absorb_q(d, 2, 1, 5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_q(d, 2, 0, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_absorb_q(d, 2, 1, 1, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_combine(d, 2, 1, FAKE, 0, FAKE, FAKE, FAKE, FAKE, None) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_combine(d, 2, 1, None, 4, FAKE, FAKE, FAKE, FAKE, None) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_combine(d, 2, 1, FAKE, 4, FAKE, FAKE, None, FAKE, None) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_out_proj(d, 2, 1, FAKE, 3, FAKE, FAKE, None) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_out_proj(d, 2, 1, None, 1, FAKE, FAKE, None) == bd.MLA_ERR_INVALID_ARG
    cop = lib.mla_combine_out_proj
    assert cop(d, 2, 1, FAKE, 0, FAKE, FAKE, 1, FAKE, FAKE, None, None) == bd.MLA_ERR_INVALID_ARG
    assert cop(d, 2, 1, FAKE, 4, FAKE, FAKE, 7, FAKE, FAKE, None, None) == bd.MLA_ERR_INVALID_ARG
    assert cop(d, 2, 1, FAKE, 4, FAKE, FAKE, 1, None, FAKE, None, None) == bd.MLA_ERR_INVALID_ARG
    assert cop(d, 2, 1, FAKE, 4, FAKE, FAKE, 1, FAKE, None, None, None) == bd.MLA_ERR_INVALID_ARG
    # fp32 weights are not compiled for the fused pass: refused before any launch
    assert cop(d, 2, 1, FAKE, 4, FAKE, FAKE, 0, FAKE, FAKE, None, None) == bd.MLA_ERR_UNSUPPORTED
    assert cop(d, 0, 1, None, 4, None, None, 1, None, None, None, None) == 0
    c = _cache()
    cr = ctypes.byref(c)
    assert lib.mla_cache_append(d, cr, -1, FAKE, FAKE, FAKE, 512, FAKE, 64, None) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_cache_append(d, cr, 3, FAKE, FAKE, FAKE, 100, FAKE, 64, None) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_cache_append(d, cr, 3, None, FAKE, FAKE, 512, FAKE, 64, None) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_cache_append(d, cr, 0, None, None, None, 0, None, 0, None) == 0
    # the fused append + absorption checks both argument sets before anything is enqueued
    aa = lib.mla_append_absorb_q
    absorb_ok = (2, 1, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    append_ok = (3, FAKE, FAKE, FAKE, 512, FAKE, 64)
    assert aa(d, cr, 3, FAKE, FAKE, FAKE, 100, FAKE, 64, *absorb_ok) == bd.MLA_ERR_INVALID_ARG
    assert aa(d, cr, -1, FAKE, FAKE, FAKE, 512, FAKE, 64, *absorb_ok) == bd.MLA_ERR_INVALID_ARG
    assert aa(d, None, *append_ok, *absorb_ok) == bd.MLA_ERR_INVALID_ARG
    assert aa(d, cr, *append_ok, 2, 0, 1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == bd.MLA_ERR_INVALID_ARG
    assert aa(d, cr, *append_ok, 2, 1, 5, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == bd.MLA_ERR_INVALID_ARG
    assert aa(d, cr, *append_ok, 2, 1, 1, FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == bd.MLA_ERR_INVALID_ARG
    assert aa(d, cr, 0, None, None, None, 0, None, 0, 0, 1, 1, None, None, None, None, None, None, None) == 0


def test_binding_refuses_host_tensors(lib):
    torch = pytest.importorskip("torch")
    dims = mla.Dims(4, 64, 16, 32, 32)
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        mla.mla_out_proj(dims, x, torch.zeros(4, 64, 32), torch.zeros(1, 1, 4, 32))


def test_cache_row_bytes(lib):
    small = bd._Dims(4, 64, 16, 32, 32, 0.0, 0.0)
    assert lib.mla_cache_row_bytes(ctypes.byref(V3), bd.FP8_E4M3) == 512 + 128 + 16
    assert lib.mla_cache_row_bytes(ctypes.byref(V3), bd.BF16) == 1152
    assert lib.mla_cache_row_bytes(ctypes.byref(V3), bd.F32) == 2304
    assert lib.mla_cache_row_bytes(ctypes.byref(small), bd.FP8_E4M3) == -1   # d_c not a multiple of 128
    assert lib.mla_cache_row_bytes(ctypes.byref(V3), 7) == -1
    assert lib.mla_cache_row_bytes(None, bd.BF16) == -1


def test_fp8_cache_argument_checks(lib):
    """fp8 is a cache dtype only, and needs d_c % 128 == 0."""
    small = bd._Dims(4, 64, 16, 32, 32, 0.0, 0.0)
    c = _cache(dtype=bd.FP8_E4M3, seq_stride=656 * 16)
    st = lib.mla_decode(ctypes.byref(small), 2, 1, FAKE, FAKE, ctypes.byref(c), FAKE, 4, FAKE, FAKE, None)
    assert st == bd.MLA_ERR_INVALID_ARG
    st = lib.mla_cache_append(ctypes.byref(small), ctypes.byref(c), 1, FAKE, FAKE, FAKE, 64, FAKE, 16, None)
    assert st == bd.MLA_ERR_INVALID_ARG
    # queries and weights are never fp8
    st = lib.mla_absorb_q(ctypes.byref(V3), 1, 1, bd.FP8_E4M3, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == bd.MLA_ERR_INVALID_ARG
    st = lib.mla_out_proj(ctypes.byref(V3), 1, 1, FAKE, bd.FP8_E4M3, FAKE, FAKE, None)
    assert st == bd.MLA_ERR_INVALID_ARG
    # a valid fp8 cache with a bad split count is still rejected on the host
    st = lib.mla_decode(ctypes.byref(V3), 2, 1, FAKE, FAKE, ctypes.byref(c), FAKE, 0, FAKE, FAKE, None)
    assert st == bd.MLA_ERR_INVALID_ARG


def test_prefill_argument_checks(lib):
    """mla_prefill / mla_prefill_weights / mla_prefill_workspace_bytes reject
    bad arguments on the host; shapes outside the compiled set (non-V3 head
    dims, fp8 or paged caches, sizes past the 32-bit buffer offsets) are
    MLA_ERR_UNSUPPORTED."""
    d = ctypes.byref(V3)
    small = ctypes.byref(bd._Dims(4, 64, 16, 32, 32, 0.0, 0.0))
    ws_bytes = lib.mla_prefill_workspace_bytes(d, 2, 100)
    assert ws_bytes == 2 * 100 * 128 * 256 * 2
    assert lib.mla_prefill_workspace_bytes(d, -1, 100) == -1
    assert lib.mla_prefill_workspace_bytes(None, 2, 100) == -1
    c = _cache(seq_stride=576 * 100)
    cr = ctypes.byref(c)

    def call(dims=d, B=2, n_q=10, max_ctx=100, cache=cr, ws=FAKE, ws_bytes=ws_bytes, q_nope=FAKE, out=FAKE):
        return lib.mla_prefill(dims, B, n_q, max_ctx, q_nope, FAKE, FAKE, cache, FAKE, ws, ws_bytes, FAKE, out,
                               None, None)

    assert call(B=0, q_nope=None, out=None, ws=None, ws_bytes=0) == 0
    assert call(n_q=0) == bd.MLA_ERR_INVALID_ARG
    assert call(B=-1) == bd.MLA_ERR_INVALID_ARG
    assert call(max_ctx=5) == bd.MLA_ERR_INVALID_ARG                    # fewer cached rows than queries
    assert call(q_nope=None) == bd.MLA_ERR_INVALID_ARG
    assert call(out=None) == bd.MLA_ERR_INVALID_ARG
    assert call(ws=None) == bd.MLA_ERR_INVALID_ARG
    assert call(ws_bytes=ws_bytes - 1) == bd.MLA_ERR_INVALID_ARG         # workspace too small
    assert call(ws=ctypes.c_void_p(0x10008)) == bd.MLA_ERR_INVALID_ARG   # not 16-byte aligned
    assert call(cache=None) == bd.MLA_ERR_INVALID_ARG
    short = _cache(seq_stride=576 * 99)                                   # max_ctx rows do not fit
    assert call(cache=ctypes.byref(short)) == bd.MLA_ERR_INVALID_ARG
    paged = _cache(block_size=64, block_table=0x30000, max_blocks=4)
    assert call(cache=ctypes.byref(paged)) == bd.MLA_ERR_UNSUPPORTED
    fp8 = _cache(dtype=bd.FP8_E4M3, seq_stride=656 * 100)
    assert call(cache=ctypes.byref(fp8)) == bd.MLA_ERR_UNSUPPORTED
    small_cache = _cache(seq_stride=80 * 100)
    small_ws = lib.mla_prefill_workspace_bytes(small, 2, 100)
    assert call(dims=small, cache=ctypes.byref(small_cache), ws_bytes=small_ws) == bd.MLA_ERR_UNSUPPORTED
    # past the 32-bit buffer offsets of the workspace rows
    big = 1 << 20
    huge = _cache(seq_stride=576 * big)
    assert call(max_ctx=big, cache=ctypes.byref(huge), ws_bytes=lib.mla_prefill_workspace_bytes(d, 2, big)) \
        == bd.MLA_ERR_UNSUPPORTED
    assert lib.mla_prefill_weights(d, None, FAKE, FAKE, None) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_prefill_weights(small, FAKE, FAKE, FAKE, None) == bd.MLA_ERR_UNSUPPORTED


def test_hip_error_detail_without_a_launch(lib):
    # no call on this thread has failed a launch yet
    assert lib.mla_last_hip_error() == 0
    assert lib.mla_hip_error_name(0) == b"hipSuccess"
    assert lib.mla_hip_error_name(100) == b"hipErrorNoDevice"
    assert lib.mla_hip_error_name(98) == b"hipErrorInvalidDeviceFunction"
    # an argument error is not a HIP error and leaves the record alone
    assert lib.mla_decode(None, 2, 1, FAKE, FAKE, None, FAKE, 4, FAKE, FAKE, None) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_last_hip_error() == 0


def test_binding_names_the_hip_error(monkeypatch):
    # the binding turns MLA_ERR_HIP into a message that names the HIP error
    class FakeLib:
        def mla_status_string(self, s):
            return b"HIP launch error"

        def mla_last_hip_error(self):
            return 98

        def mla_hip_error_name(self, c):
            return b"hipErrorInvalidDeviceFunction"
    monkeypatch.setattr(bd, "load_library", lambda *a, **k: FakeLib())
    with pytest.raises(bd.MlaError, match=r"hipErrorInvalidDeviceFunction \(98\)"):
        bd._check("mla_decode", bd.MLA_ERR_HIP)


def test_misaligned_vector_buffers_are_rejected(lib):
    c = _cache()
    d = ctypes.byref(V3)
    odd16, odd8 = ctypes.c_void_p(0x10008), ctypes.c_void_p(0x10004)
    base = [d, 2, 1, FAKE, FAKE, ctypes.byref(c), FAKE, 4, FAKE, FAKE, None]
    for idx, bad in ((3, odd16), (4, odd16), (8, odd16), (9, odd8)):
        args = list(base)
        args[idx] = bad
        assert lib.mla_decode(*args) == bd.MLA_ERR_INVALID_ARG, idx
    # combine: u_part, u 16 bytes, lse_part 8 bytes
    assert lib.mla_combine(d, 2, 1, FAKE, 4, odd16, FAKE, FAKE, None, None) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_combine(d, 2, 1, FAKE, 4, FAKE, odd8, FAKE, None, None) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_combine(d, 2, 1, FAKE, 4, FAKE, FAKE, odd16, None, None) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_out_proj(d, 2, 1, odd16, 1, FAKE, FAKE, None) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_out_proj(d, 2, 1, FAKE, 1, odd16, FAKE, None) == bd.MLA_ERR_INVALID_ARG
    assert lib.mla_combine_out_proj(d, 2, 1, FAKE, 4, odd16, FAKE, 1, FAKE, FAKE, None, None) == \
        bd.MLA_ERR_INVALID_ARG
    assert lib.mla_combine_out_proj(d, 2, 1, FAKE, 4, FAKE, odd8, 1, FAKE, FAKE, None, None) == \
        bd.MLA_ERR_INVALID_ARG


def test_contiguous_stride_below_one_row_is_rejected(lib):
    d = ctypes.byref(V3)
    for stride in (0, 575, -1):
        c = _cache(seq_stride=stride)
        assert lib.mla_decode(d, 1, 1, FAKE, FAKE, ctypes.byref(c), FAKE, 4, FAKE, FAKE, None) == \
            bd.MLA_ERR_INVALID_ARG, stride
    # fp8 rows: the stride counts bytes, one row is 656 bytes at V3 dims
    c = _cache(dtype=2, seq_stride=655)
    assert lib.mla_decode(d, 1, 1, FAKE, FAKE, ctypes.byref(c), FAKE, 4, FAKE, FAKE, None) == bd.MLA_ERR_INVALID_ARG


def test_noalloc_rejects_inputs_beyond_its_scratch(lib):
    # host-side size check, before any HIP call: (num_splits + B - 1) partial
    # slots of n_q * n_h rows beyond MLA_NOALLOC_SCRATCH_BYTES
    c = _cache()
    d = ctypes.byref(V3)
    args = lambda B, ns: (d, B, 1, FAKE, FAKE, ctypes.byref(c), FAKE, ns, 1, FAKE, FAKE, None, None)
    assert lib.mla_decode_out_noalloc(*args(2, 1 << 20)) == bd.MLA_ERR_TOO_LARGE
    assert lib.mla_decode_out_noalloc(*args(2, 510)) == bd.MLA_ERR_TOO_LARGE     # 511 slots of 128 rows
    assert lib.mla_status_string(bd.MLA_ERR_TOO_LARGE).startswith(b"input needs more")
    # argument errors come first, as for mla_decode / mla_combine_out_proj
    assert lib.mla_decode_out_noalloc(d, 2, 1, FAKE, FAKE, ctypes.byref(c), FAKE, 4, 1, None, FAKE, None, None) == \
        bd.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_out_noalloc(d, 2, 1, FAKE, FAKE, ctypes.byref(c), FAKE, 4, 1, FAKE, None, None, None) == \
        bd.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_out_noalloc(d, 2, 1, FAKE, FAKE, ctypes.byref(c), FAKE, 0, 1, FAKE, FAKE, None, None) == \
        bd.MLA_ERR_INVALID_ARG
    assert lib.mla_decode_out_noalloc(d, 0, 1, None, None, ctypes.byref(c), None, 4, 1, None, None, None, None) == 0
