"""GPU parity of the fp8 e4m3 latent cache against the oracle, through the C ABI.

The cache rows are written by the library's own append (mla_cache_append with
an fp8 cache quantises them); the oracle quantises the same seeded bf16
latents with its own encoder (oracle.fp8_quantize_latent).
  - codes and scales: bit-exact (integer results, both sides decide them on
    exact values: x / 2^k is exact in fp32 and fp64);
  - the bf16 positional key: the oracle's fp64 rotation to bf16 resolution,
    as for bf16 caches;
  - decode: the oracle's decode over its dequantised latents, with the bf16
    tolerance (1e-2 max vector relative error): the quantisation itself is
    modelled exactly, so the remaining error is the bf16 rounding of q_lat,
    q_pe and the softmax weights, as on the bf16 path.
Unused cache slots hold 0xFF bytes (NaN codes, NaN bf16 keys, NaN scales).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.test_gpu_parity import _check, _need_gpu, _run

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RB = 512 + 128 + 16   # fp8 row bytes at V3 dims


def _fp8(**kw):
    return W.with_fp8_cache(W.custom(**kw))


def _rows_of(st, w, b):
    """Bytes of the cached rows of sequence b, [ctx][row bytes] uint8."""
    data = st["cache"].data.cpu().numpy()
    n = int(st["ctx_host"][b])
    if not w.block_size:
        return data[b, :n]
    tbl = st["block_table_host"]
    t = np.arange(n)
    return data[tbl[b, t // w.block_size], t % w.block_size]


def _check_rows(w, st, b, rows_bytes):
    rows = W.cache_rows(w, b, 0, int(st["ctx_host"][b]))
    codes, scales = oracle.fp8_quantize_latent(rows["c_kv"])
    np.testing.assert_array_equal(rows_bytes[:, : w.d_c], codes)
    got_scales = np.ascontiguousarray(rows_bytes[:, w.d_c + 2 * w.d_rope:]).view(np.float32)
    np.testing.assert_array_equal(got_scales, scales)
    key = np.ascontiguousarray(rows_bytes[:, w.d_c: w.d_c + 2 * w.d_rope]).view(np.uint16)
    key = W.bf16_bits_to_f32(key).astype(np.float64)
    ref = oracle.rope_rotate(rows["k_rope_raw"], np.arange(len(key)), w.rope_base)
    assert np.abs(key - ref).max() <= 2 ** -8 * np.abs(ref).max()


@pytest.mark.parametrize("block_size", [0, 64])
def test_fp8_append_matches_oracle_codes(block_size):
    _need_gpu()
    from workloads.device import stage
    w = _fp8(name="fp8_append", seed=41, batch=3, n_q=1, ctx=None, ctx_range=(1, 1), block_size=block_size)
    st = stage(w, ctx=np.array([300, 1, 130], np.int32))
    for b in range(w.batch):
        print(f"  seq {b} ctx {st['ctx_host'][b]}", flush=True)
        _check_rows(w, st, b, _rows_of(st, w, b))
    if not block_size:   # rows past each context untouched
        data = st["cache"].data.cpu().numpy()
        for b in range(w.batch):
            assert (data[b, int(st["ctx_host"][b]):] == 0xFF).all()


def test_fp8_append_special_tiles():
    """Tiles that hit the scale rule's corners and the encoder's rounding:
    all zeros, a largest magnitude of exactly 448 * 2^k and just above it,
    values that fall halfway between two codes (ties to even), a tile far
    below 1, negative zeros and bf16 subnormals next to large values."""
    _need_gpu()
    import mla_latent_kv_02_amd as mla
    dims = mla.Dims(128, 512, 64, 128, 128)
    n = 6
    x = np.zeros((n, 512), np.float32)
    rng = np.random.default_rng(43)
    x[1] = rng.standard_normal(512).astype(np.float32)
    x[1, 0:128] *= 0.0                                   # an all-zero tile
    x[1, 128] = 448 * 2.0 ** -3                          # amax = 448 * 2^-3 exactly -> scale 2^-3
    x[1, 256] = np.float32(448 * 2.0 ** -3) * np.float32(1.0078125)   # just above -> scale 2^-2
    # ties with scale 1 (amax 448): 8.5 and 9.5 lie halfway between codes of 8/9 and 9/10, 17
    # between 16 and 18, 2^-10 between 0 and the smallest subnormal 2^-9, 3 * 2^-10 between
    # 2^-9 and 2^-8; each goes to the code with the even mantissa
    x[2, :128] = 0.0
    x[2, 0] = 448.0
    x[2, 1:9] = [8.5, 9.5, -8.5, -9.5, 2.0 ** -10, -(2.0 ** -10), 3 * 2.0 ** -10, 17.0]
    x[3] = rng.standard_normal(512).astype(np.float32) * np.float32(1e-3)
    x[4] = -0.0
    x[4, 5] = 300.0
    x[4, 6] = 2.0 ** -130                               # bf16 subnormal beside a large value
    x[5] = rng.standard_normal(512).astype(np.float32) * np.float32(3e4)
    x = W.round_to_bf16(x)
    k_raw = W.round_to_bf16(rng.standard_normal((n, 64)).astype(np.float32))
    data = torch.full((1, n, RB), 0xFF, dtype=torch.uint8, device="cuda")
    cache = mla.LatentCache(data=data, ctx_lens=torch.tensor([n], dtype=torch.int32, device="cuda"))
    seq = torch.zeros(n, dtype=torch.int32, device="cuda")
    pos = torch.arange(n, dtype=torch.int32, device="cuda")
    xt = torch.from_numpy(x).to(torch.bfloat16).cuda()
    kt = torch.from_numpy(k_raw).to(torch.bfloat16).cuda()
    mla.mla_cache_append(dims, cache, seq, pos, xt, kt)
    torch.cuda.synchronize()
    got = data[0].cpu().numpy()
    codes, scales = oracle.fp8_quantize_latent(x)
    np.testing.assert_array_equal(got[:, :512], codes)
    np.testing.assert_array_equal(np.ascontiguousarray(got[:, 640:]).view(np.float32), scales)
    assert scales[1, 0] == 1.0 and scales[1, 1] == 2.0 ** -3 and scales[1, 2] == 2.0 ** -2
    assert list(codes[2, 1:9]) == [0x50, 0x52, 0xD0, 0xD2, 0x00, 0x00, 0x02, 0x58]


@pytest.mark.parametrize("num_splits", [1, 4, 9])
def test_fp8_v3_contiguous_ragged(num_splits):
    _need_gpu()
    from workloads.device import stage
    w = _fp8(name="fp8_small", seed=44, batch=3, n_q=1, ctx=None, ctx_range=(1, 1))
    st = stage(w, ctx=np.array([300, 1, 130], np.int32))
    got = _run(st, num_splits)
    _check(w, st, got)


@pytest.mark.parametrize("num_splits", [1, 5])
def test_fp8_v3_two_query_tokens(num_splits):
    _need_gpu()
    from workloads.device import stage
    w = _fp8(name="fp8_nq2", seed=45, batch=3, n_q=2, ctx=None, ctx_range=(1, 1))
    st = stage(w, ctx=np.array([257, 2, 66], np.int32))
    got = _run(st, num_splits)
    _check(w, st, got)


@pytest.mark.parametrize("block_size,num_splits",
                         [(64, 1), (64, 3), (16, 1), (16, 5), (40, 4), (96, 3), (96, 7), (256, 2)])
def test_fp8_v3_paged(block_size, num_splits):
    """Paged fp8 caches: block sizes that are multiples of 32 tokens (64, 96,
    256: buffer loads from the lowest block; segments cut at tokens that are
    not multiples of 32 start their stages below the cut and mask the tokens
    before it), and 16 and 40 (the generic layout, per-lane row addresses);
    0xFF in every unused pool byte."""
    _need_gpu()
    from workloads.device import stage
    w = _fp8(name=f"fp8_paged_b{block_size}", seed=46 + block_size, batch=4, n_q=1, ctx=None,
             ctx_range=(1, 1), block_size=block_size)
    st = stage(w, ctx=np.array([200, 64, 65, 1], np.int32))
    assert (st["cache"].data == 0xFF).any()
    got = _run(st, num_splits)
    _check(w, st, got)


@pytest.mark.parametrize("num_splits", [1, 4])
def test_fp8_v3_three_query_tokens_paged(num_splits):
    _need_gpu()
    from workloads.device import stage
    w = _fp8(name="fp8_nq3", seed=47, batch=2, n_q=3, ctx=None, ctx_range=(1, 1), block_size=64)
    st = stage(w, ctx=np.array([131, 3], np.int32))
    got = _run(st, num_splits)
    _check(w, st, got)


def test_fp8_generic_path_small_dims():
    """fp8 rows through the generic kernel: d_c = 256, 8 heads (not a multiple
    of 32), paged with 16-token blocks and contiguous."""
    _need_gpu()
    from workloads.device import stage
    for bs in (0, 16):
        w = _fp8(name="fp8_generic", seed=48, batch=2, n_q=2, n_h=8, d_c=256, d_rope=32, d_nope=32, d_v=32,
                 ctx=None, ctx_range=(1, 1), block_size=bs)
        st = stage(w, ctx=np.array([97, 3], np.int32))
        for ns in (1, 4):
            got = _run(st, ns)
            _check(w, st, got)


def test_fp8_paged_pool_over_4gib():
    """An fp8 pool over 4 GiB (110000 blocks of 64 rows of 656 bytes):
    sequence 0's blocks at both ends of the pool (its segments take the
    generic layout's 64-bit addresses), sequence 1's neighbours (32-bit buffer
    offsets from its lowest block), both in one launch."""
    _need_gpu()
    import mla_latent_kv_02_amd as mla
    from workloads.device import stage
    w = _fp8(name="fp8_bigpool", seed=49, batch=2, n_q=1, ctx=None, ctx_range=(1, 1), block_size=64)
    st = stage(w, ctx=np.array([200, 100], np.int32))
    n_blocks = 110000
    assert n_blocks * 64 * RB > 2 ** 32
    big = torch.empty((n_blocks, 64, RB), dtype=torch.uint8, device="cuda")
    old = st["block_table_host"]
    new = np.full_like(old, -1)
    new[0, :4] = [0, n_blocks - 1, 1, n_blocks - 2]
    new[1, :2] = [60000, 60001]
    for b, nb in ((0, 4), (1, 2)):
        for k in range(nb):
            big[int(new[b, k])] = st["cache"].data[int(old[b, k])]
    st = dict(st, cache=mla.LatentCache(data=big, ctx_lens=st["cache"].ctx_lens,
                                        block_table=torch.from_numpy(new).cuda(), block_size=64))
    for ns in (1, 3):
        got = _run(st, ns)
        _check(w, st, got)
    del big
    torch.cuda.empty_cache()


@pytest.mark.parametrize("block_size", [0, 64])
def test_fp8_append_absorb_matches_separate_calls(block_size):
    """The fused append + absorption writes the same fp8 rows, q_lat and q_pe,
    bit for bit, as mla_cache_append then mla_absorb_q; the new rows are the
    oracle's codes and scales."""
    _need_gpu()
    import mla_latent_kv_02_amd as mla
    from workloads.device import stage
    w = _fp8(name="fp8_append_absorb", seed=50, batch=5, n_q=1, ctx=None, ctx_range=(1, 1),
             block_size=block_size)
    st = stage(w, ctx=np.array([130, 3, 64, 1000, 77], np.int32))
    ctx = st["ctx_host"]
    n = w.batch
    g = torch.Generator().manual_seed(51)
    raw = torch.randn(n, w.row, generator=g).to(torch.bfloat16).cuda()
    seq = torch.arange(n, dtype=torch.int32).cuda()
    pos_host = (ctx - 1).astype(np.int32)
    pos = torch.from_numpy(pos_host).cuda()
    d = st["dims"]
    outs = []
    for fused in (False, True):
        cache = mla.LatentCache(data=st["cache"].data.clone(), ctx_lens=st["cache"].ctx_lens,
                                block_table=st["cache"].block_table, block_size=st["cache"].block_size)
        q_lat = torch.full((w.batch, w.n_q, w.n_h, w.d_c), float("nan"), dtype=torch.bfloat16, device="cuda")
        q_pe = torch.full((w.batch, w.n_q, w.n_h, w.d_rope), float("nan"), dtype=torch.bfloat16, device="cuda")
        if fused:
            mla.mla_append_absorb_q(d, cache, seq, pos, raw[:, :w.d_c], raw[:, w.d_c:], st["q_nope"],
                                    st["q_rope"], st["positions"], st["w_uk"], q_lat, q_pe)
        else:
            mla.mla_cache_append(d, cache, seq, pos, raw[:, :w.d_c], raw[:, w.d_c:])
            mla.mla_absorb_q(d, st["q_nope"], st["q_rope"], st["positions"], st["w_uk"], q_lat, q_pe)
        torch.cuda.synchronize()
        outs.append((cache.data, q_lat.view(torch.int16), q_pe.view(torch.int16)))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)
    data = outs[1][0].cpu().numpy()
    tbl = st.get("block_table_host")
    raw_h = raw.float().cpu().numpy()
    codes, scales = oracle.fp8_quantize_latent(raw_h[:, : w.d_c])
    for b in range(n):
        t = int(pos_host[b])
        row = data[b, t] if not block_size else data[tbl[b, t // block_size], t % block_size]
        np.testing.assert_array_equal(row[: w.d_c], codes[b])
        np.testing.assert_array_equal(np.ascontiguousarray(row[w.d_c + 2 * w.d_rope:]).view(np.float32), scales[b])
