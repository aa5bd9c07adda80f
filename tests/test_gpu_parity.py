"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Small cases that the oracle finishes in seconds, spanning several 64-token
tiles, ragged tails, contexts of one token, two query tokens (causal within
the pair), paged caches with NaN in every unused slot, many split counts and
empty work units.  Tolerances: max vector relative error 1e-4 for fp32
workloads and 1e-2 for bf16 workloads (the bf16 path rounds q_lat, the
rotated positional key and the softmax weights to bf16 as MFMA operands and
accumulates in fp32).
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests._metrics import scalar_err, vec_rel_err
from tests.plan_ref import Plan

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _tol(w):
    return 1e-4 if w.dtype == "f32" else 1e-2


def _run(st, num_splits):
    import mla_latent_kv_02_amd as mla
    from mla_latent_kv_02_amd.step import DecodeStep
    w = st["workload"]
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    step = DecodeStep(st["dims"], w.batch, w.n_q, num_splits, tdt)
    step.run(st["q_nope"], st["q_rope"], st["positions"], st["w_uk"], st["w_uv"], st["cache"])
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    got = {"q_lat": f(step.q_lat), "q_pe": f(step.q_pe), "u": f(step.u), "lse": f(step.lse),
           "o": f(step.out), "u_part": f(step.u_part), "lse_part": f(step.lse_part)}
    if w.dtype == "bf16" and w.d_c == 512 and w.d_v == 128:
        # the same partials through the fused merge + up-projection
        out2 = torch.full_like(step.out, float("nan"))
        lse2 = torch.full_like(step.lse, float("nan"))
        mla.mla_combine_out_proj(st["dims"], st["cache"].ctx_lens, num_splits, step.u_part, step.lse_part,
                                 st["w_uv"], out2, lse2)
        torch.cuda.synchronize()
        got["o_fused"], got["lse_fused"] = f(out2), f(lse2)
    return got


def _oracle(w, st, b, heads=None):
    rows = W.cache_rows(w, b, 0, int(st["ctx_host"][b]))
    c_kv = rows["c_kv"]
    if w.cache_dtype == "fp8":   # the latents as an fp8 cache holds them
        c_kv = oracle.fp8_dequantize_latent(*oracle.fp8_quantize_latent(c_kv))
    wt = W.weights(w)
    q = W.queries(w)
    return oracle.decode_sequence(q["q_nope"][b], q["q_rope"][b], st["positions_host"][b], c_kv,
                                  rows["k_rope_raw"], wt["w_uk"], wt["w_uv"], w.sm_scale, w.rope_base,
                                  heads=heads)


def _check(w, st, got, seqs=None, heads=None):
    tol = _tol(w)
    seqs = range(w.batch) if seqs is None else seqs
    hsel = slice(None) if heads is None else list(heads)
    for b in seqs:
        ref = _oracle(w, st, b, heads)
        errs = {
            "q_lat": vec_rel_err(got["q_lat"][b][:, hsel], ref["q_lat"]),
            "q_pe": vec_rel_err(got["q_pe"][b][:, hsel], ref["q_pe"]),
            "u": vec_rel_err(got["u"][b][:, hsel], ref["u"]),
            "o": vec_rel_err(got["o"][b][:, hsel], ref["o"]),
            "lse": scalar_err(got["lse"][b][:, hsel], ref["lse"]),
        }
        if "o_fused" in got:
            errs["o_fused"] = vec_rel_err(got["o_fused"][b][:, hsel], ref["o"])
            errs["lse_fused"] = scalar_err(got["lse_fused"][b][:, hsel], ref["lse"])
        print(f"  seq {b} ctx {st['ctx_host'][b]}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()),
              flush=True)
        for k, v in errs.items():
            assert v <= tol, (b, k, v)


def test_synth_device_rows_match_host():
    _need_gpu()
    w = W.get("v3_b64")
    seq = np.array([0, 5, 63, 17], np.int32)
    tok = np.array([0, 4097, 8191, 12], np.int32)
    table = torch.from_numpy(W.normal_table_bf16_bits().view(np.int16)).cuda()
    out = torch.empty((4, w.row), dtype=torch.bfloat16, device="cuda")
    sd, td = torch.from_numpy(seq).cuda(), torch.from_numpy(tok).cuda()
    W.fill_cache_rows_device(w, sd.data_ptr(), td.data_ptr(), 4, table.data_ptr(), out.data_ptr(),
                             torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    for k in range(4):
        r = W.cache_rows(w, int(seq[k]), int(tok[k]), int(tok[k]) + 1)
        host = np.concatenate([r["c_kv"], r["k_rope_raw"]], axis=1)[0]
        np.testing.assert_array_equal(W.bf16_bits_to_f32(got[k]), host)


@pytest.mark.parametrize("num_splits", [1, 3, 7])
def test_tiny_fp32(num_splits):
    _need_gpu()
    from workloads.device import stage
    w = W.get("tiny_fp32")
    st = stage(w)
    got = _run(st, num_splits)
    _check(w, st, got)


@pytest.mark.parametrize("num_splits", [1, 4, 9])
def test_v3_contiguous_ragged(num_splits):
    _need_gpu()
    from workloads.device import stage
    w = W.custom(name="v3_small", seed=21, batch=3, n_q=1, ctx=None, ctx_range=(1, 1))
    st = stage(w, ctx=np.array([300, 1, 130], np.int32))
    got = _run(st, num_splits)
    _check(w, st, got)


@pytest.mark.parametrize("num_splits", [1, 5])
def test_v3_two_query_tokens(num_splits):
    _need_gpu()
    from workloads.device import stage
    w = W.custom(name="v3_nq2", seed=22, batch=3, n_q=2, ctx=None, ctx_range=(1, 1))
    st = stage(w, ctx=np.array([257, 2, 66], np.int32))
    got = _run(st, num_splits)
    _check(w, st, got)


@pytest.mark.parametrize("num_splits", [1, 3, 6])
def test_v3_paged_nan_poisoned(num_splits):
    _need_gpu()
    from workloads.device import stage
    w = W.custom(name="v3_paged_small", seed=23, batch=4, n_q=1, ctx=None, ctx_range=(1, 1), block_size=64)
    st = stage(w, ctx=np.array([200, 64, 65, 1], np.int32))
    # every unused slot of the pool holds NaN
    assert torch.isnan(st["cache"].data.float()).any()
    got = _run(st, num_splits)
    _check(w, st, got)


@pytest.mark.parametrize("block_size,num_splits", [(16, 1), (16, 5), (40, 1), (40, 4), (96, 3), (96, 11)])
def test_v3_paged_block_sizes(block_size, num_splits):
    """Block sizes that are not a multiple of the 32-token stage (16, 40: the
    generic layout, per-lane row addresses) and one that is a multiple but not
    a power of two (96; with 11 splits the batch is cut at tokens 77 and 27,
    not multiples of 32, so stage 0 of the segments after the cuts starts
    before their first token and masks the tokens before it), NaN in every
    unused pool slot."""
    _need_gpu()
    from workloads.device import stage
    w = W.custom(name=f"v3_paged_b{block_size}", seed=30 + block_size, batch=3, n_q=1, ctx=None,
                 ctx_range=(1, 1), block_size=block_size)
    st = stage(w, ctx=np.array([150, 17, 97], np.int32))
    got = _run(st, num_splits)
    _check(w, st, got)


def test_v3_paged_pool_over_4gib():
    """A 4.4 GB pool (60000 blocks of 64 tokens): sequence 0's blocks sit at both
    ends of the pool, more than 4 GiB apart (its segments take 64-bit row
    addresses), sequence 1's are neighbours (32-bit buffer offsets from its
    lowest block), both in one launch."""
    _need_gpu()
    import mla_latent_kv_02_amd as mla
    from workloads.device import stage
    w = W.custom(name="v3_bigpool", seed=37, batch=2, n_q=1, ctx=None, ctx_range=(1, 1), block_size=64)
    st = stage(w, ctx=np.array([200, 100], np.int32))
    n_blocks = 60000
    assert n_blocks * 64 * w.row * 2 > 2 ** 32
    big = torch.empty((n_blocks, 64, w.row), dtype=torch.bfloat16, device="cuda")
    old = st["block_table_host"]
    new = np.full_like(old, -1)
    new[0, :4] = [0, n_blocks - 1, 1, n_blocks - 2]
    new[1, :2] = [30000, 30001]
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


@pytest.mark.parametrize("num_splits", [1, 4])
def test_v3_three_query_tokens_paged(num_splits):
    """Three query tokens per sequence (three row groups, causal within the
    triple) on a paged cache."""
    _need_gpu()
    from workloads.device import stage
    w = W.custom(name="v3_nq3", seed=35, batch=2, n_q=3, ctx=None, ctx_range=(1, 1), block_size=64)
    st = stage(w, ctx=np.array([131, 3], np.int32))
    got = _run(st, num_splits)
    _check(w, st, got)


def test_fp32_paged_generic_path():
    _need_gpu()
    from workloads.device import stage
    w = W.custom(name="f32_paged", seed=36, batch=2, n_q=2, n_h=4, d_c=64, d_rope=16, d_nope=32, d_v=32,
                 dtype="f32", ctx=None, ctx_range=(1, 1), block_size=16)
    st = stage(w, ctx=np.array([70, 2], np.int32))
    for ns in (1, 5):
        got = _run(st, ns)
        _check(w, st, got)


def test_generic_path_bf16_small_dims():
    _need_gpu()
    from workloads.device import stage
    w = W.custom(name="bf16_small", seed=24, batch=2, n_q=2, n_h=4, d_c=64, d_rope=16, d_nope=32, d_v=32,
                 ctx=None, ctx_range=(1, 1))
    st = stage(w, ctx=np.array([97, 3], np.int32))
    for ns in (1, 4):
        got = _run(st, ns)
        _check(w, st, got)


def test_split_invariance_and_determinism():
    """Splitting the tokens into more work units changes nothing but rounding.
    On the fp32 path that is fp32 rounding; on the bf16 MFMA path the softmax
    weights are rounded to bf16 against each unit's own running maximum, so
    different splits round differently (bf16 level, ~2^-9).  Reruns with the
    same split are bit-identical (fixed reduction order)."""
    _need_gpu()
    from workloads.device import stage
    wt = W.get("tiny_fp32")
    st = stage(wt)
    one, many = _run(st, 1), _run(st, 13)
    assert vec_rel_err(many["u"], one["u"]) < 1e-5
    assert scalar_err(many["lse"], one["lse"]) < 1e-6
    w = W.custom(name="v3_split_inv", seed=25, batch=2, n_q=1, ctx=None, ctx_range=(1, 1))
    st = stage(w, ctx=np.array([700, 450], np.int32))
    one = _run(st, 1)
    many = _run(st, 11)
    again = _run(st, 11)
    assert vec_rel_err(many["u"], one["u"]) < 1e-2
    assert scalar_err(many["lse"], one["lse"]) < 1e-3
    for k in ("u", "lse", "o", "u_part", "lse_part"):
        np.testing.assert_array_equal(many[k], again[k])


def test_combine_alone_against_oracle():
    """Partials in the documented format (unnormalised value sum with its
    reference r, and lse) merged by mla_combine vs the oracle's merge of the
    normalised partials u_k = u_part_k * exp(r_k - lse_k)."""
    _need_gpu()
    import mla_latent_kv_02_amd as mla
    rng = np.random.default_rng(5)
    dims = mla.Dims(8, 64, 16, 32, 32)
    ctx = np.array([1000, 1, 3500, 700], np.int32)   # the third sequence meets five units
    num_splits = 6
    slots = mla.mla_num_partials(len(ctx), num_splits)
    u_norm = rng.standard_normal((slots, 1, 8, 64))
    lse = rng.standard_normal((slots, 1, 8)) * 5
    ref_shift = rng.standard_normal((slots, 1, 8)) * 3          # arbitrary references r_k
    lse[1, 0, 3] = -np.inf
    u_part = (u_norm * np.exp(lse - ref_shift)[..., None]).astype(np.float32)
    u_part[1, 0, 3] = 0
    rl = np.stack([ref_shift, lse], axis=-1).astype(np.float32)
    rl[1, 0, 3] = (0.0, -np.inf)
    u = torch.empty((4, 1, 8, 64), device="cuda")
    lse_out = torch.empty((4, 1, 8), device="cuda")
    mla.mla_combine(dims, torch.from_numpy(ctx).cuda(), num_splits, torch.from_numpy(u_part).cuda(),
                    torch.from_numpy(rl).cuda(), u, lse_out)
    torch.cuda.synchronize()
    # slots of each sequence under the documented plan
    plan = Plan(ctx, num_splits)
    base = 0
    for b in range(4):
        n = plan.parts[b]
        assert plan.slot0[b] == base
        ref_u, ref_l = oracle.merge_partials(u_norm[base:base + n], lse[base:base + n])
        assert vec_rel_err(u[b].cpu().numpy(), ref_u) < 1e-5
        assert scalar_err(lse_out[b].cpu().numpy(), ref_l) < 1e-6
        base += n
    assert base <= slots


@pytest.mark.parametrize("num_splits", [7, 50])
def test_decode_partials_follow_the_documented_plan(num_splits):
    """mla_decode writes sequence b's partials to the slots the documented
    plan gives it (tests/plan_ref.py) and to no other slot: with u_part and
    lse_part poisoned with NaN, every slot past the plan's count stays NaN,
    and each sequence's slots, normalised (u_part exp(r - lse)) and merged by
    the oracle, give the oracle's u and lse for that sequence.  Ragged
    contexts with empty ones, so that units start inside sequences and the
    cost of the extra segments moves the cuts."""
    _need_gpu()
    from mla_latent_kv_02_amd.step import DecodeStep
    from workloads.device import stage
    w = W.custom(name="plan_slots", seed=61, batch=12, n_q=1, ctx=None, ctx_range=(1, 700))
    ctx = W.context_lengths(w).copy()
    ctx[[3, 8]] = 0
    ctx[5] = 1
    st = stage(w, ctx=ctx)
    step = DecodeStep(st["dims"], w.batch, w.n_q, num_splits, torch.bfloat16)
    step.u_part.fill_(float("nan"))
    step.lse_part.fill_(float("nan"))
    step.run(st["q_nope"], st["q_rope"], st["positions"], st["w_uk"], st["w_uv"], st["cache"])
    torch.cuda.synchronize()
    u_part = step.u_part.cpu().numpy().astype(np.float64)
    rl = step.lse_part.cpu().numpy().astype(np.float64)
    plan = Plan(ctx, num_splits)
    used = sum(plan.parts)
    assert plan.cost_total > int(ctx.sum())                      # some unit starts inside a sequence
    assert np.isnan(rl[used:]).all() and np.isnan(u_part[used:]).all()
    assert not np.isnan(rl[:used]).any() and not np.isnan(u_part[:used]).any()
    for b in range(w.batch):
        if ctx[b] == 0:
            assert plan.parts[b] == 0
            continue
        sl = slice(plan.slot0[b], plan.slot0[b] + plan.parts[b])
        r, lse = rl[sl, ..., 0], rl[sl, ..., 1]
        fin = np.isfinite(lse)
        u_norm = np.where(fin[..., None], u_part[sl] * np.exp(np.where(fin, r - lse, 0.0))[..., None], 0.0)
        u_m, lse_m = oracle.merge_partials(u_norm, lse)
        ref = _oracle(w, st, b)
        assert vec_rel_err(u_m, ref["u"]) <= 1e-2, b
        assert scalar_err(lse_m, ref["lse"]) <= 1e-2, b


# (heads, sequences), two query tokens each: 16 x 40 -> 80 query rows in blocks
# of 4 with eight lanes per row, workgroups of one row block; the others take
# workgroups of two row blocks (one-block workgroups of 32 rows would need more
# than one round over 256 CUs):
# 128 x 55 -> 110 rows, the second workgroup's second block ragged (14 rows);
# 128 x 45 -> 90 rows, the second workgroup's second block past the batch end;
# 96 x 50 -> 100 rows in blocks of 16 with two lanes per row, the last
# workgroup's second block past the end.
@pytest.mark.parametrize("n_h,B", [(16, 40), (128, 55), (128, 45), (96, 50)])
@pytest.mark.parametrize("num_splits", [1, 7, 50])
def test_combine_out_proj_against_oracle(num_splits, n_h, B):
    """mla_combine_out_proj on partials in the documented format, two query
    tokens a sequence, one empty partial: against the oracle's merge of the
    normalised partials followed by its W_UV product."""
    _need_gpu()
    import mla_latent_kv_02_amd as mla
    rng = np.random.default_rng(31 + num_splits + n_h + B)
    d_c, d_v, n_q = 512, 128, 2
    dims = mla.Dims(n_h, d_c, 64, 128, d_v)
    ctx = rng.integers(1, 4000, size=B).astype(np.int32)   # one to four partials a sequence
    ctx[3] = 1
    slots = mla.mla_num_partials(B, num_splits)
    u_norm = rng.standard_normal((slots, n_q, n_h, d_c))
    lse = rng.standard_normal((slots, n_q, n_h)) * 4
    ref_shift = lse + rng.standard_normal((slots, n_q, n_h))      # references near lse
    lse[0, 1, 5] = -np.inf
    u_part = (u_norm * np.exp(lse - ref_shift)[..., None]).astype(np.float32)
    u_part[0, 1, 5] = 0
    rl = np.stack([ref_shift, lse], axis=-1).astype(np.float32)
    rl[0, 1, 5] = (0.0, -np.inf)
    wuv = W.round_to_bf16((rng.standard_normal((n_h, d_c, d_v)) / np.sqrt(d_c)).astype(np.float32))
    out = torch.full((B, n_q, n_h, d_v), float("nan"), device="cuda")
    lse_out = torch.full((B, n_q, n_h), float("nan"), device="cuda")
    mla.mla_combine_out_proj(dims, torch.from_numpy(ctx).cuda(), num_splits, torch.from_numpy(u_part).cuda(),
                             torch.from_numpy(rl).cuda(), torch.from_numpy(wuv).cuda().bfloat16(), out, lse_out)
    torch.cuda.synchronize()
    out, lse_out = out.cpu().numpy(), lse_out.cpu().numpy()
    plan = Plan(ctx, num_splits)
    base = 0
    for b in range(B):
        n = plan.parts[b]
        assert plan.slot0[b] == base
        ref_u, ref_l = oracle.merge_partials(u_norm[base:base + n], lse[base:base + n])
        ref_o = oracle.value_up_projection(ref_u, wuv)
        assert vec_rel_err(out[b], ref_o) < 1e-4, b
        assert scalar_err(lse_out[b], ref_l) < 1e-5, b
        base += n
    assert base <= slots


@pytest.mark.parametrize("n_h,B", [(16, 40), (128, 45)])
def test_merge_without_lse_output(n_h, B):
    """mla_combine and mla_combine_out_proj with no lse output (a NULL pointer
    at the C ABI): the other outputs are bit-identical to the calls with one,
    for workgroups of one row block (16 heads) and of two (128 heads)."""
    _need_gpu()
    import mla_latent_kv_02_amd as mla
    rng = np.random.default_rng(77 + n_h)
    d_c, d_v, n_q, num_splits = 512, 128, 2, 7
    dims = mla.Dims(n_h, d_c, 64, 128, d_v)
    ctx = torch.from_numpy(rng.integers(1, 4000, size=B).astype(np.int32)).cuda()
    slots = mla.mla_num_partials(B, num_splits)
    lse = rng.standard_normal((slots, n_q, n_h)) * 4
    ref = lse + rng.standard_normal((slots, n_q, n_h))
    u_part = torch.from_numpy((rng.standard_normal((slots, n_q, n_h, d_c)) * np.exp(lse - ref)[..., None])
                              .astype(np.float32)).cuda()
    rl = torch.from_numpy(np.stack([ref, lse], axis=-1).astype(np.float32)).cuda()
    wuv = torch.from_numpy(W.round_to_bf16((rng.standard_normal((n_h, d_c, d_v)) / np.sqrt(d_c))
                                           .astype(np.float32))).cuda().bfloat16()
    outs = []
    for with_lse in (True, False):
        u = torch.full((B, n_q, n_h, d_c), float("nan"), device="cuda")
        o = torch.full((B, n_q, n_h, d_v), float("nan"), device="cuda")
        l1 = torch.full((B, n_q, n_h), float("nan"), device="cuda") if with_lse else None
        l2 = torch.full((B, n_q, n_h), float("nan"), device="cuda") if with_lse else None
        mla.mla_combine(dims, ctx, num_splits, u_part, rl, u, l1)
        mla.mla_combine_out_proj(dims, ctx, num_splits, u_part, rl, wuv, o, l2)
        torch.cuda.synchronize()
        outs.append((u.cpu(), o.cpu()))
        if with_lse:
            assert torch.isfinite(l1).all() and torch.allclose(l1, l2, rtol=1e-5, atol=1e-5)
    assert torch.isfinite(outs[0][0]).all() and torch.isfinite(outs[0][1]).all()
    assert torch.equal(outs[0][0], outs[1][0])
    assert torch.equal(outs[0][1], outs[1][1])


# 16 heads x 10 rows: workgroups of one row block; 128 heads x 90 rows:
# workgroups of two, the last one's second block past the batch end
@pytest.mark.parametrize("n_h,B", [(16, 5), (128, 45)])
def test_out_proj_alone_against_oracle(n_h, B):
    _need_gpu()
    import mla_latent_kv_02_amd as mla
    rng = np.random.default_rng(6 + n_h)
    dims = mla.Dims(n_h, 512, 64, 128, 128)
    u = rng.standard_normal((B, 2, n_h, 512)).astype(np.float32)
    wuv = W.round_to_bf16((rng.standard_normal((n_h, 512, 128)) / np.sqrt(512)).astype(np.float32))
    out = torch.full((B, 2, n_h, 128), float("nan"), device="cuda")
    mla.mla_out_proj(dims, torch.from_numpy(u).cuda(), torch.from_numpy(wuv).cuda().bfloat16(), out)
    torch.cuda.synchronize()
    ref = oracle.value_up_projection(u, wuv)
    assert vec_rel_err(out.cpu().numpy(), ref) < 1e-4


def test_cache_append_rotates_positional_key():
    _need_gpu()
    from workloads.device import stage
    w = W.custom(name="append", seed=26, batch=2, n_q=1, ctx=None, ctx_range=(1, 1))
    ctx = np.array([70, 5], np.int32)
    st = stage(w, ctx=ctx)
    data = st["cache"].data.float().cpu().numpy()
    for b in range(2):
        rows = W.cache_rows(w, b, 0, int(ctx[b]))
        np.testing.assert_array_equal(data[b, :ctx[b], :512], rows["c_kv"])
        ref = oracle.rope_rotate(rows["k_rope_raw"], np.arange(ctx[b]), 10000.0)
        assert np.abs(data[b, :ctx[b], 512:] - ref).max() <= 2 ** -8 * np.abs(ref).max()
        assert np.isnan(data[b, ctx[b]:]).all()


def test_graph_replay_matches_eager():
    """The step captured once in a HIP graph and replayed: every replay writes
    the same outputs as the eager step (outputs poisoned with NaN by eager work
    before each replay), for both the fused and the separate merge."""
    _need_gpu()
    from workloads.device import stage
    from mla_latent_kv_02_amd.step import DecodeStep
    w = W.custom(name="v3_graph", seed=27, batch=3, n_q=2, ctx=None, ctx_range=(1, 1))
    st = stage(w, ctx=np.array([300, 2, 97], np.int32))
    for fused in (True, False):
        step = DecodeStep(st["dims"], w.batch, w.n_q, 5, torch.bfloat16)
        args = (st["q_nope"], st["q_rope"], st["positions"], st["w_uk"], st["w_uv"], st["cache"])
        step.run(*args, fused_tail=fused)
        torch.cuda.synchronize()
        ref_o, ref_l = step.out.clone(), step.lse.clone()
        graph = step.capture(*args, fused_tail=fused)
        for rep in range(3):
            step.out.fill_(float("nan"))
            step.lse.fill_(float("nan"))
            step.u_part.fill_(float("nan"))
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(step.out, ref_o), (fused, rep)
            assert torch.equal(step.lse, ref_l), (fused, rep)


@pytest.mark.parametrize("name,block_size,n_q", [("v3", 0, 1), ("v3", 64, 2), ("tiny", 0, 1)])
def test_append_absorb_matches_separate_calls(name, block_size, n_q):
    """mla_append_absorb_q writes the same cache rows, q_lat and q_pe, bit for
    bit, as mla_cache_append followed by mla_absorb_q (one launch for the bf16
    V3 shapes, two for the fp32 tiny shapes); the new rows' positional keys
    are the oracle's rotation to bf16/fp32 resolution."""
    _need_gpu()
    import mla_latent_kv_02_amd as mla
    from workloads.device import stage
    if name == "tiny":
        w = W.get("tiny_fp32")
        st = stage(w)
    else:
        w = W.custom(name="append_absorb", seed=28, batch=5, n_q=n_q, ctx=None, ctx_range=(1, 1),
                     block_size=block_size)
        st = stage(w, ctx=np.array([130, 3, 64, 1000, 77], np.int32)[: w.batch])
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    ctx = st["ctx_host"]
    # one new row per sequence, written over its last cached token
    n = w.batch
    g = torch.Generator().manual_seed(29)
    raw = torch.randn(n, w.row, generator=g).to(tdt).cuda()
    seq = torch.arange(n, dtype=torch.int32).cuda()
    pos_host = (ctx - 1).astype(np.int32)
    pos = torch.from_numpy(pos_host).cuda()
    d = st["dims"]
    outs = []
    for fused in (False, True):
        cache = mla.LatentCache(data=st["cache"].data.clone(), ctx_lens=st["cache"].ctx_lens,
                                block_table=st["cache"].block_table, block_size=st["cache"].block_size)
        q_lat = torch.full((w.batch, w.n_q, w.n_h, w.d_c), float("nan"), dtype=tdt, device="cuda")
        q_pe = torch.full((w.batch, w.n_q, w.n_h, w.d_rope), float("nan"), dtype=tdt, device="cuda")
        if fused:
            mla.mla_append_absorb_q(d, cache, seq, pos, raw[:, :w.d_c], raw[:, w.d_c:], st["q_nope"],
                                    st["q_rope"], st["positions"], st["w_uk"], q_lat, q_pe)
        else:
            mla.mla_cache_append(d, cache, seq, pos, raw[:, :w.d_c], raw[:, w.d_c:])
            mla.mla_absorb_q(d, st["q_nope"], st["q_rope"], st["positions"], st["w_uk"], q_lat, q_pe)
        torch.cuda.synchronize()
        outs.append((cache, q_lat, q_pe))
    bits = (lambda t: t.view(torch.int16)) if tdt == torch.bfloat16 else (lambda t: t.view(torch.int32))
    for a, b in zip(outs[0], outs[1]):
        ta, tb = (a.data, b.data) if isinstance(a, mla.LatentCache) else (a, b)
        assert torch.equal(bits(ta), bits(tb))
    cache = outs[1][0]
    data = cache.data.float().cpu().numpy()
    tbl = None if cache.block_table is None else cache.block_table.cpu().numpy()
    raw_h = raw.float().cpu().numpy().astype(np.float64)
    for b in range(n):
        t = int(pos_host[b])
        row = data[b, t] if tbl is None else data[tbl[b, t // w.block_size], t % w.block_size]
        np.testing.assert_array_equal(row[: w.d_c], raw_h[b, : w.d_c])
        ref = oracle.rope_rotate(raw_h[b : b + 1, w.d_c :], np.array([t]), w.rope_base)[0]
        assert np.abs(row[w.d_c :] - ref).max() <= (2 ** -8 if tdt == torch.bfloat16 else 1e-6) * np.abs(ref).max()
