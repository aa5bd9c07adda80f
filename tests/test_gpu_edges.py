"""GPU cases at the edges of the split-KV plan, the decode kernel's redo path
and the cache descriptor, against the fp64 oracle (tolerance 1e-2, bf16
operands):

- a batch of 300 sequences: the plan walk takes sequences in chunks of 256,
  so work-unit boundaries and partial slots fall in both chunks (or a unit
  runs across the chunk boundary); short ragged contexts, two of 1500 tokens,
  some empty (a query that sees no token gives u = 0, o = 0, lse = -inf);
- one late token whose latent row is 2048 e_j: its scores pass many rows'
  reference by far more than the kernel's headroom, so those segments are
  computed again with the true maximum.  Over paged caches whose segment
  spans more than the 64-block id window (the window reloads before the
  spike) and over fp8 caches (2048 e_j is exact under the power-of-two tile
  scales), at 1 and 4 splits; per-head tolerance 1e-2 plus the bf16 rounding
  of the spike's own score where its softmax share is partial (derived in
  the test);
- descriptor breaches the kernels keep memory-safe: an append to a position
  without a reserved block writes nothing; decode takes a range with a
  negative block id, or one that runs past the table row, as empty.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests._metrics import scalar_err, vec_rel_err
from tests.plan_ref import Plan
from tests.test_gpu_parity import _need_gpu, torch

pytestmark = pytest.mark.gpu


def _f(t):
    return t.float().cpu().numpy().astype(np.float64)


def _decode(st, num_splits):
    """The step through both merges: combine + out_proj and the fused one."""
    import mla_latent_kv_02_amd as mla
    from mla_latent_kv_02_amd.step import DecodeStep
    w = st["workload"]
    step = DecodeStep(st["dims"], w.batch, w.n_q, num_splits, torch.bfloat16)
    step.run(st["q_nope"], st["q_rope"], st["positions"], st["w_uk"], st["w_uv"], st["cache"])
    out2 = torch.full_like(step.out, float("nan"))
    lse2 = torch.full_like(step.lse, float("nan"))
    mla.mla_combine_out_proj(st["dims"], st["cache"].ctx_lens, num_splits, step.u_part, step.lse_part,
                             st["w_uv"], out2, lse2)
    torch.cuda.synchronize()
    return {"u": _f(step.u), "lse": _f(step.lse), "o": _f(step.out), "o_fused": _f(out2), "lse_fused": _f(lse2)}


_INPUTS = {}
_REFS = {}


def _inputs(w):
    """Weights and queries of a workload, drawn once per test session."""
    key = (w.name, w.seed, w.batch)
    if key not in _INPUTS:
        _INPUTS[key] = (W.weights(w), W.queries(w))
    return _INPUTS[key]


def _ref(w, b, ctx, positions, spike=None):
    """The oracle's decode of sequence b (memoised: the same sequence serves
    several split counts)."""
    key = (w.name, w.seed, w.cache_dtype, b, ctx, tuple(np.asarray(positions).tolist()), spike)
    if key not in _REFS:
        _REFS[key] = _ref_uncached(w, b, ctx, positions, spike)
    return _REFS[key]


def _ref_uncached(w, b, ctx, positions, spike):
    rows = W.cache_rows(w, b, 0, ctx)
    c_kv = rows["c_kv"]
    if spike is not None:
        t, j, v = spike
        c_kv[t] = 0.0
        c_kv[t, j] = v
    if w.cache_dtype == "fp8":   # the latents as the fp8 cache holds them
        c_kv = oracle.fp8_dequantize_latent(*oracle.fp8_quantize_latent(c_kv))
    wt, q = _inputs(w)
    return oracle.decode_sequence(q["q_nope"][b], q["q_rope"][b], positions, c_kv, rows["k_rope_raw"],
                                  wt["w_uk"], wt["w_uv"], w.sm_scale, w.rope_base)


def _assert_close(got, ref, b, label=""):
    errs = {"u": vec_rel_err(got["u"][b], ref["u"]), "o": vec_rel_err(got["o"][b], ref["o"]),
            "o_fused": vec_rel_err(got["o_fused"][b], ref["o"]), "lse": scalar_err(got["lse"][b], ref["lse"]),
            "lse_fused": scalar_err(got["lse_fused"][b], ref["lse"])}
    for k, v in errs.items():
        assert v <= 1e-2, (label, b, k, v)
    return errs


def _assert_empty(got, b, label=""):
    for k in ("u", "o", "o_fused"):
        assert np.all(got[k][b] == 0.0), (label, b, k)
    for k in ("lse", "lse_fused"):
        assert np.all(np.isneginf(got[k][b])), (label, b, k)


@pytest.mark.parametrize("num_splits", [13, 64, 256])
def test_batch_over_one_plan_chunk(num_splits):
    _need_gpu()
    from workloads.device import stage
    w = W.custom(name="b300", seed=91, batch=300, n_q=1, ctx=None, ctx_range=(0, 40))
    ctx = W.context_lengths(w).copy()
    ctx[[5, 200, 255, 256, 299]] = 0
    ctx[[1, 257]] = 1
    ctx[[40, 270]] = 1500   # longer than a unit at 64 and 256 splits
    st = stage(w, ctx=ctx)
    total = int(ctx.sum())
    # the plan cuts sequences of both chunks, or runs a unit across the chunk boundary
    plan = Plan(ctx, num_splits)
    straddle = [b for b in range(w.batch) if plan.parts[b] > 1]
    spanning = [u for u in range(num_splits) if {b < 256 for b, *_ in plan.segments(u)} == {True, False}]
    assert any(b < 256 for b in straddle) and (any(b >= 256 for b in straddle) or spanning)
    got = _decode(st, num_splits)
    worst = 0.0
    for b in range(w.batch):
        if ctx[b] == 0:
            _assert_empty(got, b, "empty sequence")
            continue
        errs = _assert_close(got, _ref(w, b, int(ctx[b]), st["positions_host"][b]), b)
        worst = max(worst, max(errs.values()))
    print(f"  300 sequences, {total} tokens, num_splits {num_splits}: worst error {worst:.2e}", flush=True)


def _write_row(st, b, t, c_row):
    """Row t of sequence b becomes [c_row | the workload's own rotated key]
    through the library's append (quantised there for an fp8 cache)."""
    import mla_latent_kv_02_amd as mla
    w = st["workload"]
    rows = W.cache_rows(w, b, t, t + 1)
    raw = np.concatenate([c_row[None, :], rows["k_rope_raw"]], axis=1).astype(np.float32)
    rt = torch.from_numpy(raw).cuda().bfloat16()
    sid = torch.tensor([b], dtype=torch.int32, device="cuda")
    pos = torch.tensor([t], dtype=torch.int32, device="cuda")
    mla.mla_cache_append(st["dims"], st["cache"], sid, pos, rt[:, :w.d_c], rt[:, w.d_c:])


@pytest.mark.parametrize("layout,num_splits", [
    ("paged16", 1), ("paged16", 4), ("paged64", 1), ("paged64", 4), ("fp8", 1), ("fp8", 4), ("fp8_paged64", 1)])
def test_late_spike_redo_path(layout, num_splits):
    _need_gpu()
    from workloads.device import stage
    bs = {"paged16": 16, "paged64": 64, "fp8": 0, "fp8_paged64": 64}[layout]
    ctx = np.array([1500, 700] if bs == 16 else [4700, 1300], np.int32)
    w = W.custom(name=f"spike_{layout}", seed=92 + bs, batch=2, n_q=1, ctx=None, ctx_range=(1, 1), block_size=bs)
    if layout.startswith("fp8"):
        w = W.with_fp8_cache(w)
    if bs:   # the long segment spans more blocks than the id window holds
        assert ctx[0] // bs > 64
    st = stage(w, ctx=ctx)
    spikes = {0: (int(ctx[0]) - 60, 5, 2048.0), 1: (int(ctx[1]) // 2, 300, -2048.0)}
    for b, (t, j, v) in spikes.items():
        c = np.zeros(w.d_c, np.float32)
        c[j] = v
        _write_row(st, b, t, c)
    torch.cuda.synchronize()
    got = _decode(st, num_splits)
    for b in range(w.batch):
        ref = _ref(w, b, int(ctx[b]), st["positions_host"][b], spike=spikes[b])
        # the redo path runs: the spike lifts many heads' lse (hence their row
        # maximum) above anything before it by more than the 64 log2 units of
        # headroom the kernel's reference allows
        bulk = _ref(w, b, int(ctx[b]), st["positions_host"][b])["lse"]
        assert int((ref["lse"] - bulk > 64 * np.log(2)).sum()) >= 10
        # Per head: the absorbed path rounds q_lat to bf16, so the spike's own
        # score s carries an error ds <= 2^-9 |s| (2^-8 (|s| + 1) with slack for
        # the positional term).  That moves the spike's softmax share p by
        # p (1 - p) ds, hence u by |v| p (1 - p) ds along e_j, which is compared
        # with max|u|.  From the oracle: p = 1 - exp(bulk - lse) (the one
        # replaced ordinary token aside), s = lse + ln p.  Heads the spike
        # dominates (p ~ 1: the redo path) or barely touches keep 1e-2.
        vj = abs(spikes[b][2])
        p = np.clip(1.0 - np.exp(bulk - ref["lse"]), 1e-300, 1.0)
        s_spike = ref["lse"] + np.log(p)
        ds = 2.0 ** -8 * (np.abs(s_spike) + 1.0)
        tol = 1e-2 + vj * p * (1.0 - p) * ds / np.abs(ref["u"]).max(-1)       # [n_q][n_h]
        worst = {}
        for k, key in (("u", "u"), ("o", "o"), ("o_fused", "o")):
            for jq in range(w.n_q):
                for h in range(w.n_h):
                    e = vec_rel_err(got[k][b][jq, h][None], ref[key][jq, h][None])
                    assert e <= tol[jq, h], (layout, b, k, jq, h, e, tol[jq, h], p[jq, h])
                    worst[k] = max(worst.get(k, 0.0), e)
        for k in ("lse", "lse_fused"):
            e = scalar_err(got[k][b], ref["lse"])
            assert e <= 1e-2, (layout, b, k, e)
            worst[k] = e
        dominated = int((p > 0.99).sum())
        print(f"  {layout} splits {num_splits} seq {b}: spike dominates {dominated} heads; max tol "
              f"{tol.max():.3f}; " + " ".join(f"{k}={v:.2e}" for k, v in worst.items()), flush=True)


@pytest.mark.parametrize("bs", [16, 64])
def test_append_without_a_block_writes_nothing(bs, monkeypatch):
    _need_gpu()
    import mla_latent_kv_02_amd as mla
    from mla_latent_kv_02_amd.contract import ContractError
    from workloads.device import stage
    w = W.custom(name=f"noblock{bs}", seed=95, batch=2, n_q=1, ctx=None, ctx_range=(1, 1), block_size=bs)
    ctx = np.array([3 * bs - 5, bs + 3], np.int32)      # table rows of 3 blocks; sequence 1 holds 2
    st = stage(w, ctx=ctx)
    table = st["block_table_host"]
    assert table.shape[1] == 3 and table[1, 2] == -1
    before = st["cache"].data.view(torch.int16).clone()
    # sequence 1 at a position in its unreserved third block, sequence 0 past
    # the table row, a negative position: nothing is written
    sid = torch.tensor([1, 0, 0], dtype=torch.int32, device="cuda")
    pos = torch.tensor([2 * bs + 1, 3 * bs, -1], dtype=torch.int32, device="cuda")
    raw = torch.randn((3, w.row), device="cuda").bfloat16()
    # the host-side contract check names the first breach (and launches nothing)
    monkeypatch.setenv("MLA_CHECK_CONTRACT", "1")
    with pytest.raises(ContractError, match="goes to block id -1"):
        mla.mla_cache_append(st["dims"], st["cache"], sid[:1], pos[:1], raw[:1, :w.d_c], raw[:1, w.d_c:])
    with pytest.raises(ContractError, match=f"positions\\[1\\] = {3 * bs} outside"):
        mla.mla_cache_append(st["dims"], st["cache"], sid, pos, raw[:, :w.d_c], raw[:, w.d_c:])
    torch.cuda.synchronize()
    assert torch.equal(st["cache"].data.view(torch.int16), before)
    # without it, the kernel's own guards keep the breach from writing
    monkeypatch.setenv("MLA_CHECK_CONTRACT", "0")
    mla.mla_cache_append(st["dims"], st["cache"], sid, pos, raw[:, :w.d_c], raw[:, w.d_c:])
    torch.cuda.synchronize()
    assert torch.equal(st["cache"].data.view(torch.int16), before)
    # control: a position with a block is written
    mla.mla_cache_append(st["dims"], st["cache"], sid[:1], torch.tensor([bs], dtype=torch.int32, device="cuda"),
                         raw[:1, :w.d_c], raw[:1, w.d_c:])
    torch.cuda.synchronize()
    assert not torch.equal(st["cache"].data.view(torch.int16), before)


@pytest.mark.parametrize("bs", [16, 64])
def test_decode_range_the_descriptor_cannot_place_is_empty(bs, monkeypatch):
    _need_gpu()
    from mla_latent_kv_02_amd.contract import ContractError
    from workloads.device import stage
    w = W.custom(name=f"badtable{bs}", seed=96, batch=3, n_q=1, ctx=None, ctx_range=(1, 1), block_size=bs)
    ctx = np.array([4 * bs - 7, 3 * bs + 2, 2 * bs + 9], np.int32)
    st = stage(w, ctx=ctx)
    max_blocks = st["block_table_host"].shape[1]
    # sequence 1: a block in the middle of its range is not reserved (-1)
    st["cache"].block_table[1, 1] = -1
    # sequence 2: the context runs past the table row (max_blocks * bs tokens)
    long_ctx = max_blocks * bs + 5
    st["cache"].ctx_lens[2] = long_ctx
    st["positions"][2, 0] = long_ctx - 1
    torch.cuda.synchronize()
    monkeypatch.setenv("MLA_CHECK_CONTRACT", "1")
    with pytest.raises(ContractError, match=f"ctx_lens\\[2\\] = {long_ctx} outside"):
        _decode(st, num_splits=1)
    st["cache"].ctx_lens[2] = int(ctx[2])
    with pytest.raises(ContractError, match="sequence 1: block 1 .* has id -1"):
        _decode(st, num_splits=1)
    st["cache"].ctx_lens[2] = long_ctx
    monkeypatch.setenv("MLA_CHECK_CONTRACT", "0")
    got = _decode(st, num_splits=1)
    _assert_close(got, _ref(w, 0, int(ctx[0]), st["positions_host"][0]), 0, "valid sequence")
    _assert_empty(got, 1, "negative block id")
    _assert_empty(got, 2, "past the table row")
