"""GPU parity of prefill / chunked prefill (mla_prefill) against the oracle.

The oracle's decode_sequence rebuilds K_i = [C W_UK_i | RoPE(k_raw)] and
V_i = C W_UV_i and runs the causal softmax for every query token: exactly
the prefill definition.  The GPU path rebuilds the per-head keys and values
into the workspace (bf16) and runs the causal attention; tolerance as for
the bf16 decode path (1e-2 max vector relative error; lse absolute 1e-2).
The oracle is run on a subset of heads to keep it fast; the GPU computes
all 128.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests._metrics import scalar_err, vec_rel_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

HEADS = [0, 1, 37, 64, 127]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _prefill(st):
    """max_ctx = the cache's rows per sequence (NaN past each context)."""
    import mla_latent_kv_02_amd as mla
    w = st["workload"]
    max_ctx = st["cache"].data.shape[1]
    d = st["dims"]
    w_kv = torch.empty((w.n_h, w.d_nope + w.d_v, w.d_c), dtype=torch.bfloat16, device="cuda")
    mla.mla_prefill_weights(d, st["w_uk"], st["w_uv"], w_kv)
    ws = torch.full((mla.mla_prefill_workspace_bytes(d, w.batch, max_ctx) // 2,), float("nan"),
                    dtype=torch.bfloat16, device="cuda")
    q_pe = torch.full((w.batch, w.n_q, w.n_h, w.d_rope), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = torch.full((w.batch, w.n_q, w.n_h, w.d_v), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((w.batch, w.n_q, w.n_h), float("nan"), dtype=torch.float32, device="cuda")
    mla.mla_prefill(d, max_ctx, st["q_nope"], st["q_rope"], st["positions"], st["cache"], w_kv, ws, q_pe, out, lse)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().astype(np.float64)
    return {"w_kv": w_kv, "kv": ws.view(w.batch, max_ctx, w.n_h, w.d_nope + w.d_v), "q_pe": f(q_pe),
            "o": f(out), "lse": f(lse)}


def _check(w, st, got, heads=HEADS, spikes=None, keys=("o", "lse", "q_pe")):
    """spikes: {sequence: (token, latent index j, value)}: the test set that
    token's latent row to value * e_j on the device."""
    wt, q = W.weights(w), W.queries(w)
    for b in range(w.batch):
        ctx = int(st["ctx_host"][b])
        rows = W.cache_rows(w, b, 0, ctx)
        if spikes and b in spikes:
            t, j, v = spikes[b]
            rows["c_kv"][t] = 0.0
            rows["c_kv"][t, j] = v
        ref = oracle.decode_sequence(q["q_nope"][b], q["q_rope"][b], st["positions_host"][b], rows["c_kv"],
                                     rows["k_rope_raw"], wt["w_uk"], wt["w_uv"], w.sm_scale, w.rope_base,
                                     heads=heads)
        errs = {"o": vec_rel_err(got["o"][b][:, heads], ref["o"])}
        if "lse" in keys:
            errs["lse"] = scalar_err(got["lse"][b][:, heads], ref["lse"])
        if "q_pe" in keys:
            errs["q_pe"] = vec_rel_err(got["q_pe"][b][:, heads], ref["q_pe"])
        print(f"  seq {b} ctx {ctx} n_q {w.n_q}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
        for k, v in errs.items():
            assert v <= 1e-2, (b, k, v)


def test_prefill_weights_layout():
    _need_gpu()
    from workloads.device import stage
    w = W.custom(name="pf_w", seed=61, batch=1, n_q=1, ctx=None, ctx_range=(1, 1))
    st = stage(w, ctx=np.array([4], np.int32))
    got = _prefill(st)["w_kv"].view(torch.int16).cpu().numpy()
    uk = st["w_uk"].view(torch.int16).cpu().numpy()
    uv = st["w_uv"].view(torch.int16).cpu().numpy()
    np.testing.assert_array_equal(got[:, :128, :], uk.transpose(0, 2, 1))
    np.testing.assert_array_equal(got[:, 128:, :], uv.transpose(0, 2, 1))


@pytest.mark.parametrize("ctx,n_q", [([200, 200], 200), ([300, 257], 100), ([130, 64], 64), ([64, 1], 1),
                                     ([333], 290)])
def test_prefill_matches_oracle(ctx, n_q):
    """Whole prompts (n_q = ctx), chunks after a prefix, a whole prompt next to a
    chunk, a single token; query counts that are not multiples of the 128-row
    block (290 spans three blocks), contexts that are not multiples of the
    32-token stage.  The cache past each context is NaN."""
    _need_gpu()
    from workloads.device import stage
    w = W.custom(name="pf", seed=62, batch=len(ctx), n_q=n_q, ctx=None, ctx_range=(1, 1))
    st = stage(w, ctx=np.array(ctx, np.int32))
    got = _prefill(st)
    _check(w, st, got)


def test_prefill_reconstruction_in_workspace():
    """The workspace rows t < ctx hold c_t W_UK_i | c_t W_UV_i (bf16 rounding of
    an fp32-accumulated product), checked on sampled (token, head) pairs."""
    _need_gpu()
    from workloads.device import stage
    w = W.custom(name="pf_kv", seed=63, batch=2, n_q=40, ctx=None, ctx_range=(1, 1))
    st = stage(w, ctx=np.array([97, 40], np.int32))
    got = _prefill(st)
    kv = got["kv"].float().cpu().numpy().astype(np.float64)
    wt = W.weights(w)
    rng = np.random.default_rng(64)
    for b in range(2):
        rows = W.cache_rows(w, b, 0, int(st["ctx_host"][b]))
        for _ in range(12):
            t = int(rng.integers(0, len(rows["c_kv"])))
            i = int(rng.integers(0, w.n_h))
            k = oracle.reconstruct_keys(rows["c_kv"][t:t + 1], wt["w_uk"], i)[0]
            v = oracle.reconstruct_values(rows["c_kv"][t:t + 1], wt["w_uv"], i)[0]
            ref = np.concatenate([k, v])
            assert np.abs(kv[b, t, i] - ref).max() <= 2 ** -8 * np.abs(ref).max() + 1e-6, (b, t, i)


def test_prefill_agrees_with_the_decode_path():
    """The same queries through mla_decode + merge + up-projection (absorbed
    form) and through mla_prefill (rebuilt K/V): both equal the oracle, so they
    agree with each other to the bf16 tolerance (checked on every head)."""
    _need_gpu()
    from mla_latent_kv_02_amd.step import DecodeStep
    from workloads.device import stage
    w = W.custom(name="pf_dec", seed=65, batch=2, n_q=3, ctx=None, ctx_range=(1, 1))
    st = stage(w, ctx=np.array([150, 33], np.int32))
    got = _prefill(st)
    step = DecodeStep(st["dims"], w.batch, w.n_q, 4, torch.bfloat16)
    step.run(st["q_nope"], st["q_rope"], st["positions"], st["w_uk"], st["w_uv"], st["cache"])
    torch.cuda.synchronize()
    dec = step.out.float().cpu().numpy().astype(np.float64)
    assert vec_rel_err(got["o"], dec) <= 2e-2
    _check(w, st, got)


def test_late_large_score_prefill_and_decode():
    """One late token's latent row is 2048 e_j (a power of two times a unit
    vector), so its rebuilt key and value are 2048 times rows of the bf16
    weights: exact in bf16, and the prefill scores stay exact to fp32
    accumulation.  Its scores (about +-100 in log2 units) pass many rows'
    running maximum by far more than the kernels' headroom in a late stage: the
    prefill accumulator is rescaled there, and the decode kernel computes those
    rows' segment again with the true maximum as reference.  In the absorbed
    decode path the spike's score carries the bf16 rounding of q_lat[j]
    (relative 2^-9), which matters only where that score is near the row's
    other scores, i.e. small.  Both paths against the oracle on the same rows;
    the queries before the token do not see it."""
    _need_gpu()
    from mla_latent_kv_02_amd.step import DecodeStep
    from workloads.device import stage
    w = W.custom(name="pf_spike", seed=66, batch=2, n_q=64, ctx=None, ctx_range=(1, 1))
    st = stage(w, ctx=np.array([300, 150], np.int32))
    spikes = {0: (260, 5, 2048.0), 1: (120, 300, -2048.0)}
    for b, (t, j, v) in spikes.items():
        st["cache"].data[b, t, :w.d_c] = 0
        st["cache"].data[b, t, j] = v
    torch.cuda.synchronize()
    _check(w, st, _prefill(st), spikes=spikes)
    for num_splits in (1, 4):
        step = DecodeStep(st["dims"], w.batch, w.n_q, num_splits, torch.bfloat16)
        step.run(st["q_nope"], st["q_rope"], st["positions"], st["w_uk"], st["w_uv"], st["cache"])
        torch.cuda.synchronize()
        dec = step.out.float().cpu().numpy().astype(np.float64)
        _check(w, st, {"o": dec}, spikes=spikes, keys=("o",))


@pytest.mark.parametrize("batch,ctx,n_q", [(1, 4096, 4096), (4, 8192, 1024)], ids=["prompt4k", "chunk1k"])
def test_prefill_full_size_sampled(batch, ctx, n_q):
    """The two benchmark shapes (a 4096-token prompt; 1024-token chunks after
    7168 cached tokens, 4 sequences) through the same entry point the bench
    times, checked against the oracle on sampled query rows (the first and last
    of the chunk, both sides of a 128-row block boundary, the middle) and
    heads; the oracle rebuilds K/V of those heads over the whole context."""
    _need_gpu()
    from workloads.device import stage
    w = W.custom(name=f"pf_full_{ctx}_{n_q}", seed=81, batch=batch, n_q=n_q, ctx=ctx)
    st = stage(w)
    got = _prefill(st)
    wt, q = W.weights(w), W.queries(w)
    rows_q = sorted({0, 127, 128, n_q // 2, n_q - 1})
    heads = [0, 77, 127]
    for b in range(batch):
        rows = W.cache_rows(w, b, 0, ctx)
        ref = oracle.decode_sequence(q["q_nope"][b][rows_q], q["q_rope"][b][rows_q],
                                     st["positions_host"][b][rows_q], rows["c_kv"], rows["k_rope_raw"],
                                     wt["w_uk"], wt["w_uv"], w.sm_scale, w.rope_base, heads=heads)
        o = got["o"][b][rows_q][:, heads]
        lse = got["lse"][b][rows_q][:, heads]
        errs = {"o": vec_rel_err(o, ref["o"]), "lse": scalar_err(lse, ref["lse"])}
        print(f"  seq {b} ctx {ctx} rows {rows_q}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
        for k, v in errs.items():
            assert v <= 1e-2, (b, k, v)
