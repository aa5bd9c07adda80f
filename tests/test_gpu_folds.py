"""GPU parity of the weight folds against the fp64 oracle, through the C ABI.

Value side [Huny §3.2]: W_comb,i = W_i^UV W_i^O (mla_fold_out) and the layer
output through it (mla_out_proj_folded) or without it (mla_out_proj, then
mla_o_proj).  Query side [Paldyn, section MLA]: W_KQ,i = W_i^UQ (W_i^UK)^T
(mla_fold_q) and q_lat from the compressed query (mla_absorb_q_folded).
V3 head shapes (n_h=128, d_c=512, d_nope=d_v=128), d_q=1536, d_model up to
7168.  Weights bf16, N(0, 1/fan_in); tolerance 1e-2 max vector relative error
(bf16 operands, fp32 accumulation; the folded weights add one bf16 rounding);
the folded matrices are checked on sampled entries, each a plain dot product.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from tests._metrics import vec_rel_err

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _dev_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).cuda()


@pytest.mark.parametrize("d_model", [1024, 7168])
def test_output_fold_and_layer_output(d_model):
    _need_gpu()
    import mla_latent_kv_02_amd as mla
    from workloads.device import dims_of
    w = W.custom(name="fold_out", seed=50, batch=3, n_q=2, ctx=1)
    dims = dims_of(w)
    rng = np.random.default_rng(51)
    w_uv = W.weights(w)["w_uv"]                                    # [n_h][d_c][d_v], bf16 values
    w_o = W.round_to_bf16((rng.standard_normal((w.n_h, w.d_v, d_model)) /
                           np.sqrt(w.n_h * w.d_v)).astype(np.float32))     # W_i^O blocks
    u = rng.standard_normal((w.batch, w.n_q, w.n_h, w.d_c)).astype(np.float32)
    w_uv_d, w_o_d = _dev_bf16(w_uv), _dev_bf16(w_o.transpose(2, 0, 1))    # w_o as [d_model][n_h][d_v]
    u_d = torch.from_numpy(u).cuda()
    w_comb = torch.empty((d_model, w.n_h, w.d_c), dtype=torch.bfloat16, device="cuda")
    mla.mla_fold_out(dims, w_uv_d, w_o_d, w_comb)
    y_f = torch.full((w.batch, w.n_q, d_model), float("nan"), device="cuda")
    mla.mla_out_proj_folded(dims, u_d, w_comb, y_f)
    o = torch.empty((w.batch, w.n_q, w.n_h, w.d_v), device="cuda")
    mla.mla_out_proj(dims, u_d, w_uv_d, o)
    y_u = torch.full((w.batch, w.n_q, d_model), float("nan"), device="cuda")
    mla.mla_o_proj(dims, o, w_o_d, y_u)
    torch.cuda.synchronize()
    ref = oracle.output_projection(oracle.value_up_projection(u.astype(np.float64), w_uv), w_o)
    e_f = vec_rel_err(y_f.cpu().numpy(), ref)
    e_u = vec_rel_err(y_u.cpu().numpy(), ref)
    # sampled entries of the folded matrix, each one dot product of length d_v
    wc = w_comb.float().cpu().numpy()
    idx = rng.integers(0, [d_model, w.n_h, w.d_c], size=(256, 3))
    got = np.array([wc[n, i, c] for n, i, c in idx])
    want = np.array([w_uv[i, c, :].astype(np.float64) @ w_o[i, :, n] for n, i, c in idx])
    e_c = np.abs(got - want).max() / np.abs(want).max()
    print(f"  d_model {d_model}: folded y {e_f:.2e}, unfolded y {e_u:.2e}, W_comb samples {e_c:.2e}", flush=True)
    assert e_f <= 1e-2 and e_u <= 1e-2 and e_c <= 1e-2


def test_query_fold_and_folded_absorption():
    _need_gpu()
    import mla_latent_kv_02_amd as mla
    from workloads.device import dims_of
    w = W.custom(name="fold_q", seed=52, batch=3, n_q=2, ctx=1)
    dims = dims_of(w)
    d_q = 1536
    rng = np.random.default_rng(53)
    w_uk = W.weights(w)["w_uk"]                                    # [n_h][d_c][d_nope]
    w_uq = W.round_to_bf16((rng.standard_normal((w.n_h, d_q, w.d_nope)) / np.sqrt(d_q)).astype(np.float32))
    c_q = W.round_to_bf16(rng.standard_normal((w.batch, w.n_q, d_q)).astype(np.float32))
    q_rope = W.round_to_bf16(rng.standard_normal((w.batch, w.n_q, w.n_h, w.d_rope)).astype(np.float32))
    pos = rng.integers(0, 100000, size=(w.batch, w.n_q)).astype(np.int32)
    w_kq = torch.empty((w.n_h, w.d_c, d_q), dtype=torch.bfloat16, device="cuda")
    mla.mla_fold_q(dims, _dev_bf16(w_uq.transpose(1, 0, 2)), _dev_bf16(w_uk), w_kq)   # w_uq as [d_q][n_h][d_nope]
    q_lat = torch.empty((w.batch, w.n_q, w.n_h, w.d_c), dtype=torch.bfloat16, device="cuda")
    q_pe = torch.empty((w.batch, w.n_q, w.n_h, w.d_rope), dtype=torch.bfloat16, device="cuda")
    mla.mla_absorb_q_folded(dims, _dev_bf16(c_q), _dev_bf16(q_rope), torch.from_numpy(pos).cuda(), w_kq, q_lat, q_pe)
    torch.cuda.synchronize()
    ref_lat = oracle.absorb_query(oracle.query_from_compressed(c_q.astype(np.float64), w_uq), w_uk)
    ref_pe = np.stack([[oracle.rope_rotate(q_rope[b, j], np.full(w.n_h, pos[b, j]), w.rope_base)
                        for j in range(w.n_q)] for b in range(w.batch)])
    e_lat = vec_rel_err(q_lat.float().cpu().numpy(), ref_lat)
    e_pe = vec_rel_err(q_pe.float().cpu().numpy(), ref_pe)
    kq = w_kq.float().cpu().numpy()
    idx = rng.integers(0, [w.n_h, w.d_c, d_q], size=(256, 3))
    got = np.array([kq[i, c, q] for i, c, q in idx])
    want = np.array([w_uq[i, q, :].astype(np.float64) @ w_uk[i, c, :] for i, c, q in idx])
    e_kq = np.abs(got - want).max() / np.abs(want).max()
    print(f"  q_lat {e_lat:.2e}, q_pe {e_pe:.2e}, W_KQ samples {e_kq:.2e}", flush=True)
    assert e_lat <= 1e-2 and e_pe <= 1e-2 and e_kq <= 1e-2


def test_products_over_ragged_tiles_and_k_slices():
    """The per-step products at shapes that cut their tiles: 70 query rows (a
    second, ragged 64-row tile), d_model 300 (a 256-column tile and a ragged
    one in which three of the four waves hold no column), K = n_h d_v = 16384
    and n_h d_c = 65536 cut into slices added into C (fp32 C), and the folded
    absorption's 128 head products over 70 rows (bf16 C, one slice)."""
    _need_gpu()
    import mla_latent_kv_02_amd as mla
    from workloads.device import dims_of
    w = W.custom(name="fold_tiles", seed=54, batch=35, n_q=2, ctx=1)
    dims = dims_of(w)
    d_model, d_q = 300, 1536
    rng = np.random.default_rng(55)
    w_uv = W.weights(w)["w_uv"]
    w_o = W.round_to_bf16((rng.standard_normal((w.n_h, w.d_v, d_model)) /
                           np.sqrt(w.n_h * w.d_v)).astype(np.float32))
    u = rng.standard_normal((w.batch, w.n_q, w.n_h, w.d_c)).astype(np.float32)
    o = rng.standard_normal((w.batch, w.n_q, w.n_h, w.d_v)).astype(np.float32)
    w_uv_d, w_o_d = _dev_bf16(w_uv), _dev_bf16(w_o.transpose(2, 0, 1))
    y_o = torch.full((w.batch, w.n_q, d_model), float("nan"), device="cuda")
    mla.mla_o_proj(dims, torch.from_numpy(o).cuda(), w_o_d, y_o)
    w_comb = torch.empty((d_model, w.n_h, w.d_c), dtype=torch.bfloat16, device="cuda")
    mla.mla_fold_out(dims, w_uv_d, w_o_d, w_comb)
    y_f = torch.full((w.batch, w.n_q, d_model), float("nan"), device="cuda")
    mla.mla_out_proj_folded(dims, torch.from_numpy(u).cuda(), w_comb, y_f)
    w_uk = W.weights(w)["w_uk"]
    w_uq = W.round_to_bf16((rng.standard_normal((w.n_h, d_q, w.d_nope)) / np.sqrt(d_q)).astype(np.float32))
    c_q = W.round_to_bf16(rng.standard_normal((w.batch, w.n_q, d_q)).astype(np.float32))
    q_rope = W.round_to_bf16(rng.standard_normal((w.batch, w.n_q, w.n_h, w.d_rope)).astype(np.float32))
    pos = rng.integers(0, 100000, size=(w.batch, w.n_q)).astype(np.int32)
    w_kq = torch.empty((w.n_h, w.d_c, d_q), dtype=torch.bfloat16, device="cuda")
    mla.mla_fold_q(dims, _dev_bf16(w_uq.transpose(1, 0, 2)), _dev_bf16(w_uk), w_kq)
    q_lat = torch.full((w.batch, w.n_q, w.n_h, w.d_c), float("nan"), dtype=torch.bfloat16, device="cuda")
    q_pe = torch.empty((w.batch, w.n_q, w.n_h, w.d_rope), dtype=torch.bfloat16, device="cuda")
    mla.mla_absorb_q_folded(dims, _dev_bf16(c_q), _dev_bf16(q_rope), torch.from_numpy(pos).cuda(), w_kq, q_lat, q_pe)
    torch.cuda.synchronize()
    e_o = vec_rel_err(y_o.cpu().numpy(), oracle.output_projection(o.astype(np.float64), w_o))
    ref_f = oracle.output_projection(oracle.value_up_projection(u.astype(np.float64), w_uv), w_o)
    e_f = vec_rel_err(y_f.cpu().numpy(), ref_f)
    ref_lat = oracle.absorb_query(oracle.query_from_compressed(c_q.astype(np.float64), w_uq), w_uk)
    e_lat = vec_rel_err(q_lat.float().cpu().numpy(), ref_lat)
    print(f"  o W_O^T {e_o:.2e}, u W_comb^T {e_f:.2e}, c_q W_KQ^T {e_lat:.2e}", flush=True)
    assert e_o <= 1e-2 and e_f <= 1e-2 and e_lat <= 1e-2
