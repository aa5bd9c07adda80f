"""Multi-step decode over a growing paged cache (DecodeSession): every step's
output against the fp64 oracle over all rows appended so far, with blocks of 16
tokens so that sequences cross block boundaries while they grow, and a
sequence released mid-run whose slot takes a new, shorter sequence.
Tolerance as for the other bf16 parity cases: 1e-2 max vector relative error."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests._metrics import scalar_err, vec_rel_err

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("n_q", [1, 2])
def test_session_steps_against_oracle(n_q):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_latent_kv_02_amd as mla
    from mla_latent_kv_02_amd.step import DecodeSession
    from workloads.device import dims_of, to_device
    w = W.custom(name="session", seed=40 + n_q, batch=3, n_q=n_q, ctx=1, block_size=16)
    dims = dims_of(w)
    wt = W.weights(w)
    w_uk, w_uv = to_device(wt["w_uk"], "bf16", "cuda"), to_device(wt["w_uv"], "bf16", "cuda")
    rng = np.random.default_rng(100 + n_q)
    bf = lambda *shape: W.round_to_bf16(rng.standard_normal(shape).astype(np.float32))
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()
    B, H = w.batch, w.n_h
    sess = DecodeSession(dims, B, n_q, num_splits=5, dtype=torch.bfloat16, n_blocks=24, block_size=16,
                         max_blocks=8)
    rows_c = [np.zeros((0, w.d_c), np.float32) for _ in range(B)]
    rows_r = [np.zeros((0, w.d_rope), np.float32) for _ in range(B)]

    def prefill(b, n):
        c, r = bf(n, w.d_c), bf(n, w.d_rope)
        start = len(rows_c[b])
        sess.append(np.full(n, b), np.arange(start, start + n), dev(c), dev(r))
        rows_c[b] = np.concatenate([rows_c[b], c])
        rows_r[b] = np.concatenate([rows_r[b], r])

    for b, n in enumerate((5, 31, 16)):
        prefill(b, n)
    for it in range(7):
        if it == 3:                       # sequence 1 ends; its slot takes a new sequence of 9 tokens
            free_before = sess.pool.free_count
            sess.release(1)
            assert sess.pool.free_count > free_before
            rows_c[1] = np.zeros((0, w.d_c), np.float32)
            rows_r[1] = np.zeros((0, w.d_rope), np.float32)
            prefill(1, 9)
        c_new, r_new = bf(B, n_q, w.d_c), bf(B, n_q, w.d_rope)
        qn, qr = bf(B, n_q, H, w.d_nope), bf(B, n_q, H, w.d_rope)
        ctx_before = sess.ctx.copy()
        out = sess.step(dev(c_new), dev(r_new), dev(qn), dev(qr), w_uk, w_uv)
        torch.cuda.synchronize()
        got_o = out.cpu().numpy().astype(np.float64)
        got_l = sess.work.lse.cpu().numpy().astype(np.float64)
        for b in range(B):
            rows_c[b] = np.concatenate([rows_c[b], c_new[b]])
            rows_r[b] = np.concatenate([rows_r[b], r_new[b]])
            qpos = ctx_before[b] + np.arange(n_q)
            ref = oracle.decode_sequence(qn[b], qr[b], qpos, rows_c[b], rows_r[b], wt["w_uk"], wt["w_uv"],
                                         w.sm_scale, w.rope_base)
            eo, el = vec_rel_err(got_o[b], ref["o"]), scalar_err(got_l[b], ref["lse"])
            print(f"  step {it} seq {b} ctx {len(rows_c[b])}: o={eo:.2e} lse={el:.2e}", flush=True)
            assert eo <= 1e-2 and el <= 1e-2, (it, b, eo, el)
        assert (sess.ctx == np.array([len(r) for r in rows_c])).all()
    # every block a sequence holds is its own, and the table on the device is the pool's
    held = sess.pool.table[sess.pool.table >= 0]
    assert len(held) == len(set(held.tolist()))
    np.testing.assert_array_equal(sess.table_dev.cpu().numpy(), sess.pool.table)
