"""The decode step for callers that cannot allocate (mla_decode_out_noalloc),
through the C ABI, against the entry points it stands for: mla_decode into
caller-allocated partials followed by mla_combine_out_proj.  Two calls in a
row, the second with a smaller input (fewer sequences, shorter contexts,
fewer splits), so the second runs over a scratch that still holds the first
call's partials; the outputs must be identical (the same kernels on the same
inputs), which meets any tolerance.  A size beyond the scratch is refused
before anything is enqueued."""
import numpy as np
import pytest

import workloads as W
from tests.test_gpu_parity import _need_gpu, torch

pytestmark = pytest.mark.gpu


CALLS = [
    # (batch, contexts, n_q, block_size, num_splits)
    (6, [900, 35, 640, 2, 777, 300], 2, 64, 11),
    (3, [130, 64, 2], 1, 0, 4),
]


def test_noalloc_matches_the_allocating_path():
    _need_gpu()
    import mla_latent_kv_02_amd as mla
    from mla_latent_kv_02_amd.step import DecodeStep
    from workloads.device import stage
    for call, (B, ctx, n_q, bs, ns) in enumerate(CALLS):
        w = W.custom(name=f"noalloc{call}", seed=97 + call, batch=B, n_q=n_q, ctx=None, ctx_range=(1, 1),
                     block_size=bs)
        st = stage(w, ctx=np.array(ctx, np.int32))
        d = st["dims"]
        step = DecodeStep(d, B, n_q, ns, torch.bfloat16)
        mla.mla_absorb_q(d, st["q_nope"], st["q_rope"], st["positions"], st["w_uk"], step.q_lat, step.q_pe)
        # the allocating path
        mla.mla_decode(d, step.q_lat, step.q_pe, st["cache"], st["positions"], ns, step.u_part, step.lse_part)
        mla.mla_combine_out_proj(d, st["cache"].ctx_lens, ns, step.u_part, step.lse_part, st["w_uv"], step.out,
                                 step.lse)
        # the step without allocation
        out = torch.full_like(step.out, float("nan"))
        lse = torch.full_like(step.lse, float("nan"))
        mla.mla_decode_out_noalloc(d, step.q_lat, step.q_pe, st["cache"], st["positions"], ns, st["w_uv"], out, lse)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all() and torch.isfinite(lse).all()
        assert torch.equal(out, step.out), (call, float((out - step.out).abs().max()))
        assert torch.equal(lse, step.lse), call
        print(f"  call {call}: B={B} n_q={n_q} block {bs} splits {ns}: identical", flush=True)
    # beyond the scratch: refused on the host
    with pytest.raises(mla.MlaError) as e:
        mla.mla_decode_out_noalloc(d, step.q_lat, step.q_pe, st["cache"], st["positions"], 600, st["w_uv"], out)
    assert e.value.status == 5
