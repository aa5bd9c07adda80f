"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own formulas: printed figures
from the pages (tests/golden), closed forms, invariants, a pure-Python
brute force on tiny inputs, a library routine (torch SDPA in fp64), and the
absorption identity the pages verify.  The mutation tests at the end plant
plausible mistakes in copies of the oracle and check that a pin fails.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import mla_oracle as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _problem(seed, n_q=1, n_h=3, d_c=8, d_nope=4, d_rope=4, d_v=5, S=7, base=10000.0):
    r = _rng(seed)
    return dict(
        q_nope=r.standard_normal((n_q, n_h, d_nope)),
        q_rope=r.standard_normal((n_q, n_h, d_rope)),
        q_positions=np.arange(S - n_q, S),
        c_kv=r.standard_normal((S, d_c)),
        k_rope_raw=r.standard_normal((S, d_rope)),
        w_uk=r.standard_normal((n_h, d_c, d_nope)) / math.sqrt(d_c),
        w_uv=r.standard_normal((n_h, d_c, d_v)) / math.sqrt(d_c),
        sm_scale=1.0 / math.sqrt(d_nope + d_rope),
        rope_base=base,
    )


# ------------------------------------------------------------ brute force
def brute_force(q_nope, q_rope, q_positions, c_kv, k_rope_raw, w_uk, w_uv, sm_scale, rope_base,
                kv_positions=None):
    """Scalar-loop MLA decode written from the definitions with the math module."""
    n_q, n_h, d_nope = len(q_nope), len(q_nope[0]), len(q_nope[0][0])
    d_rope = len(q_rope[0][0])
    S, d_c = len(c_kv), len(c_kv[0])
    d_v = len(w_uv[0][0])
    kvp = list(range(S)) if kv_positions is None else [int(p) for p in kv_positions]

    def rot(x, p):
        y = [0.0] * d_rope
        for k in range(d_rope // 2):
            theta = rope_base ** (-(2.0 * k) / d_rope)
            a = p * theta
            y[2 * k] = x[2 * k] * math.cos(a) - x[2 * k + 1] * math.sin(a)
            y[2 * k + 1] = x[2 * k] * math.sin(a) + x[2 * k + 1] * math.cos(a)
        return y

    out = {"o": [], "u": [], "lse": [], "q_lat": [], "q_pe": []}
    kr = [rot(list(k_rope_raw[s]), kvp[s]) for s in range(S)]
    for j in range(n_q):
        o_j, u_j, l_j, ql_j, qp_j = [], [], [], [], []
        for i in range(n_h):
            qpe = rot(list(q_rope[j][i]), int(q_positions[j]))
            qlat = [sum(q_nope[j][i][k] * w_uk[i][c][k] for k in range(d_nope)) for c in range(d_c)]
            scores = []
            for s in range(S):
                if kvp[s] > q_positions[j]:
                    continue
                kc = [sum(c_kv[s][c] * w_uk[i][c][k] for c in range(d_c)) for k in range(d_nope)]
                dot = sum(q_nope[j][i][k] * kc[k] for k in range(d_nope))
                dot += sum(qpe[r] * kr[s][r] for r in range(d_rope))
                scores.append((s, dot * sm_scale))
            m = max(v for _, v in scores)
            z = sum(math.exp(v - m) for _, v in scores)
            probs = [(s, math.exp(v - m) / z) for s, v in scores]
            o = [sum(p * sum(c_kv[s][c] * w_uv[i][c][v] for c in range(d_c)) for s, p in probs)
                 for v in range(d_v)]
            u = [sum(p * c_kv[s][c] for s, p in probs) for c in range(d_c)]
            o_j.append(o), u_j.append(u), l_j.append(m + math.log(z)), ql_j.append(qlat), qp_j.append(qpe)
        for key, val in zip(("o", "u", "lse", "q_lat", "q_pe"), (o_j, u_j, l_j, ql_j, qp_j)):
            out[key].append(val)
    return {k: np.array(v) for k, v in out.items()}


def _compare_to_brute(decode_fn, prob, tol=1e-12):
    got = decode_fn(**prob)
    ref = brute_force(**prob)
    for key in ("o", "u", "lse", "q_lat", "q_pe"):
        scale = max(1.0, float(np.abs(ref[key]).max()))
        err = float(np.abs(np.asarray(got[key]) - ref[key]).max()) / scale
        if not err <= tol:
            return False, key, err
    return True, None, 0.0


@pytest.mark.parametrize("n_q", [1, 2, 3])
@pytest.mark.parametrize("seed", [0, 1])
def test_brute_force_tiny(n_q, seed):
    prob = _problem(seed, n_q=n_q, n_h=2, d_c=4, d_nope=2, d_rope=4, d_v=3, S=5)
    ok, key, err = _compare_to_brute(om.decode_sequence, prob, tol=1e-13)
    assert ok, (key, err)


def test_brute_force_explicit_positions():
    prob = _problem(3, n_q=2, n_h=2, d_c=4, d_nope=2, d_rope=2, d_v=3, S=5)
    kvp = np.array([7, 2, 9, 4, 11])
    prob["q_positions"] = np.array([9, 10])
    got = om.decode_sequence(kv_positions=kvp, **prob)
    ref = brute_force(kv_positions=kvp, **prob)
    for key in ("o", "u", "lse"):
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------ cache figures
def _mib_8k(kind):
    per = {"mha": oracle.mha_cache_bytes_per_token(128, 128, 2),
           "mqa": oracle.gqa_cache_bytes_per_token(1, 128, 2),
           "gqa8": oracle.gqa_cache_bytes_per_token(8, 128, 2),
           "mla": oracle.mla_cache_bytes_per_token(512, 64, 2)}[kind]
    return per * 8192 / 2 ** 20


def test_cache_arithmetic_matches_pages():
    cases = json.load(open(os.path.join(GOLDEN, "cache_arithmetic.json")))["cases"]
    mla = oracle.mla_cache_bytes_per_token(512, 64, 2)
    mha = oracle.mha_cache_bytes_per_token(128, 128, 2)
    gqa8 = oracle.gqa_cache_bytes_per_token(8, 128, 2)
    for c in cases:
        k = c["kind"]
        if k == "mha_bytes":
            assert oracle.mha_cache_bytes_per_token(c["n_h"], c["d_h"], c["b"]) == c["printed"], c
        elif k == "mla_bytes":
            assert oracle.mla_cache_bytes_per_token(c["d_c"], c["d_rope"], c["b"]) == c["printed"], c
        elif k == "mla_elems":
            assert oracle.mla_cache_elements_per_token(c["d_c"], c["d_rope"]) == c["printed"], c
        elif k == "mha_elems":
            assert oracle.mha_cache_bytes_per_token(c["n_h"], c["d_h"], 1) == c["printed"], c
        elif k == "reduction_vs_mha_pct":
            assert round(100 * (1 - mla / mha), c["decimals"]) == c["printed"], c
        elif k == "reduction_vs_gqa8_pct":
            assert round(100 * (1 - mla / gqa8), c["decimals"]) == c["printed"], c
        elif k == "gqa_bytes":
            assert oracle.gqa_cache_bytes_per_token(c["n_kv"], c["d_h"], c["b"]) == c["printed"], c
        elif k == "mib_8k":
            assert _mib_8k(c["per_token"]) == c["printed"], c
        elif k == "share_pct":
            share = oracle.mla_cache_elements_per_token(512, 64) / oracle.mha_cache_bytes_per_token(128, 128, 1)
            assert round(100 * share, c["decimals"]) == c["printed"], c
        elif k == "paged_block_bytes":
            nbytes = c["tokens"] * c["layers"] * oracle.mla_cache_bytes_per_token(c["d_c"], c["d_rope"], c["b"])
            assert round(nbytes / 1e6, c["decimals"]) == c["printed_mb"], c
        else:
            raise AssertionError(f"unknown case {k}")
    # exact forms behind the rounded percentages
    assert 1 - mla / mha == 0.982421875 and 1 - mla / gqa8 == 0.71875


# ------------------------------------------------------------------ RoPE
def test_rope_identity_and_norm():
    r = _rng(5)
    x = r.standard_normal((10, 64))
    np.testing.assert_array_equal(om.rope_rotate(x, 0, 10000.0), x)
    for pos in (1, 17, 131071):
        y = om.rope_rotate(x, pos, 10000.0)
        np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14)
        # each plane keeps its own norm
        np.testing.assert_allclose(y[:, 0::2] ** 2 + y[:, 1::2] ** 2, x[:, 0::2] ** 2 + x[:, 1::2] ** 2,
                                   rtol=1e-12, atol=1e-14)


def test_rope_composition_and_relative_form():
    r = _rng(6)
    q, k = r.standard_normal(64), r.standard_normal(64)
    for a, b in ((3, 5), (100, 4000), (65535, 65536)):
        np.testing.assert_allclose(om.rope_rotate(om.rope_rotate(q, a, 1e4), b, 1e4),
                                   om.rope_rotate(q, a + b, 1e4), rtol=1e-9, atol=1e-9)
    # <R_m q, R_n k> depends only on m - n
    m, n = 40, 13
    ref = om.rope_rotate(q, m, 1e4) @ om.rope_rotate(k, n, 1e4)
    for d in (1, 7, 1000):
        np.testing.assert_allclose(om.rope_rotate(q, m + d, 1e4) @ om.rope_rotate(k, n + d, 1e4), ref,
                                   rtol=1e-9, atol=1e-11)


def test_rope_closed_form_planes():
    # plane 0 always has theta = 1: e_0 -> (cos p, sin p), e_1 -> (-sin p, cos p)
    for p in (1, 2, 255, 131071):
        y = om.rope_rotate(np.array([1.0, 0.0, 0.0, 0.0]), p, 10000.0)
        np.testing.assert_allclose(y, [math.cos(p), math.sin(p), 0, 0], atol=1e-12)
        y = om.rope_rotate(np.array([0.0, 1.0, 0.0, 0.0]), p, 10000.0)
        np.testing.assert_allclose(y, [-math.sin(p), math.cos(p), 0, 0], atol=1e-12)
        # plane 1 of a 4-wide key rotates at 10000^(-1/2) = 0.01 rad per position
        y = om.rope_rotate(np.array([0.0, 0.0, 1.0, 0.0]), p, 10000.0)
        np.testing.assert_allclose(y, [0, 0, math.cos(0.01 * p), math.sin(0.01 * p)], atol=1e-9)


# ----------------------------------------------------- absorption identity
def _absorbed_decode(q_nope, q_rope, q_positions, c_kv, k_rope_raw, w_uk, w_uv, sm_scale, rope_base):
    """The pages' 'Method B': scores against the latent cache, then u W_UV."""
    q_lat = oracle.absorb_query(q_nope, w_uk)
    q_pe = oracle.rope_rotate(q_rope, np.asarray(q_positions)[:, None], rope_base)
    k_r = oracle.rope_rotate(k_rope_raw, np.arange(len(c_kv)), rope_base)
    logits = (np.einsum("jic,sc->jis", q_lat, c_kv) + np.einsum("jir,sr->jis", q_pe, k_r)) * sm_scale
    vis = np.arange(len(c_kv))[None, None, :] <= np.asarray(q_positions)[:, None, None]
    logits = np.where(vis, logits, -np.inf)
    m = logits.max(-1, keepdims=True)
    p = np.exp(logits - m)
    p /= p.sum(-1, keepdims=True)
    u = np.einsum("jis,sc->jic", p, c_kv)
    return logits, p, u, oracle.value_up_projection(u, w_uv)


def test_absorption_matches_reconstruction_v3_shapes():
    """Case 4 of the pages at DeepSeek-V3 head shapes (fewer heads and tokens)."""
    g = json.load(open(os.path.join(GOLDEN, "absorption_case4.json")))
    prob = _problem(7, n_q=1, n_h=4, d_c=512, d_nope=128, d_rope=64, d_v=128, S=64)
    ref = oracle.decode_sequence(**prob)
    logits, p, u, o = _absorbed_decode(**prob)
    lim = g["allowed_factor"]
    # logits: reconstructed-key scores computed independently per head
    for i in range(4):
        kc = oracle.reconstruct_keys(prob["c_kv"], prob["w_uk"], i)
        k_r = oracle.rope_rotate(prob["k_rope_raw"], np.arange(64), 1e4)
        q_pe = oracle.rope_rotate(prob["q_rope"][0, i], prob["q_positions"][0], 1e4)
        rec = (prob["q_nope"][0, i] @ kc.T + q_pe @ k_r.T) * prob["sm_scale"]
        assert np.abs(rec - logits[0, i]).max() <= lim * g["printed_max_abs_deviation"]["logits"]
    assert np.abs(o - ref["o"]).max() <= lim * g["printed_max_abs_deviation"]["output"]
    assert np.abs(u - ref["u"]).max() <= 1e-13
    np.testing.assert_allclose(np.log(np.exp(logits - logits.max(-1, keepdims=True)).sum(-1))
                               + logits.max(-1), ref["lse"], rtol=1e-13)


def test_value_side_identity():
    """P (C W_UV) == (P C) W_UV  [value absorption]."""
    prob = _problem(8, n_q=2, n_h=3, d_c=16, d_nope=8, d_rope=4, d_v=6, S=20)
    ref = oracle.decode_sequence(**prob)
    np.testing.assert_allclose(oracle.value_up_projection(ref["u"], prob["w_uv"]), ref["o"],
                               rtol=1e-12, atol=1e-14)


def test_output_fold_against_scalar_loops():
    """Layer output through the fold, sum_i u_i (W_i^UV W_i^O), and without it,
    sum_i (u_i W_i^UV) W_i^O [Huny §3.2], both equal plain scalar loops over
    every index; a transposed W_i^O block (square, so shapes cannot catch it)
    changes the result."""
    rng = np.random.default_rng(41)
    n_h, d_c, d_v, d = 3, 5, 4, 6
    u = rng.standard_normal((2, n_h, d_c))
    w_uv = rng.standard_normal((n_h, d_c, d_v))
    w_o = rng.standard_normal((n_h, d_v, d))
    brute = np.zeros((2, d))
    for m in range(2):
        for n in range(d):
            acc = 0.0
            for i in range(n_h):
                for c in range(d_c):
                    for v in range(d_v):
                        acc += u[m, i, c] * w_uv[i, c, v] * w_o[i, v, n]
            brute[m, n] = acc
    unfolded = oracle.output_projection(oracle.value_up_projection(u, w_uv), w_o)
    comb = oracle.fold_output(w_uv, w_o)
    folded = sum(u[:, i, :] @ comb[i] for i in range(n_h))
    np.testing.assert_allclose(unfolded, brute, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(folded, brute, rtol=1e-12, atol=1e-12)
    w_sq = rng.standard_normal((n_h, d_v, d_v))
    o = oracle.value_up_projection(u, w_uv)
    assert np.abs(oracle.output_projection(o, w_sq) - oracle.output_projection(o, w_sq.transpose(0, 2, 1))).max() > 0.1


def test_query_fold_against_scalar_loops():
    """q_lat from the compressed query through the fold, c_q W_i^UQ (W_i^UK)^T
    [Paldyn, section MLA], equals plain loops and the two-step path (content
    query, then the absorption of decode_sequence)."""
    rng = np.random.default_rng(42)
    n_h, d_q, d_nope, d_c = 2, 6, 4, 5
    c_q = rng.standard_normal((3, d_q))
    w_uq = rng.standard_normal((n_h, d_q, d_nope))
    w_uk = rng.standard_normal((n_h, d_c, d_nope))
    brute = np.zeros((3, n_h, d_c))
    for m in range(3):
        for i in range(n_h):
            for c in range(d_c):
                brute[m, i, c] = sum(c_q[m, q] * w_uq[i, q, k] * w_uk[i, c, k]
                                     for q in range(d_q) for k in range(d_nope))
    kq = oracle.fold_query(w_uq, w_uk)
    folded = np.stack([c_q @ kq[i] for i in range(n_h)], axis=1)
    np.testing.assert_allclose(folded, brute, rtol=1e-12, atol=1e-12)
    q_nope = oracle.query_from_compressed(c_q, w_uq)
    np.testing.assert_allclose(oracle.absorb_query(q_nope, w_uk), brute, rtol=1e-12, atol=1e-12)
    # through a decode step (one token, arbitrary cache): its absorbed query is the same
    S, d_rope, d_v = 4, 4, 3
    ref = oracle.decode_sequence(q_nope, rng.standard_normal((3, n_h, d_rope)), np.array([3, 3, 3]),
                                 rng.standard_normal((S, d_c)), rng.standard_normal((S, d_rope)), w_uk,
                                 rng.standard_normal((n_h, d_c, d_v)), 0.3, 10000.0)
    np.testing.assert_allclose(ref["q_lat"], brute, rtol=1e-12, atol=1e-12)


def test_decomposition_single_token_closed_form():
    """S = 1: softmax weight 1, so o = c_0 W_UV, u = c_0 and lse = the one score,
    which is the sum of the content and positional dot products."""
    prob = _problem(9, n_q=1, n_h=3, d_c=16, d_nope=8, d_rope=8, d_v=6, S=1)
    ref = oracle.decode_sequence(**prob)
    c0 = prob["c_kv"][0]
    for i in range(3):
        np.testing.assert_allclose(ref["u"][0, i], c0, rtol=1e-15)
        np.testing.assert_allclose(ref["o"][0, i], c0 @ prob["w_uv"][i], rtol=1e-13)
        content = prob["q_nope"][0, i] @ (c0 @ prob["w_uk"][i])
        rope = prob["q_rope"][0, i] @ prob["k_rope_raw"][0]   # same position 0: R_0 = I
        assert abs(ref["lse"][0, i] - (content + rope) * prob["sm_scale"]) <= 1e-13
        split = content * prob["sm_scale"] + rope * prob["sm_scale"]
        assert abs(ref["lse"][0, i] - split) <= 8.88e-16 * 100


def test_zero_query_is_uniform_average():
    prob = _problem(10, n_q=1, n_h=2, d_c=8, d_nope=4, d_rope=4, d_v=5, S=9)
    prob["q_nope"][:] = 0
    prob["q_rope"][:] = 0
    ref = oracle.decode_sequence(**prob)
    for i in range(2):
        np.testing.assert_allclose(ref["u"][0, i], prob["c_kv"].mean(0), rtol=1e-13)
        assert abs(ref["lse"][0, i] - math.log(9)) < 1e-14


def test_dominant_score_selects_one_token():
    prob = _problem(11, n_q=1, n_h=1, d_c=8, d_nope=8, d_rope=4, d_v=5, S=6)
    prob["k_rope_raw"][:] = 0
    prob["w_uk"][0] = np.eye(8)
    prob["q_nope"][0, 0] = np.ones(8)
    c = _rng(1).standard_normal((6, 8)) * 0.1
    c[3] += 60.0 / (8 * prob["sm_scale"])           # score of token 3 is ~60 above the rest
    prob["c_kv"] = c
    ref = oracle.decode_sequence(**prob)
    # the other weights are ~exp(-60) ~ 1e-26: below one ulp of c[3]
    assert np.abs(ref["u"][0, 0] - c[3]).max() <= 4e-16 * np.abs(c[3]).max()


def test_constant_latents_give_constant_u():
    """Weights sum to one: if every cached latent is the same vector, u is it."""
    prob = _problem(12, n_q=2, n_h=3, d_c=8, d_nope=4, d_rope=6, d_v=5, S=11)
    prob["c_kv"] = np.tile(_rng(2).standard_normal(8), (11, 1))
    ref = oracle.decode_sequence(**prob)
    np.testing.assert_allclose(ref["u"], np.broadcast_to(prob["c_kv"][0], ref["u"].shape), rtol=1e-13)


def test_token_permutation_invariance():
    prob = _problem(13, n_q=2, n_h=2, d_c=8, d_nope=4, d_rope=4, d_v=5, S=12)
    ref = oracle.decode_sequence(**prob)
    perm = _rng(3).permutation(12)
    p2 = dict(prob)
    p2["c_kv"] = prob["c_kv"][perm]
    p2["k_rope_raw"] = prob["k_rope_raw"][perm]
    got = oracle.decode_sequence(kv_positions=np.arange(12)[perm], **p2)
    for key in ("o", "u", "lse"):
        np.testing.assert_allclose(got[key], ref[key], rtol=1e-12, atol=1e-14)


def test_causal_mask_pair():
    """n_q = 2: the first query does not see the second query's token."""
    prob = _problem(14, n_q=2, n_h=2, d_c=8, d_nope=4, d_rope=4, d_v=5, S=10)
    ref = oracle.decode_sequence(**prob)
    p1 = {k: (v[:1] if k in ("q_nope", "q_rope", "q_positions") else v) for k, v in prob.items()}
    p1["c_kv"], p1["k_rope_raw"] = prob["c_kv"][:9], prob["k_rope_raw"][:9]
    got = oracle.decode_sequence(**p1)
    for key in ("o", "u", "lse"):
        np.testing.assert_allclose(got[key][0], ref[key][0], rtol=1e-13)


def test_prefill_chunk_brute_force():
    """A prefill chunk: the last 6 of 8 cached tokens are queries, each attending
    causally to every cached token up to its own position."""
    prob = _problem(30, n_q=6, n_h=2, d_c=4, d_nope=2, d_rope=4, d_v=3, S=8)
    ok, key, err = _compare_to_brute(oracle.decode_sequence, prob, tol=1e-13)
    assert ok, (key, err)


def test_prefill_rows_are_single_query_decodes():
    """Row j of a chunk of 8 equals one decode query at position pos_j over the
    cache cut after pos_j (queries are independent; the causal mask is the cut)."""
    prob = _problem(31, n_q=8, n_h=3, d_c=8, d_nope=4, d_rope=4, d_v=5, S=20)
    ref = oracle.decode_sequence(**prob)
    for j in range(8):
        pos = int(prob["q_positions"][j])
        one = dict(prob, q_nope=prob["q_nope"][j:j + 1], q_rope=prob["q_rope"][j:j + 1],
                   q_positions=prob["q_positions"][j:j + 1], c_kv=prob["c_kv"][:pos + 1],
                   k_rope_raw=prob["k_rope_raw"][:pos + 1])
        got = oracle.decode_sequence(**one)
        for key in ("o", "u", "lse"):
            np.testing.assert_allclose(got[key][0], ref[key][j], rtol=1e-13, atol=1e-15)


def test_low_rank_bound():
    """Keys rebuilt from d_c-wide latents span at most d_c dimensions (case 2)."""
    r = _rng(15)
    S, d_c, n_h, d_nope = 600, 128, 4, 128
    c = r.standard_normal((S, d_c))
    w = r.standard_normal((n_h, d_c, d_nope))
    keys = np.concatenate([oracle.reconstruct_keys(c, w, i) for i in range(n_h)], axis=1)
    assert keys.shape == (600, 512)
    assert np.linalg.matrix_rank(keys) == d_c


def test_split_merge_equals_full_softmax():
    prob = _problem(16, n_q=2, n_h=3, d_c=8, d_nope=4, d_rope=4, d_v=5, S=23)
    ref = oracle.decode_sequence(**prob)
    bounds = [(0, 5), (5, 6), (6, 6), (6, 22), (22, 23)]   # includes an empty and a masked-for-j=0 chunk
    us, ls = [], []
    for t0, t1 in bounds:
        part = oracle.decode_sequence(token_range=(t0, t1), **prob)
        us.append(part["u"]), ls.append(part["lse"])
    assert np.isneginf(ls[2]).all() and np.isneginf(ls[4][0]).all()
    u, lse = oracle.merge_partials(np.stack(us), np.stack(ls))
    np.testing.assert_allclose(u, ref["u"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(lse, ref["lse"], rtol=1e-13)
    # all chunks empty -> u = 0, lse = -inf
    u0, l0 = oracle.merge_partials(np.zeros((3, 2, 4)), np.full((3, 2), -np.inf))
    assert (u0 == 0).all() and np.isneginf(l0).all()


def test_torch_sdpa_fp64_cross_check():
    torch = pytest.importorskip("torch")
    prob = _problem(17, n_q=2, n_h=3, d_c=16, d_nope=8, d_rope=8, d_v=6, S=13)
    ref = oracle.decode_sequence(**prob)
    S = 13
    k_r = oracle.rope_rotate(prob["k_rope_raw"], np.arange(S), 1e4)
    q_pe = oracle.rope_rotate(prob["q_rope"], prob["q_positions"][:, None], 1e4)
    mask = torch.tensor(np.arange(S)[None, :] <= prob["q_positions"][:, None])
    for i in range(3):
        K = np.concatenate([oracle.reconstruct_keys(prob["c_kv"], prob["w_uk"], i), k_r], 1)
        V = oracle.reconstruct_values(prob["c_kv"], prob["w_uv"], i)
        Q = np.concatenate([prob["q_nope"][:, i], q_pe[:, i]], 1)
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(Q)[None], torch.tensor(K)[None], torch.tensor(V)[None],
            attn_mask=mask[None], scale=prob["sm_scale"])[0].numpy()
        np.testing.assert_allclose(ref["o"][:, i], o, rtol=1e-12, atol=1e-14)


# ------------------------------------------------------------- mutations
def _mutant_decode(mutation):
    """A copy of the oracle's decode with one planted mistake."""
    orig_rope = om.rope_rotate

    def rope_bad(x, pos, base):
        y = orig_rope(x, pos, base)
        if mutation == "rope_sign":
            return orig_rope(x, -np.asarray(pos), base)
        if mutation == "rope_halves":
            x = np.asarray(x, np.float64)
            d = x.shape[-1]
            perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
            inv = np.argsort(perm)
            return orig_rope(x[..., inv], pos, base)[..., perm]
        return y

    def decode(**prob):
        p = dict(prob)
        if mutation == "no_scale":
            p["sm_scale"] = 1.0
        if mutation == "drop_rope":
            p["q_rope"] = np.zeros_like(p["q_rope"])
        if mutation == "transpose_wuv":
            p["w_uv"] = np.ascontiguousarray(np.transpose(p["w_uv"][:, :p["w_uv"].shape[2], :], (0, 2, 1)))
        om.rope_rotate = rope_bad
        try:
            out = om.decode_sequence(**p)
        finally:
            om.rope_rotate = orig_rope
        if mutation == "off_by_one_mask":
            p2 = dict(p)
            p2["q_positions"] = np.asarray(p["q_positions"]) - 1
            out = om.decode_sequence(**p2)
        return out
    return decode


@pytest.mark.parametrize("mutation", ["rope_sign", "rope_halves", "no_scale", "drop_rope",
                                      "off_by_one_mask", "transpose_wuv"])
def test_planted_mistakes_fail_brute_force(mutation):
    prob = _problem(18, n_q=2, n_h=2, d_c=4, d_nope=2, d_rope=4, d_v=4, S=6)
    ok, _, _ = _compare_to_brute(_mutant_decode(mutation), prob, tol=1e-10)
    assert not ok, f"planted mistake {mutation} was not detected"


# ------------------------------------------------------------------ fp8 latent cache
def test_e4m3_format_definition():
    """Closed forms of the e4m3 format: 448 largest, 2^-6 smallest normal,
    2^-9 smallest subnormal, 1.0 at exponent field 7, two NaN codes, symmetric,
    127 increasing non-negative finite values."""
    v = oracle.e4m3_value(np.arange(256))
    assert v[0x7E] == 448.0 and v[0x08] == 2.0 ** -6 and v[0x01] == 2.0 ** -9 and v[0x38] == 1.0
    assert v[0x07] == 7 / 8 * 2.0 ** -6 and v[0x3F] == 1.875 and v[0x40] == 2.0
    assert np.isnan(v).sum() == 2 and np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    np.testing.assert_array_equal(v[0x80:0xFF], -v[0x00:0x7F])
    assert (np.diff(v[:0x7F]) > 0).all()


def test_e4m3_encode_rounds_to_nearest_even():
    v = oracle.e4m3_value(np.arange(256))
    finite = [c for c in range(256) if not np.isnan(v[c]) and c != 0x80]
    np.testing.assert_array_equal(oracle.e4m3_encode(v[finite]), finite)
    assert oracle.e4m3_encode(np.array([-0.0]))[0] == 0x00          # zero keeps no sign
    pos = v[:0x7F]
    mid = (pos[:-1] + pos[1:]) / 2
    lo = np.arange(0x7E)
    even = np.where(lo % 2 == 0, lo, lo + 1)
    np.testing.assert_array_equal(oracle.e4m3_encode(mid), even)     # ties go to the even code
    np.testing.assert_array_equal(oracle.e4m3_encode(np.nextafter(mid, 0)), lo)
    np.testing.assert_array_equal(oracle.e4m3_encode(np.nextafter(mid, 1e9)), lo + 1)
    np.testing.assert_array_equal(oracle.e4m3_encode(-mid), np.where(even == 0, 0, even | 0x80))
    np.testing.assert_array_equal(oracle.e4m3_encode(np.array([500.0, -1e9])), [0x7E, 0xFE])   # clamped


def test_fp8_tile_scale_is_the_smallest_sufficient_power_of_two():
    amax = np.array([448.0, 448.0001, 224.0, 224.0001, 1.0, 3.9, 1e-30, 0.0, 7e5], dtype=np.float32)
    sc = oracle.fp8_tile_scale(amax)
    np.testing.assert_array_equal(sc, [1.0, 2.0, 0.5, 1.0, 2.0 ** -8, 2.0 ** -6, 2.0 ** -108, 1.0, 2.0 ** 11])
    # the lower bound 2^-126 (a normal fp32 scale) for tiles below 448 * 2^-126
    tiny = np.array([448 * 2.0 ** -126, 447 * 2.0 ** -126, 1e-40], dtype=np.float32)
    np.testing.assert_array_equal(oracle.fp8_tile_scale(tiny), [2.0 ** -126] * 3)
    k = np.log2(sc[amax > 0].astype(np.float64))
    assert (k == np.round(k)).all()
    a = amax[amax > 0].astype(np.float64)
    assert (a <= 448 * 2.0 ** k).all() and (a > 448 * 2.0 ** (k - 1)).all()


def test_fp8_latent_quantisation():
    """Per-tile power-of-two scales: the largest magnitude of every tile lands
    in [224, 448], an all-zero tile gets scale 1 and zero codes, every value is
    recovered within half an e4m3 step of its tile's scale, and a normal-range
    value within 2^-4 of itself."""
    rng = np.random.default_rng(60)
    x = oracle_round_bf16(rng.standard_normal((5, 512)).astype(np.float32) * np.float32(3.0))
    x[2, 128:256] = 0.0
    x[3, 0:128] *= np.float32(1e-3)           # a small tile keeps its own resolution
    codes, scales = oracle.fp8_quantize_latent(x)
    assert codes.dtype == np.uint8 and scales.shape == (5, 4)
    assert scales[2, 1] == 1.0 and (codes[2, 128:256] == 0).all()
    for s in range(5):
        for g in range(4):
            tile = x[s, 128 * g:128 * (g + 1)]
            if not tile.any():
                continue
            k = int(np.argmax(np.abs(tile)))
            top = oracle.e4m3_value(int(codes[s, 128 * g + k]))
            assert 224 <= abs(top) <= 448 and np.sign(top) == np.sign(tile[k])
    deq = oracle.fp8_dequantize_latent(codes, scales)
    v = oracle.e4m3_value(np.arange(0x7F))
    step = np.diff(v)                                # spacing above each non-negative code
    a = np.abs(oracle.e4m3_value(codes.astype(np.int64)))
    idx = np.clip(np.searchsorted(v, a), 0, 0x7D)
    bound = np.repeat(scales, 128, axis=1) * step[idx] / 2 * (1 + 1e-6)
    assert (np.abs(deq - x) <= bound + 1e-30).all()
    # the small tile's error follows its own largest value (half a top-binade step, 16 of 256)
    assert np.abs(deq[3, :128] - x[3, :128]).max() <= np.abs(x[3, :128]).max() / 16 * (1 + 1e-6)
    normal = np.abs(x) >= np.repeat(scales, 128, axis=1) * 2.0 ** -6
    assert (np.abs(deq - x)[normal] <= np.abs(x)[normal] * 2.0 ** -4 * (1 + 1e-9)).all()


def oracle_round_bf16(x):
    import workloads as W
    return W.round_to_bf16(x)
