"""Plain fp64 definition of one MLA decode step (reconstruct-then-attend).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library.  It shares no code with
the HIP path.

Pages cited (by title):
  [Huny]    "Multi-Head Latent Attention(MLA) 아키텍처 해부: Low-Rank 압축부터
            Decoupled RoPE·Weight Absorption(행렬 흡수)과 KV Cache 93% 절감
            원리까지", Huny's Dev Blog (blog.huny.dev).
  [Tbr8]    "DeepSeek MLA（多头潜在注意力）深度解析", tbr8.org.
  [Ingu627] the MLA / SGLang article on ingu627.github.io.
  [Ikmyung] the attention / MHA / GQA / DeepSeek MLA guide on ikmyungterran.us.
  [Paldyn]  "MQA와 GQA: KV 캐시 경량화 전략", ailab.paldyn.com.

What is computed.  For one sequence whose cache holds, per token s, the latent
c_s (d_c values) and the positional key before rotation (d_rope values):

  * keys and values are rebuilt explicitly per head i:
        k^C_{s,i} = c_s W_i^UK,  v_{s,i} = c_s W_i^UV          [Huny §1.2]
    and the positional key, shared by all heads, is rotated to its position:
        k^R_s = RoPE(k_raw_s, s)                                [Huny §2.2]
  * each query head is [q^C_i | RoPE(q^R_i, p)] and each key [k^C_{s,i} | k^R_s]
    (concatenation)                                              [Huny §2.2]
  * textbook attention softmax(q k^T / sqrt(d_k)) v with d_k the query/key
    width d_nope + d_rope                                 [Ikmyung §1.3, §1.4]
    over the tokens at positions <= p (causal).
The absorbed quantities that the fast path produces are also returned, each
from its plain definition: q_lat = q^C (W^UK)^T (the absorbed query,
[Huny §3.1]), u = a C (attention weights times the latent cache, [Huny §3.2])
and lse = log sum_s exp(score_s), the log of the softmax normaliser.

Readings where the pages leave a step open (each is also listed in the design
notes):
  * RoPE pairs adjacent elements (2k, 2k+1) and rotates the pair by
    pos * theta_k with theta_k = base^(-2k/d_rope); the pages only say that
    R_t is an orthogonal, position-dependent rotation of 2-D planes.
  * The cached positional key is stored already rotated (k^R_s = RoPE(...)
    is what the cache holds, [Huny §2.2]); this module rotates the raw key.
  * One positional key shared by all heads ([Huny §2.2], [Ikmyung §7.2]).
  * Scale 1/sqrt(d_nope + d_rope), no extra long-context factor.
  * An empty softmax row (no visible token) gives u = 0, o = 0, lse = -inf.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


# --------------------------------------------------------------- RoPE
def rope_inverse_frequencies(d_rope: int, base: float) -> np.ndarray:
    """theta_k = base^(-2k/d_rope), k = 0 .. d_rope/2 - 1 (fp64)."""
    if d_rope % 2:
        raise ValueError("d_rope must be even")
    k = np.arange(d_rope // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * k / d_rope)


def rope_rotate(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate each plane (x_2k, x_2k+1) of the last axis by angle pos*theta_k.

    ``pos`` broadcasts against x.shape[:-1].  R_t is orthogonal and
    position-dependent [Huny §2.1]; the pairing and frequencies are the
    reading stated in the module docstring.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    theta = rope_inverse_frequencies(d, base)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta  # [..., d/2]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)), dtype=np.float64)
    y[..., 0::2] = x0 * c - x1 * s
    y[..., 1::2] = x0 * s + x1 * c
    return y


# --------------------------------------------------------- projections
def absorb_query(q_nope: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """q_lat[..., i, :] = q^C_i (W_i^UK)^T  [Huny §3.1; Tbr8 §5.3; Ikmyung §6].

    q_nope: [..., n_h, d_nope]; w_uk: [n_h, d_c, d_nope] -> [..., n_h, d_c].
    """
    q = np.asarray(q_nope, dtype=np.float64)
    w = np.asarray(w_uk, dtype=np.float64)
    out = np.empty(q.shape[:-1] + (w.shape[1],), dtype=np.float64)
    for i in range(w.shape[0]):
        out[..., i, :] = q[..., i, :] @ w[i].T
    return out


def reconstruct_keys(c_kv: np.ndarray, w_uk: np.ndarray, head: int) -> np.ndarray:
    """K^C_i = C^KV W_i^UK: [S, d_c] -> [S, d_nope]  [Huny §1.2; Tbr8 §5.1]."""
    return np.asarray(c_kv, dtype=np.float64) @ np.asarray(w_uk[head], dtype=np.float64)


def reconstruct_values(c_kv: np.ndarray, w_uv: np.ndarray, head: int) -> np.ndarray:
    """V_i = C^KV W_i^UV: [S, d_c] -> [S, d_v]  [Huny §1.2; Tbr8 §5.1]."""
    return np.asarray(c_kv, dtype=np.float64) @ np.asarray(w_uv[head], dtype=np.float64)


def value_up_projection(u: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """o[..., i, :] = u_i W_i^UV  [Huny §3.2]: [..., n_h, d_c] -> [..., n_h, d_v]."""
    u = np.asarray(u, dtype=np.float64)
    w = np.asarray(w_uv, dtype=np.float64)
    out = np.empty(u.shape[:-1] + (w.shape[2],), dtype=np.float64)
    for i in range(w.shape[0]):
        out[..., i, :] = u[..., i, :] @ w[i]
    return out


# --------------------------------------------------------------- weight folds
def output_projection(o: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """Layer output: the heads' outputs concatenated times W^O, i.e.
    y = sum_i o_i W_i^O with W_i^O the d_v x d block of head i [Huny §3.2].
    o [..., n_h, d_v], w_o [n_h, d_v, d] -> [..., d]."""
    o = np.asarray(o, dtype=np.float64)
    w = np.asarray(w_o, dtype=np.float64)
    y = np.zeros(o.shape[:-2] + (w.shape[2],), dtype=np.float64)
    for i in range(w.shape[0]):
        y += o[..., i, :] @ w[i]
    return y


def fold_output(w_uv: np.ndarray, w_o: np.ndarray) -> np.ndarray:
    """W_{i,comb} = W_i^UV W_i^O per head, formed offline so that the layer
    output is u_i W_{i,comb} summed over heads [Huny §3.2].
    w_uv [n_h, d_c, d_v], w_o [n_h, d_v, d] -> [n_h, d_c, d]."""
    w_uv = np.asarray(w_uv, dtype=np.float64)
    w_o = np.asarray(w_o, dtype=np.float64)
    return np.stack([w_uv[i] @ w_o[i] for i in range(w_uv.shape[0])])


def query_from_compressed(c_q: np.ndarray, w_uq: np.ndarray) -> np.ndarray:
    """q^C_i = c_q W_i^UQ, the per-head content query from the compressed
    query [Huny §1]; c_q [..., d_q], w_uq [n_h, d_q, d_nope] -> [..., n_h, d_nope]."""
    c = np.asarray(c_q, dtype=np.float64)
    w = np.asarray(w_uq, dtype=np.float64)
    return np.stack([c @ w[i] for i in range(w.shape[0])], axis=-2)


def fold_query(w_uq: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """W_{KQ,i} = W_i^UQ (W_i^UK)^T per head: the key expansion folded into the
    query projection [Paldyn, section MLA], so that q_lat = c_q W_{KQ,i}.
    w_uq [n_h, d_q, d_nope], w_uk [n_h, d_c, d_nope] -> [n_h, d_q, d_c]."""
    w_uq = np.asarray(w_uq, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    return np.stack([w_uq[i] @ w_uk[i].T for i in range(w_uq.shape[0])])


# --------------------------------------------------------------- decode
def decode_sequence(q_nope, q_rope, q_positions, c_kv, k_rope_raw, w_uk, w_uv,
                    sm_scale: float, rope_base: float,
                    kv_positions: Optional[np.ndarray] = None,
                    heads: Optional[Sequence[int]] = None,
                    token_range: Optional[tuple] = None) -> dict:
    """One decode step of one sequence, keys and values rebuilt explicitly.

    q_nope [n_q][n_h][d_nope], q_rope [n_q][n_h][d_rope] (before rotation),
    q_positions [n_q]; c_kv [S][d_c], k_rope_raw [S][d_rope] (before rotation),
    kv_positions [S] (default 0..S-1); w_uk [n_h][d_c][d_nope],
    w_uv [n_h][d_c][d_v].  ``heads`` restricts the computation to a subset of
    heads (outputs are indexed by position in ``heads``); ``token_range`` =
    (t0, t1) restricts attention to cache rows t0..t1-1, giving the partial
    (u, lse) of that chunk of the softmax.

    Returns o [n_q][h][d_v], u [n_q][h][d_c], lse [n_q][h], q_lat
    [n_q][h][d_c], q_pe [n_q][h][d_rope] (all fp64).
    """
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_rope = np.asarray(q_rope, dtype=np.float64)
    qpos = np.asarray(q_positions, dtype=np.int64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_raw = np.asarray(k_rope_raw, dtype=np.float64)
    S = c_kv.shape[0]
    kvpos = np.arange(S, dtype=np.int64) if kv_positions is None else np.asarray(kv_positions, np.int64)
    if token_range is not None:
        t0, t1 = token_range
        c_kv, k_raw, kvpos = c_kv[t0:t1], k_raw[t0:t1], kvpos[t0:t1]
    n_q = q_nope.shape[0]
    heads = list(range(q_nope.shape[1])) if heads is None else list(heads)
    d_c, d_v = c_kv.shape[1], w_uv.shape[2]

    k_r = rope_rotate(k_raw, kvpos, rope_base)                 # [S', d_rope], shared
    q_pe_all = rope_rotate(q_rope, qpos[:, None], rope_base)   # [n_q, n_h, d_rope]
    visible = kvpos[None, :] <= qpos[:, None]                  # [n_q, S']

    H = len(heads)
    o = np.zeros((n_q, H, d_v))
    u = np.zeros((n_q, H, d_c))
    lse = np.full((n_q, H), -np.inf)
    q_lat = np.empty((n_q, H, d_c))
    q_pe = np.empty((n_q, H, q_rope.shape[-1]))
    for hi, i in enumerate(heads):
        q_lat[:, hi] = q_nope[:, i] @ np.asarray(w_uk[i], dtype=np.float64).T
        q_pe[:, hi] = q_pe_all[:, i]
        if c_kv.shape[0] == 0:
            continue
        k_i = np.concatenate([reconstruct_keys(c_kv, w_uk, i), k_r], axis=1)   # [S', d_k]
        v_i = reconstruct_values(c_kv, w_uv, i)                                 # [S', d_v]
        q_i = np.concatenate([q_nope[:, i], q_pe_all[:, i]], axis=1)            # [n_q, d_k]
        scores = (q_i @ k_i.T) * sm_scale                                       # [n_q, S']
        scores = np.where(visible, scores, -np.inf)
        for j in range(n_q):
            row = scores[j]
            if not visible[j].any():
                continue
            m = row.max()
            e = np.exp(row - m)
            l = e.sum()
            p = e / l
            o[j, hi] = p @ v_i
            u[j, hi] = p @ c_kv
            lse[j, hi] = m + np.log(l)
    return {"o": o, "u": u, "lse": lse, "q_lat": q_lat, "q_pe": q_pe, "heads": heads}


def merge_partials(u_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge softmax chunks: u_parts [K][...][d_c], lse_parts [K][...].

    With L = log sum_k exp(lse_k), the merged value sum is
    sum_k exp(lse_k - L) u_k and the merged log-normaliser is L; a chunk with
    lse = -inf (no visible token) has weight 0.  This is the softmax over the
    union of the chunks written in terms of per-chunk results.
    """
    u_parts = np.asarray(u_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.exp(lse_parts - m_safe)                      # exp(-inf) = 0
    s = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, s, 1.0)), -np.inf)
    wn = np.where(finite, w / np.where(finite, s, 1.0), 0.0)
    u = (wn[..., None] * u_parts).sum(axis=0)
    return u, lse


# ------------------------------------------------------- fp8 latent cache
# The pages warn that a per-tensor fp8 scale lets outlier channels crush the
# rest of the compressed latent, and ask for per-channel or per-block (tile)
# scales instead [Huny, serving checklist, fp8 KV-cache item; Paldyn, KV-cache
# quantisation].  The reading taken here: each cached token's latent is cut
# into tiles of 128 channels, and each tile gets its own scale, the smallest
# power of two 2^k (k >= -126) with the tile's largest magnitude <= 448 * 2^k
# (448 is the largest e4m3 value).  A power of two costs a floating-point format no
# relative precision (every value keeps its 3 mantissa bits) and makes both
# directions exact: x / 2^k before rounding, code value * 2^k after.  The
# element format is
# the 8-bit e4m3 float: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa
# bits, subnormals at exponent field 0, no infinities, and the all-ones
# exponent-and-mantissa pattern reserved for NaN.
FP8_TILE = 128
FP8_MAX = 448.0


def e4m3_value(code) -> np.ndarray:
    """Value of e4m3 byte(s) per the format definition (NaN for the NaN codes)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e.astype(np.float64) - 7))
    return np.where((e == 15) & (m == 7), np.nan, sign * mag)


def e4m3_encode(x) -> np.ndarray:
    """Nearest e4m3 code to each value (ties to the even code), values first
    clamped to [-448, 448]: a search over the 127 non-negative finite codes."""
    x = np.clip(np.asarray(x, dtype=np.float64), -FP8_MAX, FP8_MAX)
    table = e4m3_value(np.arange(127))                # codes 0x00 .. 0x7E, increasing
    a = np.abs(x)
    hi = np.clip(np.searchsorted(table, a, side="left"), 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_lo, d_hi = a - table[lo], table[hi] - a
    pick = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    pick = np.where(a == table[hi], hi, pick)
    return (pick | np.where(np.signbit(x) & (pick != 0), 0x80, 0)).astype(np.uint8)


def fp8_tile_scale(amax) -> np.ndarray:
    """2^k for the smallest integer k >= -126 with amax <= 448 * 2^k (1 for
    amax = 0).  The bound keeps the scale a normal fp32 number; it binds only
    for tiles whose largest magnitude is below 448 * 2^-126 (about 5e-36)."""
    amax = np.asarray(amax, dtype=np.float64)
    k = np.zeros(amax.shape, dtype=np.int64)
    pos = amax > 0
    k[pos] = np.ceil(np.log2(amax[pos] / FP8_MAX)).astype(np.int64)
    # guard the logarithm's rounding: step k until 448 * 2^(k-1) < amax <= 448 * 2^k
    for _ in range(2):
        k = np.where(pos & (amax > FP8_MAX * 2.0 ** k), k + 1, k)
        k = np.where(pos & (amax <= FP8_MAX * 2.0 ** (k - 1)), k - 1, k)
    k = np.maximum(k, -126)
    return (2.0 ** k).astype(np.float32)


def fp8_quantize_latent(c_kv: np.ndarray):
    """Codes [S][d_c] (uint8) and scales [S][d_c/128] (fp32 powers of two) of
    cached latents: per 128-channel tile, scale = fp8_tile_scale(largest
    magnitude), code = e4m3(x / scale) (the division is exact)."""
    x = np.asarray(c_kv, dtype=np.float32)
    S, d_c = x.shape
    if d_c % FP8_TILE:
        raise ValueError("d_c must be a multiple of 128")
    tiles = x.reshape(S, d_c // FP8_TILE, FP8_TILE).astype(np.float64)
    scale = fp8_tile_scale(np.abs(tiles).max(axis=-1))
    return e4m3_encode(tiles / scale[..., None]).reshape(S, d_c), scale


def fp8_dequantize_latent(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """c_kv as the fp8 cache holds it: e4m3 value times its tile's scale (fp64)."""
    codes = np.asarray(codes)
    S, d_c = codes.shape
    v = e4m3_value(codes).reshape(S, d_c // FP8_TILE, FP8_TILE)
    return (v * np.asarray(scales, dtype=np.float64)[..., None]).reshape(S, d_c)


# ------------------------------------------------------- cache arithmetic
def mla_cache_elements_per_token(d_c: int, d_rope: int) -> int:
    """Elements cached per token per layer: c^KV plus the shared k^R [Huny §2.2]."""
    return d_c + d_rope


def mla_cache_bytes_per_token(d_c: int, d_rope: int, bytes_per_elem: int) -> int:
    """(d_c + d_R) * b bytes per token per layer [Huny §2.2]."""
    return mla_cache_elements_per_token(d_c, d_rope) * bytes_per_elem


def mha_cache_bytes_per_token(n_h: int, d_h: int, bytes_per_elem: int) -> int:
    """2 * n_h * d_h * b bytes per token per layer for full MHA [Huny §1.1]."""
    return 2 * n_h * d_h * bytes_per_elem


def gqa_cache_bytes_per_token(n_kv: int, d_h: int, bytes_per_elem: int) -> int:
    """2 * n_kv * d_h * b bytes per token per layer for grouped KV heads [Paldyn]."""
    return 2 * n_kv * d_h * bytes_per_elem
