/*
 * mla.h -- C ABI of the MI355X (gfx950) Multi-Head Latent Attention decode
 * library: one decode step with weight absorption over a latent KV cache.
 *
 * Pages cited (by title):
 *   [Huny]    "Multi-Head Latent Attention(MLA) 아키텍처 해부: Low-Rank 압축부터
 *             Decoupled RoPE·Weight Absorption(행렬 흡수)과 KV Cache 93% 절감
 *             원리까지", Huny's Dev Blog.
 *   [Tbr8]    "DeepSeek MLA（多头潜在注意力）深度解析", tbr8.org.
 *   [Ikmyung] the attention / MHA / GQA / DeepSeek MLA guide, ikmyungterran.us.
 *   [Paldyn]  "MQA와 GQA: KV 캐시 경량화 전략", ailab.paldyn.com.
 *
 * The step, per sequence b, query token j and head i:
 *   q_lat = q^C_i (W_i^UK)^T                     (key absorption, [Huny] §3.1)
 *   q_pe  = RoPE(q^R_i, position)                (decoupled RoPE, [Huny] §2.2)
 *   s_t   = scale * (q_lat . c_t + q_pe . k^R_t) for cached tokens t <= position
 *                                                 ([Huny] §2.2 score split, §3.1)
 *   a     = softmax(s)                           ([Ikmyung] §1.3-1.4)
 *   u     = sum_t a_t c_t                        (value-side absorption, [Huny] §3.2)
 *   o     = u W_i^UV                             ([Huny] §3.2)
 * The cache row of token t is [c_t (d_c) | k^R_t (d_rope)]: the latent and the
 * positional key shared by all heads, the latter stored already rotated to
 * position t ([Huny] §2.2).  Keys and values are never materialised.
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers to row-major arrays whose shape
 *     is given in the comment; the caller owns all memory.  The library never
 *     allocates, frees or synchronises; each call enqueues work on `stream`
 *     (a hipStream_t passed as void*, NULL = default stream) and returns.
 *   - Argument errors are found on the host before anything is enqueued and
 *     return MLA_ERR_INVALID_ARG; a shape the compiled kernels do not cover
 *     returns MLA_ERR_UNSUPPORTED; a failed launch returns MLA_ERR_HIP, and
 *     mla_last_hip_error() then gives the hipError_t behind it.
 *   - Arrays the kernels move in 16-byte vectors must be 16-byte aligned
 *     (each entry point names them; MLA_ERR_INVALID_ARG otherwise).  Buffers
 *     from a device allocator are; an offset view may not be.
 *   - Device-side contents (context lengths, positions, block ids) are the
 *     caller's contract and are not checked on the host: 0 <= ctx_lens[b] <=
 *     max_blocks * block_size (paged) or ctx_lens[b] * row <= seq_stride
 *     (contiguous); the id of every block holding one of a sequence's first
 *     ctx_lens[b] tokens in [0, number of blocks); for a decode step,
 *     positions[b][j] = ctx_lens[b] - n_q + j (the queries are the last n_q
 *     tokens; a negative position sees no token); append targets reserved
 *     and distinct.  The Python binding checks all of this on the host
 *     before each call when MLA_CHECK_CONTRACT=1.  The kernels keep
 *     memory safety where they can see a breach: decode treats a segment
 *     whose block ids include a negative one, or whose tokens run past
 *     max_blocks * block_size, as empty (its partial is u = 0, lse = -inf);
 *     an append skips a row whose block is missing (negative id) or lies
 *     past max_blocks.
 *   - Mutable state: the per-thread record behind mla_last_hip_error(), and
 *     the per-GPU scratch of mla_decode_out_noalloc (see there); other
 *     concurrent calls on different streams are safe when their output
 *     buffers do not overlap.
 */
#ifndef MLA_H
#define MLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,
  MLA_ERR_UNSUPPORTED = 2,
  MLA_ERR_HIP = 3,
  MLA_ERR_OUT_OF_BLOCKS = 4,   /* block pool: not enough free blocks */
  MLA_ERR_TOO_LARGE = 5         /* mla_decode_out_noalloc: the input needs more than its fixed scratch */
} mla_status_t;

/* MLA_FP8_E4M3 is a cache dtype only (see mla_cache_t); queries, weights and
 * new cache rows that go with an fp8 cache are bf16. */
typedef enum { MLA_F32 = 0, MLA_BF16 = 1, MLA_FP8_E4M3 = 2 } mla_dtype_t;

/* Head geometry.  n_h query heads; d_c latent width; d_rope positional-key
 * width (even); d_nope per-head content width of q/k; d_v per-head value
 * width.  sm_scale = 0 selects 1/sqrt(d_nope + d_rope) (the q/k width,
 * [Ikmyung] §1.3).  rope_base = 0 selects 10000.  RoPE rotates each pair of
 * adjacent elements (2k, 2k+1) by position * rope_base^(-2k/d_rope). */
typedef struct {
  int32_t n_h, d_c, d_rope, d_nope, d_v;
  float sm_scale;
  float rope_base;
} mla_dims_t;

/* Latent cache ([Huny] §2.2; paging per [Tbr8] §6.1).
 * Row of one token = d_c + d_rope elements of `dtype`: [c_kv | rotated k_rope].
 *   Contiguous (block_size == 0): token t of sequence b is the row at element
 *     offset b * seq_stride + t * (d_c + d_rope) of `data`.
 *   Paged (block_size > 0): `data` is a pool [n_blocks][block_size][row];
 *     token t of sequence b is row (t % block_size) of block
 *     block_table[b * max_blocks + t / block_size].
 * ctx_lens [B]: number of cached tokens of each sequence (the query tokens'
 * own rows included).  `data` must be 16-byte aligned.  A contiguous cache
 * needs seq_stride >= one row (d_c + d_rope elements; the fp8 row's bytes).
 * Any block size is accepted; the decode's fast paged path takes block sizes
 * that are multiples of 32 tokens (others read rows one by one, slower).
 *
 * fp8 cache (dtype MLA_FP8_E4M3; [Huny], serving checklist, fp8 KV-cache item
 * and [Paldyn], KV-cache quantisation: per-block scales rather than one
 * scale per tensor).  A row is mla_cache_row_bytes() = d_c + 2 d_rope +
 * 4 d_c/128 bytes:
 *   bytes [0, d_c)                   c_kv as e4m3 codes (OCP FP8: bias 7, max
 *                                    448, subnormals, 0x7F/0xFF NaN)
 *   bytes [d_c, d_c + 2 d_rope)      rotated k_rope, bf16 (not quantised)
 *   then d_c/128 fp32 scales         one per 128-channel tile of c_kv
 * c_kv[128 g + j] = e4m3(code) * scale[g].  Each scale is the smallest power
 * of two 2^k, k >= -126, with the tile's largest magnitude <= 448 * 2^k (1
 * for an all-zero tile), so encoding and decoding are exact scalings and every
 * element keeps the 3 mantissa bits of e4m3.  Requires d_c % 128 == 0;
 * seq_stride counts bytes. */
typedef struct {
  mla_dtype_t dtype;
  void *data;
  int64_t seq_stride;          /* elements (bytes for fp8); contiguous layout only */
  int32_t block_size;          /* 0 = contiguous */
  const int32_t *block_table;  /* [B][max_blocks], paged layout only */
  int32_t max_blocks;
  const int32_t *ctx_lens;     /* [B] */
} mla_cache_t;

/* Bytes of one cache row of the given dtype: (d_c + d_rope) * 4 or * 2 for
 * fp32 / bf16, d_c + 2 d_rope + 4 d_c/128 for MLA_FP8_E4M3; -1 for invalid
 * dims or dtype (fp8 with d_c not a multiple of 128 included). */
int64_t mla_cache_row_bytes(const mla_dims_t *dims, mla_dtype_t dtype);

/* Key absorption and query RoPE ([Huny] §3.1, §2.2; [Tbr8] §5.3).
 *   q_nope    [B][n_q][n_h][d_nope]   dtype dt
 *   q_rope    [B][n_q][n_h][d_rope]   dtype dt, before rotation
 *   positions [B][n_q]                int32, token position of each query
 *   w_uk      [n_h][d_c][d_nope]      dtype dt (W_i^UK of head i)
 *   q_lat     [B][n_q][n_h][d_c]      dtype dt, out: q^C_i (W_i^UK)^T
 *   q_pe      [B][n_q][n_h][d_rope]   dtype dt, out: rotated q^R_i
 * bf16 accumulates in fp32 and rounds the outputs to nearest even. */
mla_status_t mla_absorb_q(const mla_dims_t *dims, int32_t B, int32_t n_q, mla_dtype_t dt,
                          const void *q_nope, const void *q_rope, const int32_t *positions,
                          const void *w_uk, void *q_lat, void *q_pe, void *stream);

/* Number of partial slots mla_decode may write for a batch of B sequences
 * split into num_splits work units: num_splits + B - 1. */
int64_t mla_num_partials(int32_t B, int32_t num_splits);

/* Decode attention over the latent cache, split-KV ([Huny] §2.2, §3.1, §3.2).
 * The tokens of all sequences, taken in order (sequence 0 first), are cut
 * into num_splits consecutive ranges of about equal cost; each range is one
 * work unit.  Cost: with T = sum ctx, U = num_splits and q0 = ceil(T / U),
 * a sequence whose token prefix P_b is not a multiple of q0 starts inside a
 * unit (the unit then runs a second segment) and is preceded by 288 cost
 * positions; its tokens sit at cost positions C_b .. C_b + ctx_b - 1, C_b =
 * P_b + 288 * (such starts among sequences 0..b).  Unit w covers cost
 * positions [w Q, (w + 1) Q), Q = ceil((T + 288 E) / U), E = all such
 * starts; when every sequence starts on a multiple of q0 this is the plain
 * split into ranges of q0 tokens.  Every (sequence, work unit) pair that shares
 * tokens produces one partial over those tokens T_p: with a reference r_p
 * (any real number the kernel picks; it keeps the weights in range),
 *   u_part[p][j][i][:]   = sum_{t in T_p} exp(s_t - r_p) c_t     (not normalised)
 *   lse_part[p][j][i][0] = r_p
 *   lse_part[p][j][i][1] = log sum_{t in T_p} exp(s_t)           (natural log)
 * so that u_part * exp(r_p - lse_part[..][1]) is the softmax-weighted latent
 * of the range.  A range with no token visible to query j gives u = 0,
 * r = 0, lse = -inf.  Partials of sequence b occupy consecutive slots p in
 * order of their token ranges; the slot layout is an implementation detail
 * read by mla_combine.
 *   q_lat     [B][n_q][n_h][d_c]      cache dtype, bf16 for an fp8 cache
 *                                     (from mla_absorb_q)
 *   q_pe      [B][n_q][n_h][d_rope]   as q_lat, rotated
 *   positions [B][n_q]                query j of sequence b attends to tokens
 *                                     t <= positions[b][j]
 *   u_part    [mla_num_partials(B, num_splits)][n_q][n_h][d_c]  fp32, out
 *   lse_part  [mla_num_partials(B, num_splits)][n_q][n_h][2]    fp32, out
 * Requires 1 <= num_splits; q_lat, q_pe and u_part 16-byte aligned, lse_part
 * 8-byte aligned.  The merge is always needed, also for num_splits = 1: a
 * sequence that shares a work unit with another still gets its own partial,
 * and a partial is unnormalised (mla_combine or mla_combine_out_proj turns
 * it into u). */
mla_status_t mla_decode(const mla_dims_t *dims, int32_t B, int32_t n_q, const void *q_lat,
                        const void *q_pe, const mla_cache_t *cache, const int32_t *positions,
                        int32_t num_splits, float *u_part, float *lse_part, void *stream);

/* Log-sum-exp merge of the partials of each sequence (split-KV combine).
 * With L = log sum_k exp(lse_k) over the partials k of (b, j, i):
 *   u[b][j][i][:] = sum_k exp(r_k - L) u_part_k,   lse[b][j][i] = L,
 * i.e. the softmax over the union of the ranges ([Ikmyung] §1.4) written in
 * terms of per-range results; u = 0, lse = -inf when every partial is empty.
 * ctx_lens and num_splits must be those given to mla_decode (they fix the
 * slot layout; ctx_lens is the cache's, as mla_decode read it).
 *   u   [B][n_q][n_h][d_c] fp32, out;  lse [B][n_q][n_h] fp32, out (may be NULL)
 * u_part and u 16-byte aligned, lse_part 8-byte aligned. */
mla_status_t mla_combine(const mla_dims_t *dims, int32_t B, int32_t n_q, const int32_t *ctx_lens,
                         int32_t num_splits, const float *u_part, const float *lse_part,
                         float *u, float *lse, void *stream);

/* Value up-projection o_i = u_i W_i^UV ([Huny] §3.2).
 *   u    [B][n_q][n_h][d_c]   fp32
 *   w_uv [n_h][d_c][d_v]      dtype w_dt
 *   out  [B][n_q][n_h][d_v]   fp32, out
 * With bf16 weights the fp32 u is split into a bf16 high part and a bf16
 * residual and both are multiplied (fp32 accumulation).  u and w_uv 16-byte
 * aligned. */
mla_status_t mla_out_proj(const mla_dims_t *dims, int32_t B, int32_t n_q, const float *u,
                          mla_dtype_t w_dt, const void *w_uv, float *out, void *stream);

/* The merge of mla_combine followed by the value up-projection of
 * mla_out_proj, in one pass over the partials ([Huny] §3.2, [Ikmyung] §1.4):
 *   out[b][j][i][:] = (sum_k exp(r_k - L) u_part_k) W_i^UV,   lse[b][j][i] = L,
 * L = log sum_k exp(lse_k) over the partials k of (b, j, i).  The merged u is
 * not stored.  Arguments as for mla_combine and mla_out_proj; lse may be
 * NULL; u_part and w_uv 16-byte aligned, lse_part 8-byte aligned.  Compiled for bf16 weights with d_c = 512 and d_v = 128; other shapes
 * return MLA_ERR_UNSUPPORTED (use mla_combine, then mla_out_proj). */
mla_status_t mla_combine_out_proj(const mla_dims_t *dims, int32_t B, int32_t n_q, const int32_t *ctx_lens,
                                  int32_t num_splits, const float *u_part, const float *lse_part,
                                  mla_dtype_t w_dt, const void *w_uv, float *out, float *lse,
                                  void *stream);

/* Write n new tokens into the cache: token k belongs to sequence seq_ids[k]
 * at position positions[k]; its row becomes [c_kv_new[k] | RoPE(k_rope_new[k],
 * positions[k])] ([Huny] §2.2: the positional key is cached rotated).  Inputs
 * have the cache dtype (bf16 for an fp8 cache, whose rows are quantised as
 * mla_cache_t states: per-tile power-of-two scale, codes rounded to nearest
 * with ties to even); row k of c_kv_new starts at element k * c_kv_stride
 * and row k of k_rope_new at element k * k_rope_stride.  The caller makes
 * sure the destination rows exist (block table filled).  ctx_lens is not
 * read or updated. */
mla_status_t mla_cache_append(const mla_dims_t *dims, const mla_cache_t *cache, int32_t n,
                              const int32_t *seq_ids, const int32_t *positions,
                              const void *c_kv_new, int64_t c_kv_stride,
                              const void *k_rope_new, int64_t k_rope_stride, void *stream);

/* mla_cache_append (n new tokens, positions new_positions) followed by
 * mla_absorb_q (B sequences, n_q query tokens, positions), with the same
 * results as the two calls made in that order on one stream.  For the V3
 * shapes (bf16, d_nope = 128, d_c a multiple of 256) with a bf16 or fp8 cache both
 * run in a single launch: a decode step's new rows cost no launch of their
 * own ([Huny] §2.2 for the cached row, §3.1 for the absorbed query).  Every
 * argument of both calls is checked before anything is enqueued; n = 0 or
 * B = 0 skips that part. */
mla_status_t mla_append_absorb_q(const mla_dims_t *dims, const mla_cache_t *cache, int32_t n,
                                 const int32_t *seq_ids, const int32_t *new_positions,
                                 const void *c_kv_new, int64_t c_kv_stride, const void *k_rope_new,
                                 int64_t k_rope_stride, int32_t B, int32_t n_q, mla_dtype_t dt,
                                 const void *q_nope, const void *q_rope, const int32_t *positions,
                                 const void *w_uk, void *q_lat, void *q_pe, void *stream);

/* ---- Prefill and chunked prefill ([Huny] §1 and §2.2: k^C_i = c W_i^UK,
 * v_i = c W_i^UV, key [k^C_i | k^R]; [Tbr8] §5.2: prefill is compute-bound, so
 * the per-head keys and values are rebuilt once per call instead of absorbing
 * W^UK into every query).  The last n_q cached tokens of each sequence are
 * queries; each attends causally to the cached tokens t <= its position:
 *   kv[b][t][i][0:d_nope]   = c_t W_i^UK       (bf16 into `workspace`)
 *   kv[b][t][i][d_nope:]    = c_t W_i^UV
 *   s_t = scale * ([q^C_i | RoPE(q^R_i, pos)] . [kv[b][t][i][0:d_nope] | k^R_t])
 *   out[b][j][i][:] = sum_t softmax(s)_t kv[b][t][i][d_nope:],   lse = log sum_t exp(s_t)
 * i.e. o = a (C W_i^UV), the same output as mla_decode + mla_combine +
 * mla_out_proj for the same queries.  Compiled for bf16, d_nope = d_v = 128,
 * d_rope = 64, d_c a multiple of 64, a contiguous cache; other shapes return
 * MLA_ERR_UNSUPPORTED. */

/* w_kv [n_h][d_nope + d_v][d_c] bf16, out: w_kv[i][d][c] = W_i^UK[c][d] for
 * d < d_nope, W_i^UV[c][d - d_nope] otherwise (the latent index innermost, the
 * layout the reconstruction reads).  w_uk [n_h][d_c][d_nope], w_uv [n_h][d_c][d_v]. */
mla_status_t mla_prefill_weights(const mla_dims_t *dims, const void *w_uk, const void *w_uv, void *w_kv,
                                 void *stream);

/* Bytes of the workspace of mla_prefill: B * max_ctx * n_h * (d_nope + d_v) * 2
 * (kv [B][max_ctx][n_h][d_nope + d_v] bf16); -1 for invalid arguments. */
int64_t mla_prefill_workspace_bytes(const mla_dims_t *dims, int32_t B, int32_t max_ctx);

/*   q_nope    [B][n_q][n_h][d_nope]   bf16
 *   q_rope    [B][n_q][n_h][d_rope]   bf16, before rotation
 *   positions [B][n_q]                query j of sequence b sits at positions[b][j]
 *                                     (normally ctx_lens[b] - n_q + j)
 *   cache                             bf16, contiguous; ctx_lens[b] <= max_ctx and
 *                                     max_ctx rows per sequence fit in seq_stride
 *   w_kv      from mla_prefill_weights
 *   workspace >= mla_prefill_workspace_bytes(dims, B, max_ctx) bytes, 16-byte
 *             aligned; holds kv [B][max_ctx][n_h][d_nope + d_v] on return
 *             (rows t >= ctx_lens[b] hold whatever the cache rows there give)
 *   q_pe      [B][n_q][n_h][d_rope]   bf16, out: RoPE(q_rope, positions)
 *   out       [B][n_q][n_h][d_v]      fp32, out
 *   lse       [B][n_q][n_h]           fp32, out (may be NULL)
 * Requires 1 <= n_q <= max_ctx and (max_ctx + 64) * n_h * (d_nope + d_v) * 2 < 2^32. */
mla_status_t mla_prefill(const mla_dims_t *dims, int32_t B, int32_t n_q, int32_t max_ctx, const void *q_nope,
                         const void *q_rope, const int32_t *positions, const mla_cache_t *cache,
                         const void *w_kv, void *workspace, int64_t workspace_bytes, void *q_pe, float *out,
                         float *lse, void *stream);

/* ---- Weight folds ([Huny] §3.2, "Value 투영과 Output 투영의 결합 행렬 흡수":
 * W_i,comb = W_i^UV W_i^O is formed offline and the layer output is one
 * product with it; [Paldyn], section "MLA": the matrix that expands the keys
 * can be multiplied into the query projection the same way).  All operands
 * bf16, fp32 accumulation; arrays 16-byte aligned; MLA_ERR_UNSUPPORTED when
 * d_v, d_nope, d_q or n_h * d_c (the contraction lengths) are not multiples
 * of 16.  The folded matrices are stored with their contraction index
 * innermost, the layout the per-step products read.
 *
 * W^O enters as a linear layer's weight: w_o [d_model][n_h][d_v], i.e.
 * w_o[n][i][v] = (W_i^O)[v][n] with W_i^O the d_v x d_model block of head i. */
/* w_comb [d_model][n_h][d_c], out: w_comb[n][i][c] = (W_i^UV W_i^O)[c][n]. */
mla_status_t mla_fold_out(const mla_dims_t *dims, int32_t d_model, const void *w_uv, const void *w_o,
                          void *w_comb, void *stream);
/* Layer output through the fold: y[b][j][:] = sum_i u[b][j][i][:] W_i,comb.
 *   u [B][n_q][n_h][d_c] fp32 (split into bf16 high + residual, ~fp32 accuracy),
 *   y [B][n_q][d_model] fp32, out.
 * For few rows the contraction is cut into slices added into y with atomic
 * adds (y is cleared first), in no fixed order: y can differ in its last bits
 * from call to call.  The same holds for mla_o_proj. */
mla_status_t mla_out_proj_folded(const mla_dims_t *dims, int32_t d_model, int32_t B, int32_t n_q,
                                 const float *u, const void *w_comb, float *y, void *stream);
/* The same layer output without the fold: y[b][j][:] = sum_i o[b][j][i][:] W_i^O,
 *   o [B][n_q][n_h][d_v] fp32 (mla_out_proj's output), y [B][n_q][d_model] fp32. */
mla_status_t mla_o_proj(const mla_dims_t *dims, int32_t d_model, int32_t B, int32_t n_q, const float *o,
                        const void *w_o, float *y, void *stream);
/* Query fold: q^C_i = c_q W_i^UQ with c_q the d_q-wide compressed query and
 *   w_uq [d_q][n_h][d_nope] (W^UQ, head i's columns at [.][i][.]);
 *   w_kq [n_h][d_c][d_q], out: w_kq[i][c][q] = (W_i^UQ (W_i^UK)^T)[q][c]. */
mla_status_t mla_fold_q(const mla_dims_t *dims, int32_t d_q, const void *w_uq, const void *w_uk, void *w_kq,
                        void *stream);
/* mla_absorb_q from the compressed query through the fold:
 *   q_lat[b][j][i][:] = c_q[b][j][:] W_i^UQ (W_i^UK)^T,  q_pe = RoPE(q_rope) as in mla_absorb_q.
 *   c_q [B][n_q][d_q] bf16; q_rope, positions, q_lat, q_pe as for mla_absorb_q (bf16). */
mla_status_t mla_absorb_q_folded(const mla_dims_t *dims, int32_t d_q, int32_t B, int32_t n_q, const void *c_q,
                                 const void *q_rope, const int32_t *positions, const void *w_kq, void *q_lat,
                                 void *q_pe, void *stream);

/* ---- Block pool of a paged cache ([Paldyn], section "PagedAttention과 연속
 * 배칭": blocks are taken as a sequence grows and handed back when it ends).
 * Host-only functions (no GPU call) on HOST memory that the caller provides
 * and owns: mla_block_pool_bytes() bytes, 4-byte aligned.  Block ids are
 * handed out lowest first from a fresh pool; released blocks are reused
 * first (last released, first taken).  The table (host, [B][max_blocks]
 * int32, -1 past a sequence's blocks) is what the caller copies into the
 * device block table of mla_cache_t.  Not thread-safe: one owner at a time. */
int64_t mla_block_pool_bytes(int32_t n_blocks, int32_t B, int32_t max_blocks);   /* -1 if invalid */
/* Set up an empty pool of n_blocks blocks of block_size tokens for B sequences
 * of at most max_blocks blocks each. */
mla_status_t mla_block_pool_init(void *pool, int64_t bytes, int32_t n_blocks, int32_t block_size,
                                 int32_t B, int32_t max_blocks);
/* Give sequence b blocks for n_tokens tokens in all (it never shrinks).
 * MLA_ERR_OUT_OF_BLOCKS, with nothing taken, if the free blocks do not
 * suffice; MLA_ERR_INVALID_ARG if it would need more than max_blocks. */
mla_status_t mla_block_pool_reserve(void *pool, int32_t b, int32_t n_tokens);
/* mla_block_pool_reserve(pool, b, n_tokens[b]) for every sequence b with
 * n_tokens[b] >= 0 (host array of B entries), all or nothing: if the free
 * blocks do not cover every request, MLA_ERR_OUT_OF_BLOCKS and nothing is
 * taken. */
mla_status_t mla_block_pool_reserve_all(void *pool, const int32_t *n_tokens);
/* Return every block of sequence b to the pool; its table row becomes -1. */
mla_status_t mla_block_pool_release(void *pool, int32_t b);
/* The host block table inside the pool memory (NULL if pool is not one). */
const int32_t *mla_block_pool_table(const void *pool);
/* Number of free blocks (-1 if pool is not one). */
int32_t mla_block_pool_free_count(const void *pool);

/* ---- The decode step for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same work and results as mla_decode followed by mla_combine_out_proj, with
 * the split-KV partials in device memory the library holds instead of
 * caller-provided u_part / lse_part.  It calls no allocator.
 *   - Arguments as for mla_decode (q_lat, q_pe, cache, positions, num_splits)
 *     and mla_combine_out_proj (w_dt, w_uv, out, lse; lse may be NULL).
 *     Compiled for what mla_combine_out_proj covers (bf16 weights, d_c = 512,
 *     d_v = 128); other shapes return MLA_ERR_UNSUPPORTED.
 *   - With rows = (num_splits + B - 1) * n_q * n_h partial rows, the
 *     partials take 4 d_c * rows bytes rounded up to a multiple of 256, plus
 *     8 * rows; more than MLA_NOALLOC_SCRATCH_BYTES (128 MiB) returns
 *     MLA_ERR_TOO_LARGE before anything is enqueued.  At V3 shapes that is
 *     510 partial slots for n_q * n_h = 128 (num_splits 256 with B up to 255),
 *     255 for n_q * n_h = 256.
 *   - One scratch per GPU, shared by every call on that GPU and kept until the
 *     process ends (the first call on a device looks up its address there).
 *     It keeps the last call's contents, and nothing in it needs to start at
 *     zero.  Calls that overlap on one GPU (different streams, or host
 *     threads without ordering) race on it: order them. */
#define MLA_NOALLOC_SCRATCH_BYTES (128LL << 20)
mla_status_t mla_decode_out_noalloc(const mla_dims_t *dims, int32_t B, int32_t n_q, const void *q_lat,
                                    const void *q_pe, const mla_cache_t *cache, const int32_t *positions,
                                    int32_t num_splits, mla_dtype_t w_dt, const void *w_uv, float *out,
                                    float *lse, void *stream);

/* Static description of a status code. */
const char *mla_status_string(mla_status_t status);

/* The hipError_t (as an integer) behind the last MLA_ERR_HIP returned to the
 * calling thread; 0 (hipSuccess) if there was none.  A later MLA_ERR_HIP
 * overwrites it; other results leave it. */
int32_t mla_last_hip_error(void);

/* Static name of a hipError_t value (hipGetErrorName), e.g. for
 * mla_last_hip_error(); needs no GPU. */
const char *mla_hip_error_name(int32_t code);

/* Library version string. */
const char *mla_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H */
