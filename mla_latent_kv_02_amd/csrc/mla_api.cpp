// C ABI of the MLA decode library: argument validation and kernel dispatch.
// Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <atomic>
#include <climits>
#include <cstring>
#include <mutex>

#include "../../include/mla.h"
#include "launch.h"

namespace {

constexpr int kMaxSplits = 1 << 20;

bool dims_ok(const mla_dims_t* d) {
  return d && d->n_h >= 1 && d->d_c >= 8 && d->d_c % 8 == 0 && d->d_rope >= 2 && d->d_rope % 8 == 0 &&
         d->d_nope >= 1 && d->d_v >= 1 && d->n_h <= 65535 && d->d_c <= (1 << 16) &&
         d->d_rope <= (1 << 16) && d->d_nope <= (1 << 16) && d->d_v <= (1 << 16) &&
         isfinite(d->sm_scale) && d->sm_scale >= 0.f && isfinite(d->rope_base) && d->rope_base >= 0.f;
}
// The value of an enum argument as the integer the caller passed: a C caller
// may pass any int, and reading one outside the enumerators' range as the
// enum type is undefined in C++, so enums from the ABI are only compared as
// integers.
template <typename E>
int32_t as_int(const E& e) {
  static_assert(sizeof(E) == sizeof(int32_t), "ABI enums are 32-bit");
  int32_t v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

bool dtype_ok(int32_t t) { return t == MLA_F32 || t == MLA_BF16; }
bool cache_dtype_ok(int32_t t) { return dtype_ok(t) || t == MLA_FP8_E4M3; }
// bytes of one cache row; -1 if the dtype does not fit the dims
int64_t row_bytes(const mla_dims_t* d, int32_t t) {
  if (t == MLA_FP8_E4M3) return d->d_c % 128 ? -1 : (int64_t)d->d_c + 2 * d->d_rope + 4 * (d->d_c / 128);
  if (t == MLA_BF16) return 2 * (int64_t)(d->d_c + d->d_rope);
  if (t == MLA_F32) return 4 * (int64_t)(d->d_c + d->d_rope);
  return -1;
}
float scale_of(const mla_dims_t* d) {
  return d->sm_scale > 0.f ? d->sm_scale : 1.0f / sqrtf((float)(d->d_nope + d->d_rope));
}
float base_of(const mla_dims_t* d) { return d->rope_base > 0.f ? d->rope_base : 10000.0f; }

bool cache_ok(const mla_cache_t* c, const mla_dims_t* d) {
  if (!c || !c->data || !c->ctx_lens || !cache_dtype_ok(as_int(c->dtype))) return false;
  const int64_t rb = row_bytes(d, as_int(c->dtype));
  if (rb < 0) return false;
  if (reinterpret_cast<uintptr_t>(c->data) % 16) return false;
  if (c->block_size < 0) return false;
  if (c->block_size > 0) return c->block_table && c->max_blocks >= 1;
  // contiguous: a sequence holds at least one row (seq_stride counts elements,
  // bytes for fp8 rows)
  const int64_t row_units = as_int(c->dtype) == MLA_FP8_E4M3 ? rb : d->d_c + d->d_rope;
  return c->seq_stride >= row_units;
}

mla::CacheView view_of(const mla_cache_t* c, const mla_dims_t* d) {
  mla::CacheView v;
  v.data = c->data;
  v.seq_stride = c->seq_stride;
  v.block_table = c->block_table;
  v.block_size = c->block_size;
  v.max_blocks = c->max_blocks;
  // elements per row; for fp8 rows (mixed element types) the unit is the byte
  v.row = as_int(c->dtype) == MLA_FP8_E4M3 ? (int32_t)row_bytes(d, MLA_FP8_E4M3) : d->d_c + d->d_rope;
  return v;
}

// The HIP error behind the last MLA_ERR_HIP this thread got (hipSuccess if none).
thread_local hipError_t t_last_hip_error = hipSuccess;

mla_status_t from_hip(hipError_t e) {
  if (e == hipSuccess) return MLA_OK;
  t_last_hip_error = e;
  return MLA_ERR_HIP;
}
bool al16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }
bool al8(const void* p) { return reinterpret_cast<uintptr_t>(p) % 8 == 0; }

// Checks the arguments of mla_absorb_q and fills *p (p->B == 0: nothing to do).
mla_status_t absorb_args(const mla_dims_t* dims, int32_t B, int32_t n_q, int32_t dt, const void* q_nope,
                         const void* q_rope, const int32_t* positions, const void* w_uk, void* q_lat, void* q_pe,
                         mla::AbsorbParams* p) {
  if (!dims_ok(dims) || B < 0 || n_q < 1 || !dtype_ok(dt)) return MLA_ERR_INVALID_ARG;
  p->B = 0;
  if (B == 0) return MLA_OK;
  if (!q_nope || !q_rope || !positions || !w_uk || !q_lat || !q_pe) return MLA_ERR_INVALID_ARG;
  if ((int64_t)B * n_q > (1 << 24)) return MLA_ERR_UNSUPPORTED;
  if ((size_t)16 * dims->d_nope * sizeof(float) > 64 * 1024) return MLA_ERR_UNSUPPORTED;
  p->q_nope = q_nope; p->q_rope = q_rope; p->positions = positions; p->w_uk = w_uk;
  p->q_lat = q_lat; p->q_pe = q_pe;
  p->B = B; p->n_q = n_q; p->n_h = dims->n_h; p->d_c = dims->d_c; p->d_rope = dims->d_rope;
  p->d_nope = dims->d_nope; p->bf16 = dt == MLA_BF16; p->rope_base = base_of(dims);
  return MLA_OK;
}

// Checks the arguments of mla_cache_append and fills *p (p->n == 0: nothing to do).
mla_status_t append_args(const mla_dims_t* dims, const mla_cache_t* cache, int32_t n, const int32_t* seq_ids,
                         const int32_t* positions, const void* c_kv_new, int64_t c_kv_stride,
                         const void* k_rope_new, int64_t k_rope_stride, mla::AppendParams* p) {
  if (!dims_ok(dims) || n < 0 || !cache_ok(cache, dims)) return MLA_ERR_INVALID_ARG;
  p->n = 0;
  if (n == 0) return MLA_OK;
  if (!seq_ids || !positions || !c_kv_new || !k_rope_new) return MLA_ERR_INVALID_ARG;
  if (c_kv_stride < dims->d_c || k_rope_stride < dims->d_rope) return MLA_ERR_INVALID_ARG;
  p->cache = view_of(cache, dims);
  p->cache_data = cache->data;
  p->n = n; p->seq_ids = seq_ids; p->positions = positions;
  p->c_kv = c_kv_new; p->c_kv_stride = c_kv_stride; p->k_rope = k_rope_new; p->k_rope_stride = k_rope_stride;
  p->d_c = dims->d_c; p->d_rope = dims->d_rope; p->bf16 = as_int(cache->dtype) == MLA_BF16;
  p->fp8 = as_int(cache->dtype) == MLA_FP8_E4M3;
  p->rope_base = base_of(dims);
  return MLA_OK;
}

mla_status_t launch_absorb_any(const mla::AbsorbParams& p, hipStream_t stream) {
  if (mla::absorb_mfma_ok(p)) return from_hip(mla::launch_absorb_mfma(p, stream));
  return from_hip(mla::launch_absorb(p, stream));
}

// Checks the arguments of mla_decode other than the partials and fills *p
// (p->B == 0: nothing to do; u_part and lse_part are left for the caller).
mla_status_t decode_args(const mla_dims_t* dims, int32_t B, int32_t n_q, const void* q_lat, const void* q_pe,
                         const mla_cache_t* cache, const int32_t* positions, int32_t num_splits,
                         mla::DecodeParams* p) {
  if (!dims_ok(dims) || B < 0 || n_q < 1 || num_splits < 1 || num_splits > kMaxSplits)
    return MLA_ERR_INVALID_ARG;
  p->B = 0;
  if (B == 0) return MLA_OK;
  if (!q_lat || !q_pe || !positions || !cache_ok(cache, dims)) return MLA_ERR_INVALID_ARG;
  // the kernels read q_lat and q_pe in 16-byte vectors
  if (!al16(q_lat) || !al16(q_pe)) return MLA_ERR_INVALID_ARG;
  if ((int64_t)n_q * dims->n_h > 65535) return MLA_ERR_UNSUPPORTED;
  p->q_lat = q_lat; p->q_pe = q_pe; p->cache = view_of(cache, dims); p->ctx_lens = cache->ctx_lens;
  p->positions = positions; p->u_part = nullptr; p->lse_part = nullptr;
  p->B = B; p->n_q = n_q; p->n_h = dims->n_h; p->d_c = dims->d_c; p->d_rope = dims->d_rope;
  p->num_splits = num_splits; p->bf16 = as_int(cache->dtype) == MLA_BF16;
  p->fp8 = as_int(cache->dtype) == MLA_FP8_E4M3;
  p->sm_scale = scale_of(dims);
  if (!((p->bf16 || p->fp8) && p->d_c == 512 && p->d_rope == 64 && p->n_h % 32 == 0) &&
      (p->d_c + p->d_rope > 2048 || p->d_c > 1024))
    return MLA_ERR_UNSUPPORTED;
  return MLA_OK;
}

// The decode kernel for the shapes of p: the MFMA kernel for the V3 row (bf16
// or fp8 cache), the generic one otherwise.
mla_status_t launch_decode_any(const mla::DecodeParams& p, hipStream_t stream) {
  const bool fast = (p.bf16 || p.fp8) && p.d_c == 512 && p.d_rope == 64 && p.n_h % 32 == 0;
  if (fast) return from_hip(mla::launch_decode_mfma(p, stream));
  return from_hip(mla::launch_decode_generic(p, stream));
}

}  // namespace

extern "C" {

const char* mla_status_string(mla_status_t s) {
  switch (as_int(s)) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARG: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case MLA_ERR_HIP: return "HIP launch error";
    case MLA_ERR_OUT_OF_BLOCKS: return "block pool has too few free blocks";
    case MLA_ERR_TOO_LARGE: return "input needs more than the fixed scratch of the no-allocation entry point";
  }
  return "unknown status";
}

const char* mla_version(void) { return "mla-mi355x 0.2.0 (gfx950)"; }

int32_t mla_last_hip_error(void) { return (int32_t)t_last_hip_error; }

const char* mla_hip_error_name(int32_t code) {
  // hipError_t's enumerators span 0 .. 1054, so its values are 0 .. 2047; an
  // integer outside that is no hipError_t at all
  if (code < 0 || code > 2047) return "not a HIP error code";
  return hipGetErrorName(static_cast<hipError_t>(code));
}

int64_t mla_cache_row_bytes(const mla_dims_t* dims, mla_dtype_t dtype) {
  if (!dims_ok(dims) || !cache_dtype_ok(as_int(dtype))) return -1;
  return row_bytes(dims, as_int(dtype));
}

int64_t mla_num_partials(int32_t B, int32_t num_splits) {
  if (B < 0 || num_splits < 1) return -1;
  return B == 0 ? 0 : (int64_t)num_splits + B - 1;
}

mla_status_t mla_absorb_q(const mla_dims_t* dims, int32_t B, int32_t n_q, mla_dtype_t dt,
                          const void* q_nope, const void* q_rope, const int32_t* positions,
                          const void* w_uk, void* q_lat, void* q_pe, void* stream) {
  mla::AbsorbParams p;
  const mla_status_t st = absorb_args(dims, B, n_q, as_int(dt), q_nope, q_rope, positions, w_uk, q_lat, q_pe, &p);
  if (st != MLA_OK || p.B == 0) return st;
  return launch_absorb_any(p, (hipStream_t)stream);
}

mla_status_t mla_decode(const mla_dims_t* dims, int32_t B, int32_t n_q, const void* q_lat,
                        const void* q_pe, const mla_cache_t* cache, const int32_t* positions,
                        int32_t num_splits, float* u_part, float* lse_part, void* stream) {
  mla::DecodeParams p;
  const mla_status_t st = decode_args(dims, B, n_q, q_lat, q_pe, cache, positions, num_splits, &p);
  if (st != MLA_OK || p.B == 0) return st;
  if (!u_part || !lse_part) return MLA_ERR_INVALID_ARG;
  // the kernels store u_part in 16-byte vectors, lse_part in pairs
  if (!al16(u_part) || !al8(lse_part)) return MLA_ERR_INVALID_ARG;
  p.u_part = u_part;
  p.lse_part = lse_part;
  return launch_decode_any(p, (hipStream_t)stream);
}

mla_status_t mla_combine(const mla_dims_t* dims, int32_t B, int32_t n_q, const int32_t* ctx_lens,
                         int32_t num_splits, const float* u_part, const float* lse_part, float* u,
                         float* lse, void* stream) {
  if (!dims_ok(dims) || B < 0 || n_q < 1 || num_splits < 1 || num_splits > kMaxSplits)
    return MLA_ERR_INVALID_ARG;
  if (B == 0) return MLA_OK;
  if (!ctx_lens || !u_part || !lse_part || !u) return MLA_ERR_INVALID_ARG;
  if (!al16(u_part) || !al8(lse_part) || !al16(u)) return MLA_ERR_INVALID_ARG;
  if ((int64_t)n_q * dims->n_h > 65535 * 4) return MLA_ERR_UNSUPPORTED;
  mla::CombineParams p;
  p.ctx_lens = ctx_lens; p.u_part = u_part; p.lse_part = lse_part; p.u = u; p.lse = lse;
  p.B = B; p.n_q = n_q; p.n_h = dims->n_h; p.d_c = dims->d_c; p.num_splits = num_splits;
  return from_hip(mla::launch_combine(p, (hipStream_t)stream));
}

mla_status_t mla_out_proj(const mla_dims_t* dims, int32_t B, int32_t n_q, const float* u,
                          mla_dtype_t w_dt, const void* w_uv, float* out, void* stream) {
  if (!dims_ok(dims) || B < 0 || n_q < 1 || !dtype_ok(as_int(w_dt))) return MLA_ERR_INVALID_ARG;
  if (B == 0) return MLA_OK;
  if (!u || !w_uv || !out) return MLA_ERR_INVALID_ARG;
  if (!al16(u) || !al16(w_uv)) return MLA_ERR_INVALID_ARG;
  if ((size_t)16 * dims->d_c * sizeof(float) > 64 * 1024) return MLA_ERR_UNSUPPORTED;
  mla::OutProjParams p;
  p.u = u; p.w_uv = w_uv; p.out = out;
  p.B = B; p.n_q = n_q; p.n_h = dims->n_h; p.d_c = dims->d_c; p.d_v = dims->d_v;
  p.bf16 = as_int(w_dt) == MLA_BF16;
  if (mla::tail_mfma_ok(p.d_c, p.d_v, p.bf16)) {
    mla::TailParams t{};
    t.u = u; t.w_uv = w_uv; t.out = out;
    t.B = B; t.n_q = n_q; t.n_h = p.n_h; t.d_c = p.d_c; t.d_v = p.d_v;
    return from_hip(mla::launch_tail_mfma(t, false, (hipStream_t)stream));
  }
  if (mla::out_proj_mfma_ok(p)) return from_hip(mla::launch_out_proj_mfma(p, (hipStream_t)stream));
  return from_hip(mla::launch_out_proj(p, (hipStream_t)stream));
}

mla_status_t mla_combine_out_proj(const mla_dims_t* dims, int32_t B, int32_t n_q, const int32_t* ctx_lens,
                                  int32_t num_splits, const float* u_part, const float* lse_part,
                                  mla_dtype_t w_dt, const void* w_uv, float* out, float* lse, void* stream) {
  if (!dims_ok(dims) || B < 0 || n_q < 1 || num_splits < 1 || num_splits > kMaxSplits || !dtype_ok(as_int(w_dt)))
    return MLA_ERR_INVALID_ARG;
  if (B == 0) return MLA_OK;
  if (!ctx_lens || !u_part || !lse_part || !w_uv || !out) return MLA_ERR_INVALID_ARG;
  if (!al16(u_part) || !al8(lse_part) || !al16(w_uv)) return MLA_ERR_INVALID_ARG;
  if (!mla::tail_mfma_ok(dims->d_c, dims->d_v, as_int(w_dt) == MLA_BF16)) return MLA_ERR_UNSUPPORTED;
  mla::TailParams p{};
  p.ctx_lens = ctx_lens; p.u_part = u_part; p.lse_part = lse_part; p.w_uv = w_uv; p.out = out; p.lse = lse;
  p.B = B; p.n_q = n_q; p.n_h = dims->n_h; p.d_c = dims->d_c; p.d_v = dims->d_v; p.num_splits = num_splits;
  return from_hip(mla::launch_tail_mfma(p, true, (hipStream_t)stream));
}

mla_status_t mla_cache_append(const mla_dims_t* dims, const mla_cache_t* cache, int32_t n,
                              const int32_t* seq_ids, const int32_t* positions,
                              const void* c_kv_new, int64_t c_kv_stride, const void* k_rope_new,
                              int64_t k_rope_stride, void* stream) {
  mla::AppendParams p;
  const mla_status_t st = append_args(dims, cache, n, seq_ids, positions, c_kv_new, c_kv_stride, k_rope_new,
                                      k_rope_stride, &p);
  if (st != MLA_OK || p.n == 0) return st;
  return from_hip(mla::launch_cache_append(p, (hipStream_t)stream));
}

mla_status_t mla_append_absorb_q(const mla_dims_t* dims, const mla_cache_t* cache, int32_t n,
                                 const int32_t* seq_ids, const int32_t* new_positions, const void* c_kv_new,
                                 int64_t c_kv_stride, const void* k_rope_new, int64_t k_rope_stride, int32_t B,
                                 int32_t n_q, mla_dtype_t dt, const void* q_nope, const void* q_rope,
                                 const int32_t* positions, const void* w_uk, void* q_lat, void* q_pe,
                                 void* stream) {
  mla::AppendParams ap;
  mla::AbsorbParams p;
  mla_status_t st = append_args(dims, cache, n, seq_ids, new_positions, c_kv_new, c_kv_stride, k_rope_new,
                                k_rope_stride, &ap);
  if (st != MLA_OK) return st;
  st = absorb_args(dims, B, n_q, as_int(dt), q_nope, q_rope, positions, w_uk, q_lat, q_pe, &p);
  if (st != MLA_OK) return st;
  const hipStream_t s = (hipStream_t)stream;
  if (p.B > 0 && mla::absorb_mfma_ok(p)) return from_hip(mla::launch_append_absorb_mfma(p, &ap, s));
  if (ap.n > 0) {
    st = from_hip(mla::launch_cache_append(ap, s));
    if (st != MLA_OK) return st;
  }
  return p.B > 0 ? launch_absorb_any(p, s) : MLA_OK;
}

// ---- prefill
namespace {
bool prefill_dims_ok(const mla_dims_t* d) {
  return d->d_nope == 128 && d->d_v == 128 && d->d_rope == 64 && d->d_c % 64 == 0;
}
}  // namespace

mla_status_t mla_prefill_weights(const mla_dims_t* dims, const void* w_uk, const void* w_uv, void* w_kv,
                                 void* stream) {
  if (!dims_ok(dims) || !w_uk || !w_uv || !w_kv) return MLA_ERR_INVALID_ARG;
  if (!prefill_dims_ok(dims) || dims->n_h > 65535) return MLA_ERR_UNSUPPORTED;
  return from_hip(mla::launch_prefill_weights(static_cast<const uint16_t*>(w_uk), static_cast<const uint16_t*>(w_uv),
                                              static_cast<uint16_t*>(w_kv), dims->n_h, dims->d_c, (hipStream_t)stream));
}

int64_t mla_prefill_workspace_bytes(const mla_dims_t* dims, int32_t B, int32_t max_ctx) {
  if (!dims_ok(dims) || B < 0 || max_ctx < 0) return -1;
  return (int64_t)B * max_ctx * dims->n_h * (dims->d_nope + dims->d_v) * 2;
}

mla_status_t mla_prefill(const mla_dims_t* dims, int32_t B, int32_t n_q, int32_t max_ctx, const void* q_nope,
                         const void* q_rope, const int32_t* positions, const mla_cache_t* cache,
                         const void* w_kv, void* workspace, int64_t workspace_bytes, void* q_pe, float* out,
                         float* lse, void* stream) {
  if (!dims_ok(dims) || B < 0 || n_q < 1 || max_ctx < n_q) return MLA_ERR_INVALID_ARG;
  if (B == 0) return MLA_OK;
  if (!q_nope || !q_rope || !positions || !w_kv || !workspace || !q_pe || !out || !cache_ok(cache, dims))
    return MLA_ERR_INVALID_ARG;
  if (workspace_bytes < mla_prefill_workspace_bytes(dims, B, max_ctx) || !al16(workspace))
    return MLA_ERR_INVALID_ARG;
  if (!prefill_dims_ok(dims) || as_int(cache->dtype) != MLA_BF16 || cache->block_size != 0) return MLA_ERR_UNSUPPORTED;
  if (cache->seq_stride < (int64_t)max_ctx * (dims->d_c + dims->d_rope)) return MLA_ERR_INVALID_ARG;
  const int64_t kv_tok = (int64_t)dims->n_h * (dims->d_nope + dims->d_v) * 2;
  if ((int64_t)(max_ctx + 64) * kv_tok >= (1LL << 32) || (int64_t)(max_ctx + 64) * (dims->d_c + dims->d_rope) * 2 >=
      (1LL << 31) || B > 65535 || (int64_t)B * n_q > (1 << 24))
    return MLA_ERR_UNSUPPORTED;
  const hipStream_t s = (hipStream_t)stream;
  mla::AbsorbParams ap;
  ap.q_nope = nullptr; ap.q_rope = q_rope; ap.positions = positions; ap.w_uk = nullptr;
  ap.q_lat = nullptr; ap.q_pe = q_pe;
  ap.B = B; ap.n_q = n_q; ap.n_h = dims->n_h; ap.d_c = dims->d_c; ap.d_rope = dims->d_rope; ap.d_nope = dims->d_nope;
  ap.bf16 = true; ap.rope_base = base_of(dims);
  mla_status_t st = from_hip(mla::launch_rope_q(ap, s));
  if (st != MLA_OK) return st;
  mla::PrefillParams p;
  p.q_nope = q_nope; p.q_pe = q_pe; p.positions = positions; p.ctx_lens = cache->ctx_lens;
  p.cache = view_of(cache, dims); p.w_kv = w_kv; p.kv = workspace; p.out = out; p.lse = lse;
  p.B = B; p.n_q = n_q; p.n_h = dims->n_h; p.d_c = dims->d_c; p.max_ctx = max_ctx; p.sm_scale = scale_of(dims);
  return from_hip(mla::launch_prefill(p, s));
}

// ---- weight folds and the products that use them
namespace {
// the launch grid of a product: (N/32, M/64, batch) blocks
mla_status_t run_gemm(const mla::GemmNT& g, void* stream) {
  if ((g.M + 63) / 64 > 65535 || g.batch > 65535) return MLA_ERR_UNSUPPORTED;
  return from_hip(mla::launch_gemm_nt(g, (hipStream_t)stream));
}
mla::GemmNT gemm(const void* A, int64_t lda, int64_t sA, const void* B, int64_t ldb, int64_t sB, void* C,
                 int64_t ldc, int64_t sC, int M, int N, int K, int batch, bool a_f32, bool c_bf16) {
  mla::GemmNT g;
  g.A = A; g.lda = lda; g.strideA = sA;
  g.B = static_cast<const uint16_t*>(B); g.ldb = ldb; g.strideB = sB;
  g.C = C; g.ldc = ldc; g.strideC = sC;
  g.M = M; g.N = N; g.K = K; g.batch = batch; g.a_f32 = a_f32; g.c_bf16 = c_bf16;
  return g;
}
}  // namespace

mla_status_t mla_fold_out(const mla_dims_t* dims, int32_t d_model, const void* w_uv, const void* w_o,
                          void* w_comb, void* stream) {
  if (!dims_ok(dims) || d_model < 1 || !w_uv || !w_o || !w_comb) return MLA_ERR_INVALID_ARG;
  const int n_h = dims->n_h, d_c = dims->d_c, d_v = dims->d_v;
  if (d_v % 16 || !al16(w_uv) || !al16(w_o) || !al16(w_comb) || (int64_t)d_model * n_h * d_c > (1LL << 40))
    return MLA_ERR_UNSUPPORTED;
  // z = head i: C[n][c] = sum_v w_o[n][i][v] w_uv[i][c][v], written to w_comb[n][i][c]
  return run_gemm(
      gemm(w_o, (int64_t)n_h * d_v, d_v, w_uv, d_v, (int64_t)d_c * d_v, w_comb, (int64_t)n_h * d_c, d_c, d_model,
           d_c, d_v, n_h, false, true), stream);
}

mla_status_t mla_out_proj_folded(const mla_dims_t* dims, int32_t d_model, int32_t B, int32_t n_q, const float* u,
                                 const void* w_comb, float* y, void* stream) {
  if (!dims_ok(dims) || d_model < 1 || B < 0 || n_q < 1) return MLA_ERR_INVALID_ARG;
  if (B == 0) return MLA_OK;
  if (!u || !w_comb || !y) return MLA_ERR_INVALID_ARG;
  const int64_t K = (int64_t)dims->n_h * dims->d_c;
  if (K % 16 || K > INT32_MAX || !al16(u) || !al16(w_comb) || (int64_t)B * n_q > INT32_MAX / 2)
    return MLA_ERR_UNSUPPORTED;
  return run_gemm(gemm(u, K, 0, w_comb, K, 0, y, d_model, 0, B * n_q, d_model, (int)K, 1, true, false), stream);
}

mla_status_t mla_o_proj(const mla_dims_t* dims, int32_t d_model, int32_t B, int32_t n_q, const float* o,
                        const void* w_o, float* y, void* stream) {
  if (!dims_ok(dims) || d_model < 1 || B < 0 || n_q < 1) return MLA_ERR_INVALID_ARG;
  if (B == 0) return MLA_OK;
  if (!o || !w_o || !y) return MLA_ERR_INVALID_ARG;
  const int64_t K = (int64_t)dims->n_h * dims->d_v;
  if (K % 16 || K > INT32_MAX || !al16(o) || !al16(w_o) || (int64_t)B * n_q > INT32_MAX / 2)
    return MLA_ERR_UNSUPPORTED;
  return run_gemm(gemm(o, K, 0, w_o, K, 0, y, d_model, 0, B * n_q, d_model, (int)K, 1, true, false), stream);
}

mla_status_t mla_fold_q(const mla_dims_t* dims, int32_t d_q, const void* w_uq, const void* w_uk, void* w_kq,
                        void* stream) {
  if (!dims_ok(dims) || d_q < 1 || !w_uq || !w_uk || !w_kq) return MLA_ERR_INVALID_ARG;
  const int n_h = dims->n_h, d_c = dims->d_c, d_nope = dims->d_nope;
  if (d_nope % 16 || !al16(w_uq) || !al16(w_uk) || !al16(w_kq)) return MLA_ERR_UNSUPPORTED;
  // z = head i: C[c][q] = sum_k w_uk[i][c][k] w_uq[q][i][k], written to w_kq[i][c][q]
  return run_gemm(
      gemm(w_uk, d_nope, (int64_t)d_c * d_nope, w_uq, (int64_t)n_h * d_nope, d_nope, w_kq, d_q,
           (int64_t)d_c * d_q, d_c, d_q, d_nope, n_h, false, true), stream);
}

mla_status_t mla_absorb_q_folded(const mla_dims_t* dims, int32_t d_q, int32_t B, int32_t n_q, const void* c_q,
                                 const void* q_rope, const int32_t* positions, const void* w_kq, void* q_lat,
                                 void* q_pe, void* stream) {
  if (!dims_ok(dims) || d_q < 1 || B < 0 || n_q < 1) return MLA_ERR_INVALID_ARG;
  if (B == 0) return MLA_OK;
  if (!c_q || !q_rope || !positions || !w_kq || !q_lat || !q_pe) return MLA_ERR_INVALID_ARG;
  const int n_h = dims->n_h, d_c = dims->d_c;
  if (d_q % 16 || !al16(c_q) || !al16(w_kq) || (int64_t)B * n_q > (1 << 24)) return MLA_ERR_UNSUPPORTED;
  // z = head i: q_lat[m][i][c] = sum_q c_q[m][q] w_kq[i][c][q]
  mla_status_t st = run_gemm(
      gemm(c_q, d_q, 0, w_kq, d_q, (int64_t)d_c * d_q, q_lat, (int64_t)n_h * d_c, d_c, B * n_q, d_c, d_q, n_h,
           false, true), stream);
  if (st != MLA_OK) return st;
  mla::AbsorbParams p;
  p.q_nope = nullptr; p.q_rope = q_rope; p.positions = positions; p.w_uk = nullptr;
  p.q_lat = q_lat; p.q_pe = q_pe;
  p.B = B; p.n_q = n_q; p.n_h = n_h; p.d_c = d_c; p.d_rope = dims->d_rope; p.d_nope = dims->d_nope;
  p.bf16 = true; p.rope_base = base_of(dims);
  return from_hip(mla::launch_rope_q(p, (hipStream_t)stream));
}

// ---- the decode step without allocation (mla_decode_out_noalloc)
namespace {
// The split-KV partials of mla_decode_out_noalloc: u_part, then lse_part at
// the next 256-byte boundary.  One copy per GPU, in device memory that the
// library's code object holds until the process ends.  In host code the name
// `scratch` is a host-side stand-in, not a device address: what the kernels
// get is the address hipGetSymbolAddress returns on the current device.
constexpr size_t kScratchBytes = (size_t)MLA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];   // per device, set once
std::mutex g_scratch_mutex;

// The device address of `scratch` on the current device, looked up (with that
// device current) on the first call there.
hipError_t scratch_on_current_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}
}  // namespace

mla_status_t mla_decode_out_noalloc(const mla_dims_t* dims, int32_t B, int32_t n_q, const void* q_lat,
                                    const void* q_pe, const mla_cache_t* cache, const int32_t* positions,
                                    int32_t num_splits, mla_dtype_t w_dt, const void* w_uv, float* out,
                                    float* lse, void* stream) {
  mla::DecodeParams p;
  mla_status_t st = decode_args(dims, B, n_q, q_lat, q_pe, cache, positions, num_splits, &p);
  if (st != MLA_OK || p.B == 0) return st;
  if (!dtype_ok(as_int(w_dt)) || !w_uv || !out || !al16(w_uv)) return MLA_ERR_INVALID_ARG;
  if (!mla::tail_mfma_ok(dims->d_c, dims->d_v, as_int(w_dt) == MLA_BF16)) return MLA_ERR_UNSUPPORTED;
  // partial rows of the plan; u_part rows of d_c fp32, lse_part rows of 2 fp32
  const int64_t rows = ((int64_t)num_splits + B - 1) * n_q * dims->n_h;
  const int64_t u_bytes = (rows * dims->d_c * 4 + 255) / 256 * 256;
  if (u_bytes + rows * 2 * 4 > (int64_t)kScratchBytes) return MLA_ERR_TOO_LARGE;
  void* base = nullptr;
  st = from_hip(scratch_on_current_device(&base));
  if (st != MLA_OK) return st;
  p.u_part = static_cast<float*>(base);
  p.lse_part = reinterpret_cast<float*>(static_cast<unsigned char*>(base) + u_bytes);
  const hipStream_t s = (hipStream_t)stream;
  st = launch_decode_any(p, s);
  if (st != MLA_OK) return st;
  // every partial the merge reads was written by the decode above: nothing in
  // the scratch has to start at zero
  mla::TailParams t{};
  t.ctx_lens = cache->ctx_lens; t.u_part = p.u_part; t.lse_part = p.lse_part; t.w_uv = w_uv; t.out = out;
  t.lse = lse; t.B = B; t.n_q = n_q; t.n_h = dims->n_h; t.d_c = dims->d_c; t.d_v = dims->d_v;
  t.num_splits = num_splits;
  return from_hip(mla::launch_tail_mfma(t, true, s));
}

}  // extern "C"
