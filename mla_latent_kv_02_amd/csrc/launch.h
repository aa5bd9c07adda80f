// Internal launchers: host-side entry points of the kernels (no validation;
// the C ABI in mla_api.cpp checks every argument first).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_device.h"

namespace mla {

struct DecodeParams {
  const void* q_lat;
  const void* q_pe;
  CacheView cache;
  const int32_t* ctx_lens;
  const int32_t* positions;
  float* u_part;
  float* lse_part;
  int B, n_q, n_h, d_c, d_rope, num_splits;
  bool bf16;             // bf16 cache (queries bf16)
  bool fp8;              // fp8 e4m3 cache (queries bf16); neither: fp32
  float sm_scale;
};

// bf16 or fp8 cache, d_c = 512, d_rope = 64, n_h % 32 == 0.
hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream);
int decode_mfma_smem_bytes(bool fp8);
// Any dims, fp32, bf16 or fp8 cache (fp32 arithmetic).
hipError_t launch_decode_generic(const DecodeParams& p, hipStream_t stream);

struct CombineParams {
  const int32_t* ctx_lens;
  const float* u_part;
  const float* lse_part;
  float* u;
  float* lse;
  int B, n_q, n_h, d_c, num_splits;
};
hipError_t launch_combine(const CombineParams& p, hipStream_t stream);

struct AbsorbParams {
  const void* q_nope;
  const void* q_rope;
  const int32_t* positions;
  const void* w_uk;
  void* q_lat;
  void* q_pe;
  int B, n_q, n_h, d_c, d_rope, d_nope;
  bool bf16;
  float rope_base;
};
hipError_t launch_absorb(const AbsorbParams& p, hipStream_t stream);
bool absorb_mfma_ok(const AbsorbParams& p);
hipError_t launch_absorb_mfma(const AbsorbParams& p, hipStream_t stream);
// q_pe = RoPE(q_rope) alone (fp64 angles), fp32 or bf16.
hipError_t launch_rope_q(const AbsorbParams& p, hipStream_t stream);

struct OutProjParams {
  const float* u;
  const void* w_uv;
  float* out;
  int B, n_q, n_h, d_c, d_v;
  bool bf16;
};
hipError_t launch_out_proj(const OutProjParams& p, hipStream_t stream);
bool out_proj_mfma_ok(const OutProjParams& p);
hipError_t launch_out_proj_mfma(const OutProjParams& p, hipStream_t stream);

// Value up-projection o = u W_i^UV, u either given or merged on the fly from
// the split-KV partials (the merge of mla_combine; u is then never stored).
struct TailParams {
  const float* u;              // [M][n_h][d_c] (no partials)
  const int32_t* ctx_lens;     // partials: plan of mla_decode
  const float* u_part;
  const float* lse_part;
  const void* w_uv;            // bf16 [n_h][d_c][d_v]
  float* out;                  // [M][n_h][d_v]
  float* lse;                  // [M][n_h] or null (partials only)
  int B, n_q, n_h, d_c, d_v, num_splits;
};
bool tail_mfma_ok(int d_c, int d_v, bool bf16_weights);
hipError_t launch_tail_mfma(const TailParams& p, bool from_partials, hipStream_t stream);

struct AppendParams {
  CacheView cache;
  void* cache_data;
  int n;
  const int32_t* seq_ids;
  const int32_t* positions;
  const void* c_kv;
  int64_t c_kv_stride;
  const void* k_rope;
  int64_t k_rope_stride;
  int d_c, d_rope;
  bool bf16;             // bf16 cache and inputs
  bool fp8;              // fp8 cache, bf16 inputs; neither: fp32
  float rope_base;
};
hipError_t launch_cache_append(const AppendParams& p, hipStream_t stream);
// mla_cache_append then the bf16 MFMA absorption, in one launch where the
// absorption takes its one-pass kernel and the cache is bf16 (ap may be null).
hipError_t launch_append_absorb_mfma(const AbsorbParams& p, const AppendParams* ap, hipStream_t stream);

// C[z][m][n] = sum_k A[z][m][k] B[z][n][k] (k contiguous in both operands).
// A: fp32 (a_f32) or bf16; B: bf16; C: bf16 (c_bf16) or fp32.  Strides in
// elements; requires K % 16 == 0, lda and ldb multiples of 8 and 16-byte
// aligned rows.
struct GemmNT {
  const void* A;
  int64_t lda, strideA;
  const uint16_t* B;
  int64_t ldb, strideB;
  void* C;
  int64_t ldc, strideC;
  int M, N, K, batch;
  bool a_f32, c_bf16;
};
hipError_t launch_gemm_nt(const GemmNT& g, hipStream_t stream);

// Prefill: reconstruction of [c W_i^UK | c W_i^UV] for tokens 0 .. max_ctx-1
// into kv [B][max_ctx][n_h][256], then causal attention of the n_q query rows
// of every sequence (V3 head shapes, bf16, contiguous cache).
struct PrefillParams {
  const void* q_nope;       // [B][n_q][n_h][128]
  const void* q_pe;         // [B][n_q][n_h][64], rotated
  const int32_t* positions; // [B][n_q]
  const int32_t* ctx_lens;  // [B]
  CacheView cache;
  const void* w_kv;         // [n_h][256][d_c]
  void* kv;
  float* out;
  float* lse;
  int B, n_q, n_h, d_c, max_ctx;
  float sm_scale;
};
hipError_t launch_prefill_weights(const uint16_t* w_uk, const uint16_t* w_uv, uint16_t* w_kv, int n_h, int d_c,
                                  hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream);

}  // namespace mla
