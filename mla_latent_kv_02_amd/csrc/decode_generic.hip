// Decode attention for any head geometry and for fp32, bf16 or fp8 caches, in
// fp32 arithmetic.  Used where the MFMA kernel's fixed shape (bf16 or fp8,
// d_c = 512, d_rope = 64, heads in groups of 32) does not apply.
//
// Same method as the MFMA kernel ([Huny] = "Multi-Head Latent Attention(MLA)
// 아키텍처 해부", Huny's Dev Blog, §2.2 and §3): scores against the cached rows
// [c_t | k^R_t] with the absorbed query, online softmax, value sum in the
// latent space.  One workgroup handles one query row (query token j, head i)
// of one work unit: each thread scores one token of a 256-token tile, then
// each thread accumulates the latent dimensions it owns over the tile.

#include "mla_device.h"
#include "launch.h"
#include "fp8.h"

namespace mla {
namespace {

constexpr int NT = 256;
constexpr int MAX_ROW = 2048;       // d_c + d_rope
constexpr int MAX_DC_PER_THREAD = 4;  // d_c <= 1024

__device__ __forceinline__ float block_max(float v, float* red) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v = fmaxf(v, __shfl_xor(v, d, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

// Element access to one cache row: latent element e (< d_c) and positional-key
// element e (< d_rope), as fp32.  Queries have type Q.
template <typename T>
struct RowFmt {
  using Q = T;
  using Unit = T;   // unit of cache_row_offset
  __device__ __forceinline__ static float lat(const Unit* row, int e, const DecodeParams&) {
    return Elem<T>::load(row, e);
  }
  __device__ __forceinline__ static float rope(const Unit* row, int e, const DecodeParams& p) {
    return Elem<T>::load(row, p.d_c + e);
  }
};
// fp8 rows (bytes): e4m3 code times its tile's power-of-two scale (exact in
// fp32); the positional key is bf16.
struct Fp8Fmt {
  using Q = uint16_t;
  using Unit = unsigned char;
  __device__ __forceinline__ static float lat(const Unit* row, int e, const DecodeParams& p) {
    const float* scales = reinterpret_cast<const float*>(row + p.d_c + 2 * p.d_rope);
    return e4m3_value<0>(row[e]) * scales[e / kFp8Tile];
  }
  __device__ __forceinline__ static float rope(const Unit* row, int e, const DecodeParams& p) {
    return bf16_to_f32(reinterpret_cast<const uint16_t*>(row + p.d_c)[e]);
  }
};

template <typename F>
__global__ __launch_bounds__(NT) void decode_generic_kernel(DecodeParams p) {
  using T = typename F::Unit;
  using Q = typename F::Q;
  __shared__ float q_s[MAX_ROW];
  __shared__ float p_s[NT];
  __shared__ float red[4];
  __shared__ PlanScratch<NT> plan;
  const T* cache = static_cast<const T*>(p.cache.data);
  const Q* q_lat = static_cast<const Q*>(p.q_lat);
  const Q* q_pe = static_cast<const Q*>(p.q_pe);
  const int w = blockIdx.x;
  const int r = blockIdx.y;              // query row = j * n_h + i
  const int jq = r / p.n_h, ih = r % p.n_h;
  const int tid = threadIdx.x;
  const int row = p.d_c + p.d_rope;
  const float scale_log2 = p.sm_scale * kLog2e;

  for_each_segment<NT>(p.ctx_lens, p.B, p.num_splits, w, &plan, [&](int b, int t0, int t1, int slot) {
    const int64_t qrow = ((int64_t)b * p.n_q + jq) * p.n_h + ih;
    for (int e = tid; e < row; e += NT)
      q_s[e] = e < p.d_c ? Elem<Q>::load(q_lat, qrow * p.d_c + e)
                         : Elem<Q>::load(q_pe, qrow * p.d_rope + (e - p.d_c));
    const int qpos = p.positions[(int64_t)b * p.n_q + jq];
    // a range whose rows the descriptor cannot place is taken as empty
    const int t_end = segment_rows_placed(p.cache, b, t0, t1, tid & 63) ? t1 : t0;
    const int limit = qpos + 1 < t_end ? qpos + 1 : t_end;
    __syncthreads();
    float acc[MAX_DC_PER_THREAD] = {0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    for (int tt = t0; tt < limit; tt += NT) {
      const int tok = tt + tid;
      float x = -INFINITY;
      if (tok < limit) {
        const T* kr = cache + cache_row_offset(p.cache, b, tok);
        float dot = 0.f;
        for (int e = 0; e < p.d_c; ++e) dot = fmaf(q_s[e], F::lat(kr, e, p), dot);
        for (int e = 0; e < p.d_rope; ++e) dot = fmaf(q_s[p.d_c + e], F::rope(kr, e, p), dot);
        x = dot * scale_log2;
      }
      const float mt = block_max(x, red);
      const float m_new = fmaxf(m_run, mt);
      const float alpha = exp2f(m_run - m_new);   // m_new is finite: tile has a visible token
      const float pt = exp2f(x - m_new);
      p_s[tid] = pt;
      l_run = l_run * alpha + block_sum(pt, red);
      m_run = m_new;
      __syncthreads();
      const int n_here = limit - tt < NT ? limit - tt : NT;
#pragma unroll
      for (int k = 0; k < MAX_DC_PER_THREAD; ++k) acc[k] *= alpha;
      for (int t = 0; t < n_here; ++t) {
        const float pw = p_s[t];
        const T* kr = cache + cache_row_offset(p.cache, b, tt + t);
#pragma unroll
        for (int k = 0; k < MAX_DC_PER_THREAD; ++k) {
          const int d = tid + k * NT;
          if (d < p.d_c) acc[k] = fmaf(pw, F::lat(kr, d, p), acc[k]);
        }
      }
      __syncthreads();
    }
    const int64_t prow = ((int64_t)slot * p.n_q + jq) * p.n_h + ih;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int k = 0; k < MAX_DC_PER_THREAD; ++k) {
      const int d = tid + k * NT;
      if (d < p.d_c) p.u_part[prow * p.d_c + d] = acc[k] * inv;
    }
    if (tid == 0) {
      // normalised partial: reference r = lse
      const float lse = l_run > 0.f ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
      p.lse_part[2 * prow] = l_run > 0.f ? lse : 0.f;
      p.lse_part[2 * prow + 1] = lse;
    }
    __syncthreads();
  });
}

}  // namespace

hipError_t launch_decode_generic(const DecodeParams& p, hipStream_t stream) {
  if (p.d_c + p.d_rope > MAX_ROW || p.d_c > NT * MAX_DC_PER_THREAD) return hipErrorInvalidValue;
  dim3 grid(p.num_splits, p.n_q * p.n_h);
  if (p.fp8)
    hipLaunchKernelGGL(decode_generic_kernel<Fp8Fmt>, grid, dim3(NT), 0, stream, p);
  else if (p.bf16)
    hipLaunchKernelGGL(decode_generic_kernel<RowFmt<uint16_t>>, grid, dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_generic_kernel<RowFmt<float>>, grid, dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
