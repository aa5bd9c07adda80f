// Value up-projection o_i = u_i W_i^UV ([Huny] = "Multi-Head Latent
// Attention(MLA) 아키텍처 해부", Huny's Dev Blog, §3.2): the attention-weighted
// latent u_i is mapped to the head's value space once per query, instead of
// mapping every cached latent.  fp32 arithmetic; weights fp32 or bf16.

#include "mla_device.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int NT = 128;
constexpr int MROWS = 16;

// grid (n_h, v-blocks of 128, m-blocks of 16); thread = one output column v.
template <typename T>
__global__ __launch_bounds__(NT) void out_proj_kernel(OutProjParams p) {
  extern __shared__ float u_s[];     // [MROWS][d_c]
  const T* w = static_cast<const T*>(p.w_uv);
  const int i = blockIdx.x;
  const int v = blockIdx.y * NT + threadIdx.x;
  const int m0 = blockIdx.z * MROWS;
  const int M = p.B * p.n_q;
  const int mrows = M - m0 < MROWS ? M - m0 : MROWS;
  for (int e = threadIdx.x; e < mrows * p.d_c; e += NT) {
    const int mm = e / p.d_c, c = e % p.d_c;
    u_s[e] = p.u[((int64_t)(m0 + mm) * p.n_h + i) * p.d_c + c];
  }
  __syncthreads();
  if (v >= p.d_v) return;
  float acc[MROWS];
#pragma unroll
  for (int mm = 0; mm < MROWS; ++mm) acc[mm] = 0.f;
  const int64_t wbase = (int64_t)i * p.d_c * p.d_v + v;
  for (int c = 0; c < p.d_c; ++c) {
    const float wv = Elem<T>::load(w, wbase + (int64_t)c * p.d_v);
#pragma unroll
    for (int mm = 0; mm < MROWS; ++mm) acc[mm] = fmaf(u_s[mm * p.d_c + c], wv, acc[mm]);
  }
  for (int mm = 0; mm < mrows; ++mm) p.out[((int64_t)(m0 + mm) * p.n_h + i) * p.d_v + v] = acc[mm];
}

}  // namespace

hipError_t launch_out_proj(const OutProjParams& p, hipStream_t stream) {
  const int M = p.B * p.n_q;
  dim3 grid(p.n_h, (p.d_v + NT - 1) / NT, (M + MROWS - 1) / MROWS);
  const size_t smem = sizeof(float) * MROWS * p.d_c;
  if (p.bf16)
    hipLaunchKernelGGL(out_proj_kernel<uint16_t>, grid, dim3(NT), smem, stream, p);
  else
    hipLaunchKernelGGL(out_proj_kernel<float>, grid, dim3(NT), smem, stream, p);
  return hipGetLastError();
}

}  // namespace mla
