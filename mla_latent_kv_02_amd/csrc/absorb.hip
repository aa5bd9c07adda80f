// Key absorption q_lat = q^C_i (W_i^UK)^T and the query-side RoPE.
//
// [Huny] ("Multi-Head Latent Attention(MLA) 아키텍처 해부", Huny's Dev Blog)
// §3.1: folding W_i^UK into the query turns the score against the rebuilt key
// into a score against the cached latent.  §2.2: only the d_rope-wide
// positional part of the query is rotated.  RoPE pairs adjacent elements
// (2k, 2k+1) and rotates them by position * base^(-2k/d_rope); the angle is
// formed and reduced in fp64 so that positions up to 2^31 keep full accuracy.

#include "mla_device.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int NT = 256;
constexpr int MROWS = 16;           // query rows per workgroup

// q_lat[m][i][c] = sum_k q_nope[m][i][k] * W[i][c][k]; grid (n_h, c-blocks, m-blocks).
template <typename T>
__global__ __launch_bounds__(NT) void absorb_kernel(AbsorbParams p) {
  extern __shared__ float q_s[];    // [MROWS][d_nope]
  const T* q_nope = static_cast<const T*>(p.q_nope);
  const T* w = static_cast<const T*>(p.w_uk);
  T* q_lat = static_cast<T*>(p.q_lat);
  const int i = blockIdx.x;
  const int c = blockIdx.y * NT + threadIdx.x;
  const int m0 = blockIdx.z * MROWS;
  const int M = p.B * p.n_q;
  const int mrows = M - m0 < MROWS ? M - m0 : MROWS;
  for (int e = threadIdx.x; e < mrows * p.d_nope; e += NT) {
    const int mm = e / p.d_nope, k = e % p.d_nope;
    q_s[e] = Elem<T>::load(q_nope, ((int64_t)(m0 + mm) * p.n_h + i) * p.d_nope + k);
  }
  __syncthreads();
  if (c >= p.d_c) return;
  float acc[MROWS];
#pragma unroll
  for (int mm = 0; mm < MROWS; ++mm) acc[mm] = 0.f;
  const int64_t wrow = ((int64_t)i * p.d_c + c) * p.d_nope;
  for (int k = 0; k < p.d_nope; ++k) {
    const float wv = Elem<T>::load(w, wrow + k);
#pragma unroll
    for (int mm = 0; mm < MROWS; ++mm) acc[mm] = fmaf(q_s[mm * p.d_nope + k], wv, acc[mm]);
  }
  for (int mm = 0; mm < mrows; ++mm)
    Elem<T>::store(q_lat, ((int64_t)(m0 + mm) * p.n_h + i) * p.d_c + c, acc[mm]);
}

// q_pe[m][i][2k:2k+2] = rotation of q_rope[m][i][2k:2k+2] by positions[m] * theta_k.
template <typename T>
__global__ __launch_bounds__(NT) void rope_q_kernel(AbsorbParams p) {
  const int half = p.d_rope / 2;
  const int64_t n = (int64_t)p.B * p.n_q * p.n_h * half;
  const int64_t idx = (int64_t)blockIdx.x * NT + threadIdx.x;
  if (idx >= n) return;
  const int k = (int)(idx % half);
  const int64_t mi = idx / half;                 // (m, i)
  const int64_t m = mi / p.n_h;
  const T* src = static_cast<const T*>(p.q_rope);
  T* dst = static_cast<T*>(p.q_pe);
  const double theta = pow((double)p.rope_base, -2.0 * k / p.d_rope);
  double sd, cd;
  sincos((double)p.positions[m] * theta, &sd, &cd);
  const int64_t off = mi * p.d_rope + 2 * k;
  const float x0 = Elem<T>::load(src, off), x1 = Elem<T>::load(src, off + 1);
  const float c = (float)cd, s = (float)sd;
  Elem<T>::store(dst, off, x0 * c - x1 * s);
  Elem<T>::store(dst, off + 1, x0 * s + x1 * c);
}

}  // namespace

hipError_t launch_absorb(const AbsorbParams& p, hipStream_t stream) {
  const int M = p.B * p.n_q;
  dim3 grid(p.n_h, (p.d_c + NT - 1) / NT, (M + MROWS - 1) / MROWS);
  const size_t smem = sizeof(float) * MROWS * p.d_nope;
  const int64_t nrope = (int64_t)M * p.n_h * (p.d_rope / 2);
  const int rgrid = (int)((nrope + NT - 1) / NT);
  if (p.bf16) {
    hipLaunchKernelGGL(absorb_kernel<uint16_t>, grid, dim3(NT), smem, stream, p);
    hipLaunchKernelGGL(rope_q_kernel<uint16_t>, dim3(rgrid), dim3(NT), 0, stream, p);
  } else {
    hipLaunchKernelGGL(absorb_kernel<float>, grid, dim3(NT), smem, stream, p);
    hipLaunchKernelGGL(rope_q_kernel<float>, dim3(rgrid), dim3(NT), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace mla
