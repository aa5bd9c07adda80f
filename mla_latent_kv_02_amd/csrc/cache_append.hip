// Latent-cache append: the row of a new token is [c_kv | RoPE(k_rope, pos)]
// ([Huny] = "Multi-Head Latent Attention(MLA) 아키텍처 해부", Huny's Dev Blog,
// §2.2: the positional key k^R_t = RoPE(h_t W_kR) is what is cached, shared
// by all heads).  The rotation pairs adjacent elements; the angle is formed
// and reduced in fp64, as on the query side.

#include "mla_device.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int NT = 256;

// grid (n_tokens, ceil(row/2 / NT)); thread = one element pair of one row.
template <typename T>
__global__ __launch_bounds__(NT) void cache_append_kernel(AppendParams p) {
  const int k = blockIdx.x;
  const int pair = blockIdx.y * NT + threadIdx.x;
  const int row = p.d_c + p.d_rope;
  if (2 * pair >= row) return;
  const int b = p.seq_ids[k];
  const int pos = p.positions[k];
  T* dst = static_cast<T*>(p.cache_data) + cache_row_offset(p.cache, b, pos);
  const int e = 2 * pair;
  if (e < p.d_c) {
    const T* src = static_cast<const T*>(p.c_kv) + (int64_t)k * p.c_kv_stride + e;
    dst[e] = src[0];
    dst[e + 1] = src[1];
  } else {
    const int r = e - p.d_c;
    const T* src = static_cast<const T*>(p.k_rope) + (int64_t)k * p.k_rope_stride + r;
    const double theta = pow((double)p.rope_base, -(double)r / p.d_rope);   // r = 2k
    float c, s;
    if (sizeof(T) == 2) {
      sincos_turns(pos, theta * kInv2Pi, &s, &c);   // bf16 rows: fp32 sin/cos of the fp64-reduced angle
    } else {
      double sd, cd;
      sincos((double)pos * theta, &sd, &cd);
      c = (float)cd;
      s = (float)sd;
    }
    const float x0 = Elem<T>::load(src, 0), x1 = Elem<T>::load(src, 1);
    Elem<T>::store(dst, e, x0 * c - x1 * s);
    Elem<T>::store(dst, e + 1, x0 * s + x1 * c);
  }
}

}  // namespace

hipError_t launch_cache_append(const AppendParams& p, hipStream_t stream) {
  if (p.n == 0) return hipSuccess;
  const int pairs = (p.d_c + p.d_rope) / 2;
  dim3 grid(p.n, (pairs + NT - 1) / NT);
  if (p.bf16)
    hipLaunchKernelGGL(cache_append_kernel<uint16_t>, grid, dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL(cache_append_kernel<float>, grid, dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
