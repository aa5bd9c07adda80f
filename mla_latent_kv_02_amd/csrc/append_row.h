// One element pair of a new latent-cache row, shared by the append kernel and
// the append role of the fused append + absorption launch.  The row of a new
// token is [c_kv | RoPE(k_rope, pos)] ([Huny] = "Multi-Head Latent
// Attention(MLA) 아키텍처 해부", Huny's Dev Blog, §2.2: the positional key
// k^R_t = RoPE(h_t W_kR) is what is cached, shared by all heads).  The
// rotation pairs adjacent elements; the angle is formed and reduced in fp64,
// as on the query side.
#pragma once
#include "mla_device.h"
#include "launch.h"

namespace mla {

// Element pair `pair` (elements 2 pair, 2 pair + 1) of new row k.  Requires
// 2 * pair < d_c + d_rope.
template <typename T>
__device__ __forceinline__ void append_pair(const AppendParams& p, int k, int pair) {
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

}  // namespace mla
