// Writers of new latent-cache rows (one element pair of an fp32 / bf16 row,
// or a whole fp8 row per wave), shared by the append kernel and the append
// role of the fused append + absorption launch.  The row of a new
// token is [c_kv | RoPE(k_rope, pos)] ([Huny] = "Multi-Head Latent
// Attention(MLA) 아키텍처 해부", Huny's Dev Blog, §2.2: the positional key
// k^R_t = RoPE(h_t W_kR) is what is cached, shared by all heads).  The
// rotation pairs adjacent elements; the angle is formed and reduced in fp64,
// as on the query side.
#pragma once
#include "mla_device.h"
#include "launch.h"
#include "fp8.h"

namespace mla {

// Rotation of the positional-key pair (x0, x1) = elements (r, r + 1) of a raw
// k_rope row (r even) to position pos.  bf16 rows (fp32_trig) take fp32 sin
// and cos of the fp64-reduced angle; fp32 rows take fp64 sin and cos.
__device__ __forceinline__ void rope_pair(int pos, int r, int d_rope, float base, bool fp32_trig, float x0,
                                          float x1, float* y0, float* y1) {
  const double theta = pow((double)base, -(double)r / d_rope);
  float c, s;
  if (fp32_trig) {
    sincos_turns(pos, theta * kInv2Pi, &s, &c);
  } else {
    double sd, cd;
    sincos((double)pos * theta, &sd, &cd);
    c = (float)cd;
    s = (float)sd;
  }
  *y0 = x0 * c - x1 * s;
  *y1 = x0 * s + x1 * c;
}

// Element pair `pair` (elements 2 pair, 2 pair + 1) of new row k.  Requires
// 2 * pair < d_c + d_rope.  A row the descriptor cannot place (no block
// reserved for it) is skipped.
template <typename T>
__device__ __forceinline__ void append_pair(const AppendParams& p, int k, int pair) {
  const int b = p.seq_ids[k];
  const int pos = p.positions[k];
  const int64_t off = cache_row_offset_checked(p.cache, b, pos);
  if (off < 0) return;   // no block reserved for this row: nothing is written
  T* dst = static_cast<T*>(p.cache_data) + off;
  const int e = 2 * pair;
  if (e < p.d_c) {
    const T* src = static_cast<const T*>(p.c_kv) + (int64_t)k * p.c_kv_stride + e;
    dst[e] = src[0];
    dst[e + 1] = src[1];
  } else {
    const int r = e - p.d_c;
    const T* src = static_cast<const T*>(p.k_rope) + (int64_t)k * p.k_rope_stride + r;
    float y0, y1;
    rope_pair(pos, r, p.d_rope, p.rope_base, sizeof(T) == 2, Elem<T>::load(src, 0), Elem<T>::load(src, 1), &y0,
              &y1);
    Elem<T>::store(dst, e, y0);
    Elem<T>::store(dst, e + 1, y1);
  }
}

// fp8 row of new token k (bf16 inputs), written by the 64 lanes of one wave:
// [codes (d_c bytes) | rotated k_rope (bf16) | d_c/128 fp32 scales].  A tile
// of 128 channels is held by 16 lanes (8 channels each), so a wave quantises
// 4 tiles per pass: the lanes of a tile reduce its largest magnitude, derive
// the power-of-two scale, then divide exactly and round each element to its
// nearest e4m3 code.  Rows are 4-byte aligned (d_c a multiple of 128, d_rope
// of 8), so codes go out as 32-bit words.
__device__ __forceinline__ void append_row_fp8(const AppendParams& p, int k, int lane) {
  const int b = p.seq_ids[k];
  const int pos = p.positions[k];
  const int64_t off = cache_row_offset_checked(p.cache, b, pos);
  if (off < 0) return;   // no block reserved for this row (the whole wave skips it)
  unsigned char* dst = static_cast<unsigned char*>(p.cache_data) + off;
  const uint16_t* src = static_cast<const uint16_t*>(p.c_kv) + (int64_t)k * p.c_kv_stride;
  const int n_tiles = p.d_c / kFp8Tile;
  float* scales = reinterpret_cast<float*>(dst + p.d_c + 2 * p.d_rope);
  for (int g0 = 0; g0 < n_tiles; g0 += 4) {
    const int g = g0 + (lane >> 4);
    const bool on = g < n_tiles;
    const int c0 = kFp8Tile * g + 8 * (lane & 15);
    float x[8];
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[j] = on ? bf16_to_f32(src[c0 + j]) : 0.f;
      amax = fmaxf(amax, fabsf(x[j]));
    }
#pragma unroll
    for (int sh = 1; sh < 16; sh <<= 1) amax = fmaxf(amax, __shfl_xor(amax, sh, 64));
    const int ke = fp8_scale_exp(amax);
    if (on) {
      uint32_t w[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j >> 2] |= e4m3_code(ldexpf(x[j], -ke)) << (8 * (j & 3));
      uint32_t* out = reinterpret_cast<uint32_t*>(dst + c0);
      out[0] = w[0];
      out[1] = w[1];
      if ((lane & 15) == 0) scales[g] = ldexpf(1.f, ke);
    }
  }
  const uint16_t* kr = static_cast<const uint16_t*>(p.k_rope) + (int64_t)k * p.k_rope_stride;
  uint16_t* rope = reinterpret_cast<uint16_t*>(dst + p.d_c);
  for (int pr = lane; 2 * pr < p.d_rope; pr += 64) {
    float y0, y1;
    rope_pair(pos, 2 * pr, p.d_rope, p.rope_base, true, bf16_to_f32(kr[2 * pr]), bf16_to_f32(kr[2 * pr + 1]), &y0,
              &y1);
    rope[2 * pr] = f32_to_bf16(y0);
    rope[2 * pr + 1] = f32_to_bf16(y1);
  }
}

}  // namespace mla
