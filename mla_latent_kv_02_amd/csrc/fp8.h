// FP8 e4m3 latent-cache codes ([Huny] = "Multi-Head Latent Attention(MLA)
// 아키텍처 해부", Huny's Dev Blog, serving checklist, fp8 KV-cache item;
// [Paldyn] = "MQA와 GQA: KV 캐시 경량화 전략", KV-cache quantisation: scales per
// channel or per block, never one per tensor).  Element format: OCP e4m3 --
// sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals at exponent
// field 0, largest finite 448, codes 0x7F / 0xFF NaN, no infinities.
// Each 128-channel tile of a cached latent row has a power-of-two scale, so
// x / scale and code * scale are exact.
#pragma once
#include "mla_device.h"

namespace mla {

constexpr int kFp8Tile = 128;

// Scale of a tile from its largest magnitude: 2^k for the smallest k >= -126
// with amax <= 448 * 2^k; 1 for an all-zero tile.  With amax = m 2^e,
// m in [0.5, 1): 448 = 0.875 * 2^9, so k = e - 9, one more when m > 0.875.
__device__ __forceinline__ int fp8_scale_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int e;
  const float m = frexpf(amax, &e);
  const int k = e - 9 + (m > 0.875f ? 1 : 0);
  return k < -126 ? -126 : k;
}

// Nearest e4m3 code of f (ties to the even code; clamped to +-448; zero and
// values that round to zero give 0x00).  f is finite.
__device__ __forceinline__ uint32_t e4m3_code(float f) {
  f = fminf(fmaxf(f, -448.f), 448.f);
  const uint32_t sign = (__float_as_uint(f) >> 24) & 0x80u;
  const float a = fabsf(f);
  uint32_t mag;
  if (a < 0.015625f) {
    // subnormal range (below 2^-6): multiples of 2^-9; rintf rounds ties to even
    mag = (uint32_t)rintf(a * 512.0f);
  } else {
    const uint32_t ua = __float_as_uint(a);
    int e = (int)(ua >> 23) - 127;
    const uint32_t man = ua & 0x7FFFFFu;
    uint32_t r = man >> 20;                   // top 3 mantissa bits
    const uint32_t rem = man & 0xFFFFFu;      // the 20 bits rounded away
    if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
    if (r == 8u) {
      r = 0u;
      ++e;
    }
    mag = ((uint32_t)(e + 7) << 3) | r;
  }
  return mag == 0u ? 0u : (sign | mag);
}

// fp32 value of the code in byte `sel` of `word` (exact).
template <int SEL>
__device__ __forceinline__ float e4m3_value(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8((int)word, SEL);
}

}  // namespace mla
