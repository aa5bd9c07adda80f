// Batched matrix product C[z] = A[z] . B[z]^T with MFMA 32x32x16 bf16 (fp32
// accumulation), for the weight folds of the pages' absorption in its full
// form ([Huny] = "Multi-Head Latent Attention(MLA) 아키텍처 해부", Huny's Dev
// Blog, §3.1: W^UK folds into the query projection; §3.2: W^UV folds into
// the output projection W^O) and for the per-step products that use them.
//
// Both operands have k contiguous in memory ("NT"): row m of A and row n of B
// are K elements each, which is the MFMA operand layout itself (a lane holds 8
// consecutive k of one row), so every operand load is one 16-byte (bf16) or
// two 16-byte (fp32) loads straight from memory into registers.  An fp32 A is
// split into bf16 high and residual parts, multiplied separately (two MFMAs),
// so the product keeps about fp32 accuracy.
//
// Workgroup = 4 waves over a 64 (m) x 32 (n) block of C: wave w takes rows
// 32(w%2) .. +32 and the k steps of half w/2 of K; the two halves are summed
// through LDS.  Each wave keeps two batches of 4 k steps of loads in flight
// (ping-pong), loading clamped (valid) addresses past the end so that every
// wait is exact; those steps are not multiplied.

#include "mla_device.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int NT = 256;
constexpr int KB = 4;   // k steps per load batch

template <bool A_F32, bool C_BF16>
__global__ __launch_bounds__(NT, 2) void gemm_nt_kernel(GemmNT g) {
  __shared__ float red[2][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mt = wave & 1, kh = wave >> 1;
  const int r = lane & 31, hk = lane >> 5;
  const int m0 = blockIdx.y * 64 + 32 * mt;
  const int n0 = blockIdx.x * 32;
  const int64_t z = blockIdx.z;
  // operand rows of this lane (clamped: rows past M or N give results that are not stored)
  const int am = m0 + r < g.M ? m0 + r : g.M - 1;
  const int bn = n0 + r < g.N ? n0 + r : g.N - 1;
  const int ksteps = g.K / 16;
  const int kbeg = kh ? ksteps / 2 : 0, kend = kh ? ksteps : ksteps / 2;
  const uint16_t* bp = g.B + z * g.strideB + (int64_t)bn * g.ldb + 8 * hk;
  const float* ap32 = static_cast<const float*>(g.A) + z * g.strideA + (int64_t)am * g.lda + 8 * hk;
  const uint16_t* ap16 = static_cast<const uint16_t*>(g.A) + z * g.strideA + (int64_t)am * g.lda + 8 * hk;

  bf16x8 b0[KB], b1[KB];
  f32x4 x0[KB][2], x1[KB][2];
  bf16x8 h0[KB], h1[KB];
  auto load = [&](int ks, bf16x8* b, f32x4 (*x)[2], bf16x8* h) {
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      int k = ks + j;
      k = k < kend ? k : kend - 1;
      b[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(bp + 16 * (int64_t)k));
      if (A_F32) {
        x[j][0] = *reinterpret_cast<const f32x4*>(ap32 + 16 * (int64_t)k);
        x[j][1] = *reinterpret_cast<const f32x4*>(ap32 + 16 * (int64_t)k + 4);
      } else {
        h[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(ap16 + 16 * (int64_t)k));
      }
    }
  };
  f32x16 acc = {};
  auto compute = [&](int ks, const bf16x8* b, const f32x4 (*x)[2], const bf16x8* h) {
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      if (ks + j >= kend) break;
      if (A_F32) {
        u16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = x[j][e >> 2][e & 3];
          hi[e] = f32_to_bf16(v);
          lo[e] = f32_to_bf16(v - bf16_to_f32(hi[e]));
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, hi), b[j], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, lo), b[j], acc, 0, 0, 0);
      } else {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h[j], b[j], acc, 0, 0, 0);
      }
    }
  };
  if (kbeg < kend) {
    load(kbeg, b0, x0, h0);
    load(kbeg + KB, b1, x1, h1);
    for (int ks = kbeg;;) {
      compute(ks, b0, x0, h0);
      load(ks + 2 * KB, b0, x0, h0);
      ks += KB;
      if (ks >= kend) break;
      compute(ks, b1, x1, h1);
      load(ks + 2 * KB, b1, x1, h1);
      ks += KB;
      if (ks >= kend) break;
    }
  }
  // acc[i] = C[m0 + 8(i/4) + 4hk + i%4][n0 + r]; sum the two k halves
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[mt][i][lane] = acc[i];
  }
  __syncthreads();
  if (kh == 0) {
    const int n = n0 + r;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = m0 + 8 * (i >> 2) + 4 * hk + (i & 3);
      const float v = acc[i] + red[mt][i][lane];
      if (m < g.M && n < g.N) {
        const int64_t o = z * g.strideC + (int64_t)m * g.ldc + n;
        if (C_BF16) static_cast<uint16_t*>(g.C)[o] = f32_to_bf16(v);
        else static_cast<float*>(g.C)[o] = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_nt(const GemmNT& g, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  const dim3 grid((g.N + 31) / 32, (g.M + 63) / 64, g.batch);
  if (g.a_f32) {
    if (g.c_bf16) hipLaunchKernelGGL((gemm_nt_kernel<true, true>), grid, dim3(NT), 0, stream, g);
    else hipLaunchKernelGGL((gemm_nt_kernel<true, false>), grid, dim3(NT), 0, stream, g);
  } else {
    if (g.c_bf16) hipLaunchKernelGGL((gemm_nt_kernel<false, true>), grid, dim3(NT), 0, stream, g);
    else hipLaunchKernelGGL((gemm_nt_kernel<false, false>), grid, dim3(NT), 0, stream, g);
  }
  return hipGetLastError();
}

}  // namespace mla
