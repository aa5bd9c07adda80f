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
// Workgroup = 2 KP waves over a 64 (m) x 32 NB (n) block of C: wave w takes
// rows 32(w%2) .. +32, the NB 32-column blocks, and the k steps of part w/2 of
// the KP parts of K; the parts are summed through LDS.  Two shapes:
//  - NB = 2, KP = 4 (8 waves): a row operand of A is loaded once per k step
//    for both column blocks, so the re-reads of A per column of C are half
//    those of a 32-column tile;
//  - NB = 1, KP = 2 (4 waves, two workgroups per CU), when 64-column tiles
//    would leave CUs without a workgroup (the skinny products here have
//    M = 64 and K up to 65536, so the grid is N / (32 NB) workgroups).
// Measured on the fold products (64 rows): c_q W_KQ^T (N = 65536, bf16 A)
// 115 -> 97 us with the wide shape; o W_O^T and u W_comb (N = 7168, fp32 A)
// are faster with the narrow one (193 against 202 us, 707 against 765 us
// for the narrow shape with four k parts).  Each wave keeps two batches of 4 k steps of loads in flight
// (ping-pong), loading clamped (valid) addresses past the end of its quarter
// so that every wait is exact; those steps are not multiplied.

#include "mla_device.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int KB = 4;             // k steps per load batch

template <bool A_F32, bool C_BF16, int NB, int KP>
__global__ __launch_bounds__(128 * KP, KP == 2 ? 2 : 1) void gemm_nt_kernel(GemmNT g) {
  __shared__ float red[KP - 1][2][NB][16][64];   // the partial sums of k parts 1 .. KP-1
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int mt = wave & 1, kp = wave >> 1;
  const int r = lane & 31, hk = lane >> 5;
  const int m0 = blockIdx.y * 64 + 32 * mt;
  const int n0 = blockIdx.x * (32 * NB);
  const int64_t z = blockIdx.z;
  // operand rows of this lane (clamped: rows past M or N give results that are not stored)
  const int am = m0 + r < g.M ? m0 + r : g.M - 1;
  const int ksteps = g.K / 16;
  const int kbeg = kp * ksteps / KP, kend = (kp + 1) * ksteps / KP;
  const uint16_t* bp[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int bn = n0 + 32 * nb + r < g.N ? n0 + 32 * nb + r : g.N - 1;
    bp[nb] = g.B + z * g.strideB + (int64_t)bn * g.ldb + 8 * hk;
  }
  const float* ap32 = static_cast<const float*>(g.A) + z * g.strideA + (int64_t)am * g.lda + 8 * hk;
  const uint16_t* ap16 = static_cast<const uint16_t*>(g.A) + z * g.strideA + (int64_t)am * g.lda + 8 * hk;

  bf16x8 b0[KB][NB], b1[KB][NB];
  f32x4 x0[KB][2], x1[KB][2];
  bf16x8 h0[KB], h1[KB];
  auto load = [&](int ks, bf16x8 (*b)[NB], f32x4 (*x)[2], bf16x8* h) {
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      int k = ks + j;
      k = k < kend ? k : kend - 1;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        b[j][nb] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(bp[nb] + 16 * (int64_t)k));
      if (A_F32) {
        x[j][0] = *reinterpret_cast<const f32x4*>(ap32 + 16 * (int64_t)k);
        x[j][1] = *reinterpret_cast<const f32x4*>(ap32 + 16 * (int64_t)k + 4);
      } else {
        h[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(ap16 + 16 * (int64_t)k));
      }
    }
  };
  f32x16 acc[NB] = {};
  auto compute = [&](int ks, const bf16x8 (*b)[NB], const f32x4 (*x)[2], const bf16x8* h) {
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
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, hi), b[j][nb], acc[nb], 0, 0, 0);
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, lo), b[j][nb], acc[nb], 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h[j], b[j][nb], acc[nb], 0, 0, 0);
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
  // acc[nb][i] = C[m0 + 8(i/4) + 4hk + i%4][n0 + 32 nb + r]; sum the k parts
  if (kp > 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[kp - 1][mt][nb][i][lane] = acc[nb][i];
  }
  __syncthreads();
  if (kp == 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int n = n0 + 32 * nb + r;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + 8 * (i >> 2) + 4 * hk + (i & 3);
        float v = acc[nb][i];
#pragma unroll
        for (int q = 0; q < KP - 1; ++q) v += red[q][mt][nb][i][lane];
        if (m < g.M && n < g.N) {
          const int64_t o = z * g.strideC + (int64_t)m * g.ldc + n;
          if (C_BF16) static_cast<uint16_t*>(g.C)[o] = f32_to_bf16(v);
          else static_cast<float*>(g.C)[o] = v;
        }
      }
    }
  }
}

}  // namespace

template <int NB, int KP>
static void launch_shape(const GemmNT& g, hipStream_t stream) {
  const dim3 grid((g.N + 32 * NB - 1) / (32 * NB), (g.M + 63) / 64, g.batch), block(128 * KP);
  if (g.a_f32) {
    if (g.c_bf16) hipLaunchKernelGGL((gemm_nt_kernel<true, true, NB, KP>), grid, block, 0, stream, g);
    else hipLaunchKernelGGL((gemm_nt_kernel<true, false, NB, KP>), grid, block, 0, stream, g);
  } else {
    if (g.c_bf16) hipLaunchKernelGGL((gemm_nt_kernel<false, true, NB, KP>), grid, block, 0, stream, g);
    else hipLaunchKernelGGL((gemm_nt_kernel<false, false, NB, KP>), grid, block, 0, stream, g);
  }
}

hipError_t launch_gemm_nt(const GemmNT& g, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  // 64-column tiles only when they still give every CU a workgroup
  const int64_t wide = (int64_t)((g.N + 63) / 64) * ((g.M + 63) / 64) * g.batch;
  if (wide >= 256) launch_shape<2, 4>(g, stream);
  else launch_shape<1, 2>(g, stream);
  return hipGetLastError();
}

}  // namespace mla
