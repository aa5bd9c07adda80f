// Batched matrix product C[z] = A[z] . B[z]^T with MFMA 32x32x16 bf16 (fp32
// accumulation), for the weight folds of the pages' absorption in its full
// form ([Huny] = "Multi-Head Latent Attention(MLA) 아키텍처 해부", Huny's Dev
// Blog, §3.1: W^UK folds into the query projection; §3.2: W^UV folds into
// the output projection W^O) and for the per-step products that use them.
//
// Both operands have k contiguous in memory ("NT"): row m of A and row n of B
// are K elements each.  An fp32 A is split into bf16 high and residual parts,
// multiplied separately (two MFMAs), so the product keeps about fp32 accuracy.
//
// The per-step products are skinny: M = the query rows (tens), N and K in the
// thousands, B a weight matrix read once, so the kernel is built to stream B:
//  - a workgroup (4 waves) takes a tile of 64 rows x 256 columns of C over one
//    slice of K; wave w owns columns 64w .. 64w+63 (two 32-column blocks) for
//    both 32-row blocks;
//  - K advances in stages of 64: the stage's B rows (256 x 128 bytes) and A
//    rows (64 x 64 values) go global->LDS (16-byte loads, 8 lanes per 128
//    contiguous bytes of a row) into a ring of 3 stages, 2 in flight while one
//    is multiplied; one workgroup barrier per stage;
//  - in LDS each row's 16-byte chunks are permuted (chunk c of row n at
//    c ^ s(n)) so that the MFMA operand reads (a lane takes 8 consecutive k of
//    one row) fall on distinct banks;
//  - when the tiles alone would leave CUs idle and C is fp32, K is cut into
//    slices whose partial products are added into C with atomic adds (C
//    cleared first); the order of those adds is not fixed, so such results
//    can differ in the last bits from call to call.
// Work items (z, row tile, K slice, column tile) go to consecutive workgroups
// of one XCD, so the items that run side by side there share their A rows.

#include "mla_device.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int TM = 64;            // rows of a tile (two MFMA row blocks)
constexpr int TN = 256;           // columns of a tile (two MFMA column blocks per wave)
constexpr int SK = 4;             // k steps (of 16) per stage
constexpr int B_ROW = SK * 32;    // bytes of a row of B in a stage
constexpr int B_CH = B_ROW / 16;  // its 16-byte chunks
constexpr int B_STAGE = TN * B_ROW;            // 32 KiB

template <bool A_F32>
struct GemmSmem {
  static constexpr int A_ROW = SK * 16 * (A_F32 ? 4 : 2);   // bytes of a row of A in a stage
  static constexpr int A_CH = A_ROW / 16;
  static constexpr int A_STAGE = TM * A_ROW;                 // 16 KiB (fp32) or 8 KiB (bf16)
  // ring of stages in LDS (144 or 120 KiB)
  static constexpr int NSLOT = 3;
  unsigned char b[NSLOT][B_STAGE];
  unsigned char a[NSLOT][A_STAGE];
};

struct GemmGrid {
  int n_tiles, m_tiles, ksplit;
  int items, items_pad;
};

// Chunk permutation of a stage row of CH 16-byte chunks: chunk c of row n sits
// at c ^ swz<CH>(n).  A ds_read_b128 serves 16 lanes together, here 16
// consecutive rows and one logical chunk; the 64 banks are 16 groups of 16
// bytes, and row n starts at group CH n mod 16, so 16/CH consecutive rows take
// different groups and the xor by (n / (16/CH)) mod CH moves each such run of
// rows to its own chunk: the 16 reads hit 16 different groups.
template <int CH>
__device__ __forceinline__ int swz(int n) { return (n / (16 / CH)) % CH; }

constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// s_waitcnt until at most `newer` stages of LOADS loads each are in flight
// (newer < the ring's steady count, at the end of a slice); the immediate of
// the wait is a constant, so each count has its own instruction.
template <int LOADS, int TOP>
__device__ __forceinline__ void wait_newer(int newer) {
  if constexpr (TOP < 0) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  } else {
    if (newer >= TOP) __builtin_amdgcn_s_waitcnt(waitcnt_vm(TOP * LOADS));
    else wait_newer<LOADS, TOP - 1>(newer);
  }
}

template <bool A_F32, bool C_BF16, bool ATOMIC>
__global__ __launch_bounds__(256, 1) void gemm_nt_kernel(GemmNT g, GemmGrid gr) {
  using Smem = GemmSmem<A_F32>;
  __shared__ Smem sm;
  constexpr int A_LOADS = Smem::A_STAGE / 4096;              // per wave and stage (4 or 2)
  constexpr int B_LOADS = B_STAGE / 4096;                    // per wave and stage (8)
  constexpr int NSLOT = Smem::NSLOT;
  constexpr int A_CH = Smem::A_CH;
  constexpr int LOADS = A_LOADS + B_LOADS;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 31, hk = lane >> 5;
  const int item = (blockIdx.x & 7) * (gr.items_pad / 8) + (blockIdx.x >> 3);
  if (item >= gr.items) return;
  const int nt = item % gr.n_tiles;
  int rest = item / gr.n_tiles;
  const int ks_i = rest % gr.ksplit;
  rest /= gr.ksplit;
  const int mt = rest % gr.m_tiles;
  const int64_t z = rest / gr.m_tiles;
  const int m0 = mt * TM, n0 = nt * TN;
  const int ksteps = g.K / 16;
  const int kbeg = (int)((int64_t)ks_i * ksteps / gr.ksplit);
  const int kend = (int)((int64_t)(ks_i + 1) * ksteps / gr.ksplit);
  const int nst = (kend - kbeg + SK - 1) / SK;

  // ---- this lane's global->LDS loads of a stage.  Load i of wave w fills
  // 1 KiB of the stage, 16-byte slots q = 64 (B_LOADS w + i) + lane: row
  // q / CH, stored chunk q % CH (the logical chunk of the permutation).  Rows
  // past N or M repeat the last row (their results are not stored); k steps
  // past the slice end repeat its last step (not multiplied).
  const uint16_t* Bz = g.B + z * g.strideB;
  const unsigned char* Az = static_cast<const unsigned char*>(g.A) + z * g.strideA * (A_F32 ? 4 : 2);
  auto issue = [&](int s) {
    const int slot = s % NSLOT;
    const int kb = kbeg + s * SK;
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int q = (wave * B_LOADS + i) * 64 + lane;      // 16-byte slot in the stage
      const int n = q / B_CH;
      const int c = (q % B_CH) ^ swz<B_CH>(n);             // logical chunk: k step c/2, half c%2
      int kk = kb + (c >> 1);
      kk = kk < kend ? kk : kend - 1;
      const int row = n0 + n < g.N ? n0 + n : g.N - 1;
      const uint16_t* src = Bz + (int64_t)row * g.ldb + 16 * kk + 8 * (c & 1);
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(sm.b[slot] + (wave * B_LOADS + i) * 1024), 16, 0, 2);
    }
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int q = (wave * A_LOADS + i) * 64 + lane;
      const unsigned char* src;
      if (A_F32) {
        const int m = q / A_CH;
        const int c = (q % A_CH) ^ swz<A_CH>(m);           // k step c/4, 4 values at 4(c%4)
        int kk = kb + (c >> 2);
        kk = kk < kend ? kk : kend - 1;
        const int row = m0 + m < g.M ? m0 + m : g.M - 1;
        src = Az + ((int64_t)row * g.lda + 16 * kk + 4 * (c & 3)) * 4;
      } else {
        const int m = q / A_CH;
        const int c = (q % A_CH) ^ swz<A_CH>(m);
        int kk = kb + (c >> 1);
        kk = kk < kend ? kk : kend - 1;
        const int row = m0 + m < g.M ? m0 + m : g.M - 1;
        src = Az + ((int64_t)row * g.lda + 16 * kk + 8 * (c & 1)) * 2;
      }
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(sm.a[slot] + (wave * A_LOADS + i) * 1024), 16, 0, 0);
    }
  };

  typedef __attribute__((address_space(3))) const u16x8 lds_u16x8;
  typedef __attribute__((address_space(3))) const f32x4 lds_f32x4;
  const auto L = [](const unsigned char* p) { return (__attribute__((address_space(3))) const unsigned char*)p; };
  f32x16 acc[2][2] = {};   // [row block][column block]
  auto compute = [&](int s) {
    const int slot = s % NSLOT;
    const int kb = kbeg + s * SK;
#pragma unroll
    for (int j = 0; j < SK; ++j) {
      if (kb + j >= kend) break;
      bf16x8 bo[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int n = 64 * wave + 32 * nb + r;
        const int c = 2 * j + hk;
        bo[nb] = __builtin_bit_cast(bf16x8, *(lds_u16x8*)L(sm.b[slot] + n * B_ROW + ((c ^ swz<B_CH>(n)) << 4)));
      }
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int m = 32 * mb + r;
        if (A_F32) {
          const int c = 4 * j + 2 * hk;
          const f32x4 x0 = *(lds_f32x4*)L(sm.a[slot] + m * Smem::A_ROW + ((c ^ swz<A_CH>(m)) << 4));
          const f32x4 x1 = *(lds_f32x4*)L(sm.a[slot] + m * Smem::A_ROW + (((c + 1) ^ swz<A_CH>(m)) << 4));
          u16x8 hi, lo;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = e < 4 ? x0[e] : x1[e - 4];
            hi[e] = f32_to_bf16(v);
            lo[e] = f32_to_bf16(v - bf16_to_f32(hi[e]));
          }
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) {
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, hi), bo[nb],
                                                                  acc[mb][nb], 0, 0, 0);
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, lo), bo[nb],
                                                                  acc[mb][nb], 0, 0, 0);
          }
        } else {
          const int c = 2 * j + hk;
          const bf16x8 h = __builtin_bit_cast(bf16x8, *(lds_u16x8*)L(sm.a[slot] + m * Smem::A_ROW +
                                                                      ((c ^ swz<A_CH>(m)) << 4)));
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h, bo[nb], acc[mb][nb], 0, 0, 0);
        }
      }
    }
  };

  // ---- the stage loop: NSLOT - 1 stages in flight while one is multiplied
  for (int s = 0; s < NSLOT - 1 && s < nst; ++s) issue(s);
  for (int s = 0; s < nst; ++s) {
    // stage s landed; the stages after it that are issued stay in flight
    const int newer = (nst - 1 < s + NSLOT - 2 ? nst - 1 : s + NSLOT - 2) - s;
    if (newer >= NSLOT - 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm((NSLOT - 2) * LOADS));
    else wait_newer<LOADS, NSLOT - 3>(newer);
    lds_sync();   // every wave's part of stage s is in; every wave is done with stage s-1
    if (s + NSLOT - 1 < nst) issue(s + NSLOT - 1);   // into the slot of stage s-1
    compute(s);
  }

  // acc[mb][nb][i] = C[m0 + 32 mb + 8(i/4) + 4hk + i%4][n0 + 64 wave + 32 nb + r]
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int n = n0 + 64 * wave + 32 * nb + r;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = m0 + 32 * mb + 8 * (i >> 2) + 4 * hk + (i & 3);
        if (m < g.M && n < g.N) {
          const int64_t o = z * g.strideC + (int64_t)m * g.ldc + n;
          if (C_BF16) static_cast<uint16_t*>(g.C)[o] = f32_to_bf16(acc[mb][nb][i]);
          else if (ATOMIC) atomicAdd(static_cast<float*>(g.C) + o, acc[mb][nb][i]);
          else static_cast<float*>(g.C)[o] = acc[mb][nb][i];
        }
      }
    }
}

// C[z][m][0 .. N-1] = 0 for every z, m (rows ldc apart, matrices strideC apart).
__global__ __launch_bounds__(256) void gemm_clear_kernel(float* C, int64_t ldc, int64_t strideC, int M, int N,
                                                        int64_t rows) {
  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const int64_t z = row / M, m = row % M;
    float* c = C + z * strideC + m * ldc;
    for (int n = threadIdx.x; n < N; n += 256) c[n] = 0.f;
  }
}

}  // namespace

hipError_t launch_gemm_nt(const GemmNT& g, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0 || g.batch <= 0) return hipSuccess;
  GemmGrid gr;
  gr.n_tiles = (g.N + TN - 1) / TN;
  gr.m_tiles = (g.M + TM - 1) / TM;
  const int64_t tiles = (int64_t)gr.n_tiles * gr.m_tiles * g.batch;
  const int ksteps = g.K / 16;
  // K slices (fp32 C only) when the tiles would leave CUs without a
  // workgroup: as many as keep the items within one workgroup per CU (one
  // fits: the ring takes most of the LDS), at least 16 k steps a slice
  int ks = 1;
  if (!g.c_bf16 && tiles < 256) {
    ks = (int)(256 / tiles);
    const int most = ksteps / 16 > 1 ? ksteps / 16 : 1;
    ks = ks < most ? ks : most;
  }
  gr.ksplit = ks;
  const int64_t items = tiles * ks;
  if (items > (int64_t)INT32_MAX - 8) return hipErrorInvalidConfiguration;
  gr.items = (int)items;
  gr.items_pad = (gr.items + 7) / 8 * 8;
  if (ks > 1) {
    const int64_t rows = (int64_t)g.M * g.batch;
    const int blocks = rows < 4096 ? (int)rows : 4096;
    hipLaunchKernelGGL(gemm_clear_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<float*>(g.C), g.ldc,
                       g.strideC, g.M, g.N, rows);
  }
  const dim3 grid(gr.items_pad), block(256);
  if (g.a_f32) {
    if (g.c_bf16) hipLaunchKernelGGL((gemm_nt_kernel<true, true, false>), grid, block, 0, stream, g, gr);
    else if (ks > 1) hipLaunchKernelGGL((gemm_nt_kernel<true, false, true>), grid, block, 0, stream, g, gr);
    else hipLaunchKernelGGL((gemm_nt_kernel<true, false, false>), grid, block, 0, stream, g, gr);
  } else {
    if (g.c_bf16) hipLaunchKernelGGL((gemm_nt_kernel<false, true, false>), grid, block, 0, stream, g, gr);
    else if (ks > 1) hipLaunchKernelGGL((gemm_nt_kernel<false, false, true>), grid, block, 0, stream, g, gr);
    else hipLaunchKernelGGL((gemm_nt_kernel<false, false, false>), grid, block, 0, stream, g, gr);
  }
  return hipGetLastError();
}

}  // namespace mla
