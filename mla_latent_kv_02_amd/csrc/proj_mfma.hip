// MFMA (gfx950) kernels for the two per-head projections around the decode,
// bf16 weights, fp32 accumulation.  Both are weight-bandwidth-bound skinny
// GEMMs (M = B * n_q rows, one head's weight matrix per workgroup).
//
// Key absorption q_lat = q^C_i (W_i^UK)^T ([Huny] = "Multi-Head Latent
// Attention(MLA) 아키텍처 해부", Huny's Dev Blog, §3.1).  Computed transposed,
// q_lat^T[c][m] = W_i^UK[c][:] . q^C[m][:], so that both MFMA operands are
// rows that are contiguous in memory along the contraction (d_nope): W_UK row c
// is the A operand and the query row m the B operand, 16 bytes per lane, no
// transpose.  One wave = 16 latent columns x all query rows.
//
// Value up-projection o_i = u_i W_i^UV ([Huny] §3.2).  W_i^UV is [d_c][d_v]
// with d_v contiguous, but the MFMA B operand wants d_c (the contraction)
// contiguous per lane, so 64-row chunks of W_i^UV are staged in LDS and read
// with ds_read_b64_tr_b16 (transposed 4x16 blocks).  u is fp32; it is split
// into a bf16 high part and a bf16 residual (u = hi + lo to ~2^-16) and both
// are multiplied, so the projection keeps fp32-level accuracy.

#include "mla_device.h"
#include "launch.h"
#include "append_row.h"

namespace mla {
namespace {

// ------------------------------------------------------------- absorption
// grid (n_h, d_c / 64); 4 waves, wave w -> latent columns c0 = 64*blockIdx.y + 16*w.
// Requires d_nope % 32 == 0, d_nope <= 128, d_c % 64 == 0.
constexpr int AB_MAXK = 4;            // d_nope / 32 held in registers
__global__ __launch_bounds__(256) void absorb_mfma_kernel(AbsorbParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = blockIdx.x;
  const int c0 = blockIdx.y * 64 + wave * 16;
  const int g = lane >> 4, l16 = lane & 15;
  const int M = p.B * p.n_q;
  const int ksteps = p.d_nope / 32;
  const uint16_t* w = static_cast<const uint16_t*>(p.w_uk) + ((int64_t)i * p.d_c + c0 + l16) * p.d_nope + 8 * g;
  const uint16_t* q = static_cast<const uint16_t*>(p.q_nope);
  uint16_t* out = static_cast<uint16_t*>(p.q_lat);
  bf16x8 a[AB_MAXK];
#pragma unroll
  for (int ks = 0; ks < AB_MAXK; ++ks)
    if (ks < ksteps) a[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u16x8*>(w + 32 * ks));
  for (int m0 = 0; m0 < M; m0 += 64) {
    u16x8 bq[4][AB_MAXK];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + 16 * mb + l16;
      const uint16_t* qr = q + ((int64_t)m * p.n_h + i) * p.d_nope + 8 * g;
#pragma unroll
      for (int ks = 0; ks < AB_MAXK; ++ks) {
        bq[mb][ks] = u16x8{0, 0, 0, 0, 0, 0, 0, 0};
        if (ks < ksteps && m < M) bq[mb][ks] = *reinterpret_cast<const u16x8*>(qr + 32 * ks);
      }
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + 16 * mb + l16;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < AB_MAXK; ++ks)
        if (ks < ksteps)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], __builtin_bit_cast(bf16x8, bq[mb][ks]), acc, 0, 0, 0);
      // acc[r] = q_lat[m][i][c0 + 4g + r]
      if (m < M) {
        u16x4 o4 = {f32_to_bf16(acc[0]), f32_to_bf16(acc[1]), f32_to_bf16(acc[2]), f32_to_bf16(acc[3])};
        *reinterpret_cast<u16x4*>(out + ((int64_t)m * p.n_h + i) * p.d_c + c0 + 4 * g) = o4;
      }
    }
  }
}

// Query RoPE over rows (query row m, head i) of d_rope elements.  Items are
// runs of 4 rotation planes (16 bytes of a bf16 row) when the rows allow
// (d_rope % 8 == 0 and 16-byte aligned arrays; VEC), else single planes; the
// plane index runs fastest, so a wave reads and writes contiguous bytes.  A
// grid-stride loop over a few workgroups per CU builds the frequency table
// once per workgroup (fp64).  fp32 rows take fp64 sin and cos of the angle;
// bf16 rows the fp32 sin and cos of the fp64-reduced angle in turns (about
// 1e-6 absolute, far below a bf16 step), as the one-pass kernel does.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void rope_q_rows_kernel(AbsorbParams p) {
  __shared__ double freq[64];   // turns (bf16) or radians (fp32) per unit of position
  const int half = p.d_rope / 2;
  const bool table = half <= 64;
  if (table && (int)threadIdx.x < half) {
    const double th = pow((double)p.rope_base, -2.0 * threadIdx.x / p.d_rope);
    freq[threadIdx.x] = sizeof(T) == 2 ? th * kInv2Pi : th;
  }
  __syncthreads();
  constexpr int PER = VEC ? 4 : 1;   // planes per item
  const int per_row = half / PER;
  const int64_t items = (int64_t)p.B * p.n_q * p.n_h * per_row;
  const T* src = static_cast<const T*>(p.q_rope);
  T* dst = static_cast<T*>(p.q_pe);
  for (int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x; it < items; it += (int64_t)gridDim.x * 256) {
    const int k0 = (int)(it % per_row) * PER;
    const int64_t mi = it / per_row;             // m * n_h + i
    const int pos = p.positions[mi / p.n_h];
    const int64_t off = mi * p.d_rope + 2 * k0;
    float x[2 * PER], y[2 * PER];
    if (VEC && sizeof(T) == 2) {
      const u16x8 v = *reinterpret_cast<const u16x8*>(src + off);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32(v[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 2 * PER; ++e) x[e] = Elem<T>::load(src, off + e);
    }
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int k = k0 + q;
      float c, s;
      if (sizeof(T) == 2) {
        const double turns = table ? freq[k] : pow((double)p.rope_base, -2.0 * k / p.d_rope) * kInv2Pi;
        sincos_turns(pos, turns, &s, &c);
      } else {
        const double th = table ? freq[k] : pow((double)p.rope_base, -2.0 * k / p.d_rope);
        double sd, cd;
        sincos((double)pos * th, &sd, &cd);
        c = (float)cd;
        s = (float)sd;
      }
      y[2 * q] = x[2 * q] * c - x[2 * q + 1] * s;
      y[2 * q + 1] = x[2 * q] * s + x[2 * q + 1] * c;
    }
    if (VEC && sizeof(T) == 2) {
      u16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = f32_to_bf16(y[e]);
      *reinterpret_cast<u16x8*>(dst + off) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 2 * PER; ++e) Elem<T>::store(dst, off + e, y[e]);
    }
  }
}

// Launch of the query RoPE: 16-byte items where the arrays allow.
template <typename T>
hipError_t launch_rope_rows(const AbsorbParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.n_q * p.n_h;
  if (rows == 0) return hipSuccess;
  const bool vec = sizeof(T) == 2 && p.d_rope % 8 == 0 && reinterpret_cast<uintptr_t>(p.q_rope) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(p.q_pe) % 16 == 0;
  const int64_t items = rows * (p.d_rope / 2) / (vec ? 4 : 1);
  const int64_t want = (items + 255) / 256;
  const dim3 grid((unsigned)(want < 2048 ? want : 2048));
  if (vec) hipLaunchKernelGGL((rope_q_rows_kernel<T, true>), grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((rope_q_rows_kernel<T, false>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

// ------------------------------------------- absorption + query RoPE, one pass
// grid: n_h * (d_c / 256) workgroups; workgroup (head i, slice h2) computes
// q_lat[:, i, 256 h2 .. +256] and the query RoPE of head i for the rows m with
// m % (d_c / 256) == h2.  Wave w owns latents c0 = 256 h2 + 64 w .. +64 (four
// 16-latent MFMA tiles, W_UK rows as the A operand held in registers) and walks
// the query rows 64 at a time (four 16-row tiles, the B operand).  Every load
// of a 64-row block is issued before any MFMA; the RoPE of the workgroup's rows
// runs while the first block is in flight.  C tile (latent tile t, row tile
// mt): lane l holds latents 16t + 4(l/16) + 0..3 of row 16mt + l%16, stored as
// 8 bytes (a wave writes 128 contiguous bytes of each row).
// Requires d_nope == 128, d_c % 256 == 0, bf16.
// Workgroups n_absorb and up take the append role instead: they write the new
// bf16 or fp8 cache rows of `ap` (as the append kernel does),
// on CUs beside the absorption workgroups, so that a step's append costs no
// launch of its own.
constexpr int AR_LAT = 256;           // latents per workgroup
constexpr int AR_ROPE = 8;            // RoPE items per thread whose loads go first
__global__ __launch_bounds__(256) void absorb_rope_kernel(AbsorbParams p, AppendParams ap, int n_absorb) {
  if ((int)blockIdx.x >= n_absorb) {
    if (ap.fp8) {   // one wave per new row
      const int stride = (gridDim.x - n_absorb) * 4;
      for (int k = (blockIdx.x - n_absorb) * 4 + (threadIdx.x >> 6); k < ap.n; k += stride)
        append_row_fp8(ap, k, threadIdx.x & 63);
      return;
    }
    const int pairs = (ap.d_c + ap.d_rope) / 2;
    const int64_t items = (int64_t)ap.n * pairs;
    const int64_t stride = (int64_t)(gridDim.x - n_absorb) * 256;
    for (int64_t it = (int64_t)(blockIdx.x - n_absorb) * 256 + threadIdx.x; it < items; it += stride)
      append_pair<uint16_t>(ap, (int)(it / pairs), (int)(it % pairs));
    return;
  }
  __shared__ double theta[64];
  // per wave: a 64-row x 64-latent block of q_lat (bf16, 128 bytes a row,
  // 16-byte chunk c of row r at c ^ (r % 8)) on its way to memory
  __shared__ __attribute__((aligned(16))) unsigned char qout[4][64 * 128];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nslices = p.d_c / AR_LAT;
  const int i = blockIdx.x / nslices, h2 = blockIdx.x % nslices;
  const int c0 = h2 * AR_LAT + wave * 64;
  const int g = lane >> 4, l16 = lane & 15;
  const int M = p.B * p.n_q;
  const int half = p.d_rope / 2;
  // ---- query RoPE of head i, rows m = h2, h2 + nslices, ...: the loads of
  // the first AR_ROPE items of this thread are issued before the GEMM loads,
  // so the rotation only waits for them
  const uint16_t* rsrc = static_cast<const uint16_t*>(p.q_rope);
  uint16_t* rdst = static_cast<uint16_t*>(p.q_pe);
  const int rrows = (M - h2 + nslices - 1) / nslices;
  const int ritems = rrows * half;
  auto rope_off = [&](int idx, int& m, int& k) -> int64_t {
    m = h2 + nslices * (idx / half);
    k = idx % half;
    return ((int64_t)m * p.n_h + i) * p.d_rope + 2 * k;
  };
  uint32_t rx[AR_ROPE];
  int rpos[AR_ROPE];
#pragma unroll
  for (int e = 0; e < AR_ROPE; ++e) {
    const int idx = threadIdx.x + 256 * e;
    rx[e] = 0;
    rpos[e] = 0;
    if (idx < ritems) {
      int m, k;
      const int64_t off = rope_off(idx, m, k);
      rx[e] = *reinterpret_cast<const uint32_t*>(rsrc + off);
      rpos[e] = p.positions[m];
    }
  }
  // A: W_UK[i][c0 + 16t + l16][32ks + 8g .. +8]
  const uint16_t* w = static_cast<const uint16_t*>(p.w_uk) + ((int64_t)i * p.d_c + c0 + l16) * 128 + 8 * g;
  u16x8 a[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) a[t][ks] = *reinterpret_cast<const u16x8*>(w + t * 16 * 128 + 32 * ks);
  const uint16_t* q = static_cast<const uint16_t*>(p.q_nope);
  uint16_t* out = static_cast<uint16_t*>(p.q_lat);
  auto load_b = [&](int m0, u16x8 (&bq)[4][4]) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int m = m0 + 16 * mt + l16;
      const uint16_t* qr = q + ((int64_t)(m < M ? m : 0) * p.n_h + i) * 128 + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) bq[mt][ks] = *reinterpret_cast<const u16x8*>(qr + 32 * ks);
    }
  };
  u16x8 bq[4][4];
  load_b(0, bq);
  // turns per position of plane k: base^(-2k/d_rope) / (2 pi), formed while
  // the loads above are in flight (the barrier waits for LDS only)
  if (threadIdx.x < half) theta[threadIdx.x] = pow((double)p.rope_base, -2.0 * threadIdx.x / p.d_rope) * kInv2Pi;
  lds_sync();
  auto rotate = [&](int idx, uint32_t x, int pos) {
    int m, k;
    const int64_t off = rope_off(idx, m, k);
    float sn, cs;
    sincos_turns(pos, theta[k], &sn, &cs);
    const float x0 = bf16_to_f32((uint16_t)(x & 0xFFFF)), x1 = bf16_to_f32((uint16_t)(x >> 16));
    *reinterpret_cast<uint32_t*>(rdst + off) =
        (uint32_t)f32_to_bf16(x0 * cs - x1 * sn) | ((uint32_t)f32_to_bf16(x0 * sn + x1 * cs) << 16);
  };
#pragma unroll
  for (int e = 0; e < AR_ROPE; ++e) {
    const int idx = threadIdx.x + 256 * e;
    if (idx < ritems) rotate(idx, rx[e], rpos[e]);
  }
  for (int idx = threadIdx.x + 256 * AR_ROPE; idx < ritems; idx += 256) {   // rows beyond the first 8*256 items
    int m, k;
    const int64_t off = rope_off(idx, m, k);
    rotate(idx, *reinterpret_cast<const uint32_t*>(rsrc + off), p.positions[m]);
  }
  for (int m0 = 0; m0 < M; m0 += 64) {
    // the next block's query rows are in flight while this block is computed
    u16x8 bn[4][4];
    if (m0 + 64 < M) load_b(m0 + 64, bn);
    // the block's results go through this wave's LDS block, so that each
    // store writes 8 rows x 128 contiguous bytes (from the registers a store
    // would carry 8 bytes of each of 64 rows)
    typedef __attribute__((address_space(3))) u16x4 lds_u16x4;
    typedef __attribute__((address_space(3))) const u32x4 lds_cu32x4;
    unsigned char* qo = qout[wave];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int r = 16 * mt + l16;
      f32x4 acc[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[t][ks]),
                                                           __builtin_bit_cast(bf16x8, bq[mt][ks]), acc[t], 0, 0, 0);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // latents 16t + 4g .. +3 of row r: chunk 2t + g/2, bytes 8(g%2) of it
        const u16x4 o4 = {f32_to_bf16(acc[t][0]), f32_to_bf16(acc[t][1]), f32_to_bf16(acc[t][2]),
                          f32_to_bf16(acc[t][3])};
        const int c = 2 * t + (g >> 1);
        *(lds_u16x4*)((__attribute__((address_space(3))) unsigned char*)(qo + r * 128 + ((c ^ (r & 7)) << 4) +
                                                                          8 * (g & 1))) = o4;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's block is in (only it reads it)
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int r = 8 * it + (lane >> 3), c = lane & 7;
      const u32x4 v = *(lds_cu32x4*)((__attribute__((address_space(3))) unsigned char*)(qo + r * 128 +
                                                                                        ((c ^ (r & 7)) << 4)));
      if (m0 + r < M) *reinterpret_cast<u32x4*>(out + ((int64_t)(m0 + r) * p.n_h + i) * p.d_c + c0 + 8 * c) = v;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads done before the next block's writes
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) bq[mt][ks] = bn[mt][ks];
  }
}

// --------------------------------------------------------- up-projection
constexpr int OP_MROWS = 64;          // query rows per workgroup (4 waves x 16)
constexpr int OP_KCHUNK = 64;         // rows of W_UV staged per LDS chunk
constexpr int OP_VCOLS = 32;          // value columns per workgroup
constexpr int OP_MAXV = OP_VCOLS;
constexpr int OP_PITCH = OP_MAXV * 2 + 32;  // bytes per staged row (pad against bank conflicts)

// grid (n_h, ceil(M / 64), d_v / 32); wave w -> rows m0 + 16w .. +16 and the
// workgroup's 32 value columns.  Requires d_c % 64 == 0, d_v % 32 == 0.
__global__ __launch_bounds__(256) void out_proj_mfma_kernel(OutProjParams p) {
  __shared__ __attribute__((aligned(16))) unsigned char wsm[OP_KCHUNK * OP_PITCH];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int i = blockIdx.x;
  const int M = p.B * p.n_q;
  const int m = blockIdx.y * OP_MROWS + wave * 16 + l16;     // A-operand row of this lane
  const int vblocks = OP_VCOLS / 16;
  const int v0 = blockIdx.z * OP_VCOLS;
  const uint16_t* w = static_cast<const uint16_t*>(p.w_uv) + (int64_t)i * p.d_c * p.d_v + v0;
  const float* ur = p.u + ((int64_t)(m < M ? m : 0) * p.n_h + i) * p.d_c + 8 * g;
  f32x4 acc[OP_MAXV / 16];
#pragma unroll
  for (int v = 0; v < OP_MAXV / 16; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int row_bytes = OP_VCOLS * 2;
  const int pieces = OP_KCHUNK * (row_bytes / 16);               // 16-byte pieces per chunk
  constexpr int PER_T = (OP_KCHUNK * OP_MAXV * 2 / 16 + 255) / 256;  // pieces per thread
  u16x8 stage[PER_T];
#define OP_FETCH(C0)                                                                       \
  _Pragma("unroll") for (int k = 0; k < PER_T; ++k) {                                     \
    const int e = tid + 256 * k;                                                           \
    if (e < pieces) {                                                                      \
      const int r = e / (row_bytes / 16), cc = e % (row_bytes / 16);                       \
      stage[k] = *reinterpret_cast<const u16x8*>(w + (int64_t)((C0) + r) * p.d_v + cc * 8); \
    }                                                                                      \
  }
  OP_FETCH(0)
  for (int c0 = 0; c0 < p.d_c; c0 += OP_KCHUNK) {
    __syncthreads();
#pragma unroll
    for (int k = 0; k < PER_T; ++k) {
      const int e = tid + 256 * k;
      if (e < pieces) {
        const int r = e / (row_bytes / 16), cc = e % (row_bytes / 16);
        *reinterpret_cast<u16x8*>(wsm + r * OP_PITCH + cc * 16) = stage[k];
      }
    }
    __syncthreads();
    if (c0 + OP_KCHUNK < p.d_c) { OP_FETCH(c0 + OP_KCHUNK) }
#pragma unroll
    for (int ks = 0; ks < OP_KCHUNK / 32; ++ks) {
      // A: u[m][c0 + 32ks + 8g .. +8], split into bf16 hi + lo
      f32x4 u0 = {0.f, 0.f, 0.f, 0.f}, u1 = u0;
      if (m < M) {
        u0 = *reinterpret_cast<const f32x4*>(ur + c0 + 32 * ks);
        u1 = *reinterpret_cast<const f32x4*>(ur + c0 + 32 * ks + 4);
      }
      u16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = e < 4 ? u0[e] : u1[e - 4];
        const uint16_t h = f32_to_bf16(x);
        hi[e] = h;
        lo[e] = f32_to_bf16(x - bf16_to_f32(h));
      }
      const bf16x8 ahi = __builtin_bit_cast(bf16x8, hi), alo = __builtin_bit_cast(bf16x8, lo);
      // B: W[c0 + 32ks + 8g + 4ins + (l16 >> 2)][16vb + 4(l16 & 3) .. +4], transposed read
#pragma unroll
      for (int vb = 0; vb < OP_MAXV / 16; ++vb) {
        if (vb < vblocks) {
        bf16x4 bv[2];
#pragma unroll
        for (int ins = 0; ins < 2; ++ins) {
          const int r = 32 * ks + 8 * g + 4 * ins + (l16 >> 2);
          const unsigned char* ptr = wsm + r * OP_PITCH + (16 * vb + 4 * (l16 & 3)) * 2;
          bv[ins] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (lds_bf16x4*)((__attribute__((address_space(3))) unsigned char*)ptr));
        }
        const bf16x8 b = __builtin_shufflevector(bv[0], bv[1], 0, 1, 2, 3, 4, 5, 6, 7);
        acc[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, b, acc[vb], 0, 0, 0);
        acc[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, b, acc[vb], 0, 0, 0);
        }
      }
    }
  }
#undef OP_FETCH
  // acc[vb][r] = o[m' = rowblock + 4g + r][16 vb + l16]
  const int mrow0 = blockIdx.y * OP_MROWS + wave * 16 + 4 * g;
#pragma unroll
  for (int vb = 0; vb < OP_MAXV / 16; ++vb) {
    if (vb < vblocks) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int mm = mrow0 + r;
        if (mm < M) p.out[((int64_t)mm * p.n_h + i) * p.d_v + v0 + 16 * vb + l16] = acc[vb][r];
      }
    }
  }
}

}  // namespace

hipError_t launch_rope_q(const AbsorbParams& p, hipStream_t stream) {
  return p.bf16 ? launch_rope_rows<uint16_t>(p, stream) : launch_rope_rows<float>(p, stream);
}

bool absorb_mfma_ok(const AbsorbParams& p) {
  return p.bf16 && p.d_nope % 32 == 0 && p.d_nope <= 32 * AB_MAXK && p.d_c % 64 == 0;
}

hipError_t launch_absorb_mfma(const AbsorbParams& p, hipStream_t stream) {
  return launch_append_absorb_mfma(p, nullptr, stream);
}

hipError_t launch_append_absorb_mfma(const AbsorbParams& p, const AppendParams* ap, hipStream_t stream) {
  const int M = p.B * p.n_q;
  const bool append = ap != nullptr && ap->n > 0;
  const bool one_pass = p.d_nope == 128 && p.d_c % AR_LAT == 0;
  const bool fused = one_pass && (ap != nullptr) && (ap->bf16 || ap->fp8);
  if (append && !fused) {   // the append gets a launch of its own
    const hipError_t e = launch_cache_append(*ap, stream);
    if (e != hipSuccess) return e;
  }
  if (one_pass) {
    const int n_absorb = p.n_h * (p.d_c / AR_LAT);
    AppendParams none{};
    int n_append = 0;
    if (append && fused) {
      const int64_t blocks = ap->fp8 ? ((int64_t)ap->n + 3) / 4
                                     : ((int64_t)ap->n * ((ap->d_c + ap->d_rope) / 2) + 255) / 256;
      n_append = (int)(blocks < 256 ? blocks : 256);
    }
    hipLaunchKernelGGL(absorb_rope_kernel, dim3(n_absorb + n_append), dim3(256), 0, stream, p,
                       n_append > 0 ? *ap : none, n_absorb);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(absorb_mfma_kernel, dim3(p.n_h, p.d_c / 64), dim3(256), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_rope_rows<uint16_t>(p, stream);
}

bool out_proj_mfma_ok(const OutProjParams& p) {
  return p.bf16 && p.d_c % OP_KCHUNK == 0 && p.d_v % OP_VCOLS == 0;
}

hipError_t launch_out_proj_mfma(const OutProjParams& p, hipStream_t stream) {
  const int M = p.B * p.n_q;
  dim3 grid(p.n_h, (M + OP_MROWS - 1) / OP_MROWS, p.d_v / OP_VCOLS);
  hipLaunchKernelGGL(out_proj_mfma_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
