// Decode attention over a bf16 latent cache with MFMA (gfx950).
//
// Method ([Huny] = "Multi-Head Latent Attention(MLA) 아키텍처 해부", Huny's Dev
// Blog): with the key absorbed into the query (§3.1) every head scores the
// cached rows [c_t | k^R_t] directly, s_t = q_lat.c_t + q_pe.k^R_t (§2.2
// score split), and the value sum stays in the latent space, u = sum_t a_t c_t
// (§3.2).  All heads read the same cache rows, so one workgroup serves 128
// query rows (heads x query tokens) of one sequence and streams each cache
// tile through LDS once:
//
//   S^T[tok][row]  = K_tile[tok][0:576] . [q_lat | q_pe]^T      (MFMA 16x16x32)
//   online softmax over tokens, in registers (a lane holds 2 rows x 8 tokens)
//   O^T[lat][row] += V_tile^T[lat][tok] . P^T[tok][row]          (MFMA 16x16x32)
//
// Workgroup = 4 waves; wave w owns 32 query rows (one query token, 32 heads)
// for both products.  The K operand of QK^T is read from LDS with 16-byte
// loads; the V^T operand of PV is read with ds_read_b64_tr_b16 (transposed
// 4x16 blocks), so the tile is stored once, token-major.
//
// LDS tile layout ("chunk groups"): a tile holds T=64 tokens of 72 16-byte
// chunks (576 bf16).  Chunk c of tile token t lives at 16-byte slot
//     (c / 8) * 512 + t * 8 + ((c % 8) ^ s(t)),  s(t) = ((t & 3) << 1) | ((t >> 2) & 1).
// A 1 KiB run of slots holds 8 tokens x 8 chunks, which is exactly what one
// 16-byte-per-lane global->LDS load writes; 8 lanes read 128 contiguous bytes
// of one token row (coalesced).  The xor keeps both LDS read patterns free of
// bank conflicts: 8 consecutive tokens of one chunk (QK), and 4 consecutive
// tokens of 2 neighbouring chunks (the transposed PV read).
//
// Split-KV: the workgroup walks the segments of its work unit (see
// for_each_segment) and writes one normalised partial (u, lse) per segment.

#include "mla_device.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int DC = 512;
constexpr int DR = 64;
constexpr int ROW = DC + DR;          // 576 elements
constexpr int T = 64;                 // tokens per tile
constexpr int NT = 256;               // threads per workgroup
constexpr int KSTEPS = ROW / 32;      // 18 MFMA k-steps for QK^T
constexpr int CGROUPS = ROW / 64;     // 9 chunk groups of 8 chunks
constexpr int TILE_BYTES = T * ROW * 2;  // 73728
constexpr int MBLK = DC / 16;         // 32 latent blocks of 16

struct DecodeArgs {
  const uint16_t* q_lat;   // [B][n_q][n_h][512]
  const uint16_t* q_pe;    // [B][n_q][n_h][64]
  CacheView cache;
  const int32_t* ctx_lens;
  const int32_t* positions;  // [B][n_q]
  float* u_part;           // [slots][n_q][n_h][512]
  float* lse_part;         // [slots][n_q][n_h]
  int B, n_q, n_h, num_splits, n_groups, n_work_pad;
  float scale_log2;        // sm_scale * log2(e)
};

__device__ __forceinline__ int swz(int t) { return ((t & 3) << 1) | ((t >> 2) & 1); }

struct __attribute__((aligned(16))) DecodeSmem {
  unsigned char tile[2][TILE_BYTES];
  PlanScratch<NT> plan;
};

// Issue this wave's share of the global->LDS loads of one tile: tile tokens
// 16*wave + 8*mm + lane/8 (mm = 0, 1), all 9 chunk groups.
__device__ __forceinline__ void load_tile(const DecodeArgs& a, int b, int tok0, int tok_end,
                                          unsigned char* buf, int wave, int lane) {
  const unsigned char* base = static_cast<const unsigned char*>(a.cache.data);
#pragma unroll
  for (int mm = 0; mm < 2; ++mm) {
    const int tt = 16 * wave + 8 * mm + (lane >> 3);
    int tok = tok0 + tt;
    tok = tok < tok_end ? tok : tok_end - 1;   // rows past the segment repeat a valid row
    const unsigned char* rowp = base + cache_row_offset(a.cache, b, tok) * 2;
    const int cpos = ((lane & 7) ^ swz(tt)) * 16;
#pragma unroll
    for (int cg = 0; cg < CGROUPS; ++cg) {
      unsigned char* dst = buf + cg * 8192 + (2 * wave + mm) * 1024;
      __builtin_amdgcn_global_load_lds(rowp + cg * 128 + cpos, (lds_void*)dst, 16, 0, 0);
    }
  }
}

__global__ __launch_bounds__(NT, 1) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ DecodeSmem smem;
  DecodeSmem* sm = &smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;          // lane half
  const int l32 = lane & 31;

  // block -> (work unit, row group); the groups of one unit sit 8 blocks apart
  // so that they land on the same XCD and share its L2.
  const int bid = blockIdx.x;
  const int w = (bid / (8 * a.n_groups)) * 8 + (bid & 7);
  const int g = (bid >> 3) % a.n_groups;
  if (w >= a.num_splits) return;

  const int rows = a.n_q * a.n_h;
  const int row0 = g * 128 + wave * 32;     // first query row of this wave
  const bool active = row0 < rows;
  const int jq = active ? row0 / a.n_h : 0;   // query token of this wave
  const int i0 = active ? row0 % a.n_h : 0;   // first head of this wave

  for_each_segment<NT>(a.ctx_lens, a.B, a.num_splits, w, &sm->plan,
                       [&](int b, int t0, int t1, int slot) {
    const int g4 = lane >> 4;         // lane group of 16
    const int l16 = lane & 15;
    // ---- query operand (B of QK^T): head i0 + 16*hb + l16, k = 32*ks + 8*g4 .. +8
    bf16x8 qreg[2][KSTEPS];
    int limit = t1;
    if (active) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int64_t qrow = ((int64_t)b * a.n_q + jq) * a.n_h + i0 + 16 * hb + l16;
        const u16x8* ql = reinterpret_cast<const u16x8*>(a.q_lat + qrow * DC);
        const u16x8* qp = reinterpret_cast<const u16x8*>(a.q_pe + qrow * DR);
#pragma unroll
        for (int ks = 0; ks < DC / 32; ++ks) qreg[hb][ks] = __builtin_bit_cast(bf16x8, ql[4 * ks + g4]);
#pragma unroll
        for (int ks = DC / 32; ks < KSTEPS; ++ks)
          qreg[hb][ks] = __builtin_bit_cast(bf16x8, qp[4 * (ks - DC / 32) + g4]);
      }
      const int qpos = a.positions[(int64_t)b * a.n_q + jq];
      limit = qpos + 1 < t1 ? qpos + 1 : t1;
    }
    f32x4 o[MBLK][2];
#pragma unroll
    for (int m = 0; m < MBLK; ++m) { o[m][0] = f32x4{}; o[m][1] = f32x4{}; }
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

    // per-lane LDS byte offsets that do not depend on the tile
    const int sw_qk = swz(l16 & 7);
    int qk_off[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) qk_off[r] = l16 * 128 + (((4 * r + g4) ^ sw_qk) << 4);
    const int tr_tok = 4 * g4 + (l16 >> 2);                // token (mod 32) of this lane's row
    const int sw_tr = swz(tr_tok & 7);
    const int half8 = (l16 & 1) * 8;
    const int cch = (l16 & 3) >> 1;                        // chunk within a chunk pair

    const int ntiles = (t1 - t0 + T - 1) / T;
    load_tile(a, b, t0, t1, sm->tile[0], wave, lane);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
      const int tile0 = t0 + it * T;
      unsigned char* cur = sm->tile[it & 1];
      if (it + 1 < ntiles) load_tile(a, b, tile0 + T, t1, sm->tile[(it + 1) & 1], wave, lane);
#pragma unroll 1
      for (int sub = 0; sub < 2; ++sub) {
        const int tok0 = tile0 + 32 * sub;
        if (!(active && tok0 < limit)) continue;
        unsigned char* sbuf = cur + sub * 32 * 128;
        // ------------ S^T = K . Q^T for 32 tokens: 4 chains (token block tb x head block hb),
        // K operands read from LDS PF k-steps ahead of their use.
        auto rd_k = [&](int ks, int tb) -> bf16x8 {
          const unsigned char* p = sbuf + (ks >> 1) * 8192 + tb * 2048 + qk_off[ks & 1];
          return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
              (const __attribute__((address_space(3))) unsigned char*)p);
        };
        constexpr int PF = 2;
        f32x4 sacc[2][2] = {{f32x4{}, f32x4{}}, {f32x4{}, f32x4{}}};
        bf16x8 kring[PF][2];
#pragma unroll
        for (int ks = 0; ks < PF; ++ks) { kring[ks][0] = rd_k(ks, 0); kring[ks][1] = rd_k(ks, 1); }
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          const bf16x8 k0 = kring[ks % PF][0], k1 = kring[ks % PF][1];
          if (ks + PF < KSTEPS) { kring[ks % PF][0] = rd_k(ks + PF, 0); kring[ks % PF][1] = rd_k(ks + PF, 1); }
          sacc[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qreg[0][ks], sacc[0][0], 0, 0, 0);
          sacc[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qreg[1][ks], sacc[0][1], 0, 0, 0);
          sacc[1][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qreg[0][ks], sacc[1][0], 0, 0, 0);
          sacc[1][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qreg[1][ks], sacc[1][1], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        // ------------ online softmax; lane holds heads (hb, l16), tokens 16*tb + 4*g4 + i
        bf16x8 pb[2];
        float alpha[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          float mt = -INFINITY;
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int tok = tok0 + 16 * tb + 4 * g4 + i;
              float x = sacc[tb][hb][i] * a.scale_log2;
              x = tok < limit ? x : -INFINITY;
              sacc[tb][hb][i] = x;
              mt = fmaxf(mt, x);
            }
          mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
          mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
          const float m_new = fmaxf(m_run[hb], mt);
          const float m_use = m_new == -INFINITY ? 0.f : m_new;
          alpha[hb] = __builtin_amdgcn_exp2f(m_run[hb] - m_use);
          float psum = 0.f;
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float p = __builtin_amdgcn_exp2f(sacc[tb][hb][i] - m_use);
              psum += p;
              pb[hb][4 * tb + i] = (__bf16)p;
            }
          l_run[hb] = l_run[hb] * alpha[hb] + psum;
          m_run[hb] = m_new;
        }
        if (__builtin_amdgcn_ballot_w64(alpha[0] != 1.f || alpha[1] != 1.f)) {
#pragma unroll
          for (int m = 0; m < MBLK; ++m) { o[m][0] *= alpha[0]; o[m][1] *= alpha[1]; }
        }
        // ------------ O^T += V^T . P^T: 32 latent blocks of 16, each fed by two
        // transposed LDS reads (tokens 4*g4 + r and 16 + 4*g4 + r) issued
        // PV_PF blocks ahead; the A operand serves both head blocks.
        auto rd_v = [&](int mb) -> bf16x8 {
          const int cq = 2 * (mb & 3) + cch;
          bf16x4 v[2];
#pragma unroll
          for (int ins = 0; ins < 2; ++ins) {
            const int t = 16 * ins + tr_tok;
            const unsigned char* p = sbuf + (mb >> 2) * 8192 + t * 128 + ((cq ^ sw_tr) << 4) + half8;
            v[ins] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4*)((__attribute__((address_space(3))) unsigned char*)p));
          }
          return __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
        };
        constexpr int PV_PF = 2;
        bf16x8 vring[PV_PF];
#pragma unroll
        for (int mb = 0; mb < PV_PF; ++mb) vring[mb] = rd_v(mb);
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb) {
          const bf16x8 va = vring[mb % PV_PF];
          if (mb + PV_PF < MBLK) vring[mb % PV_PF] = rd_v(mb + PV_PF);
          o[mb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[0], o[mb][0], 0, 0, 0);
          o[mb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[1], o[mb][1], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }

    // ---------------- write the partial of this segment
    if (active) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float l_tot = l_run[hb] + __shfl_xor(l_run[hb], 16, 64);
        l_tot += __shfl_xor(l_tot, 32, 64);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        const int64_t prow = ((int64_t)slot * a.n_q + jq) * a.n_h + i0 + 16 * hb + l16;
        float* up = a.u_part + prow * DC + 4 * g4;
#pragma unroll
        for (int mb = 0; mb < MBLK; ++mb)
          *reinterpret_cast<f32x4*>(up + 16 * mb) = o[mb][hb] * inv;
        if (g4 == 0)
          a.lse_part[prow] = l_tot > 0.f ? (m_run[hb] + __log2f(l_tot)) * kLn2 : -INFINITY;
      }
    }
  });
}

}  // namespace

int decode_mfma_smem_bytes() { return (int)sizeof(DecodeSmem); }

hipError_t launch_decode_mfma(const DecodeParams& p, hipStream_t stream) {
  DecodeArgs a;
  a.q_lat = static_cast<const uint16_t*>(p.q_lat);
  a.q_pe = static_cast<const uint16_t*>(p.q_pe);
  a.cache = p.cache;
  a.ctx_lens = p.ctx_lens;
  a.positions = p.positions;
  a.u_part = p.u_part;
  a.lse_part = p.lse_part;
  a.B = p.B;
  a.n_q = p.n_q;
  a.n_h = p.n_h;
  a.num_splits = p.num_splits;
  a.n_groups = (p.n_q * p.n_h + 127) / 128;
  a.n_work_pad = (p.num_splits + 7) / 8 * 8;
  a.scale_log2 = p.sm_scale * kLog2e;
  const int grid = a.n_work_pad * a.n_groups;
  hipLaunchKernelGGL(decode_mfma_kernel, dim3(grid), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
