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
// LDS stage layout ("chunk groups"): a stage holds T=32 tokens of 72 16-byte
// chunks (576 bf16).  Chunk c of stage token t lives at 16-byte slot
//     (c / 8) * 256 + t * 8 + ((c % 8) ^ s(t)),  s(t) = ((t & 3) << 1) | ((t >> 2) & 1).
// A 1 KiB run of slots holds 8 tokens x 8 chunks, which is exactly what one
// 16-byte-per-lane global->LDS load writes; 8 lanes read 128 contiguous bytes
// of one token row (coalesced).  The xor keeps both LDS read patterns free of
// bank conflicts: 8 consecutive tokens of one chunk (QK), and 4 consecutive
// tokens of 2 neighbouring chunks (the transposed PV read).
//
// Pipeline: a ring of NSTAGE stages in LDS; loads run NSTAGE - 1 stages ahead
// of the stage being used, and each wave waits (vmcnt) only for the oldest
// stage it needs.  Softmax weights exp2(s - m_ref) use a fixed per-row
// reference, so the fp32 accumulator is never rescaled; the partial is
// written unnormalised together with its reference and log-sum-exp, and the
// combine normalises (exact for any reference).
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
constexpr int T = 32;                 // tokens per pipeline stage
constexpr int NSTAGE = 4;             // LDS ring: NSTAGE - 1 stages in flight while one is used
constexpr int NT = 256;               // threads per workgroup
constexpr int KSTEPS = ROW / 32;      // 18 MFMA k-steps for QK^T
constexpr int CGROUPS = ROW / 64;     // 9 chunk groups of 8 chunks
constexpr int CG_BYTES = T * 128;     // one chunk group of a stage: 32 tokens x 128 B
constexpr int STAGE_BYTES = CGROUPS * CG_BYTES;   // 36864
constexpr int LOADS_PER_STAGE = CGROUPS;          // 16-byte-per-lane loads per wave per stage
constexpr int MBLK = DC / 16;         // 32 latent blocks of 16
constexpr float REF_HEADROOM = 64.f;  // log2 units a score may exceed its row's reference

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
  unsigned char stage[NSTAGE][STAGE_BYTES];
  bf16x8 pbuf[8][64];        // softmax weights of the stage, MFMA B-operand layout, per head block
  int flag[4];               // per wave: a score ran past its row's reference (redo needed)
  PlanScratch<NT> plan;
};

// Block id of the paged cache for token `tok` of sequence b, read with a
// scalar load (the index is wave-uniform).  Scalar loads are counted by
// lgkmcnt, so waiting for them does not drain the vector-memory queue that
// holds the in-flight stage loads.
__device__ __forceinline__ int block_id_scalar(const CacheView& c, int b, int tok) {
  const int32_t* p = c.block_table + (int64_t)b * c.max_blocks + tok / c.block_size;
  // readfirstlane returns a signed int: widen through uint32_t (zero-extend)
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)p);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uintptr_t)p >> 32));
  const uint64_t addr = (uint64_t)lo | ((uint64_t)hi << 32);
  int v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(addr) : "memory");
  return v;
}

// This wave's share of the global->LDS loads of one stage: stage tokens
// 8*wave + lane/8, all 9 chunk groups (9 loads of 1 KiB per wave).
__device__ __forceinline__ void load_stage(const DecodeArgs& a, int b, int tok0, int tok_end,
                                           unsigned char* buf, int wave, int lane) {
  const unsigned char* base = static_cast<const unsigned char*>(a.cache.data);
  const int tt = 8 * wave + (lane >> 3);
  int tok = tok0 + tt;
  tok = tok < tok_end ? tok : tok_end - 1;   // rows past the segment repeat a valid row
  int64_t off;
  const CacheView& c = a.cache;
  if (c.block_size == 0) {
    off = (int64_t)b * c.seq_stride + (int64_t)tok * ROW;
  } else if (c.block_size >= T) {
    // the stage's tokens lie in at most two blocks: those of its first and last token
    const int last = tok0 + T - 1 < tok_end - 1 ? tok0 + T - 1 : tok_end - 1;
    const int blk0 = block_id_scalar(c, b, tok0);
    const int blk1 = block_id_scalar(c, b, last);
    const int blk = tok / c.block_size == tok0 / c.block_size ? blk0 : blk1;
    off = ((int64_t)blk * c.block_size + tok % c.block_size) * ROW;
  } else {
    off = cache_row_offset(c, b, tok);
  }
  const unsigned char* rowp = base + off * 2 + ((lane & 7) ^ swz(tt)) * 16;
  unsigned char* dst = buf + wave * 1024;
#pragma unroll
  for (int cg = 0; cg < CGROUPS; ++cg)
    __builtin_amdgcn_global_load_lds(rowp + cg * 128, (lds_void*)(dst + cg * CG_BYTES), 16, 0, 0);
}

// Workgroup barrier that waits only for this wave's LDS operations (a
// __syncthreads() would also wait for every outstanding global load and so
// drain the stage pipeline).  Stage data arriving through global->LDS loads is
// covered by the explicit vmcnt waits before the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt immediates (GFX9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] << 14) that wait on vector memory only.  Issued through the
// builtin so that the compiler's own wait insertion sees them.
constexpr int kWaitVm0 = 0x0F70, kWaitVm9 = 0x0F79, kWaitVm18 = 0x4F72;

// O += A . B for one 16x16 block of the PV product, with the accumulator pinned
// to AGPRs.  O needs all 256 AGPRs; the QK^T accumulators (built-in MFMAs,
// compiled in the VGPR form) stay in VGPRs, so the allocator never moves O
// blocks between register files inside the stage loop.
__device__ __forceinline__ void pv_mfma(f32x4& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Wait states between the last PV MFMA and any other read of its accumulator
// (the compiler cannot see the MFMA inside the asm statements above).
__device__ __forceinline__ void pv_mfma_drain() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// Wait until at most `n` stages of this wave's loads are still in flight.
__device__ __forceinline__ void wait_stages_in_flight(int n) {
  if (n >= 2) __builtin_amdgcn_s_waitcnt(kWaitVm18);
  else if (n == 1) __builtin_amdgcn_s_waitcnt(kWaitVm9);
  else __builtin_amdgcn_s_waitcnt(kWaitVm0);
}
static_assert(LOADS_PER_STAGE == 9 && NSTAGE == 4, "wait counts assume 9 loads per stage, 4 stages");

// Work split inside a workgroup of 4 waves serving 128 query rows:
//   QK^T and softmax: wave w owns rows 32w .. 32w+31 (its heads' queries stay in
//     registers as the MFMA B operand);
//   PV: wave w owns latent columns 128w .. 128w+127 for all 128 rows, so each
//     V element is read from LDS once per workgroup; the softmax weights of all
//     rows come through LDS (each wave's weights are already in the B-operand
//     lane layout, so the exchange is a 16-byte copy per lane and head block).
// The accumulator O is touched only by MFMAs and by the final store: the
// weights use a fixed per-row reference (the row's maximum over the first
// stage), which needs no rescaling of O.  If a later score exceeds the
// reference by more than REF_HEADROOM (log2 units; weights stay below
// 2^REF_HEADROOM, far from fp32/bf16 overflow), the segment is computed again
// with the row's true maximum as the reference.
__global__ __launch_bounds__(NT, 1) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ DecodeSmem smem;
  DecodeSmem* sm = &smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g4 = lane >> 4;         // lane group of 16
  const int l16 = lane & 15;

  // block -> (work unit, row group); the groups of one unit sit 8 blocks apart
  // so that they land on the same XCD and share its L2.
  const int bid = blockIdx.x;
  const int w = (bid / (8 * a.n_groups)) * 8 + (bid & 7);
  const int g = (bid >> 3) % a.n_groups;
  if (w >= a.num_splits) return;

  const int rows = a.n_q * a.n_h;
  const int grow0 = g * 128;                  // first query row of the workgroup
  const int row0 = grow0 + wave * 32;         // first QK row of this wave
  const bool active = row0 < rows;
  const int jq = active ? row0 / a.n_h : 0;   // query token of this wave's QK rows

  for_each_segment<NT>(a.ctx_lens, a.B, a.num_splits, w, &sm->plan,
                       [&](int b, int t0, int t1, int slot) {
    // ---- query operand (B of QK^T): row row0 + 16*hb + l16, k = 32*ks + 8*g4 .. +8
    bf16x8 qreg[2][KSTEPS];
    int limit = t1;
    if (active) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int64_t qrow = (int64_t)b * rows + row0 + 16 * hb + l16;
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
    // the query operands must not be waited for inside the stage loop, where the
    // vector-memory counter also covers the stage loads
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    // per-lane LDS byte offsets that do not depend on the stage
    const int sw_qk = swz(l16 & 7);
    int qk_off[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) qk_off[r] = l16 * 128 + (((4 * r + g4) ^ sw_qk) << 4);
    const int tr_tok = 4 * g4 + (l16 >> 2);                // token (mod 16) of this lane's row
    const int sw_tr = swz(tr_tok & 7);
    const int half8 = (l16 & 1) * 8;
    const int cch = (l16 & 3) >> 1;                        // chunk within a chunk pair
    const int nst = (t1 - t0 + T - 1) / T;

    // m_ref: reference (log2 units) of each of the lane's two QK rows;
    // m_max: running maximum of the row's scores
    float m_ref[2] = {-INFINITY, -INFINITY}, m_max[2] = {-INFINITY, -INFINITY};
    float l_run[2];
    // O^T accumulators of this wave: latent block mb (16 latents at 128*wave + 16*mb)
    // x head block hb (rows grow0 + 16*hb .. +16)
    f32x4 o[8][8];
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int hb = 0; hb < 8; ++hb) o[mb][hb] = f32x4{};
      l_run[0] = l_run[1] = 0.f;
      bool over = false;
#pragma unroll
      for (int s = 0; s < NSTAGE - 1; ++s)
        if (s < nst) load_stage(a, b, t0 + s * T, t1, sm->stage[s], wave, lane);

      for (int it = 0; it < nst; ++it) {
        const int after = nst - 1 - it;     // stages already issued beyond this one (at most 2)
        wait_stages_in_flight(after < NSTAGE - 2 ? after : NSTAGE - 2);
        lds_barrier();
        if (it + NSTAGE - 1 < nst)
          load_stage(a, b, t0 + (it + NSTAGE - 1) * T, t1, sm->stage[(it + NSTAGE - 1) % NSTAGE], wave, lane);
        const int tok0 = t0 + it * T;
        unsigned char* sbuf = sm->stage[it % NSTAGE];
        bf16x8 pb[2] = {bf16x8{}, bf16x8{}};
        if (active && tok0 < limit) {
          // ------------ S^T = K . Q^T for 32 tokens: 4 chains (token block tb x head block hb),
          // K operands read from LDS PF k-steps ahead of their use.
          auto rd_k = [&](int ks, int tb) -> bf16x8 {
            const unsigned char* p = sbuf + (ks >> 1) * CG_BYTES + tb * 2048 + qk_off[ks & 1];
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
          // ------------ softmax weights; lane holds rows (hb, l16), tokens 16*tb + 4*g4 + i
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
            m_max[hb] = fmaxf(m_max[hb], mt);
            if (m_ref[hb] == -INFINITY) m_ref[hb] = mt;       // first visible stage of the row
            over |= mt > m_ref[hb] + REF_HEADROOM;
            const float m_use = m_ref[hb] == -INFINITY ? 0.f : m_ref[hb];
            float psum = 0.f;
#pragma unroll
            for (int tb = 0; tb < 2; ++tb)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(sacc[tb][hb][i] - m_use);
                psum += p;
                pb[hb][4 * tb + i] = (__bf16)p;
              }
            l_run[hb] += psum;
          }
        }
        // ------------ publish this wave's weights (B-operand layout)
        sm->pbuf[2 * wave][lane] = pb[0];
        sm->pbuf[2 * wave + 1][lane] = pb[1];
        lds_barrier();
        // ------------ O^T[own 128 latents][128 rows] += V^T . P^T: 8 latent blocks,
        // each fed by two transposed LDS reads and reused for the 8 head blocks.
        bf16x8 pall[8];
#pragma unroll
        for (int hb = 0; hb < 8; ++hb) pall[hb] = sm->pbuf[hb][lane];
        auto rd_v = [&](int mb) -> bf16x8 {
          const int mbg = 8 * wave + mb;                   // global latent block (16 latents)
          const int cq = 2 * (mbg & 3) + cch;
          bf16x4 v[2];
#pragma unroll
          for (int ins = 0; ins < 2; ++ins) {
            const int t = 16 * ins + tr_tok;
            const unsigned char* p = sbuf + (mbg >> 2) * CG_BYTES + t * 128 + ((cq ^ sw_tr) << 4) + half8;
            v[ins] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4*)((__attribute__((address_space(3))) unsigned char*)p));
          }
          return __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
        };
        bf16x8 va = rd_v(0);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
          const bf16x8 cur = va;
          if (mb + 1 < 8) va = rd_v(mb + 1);
#pragma unroll
          for (int hb = 0; hb < 8; ++hb) pv_mfma(o[mb][hb], cur, pall[hb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // ------------ did any row of the workgroup outgrow its reference?
      const bool wover = __builtin_amdgcn_ballot_w64(over) != 0;
      if (lane == 0) sm->flag[wave] = wover;
      __syncthreads();
      const bool redo = (sm->flag[0] | sm->flag[1] | sm->flag[2] | sm->flag[3]) != 0;
      __syncthreads();
      if (!redo) break;
      m_ref[0] = m_max[0];
      m_ref[1] = m_max[1];
    }
    pv_mfma_drain();
    // ---------------- write the partial of this segment (unnormalised; see mla.h)
    if (active) {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        float l_tot = l_run[hb] + __shfl_xor(l_run[hb], 16, 64);
        l_tot += __shfl_xor(l_tot, 32, 64);
        if (g4 == 0) {
          const int r = row0 + 16 * hb + l16;
          float2 rl;
          rl.x = l_tot > 0.f ? m_ref[hb] * kLn2 : 0.f;
          rl.y = l_tot > 0.f ? (m_ref[hb] + __log2f(l_tot)) * kLn2 : -INFINITY;
          reinterpret_cast<float2*>(a.lse_part)[(int64_t)slot * rows + r] = rl;
        }
      }
    }
#pragma unroll
    for (int hb = 0; hb < 8; ++hb) {
      const int r = grow0 + 16 * hb + l16;
      if (r < rows) {
        float* up = a.u_part + ((int64_t)slot * rows + r) * DC + 128 * wave + 4 * g4;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) *reinterpret_cast<f32x4*>(up + 16 * mb) = o[mb][hb];
      }
    }
    __syncthreads();   // all waves done with the ring and the exchange buffers
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
