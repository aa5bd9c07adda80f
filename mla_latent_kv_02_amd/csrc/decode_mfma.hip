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
//   S^T[tok][row]  = K_tile[tok][0:576] . [q_lat | q_pe]^T      (MFMA 32x32x16)
//   softmax over tokens, in registers (a lane holds 1 row x 16 tokens)
//   O^T[lat][row] += V_tile^T[lat][tok] . P^T[tok][row]          (MFMA 32x32x16)
// (32x32x16 is the full-rate bf16 MFMA shape on gfx950; 16x16x32 issues at
// half the rate.)
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
constexpr int KSTEPS = ROW / 16;      // 36 MFMA k-steps (32x32x16) for QK^T
constexpr int CGROUPS = ROW / 64;     // 9 chunk groups of 8 chunks
constexpr int CG_BYTES = T * 128;     // one chunk group of a stage: 32 tokens x 128 B
constexpr int STAGE_BYTES = CGROUPS * CG_BYTES;   // 36864
constexpr int LOADS_PER_STAGE = CGROUPS;          // 16-byte-per-lane loads per wave per stage
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
  bf16x8 pbuf[4][2][64];     // softmax weights of the stage: [head block][k-step][lane], B-operand layout
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

// O += A . B for one 32x32 block of the PV product, with the accumulator pinned
// to AGPRs.  O needs all 256 AGPRs; the QK^T accumulators (built-in MFMAs,
// compiled in the VGPR form) stay in VGPRs, so the allocator never moves O
// blocks between register files inside the stage loop.
__device__ __forceinline__ void pv_mfma(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
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
//     registers as the MFMA B operand); per stage it computes one 32-token x
//     32-row block S^T with 32x32x16 MFMAs (two accumulation chains over
//     alternate k-steps).  Lane l holds row l%32 and tokens
//     8*(i/4) + 4*(l/32) + i%4 (i < 16) of the block.
//   PV: wave w owns latent columns 128w .. 128w+127 for all 128 rows (4 x 4
//     blocks of 32x32), so each V element is read from LDS once per workgroup.
//     The k index of the PV MFMA is mapped to tokens so that a lane's own
//     softmax weights are its B operand (k = 8*(l/32) + e <-> token
//     16q + 8*(e/4) + 4*(l/32) + e%4 for k-step q), and V^T is read with the
//     same token order by transposed 4x16 LDS reads.  The weights of all rows
//     pass through LDS as 16-byte copies.
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
  const int h = lane >> 5;          // lane half
  const int l32 = lane & 31;
  const int g4 = lane >> 4;         // lane group of 16 (transposed reads)
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
    // ---- query operand (B of QK^T): row row0 + l32, k = 16*ks + 8*h .. +8
    bf16x8 qreg[KSTEPS];
    int limit = t1;
    if (active) {
      const int64_t qrow = (int64_t)b * rows + row0 + l32;
      const u16x8* ql = reinterpret_cast<const u16x8*>(a.q_lat + qrow * DC);
      const u16x8* qp = reinterpret_cast<const u16x8*>(a.q_pe + qrow * DR);
#pragma unroll
      for (int ks = 0; ks < DC / 16; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8, ql[2 * ks + h]);
#pragma unroll
      for (int ks = DC / 16; ks < KSTEPS; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8, qp[2 * (ks - DC / 16) + h]);
      const int qpos = a.positions[(int64_t)b * a.n_q + jq];
      limit = qpos + 1 < t1 ? qpos + 1 : t1;
    }
    // the query operands must not be waited for inside the stage loop, where the
    // vector-memory counter also covers the stage loads
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    // per-lane LDS byte offsets that do not depend on the stage
    const int sw_qk = swz(l32 & 7);
    int qk_off[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) qk_off[r] = l32 * 128 + (((2 * r + h) ^ sw_qk) << 4);
    const int hq = g4 >> 1;                              // k half of this lane's transposed read
    const int tr_tok = 4 * hq + (l16 >> 2);              // token (mod 8) of this lane's row
    const int sw_tr = swz(tr_tok);
    const int half8 = (l16 & 1) * 8;
    const int cch = 2 * (g4 & 1) + ((l16 & 3) >> 1);     // chunk within a group of 4
    const int nst = (t1 - t0 + T - 1) / T;

    // m_ref: reference (log2 units) of the lane's QK row; m_max: running maximum
    float m_ref = -INFINITY, m_max = -INFINITY;
    float l_run;
    // O^T accumulators of this wave: latent block mb (32 latents at 128*wave + 32*mb)
    // x head block hb (rows grow0 + 32*hb .. +32)
    f32x16 o[4][4];
    // K operand of QK^T for k-step ks from a stage buffer
    auto rd_k = [&](const unsigned char* sb, int ks) -> bf16x8 {
      const unsigned char* p = sb + (ks >> 2) * CG_BYTES + qk_off[ks & 3];
      return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(
          (const __attribute__((address_space(3))) unsigned char*)p);
    };
    // V^T operand of PV for k-step q and latent block mb (32 latents of this wave)
    auto rd_v = [&](const unsigned char* sb, int q, int mb) -> bf16x8 {
      const int mbg = 4 * wave + mb;                   // global latent block (32 latents)
      const int cq = 4 * (mbg & 1) + cch;
      bf16x4 v[2];
#pragma unroll
      for (int ins = 0; ins < 2; ++ins) {
        const int t = 16 * q + 8 * ins + tr_tok;
        const unsigned char* p = sb + (mbg >> 1) * CG_BYTES + t * 128 + ((cq ^ sw_tr) << 4) + half8;
        v[ins] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)((__attribute__((address_space(3))) unsigned char*)p));
      }
      return __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
    };
    constexpr int PF = 2;

    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) o[mb][hb] = f32x16{};
      l_run = 0.f;
      bool over = false;
#pragma unroll
      for (int s = 0; s < NSTAGE - 1; ++s)
        if (s < nst) load_stage(a, b, t0 + s * T, t1, sm->stage[s], wave, lane);

      // Software pipeline: iteration it computes S^T of stage it+1 (MFMA) while
      // it turns the scores of stage it into weights (VALU), then accumulates
      // PV of stage it.  Stage it+3 is loaded into the slot stage it-1 freed.
      // s_cur: scores of the stage whose weights come next (two MFMA chains summed).
      f32x16 s_cur = f32x16{};
      // S^T of one stage into s_cur (no overlap; pipeline fill and edges)
      auto qk_plain = [&](const unsigned char* sb) {
        f32x16 c0 = f32x16{}, c1 = f32x16{};
        bf16x8 kring[PF];
#pragma unroll
        for (int ks = 0; ks < PF; ++ks) kring[ks] = rd_k(sb, ks);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          const bf16x8 kk = kring[ks % PF];
          if (ks + PF < KSTEPS) kring[ks % PF] = rd_k(sb, ks + PF);
          if (ks & 1) c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, qreg[ks], c1, 0, 0, 0);
          else c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, qreg[ks], c0, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        s_cur = c0 + c1;
      };
      // softmax pieces on s_cur for stage tokens tok0..: scale + mask, row max, weights
      auto sm_scale_mask = [&](int tok0, float* x, float& mt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int tok = tok0 + 8 * (i >> 2) + 4 * h + (i & 3);
          const float v = s_cur[i] * a.scale_log2;
          x[i] = tok < limit ? v : -INFINITY;
          mt = fmaxf(mt, x[i]);
        }
      };
      auto sm_rowmax = [&](float& mt, bool& ov) {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
        mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        m_max = fmaxf(m_max, mt);
        if (m_ref == -INFINITY) m_ref = mt;       // first visible stage of the row
        ov |= mt > m_ref + REF_HEADROOM;
      };
      auto sm_weights = [&](const float* x, int q, bf16x8* pb, float& psum) {
        const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = __builtin_amdgcn_exp2f(x[8 * q + e] - m_use);
          psum += p;
          pb[q][e] = (__bf16)p;
        }
      };

      wait_stages_in_flight(nst - 1 < NSTAGE - 2 ? nst - 1 : NSTAGE - 2);
      lds_barrier();
      if (active && t0 < limit) qk_plain(sm->stage[0]);

      for (int it = 0; it < nst; ++it) {
        const bool has_next = it + 1 < nst;
        if (has_next) wait_stages_in_flight(it + 2 < nst ? 1 : 0);   // stage it+1 resident
        lds_barrier();
        if (it + NSTAGE - 1 < nst)
          load_stage(a, b, t0 + (it + NSTAGE - 1) * T, t1, sm->stage[(it + NSTAGE - 1) % NSTAGE], wave, lane);
        const int tok0 = t0 + it * T;
        const bool qk_now = active && tok0 < limit;                     // weights of stage it
        const bool qk_next = active && has_next && tok0 + T < limit;    // scores of stage it+1
        const unsigned char* sb_next = sm->stage[(it + 1) % NSTAGE];
        bf16x8 pb[2] = {bf16x8{}, bf16x8{}};
        float x[16];
        float psum = 0.f, mt = -INFINITY;
        if (qk_now && qk_next) {
          // ------------ S^T(it+1) by MFMA, interleaved with the softmax of stage it
          f32x16 c0 = f32x16{}, c1 = f32x16{};
          bf16x8 kring[PF];
#pragma unroll
          for (int ks = 0; ks < PF; ++ks) kring[ks] = rd_k(sb_next, ks);
#pragma unroll
          for (int ks = 0; ks < KSTEPS; ++ks) {
            const bf16x8 kk = kring[ks % PF];
            if (ks + PF < KSTEPS) kring[ks % PF] = rd_k(sb_next, ks + PF);
            if (ks & 1) c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, qreg[ks], c1, 0, 0, 0);
            else c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, qreg[ks], c0, 0, 0, 0);
            if (ks == 1) sm_scale_mask(tok0, x, mt);
            if (ks == 4) sm_rowmax(mt, over);
            if (ks == 7) sm_weights(x, 0, pb, psum);
            if (ks == 10) sm_weights(x, 1, pb, psum);
            __builtin_amdgcn_sched_barrier(0);
          }
          s_cur = c0 + c1;
        } else {
          if (qk_now) {
            sm_scale_mask(tok0, x, mt);
            sm_rowmax(mt, over);
            sm_weights(x, 0, pb, psum);
            sm_weights(x, 1, pb, psum);
          }
          if (qk_next) qk_plain(sb_next);
        }
        l_run += psum;
        // ------------ publish this wave's weights (B-operand layout, per k-step)
        sm->pbuf[wave][0][lane] = pb[0];
        sm->pbuf[wave][1][lane] = pb[1];
        lds_barrier();
        // ------------ O^T[own 128 latents][128 rows] += V^T . P^T for stage it
        const unsigned char* sb = sm->stage[it % NSTAGE];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          bf16x8 pq[4];
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) pq[hb] = sm->pbuf[hb][q][lane];
          bf16x8 va = rd_v(sb, q, 0);
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) {
            const bf16x8 cur = va;
            if (mb + 1 < 4) va = rd_v(sb, q, mb + 1);
#pragma unroll
            for (int hb = 0; hb < 4; ++hb) pv_mfma(o[mb][hb], cur, pq[hb]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      // ------------ did any row of the workgroup outgrow its reference?
      const bool wover = __builtin_amdgcn_ballot_w64(over) != 0;
      if (lane == 0) sm->flag[wave] = wover;
      __syncthreads();
      const bool redo = (sm->flag[0] | sm->flag[1] | sm->flag[2] | sm->flag[3]) != 0;
      __syncthreads();
      if (!redo) break;
      m_ref = m_max;
    }
    pv_mfma_drain();
    // ---------------- write the partial of this segment (unnormalised; see mla.h)
    if (active) {
      const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
      if (h == 0) {
        const int r = row0 + l32;
        float2 rl;
        rl.x = l_tot > 0.f ? m_ref * kLn2 : 0.f;
        rl.y = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
        reinterpret_cast<float2*>(a.lse_part)[(int64_t)slot * rows + r] = rl;
      }
    }
    // o[mb][hb][i] = u[row grow0 + 32 hb + l32][latent 128 wave + 32 mb + 8 (i/4) + 4 h + i%4]
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int r = grow0 + 32 * hb + l32;
      if (r < rows) {
        float* up = a.u_part + ((int64_t)slot * rows + r) * DC + 128 * wave + 4 * h;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4)
            *reinterpret_cast<f32x4*>(up + 32 * mb + 8 * i4) =
                f32x4{o[mb][hb][4 * i4], o[mb][hb][4 * i4 + 1], o[mb][hb][4 * i4 + 2], o[mb][hb][4 * i4 + 3]};
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
