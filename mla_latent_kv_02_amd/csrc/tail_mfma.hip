// Value up-projection o_i = u_i W_i^UV ([Huny] = "Multi-Head Latent
// Attention(MLA) 아키텍처 해부", Huny's Dev Blog, §3.2) for bf16 weights, with u
// either given (mla_out_proj) or merged on the fly from the split-KV partials
// (mla_combine_out_proj): u = sum_k exp(r_k - L) u_k, L = log sum_k exp(lse_k)
// over the partials k of a query row -- the softmax over the union of the
// partials' token ranges ([Ikmyung] §1.4).  The merged u is never written.
//
// Workgroup = (head i, NTEAM blocks of up to 32 query rows; fewer when the
// batch is small, so that the workgroups cover the CUs), all d_v = 128 value
// columns, NTEAM teams of 4 waves.  Team t takes row block t; wave w of a
// team owns the contraction slice d_c*w/4 .. d_c*(w+1)/4 (<= 128 latents):
//   1. W_i^UV is staged in LDS once for all teams (global->LDS loads, 16-byte
//      chunks xor-swizzled by row so that transposed reads hit distinct
//      banks), and the plan walk (the slots of the rows' partials) is done
//      once for the workgroup's rows;
//   2. each lane builds its row's slice of u in fp32 registers (64 values per
//      lane: row lane%32, latents 16*ks + 8*(lane/32) + 0..7), reading every
//      partial element once, all 16 loads of one partial in flight together;
//   3. u is split into a bf16 high part and a bf16 residual (u = hi + lo to
//      ~2^-16 relative) and both are multiplied with MFMA 32x32x16 against
//      W^UV read transposed from LDS (ds_read_b64_tr_b16), fp32 accumulation;
//   4. the four waves' partial products of a team are summed through LDS.
// One team (4 waves, one per SIMD) keeps two partials in flight per lane.
// Batches that would need more than one round of such workgroups over the
// 256 CUs (more than 64 rows at 128 heads) take two teams: the W^UV staging
// and the plan walk are shared by twice the rows, and the rounds halve; two
// waves then share each SIMD, so a lane keeps one partial in flight (the
// registers of a second do not fit), and the teams keep in step at the
// workgroup barriers.

#include "mla_device.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int TR = 32;            // query rows of the MFMA tile (M), and the most a team takes
constexpr int TDV = 128;          // value columns (4 MFMA column blocks of 32)
constexpr int TKW = 128;          // contraction rows per wave (d_c / 4)
constexpr int TKS = TKW / 16;     // MFMA k-steps per wave
constexpr int TROWB = TDV * 2;    // bytes of one W^UV row

template <int NTEAM>
struct __attribute__((aligned(16))) TailSmem {
  union {
    unsigned char w[4][TKW * TROWB];   // 4 x 32 KiB: the W^UV rows of each contraction slice
    float red[NTEAM][4][4][16][64];    // 64 KiB per team: each wave's [col block][acc reg][lane]
  };
  int32_t slot0[NTEAM * TR];           // the workgroup's sequences (at most NTEAM * R of them)
  int32_t nparts[NTEAM * TR];
  PlanScratch<256 * NTEAM> plan;
};
static_assert(sizeof(TailSmem<2>) <= 160 * 1024, "LDS budget");

// chunk xor of W^UV row r: a transposed read covers 4 consecutive rows x 4
// chunks (one aligned group of 4); the xor by 4(r%4) gives each row its own group
__device__ __forceinline__ int wswz(int r) { return 4 * (r & 3); }

template <bool PARTIALS, int NTEAM>
__global__ __launch_bounds__(256 * NTEAM, 1) void tail_kernel(TailParams p, int items_pad, int rows_per_block) {
  constexpr int NT = 256 * NTEAM;
  __shared__ TailSmem<NTEAM> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int team = wave8 >> 2;               // row block of the workgroup
  const int wave = wave8 & 3;                // contraction slice
  const int M = p.B * p.n_q;
  const int R = rows_per_block;              // rows per team, a power of two <= TR
  const int rblocks = (M + NTEAM * R - 1) / (NTEAM * R);
  // block -> (head, pair of row blocks); consecutive items on one XCD (block b
  // runs on XCD b % 8), so the row blocks of a head share its weights in L2
  const int item = (blockIdx.x & 7) * (items_pad / 8) + (blockIdx.x >> 3);
  if (item >= p.n_h * rblocks) return;
  const int ih = item / rblocks;
  const int mw0 = (item % rblocks) * NTEAM * R;   // first row of the workgroup
  const int m0 = mw0 + team * R;                  // first row of this team
  const int k0 = wave * TKW;                 // first latent of this wave's slice
  // the sequence lengths for the plan, loaded ahead of the weights
  const int len_tid = PARTIALS && (int)threadIdx.x < p.B ? p.ctx_lens[threadIdx.x] : 0;

  // ---- 1. W^UV rows of slice `wave` into LDS, 4 rows of 256 B per
  // instruction: team t stages rows (128/NTEAM) t .. (128/NTEAM)(t+1) - 1 of the slice
  {
    const unsigned char* src = static_cast<const unsigned char*>(p.w_uv) + ((int64_t)ih * p.d_c + k0) * TROWB;
    unsigned char* dst = sm.w[wave];
    const int rr = lane >> 4, pos = lane & 15;
#pragma unroll 4
    for (int i = 0; i < TKW / 4 / NTEAM; ++i) {
      const int it = team * (TKW / 4 / NTEAM) + i;
      const int r = 4 * it + rr;
      __builtin_amdgcn_global_load_lds(src + r * TROWB + ((pos ^ wswz(r)) << 4), (lds_void*)(dst + it * 1024),
                                       16, 0, 0);
    }
  }

  // ---- 2. this lane's query row and its slice of u.  A block with fewer than
  // 32 rows gives each row rep = 32/P lanes (P = rows rounded up to a power of
  // two): replica j of a row takes the partials k = j, j+rep, ... and the
  // replicas are summed with lane exchanges before the MFMAs (rows past the
  // block end carry copies that are never stored).
  const int rows_here = (M - m0) < R ? (M - m0) : R;   // <= 0: a team past the batch end
  int prow2 = 1;
  while (prow2 < rows_here) prow2 <<= 1;
  const int rep = PARTIALS ? TR / prow2 : 1;
  const int r = PARTIALS ? (lane & 31) % prow2 : (lane & 31);
  const int replica = PARTIALS ? (lane & 31) / prow2 : 0;
  const int hk = lane >> 5;
  const int m = m0 + r;
  const bool mvalid = m < M;
  float L = 0.f;
  int slot0 = 0, np = 1;
  const int b_lo = mw0 / p.n_q;            // the workgroup's first sequence
  if (PARTIALS) {
    const int b_hi = ((M < mw0 + NTEAM * R ? M : mw0 + NTEAM * R) - 1) / p.n_q;
    plan_slot_range<NT>(p.ctx_lens, p.B, p.num_splits, b_lo, b_hi - b_lo + 1, len_tid, &sm.plan, sm.slot0,
                        sm.nparts);
  }
  const int b = mvalid ? m / p.n_q : b_lo;
  const int jq = mvalid ? m % p.n_q : 0;
  const int64_t rows_per_slot = (int64_t)p.n_q * p.n_h;
  const int64_t rowid = (int64_t)jq * p.n_h + ih;
  if (PARTIALS) {
    slot0 = sm.slot0[b - b_lo];
    np = mvalid ? sm.nparts[b - b_lo] : 0;
  }
  f32x4 u[2 * TKS];
#pragma unroll
  for (int e = 0; e < 2 * TKS; ++e) u[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (PARTIALS) {
    // One pass over the partials with a running maximum mx of their lse:
    //   acc = sum_k exp(r_k - mx) u_k,  s = sum_k exp(lse_k - mx),
    // rescaled whenever mx grows; then L = mx + log s and u = acc / s.  Every
    // r_k <= lse_k, so no weight exceeds 1.
    const float2* lp = reinterpret_cast<const float2*>(p.lse_part);
    // this lane's partials: k = replica + j*rep, j = 0 .. nj-1, one in flight
    // per lane (two waves share a SIMD, so a CU still has 8 waves' loads in
    // flight); partial j+1 is fetched as soon as partial j is merged.
    const int nj = replica < np ? (np - replica + rep - 1) / rep : 0;
    // (one team: partial j is fetched into buffer j%2 while partial j-1 is
    // merged; the loads of a fetch are unconditional, a lane past its last
    // partial re-reading row 0 and ignoring it, so every wait is for exactly
    // the older buffer)
    auto fetch = [&](int j, f32x4* v, float2& rl) {
      const int64_t prow = j < nj ? (int64_t)(slot0 + replica + j * rep) * rows_per_slot + rowid : 0;
      rl = lp[prow];
      const f32x4* src = reinterpret_cast<const f32x4*>(p.u_part + prow * p.d_c + k0 + 8 * hk);
#pragma unroll
      for (int ks = 0; ks < TKS; ++ks) {
        v[2 * ks] = src[4 * ks];
        v[2 * ks + 1] = src[4 * ks + 1];
      }
    };
    float mx = -INFINITY, sum = 0.f;
    // branch-free, so that u keeps its registers through the loop: a partial
    // past the lane's last one, or with no visible token, gets weight 0 and
    // leaves mx (and the scale 1) unchanged
    auto merge = [&](int j, const f32x4* v, float2 rl) {
      const bool ok = j < nj && rl.y != -INFINITY;
      const float nm = ok ? fmaxf(mx, rl.y) : mx;
      const float sc = nm == mx ? 1.f : __expf(mx - nm);   // 0 while mx is -inf
      const float wk = ok ? __expf(rl.x - nm) : 0.f;
      sum = sum * sc + (ok ? __expf(rl.y - nm) : 0.f);
#pragma unroll
      for (int e = 0; e < 2 * TKS; ++e) u[e] = u[e] * sc + wk * v[e];
      mx = nm;
    };
    if constexpr (NTEAM == 1) {
      f32x4 va[2 * TKS], vb[2 * TKS];
      float2 ra, rb;
      fetch(0, va, ra);
      fetch(1, vb, rb);
      int j = 0;
      for (; j + 2 < nj; j += 2) {
        merge(j, va, ra);
        fetch(j + 2, va, ra);
        merge(j + 1, vb, rb);
        fetch(j + 3, vb, rb);
      }
      merge(j, va, ra);
      merge(j + 1, vb, rb);
    } else {
      f32x4 va[2 * TKS];
      float2 ra;
      fetch(0, va, ra);
      for (int j = 0; j < nj; ++j) {
        merge(j, va, ra);
        // (keeps the next loads behind the merge: one buffer's worth of registers)
        __builtin_amdgcn_sched_barrier(0);
        if (j + 1 < nj) fetch(j + 1, va, ra);
      }
    }
    // merge the replicas of the row (lanes xor prow2, 2*prow2, ... within the half)
    for (int sh = prow2; sh < TR; sh <<= 1) {
      const float mo = __shfl_xor(mx, sh, 64);
      const float mn = fmaxf(mx, mo);
      const float sc = mn == -INFINITY ? 0.f : __expf(mx - mn);
      sum *= sc;
#pragma unroll
      for (int e = 0; e < 2 * TKS; ++e) u[e] *= sc;
      sum += __shfl_xor(sum, sh, 64);
#pragma unroll
      for (int e = 0; e < 2 * TKS; ++e)
#pragma unroll
        for (int c = 0; c < 4; ++c) u[e][c] += __shfl_xor(u[e][c], sh, 64);
      mx = mn;
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
#pragma unroll
    for (int e = 0; e < 2 * TKS; ++e) u[e] *= inv;
    L = sum > 0.f ? mx + __logf(sum) : -INFINITY;
  } else if (mvalid) {
    const f32x4* src = reinterpret_cast<const f32x4*>(p.u + ((int64_t)m * p.n_h + ih) * p.d_c + k0 + 8 * hk);
#pragma unroll
    for (int ks = 0; ks < TKS; ++ks) {
      u[2 * ks] = src[4 * ks];
      u[2 * ks + 1] = src[4 * ks + 1];
    }
  }

  // ---- 3. MFMA: acc[nb] (rows x value columns 32nb..32nb+31) += u_slice . W^UV_slice
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's staged W^UV rows have landed
  if constexpr (NTEAM > 1) __syncthreads();   // and the other teams' parts of the slice
  const int g4 = lane >> 4, j = lane & 15;
  f32x16 acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x16{};
  const unsigned char* wl = sm.w[wave];
#pragma unroll
  for (int ks = 0; ks < TKS; ++ks) {
    u16x8 hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = e < 4 ? u[2 * ks][e] : u[2 * ks + 1][e - 4];
      const uint16_t h = f32_to_bf16(x);
      hi[e] = h;
      lo[e] = f32_to_bf16(x - bf16_to_f32(h));
    }
    const bf16x8 ahi = __builtin_bit_cast(bf16x8, hi), alo = __builtin_bit_cast(bf16x8, lo);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      // B operand: lane -> value column 32nb + 16(g4&1) + j, latents 16ks + 8(g4>>1) + 0..7
      bf16x4 bv[2];
#pragma unroll
      for (int ins = 0; ins < 2; ++ins) {
        const int kr = 16 * ks + 8 * (g4 >> 1) + 4 * ins + (j >> 2);
        const int chunk = 4 * nb + 2 * (g4 & 1) + ((j & 3) >> 1);
        const unsigned char* ptr = wl + kr * TROWB + ((chunk ^ wswz(kr)) << 4) + (j & 1) * 8;
        bv[ins] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)((__attribute__((address_space(3))) unsigned char*)ptr));
      }
      const bf16x8 bw = __builtin_shufflevector(bv[0], bv[1], 0, 1, 2, 3, 4, 5, 6, 7);
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi, bw, acc[nb], 0, 0, 0);
      acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo, bw, acc[nb], 0, 0, 0);
    }
  }

  // ---- 4. sum the team's four products; acc[nb][i] = o[row 8(i/4) + 4(lane/32) + i%4][32nb + lane%32]
  __syncthreads();   // every wave is done with the W^UV rows (the buffer is reused)
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int i = 0; i < 16; ++i) sm.red[team][wave][nb][i][lane] = acc[nb][i];
  __syncthreads();
  const int ttid = tid & (NT / NTEAM - 1);   // thread within the team
  const auto& red = sm.red[team];
#pragma unroll 4
  for (int q = 0; q < 16; ++q) {
    const int idx = q * (NT / NTEAM) + ttid;
    const int nb = idx >> 10, i = (idx >> 6) & 15, l = idx & 63;
    const float v = red[0][nb][i][l] + red[1][nb][i][l] + red[2][nb][i][l] + red[3][nb][i][l];
    const int rr = 8 * (i >> 2) + 4 * (l >> 5) + (i & 3);   // MFMA row = the lane of the A operand
    const int mm = m0 + rr;
    if (rr < rows_here) p.out[((int64_t)mm * p.n_h + ih) * TDV + 32 * nb + (l & 31)] = v;
  }
  if (PARTIALS && p.lse && wave == 0 && hk == 0 && replica == 0 && mvalid) p.lse[(int64_t)m * p.n_h + ih] = L;
}

}  // namespace

bool tail_mfma_ok(int d_c, int d_v, bool bf16_weights) {
  return bf16_weights && d_c == 4 * TKW && d_v == TDV;
}

hipError_t launch_tail_mfma(const TailParams& p, bool from_partials, hipStream_t stream) {
  const int M = p.B * p.n_q;
  // Two teams when one-team workgroups of 32 rows would take more than one
  // round over the 256 CUs.  Blocks of fewer rows when the batch is small, so
  // that the workgroups cover the CUs (the spare lanes of a block take shares
  // of its rows' partials, as replicas).  A workgroup takes nteam blocks of R rows.
  const int nteam = (int64_t)p.n_h * ((M + TR - 1) / TR) > 256 ? 2 : 1;
  int R = TR;
  while (R > 1 && (int64_t)p.n_h * ((M + nteam * R - 1) / (nteam * R)) < 256) R >>= 1;
  const int items = p.n_h * ((M + nteam * R - 1) / (nteam * R));
  const int items_pad = (items + 7) / 8 * 8;
  const dim3 grid(items_pad), block(256 * nteam);
  if (from_partials && nteam == 2)
    hipLaunchKernelGGL((tail_kernel<true, 2>), grid, block, 0, stream, p, items_pad, R);
  else if (from_partials)
    hipLaunchKernelGGL((tail_kernel<true, 1>), grid, block, 0, stream, p, items_pad, R);
  else if (nteam == 2)
    hipLaunchKernelGGL((tail_kernel<false, 2>), grid, block, 0, stream, p, items_pad, R);
  else
    hipLaunchKernelGGL((tail_kernel<false, 1>), grid, block, 0, stream, p, items_pad, R);
  return hipGetLastError();
}

}  // namespace mla
