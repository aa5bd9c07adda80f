// Prefill (and chunked prefill) of MLA attention: many query tokens per
// sequence, keys and values rebuilt per head from the cached latents.
//
// Method ([Huny] = "Multi-Head Latent Attention(MLA) 아키텍처 해부", Huny's Dev
// Blog, §1: k^C_i = c W_i^UK, v_i = c W_i^UV; §2.2: the key of head i is
// [k^C_i | k^R] with the shared rotated positional key; [Tbr8] = "DeepSeek
// MLA（多头潜在注意力）深度解析", tbr8.org, §5.2: prefill is compute-bound, so
// the up-projections cost little there, while absorption pays at decode):
//   kv[t][i] = [c_t W_i^UK | c_t W_i^UV]                 (reconstruct_gemm)
//   o_j,i    = softmax_{t <= pos_j}(q_j,i . [kv[t][i][:128] | k^R_t] * scale) kv[t][i][128:]
//                                                      (prefill_attn_kernel)
// Absorbing W^UK into the query costs 2(d_c + d_rope) + 2 d_c = 2176 FLOPs per
// (query, token, head) against 2(d_nope + d_rope) + 2 d_v = 640 here; the
// reconstruction adds 2 d_c (d_nope + d_v) n_h FLOPs per cached token once per
// call, which a chunk of many queries amortises.
//
// V3 head shapes only: d_nope = d_v = 128, d_rope = 64, bf16 operands, fp32
// accumulation.

#include <climits>

#include "mla_device.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int NT = 256;
constexpr int DN = 128, DV = 128, DR = 64;
constexpr int KVW = DN + DV;             // elements of one head's reconstructed row
constexpr int kBufferWord3 = 0x00020000; // raw buffer resource, 32-bit data format, byte offsets

// s(t) = P[(t / 2) % 8], P = (0, 4, 1, 5, 2, 6, 3, 7): 16-byte chunk c of LDS row t
// sits at slot c ^ s(t), so that 16 consecutive rows read at one chunk hit
// 16 distinct bank groups (two row parities x 8 slot values).
__device__ __forceinline__ int swz(int t) { return (0x73625140 >> (4 * ((t >> 1) & 7))) & 7; }

typedef __attribute__((address_space(3))) const bf16x8 lds_cbf16x8;
__device__ __forceinline__ bf16x8 lds_read16(const unsigned char* p) {
  return *(lds_cbf16x8*)((__attribute__((address_space(3))) const unsigned char*)p);
}

// ------------------------------------------------------------ weight layout
// w_kv[i][d][c] = W_i^UK[c][d] (d < 128), W_i^UV[c][d - 128] (d >= 128): the
// latent index innermost, the operand layout of the reconstruction product.
__global__ __launch_bounds__(NT) void prefill_weights_kernel(const uint16_t* __restrict__ w_uk,
                                                             const uint16_t* __restrict__ w_uv,
                                                             uint16_t* __restrict__ w_kv, int d_c) {
  __shared__ uint16_t tile[32][33];
  const int i = blockIdx.z;
  const int c0 = blockIdx.x * 32, d0 = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  const uint16_t* src = d0 < DN ? w_uk + (int64_t)i * d_c * DN : w_uv + (int64_t)i * d_c * DV;
  const int dd = d0 < DN ? d0 : d0 - DN;
  for (int r = ty; r < 32; r += 8) tile[r][tx] = src[(int64_t)(c0 + r) * DN + dd + tx];   // [c][d]
  lds_sync();
  for (int r = ty; r < 32; r += 8) w_kv[((int64_t)i * KVW + d0 + r) * d_c + c0 + tx] = tile[tx][r];
}

// ------------------------------------------------------- reconstruction
// kv[z][m][n] = sum_c A[z][m][c] w_kv[n][c] with A the cached latents of
// sequence z (rows m < M of the cache, the first d_c elements of each row) and
// n = i * 256 + d over all heads.  Workgroup tile 128 (m) x 256 (n), 4 waves;
// wave w takes m rows 64(w%2) .. +64 and n rows 128(w/2) .. +128 (2 x 4
// blocks of 32 x 32).  The weight rows are the MFMA's first operand.  The k
// range is streamed in chunks of 32 through a 3-stage LDS ring (72 KiB, so two
// workgroups share a CU and one's barrier waits are covered by the other's
// MFMAs): row r of a stage holds 4 chunks of 16 bytes, chunk c at slot
// c ^ ((r / 4) % 4), which spreads 16 consecutive rows read at one chunk over
// all 64 banks; a wave's 16-byte global->LDS load writes 16 rows x 64 bytes.
// (A 256 x 256 tile with 8 waves, one workgroup per CU, needs a third fewer
// L2 reads but measured slower.)
constexpr int GM = 128, GN = 256, GK = 32, GSTAGES = 3, GWAVES = (GM / 64) * (GN / 128), GNT = 64 * GWAVES;
constexpr int GWG_PER_CU = 2;
static_assert(GSTAGES == 3 || GSTAGES == 4, "the stage-top waits cover 3 or 4 stages");
constexpr int GROW = GK * 2;                                    // LDS row: 64 bytes
constexpr int GA_BYTES = GM * GROW, GB_BYTES = GN * GROW;       // 8 KiB, 16 KiB
constexpr int G_LOADS = (GM + GN) / 16 / GWAVES;                // 1 KiB loads per wave per stage: 6
__device__ __forceinline__ int gswz(int r) { return (r >> 2) & 3; }

struct GemmArgs {
  const unsigned char* a;   // cache data (bf16 rows)
  int64_t a_seq_bytes;      // bytes between sequences
  int a_row_bytes;          // bytes between rows
  const uint16_t* w;        // w_kv [N][K]
  uint16_t* c;              // kv [Z][M][N]
  int M, N, K;
  int mb, nb, tiles, tiles_per_xcd;   // tile grid: mb x nb per sequence, Z * mb * nb in all
};

// Tile order.  Workgroups are dealt to the 8 XCDs in turn, so XCD x gets
// blockIdx x, x+8, ...; it is given the consecutive tiles x*T .. x*T+T-1 of
// the order below, in which G_GROUP_M consecutive m blocks sweep the n blocks
// together (tile i of a group: m = first + i % G_GROUP_M, n = i / G_GROUP_M;
// measured on chunk1k: groups of 4 m blocks 3.76 ms a call, 8: 3.80, 16: 3.82,
// 64: 3.92, no grouping: 4.08).  The tiles an XCD runs at one time then share
// their A rows and weight rows in its L2.
constexpr int G_GROUP_M = 4;
__device__ __forceinline__ bool gemm_tile(const GemmArgs& g, int bid, int* z, int* mi, int* ni) {
  const int t = (bid & 7) * g.tiles_per_xcd + (bid >> 3);
  if (t >= g.tiles) return false;
  const int per_z = g.mb * g.nb;
  *z = t / per_z;
  const int r = t - *z * per_z;
  const int first = (r / (G_GROUP_M * g.nb)) * G_GROUP_M;
  const int gsize = g.mb - first < G_GROUP_M ? g.mb - first : G_GROUP_M;
  const int in = r - first * g.nb;
  *mi = first + in % gsize;
  *ni = in / gsize;
  return true;
}

struct __attribute__((aligned(16))) GemmSmem {
  unsigned char a[GSTAGES][GA_BYTES];
  unsigned char b[GSTAGES][GB_BYTES];
};
static_assert(GWG_PER_CU * sizeof(GemmSmem) <= 160 * 1024, "LDS of one CU");

__global__ __launch_bounds__(GNT, GWG_PER_CU) void reconstruct_gemm_kernel(GemmArgs g) {
  __shared__ GemmSmem sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  int zi, mi, ni;
  if (!gemm_tile(g, blockIdx.x, &zi, &mi, &ni)) return;
  const int m0 = __builtin_amdgcn_readfirstlane(mi * GM), n0 = __builtin_amdgcn_readfirstlane(ni * GN);
  const int64_t z = __builtin_amdgcn_readfirstlane(zi);
  // A rows past M read as zeros (buffer range); their results are not stored
  const unsigned char* abase = g.a + z * g.a_seq_bytes + (int64_t)m0 * g.a_row_bytes;
  const int a_rows = g.M - m0 < GM ? g.M - m0 : GM;
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(abase), (short)0,
                                                                      a_rows * g.a_row_bytes, kBufferWord3);
  const unsigned char* bbase = reinterpret_cast<const unsigned char*>(g.w + (int64_t)n0 * g.K);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(bbase), (short)0,
                                                                      GN * g.K * 2, kBufferWord3);
  // this lane's rows in its loads: A row 16j + lane/4 (j = wave, wave + GWAVES, ..), B likewise
  const int lr = lane >> 2, lp = lane & 3;
  const int nst = g.K / GK;
  auto issue = [&](int s) {
    const int slot = s % GSTAGES;
    const int kb = s * GROW;   // byte offset of the chunk within a row
#pragma unroll
    for (int q = 0; q < GM / 16 / GWAVES; ++q) {   // loads of A rows
      const int j = wave + GWAVES * q;
      const int r = 16 * j + lr;
      const int off = r * g.a_row_bytes + kb + ((lp ^ gswz(r)) << 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(sm.a[slot] + 1024 * j), 16, off, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < GN / 16 / GWAVES; ++q) {   // loads of weight rows
      const int j = wave + GWAVES * q;
      const int r = 16 * j + lr;
      const int off = r * g.K * 2 + kb + ((lp ^ gswz(r)) << 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(sm.b[slot] + 1024 * j), 16, off, 0, 0, 0);
    }
  };
  const int wm = wave % (GM / 64), wn = wave / (GM / 64);
  f32x16 acc[4][2];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = f32x16{};
  // operand rows of this lane and their swizzles
  int boff[4], aoff[2], bsw[4], asw[2];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int r = 128 * wn + 32 * nb + l32;
    boff[nb] = r * GROW;
    bsw[nb] = gswz(r);
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int r = 64 * wm + 32 * mb + l32;
    aoff[mb] = r * GROW;
    asw[mb] = gswz(r);
  }
  static_assert(G_LOADS * (GSTAGES - 2) < 16, "the wait count fits the low vmcnt field");
  for (int s = 0; s < GSTAGES - 1 && s < nst; ++s) issue(s);
  for (int s = 0; s < nst; ++s) {
    // this wave's loads of stage s are in; the barrier (LDS only: the loads of
    // the next stages stay in flight) makes every wave's visible and ends every
    // read of the slot stage s + GSTAGES - 1 reuses
    const int ahead = nst - 1 - s;
    if (ahead >= GSTAGES - 2) __builtin_amdgcn_s_waitcnt(0x0F70 | (G_LOADS * (GSTAGES - 2)));
    else if (GSTAGES > 3 && ahead == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | G_LOADS);
    else __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    lds_sync();
    if (s + GSTAGES - 1 < nst) issue(s + GSTAGES - 1);
    const unsigned char* sa = sm.a[s % GSTAGES];
    const unsigned char* sb = sm.b[s % GSTAGES];
#pragma unroll
    for (int kk = 0; kk < GK / 16; ++kk) {
      const int c = 2 * kk + h;
      bf16x8 bo[4], ao[2];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) bo[nb] = lds_read16(sb + boff[nb] + ((c ^ bsw[nb]) << 4));
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) ao[mb] = lds_read16(sa + aoff[mb] + ((c ^ asw[mb]) << 4));
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          acc[nb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bo[nb], ao[mb], acc[nb][mb], 0, 0, 0);
    }
  }
  // ---- results.  acc[nb][mb][i] is kv at m = m0 + 64 wm + 32 mb + l32,
  // n = n0 + 128 wn + 32 nb + 8 (i/4) + 4 h + i%4.  Stored straight from the
  // registers, a wave's store would touch 32 rows with 16 bytes each; instead
  // each wave puts its 64 x 128 block in the ring's memory (16 KiB, row r at
  // 256 r, 16-byte chunk c at c ^ (r % 16)) and writes it back 4 whole rows
  // (4 x 256 contiguous bytes) per store.
  static_assert(GWAVES * 64 * 256 <= (int)sizeof(GemmSmem), "the output blocks fit in the ring");
  lds_sync();   // every wave is done with the ring
  unsigned char* ob = reinterpret_cast<unsigned char*>(&sm) + 16384 * wave;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int r = 32 * mb + l32;
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = f32_to_bf16(acc[nb][mb][4 * q + e]);
        *reinterpret_cast<u16x4*>(ob + 256 * r + (((4 * nb + q) ^ (r & 15)) << 4) + 8 * h) = v;
      }
  }
  // this wave's block is in (only this wave reads it back; the clobber keeps
  // the reads below the writes)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const int rr = lane >> 4, cc = lane & 15;
  uint16_t* cbase = g.c + (z * g.M + m0 + 64 * wm) * (int64_t)g.N + n0 + 128 * wn + 8 * cc;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int r = 4 * it + rr;
    const u16x8 v = *reinterpret_cast<const u16x8*>(ob + 256 * r + ((cc ^ (r & 15)) << 4));
    if (m0 + 64 * wm + r < g.M) *reinterpret_cast<u16x8*>(cbase + (int64_t)r * g.N) = v;
  }
}

// ------------------------------------------------------------- attention
// One workgroup = 128 query rows (query tokens) of one head of one sequence;
// wave w owns rows 32w .. 32w+31 for the whole computation (no exchange of
// weights between waves).  The cached tokens stream through a 2-slot LDS
// ring of T = 64-token stages; a stage holds 5 chunk groups of 64 rows x 8 chunks
// (16 bytes): the key content part (2 groups, from kv), the positional key
// (1 group, from the cache row) and the value (2 groups, from kv).  Per stage:
//   S^T[tok][row] = K[tok][0:192] . [q_nope | q_pe]^T   (2 blocks of 32 tokens,
//                   two independent chains of 12 MFMA 32x32x16)
//   online softmax per row (running maximum, rescaled accumulator)
//   O^T[dv][row] += V^T[dv][tok] . P^T[tok][row]          (16 MFMA 32x32x16)
// A lane holds row l%32 and 16 tokens of each S^T block; its own weights are
// the B operand of the PV product (the k index of step q maps to tokens
// 16q + 8(e/4) + 4(l/32) + e%4, the order of the S^T layout), and V^T is read
// in the same token order by transposed LDS reads.  Two workgroups share a
// CU (80 KiB of LDS each), so one's softmax runs under the other's MFMAs.
// Stages that every row of a wave sees whole take a loop without masking.
// (Measured: one workgroup per CU with a 3-slot ring, and 32-token stages
// with S^T(s+1) interleaved with the softmax of stage s, were both slower.)
constexpr int T = 64;
constexpr int CG = T * 128;                // bytes of one chunk group (8 KiB)
constexpr int ASTAGE = 5 * CG;             // 40 KiB
constexpr int ANST = 2;                    // ring slots: ANST - 1 stages in flight ahead of use
constexpr int AWG_PER_CU = 2;
constexpr int QK_STEPS = (DN + DR) / 16;   // 12
constexpr float A_HEADROOM = 32.f;         // log2 units a weight's exponent may exceed 0
constexpr int QPF = 2;                     // QK k-steps of K operands read ahead
constexpr int A_LOADS = 10;                // 1 KiB global->LDS loads per wave per stage

struct AttnArgs {
  const uint16_t* q_nope;   // [B][n_q][n_h][128]
  const uint16_t* q_pe;     // [B][n_q][n_h][64]
  const int32_t* positions; // [B][n_q]
  const int32_t* ctx_lens;  // [B]
  const unsigned char* cache;   // bf16 rows of d_c + 64 elements
  int64_t cache_seq_bytes;
  int cache_row_bytes, rope_byte;   // row pitch, byte offset of k^R in a row
  const unsigned char* kv;  // [B][M][n_h][256] bf16
  float* out;               // [B][n_q][n_h][128]
  float* lse;               // [B][n_q][n_h] or null
  int B, n_q, n_h, M, n_qb, units, units_per_xcd;
  float scale_log2;
};

struct __attribute__((aligned(16))) AttnSmem {
  unsigned char stage[ANST][ASTAGE];
};
static_assert(AWG_PER_CU * sizeof(AttnSmem) <= 160 * 1024, "LDS of one CU");
static_assert(ANST == 2 || ANST == 3, "the stage-top wait covers 2 or 3 slots");

// Transposed 8-byte LDS read (4 bf16 of 4 consecutive rows, see the PV
// operand below) at addr + OFF.  Issued as inline asm: with the built-in, the
// compiler puts a wait for every global->LDS load in flight in front of it
// (it cannot tell that those write another stage).  The constant part of the
// address goes in the offset field, so each read costs no address arithmetic.
template <int OFF>
__device__ __forceinline__ bf16x4 lds_read_tr(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "DS offset field");
  bf16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// Byte offset, from a stage's start plus a lane's part, of the V^T read half
// `ins` of PV step q (tokens 16q .. 16q+15) and dv block db (chunk group 3 or 4).
constexpr int pv_off(int q, int db, int ins) { return (3 + (db >> 1)) * CG + (16 * q + 8 * ins) * 128; }
__device__ __forceinline__ bf16x8 cat4(bf16x4 x, bf16x4 y) {
  return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}
// V^T operands of PV step Q (tokens 16Q .. 16Q+15) for the 4 dv blocks
// (va[2 (db%2) + half] = the lane's read addresses); their data is waited for
// by pv_mfmas.
template <int Q>
__device__ __forceinline__ void pv_reads(bf16x8 (&v)[4], const uint32_t (&va)[4]) {
  v[0] = cat4(lds_read_tr<pv_off(Q, 0, 0)>(va[0]), lds_read_tr<pv_off(Q, 0, 1)>(va[1]));
  v[1] = cat4(lds_read_tr<pv_off(Q, 1, 0)>(va[2]), lds_read_tr<pv_off(Q, 1, 1)>(va[3]));
  v[2] = cat4(lds_read_tr<pv_off(Q, 2, 0)>(va[0]), lds_read_tr<pv_off(Q, 2, 1)>(va[1]));
  v[3] = cat4(lds_read_tr<pv_off(Q, 3, 0)>(va[2]), lds_read_tr<pv_off(Q, 3, 1)>(va[3]));
}
// Waits for every LDS read in flight (the operands v among them: the MFMAs
// take them through this statement, so they cannot move ahead of it).
__device__ __forceinline__ void lds_wait_operands(bf16x8 (&v)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
}
// O^T[dv][row] += V^T[dv][16 tokens] . P^T for the 4 dv blocks.
__device__ __forceinline__ void pv_mfmas(f32x16 (&o)[4], const bf16x8 (&v)[4], const bf16x8& p) {
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[db], p, o[db], 0, 0, 0);
}
// PV of one stage: the reads of step Q+1 go out before the MFMAs of step Q,
// so their latency runs under those MFMAs (the reads of step 0 were issued by
// the caller, before the softmax).
template <int Q>
__device__ __forceinline__ void pv_pipeline(f32x16 (&o)[4], bf16x8 (&v)[2][4], const bf16x8 (&p)[4],
                                            const uint32_t (&va)[4]) {
  lds_wait_operands(v[Q % 2]);
  if constexpr (Q + 1 < 4) pv_reads<Q + 1>(v[(Q + 1) % 2], va);
  __builtin_amdgcn_sched_barrier(0);
  pv_mfmas(o, v[Q % 2], p[Q]);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (Q + 1 < 4) pv_pipeline<Q + 1>(o, v, p, va);
}

__global__ __launch_bounds__(NT, AWG_PER_CU) void prefill_attn_kernel(AttnArgs a) {
  __shared__ AttnSmem sm;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  const int g4 = lane >> 4, l16 = lane & 15;
  // workgroups are dealt to the 8 XCDs in turn; XCD x takes the consecutive
  // units x*U .. x*U+U-1, i.e. the query blocks of a few heads, heaviest
  // (latest) block first, so the blocks of one head share that XCD's L2
  const int u = (blockIdx.x & 7) * a.units_per_xcd + (blockIdx.x >> 3);
  if (u >= a.units) return;
  // (readfirstlane: the compiler is told these are uniform, so the buffer
  // resources built from them stay in scalar registers)
  const int qb = __builtin_amdgcn_readfirstlane(a.n_qb - 1 - u % a.n_qb);
  const int hi = __builtin_amdgcn_readfirstlane((u / a.n_qb) % a.n_h);
  const int b = __builtin_amdgcn_readfirstlane(u / (a.n_qb * a.n_h));
  const int j0 = qb * 128;                      // first query row of the block
  // (a length outside [0, M] is a caller error; clamped, no access leaves kv)
  const int ctx = __builtin_amdgcn_readfirstlane(min(max(a.ctx_lens[b], 0), a.M));
  // rows past n_q repeat the last query (their results are not stored)
  const int jr = j0 + 32 * wave + l32;
  const int jq = jr < a.n_q ? jr : a.n_q - 1;
  const int64_t qrow = ((int64_t)b * a.n_q + jq) * a.n_h + hi;
  bf16x8 qreg[QK_STEPS];
  {
    const u16x8* qn = reinterpret_cast<const u16x8*>(a.q_nope + qrow * DN);
    const u16x8* qp = reinterpret_cast<const u16x8*>(a.q_pe + qrow * DR);
#pragma unroll
    for (int ks = 0; ks < DN / 16; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8, qn[2 * ks + h]);
#pragma unroll
    for (int ks = DN / 16; ks < QK_STEPS; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8, qp[2 * (ks - DN / 16) + h]);
  }
  // the last token the row sees: its position, within the sequence's cached tokens
  const int pos_q = a.positions[(int64_t)b * a.n_q + jq];
  const int pos = pos_q < ctx ? pos_q : ctx - 1;
  // the stage count follows the workgroup's largest position (every wave runs
  // the same stages: they share barriers); masking is decided per wave.  The
  // four waves' maxima meet in the first bytes of stage 1, before any load
  // writes there (the second barrier ends the reads).
  int pmax = pos, pmin = pos;
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) {
    pmax = max(pmax, __shfl_xor(pmax, sh, 64));
    pmin = min(pmin, __shfl_xor(pmin, sh, 64));
  }
  const int pos_min = __builtin_amdgcn_readfirstlane(pmin);
  int* xchg = reinterpret_cast<int*>(sm.stage[1]);
  if (lane == 0) xchg[wave] = pmax;
  lds_sync();
  const int pos_last = __builtin_amdgcn_readfirstlane(max(max(xchg[0], xchg[1]), max(xchg[2], xchg[3])));
  lds_sync();
  // tokens any row sees (ctx <= M, the rows kv holds, is checked by the caller)
  const int n_tok = __builtin_amdgcn_readfirstlane(pos_last + 1);
  const int nst = (n_tok + T - 1) / T;

  // loads: wave w fills rows 8w .. 8w+7 and 32+8w .. 32+8w+7 of every chunk group
  const int tt0 = 8 * wave + (lane >> 3);           // the second rows are tt0 + 32, same swizzle
  const int chunk = ((lane & 7) ^ swz(tt0)) << 4;
  const uint32_t kv_tok = (uint32_t)a.n_h * (KVW * 2);   // bytes between tokens in kv
  const unsigned char* kvb = a.kv + ((int64_t)b * a.M * a.n_h + hi) * (KVW * 2);
  const __amdgpu_buffer_rsrc_t rkv = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(kvb), (short)0,
                                                                       (int)((uint32_t)n_tok * kv_tok), kBufferWord3);
  const unsigned char* cb = a.cache + (int64_t)b * a.cache_seq_bytes;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(cb), (short)0,
                                                                      n_tok * a.cache_row_bytes, kBufferWord3);
  auto issue = [&](int s) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      unsigned char* dst = sm.stage[s % ANST] + 1024 * wave + 4096 * e;   // rows 8w + 32e ..
      const uint32_t tok = (uint32_t)(s * T + tt0 + 32 * e);   // rows past n_tok read as zeros
      const int vkv = (int)(tok * kv_tok + (uint32_t)chunk);
      const int vc = (int)(tok * (uint32_t)a.cache_row_bytes + (uint32_t)(a.rope_byte + chunk));
      // the chunk group's byte offset in the row goes in soffset: an immediate
      // offset would move the LDS destination as well
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rkv, (lds_void*)(dst + 0 * CG), 16, vkv, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rkv, (lds_void*)(dst + 1 * CG), 16, vkv, 128, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_void*)(dst + 2 * CG), 16, vc, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rkv, (lds_void*)(dst + 3 * CG), 16, vkv, 256, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rkv, (lds_void*)(dst + 4 * CG), 16, vkv, 384, 0, 0);
    }
  };

  // LDS offsets of this lane's S^T operands: token l32 of block 0; block 1 is
  // 32 rows on, with the same swizzle (s(t) has period 16)
  const int sw_qk = swz(l32);
  int qk_off[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) qk_off[r] = l32 * 128 + (((2 * r + h) ^ sw_qk) << 4);
  const int hq = g4 >> 1;
  const int tr_tok = 4 * hq + (l16 >> 2);
  const int sw_tr0 = swz(tr_tok), sw_tr1 = swz(8 + tr_tok);
  const int half8 = (l16 & 1) * 8;
  const int cch = 2 * (g4 & 1) + ((l16 & 3) >> 1);
  // Per-lane parts of the addresses of the transposed V reads, one per
  // (dv block parity, read half); the rest of each address is a constant that
  // goes in the instruction's offset field (see pv_reads).
  uint32_t v_lane[4];
#pragma unroll
  for (int d1 = 0; d1 < 2; ++d1)
#pragma unroll
    for (int ins = 0; ins < 2; ++ins)
      v_lane[2 * d1 + ins] = tr_tok * 128 + (((4 * d1 + cch) ^ (ins ? sw_tr1 : sw_tr0)) << 4) + half8;

  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  // score i of block k is token 32k + 8(i/4) + 4h + i%4 of the stage: visible while <= pos
  const int lim = pos - 4 * h;

  // One stage: S^T, online softmax (log2 units; the scale is folded into the
  // exponent's fma, the row maximum of the raw scores scaled once), PV.
  // MASKED: some row of this wave may not see every token of the stage.
  auto stage = [&](int s, auto masked_tag) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    // this wave's loads of stage s are in (those of stage s+1 may fly); the
    // barrier makes every wave's visible and ends every read of stage s-1,
    // whose slot stage s + ANST - 1 reuses
    if (ANST == 3 && s + 1 < nst) __builtin_amdgcn_s_waitcnt(0x0F70 | A_LOADS);   // vmcnt(10)
    else __builtin_amdgcn_s_waitcnt(0x0F70);                                       // vmcnt(0)
    lds_sync();
    if (s + ANST - 1 < nst) issue(s + ANST - 1);
    const unsigned char* sb = sm.stage[s % ANST];
    // S^T: K operands read QPF k-steps ahead of their MFMAs (the fences keep
    // that order; the compiler's waits then cover only the oldest reads)
    f32x16 st[2] = {f32x16{}, f32x16{}};
    auto rd_k = [&](int ks, int k) { return lds_read16(sb + (ks >> 2) * CG + 4096 * k + qk_off[ks & 3]); };
    bf16x8 kr[QPF][2];
#pragma unroll
    for (int ks = 0; ks < QPF; ++ks) {
      kr[ks][0] = rd_k(ks, 0);
      kr[ks][1] = rd_k(ks, 1);
    }
#pragma unroll
    for (int ks = 0; ks < QK_STEPS; ++ks) {
      const bf16x8 a0 = kr[ks % QPF][0], a1 = kr[ks % QPF][1];
      if (ks + QPF < QK_STEPS) {
        kr[ks % QPF][0] = rd_k(ks + QPF, 0);
        kr[ks % QPF][1] = rd_k(ks + QPF, 1);
      }
      st[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qreg[ks], st[0], 0, 0, 0);
      st[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qreg[ks], st[1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the V^T operands of PV step 0 go out now, under the softmax
    const uint32_t sbase = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const unsigned char*)sb);
    const uint32_t va[4] = {sbase + v_lane[0], sbase + v_lane[1], sbase + v_lane[2], sbase + v_lane[3]};
    bf16x8 vv[2][4];
    pv_reads<0>(vv[0], va);
    float mt = -INFINITY;
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if constexpr (MASKED) {
          const int rel = 32 * k + 8 * (i >> 2) + (i & 3);
          st[k][i] = s * T + rel <= lim ? st[k][i] : -INFINITY;
        }
        mt = fmaxf(mt, st[k][i]);
      }
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
      mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * a.scale_log2;
    }
    // The row's reference m_run moves only when the stage maximum passes it by
    // more than A_HEADROOM (and at the row's first visible stage, m_run =
    // -inf): weights are then at most 2^A_HEADROOM, and the accumulator is
    // rescaled rarely instead of at every new maximum.  Weights and their sum
    // share the reference, so the normalised result does not depend on it.
    // Masked stages: rows with nothing visible yet keep m = -inf, weights 0
    // and alpha 1 (in a whole stage every score is finite).
    const bool grow = mt > m_run + A_HEADROOM;
    const float m_new = grow ? mt : m_run;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - mt) : 1.f;
    const float neg = MASKED && m_new == -INFINITY ? 0.f : -m_new;
    m_run = m_new;
    float psum = 0.f;
    bf16x8 pb[4];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(st[k][i], a.scale_log2, neg));
        psum += p;
        pb[2 * k + (i >> 3)][i & 7] = (__bf16)p;
      }
    l_run = l_run * alpha + psum;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
    }
    pv_pipeline<0>(o, vv, pb, va);
  };
  using Whole = std::integral_constant<bool, false>;
  using Masked = std::integral_constant<bool, true>;
  // stages 0 .. n_whole-1 end at or before every row's position (s*T + T-1 <= pos_min);
  // every wave runs all nst stages, so the barriers inside stay matched
  const int n_whole = min(nst, max(pos_min + 1, 0) / T);
  for (int s = 0; s < ANST - 1 && s < nst; ++s) issue(s);
  int s = 0;
  for (; s < n_whole; ++s) stage(s, Whole{});
  for (; s < nst; ++s) stage(s, Masked{});
  static_assert(A_LOADS == 10, "one stage = 10 loads per wave");
  // ---- results: o[db][i] = O[row l32][dv 32 db + 8 (i/4) + 4 h + i%4]
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (jr < a.n_q) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* op = a.out + qrow * DV + 4 * h;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4*>(op + 32 * db + 8 * q) =
            f32x4{o[db][4 * q] * inv, o[db][4 * q + 1] * inv, o[db][4 * q + 2] * inv, o[db][4 * q + 3] * inv};
    if (a.lse != nullptr && h == 0)
      a.lse[qrow] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_prefill_weights(const uint16_t* w_uk, const uint16_t* w_uv, uint16_t* w_kv, int n_h, int d_c,
                                  hipStream_t stream) {
  hipLaunchKernelGGL(prefill_weights_kernel, dim3(d_c / 32, KVW / 32, n_h), dim3(NT), 0, stream, w_uk, w_uv, w_kv,
                     d_c);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  // 1. keys' content part and values of every head, tokens 0 .. max_ctx-1
  GemmArgs g;
  g.a = static_cast<const unsigned char*>(p.cache.data);
  g.a_seq_bytes = p.cache.seq_stride * 2;
  g.a_row_bytes = p.cache.row * 2;
  g.w = static_cast<const uint16_t*>(p.w_kv);
  g.c = static_cast<uint16_t*>(p.kv);
  g.M = p.max_ctx;
  g.N = p.n_h * KVW;
  g.K = p.d_c;
  g.mb = (g.M + GM - 1) / GM;
  g.nb = g.N / GN;
  g.tiles = g.mb * g.nb * p.B;
  g.tiles_per_xcd = (g.tiles + 7) / 8;
  if (g.tiles == 0) return hipSuccess;
  hipLaunchKernelGGL(reconstruct_gemm_kernel, dim3(g.tiles_per_xcd * 8), dim3(GNT), 0, stream, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // 2. attention
  AttnArgs a;
  a.q_nope = static_cast<const uint16_t*>(p.q_nope);
  a.q_pe = static_cast<const uint16_t*>(p.q_pe);
  a.positions = p.positions;
  a.ctx_lens = p.ctx_lens;
  a.cache = static_cast<const unsigned char*>(p.cache.data);
  a.cache_seq_bytes = p.cache.seq_stride * 2;
  a.cache_row_bytes = p.cache.row * 2;
  a.rope_byte = p.d_c * 2;
  a.kv = static_cast<const unsigned char*>(p.kv);
  a.out = p.out;
  a.lse = p.lse;
  a.B = p.B;
  a.n_q = p.n_q;
  a.n_h = p.n_h;
  a.M = p.max_ctx;
  a.n_qb = (p.n_q + 127) / 128;
  a.units = p.B * p.n_h * a.n_qb;
  a.units_per_xcd = (a.units + 7) / 8;
  a.scale_log2 = p.sm_scale * kLog2e;
  hipLaunchKernelGGL(prefill_attn_kernel, dim3(a.units_per_xcd * 8), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
