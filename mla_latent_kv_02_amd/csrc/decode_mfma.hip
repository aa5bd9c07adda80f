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
//     (c / 8) * 256 + t * 8 + ((c % 8) ^ s(t)),  s(t) = P[(t / 2) % 8],
//     P = (0, 4, 1, 5, 2, 6, 3, 7).
// A 1 KiB run of slots holds 8 tokens x 8 chunks, which is exactly what one
// 16-byte-per-lane global->LDS load writes; 8 lanes read 128 contiguous bytes
// of one token row (coalesced).  The xor keeps both LDS read patterns free of
// bank conflicts on gfx950's 64 four-byte banks: a 16-byte read serves 16
// lanes per cycle, here 16 consecutive tokens of one chunk (QK), whose two
// parity classes (rows 128 B apart share a 256-byte bank period) each see all
// 8 values of s; the transposed PV read serves 32 lanes, 4 consecutive tokens
// of 4 chunks, and s(t), s(t+2) differ in bit 2 so the two tokens of a parity
// class use disjoint aligned groups of 4 chunks.  (Measured: 0 bank conflicts
// for both patterns.)
//
// Pipeline: a ring of NSTAGE stages in LDS; loads run NSTAGE - 1 stages ahead
// of the stage being used, and each wave waits (vmcnt) only for the oldest
// stage it needs.  Softmax weights exp2(s - m_ref) use a fixed per-row
// reference, so the fp32 accumulator is never rescaled; the partial is
// written unnormalised together with its reference and log-sum-exp, and the
// combine normalises (exact for any reference).
//
// Split-KV: the workgroup walks the segments of its work unit (see
// for_each_segment) and writes one partial per segment: u unnormalised, with
// its reference and log-sum-exp (the format mla.h states for mla_decode).

#include <climits>
#include <type_traits>

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
// fp8 cache rows: [512 e4m3 codes | 64 bf16 rotated k_rope | 4 fp32 scales]
constexpr int RB16 = ROW * 2;                     // bytes of a bf16 row (1152)
constexpr int RB8 = DC + 2 * DR + 4 * (DC / 128); // bytes of an fp8 row (656)
constexpr int F8_ROPE = DC, F8_SCALE = DC + 2 * DR;   // byte offsets in an fp8 row
constexpr int NRAW = 3;               // fp8: stages of raw rows in flight per wave
// A wave's part of one raw fp8 stage: the codes of its 128-channel tile for
// the 32 tokens (4 loads of 8 tokens x 128 B), the positional keys of tokens
// 8w .. 8w+7 (1 load), the tile's scale of every token (1 load of 4 B per lane).
constexpr int RAW_CODES = 0, RAW_ROPE = 4096, RAW_SCALE = 5120, RAW_WAVE_BYTES = 5376;
constexpr int FP8_LOADS_PER_STAGE = 6;
// s_waitcnt immediates (GFX9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] << 14) that wait on vector memory only.  Issued through the
// builtin so that the compiler's own wait insertion sees them.
constexpr int kWaitVm0 = 0x0F70, kWaitVm9 = 0x0F79, kWaitVm18 = 0x4F72;
constexpr int kWaitVm6 = 0x0F76, kWaitVm12 = 0x0F7C;   // fp8: 6 loads per stage
// Word 3 of a raw buffer resource on gfx9-class chips (32-bit data format, no
// swizzle, offsets in bytes); words 0-2 carry the base and the byte range.
constexpr int kBufferWord3 = 0x00020000;
// Cache-policy operand of the bf16 cache row loads: the non-temporal hint (nt,
// bit 1 on gfx940-class chips).  Every row is read once per launch; with the
// hint the paged batch's decode ran 1.5-3 % faster.  (The fp8 row loads were
// no faster with it and keep the default policy.)
constexpr int kRowLoadPolicy = 2;

struct DecodeArgs {
  const uint16_t* q_lat;   // [B][n_q][n_h][512]
  const uint16_t* q_pe;    // [B][n_q][n_h][64]
  CacheView cache;
  const int32_t* ctx_lens;
  const int32_t* positions;  // [B][n_q]
  float* u_part;           // [slots][n_q][n_h][512]
  float* lse_part;         // [slots][n_q][n_h][2]: (reference, log-sum-exp)
  int B, n_q, n_h, num_splits, n_groups, n_work_pad;
  float scale_log2;        // sm_scale * log2(e)
};

// Byte range of a buffer resource over the first n rows of rb bytes (the
// resource's range is 32 bits; the launch keeps a sequence within 4 GiB).
__device__ __forceinline__ int record_bytes(int n, int rb) {
  const int64_t v = (int64_t)n * rb;
  return (int)(uint32_t)(v < (int64_t)0xFFFFFFFF ? v : (int64_t)0xFFFFFFFF);
}

// s(t) of the stage layout: P[(t >> 1) & 7] with P packed in nibbles
__device__ __forceinline__ int swz(int t) { return (0x73625140 >> (4 * ((t >> 1) & 7))) & 7; }

struct __attribute__((aligned(16))) DecodeSmem {
  unsigned char stage[NSTAGE][STAGE_BYTES];
  bf16x8 pbuf[4][2][64];     // softmax weights of the stage: [head block][k-step][lane], B-operand layout
  int flag[4];               // per wave: a score ran past its row's reference (redo needed)
  PlanScratch<NT> plan;
};

// fp8 caches: two bf16 stages (the layout above), filled by converting the
// raw fp8 rows that each wave loads into its own part of a raw ring.
struct __attribute__((aligned(16))) DecodeSmemFp8 {
  unsigned char stage[2][STAGE_BYTES];
  unsigned char raw[NRAW][4 * RAW_WAVE_BYTES];
  bf16x8 pbuf[4][2][64];
  int flag[4];
  PlanScratch<NT> plan;
};
static_assert(sizeof(DecodeSmemFp8) <= 160 * 1024, "LDS budget");

// Cache layouts the kernel is compiled for.
enum Layout : int {
  kContiguous = 0,   // [B][seq_stride] rows; a sequence's rows (plus one stage) span < 4 GiB
  kPaged = 1,        // block table, block_size a multiple of T (a stage lies in one block)
  kAnyLayout = 2,    // any block size: per-token row lookup
};

// Paged addressing of consecutive stages of T tokens.  The block size is a
// multiple of T and every stage starts at a token that is a multiple of T
// (the kernel starts a segment's stages at the multiple of T at or below its
// first token), so a stage lies in one block: block k0 from row r0 on, with
// r0 + T <= block_size.  Stages come in order, T tokens apart, so (k0, r0)
// follows from the previous stage without a division (a restart recomputes
// it).  The block ids come from a window of 64 ids, one per lane (`ids`),
// reloaded when a stage leaves it (one vector load, waited for right there: a
// wait placed by the compiler at the uses of `ids` would sit on every stage's
// path and drain the stage loads in flight each time; this one runs once per
// 64 blocks).  locate() gives the byte offset, from the resource base at block
// blk_lo, of the stage's first row: row t < span + 1 of the stage is at
// off0 + t * rb, rows past the segment end repeat its last row (uint32
// arithmetic, exact modulo 2^32).
struct PagedCursor {
  int ids, kbase;              // lane l holds the id of block kbase + l of the sequence
  int ntok, nk, nr;            // the next stage's first token, its block index and row in it
  uint32_t off0;               // row r0 of block k0
  int r0, span, bs;
  uint32_t rb;                 // row bytes

  __device__ __forceinline__ void init(int block_size, uint32_t row_bytes) {
    kbase = INT_MIN / 2;         // no window loaded yet
    ids = 0;
    ntok = INT_MIN;              // next stage unknown
    nk = nr = 0;
    bs = block_size;
    rb = row_bytes;
  }
  __device__ __forceinline__ void locate(const CacheView& c, int b, int tok0, int tok_end, int blk_lo, int lane,
                                         uint32_t block_bytes) {
    if (tok0 != ntok) {
      nk = tok0 / bs;
      nr = tok0 - nk * bs;
    }
    const int k0 = nk;
    r0 = nr;
    span = T - 1 < tok_end - 1 - tok0 ? T - 1 : tok_end - 1 - tok0;   // last row, from tok0
    ntok = tok0 + T;
    nr = r0 + T;
    if (nr == bs) {   // the next stage starts the next block
      nr = 0;
      ++nk;
    }
    if (k0 < kbase || k0 - kbase >= 64) {
      kbase = k0;
      const int k = k0 + lane;
      ids = k <= (tok_end - 1) / bs ? c.block_table[(int64_t)b * c.max_blocks + k] : 0;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    const int blk0 = __builtin_amdgcn_readlane(ids, k0 - kbase);
    off0 = (uint32_t)(blk0 - blk_lo) * block_bytes + (uint32_t)r0 * rb;
  }
  // byte offset of stage row t (clamped to the segment's last row) plus `byte`
  __device__ __forceinline__ uint32_t row(int t, uint32_t byte) const {
    const int tt = t < span ? t : span;
    return off0 + (uint32_t)tt * rb + byte;
  }
};

// Issues this wave's share of the global->LDS loads of one stage: stage
// tokens 8*wave + lane/8, all 9 chunk groups (9 loads of 1 KiB per wave).
// Lane (token tt, chunk c%8) reads 16 bytes at chunk (c%8) ^ s(tt) of its
// row, so the LDS slot it fills is the swizzled one (see the layout above).
//
// Contiguous caches use buffer loads: the resource (SGPRs) spans the
// segment's rows of one sequence, so tokens past the segment end fall out of
// range and read as zeros (never the cache's padding); each lane keeps one
// 32-bit offset.  Paged caches (block_size a multiple of T) clamp such tokens to the last
// row of the segment and also use buffer loads, from a resource that starts at
// the lowest block of the segment (blk_lo); the caller takes this layout only
// when every block of the segment lies within 4 GiB of that one (else the
// generic layout).  The generic layout (any block size) uses 64-bit per-lane
// addresses.
template <int LAYOUT>
struct StageLoader {
  const unsigned char* base;   // contiguous: first row of the sequence; else cache base
  __amdgpu_buffer_rsrc_t rsrc;
  const CacheView* c;
  int b, tok_end, blk_lo;
  int lane_off;                // contiguous: byte offset of the lane within a stage
  int tt, chunk_off;
  int lane_;
  PagedCursor pc;
  uint32_t block_bytes;

  __device__ __forceinline__ void init(const CacheView& cache, int b_, int tok_end_, int wave, int lane,
                                       int blk_lo_) {
    c = &cache;
    b = b_;
    tok_end = tok_end_;
    blk_lo = blk_lo_;
    lane_ = lane;
    tt = 8 * wave + (lane >> 3);
    chunk_off = ((lane & 7) ^ swz(tt)) * 16;
    base = static_cast<const unsigned char*>(cache.data);
    if (LAYOUT == kContiguous) {
      base += (int64_t)b * cache.seq_stride * 2;
      rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(base), (short)0,
                                               record_bytes(tok_end, RB16), kBufferWord3);
      lane_off = tt * RB16 + chunk_off;
    } else if (LAYOUT == kPaged) {
      pc.init(cache.block_size, RB16);
      block_bytes = (uint32_t)cache.block_size * RB16;
      rsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<unsigned char*>(base + (int64_t)blk_lo * block_bytes), (short)0, (int)0xFFFFFFFF, kBufferWord3);
      lane_off = tt * RB16 + chunk_off;
    }
  }

  // per-stage addressing (scalar block lookups for paged caches), then one
  // chunk group per issue_cg call, so the 9 loads can be spread out
  uint32_t voff;
  const unsigned char* rowp;
  __device__ __forceinline__ void prepare(int tok0) {
    if (LAYOUT == kContiguous) {
      voff = (uint32_t)lane_off + (uint32_t)tok0 * (uint32_t)RB16;
      return;
    }
    if (LAYOUT == kPaged) {
      pc.locate(*c, b, tok0, tok_end, blk_lo, lane_, block_bytes);
      voff = pc.row(tt, chunk_off);
      return;
    }
    int tok = tok0 + tt;
    tok = tok < tok_end ? tok : tok_end - 1;   // rows past the segment repeat a valid row
    rowp = base + cache_row_offset(*c, b, tok) * 2 + chunk_off;
  }
  __device__ __forceinline__ void issue_cg(int cg, unsigned char* buf, int wave) {
    unsigned char* dst = buf + wave * 1024 + cg * CG_BYTES;
    if (LAYOUT == kContiguous || LAYOUT == kPaged)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, (int)voff, cg * 128, 0, kRowLoadPolicy);
    else
      __builtin_amdgcn_global_load_lds(rowp + cg * 128, (lds_void*)dst, 16, 0, kRowLoadPolicy);
  }
  __device__ __forceinline__ void issue(int tok0, unsigned char* buf, int wave) {
    prepare(tok0);
#pragma unroll
    for (int cg = 0; cg < CGROUPS; ++cg) issue_cg(cg, buf, wave);
  }
};

// The fp8 counterpart of StageLoader: wave w loads, for one stage, exactly
// the bytes it will convert (so its raw ring needs no workgroup barrier):
//   loads 0-3: codes of tile w, tokens 8i + lane/8, 16 bytes at 128w + 16(lane%8)
//              (8 lanes read 128 contiguous bytes of a row);
//   load 4:    positional key of token 8w + lane/8, chunk (lane%8) ^ s(token)
//              (already in its bf16 stage slot order);
//   load 5:    scale of tile w of token lane%32 (4 bytes; lanes 32-63 repeat).
// LDS destination: the wave's part of a raw stage, 1 KiB per load in lane
// order (the scale load 256 B).  Rows past the segment end read as zeros
// (contiguous) or repeat its last row (paged, generic), as for bf16 rows.
template <int LAYOUT>
struct Fp8Loader {
  const unsigned char* base;
  __amdgpu_buffer_rsrc_t rsrc;
  const CacheView* c;
  int b, tok_end, blk_lo, lane_, wave_;
  PagedCursor pc;
  uint32_t block_bytes;
  uint32_t lc[3];              // contiguous: lane offsets of the codes, key and scale loads in a stage
  uint32_t sbase;              // contiguous: byte offset of the stage's first row
  uint32_t rowidx[FP8_LOADS_PER_STAGE];   // generic layout: row of load i, counted from the cache start

  __device__ __forceinline__ int token(int i) const {   // stage token of load i for this lane
    return i < 4 ? 8 * i + (lane_ >> 3) : (i == 4 ? 8 * wave_ + (lane_ >> 3) : (lane_ & 31));
  }
  __device__ __forceinline__ uint32_t byte(int i) const {   // byte offset of load i in its row
    return i < 4 ? 128 * wave_ + 16 * (lane_ & 7)
                 : (i == 4 ? F8_ROPE + 16 * ((lane_ & 7) ^ swz(8 * wave_ + (lane_ >> 3))) : F8_SCALE + 4 * wave_);
  }
  __device__ __forceinline__ void init(const CacheView& cache, int b_, int tok_end_, int wave, int lane,
                                       int blk_lo_) {
    c = &cache;
    b = b_;
    tok_end = tok_end_;
    blk_lo = blk_lo_;
    lane_ = lane;
    wave_ = wave;
    base = static_cast<const unsigned char*>(cache.data);
    if (LAYOUT == kContiguous) {
      base += (int64_t)b * cache.seq_stride;    // bytes
      rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(base), (short)0,
                                               record_bytes(tok_end, RB8), kBufferWord3);
#pragma unroll
      for (int k = 0; k < 3; ++k) lc[k] = (uint32_t)token(k == 0 ? 0 : k + 3) * RB8 + byte(k == 0 ? 0 : k + 3);
    } else if (LAYOUT == kPaged) {
      pc.init(cache.block_size, RB8);
      block_bytes = (uint32_t)cache.block_size * RB8;
      rsrc = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<unsigned char*>(base + (int64_t)blk_lo * block_bytes), (short)0, (int)0xFFFFFFFF, kBufferWord3);
    }
  }
  // per-stage state: uniform values only, except the generic layout's pointers
  __device__ __forceinline__ void prepare(int tok0) {
    if (LAYOUT == kContiguous) {
      sbase = (uint32_t)tok0 * RB8;
    } else if (LAYOUT == kPaged) {
      pc.locate(*c, b, tok0, tok_end, blk_lo, lane_, block_bytes);
    } else {
#pragma unroll
      for (int i = 0; i < FP8_LOADS_PER_STAGE; ++i) {
        int tok = tok0 + token(i);
        tok = tok < tok_end ? tok : tok_end - 1;
        rowidx[i] = (uint32_t)(cache_row_offset(*c, b, tok) / RB8);   // rows counted in bytes
      }
    }
  }
  // load i of the prepared stage into `dst`, this wave's part of a raw stage
  __device__ __forceinline__ void issue_cg(int i, unsigned char* dst, int) {
    lds_void* d = (lds_void*)(dst + (i < 4 ? RAW_CODES + 1024 * i : (i == 4 ? RAW_ROPE : RAW_SCALE)));
    if (LAYOUT == kContiguous || LAYOUT == kPaged) {
      int vo, so;
      if (LAYOUT == kContiguous) {
        vo = (int)lc[i < 4 ? 0 : i - 3];
        so = (int)(sbase + (i < 4 ? 8u * i * RB8 : 0u));
      } else {
        // the per-lane parts of the six loads' offsets are formed here, from
        // an opaque copy of the lane index, so the compiler cannot hoist them
        // out of the stage loop (twelve more live registers there spill)
        int ln = lane_;
        asm volatile("" : "+v"(ln));
        const int q = ln >> 3, p = ln & 7;
        const int t = i < 4 ? 8 * i + q : (i == 4 ? 8 * wave_ + q : (ln & 31));
        const uint32_t by = i < 4 ? 128 * wave_ + 16 * p
                                  : (i == 4 ? F8_ROPE + 16 * (p ^ swz(8 * wave_ + q)) : F8_SCALE + 4 * wave_);
        vo = (int)pc.row(t, by);
        so = 0;
      }
      if (i < 5) __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, d, 16, vo, so, 0, 0);
      else __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, d, 4, vo, so, 0, 0);
    } else {
      const unsigned char* src = base + (uint64_t)rowidx[i] * RB8 + byte(i);
      if (i < 5) __builtin_amdgcn_global_load_lds(src, d, 16, 0, 0);
      else __builtin_amdgcn_global_load_lds(src, d, 4, 0, 0);
    }
  }
  __device__ __forceinline__ void issue(int tok0, unsigned char* dst, int wave) {
    prepare(tok0);
#pragma unroll
    for (int i = 0; i < FP8_LOADS_PER_STAGE; ++i) issue_cg(i, dst, wave);
  }
};

// Converts this wave's part of a raw fp8 stage into the bf16 stage `bf`: the
// 128 latents of tile w (chunk groups 2w, 2w+1) of all 32 tokens, and the
// positional keys of tokens 8w .. 8w+7 (chunk group 8).  A lane converts the
// 16-byte pieces it loaded: piece i holds latents 128w + 16(lane%8) .. +16 of
// token 8i + lane/8, i.e. bf16 chunks 2(lane%8) and 2(lane%8)+1 of the tile.
// Codes times the power-of-two scale are exact in bf16 (3 of its 7 mantissa
// bits; the scaled conversion applies the scale as an exponent offset).
__device__ __forceinline__ void convert_fp8_stage(const unsigned char* rw, unsigned char* bf, int wave, int lane) {
  typedef __attribute__((address_space(3))) const u32x4 lds_cu32x4;
  typedef __attribute__((address_space(3))) const float lds_cf32;
  typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  const auto L = [](const unsigned char* p) { return (__attribute__((address_space(3))) unsigned char*)p; };
  // The lane-dependent offsets below are cheap to form; an opaque copy of the
  // lane index keeps the compiler from hoisting them out of the stage loop,
  // where they would hold registers for the whole loop.
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const int p8 = ln & 7, tq = ln >> 3;
  // token 8i + tq: s(8i + tq) = s(tq) for even i and s(tq) ^ 2 for odd i
  // (P[x + 4] = P[x] ^ 2), so the write slots of both chunks of every piece
  // are x, x^1, x^2, x^3 with x = 2(p8 % 4) ^ s(tq), plus 1024 i.
  const int x = (2 * (p8 & 3)) ^ swz(tq);
  unsigned char* wbase = bf + (2 * wave + (p8 >> 2)) * CG_BYTES + tq * 128;
  const unsigned char* rbase = rw + RAW_CODES + 16 * ln;
  const unsigned char* sbase = rw + RAW_SCALE + 4 * tq;
  // every read first (the raw and bf16 stages could alias as far as the
  // compiler knows, so it would not move a read above an earlier write)
  float sc[4];
  u32x4 w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sc[i] = *(lds_cf32*)L(sbase + 32 * i);
    w[i] = *(lds_cu32x4*)L(rbase + 1024 * i);
  }
  const u32x4 key = *(lds_cu32x4*)L(rw + RAW_ROPE + 16 * ln);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bf16x8 o[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const auto a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i][2 * h], sc[i], false);
      const auto a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i][2 * h], sc[i], true);
      const auto a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i][2 * h + 1], sc[i], false);
      const auto a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i][2 * h + 1], sc[i], true);
      o[h] = bf16x8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
    }
    const int xi = x ^ (i & 1 ? 2 : 0);
    *(lds_bf16x8*)L(wbase + 1024 * i + (xi << 4)) = o[0];
    *(lds_bf16x8*)L(wbase + 1024 * i + ((xi ^ 1) << 4)) = o[1];
  }
  *(lds_u32x4*)L(bf + 8 * CG_BYTES + 1024 * wave + 16 * ln) = key;
}

// Paged cache, tokens t0..t1-1 of sequence b: the lowest block id among their
// blocks, and whether all of them lie within 4 GiB of it (kSpanNear: 32-bit
// buffer offsets from it reach every row) or not (kSpanFar); kSpanInvalid if
// the descriptor cannot place them (a block past the table row, or a negative
// id).  Each wave reads the block table entries itself and reduces them across
// its lanes; the result is the same in every wave.
enum SpanKind : int { kSpanNear = 0, kSpanFar = 1, kSpanInvalid = 2 };
__device__ __forceinline__ int paged_span(const CacheView& c, int b, int t0, int t1, int lane, int row_bytes,
                                          int* blk_lo) {
  const int bs = c.block_size;
  const int k0 = t0 / bs, k1 = (t1 - 1) / bs;
  if (k1 >= c.max_blocks) return kSpanInvalid;
  int lo = INT_MAX, hi = INT_MIN;
  for (int k = k0 + lane; k <= k1; k += 64) {
    const int id = c.block_table[(int64_t)b * c.max_blocks + k];
    lo = id < lo ? id : lo;
    hi = id > hi ? id : hi;
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) {
    const int ol = __shfl_xor(lo, sh, 64), oh = __shfl_xor(hi, sh, 64);
    lo = ol < lo ? ol : lo;
    hi = oh > hi ? oh : hi;
  }
  *blk_lo = __builtin_amdgcn_readfirstlane(lo);
  if (*blk_lo < 0) return kSpanInvalid;
  const int64_t span = ((int64_t)__builtin_amdgcn_readfirstlane(hi) - *blk_lo + 1) * bs * row_bytes;
  return span <= (int64_t)0xFFFFFFFF ? kSpanNear : kSpanFar;
}

// Workgroup barrier that waits only for this wave's LDS operations (a
// __syncthreads() would also wait for every outstanding global load and so
// drain the stage pipeline).  Stage data arriving through global->LDS loads is
// covered by the explicit vmcnt waits before the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

static_assert(FP8_LOADS_PER_STAGE == 6 && NRAW == 3, "fp8 wait counts assume 6 loads per stage, 3 raw stages");

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
//     32-row block S^T with one chain of 36 32x32x16 MFMAs.  Lane l holds row l%32 and tokens
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
//
// fp8 caches (FP8): the bf16 stages alternate between two buffers; wave w
// converts tile w of raw stage it+2 into the buffer of stage it right after
// its own PV of stage it (which reads only tile w of that buffer, and the QK
// reads of it ended at the previous iteration's second barrier), so the
// conversion needs no barrier of its own: the next iteration's first barrier
// publishes it.  Raw stage it+1+NRAW is loaded during the QK of iteration it.
template <int LAYOUT, bool FP8>
__global__ __launch_bounds__(NT, 1) void decode_mfma_kernel(DecodeArgs a) {
  using Smem = std::conditional_t<FP8, DecodeSmemFp8, DecodeSmem>;
  __shared__ Smem smem;
  Smem* sm = &smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;          // lane half
  const int l32 = lane & 31;
  const int g4 = lane >> 4;         // lane group of 16 (transposed reads)
  const int l16 = lane & 15;

  // block -> (work unit, row group).  Workgroups are dealt to the 8 XCDs in
  // turn (block b runs on XCD b % 8), so XCD x gets blocks x, x+8, ...; they
  // take the consecutive work units x*U .. x*U+U-1 (U = units per XCD), all
  // row groups of a unit together.  The units of one sequence then share an
  // L2: its query rows are fetched from memory once per XCD, and the row
  // groups of a unit read the same cache tiles.
  const int bid = blockIdx.x;
  const int units_per_xcd = a.n_work_pad / 8;
  const int j = bid >> 3;
  const int w = (bid & 7) * units_per_xcd + j / a.n_groups;
  const int g = j % a.n_groups;
  if (w >= a.num_splits) return;

  const int rows = a.n_q * a.n_h;
  const int grow0 = g * 128;                  // first query row of the workgroup
  const int row0 = grow0 + wave * 32;         // first QK row of this wave
  const bool active = row0 < rows;
  const int jq = active ? row0 / a.n_h : 0;   // query token of this wave's QK rows

  // one segment (tokens t0_seg..t1-1 of sequence b, partial slot `slot`), its
  // cache rows read through the stage loader of layout SL.  Stages cover T
  // tokens from t0; in the paged layout t0 is the multiple of T at or below
  // t0_seg (so that no stage meets two blocks) and the scores of the tokens
  // before t0_seg, all in stage 0, are masked.
  auto segment = [&](auto layout_tag, int b, int t0_seg, int t1, int slot, int blk_lo) {
    constexpr int SL = decltype(layout_tag)::value;
    const int t0 = SL == kPaged ? (t0_seg & ~(T - 1)) : t0_seg;
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
    // Wait for the query rows before the first stage loads go out.  The
    // stage loop reads these registers in every iteration; without a wait
    // that covers them on every path, the compiler puts vector-memory waits
    // in front of their uses inside the loop, and such a wait also waits for
    // the stage loads issued just before it (the counter completes in order),
    // which drains the prefetch pipeline once per stage.
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    std::conditional_t<FP8, Fp8Loader<SL>, StageLoader<SL>> ld;
    ld.init(a.cache, b, t1, wave, lane, blk_lo);
    // bf16 stage s (ring of NSTAGE, or two buffers for fp8); this wave's part of raw stage s
    auto stage_buf = [&](int s) -> unsigned char* {
      if constexpr (FP8) return sm->stage[s & 1];
      else return sm->stage[s % NSTAGE];
    };
    auto raw_buf = [&](int s) -> unsigned char* {
      if constexpr (FP8) return sm->raw[s % NRAW] + wave * RAW_WAVE_BYTES;
      else return nullptr;
    };
    // fp8: wait until raw stage s (of stages issued up to `last`) has landed, then convert it
    auto convert_stage = [&](int s, int last) {
      const int after = last - s;   // stages issued after s, still allowed in flight
      if (after >= 2) __builtin_amdgcn_s_waitcnt(kWaitVm12);
      else if (after == 1) __builtin_amdgcn_s_waitcnt(kWaitVm6);
      else __builtin_amdgcn_s_waitcnt(kWaitVm0);
      convert_fp8_stage(raw_buf(s), stage_buf(s), wave, lane);
    };
    // per-lane LDS byte offsets that do not depend on the stage
    const int sw_qk = swz(l32);
    int qk_off[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) qk_off[r] = l32 * 128 + (((2 * r + h) ^ sw_qk) << 4);
    const int hq = g4 >> 1;                              // k half of this lane's transposed read
    const int tr_tok = 4 * hq + (l16 >> 2);              // token (mod 8) of this lane's row
    const int sw_tr0 = swz(tr_tok), sw_tr1 = swz(8 + tr_tok);   // s(t) of t = 16q + 8ins + tr_tok
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
        const unsigned char* p = sb + (mbg >> 1) * CG_BYTES + t * 128 + ((cq ^ (ins ? sw_tr1 : sw_tr0)) << 4) + half8;
        v[ins] = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4*)((__attribute__((address_space(3))) unsigned char*)p));
      }
      return __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3, 4, 5, 6, 7);
    };
    constexpr int PF = 2;          // K operands read ahead of their MFMA

    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) o[mb][hb] = f32x16{};
      l_run = 0.f;
      bool over = false;
      if constexpr (!FP8) {
#pragma unroll
        for (int s = 0; s < NSTAGE - 1; ++s)
          if (s < nst) ld.issue(t0 + s * T, stage_buf(s), wave);
      } else {
#pragma unroll
        for (int s = 0; s < NRAW; ++s)
          if (s < nst) ld.issue(t0 + s * T, raw_buf(s), wave);
      }

      // Pipeline, iteration it: publish the weights of stage it (computed in
      // the previous iteration), S^T of stage it+1 (MFMA only), then PV of
      // stage it with the softmax of stage it+1 spread between its MFMAs, one
      // small piece after each (the VALU work then runs while the matrix core
      // is busy).  Stage it+3 is loaded into the slot stage it-1 freed.
      f32x16 s_nx = f32x16{};            // scores of the stage whose weights come next
      bf16x8 pb[2] = {bf16x8{}, bf16x8{}};   // weights of the stage about to be published
      // S^T of one stage into s_nx: one MFMA accumulation chain (dependent
      // 32x32x16 MFMAs issue back to back; a single chain also spares the sum
      // of several partial accumulators)
      // With LOADS, the 9 loads of a later stage (prepared in ld) are issued
      // one per 4 k-steps, so their issue overlaps the MFMAs.
      auto qk = [&](const unsigned char* sb, auto loads_tag, unsigned char* ldst) {
        constexpr bool LOADS = decltype(loads_tag)::value;
        f32x16 acc = f32x16{};
        bf16x8 kring[PF];
#pragma unroll
        for (int ks = 0; ks < PF; ++ks) kring[ks] = rd_k(sb, ks);
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) {
          const bf16x8 kk = kring[ks % PF];
          if (ks + PF < KSTEPS) kring[ks % PF] = rd_k(sb, ks + PF);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, qreg[ks], acc, 0, 0, 0);
          if constexpr (LOADS && !FP8) {
            if ((ks & 3) == 1) ld.issue_cg(ks >> 2, ldst, wave);
          } else if constexpr (LOADS) {
            if (ks % 6 == 1) ld.issue_cg(ks / 6, ldst, wave);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        s_nx = acc;
      };
      using NoLoads = std::integral_constant<bool, false>;
      using WithLoads = std::integral_constant<bool, true>;
      // Softmax of the raw scores in s_nx in small pieces of a few VALU ops,
      // one after each PV MFMA of the previous stage, so that the VALU work
      // runs while the matrix core is busy.  Two schedules:
      //  - masked (stages that reach the row's limit, and stage 0; 30 pieces):
      //    0-7 mask scores of tokens at or past the limit (lim = limit minus the
      //    lane's base token; INT_MIN masks all, leaving the weights zero) and,
      //    in stage 0, of tokens before the segment's first (lo = t0_seg minus
      //    the lane's base token), 8-11 lane
      //    maximum, 12 row maximum (the two lanes holding a row exchange
      //    theirs), 13 reference update, 14-29 one weight exp2(s*scale - m_ref);
      //  - visible (every token of the stage visible; 27 pieces), staggered so
      //    that no piece waits on its own results: 0-3 maxima of 4 scores, 4
      //    lane maximum, 5 exchange, 6 row maximum, 7-8 reference update, then
      //    piece 9+i forms the exponent of score i, takes exp2 of score i-1
      //    and accumulates score i-2 (into one of two sums) and its bf16 weight.
      constexpr int PIECES_MASKED = 30, PIECES_VISIBLE = 27;
      float mt = -INFINITY, neg_m = 0.f;
      float psum[2] = {0.f, 0.f};
      float t4[4];
      unsigned sw_mt[2];
      auto sm_piece = [&](int k, int lim, int lo) {
        if (k < 8) {
#pragma unroll
          for (int e = 2 * k; e < 2 * k + 2; ++e) {
            const int rel = 8 * (e >> 2) + (e & 3);      // token of s_nx[e] minus the lane's base token
            s_nx[e] = (rel < lim && rel >= lo) ? s_nx[e] : -INFINITY;
          }
        } else if (k < 12) {
          const int j = k - 8;
          mt = fmaxf(mt, fmaxf(fmaxf(s_nx[4 * j], s_nx[4 * j + 1]), fmaxf(s_nx[4 * j + 2], s_nx[4 * j + 3])));
        } else if (k == 12) {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
          mt = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1])) * a.scale_log2;
        } else if (k == 13) {
          m_max = fmaxf(m_max, mt);
          if (m_ref == -INFINITY) m_ref = mt;       // first visible stage of the row
          over |= mt > m_ref + REF_HEADROOM;
          neg_m = m_ref == -INFINITY ? 0.f : -m_ref;
        } else if (k < PIECES_MASKED) {
          const int e = k - 14;
          const float pv = __builtin_amdgcn_exp2f(fmaf(s_nx[e], a.scale_log2, neg_m));
          psum[e & 1] += pv;
          pb[e >> 3][e & 7] = (__bf16)pv;
        }
      };
      auto sm_piece_visible = [&](int k) {
        if (k < 4) {
          t4[k] = fmaxf(fmaxf(s_nx[4 * k], s_nx[4 * k + 1]), fmaxf(s_nx[4 * k + 2], s_nx[4 * k + 3]));
        } else if (k == 4) {
          mt = fmaxf(fmaxf(t4[0], t4[1]), fmaxf(t4[2], t4[3]));
        } else if (k == 5) {
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mt), __float_as_uint(mt), false, false);
          sw_mt[0] = sw[0];
          sw_mt[1] = sw[1];
        } else if (k == 6) {
          mt = fmaxf(__uint_as_float(sw_mt[0]), __uint_as_float(sw_mt[1])) * a.scale_log2;
        } else if (k == 7) {
          m_max = fmaxf(m_max, mt);
          if (m_ref == -INFINITY) m_ref = mt;       // first visible stage of the row
        } else if (k == 8) {
          over |= mt > m_ref + REF_HEADROOM;
          neg_m = -m_ref;                            // finite: this stage has visible tokens
        } else if (k < PIECES_VISIBLE) {
          const int i = k - 9;
          if (i < 16) s_nx[i] = fmaf(s_nx[i], a.scale_log2, neg_m);
          if (i >= 1 && i <= 16) s_nx[i - 1] = __builtin_amdgcn_exp2f(s_nx[i - 1]);
          if (i >= 2) {
            const int e = i - 2;
            psum[e & 1] += s_nx[e];
            pb[e >> 3][e & 7] = (__bf16)s_nx[e];
          }
        }
      };
      // base token of this lane's scores within a stage: 8*(i/4) + 4*h + i%4 for score i
      auto lane_lim = [&](int tok0) { return limit - tok0 - 4 * h; };

      // ---- prologue: scores and weights of stage 0
      if constexpr (!FP8) {
        wait_stages_in_flight(nst - 1 < NSTAGE - 2 ? nst - 1 : NSTAGE - 2);
      } else {
        // stages 0 and 1 into the two bf16 buffers; raw stage NRAW reuses stage 0's slot
        int last = nst - 1 < NRAW - 1 ? nst - 1 : NRAW - 1;
        convert_stage(0, last);
        if (NRAW < nst) {
          ld.issue(t0 + NRAW * T, raw_buf(NRAW), wave);
          last = NRAW;
        }
        if (nst > 1) convert_stage(1, last);
      }
      lds_barrier();
      if (active && t0_seg < limit) {
        qk(stage_buf(0), NoLoads{}, nullptr);
        const int lim = lane_lim(t0);
        const int lo = t0_seg - t0 - 4 * h;
#pragma unroll
        for (int k = 0; k < PIECES_MASKED; ++k) sm_piece(k, lim, lo);
        l_run += psum[0] + psum[1];
      }

      // O^T[own 128 latents][128 rows] += V^T . P^T for one stage, with the
      // softmax pieces of the next stage after the MFMAs
      auto pv_stage = [&](const unsigned char* sb, auto visible_tag, int lim) {
        constexpr bool VISIBLE = decltype(visible_tag)::value;
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
            for (int hb = 0; hb < 4; ++hb) {
              pv_mfma(o[mb][hb], cur, pq[hb]);
              if (VISIBLE) sm_piece_visible(16 * q + 4 * mb + hb);
              else sm_piece(16 * q + 4 * mb + hb, lim, 0);   // (stages past 0 start inside the segment)
              __builtin_amdgcn_sched_barrier(0);
            }
          }
        }
      };
      using Visible = std::integral_constant<bool, true>;
      using Masked = std::integral_constant<bool, false>;

      // one iteration of the stage loop; VISIBLE: the next stage's tokens are
      // all visible to this wave's rows (its softmax needs no mask)
      auto iteration = [&](int it, auto visible_tag) {
        constexpr bool VISIBLE = decltype(visible_tag)::value;
        const bool has_next = it + 1 < nst;
        // addresses of the stage to load first, ahead of the waits (a paged cache
        // takes its block ids from the register window, reloaded now and then):
        // bf16 stage it+3 into the ring slot stage it-1 freed; fp8 raw stage
        // it+1+NRAW into the raw slot of stage it+1 (converted last iteration)
        const int ld_stage = FP8 ? it + 1 + NRAW : it + NSTAGE - 1;
        // fp8 rows in the generic layout: the 6 loads go out at once (their
        // per-lane rows would otherwise stay live through the QK chain)
        constexpr bool kIssueNow = FP8 && SL == kAnyLayout;
        const bool do_load = ld_stage < nst;
        if (do_load) {
          if constexpr (kIssueNow) ld.issue(t0 + ld_stage * T, raw_buf(ld_stage), wave);
          else ld.prepare(t0 + ld_stage * T);
        }
        if constexpr (!FP8) {
          if (has_next) wait_stages_in_flight(it + 2 < nst ? 1 : 0);   // stage it+1 resident
        }
        lds_barrier();   // every wave is done with the weights of stage it-1 (fp8: and
                         // has converted its part of stage it+1)
        // ------------ publish the weights of stage it (B-operand layout, per k-step)
        sm->pbuf[wave][0][lane] = pb[0];
        sm->pbuf[wave][1][lane] = pb[1];
        pb[0] = bf16x8{};
        pb[1] = bf16x8{};
        // the loads ride along with the MFMAs of S^T(it+1) when there are any
        unsigned char* ldst = FP8 ? raw_buf(ld_stage) : stage_buf(ld_stage);
        const int tok_nx = t0 + (it + 1) * T;
        const bool qk_next = VISIBLE || (active && has_next && tok_nx < limit);    // scores of stage it+1
        if (qk_next) {
          if (do_load && !kIssueNow) qk(stage_buf(it + 1), WithLoads{}, ldst);
          else qk(stage_buf(it + 1), NoLoads{}, nullptr);
        } else if (do_load && !kIssueNow) {
#pragma unroll
          for (int cg = 0; cg < (FP8 ? FP8_LOADS_PER_STAGE : CGROUPS); ++cg) ld.issue_cg(cg, ldst, wave);
        }
        lds_barrier();   // weights of stage it visible to all waves
        const unsigned char* sb = stage_buf(it);
        mt = -INFINITY;
        psum[0] = psum[1] = 0.f;
        pv_stage(sb, visible_tag, qk_next ? lane_lim(tok_nx) : INT_MIN);
        l_run += psum[0] + psum[1];
        if constexpr (FP8) {
          // stage it+2 into the buffer of stage it (this wave's tile is done)
          if (it + 2 < nst) convert_stage(it + 2, it + 1 + NRAW < nst - 1 ? it + 1 + NRAW : nst - 1);
        }
      };
      // Iterations whose next stage is entirely visible (stage it+1 ends at or
      // before the limit) take the unmasked schedule; every wave runs the same
      // number of iterations, so the barriers inside stay matched.
      int it_vis = active ? (limit - t0) / T - 1 : 0;   // iterations it < it_vis are visible
      it_vis = it_vis < 0 ? 0 : (it_vis > nst ? nst : it_vis);
      int it = 0;
      for (; it < it_vis; ++it) iteration(it, Visible{});
      for (; it < nst; ++it) iteration(it, Masked{});
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
    // o[mb][hb][i] = u[row grow0 + 32 hb + l32][latent 128 wave + 32 mb + 8 (i/4) + 4 h + i%4].
    // Stored straight from the registers, an instruction would touch 32 rows
    // with 32 bytes each (one L2 request per run).  Instead, per head block hb,
    // each wave puts its 32 rows x 128 latents (16 KiB: row r at 512 r,
    // 16-byte chunk c at c ^ r) in the stage memory (the ring; the two bf16
    // stages over an fp8 cache) and stores them back as 2 rows of 512
    // contiguous bytes per instruction.
    lds_barrier();   // every wave is done with the ring
    // (lane offsets from an opaque copy of the lane index: the compiler cannot
    // hoist them out of the segment, where they would stay live through the
    // stage loop)
    int lane_o;
    asm volatile("v_mov_b32 %0, %1" : "=v"(lane_o) : "v"(lane));
    const int ol32 = lane_o & 31, oh = (lane_o >> 5) & 1;
    unsigned char* ob = &sm->stage[0][0] + 16384 * wave;
    static_assert(4 * 16384 <= (int)sizeof(sm->stage), "the staging blocks fit in the stage memory");
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int c = 8 * mb + 2 * i4 + oh;
          *reinterpret_cast<f32x4*>(ob + 512 * ol32 + ((c ^ ol32) << 4)) =
              f32x4{o[mb][hb][4 * i4], o[mb][hb][4 * i4 + 1], o[mb][hb][4 * i4 + 2], o[mb][hb][4 * i4 + 3]};
          __builtin_amdgcn_sched_barrier(0);   // accumulator reads one block at a time
        }
      // this wave's block is in (only this wave reads it; the clobber keeps
      // the reads below the writes and the next block's writes below the reads)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // instruction it stores rows 2 it + oh of the block, 16 bytes per lane;
      // the 16 reads go out together, then the stores (one read at a time,
      // each store waited for its read's full latency)
      float* const ub = a.u_part + ((int64_t)slot * rows + grow0 + 32 * hb) * DC + 128 * wave;
      const int lo = oh * DC + 4 * ol32;
      f32x4 v[16];
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int rr = 2 * it + oh;
        v[it] = *reinterpret_cast<const f32x4*>(ob + 512 * rr + ((ol32 ^ rr) << 4));
      }
#pragma unroll
      for (int it = 0; it < 16; ++it) {
        const int rr = 2 * it + oh;
        if (grow0 + 32 * hb + rr < rows) *reinterpret_cast<f32x4*>(ub + 2 * DC * it + lo) = v[it];
      }
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    // (the segment walker's barrier after this call keeps the ring and the
    // exchange buffers until every wave is done with them)
  };
  using Contig = std::integral_constant<int, kContiguous>;
  using Paged = std::integral_constant<int, kPaged>;
  using Any = std::integral_constant<int, kAnyLayout>;
  for_each_segment<NT>(a.ctx_lens, a.B, a.num_splits, w, &sm->plan, [&](int b, int t0, int t1, int slot) {
    // (a range the descriptor cannot place is taken as empty: its partial is
    // u = 0, lse = -inf, and no row of it is read)
    if constexpr (LAYOUT == kContiguous) {
      segment(Contig{}, b, t0, t1, slot, 0);
    } else if constexpr (LAYOUT == kPaged) {
      int blk_lo = 0;
      const int span = paged_span(a.cache, b, t0, t1, lane, FP8 ? RB8 : RB16, &blk_lo);
      // one call site per layout: a second inlined copy of the segment body
      // costs the whole kernel registers (spills in the stage loop)
      if (span == kSpanNear) segment(Paged{}, b, t0, t1, slot, blk_lo);
      else segment(Any{}, b, t0, span == kSpanFar ? t1 : t0, slot, 0);   // blocks 4 GiB or more apart
    } else {
      const bool placed = segment_rows_placed(a.cache, b, t0, t1, lane);
      segment(Any{}, b, t0, placed ? t1 : t0, slot, 0);
    }
  });
}

}  // namespace

int decode_mfma_smem_bytes(bool fp8) { return fp8 ? (int)sizeof(DecodeSmemFp8) : (int)sizeof(DecodeSmem); }

template <bool FP8>
static void launch_decode_layout(const DecodeArgs& a, const DecodeParams& p, int grid, hipStream_t stream) {
  const int64_t rb = FP8 ? RB8 : RB16;
  const int64_t stride_bytes = p.cache.seq_stride * (FP8 ? 1 : 2);
  // buffer offsets are 32-bit: a sequence plus one stage of overrun must fit
  if (p.cache.block_size == 0 && stride_bytes + (int64_t)T * rb <= (int64_t)0xFFFFFFFF)
    hipLaunchKernelGGL((decode_mfma_kernel<kContiguous, FP8>), dim3(grid), dim3(NT), 0, stream, a);
  else if (p.cache.block_size % T == 0)
    hipLaunchKernelGGL((decode_mfma_kernel<kPaged, FP8>), dim3(grid), dim3(NT), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<kAnyLayout, FP8>), dim3(grid), dim3(NT), 0, stream, a);
}

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
  if (p.fp8) launch_decode_layout<true>(a, p, grid, stream);
  else launch_decode_layout<false>(a, p, grid, stream);
  return hipGetLastError();
}

}  // namespace mla
