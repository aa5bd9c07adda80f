// Device-side helpers shared by the gfx950 kernels of the MLA decode library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------ bf16 <-> fp32
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ __forceinline__ static void store(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// ------------------------------------------------------------------- RoPE
// sin and cos of the angle pos * theta, given turns = theta / (2 pi): the angle
// in turns and its reduction to [-1/2, 1/2] are fp64; the sine and cosine of
// the reduced angle use the fp32 hardware instructions, which take turns.
// Accurate to ~1e-6 absolute, far below the bf16 resolution of the outputs
// that use it.
__device__ __forceinline__ void sincos_turns(int pos, double turns, float* s, float* c) {
  const double v = (double)pos * turns;
  const float f = (float)(v - rint(v));
  *s = __builtin_amdgcn_sinf(f);
  *c = __builtin_amdgcn_cosf(f);
}
constexpr double kInv2Pi = 0.15915494309189535;

// --------------------------------------------------------- cache addressing
struct CacheView {
  const void* data;
  int64_t seq_stride;        // elements (contiguous)
  const int32_t* block_table;
  int32_t block_size;        // 0 = contiguous
  int32_t max_blocks;
  int32_t row;               // elements per token row (d_c + d_rope)
};

// Element offset of the row of token t of sequence b.
__device__ __forceinline__ int64_t cache_row_offset(const CacheView& c, int b, int t) {
  if (c.block_size == 0) return (int64_t)b * c.seq_stride + (int64_t)t * c.row;
  const int blk = c.block_table[(int64_t)b * c.max_blocks + t / c.block_size];
  return ((int64_t)blk * c.block_size + (t % c.block_size)) * (int64_t)c.row;
}

// As cache_row_offset, or -1 where the descriptor cannot place the row: a
// negative position, or (paged) a block past the table row or a negative
// block id (a block the caller has not reserved).
__device__ __forceinline__ int64_t cache_row_offset_checked(const CacheView& c, int b, int t) {
  if (t < 0) return -1;
  if (c.block_size == 0) return (int64_t)b * c.seq_stride + (int64_t)t * c.row;
  const int k = t / c.block_size;
  if (k >= c.max_blocks) return -1;
  const int blk = c.block_table[(int64_t)b * c.max_blocks + k];
  if (blk < 0) return -1;
  return ((int64_t)blk * c.block_size + (t % c.block_size)) * (int64_t)c.row;
}

// Whether every row of tokens t0..t1-1 (t0 < t1) of sequence b is placed by a
// paged descriptor: the range's blocks lie within the table row and none of
// their ids is negative.  The lanes of the calling wave read the table row
// together; the result is the same in every lane (and in every wave that
// asks).  Contiguous caches: true.
__device__ __forceinline__ bool segment_rows_placed(const CacheView& c, int b, int t0, int t1, int lane) {
  if (c.block_size == 0) return true;
  const int k0 = t0 / c.block_size, k1 = (t1 - 1) / c.block_size;
  if (k1 >= c.max_blocks) return false;
  int bad = 0;
  for (int k = k0 + lane; k <= k1; k += 64) bad |= c.block_table[(int64_t)b * c.max_blocks + k] < 0;
  return __builtin_amdgcn_ballot_w64(bad != 0) == 0;
}

// ------------------------------------------------------ split-KV work plan
// Work units are equal ranges of a cost line on which the tokens of all
// sequences lie in order (U = num_splits, T = the sum of the lengths):
//   - the token cut q0 = ceil(T / U) marks where a plain token split would
//     cut; sequence b (token prefix P_b, length L_b > 0) starts inside a unit
//     when P_b is not a multiple of q0 (f_b = 1);
//   - such a start costs the unit that meets it a second segment (query rows,
//     pipeline start, one more partial written), counted as kSegmentCost
//     tokens placed in front of the sequence's tokens: b's tokens occupy cost
//     positions C_b .. C_b + L_b - 1, C_b = P_b + kSegmentCost * sum_{b' <= b} f_b';
//   - unit w covers cost positions [w Q, (w + 1) Q), Q = ceil((T + kSegmentCost E) / U)
//     with E = sum_b f_b.
// Sequence b meets units C_b / Q .. (C_b + L_b - 1) / Q and owns that many
// consecutive partial slots starting at the sum of the counts of the
// sequences before it.  When every sequence starts on a multiple of q0, E = 0
// and this is the plain token split.
constexpr int64_t kSegmentCost = 288;

__device__ __forceinline__ int64_t plan_chunk(int64_t total, int num_splits) {
  int64_t q = (total + num_splits - 1) / num_splits;
  return q > 0 ? q : 1;
}
__device__ __forceinline__ int plan_parts(int64_t prefix, int64_t len, int64_t q) {
  return len > 0 ? (int)((prefix + len - 1) / q - prefix / q + 1) : 0;
}

// Workgroup barrier for data exchanged through LDS only: waits for this
// wave's LDS operations, not for its outstanding global loads (which
// __syncthreads() also waits for, draining whatever is in flight).
__device__ __forceinline__ void lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Inclusive scan of one int64 per thread over a workgroup of NT threads
// (NT a multiple of 64).  `scratch` holds NT/64 + 1 int64 values.  Returns the
// inclusive prefix; *total receives the workgroup sum.
template <int NT>
__device__ __forceinline__ int64_t block_scan_incl(int64_t v, int64_t* scratch, int64_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int64_t o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  if (lane == 63) scratch[wave] = v;
  lds_sync();
  if (threadIdx.x == 0) {
    int64_t run = 0;
    for (int w = 0; w < NT / 64; ++w) { int64_t s = scratch[w]; scratch[w] = run; run += s; }
    scratch[NT / 64] = run;
  }
  lds_sync();
  v += scratch[wave];
  *total = scratch[NT / 64];
  lds_sync();
  return v;
}

}  // namespace mla

namespace mla {

// LDS scratch used by the workgroup-level plan walk.
template <int NT>
struct PlanScratch {
  int64_t scan[NT / 64 + 1];
  int64_t prefix[NT];
  int32_t len[NT];
  int32_t slot[NT];
  int32_t first, last;
};

// Positions of one chunk of NT sequences on the cost line (this thread's
// sequence has length len; run and frun are the token count and the number
// of inside starts of the sequences before the chunk): *p = P_b, *cp = C_b;
// *tot_len and *tot_f receive the chunk's sums.
template <int NT>
__device__ __forceinline__ void plan_positions(int64_t len, int64_t run, int64_t frun, int64_t q0, int64_t* scan,
                                               int64_t* p, int64_t* cp, int64_t* tot_len, int64_t* tot_f) {
  *p = run + block_scan_incl<NT>(len, scan, tot_len) - len;
  const int64_t f = len > 0 && *p % q0 != 0 ? 1 : 0;
  *cp = *p + kSegmentCost * (frun + block_scan_incl<NT>(f, scan, tot_f));
}

// The plan's token cut q0, unit width Q and cost-line length, and the
// positions of the first chunk of NT sequences (this thread's C_b and the
// chunk's sums), which the walks below reuse.  len0 is ctx_lens[threadIdx.x]
// (0 past B), loaded by the caller.  All NT threads must call this together.
struct PlanGeometry {
  int64_t q0, Q, cost_total;
  int64_t cp0, tot_len0, tot_f0;
};
template <int NT>
__device__ void plan_geometry(const int32_t* __restrict__ ctx_lens, int B, int num_splits, int len0,
                              PlanScratch<NT>* sc, PlanGeometry* g) {
  const int tid = threadIdx.x;
  const int64_t p0 = block_scan_incl<NT>((int64_t)len0, sc->scan, &g->tot_len0) - len0;
  int64_t total = g->tot_len0;
  if (B > NT) {   // the token total needs the other chunks too
    int64_t part = 0, rest;
    for (int b = tid + NT; b < B; b += NT) part += ctx_lens[b];
    block_scan_incl<NT>(part, sc->scan, &rest);
    total += rest;
  }
  g->q0 = plan_chunk(total, num_splits);
  const int64_t f0 = len0 > 0 && p0 % g->q0 != 0 ? 1 : 0;
  g->cp0 = p0 + kSegmentCost * block_scan_incl<NT>(f0, sc->scan, &g->tot_f0);
  int64_t run = g->tot_len0, frun = g->tot_f0;
  for (int c0 = NT; c0 < B; c0 += NT) {
    const int b = c0 + tid;
    const int64_t len = b < B ? ctx_lens[b] : 0;
    int64_t p, cp, tot_len, tot_f;
    plan_positions<NT>(len, run, frun, g->q0, sc->scan, &p, &cp, &tot_len, &tot_f);
    run += tot_len;
    frun += tot_f;
  }
  g->cost_total = total + kSegmentCost * frun;
  g->Q = plan_chunk(g->cost_total, num_splits);
}

// C_b of this thread's sequence in the chunk starting at c0, and the chunk's sums.
template <int NT>
__device__ __forceinline__ void plan_chunk_positions(const PlanGeometry& g, int c0, int64_t len, int64_t run,
                                                     int64_t frun, int64_t* scan, int64_t* cp, int64_t* tot_len,
                                                     int64_t* tot_f) {
  if (c0 == 0) {
    *cp = g.cp0;
    *tot_len = g.tot_len0;
    *tot_f = g.tot_f0;
  } else {
    int64_t p;
    plan_positions<NT>(len, run, frun, g.q0, scan, &p, cp, tot_len, tot_f);
  }
}

// Calls f(b, t0, t1, slot) for every segment of work unit w: the tokens
// t0..t1-1 of sequence b that fall into the unit, and the partial slot they
// own.  Segments come in sequence order.  All NT threads of the workgroup
// must call this together; f is called uniformly.
template <int NT, typename F>
__device__ void for_each_segment(const int32_t* __restrict__ ctx_lens, int B, int num_splits, int w,
                                 PlanScratch<NT>* sc, F&& f) {
  const int tid = threadIdx.x;
  const int len0 = tid < B ? ctx_lens[tid] : 0;
  PlanGeometry g;
  plan_geometry<NT>(ctx_lens, B, num_splits, len0, sc, &g);
  const int64_t q = g.Q;
  const int64_t a = (int64_t)w * q;
  const int64_t e = a + q < g.cost_total ? a + q : g.cost_total;
  if (a >= e) return;
  int64_t run = 0, frun = 0, slot_run = 0;
  for (int c0 = 0; c0 < B; c0 += NT) {
    const int b = c0 + tid;
    const int64_t len = c0 == 0 ? len0 : (b < B ? ctx_lens[b] : 0);
    int64_t cp, tot_len, tot_f, tot_np;
    plan_chunk_positions<NT>(g, c0, len, run, frun, sc->scan, &cp, &tot_len, &tot_f);
    const int64_t np = plan_parts(cp, len, q);
    const int64_t sb = slot_run + block_scan_incl<NT>(np, sc->scan, &tot_np) - np;
    if (tid == 0) { sc->first = NT; sc->last = -1; }
    __syncthreads();
    const bool hit = len > 0 && cp < e && cp + len > a;
    sc->prefix[tid] = cp;
    sc->len[tid] = (int32_t)len;
    sc->slot[tid] = (int32_t)(sb + (w - cp / q));
    if (hit) { atomicMin(&sc->first, tid); atomicMax(&sc->last, tid); }
    __syncthreads();
    // the segment values are the same in every lane: keep them in scalar
    // registers so that everything derived from them stays scalar too
    const int first = __builtin_amdgcn_readfirstlane(sc->first);
    const int last = __builtin_amdgcn_readfirstlane(sc->last);
    for (int k = first; k <= last; ++k) {
      const int64_t pk = sc->prefix[k];
      const int64_t lo = a > pk ? a : pk;
      const int64_t hi = e < pk + sc->len[k] ? e : pk + sc->len[k];
      const int t0 = __builtin_amdgcn_readfirstlane((int)(lo - pk));
      const int t1 = __builtin_amdgcn_readfirstlane((int)(hi - pk));
      const int slot = __builtin_amdgcn_readfirstlane(sc->slot[k]);
      // LDS-only barrier: the plan scratch is read; global stores of the
      // previous segment may still be in flight
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      f(c0 + k, t0, t1, slot);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    run += tot_len;
    frun += tot_f;
    slot_run += tot_np;
    if (run + kSegmentCost * frun >= e) break;   // later sequences start at or past the unit's end
  }
}

// For the n (<= NT) sequences b_lo .. b_lo + n - 1: first partial slot and
// number of partials, written to slot0[] and nparts[] (n entries each, LDS).
// len_tid = ctx_lens[threadIdx.x] (0 for threadIdx.x >= B), loaded by the
// caller: issued before the caller's other global loads, the wait for it does
// not wait for them.  All NT threads of the workgroup must call this together.
template <int NT>
__device__ void plan_slot_range(const int32_t* __restrict__ ctx_lens, int B, int num_splits, int b_lo, int n,
                                int len_tid, PlanScratch<NT>* sc, int* slot0, int* nparts) {
  const int tid = threadIdx.x;
  PlanGeometry g;
  plan_geometry<NT>(ctx_lens, B, num_splits, len_tid, sc, &g);
  int64_t run = 0, frun = 0, slot_run = 0;
  for (int c0 = 0; c0 < b_lo + n; c0 += NT) {
    const int k = c0 + tid;
    const int64_t len = c0 == 0 ? len_tid : (k < B ? ctx_lens[k] : 0);
    int64_t cp, tot_len, tot_f, tot_np;
    plan_chunk_positions<NT>(g, c0, len, run, frun, sc->scan, &cp, &tot_len, &tot_f);
    const int64_t np = plan_parts(cp, len, g.Q);
    const int64_t sb = slot_run + block_scan_incl<NT>(np, sc->scan, &tot_np) - np;
    if (k >= b_lo && k < b_lo + n) { slot0[k - b_lo] = (int32_t)sb; nparts[k - b_lo] = (int32_t)np; }
    run += tot_len;
    frun += tot_f;
    slot_run += tot_np;
  }
  lds_sync();
}

// For sequence b: first partial slot and number of partials (0 if empty).
template <int NT>
__device__ void plan_lookup(const int32_t* __restrict__ ctx_lens, int B, int num_splits, int b,
                            PlanScratch<NT>* sc, int* slot_base, int* n_parts) {
  const int tid = threadIdx.x;
  const int len0 = tid < B ? ctx_lens[tid] : 0;
  PlanGeometry g;
  plan_geometry<NT>(ctx_lens, B, num_splits, len0, sc, &g);
  int64_t run = 0, frun = 0, slot_run = 0;
  for (int c0 = 0; c0 <= b; c0 += NT) {
    const int k = c0 + tid;
    const int64_t len = c0 == 0 ? len0 : (k < B ? ctx_lens[k] : 0);
    int64_t cp, tot_len, tot_f, tot_np;
    plan_chunk_positions<NT>(g, c0, len, run, frun, sc->scan, &cp, &tot_len, &tot_f);
    const int64_t np = plan_parts(cp, len, g.Q);
    const int64_t sb = slot_run + block_scan_incl<NT>(np, sc->scan, &tot_np) - np;
    if (k == b) { sc->slot[0] = (int32_t)sb; sc->len[0] = (int32_t)np; }
    run += tot_len;
    frun += tot_f;
    slot_run += tot_np;
  }
  __syncthreads();
  *slot_base = sc->slot[0];
  *n_parts = sc->len[0];
  __syncthreads();
}

}  // namespace mla
