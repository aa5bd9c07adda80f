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
// The tokens of all sequences, in order, are cut into ranges of Q tokens
// (Q = ceil(total / num_splits)); range w is work unit w.  Sequence b (prefix
// P_b, length L_b > 0) meets work units P_b / Q .. (P_b + L_b - 1) / Q and owns
// that many consecutive partial slots starting at slot_base(b), the sum of the
// counts of the sequences before it.
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

// Calls f(b, t0, t1, slot) for every segment of work unit w: the tokens
// t0..t1-1 of sequence b that fall into the unit, and the partial slot they
// own.  Segments come in sequence order.  All NT threads of the workgroup
// must call this together; f is called uniformly.
template <int NT, typename F>
__device__ void for_each_segment(const int32_t* __restrict__ ctx_lens, int B, int num_splits, int w,
                                 PlanScratch<NT>* sc, F&& f) {
  const int tid = threadIdx.x;
  int64_t part = 0;
  for (int b = tid; b < B; b += NT) part += ctx_lens[b];
  int64_t total;
  block_scan_incl<NT>(part, sc->scan, &total);
  const int64_t q = plan_chunk(total, num_splits);
  const int64_t a = (int64_t)w * q;
  const int64_t e = a + q < total ? a + q : total;
  if (a >= e) return;
  int64_t run = 0, slot_run = 0;
  for (int c0 = 0; c0 < B; c0 += NT) {
    const int b = c0 + tid;
    const int64_t len = b < B ? ctx_lens[b] : 0;
    int64_t tot_len, tot_np;
    const int64_t p = run + block_scan_incl<NT>(len, sc->scan, &tot_len) - len;
    const int64_t np = plan_parts(p, len, q);
    const int64_t sb = slot_run + block_scan_incl<NT>(np, sc->scan, &tot_np) - np;
    if (tid == 0) { sc->first = NT; sc->last = -1; }
    __syncthreads();
    const bool hit = len > 0 && p < e && p + len > a;
    sc->prefix[tid] = p;
    sc->len[tid] = (int32_t)len;
    sc->slot[tid] = (int32_t)(sb + (w - p / q));
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
    slot_run += tot_np;
    if (run >= e) break;
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
  int64_t part = len_tid;
  for (int k = tid + NT; k < B; k += NT) part += ctx_lens[k];
  int64_t total;
  block_scan_incl<NT>(part, sc->scan, &total);
  const int64_t q = plan_chunk(total, num_splits);
  int64_t run = 0, slot_run = 0;
  for (int c0 = 0; c0 < b_lo + n; c0 += NT) {
    const int k = c0 + tid;
    const int64_t len = c0 == 0 ? len_tid : (k < B ? ctx_lens[k] : 0);
    int64_t tot_len, tot_np;
    const int64_t p = run + block_scan_incl<NT>(len, sc->scan, &tot_len) - len;
    const int64_t np = plan_parts(p, len, q);
    const int64_t sb = slot_run + block_scan_incl<NT>(np, sc->scan, &tot_np) - np;
    if (k >= b_lo && k < b_lo + n) { slot0[k - b_lo] = (int32_t)sb; nparts[k - b_lo] = (int32_t)np; }
    run += tot_len;
    slot_run += tot_np;
  }
  lds_sync();
}

// For sequence b: first partial slot and number of partials (0 if empty).
template <int NT>
__device__ void plan_lookup(const int32_t* __restrict__ ctx_lens, int B, int num_splits, int b,
                            PlanScratch<NT>* sc, int* slot_base, int* n_parts) {
  const int tid = threadIdx.x;
  int64_t part = 0;
  for (int k = tid; k < B; k += NT) part += ctx_lens[k];
  int64_t total;
  block_scan_incl<NT>(part, sc->scan, &total);
  const int64_t q = plan_chunk(total, num_splits);
  int64_t run = 0, slot_run = 0;
  for (int c0 = 0; c0 <= b; c0 += NT) {
    const int k = c0 + tid;
    const int64_t len = k < B ? ctx_lens[k] : 0;
    int64_t tot_len, tot_np;
    const int64_t p = run + block_scan_incl<NT>(len, sc->scan, &tot_len) - len;
    const int64_t np = plan_parts(p, len, q);
    const int64_t sb = slot_run + block_scan_incl<NT>(np, sc->scan, &tot_np) - np;
    if (k == b) { sc->slot[0] = (int32_t)sb; sc->len[0] = (int32_t)np; }
    run += tot_len;
    slot_run += tot_np;
  }
  __syncthreads();
  *slot_base = sc->slot[0];
  *n_parts = sc->len[0];
  __syncthreads();
}

}  // namespace mla
