// Device implementation of the seeded synthetic-input generator in
// workloads/__init__.py: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel
// Random Numbers: As Easy as 1, 2, 3", SC'11) + a 65536-entry quantile table
// of the standard normal.  It holds no attention arithmetic; it only fills raw
// cache rows so that multi-gigabyte caches need not be built on the host.
// Row k of the output is element-for-element identical to
// workloads.cache_rows(w, seq_ids[k], tok[k], tok[k] + 1).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
  }
}

// grid (n_tokens, ceil(row/8 / 64)); thread = 8 consecutive elements of one row.
__global__ __launch_bounds__(64) void fill_rows_kernel(uint32_t seed, uint32_t stream, int row, int n,
                                                       const int32_t* seq_ids, const int32_t* tok,
                                                       const uint16_t* table, uint16_t* out) {
  const int k = blockIdx.x;
  const int blk = blockIdx.y * 64 + threadIdx.x;
  if (k >= n || blk * 8 >= row) return;
  uint32_t c[4] = {(uint32_t)blk, (uint32_t)tok[k], (uint32_t)seq_ids[k], 0u};
  philox4x32_10(c, seed, stream);
  uint16_t* dst = out + (int64_t)k * row + blk * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (blk * 8 + e >= row) break;
    const uint32_t word = c[e >> 1];
    const uint32_t lane = (e & 1) ? (word >> 16) : (word & 0xFFFFu);
    dst[e] = table[lane];
  }
}

}  // namespace

// Returns 0, -1 for an invalid argument, or the hipError_t of a failed launch
// (synth_error_name gives its name).
extern "C" int synth_fill_cache_rows(uint32_t seed, int32_t stream_id, int32_t row, int32_t n_tokens,
                                     const int32_t* seq_ids, const int32_t* tok, const uint16_t* table,
                                     uint16_t* out, void* stream) {
  if (n_tokens < 0 || row <= 0 || !seq_ids || !tok || !table || !out) return -1;
  if (n_tokens == 0) return 0;
  dim3 grid(n_tokens, (row / 8 + 63) / 64 + 1);
  hipLaunchKernelGGL(fill_rows_kernel, grid, dim3(64), 0, (hipStream_t)stream, seed, (uint32_t)stream_id,
                     row, n_tokens, seq_ids, tok, table, out);
  return (int)hipGetLastError();
}

extern "C" const char* synth_error_name(int code) { return hipGetErrorName((hipError_t)code); }
