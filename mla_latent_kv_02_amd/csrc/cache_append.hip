// Latent-cache append kernels: one thread per element pair of a new row for
// fp32 and bf16 caches (the pair itself is written by append_pair), one wave
// per new row for fp8 caches (the row's tiles are quantised together).

#include "append_row.h"

namespace mla {
namespace {

constexpr int NT = 256;

// grid (n_tokens, ceil(row/2 / NT)); thread = one element pair of one row.
template <typename T>
__global__ __launch_bounds__(NT) void cache_append_kernel(AppendParams p) {
  const int k = blockIdx.x;
  const int pair = blockIdx.y * NT + threadIdx.x;
  if (2 * pair >= p.d_c + p.d_rope) return;
  append_pair<T>(p, k, pair);
}

// grid ceil(n / 4); one wave per new row (append_row_fp8).
__global__ __launch_bounds__(NT) void cache_append_fp8_kernel(AppendParams p) {
  const int k = blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
  if (k < p.n) append_row_fp8(p, k, threadIdx.x & 63);
}

}  // namespace

hipError_t launch_cache_append(const AppendParams& p, hipStream_t stream) {
  if (p.n == 0) return hipSuccess;
  if (p.fp8) {
    hipLaunchKernelGGL(cache_append_fp8_kernel, dim3((p.n + NT / 64 - 1) / (NT / 64)), dim3(NT), 0, stream, p);
    return hipGetLastError();
  }
  const int pairs = (p.d_c + p.d_rope) / 2;
  dim3 grid(p.n, (pairs + NT - 1) / NT);
  if (p.bf16)
    hipLaunchKernelGGL(cache_append_kernel<uint16_t>, grid, dim3(NT), 0, stream, p);
  else
    hipLaunchKernelGGL(cache_append_kernel<float>, grid, dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
