// Split-KV combine: log-sum-exp merge of the per-work-unit partials of each
// sequence.  Partial k of a query row holds u_k = sum_t exp(s_t - r_k) c_t
// over its token range, its reference r_k and lse_k = log sum_t exp(s_t).
// With L = log sum_k exp(lse_k), the merged value sum is
// sum_k exp(r_k - L) u_k -- the softmax over the union of the ranges.
//
// One wave per query row; lanes cover the latent dimension with 16-byte
// loads, so each partial row (d_c floats) is read once, coalesced.

#include "mla_device.h"
#include "launch.h"

namespace mla {
namespace {

constexpr int NT = 256;

__global__ __launch_bounds__(NT) void combine_kernel(CombineParams p) {
  __shared__ PlanScratch<NT> plan;
  const int b = blockIdx.y;
  int slot0, nparts;
  plan_lookup<NT>(p.ctx_lens, p.B, p.num_splits, b, &plan, &slot0, &nparts);
  const int lane = threadIdx.x & 63;
  const int rows = p.n_q * p.n_h;
  const int r = blockIdx.x * (NT / 64) + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int64_t stride_rows = rows;   // partial slot stride, in rows

  const float2* lp = reinterpret_cast<const float2*>(p.lse_part);   // (r_k, lse_k)
  float m = -INFINITY;
  for (int k = lane; k < nparts; k += 64) m = fmaxf(m, lp[(int64_t)(slot0 + k) * stride_rows + r].y);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
  float s = 0.f;
  if (m != -INFINITY)
    for (int k = lane; k < nparts; k += 64) s += expf(lp[(int64_t)(slot0 + k) * stride_rows + r].y - m);
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
  const float L = m != -INFINITY ? m + logf(s) : -INFINITY;

  const int64_t orow = (int64_t)b * rows + r;
  float* uo = p.u + orow * p.d_c;
  for (int c4 = lane; c4 < p.d_c / 4; c4 += 64) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (m != -INFINITY) {
      for (int k = 0; k < nparts; ++k) {
        const int64_t prow = (int64_t)(slot0 + k) * stride_rows + r;
        const float2 rl = lp[prow];
        if (rl.y == -INFINITY) continue;
        const float wk = expf(rl.x - L);
        acc += wk * reinterpret_cast<const f32x4*>(p.u_part + prow * p.d_c)[c4];
      }
    }
    reinterpret_cast<f32x4*>(uo)[c4] = acc;
  }
  if (p.lse && lane == 0) p.lse[orow] = L;
}

}  // namespace

hipError_t launch_combine(const CombineParams& p, hipStream_t stream) {
  const int rows = p.n_q * p.n_h;
  dim3 grid((rows + NT / 64 - 1) / (NT / 64), p.B);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(NT), 0, stream, p);
  return hipGetLastError();
}

}  // namespace mla
