// Streaming-rate probes for the bench (bench.py --stream-probe-mib): how fast
// this chip reads HBM at all, the reference the decode kernel's rates are set
// against.  Timing only; nothing here computes anything of the method.
//
//   probe_stream_read: each of 256 workgroups (4 waves) reads its contiguous
//     share of a buffer with 16-byte loads, 8 in flight per lane, plain or
//     non-temporal.
//   probe_stream_rows: the decode kernel's load schedule with its work taken
//     out: rows of 1152 bytes in blocks of 64 rows (72 KiB) taken in the order
//     of a block table, 32-row stages of 36 KiB loaded global->LDS into a ring
//     of 4 (wave w reads rows 8w..8w+7 of a stage, 128 contiguous bytes per 8
//     lanes), three stages issued ahead, two workgroup barriers per stage.
//
// Every address stays inside the buffer: block ids are taken modulo the
// block count, reads past a share are masked.  LDS slots are in bounds by
// construction.

#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRowBytes = 1152, kBlockRows = 64, kStageRows = 32;
constexpr int kStageBytes = kStageRows * kRowBytes;   // 36 KiB
constexpr int kBlockBytes = kBlockRows * kRowBytes;   // 72 KiB

template <bool NT>
__global__ __launch_bounds__(256, 1) void read_kernel(const u32x4* __restrict__ src, int64_t n16, int64_t per_wg,
                                                      unsigned* sink) {
  const int64_t lo = (int64_t)blockIdx.x * per_wg;
  const int64_t hi = lo + per_wg < n16 ? lo + per_wg : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t i = lo + threadIdx.x; i < hi; i += 256 * 8) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t j = i + 256 * u;
      v[u] = j < hi ? (NT ? __builtin_nontemporal_load(src + j) : src[j]) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  if (acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u) sink[threadIdx.x] = acc[2];   // keeps the loads
}

// workgroup barrier that waits for LDS operations only (a full __syncthreads
// would also wait for the stage loads in flight)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <bool NT>
__global__ __launch_bounds__(256, 1) void rows_kernel(const unsigned char* __restrict__ src,
                                                      const int32_t* __restrict__ blocks, int32_t n_blocks,
                                                      int32_t stages_per_wg, unsigned* sink) {
  __shared__ __attribute__((aligned(16))) unsigned char ring[4][kStageBytes];
  const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int64_t first = (int64_t)blockIdx.x * stages_per_wg;
  const int row = 8 * wave + (lane >> 3);
  auto issue = [&](int s) {
    const int64_t gs = first + s;
    int32_t blk = blocks[(gs >> 1) % n_blocks] % n_blocks;
    blk = blk < 0 ? blk + n_blocks : blk;
    const unsigned char* p = src + (int64_t)blk * kBlockBytes + (gs & 1) * kStageBytes + row * kRowBytes +
                             (lane & 7) * 16;
    unsigned char* d = ring[s & 3] + wave * 1024;
#pragma unroll
    for (int i = 0; i < 9; ++i)
      __builtin_amdgcn_global_load_lds(p + i * 128, (lds_void*)(d + i * 4096), 16, 0, NT ? 2 : 0);
  };
  const int nst = stages_per_wg;
  for (int s = 0; s < 3 && s < nst; ++s) issue(s);
  unsigned acc = 0;
  for (int it = 0; it < nst; ++it) {
    // stage it resident (the decode waits one iteration earlier, for it+1)
    if (it + 2 < nst) __builtin_amdgcn_s_waitcnt(0x4F72);        // vmcnt(18)
    else if (it + 1 < nst) __builtin_amdgcn_s_waitcnt(0x0F79);   // vmcnt(9)
    else __builtin_amdgcn_s_waitcnt(0x0F70);                     // vmcnt(0)
    lds_barrier();
    if (it + 3 < nst) issue(it + 3);
    acc += *(volatile __attribute__((address_space(3))) unsigned*)(
        (__attribute__((address_space(3))) unsigned char*)(ring[it & 3] + 4 * t));
    lds_barrier();
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  if (acc == 0x12345679u) sink[t] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16) at `src`, plain or non-temporal.  `sink`:
// 256 unsigned of device memory (written only for one impossible checksum).
extern "C" int probe_stream_read(const void* src, int64_t bytes, int32_t nontemporal, void* sink, void* stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16) return 1;
  const int64_t n16 = bytes / 16;
  const int64_t per_wg = (n16 + 255) / 256;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nontemporal)
    read_kernel<true><<<256, 256, 0, s>>>(static_cast<const u32x4*>(src), n16, per_wg, static_cast<unsigned*>(sink));
  else
    read_kernel<false><<<256, 256, 0, s>>>(static_cast<const u32x4*>(src), n16, per_wg, static_cast<unsigned*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// Streams n_blocks blocks of 64 rows x 1152 bytes at `src` (n_blocks * 73728
// bytes) in the order of `blocks` (n_blocks device int32), over 256
// workgroups: n_blocks * 2 must be a multiple of 256.
extern "C" int probe_stream_rows(const void* src, const int32_t* blocks, int32_t n_blocks, int32_t nontemporal,
                                 void* sink, void* stream) {
  if (!src || !blocks || !sink || n_blocks <= 0 || (2 * (int64_t)n_blocks) % 256) return 1;
  const int32_t stages_per_wg = (int32_t)(2 * (int64_t)n_blocks / 256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned char* p = static_cast<const unsigned char*>(src);
  if (nontemporal)
    rows_kernel<true><<<256, 256, 0, s>>>(p, blocks, n_blocks, stages_per_wg, static_cast<unsigned*>(sink));
  else
    rows_kernel<false><<<256, 256, 0, s>>>(p, blocks, n_blocks, stages_per_wg, static_cast<unsigned*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
