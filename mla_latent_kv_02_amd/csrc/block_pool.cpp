// Block pool of a paged latent cache ([Paldyn] = "MQA와 GQA: KV 캐시 경량화
// 전략", ailab.paldyn.com, section "PagedAttention과 연속 배칭": the cache is
// cut into small fixed-size blocks that a sequence takes as it grows, and the
// blocks of a finished sequence go straight back to the free list for the next
// one).  Host code only: it decides which physical block holds which tokens and
// keeps the block table in host memory; the caller copies the table to the
// device buffer that mla_cache_t.block_table points at.
//
// The pool lives entirely in memory the caller provides (int32 words):
//   [0..7]                 header: magic, n_blocks, block_size, B, max_blocks, n_free, 0, 0
//   [8 .. 8+n_blocks)      free stack; the next block handed out is free[n_free - 1]
//   [.. + B)               blocks held by each sequence
//   [.. + B*max_blocks)    block table [B][max_blocks], -1 past a sequence's blocks
#include <stdint.h>

#include "../../include/mla.h"

namespace {

constexpr int32_t kMagic = 0x4d4c4250;   // "MLBP"
constexpr int kHeader = 8;

struct View {
  int32_t* w;
  int32_t& n_blocks() { return w[1]; }
  int32_t& block_size() { return w[2]; }
  int32_t& B() { return w[3]; }
  int32_t& max_blocks() { return w[4]; }
  int32_t& n_free() { return w[5]; }
  int32_t* free_stack() { return w + kHeader; }
  int32_t* held() { return w + kHeader + n_blocks(); }
  int32_t* table() { return held() + B(); }
};

bool view_of(void* pool, View* v) {
  if (!pool || reinterpret_cast<uintptr_t>(pool) % 4) return false;
  v->w = static_cast<int32_t*>(pool);
  return v->w[0] == kMagic;
}

}  // namespace

extern "C" {

int64_t mla_block_pool_bytes(int32_t n_blocks, int32_t B, int32_t max_blocks) {
  if (n_blocks < 0 || B < 0 || max_blocks < 1) return -1;
  return 4 * ((int64_t)kHeader + n_blocks + B + (int64_t)B * max_blocks);
}

mla_status_t mla_block_pool_init(void* pool, int64_t bytes, int32_t n_blocks, int32_t block_size, int32_t B,
                                 int32_t max_blocks) {
  const int64_t need = mla_block_pool_bytes(n_blocks, B, max_blocks);
  if (!pool || reinterpret_cast<uintptr_t>(pool) % 4 || block_size < 1 || need < 0 || bytes < need)
    return MLA_ERR_INVALID_ARG;
  View v{static_cast<int32_t*>(pool)};
  v.w[0] = kMagic;
  v.n_blocks() = n_blocks;
  v.block_size() = block_size;
  v.B() = B;
  v.max_blocks() = max_blocks;
  v.n_free() = n_blocks;
  v.w[6] = v.w[7] = 0;
  for (int32_t i = 0; i < n_blocks; ++i) v.free_stack()[i] = n_blocks - 1 - i;   // block 0 first
  for (int32_t b = 0; b < B; ++b) v.held()[b] = 0;
  for (int64_t i = 0; i < (int64_t)B * max_blocks; ++i) v.table()[i] = -1;
  return MLA_OK;
}

mla_status_t mla_block_pool_reserve(void* pool, int32_t b, int32_t n_tokens) {
  View v;
  if (!view_of(pool, &v) || b < 0 || b >= v.B() || n_tokens < 0) return MLA_ERR_INVALID_ARG;
  const int64_t need = ((int64_t)n_tokens + v.block_size() - 1) / v.block_size();
  if (need > v.max_blocks()) return MLA_ERR_INVALID_ARG;
  const int32_t have = v.held()[b];
  if (need <= have) return MLA_OK;
  if (need - have > v.n_free()) return MLA_ERR_OUT_OF_BLOCKS;   // nothing taken
  int32_t* row = v.table() + (int64_t)b * v.max_blocks();
  for (int32_t k = have; k < need; ++k) row[k] = v.free_stack()[--v.n_free()];
  v.held()[b] = (int32_t)need;
  return MLA_OK;
}

mla_status_t mla_block_pool_reserve_all(void* pool, const int32_t* n_tokens) {
  View v;
  if (!view_of(pool, &v) || !n_tokens) return MLA_ERR_INVALID_ARG;
  int64_t extra = 0;
  for (int32_t b = 0; b < v.B(); ++b) {
    if (n_tokens[b] < 0) continue;
    const int64_t need = ((int64_t)n_tokens[b] + v.block_size() - 1) / v.block_size();
    if (need > v.max_blocks()) return MLA_ERR_INVALID_ARG;
    if (need > v.held()[b]) extra += need - v.held()[b];
  }
  if (extra > v.n_free()) return MLA_ERR_OUT_OF_BLOCKS;   // nothing taken
  for (int32_t b = 0; b < v.B(); ++b)
    if (n_tokens[b] >= 0) mla_block_pool_reserve(pool, b, n_tokens[b]);
  return MLA_OK;
}

mla_status_t mla_block_pool_release(void* pool, int32_t b) {
  View v;
  if (!view_of(pool, &v) || b < 0 || b >= v.B()) return MLA_ERR_INVALID_ARG;
  int32_t* row = v.table() + (int64_t)b * v.max_blocks();
  for (int32_t k = v.held()[b] - 1; k >= 0; --k) {   // the last block taken is the next handed out
    v.free_stack()[v.n_free()++] = row[k];
    row[k] = -1;
  }
  v.held()[b] = 0;
  return MLA_OK;
}

const int32_t* mla_block_pool_table(const void* pool) {
  View v;
  if (!view_of(const_cast<void*>(pool), &v)) return nullptr;
  return v.table();
}

int32_t mla_block_pool_free_count(const void* pool) {
  View v;
  if (!view_of(const_cast<void*>(pool), &v)) return -1;
  return v.n_free();
}

}  // extern "C"
