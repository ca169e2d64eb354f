// cache_dev.h -- plan and launcher of the cache of selected rows (cache.hip).
#pragma once
#include "ckv_dev.h"

namespace ckv {

constexpr int kMaxCacheR = 8;
constexpr int kMaxCacheB = 4096;          // largest budget the cache plan holds in registers
struct CachePlan {
    int H, C, c_cap, n_sink, B, R, dtype, rows;
    int64_t L, token_base, t_cap, kv_head_stride, kv_rows;
    int32_t *src;             // workspace [H][rows]: source of every new slot
    int32_t *tot;             // workspace [H]: slots in use after the step
};
hipError_t launch_cache_step(const CachePlan &p, int64_t step, const int32_t *idx,
                             const int32_t *n_sel, const int32_t *assign,
                             const int32_t *offsets, const int32_t *tokens, const void *Kh,
                             const void *Vh, int32_t *ring, void *cache_K, void *cache_V,
                             int32_t *cache_tok, int32_t *idx_cache, int32_t *stats,
                             hipStream_t s);

}  // namespace ckv
