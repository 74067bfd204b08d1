// paged_skip.h - internal launch interface of dynamic block skipping over a paged
// cache (decode.hip); `cache` is the fixed-length page table, records in `pool`
// (pool == null: the contiguous cache, as launch_summaries / launch_decode_skip).
#pragma once
#include "kernels.h"

namespace tria {

hipError_t launch_summaries_paged(const Shape& s, int64_t ctx_len, const void* cache, int64_t cache_bytes, void* sums,
                                  const void* pool, int64_t pool_bytes, hipStream_t stream);
hipError_t launch_decode_skip_paged(const Shape& s, int64_t ctx_len, const void* cache, int64_t cache_bytes,
                                    const void* sums, const void* q, const float* thresholds, float sm_scale,
                                    float* out, void* workspace, const void* pool, int64_t pool_bytes,
                                    hipStream_t stream);

}  // namespace tria
