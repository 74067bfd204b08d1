// paged_skip.h - internal launch interface of dynamic block skipping over a paged
// cache or a variable-length cache (decode.hip): with a pool, `cache` is the
// fixed-length page table and the records are in `pool`; without, the contiguous cache.
#pragma once
#include "kernels.h"

namespace tria {

// varlen: a version-3 (contiguous) cache, each pair's ctx_len from its directory entry
// (ctx_len = seq_len sizes the index and the workspace).
hipError_t launch_summaries_paged(const Shape& s, int64_t ctx_len, const void* cache, int64_t cache_bytes, void* sums,
                                  const void* pool, int64_t pool_bytes, bool varlen, hipStream_t stream);
hipError_t launch_decode_skip_paged(const Shape& s, int64_t ctx_len, const void* cache, int64_t cache_bytes,
                                    const void* sums, const void* q, const float* thresholds, float sm_scale,
                                    float* out, void* workspace, const void* pool, int64_t pool_bytes, bool varlen,
                                    hipStream_t stream);

}  // namespace tria
