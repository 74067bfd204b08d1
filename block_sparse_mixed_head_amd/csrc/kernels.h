// kernels.h - internal launch interface between the C-ABI layer (capi.cpp) and the
// gfx950 kernels.  Not part of the public ABI; shapes here are already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tria {

struct Shape {
  int batch, hq, hkv, d, blk;
  int64_t n;
};

// Per-row symmetric int8 / int4 quantisation of Q and K (one launch for both; q null:
// K only, the Q outputs untouched).
hipError_t launch_quantize(const Shape& s, const void* q, const void* k, int8_t* q8, uint8_t* q4,
                           float* q8s, float* q4s, int8_t* k8, uint8_t* k4, float* k8s, float* k4s,
                           hipStream_t stream);

// Fused block-sparse prefill over the unit records of a schedule (device memory).
// qraw (device bf16 Q, or null): the kernel quantises each unit's query rows itself
// (same codes as launch_quantize) and q8 .. q4s are not read.
// seqs (device, or null): {start, length} of n_seqs sequences packed along the rows of
// one batch element (s.batch == 1, s.n = total rows); a unit's b is its sequence.
// header: the device schedule (64-byte header, then the n_units records, then, for a
// variable-length batch, the n_seqs {start, length} records); version and nb: what
// its header must hold.
hipError_t launch_prefill(const Shape& s, const int32_t* header, int version, int64_t nb, int64_t n_units,
                          const int32_t* seqs, int n_seqs, const int8_t* q8, const uint8_t* q4, const float* q8s,
                          const float* q4s, const void* qraw, const int8_t* k8, const uint8_t* k4, const float* k8s,
                          const float* k4s, const void* v, float sm_scale, float* out, float* lse, hipStream_t stream);

// Per-KV-head policy passed by value to the cache kernels.
struct KvPolicy {
  int32_t hi[128];
  int32_t keep[128];
};

// Cache geometry shared by the packer and decode launchers (host side).
struct CacheGeom {
  int64_t ctx_len;
  int32_t cur_block;     // c = (ctx_len - 1) / blk
  int64_t data_offset;   // first record byte
  int64_t rec8_bytes;    // 2*B*d + 8*B
  int64_t rec4_bytes;    // B*d + 8*B
  int64_t batch_bytes;   // record bytes of one batch element (all KV heads)
  int64_t total_bytes;
};

// Packs the cache for g.ctx_len.  Update mode (old_cache non-null): old_cache holds the
// cache for old_geo->ctx_len = g.ctx_len - 1 with the same policy and K/V; records it
// holds for the same block and precision are reused (skipped in place, else copied).
// only_current: in place, same current block: only the new token's row (append kernel).
hipError_t launch_pack(const Shape& s, const KvPolicy& pol, const CacheGeom& g, const void* k,
                       const void* v, void* cache, const void* old_cache, const CacheGeom* old_geo,
                       bool only_current, hipStream_t stream);

// Variable-length batch (s.batch <= kMaxVarlenBatch): sequence b holds ctxs[b] tokens
// (host array); geo: data offset, record sizes, cur_block of the longest sequence and
// total_bytes.  Writes the version-3 header and directory, then the records.
constexpr int kMaxVarlenBatch = 256;
hipError_t launch_pack_varlen(const Shape& s, const KvPolicy& pol, const CacheGeom& geo, const int64_t* ctxs,
                              const void* k, const void* v, void* cache, hipStream_t stream);

// Decode: split-KV partials into `workspace`, then a merge into `out`.
// decode_units_fit: the work split counts 32-token units in int32.
bool decode_units_fit(const Shape& s, int64_t ctx_len);
int64_t decode_workspace_bytes(const Shape& s, int64_t ctx_len);
// varlen: a version-3 cache (each directory entry holds its sequence's ctx_len; the
// ctx_len argument is then ignored).
hipError_t launch_decode(const Shape& s, int64_t ctx_len, const void* cache, int64_t cache_bytes,
                         const void* q, float sm_scale, float* out, void* workspace, bool varlen,
                         hipStream_t stream);
// The decode's scratch for callers that cannot allocate (decode.hip): a file-scope
// device array of decode_scratch_capacity() bytes; decode_scratch(&p) gives its
// address on the current device (looked up once per device).
int64_t decode_scratch_capacity();
hipError_t decode_scratch(void** ptr);

// Dynamic block skipping (decode.hip): the statistics index of a version-2 cache,
// the keep bits of every stored record (uint32 [pairs][cur_block + 1]), and the
// decode that reads only kept records.  q, thresholds: device.
int64_t summaries_bytes(const Shape& s, int64_t ctx_len);
int64_t skip_workspace_bytes(const Shape& s, int64_t ctx_len);
hipError_t launch_summaries(const Shape& s, int64_t ctx_len, const void* cache, int64_t cache_bytes, void* sums,
                            hipStream_t stream);
hipError_t launch_skip_masks(const Shape& s, int64_t ctx_len, const void* cache, int64_t cache_bytes,
                             const void* sums, const void* q, const float* thresholds, float sm_scale,
                             uint32_t* masks, hipStream_t stream);
hipError_t launch_decode_skip(const Shape& s, int64_t ctx_len, const void* cache, int64_t cache_bytes,
                              const void* sums, const void* q, const float* thresholds, float sm_scale, float* out,
                              void* workspace, hipStream_t stream);

// Paged cache (decode.hip): decode over a version-4 page table and a page pool.
hipError_t launch_decode_paged(const Shape& s, int64_t ctx_len, const void* table, int64_t table_bytes,
                               const void* pool, int64_t pool_bytes, const void* q, float sm_scale, float* out,
                               void* workspace, bool varlen, hipStream_t stream);
// Paged cache (pack.hip): records of the table for geo.ctx_len into the pool; records an
// old table maps to the same page and (block, precision) are left as they are.
hipError_t launch_pack_paged(const Shape& s, const KvPolicy& pol, const CacheGeom& geo, const void* k, const void* v,
                             const void* table, int64_t table_bytes, const void* old_table, int64_t old_table_bytes,
                             void* pool, int64_t pool_bytes, hipStream_t stream);

hipError_t launch_pack_paged_varlen(const Shape& s, const KvPolicy& pol, const CacheGeom& geo, const int64_t* ctxs,
                                    const void* k, const void* v, const void* table, int64_t table_bytes,
                                    const void* old_table, int64_t old_table_bytes, void* pool, int64_t pool_bytes,
                                    hipStream_t stream);

// Measured ceilings (peaks.hip): an MFMA issue loop (kind 0: i8 16x16x64, 1: bf16
// 16x16x32) and a non-temporal streaming read.  Work of one launch in ops / flops.
double peak_mfma_work(int kind, int iters);
hipError_t launch_peak_mfma(int kind, int iters, int* sink, hipStream_t stream);
int64_t peak_read_align();
hipError_t launch_peak_read(const void* src, int64_t bytes, int* sink, hipStream_t stream);

}  // namespace tria
