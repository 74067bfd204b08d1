// capi.cpp - the C ABI declared in include/tria.h: argument validation, the host
// policy expander, size queries and kernel launches.  Nothing here allocates
// device memory; device work is enqueued on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <queue>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "kernels.h"
#include "paged_skip.h"
#include "tria.h"

namespace {

thread_local std::string g_error;

tria_status fail(tria_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
tria_status fail(tria_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  if (getenv("TRIA_LOG")) fprintf(stderr, "tria: %s\n", buf);
  return st;
}

tria_status ok() {
  g_error.clear();
  return TRIA_OK;
}

tria_status check_dims(const tria_dims* d) {
  if (!d) return fail(TRIA_ERR_INVALID_ARG, "dims is NULL");
  if (d->reserved != 0) return fail(TRIA_ERR_INVALID_ARG, "dims.reserved must be 0");
  if (d->batch < 1 || d->n_q_heads < 1 || d->n_kv_heads < 1 || d->seq_len < 1)
    return fail(TRIA_ERR_INVALID_ARG, "batch, heads and seq_len must be >= 1");
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(TRIA_ERR_INVALID_ARG, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", d->n_q_heads,
                d->n_kv_heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(TRIA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d->head_dim);
  if (d->block != 64 && d->block != 128)
    return fail(TRIA_ERR_UNSUPPORTED, "block %d not supported (64 or 128)", d->block);
  if (d->n_kv_heads > TRIA_MAX_KV_HEADS)
    return fail(TRIA_ERR_UNSUPPORTED, "n_kv_heads %d above %d", d->n_kv_heads, TRIA_MAX_KV_HEADS);
  const int64_t nb = (d->seq_len + d->block - 1) / d->block;
  if ((int64_t)d->batch * d->n_q_heads * nb > INT32_MAX)
    return fail(TRIA_ERR_UNSUPPORTED, "too many (batch, head, block) units");
  return TRIA_OK;
}

tria_status check_policy(const int32_t* hi, const int32_t* keep, int32_t n) {
  if (!hi || !keep) return fail(TRIA_ERR_INVALID_ARG, "hi/keep is NULL");
  for (int32_t h = 0; h < n; ++h) {
    if (hi[h] < 0 || keep[h] < hi[h])
      return fail(TRIA_ERR_INVALID_ARG, "head %d: need 0 <= hi (%d) <= keep (%d)", h, hi[h], keep[h]);
  }
  return TRIA_OK;
}

tria::Shape shape_of(const tria_dims* d) {
  return tria::Shape{d->batch, d->n_q_heads, d->n_kv_heads, d->head_dim, d->block, d->seq_len};
}

// Per-KV-head boundaries (merged by group maximum when given per query head).
tria_status kv_policy(const tria_dims* d, const int32_t* hi, const int32_t* keep, int32_t n_policy,
                      tria::KvPolicy& pol) {
  if (n_policy != d->n_kv_heads && n_policy != d->n_q_heads)
    return fail(TRIA_ERR_INVALID_ARG, "n_policy_heads %d must be n_kv_heads (%d) or n_q_heads (%d)", n_policy,
                d->n_kv_heads, d->n_q_heads);
  tria_status st = check_policy(hi, keep, n_policy);
  if (st != TRIA_OK) return st;
  std::memset(&pol, 0, sizeof pol);
  const int G = n_policy == d->n_kv_heads ? 1 : d->n_q_heads / d->n_kv_heads;
  for (int h = 0; h < n_policy; ++h) {
    const int g = h / G;
    pol.hi[g] = std::max(pol.hi[g], hi[h]);
    pol.keep[g] = std::max(pol.keep[g], keep[h]);
  }
  return TRIA_OK;
}

struct Stored {
  int64_t n8, n4;
};

// Stored blocks of one KV head for current block c (the tile rule for query block c).
Stored stored_count(int64_t c, int64_t hi, int64_t keep) {
  const int64_t lo8 = (c - hi >= 2) ? c - hi : 0;
  const int64_t sink = lo8 > 0 ? 1 : 0;
  int64_t lo4 = std::max<int64_t>(1, c - keep), hi4 = c - hi - 1;
  const int64_t n4 = lo4 > hi4 ? 0 : hi4 - lo4 + 1;
  return Stored{c - lo8 + 1 + sink, n4};
}

tria::CacheGeom cache_geom(const tria_dims* d, const tria::KvPolicy& pol, int64_t ctx_len) {
  tria::CacheGeom g;
  g.ctx_len = ctx_len;
  g.cur_block = (int32_t)((ctx_len - 1) / d->block);
  g.data_offset = (64 + 64LL * d->batch * d->n_kv_heads + 255) / 256 * 256;
  g.rec8_bytes = 2LL * d->block * d->head_dim + 8LL * d->block;
  g.rec4_bytes = (int64_t)d->block * d->head_dim + 8LL * d->block;
  int64_t per_batch = 0;
  for (int gk = 0; gk < d->n_kv_heads; ++gk) {
    const Stored s = stored_count(g.cur_block, pol.hi[gk], pol.keep[gk]);
    per_batch += s.n8 * g.rec8_bytes + s.n4 * g.rec4_bytes;
  }
  g.batch_bytes = per_batch;
  g.total_bytes = g.data_offset + per_batch * d->batch;
  return g;
}

tria_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(TRIA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Whole tiles of one head's policy summed over all query blocks (the tile rule:
// int8 = block 0, the diagonal and distances <= hi; int4 = distances in (hi, keep]).
void policy_tiles(int64_t nb, int64_t hi, int64_t keep, int64_t& t8, int64_t& t4) {
  t8 = t4 = 0;
  for (int64_t qb = 0; qb < nb; ++qb) {
    const int64_t lo8 = qb - hi >= 2 ? qb - hi : 0;
    t8 += qb - lo8 + 1 + (lo8 > 0 ? 1 : 0);
    const int64_t lo4 = std::max<int64_t>(1, qb - keep), hi4 = qb - hi - 1;
    if (hi4 >= lo4) t4 += hi4 - lo4 + 1;
  }
}

// Cost of one head's policy: whole processed tiles (B*B query-key pairs each) weighted
// by the cost of a pair at each precision.
#pragma clang fp contract(off)  // the cost is compared bit for bit: no fused multiply-add
double policy_cost_of(const tria_dims* d, int64_t hi, int64_t keep, double c8, double c4) {
  const int64_t nb = (d->seq_len + d->block - 1) / d->block;
  int64_t t8, t4;
  policy_tiles(nb, hi, keep, t8, t4);
  const double b2 = (double)d->block * (double)d->block;
  return (c8 * (double)t8 + c4 * (double)t4) * b2;
}
#pragma clang fp contract(on)

#define NONNULL(p)                                                           \
  do {                                                                       \
    if (!(p)) return fail(TRIA_ERR_INVALID_ARG, "%s is NULL", #p);           \
  } while (0)

}  // namespace

extern "C" {

const char* tria_last_error(void) { return g_error.c_str(); }

int32_t tria_version(void) { return (1 << 16) | 0; }

// ------------------------------------------------------------------ (1) policy
// Dispatch order of the units.  The prefill launches one work group per unit in
// record order, and work group i runs on XCD i mod 8 (round-robin over the eight
// XCDs, each with its own L2).  Consecutive query blocks of one query head read
// overlapping key windows: run together on one XCD, they read each K/V tile within
// a few stages of one another, so it is fetched into that L2 about once instead of
// once per unit (the traffic beyond L2 costs power, and the part runs at its power
// limit).  So each lane (batch row b, head h) is cut into chunks of kChunk
// consecutive query blocks, taken from the last block down; a chunk's units run in
// consecutive slots of one XCD.  Chunks go, largest (most tiles) first, to the XCD
// with the least work so far among those with room for them, and each XCD runs its
// chunks largest first, so the shortest units close the dispatch.  Record r of
// XCD x goes to position 8 r + x while every XCD still has records; the rest
// follow round-robin over the XCDs that still have them.
constexpr int kXcds = 8;
constexpr int64_t kChunk = 32;

static void dispatch_order(const std::vector<int32_t>& rec, int64_t n_units, const std::vector<int64_t>& nb_of,
                           int32_t hq, int32_t* units) {
  struct Chunk {
    int64_t first, count, work;  // records first .. first + count - 1 (q-blocks descending)
  };
  // records arrive in (b, h, qb ascending) order; a lane's chunks start at its last q-block
  std::vector<Chunk> chunks;
  std::vector<int64_t> order;  // record indices, each lane's q-blocks descending
  order.reserve((size_t)n_units);
  int64_t base = 0;
  for (size_t b = 0; b < nb_of.size(); ++b)
    for (int h = 0; h < hq; ++h, base += nb_of[b])
      for (int64_t c0 = 0; c0 < nb_of[b]; c0 += kChunk) {
        Chunk c{(int64_t)order.size(), std::min(kChunk, nb_of[b] - c0), 0};
        for (int64_t i = 0; i < c.count; ++i) {
          const int64_t r = base + nb_of[b] - 1 - (c0 + i);
          order.push_back(r);
          c.work += rec[(size_t)r * 8 + 7];
        }
        chunks.push_back(c);
      }
  std::vector<size_t> by_work(chunks.size());
  for (size_t i = 0; i < by_work.size(); ++i) by_work[i] = i;
  std::stable_sort(by_work.begin(), by_work.end(),
                   [&](size_t a, size_t b) { return chunks[a].work > chunks[b].work; });
  const int64_t room = (n_units + kXcds - 1) / kXcds;
  std::vector<std::vector<size_t>> xcd(kXcds);
  int64_t work[kXcds] = {0}, count[kXcds] = {0};
  for (size_t c : by_work) {
    int best = -1;
    for (int x = 0; x < kXcds; ++x)
      if (count[x] + chunks[c].count <= room && (best < 0 || work[x] < work[best])) best = x;
    if (best < 0)  // no XCD has room for the whole chunk: the least loaded by units
      for (int x = 0; x < kXcds; ++x)
        if (best < 0 || count[x] < count[best]) best = x;
    xcd[best].push_back(c);
    work[best] += chunks[c].work;
    count[best] += chunks[c].count;
  }
  // each XCD's records (its chunks in placement order: largest first)
  std::vector<std::vector<int64_t>> seq(kXcds);
  for (int x = 0; x < kXcds; ++x)
    for (size_t c : xcd[x])
      for (int64_t i = 0; i < chunks[c].count; ++i) seq[x].push_back(order[(size_t)(chunks[c].first + i)]);
  int64_t pos = 0;
  for (size_t r = 0; pos < n_units; ++r)
    for (int x = 0; x < kXcds; ++x)
      if (r < seq[x].size()) std::memcpy(units + 8 * pos++, &rec[(size_t)seq[x][r] * 8], 32);
}

// Units of `nb_of.size()` batch rows (sequences) with nb_of[b] query blocks each,
// written after the 64-byte header at `out` in the dispatch order above.
static void expand_units(const std::vector<int64_t>& nb_of, int32_t hq, const int32_t* hi, const int32_t* keep,
                         int32_t* units) {
  int64_t n_units = 0;
  for (int64_t nb : nb_of) n_units += hq * nb;
  std::vector<int32_t> rec((size_t)n_units * 8);
  int64_t u = 0;
  for (size_t b = 0; b < nb_of.size(); ++b)
    for (int h = 0; h < hq; ++h)
      for (int64_t qb = 0; qb < nb_of[b]; ++qb, ++u) {
        const int64_t H = hi[h], K = keep[h];
        const int64_t lo8 = (qb - H >= 2) ? qb - H : 0;
        const int64_t sink = lo8 > 0 ? 1 : 0;
        int64_t lo4 = std::max<int64_t>(1, qb - K), hi4 = qb - H - 1;
        if (lo4 > hi4) {
          lo4 = 0;
          hi4 = -1;
        }
        const int64_t ntiles = (qb - lo8 + 1) + sink + (hi4 - lo4 + 1);
        int32_t* r = &rec[(size_t)u * 8];
        r[0] = (int32_t)b;
        r[1] = h;
        r[2] = (int32_t)qb;
        r[3] = (int32_t)lo8;
        r[4] = (int32_t)lo4;
        r[5] = (int32_t)hi4;
        r[6] = (int32_t)sink;
        r[7] = (int32_t)ntiles;
      }
  dispatch_order(rec, n_units, nb_of, hq, units);
}

static void schedule_header(int32_t* out, int32_t version, int32_t rows, const tria_dims* dims, int64_t nb,
                            int64_t n_units) {
  std::memset(out, 0, TRIA_SCHED_HEADER_BYTES);
  out[0] = TRIA_SCHED_MAGIC;
  out[1] = version;
  out[2] = rows;
  out[3] = dims->n_q_heads;
  out[4] = dims->n_kv_heads;
  out[5] = dims->head_dim;
  out[6] = dims->block;
  out[7] = (int32_t)nb;
  out[8] = (int32_t)n_units;
  out[10] = (int32_t)(dims->seq_len & 0xFFFFFFFF);
  out[11] = (int32_t)(dims->seq_len >> 32);
}

tria_status tria_build_policy(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                              int32_t n_policy_heads, void* sched_host, size_t sched_bytes,
                              size_t* sched_bytes_needed) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  if (n_policy_heads != dims->n_q_heads)
    return fail(TRIA_ERR_INVALID_ARG, "n_policy_heads %d != n_q_heads %d", n_policy_heads, dims->n_q_heads);
  st = check_policy(hi, keep, n_policy_heads);
  if (st != TRIA_OK) return st;
  const int64_t nb = (dims->seq_len + dims->block - 1) / dims->block;
  const int64_t n_units = (int64_t)dims->batch * dims->n_q_heads * nb;
  const size_t need = TRIA_SCHED_HEADER_BYTES + TRIA_SCHED_UNIT_BYTES * (size_t)n_units;
  if (sched_bytes_needed) *sched_bytes_needed = need;
  if (!sched_host) {
    if (sched_bytes_needed) return ok();
    return fail(TRIA_ERR_INVALID_ARG, "sched_host and sched_bytes_needed are both NULL");
  }
  if (sched_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "schedule needs %zu bytes, got %zu", need, sched_bytes);
  int32_t* out = static_cast<int32_t*>(sched_host);
  schedule_header(out, TRIA_SCHED_VERSION, dims->batch, dims, nb, n_units);
  expand_units(std::vector<int64_t>((size_t)dims->batch, nb), dims->n_q_heads, hi, keep,
               out + TRIA_SCHED_HEADER_BYTES / 4);
  return ok();
}

// Variable-length batch: checks cu_seqlens (host) against dims and returns the
// per-sequence block counts and the unit count.
static tria_status varlen_layout(const tria_dims* dims, int32_t n_seqs, const int64_t* cu, std::vector<int64_t>& nbs,
                                 int64_t& n_units) {
  if (dims->batch != 1) return fail(TRIA_ERR_INVALID_ARG, "a variable-length batch needs dims->batch == 1");
  if (n_seqs < 1) return fail(TRIA_ERR_INVALID_ARG, "n_seqs must be >= 1");
  NONNULL(cu);
  if (cu[0] != 0 || cu[n_seqs] != dims->seq_len)
    return fail(TRIA_ERR_INVALID_ARG, "cu_seqlens must start at 0 and end at seq_len (%lld)",
                (long long)dims->seq_len);
  nbs.assign((size_t)n_seqs, 0);
  n_units = 0;
  for (int32_t i = 0; i < n_seqs; ++i) {
    if (cu[i + 1] <= cu[i]) return fail(TRIA_ERR_INVALID_ARG, "sequence %d is empty or cu_seqlens decreases", i);
    nbs[i] = (cu[i + 1] - cu[i] + dims->block - 1) / dims->block;
    n_units += (int64_t)dims->n_q_heads * nbs[i];
  }
  return TRIA_OK;
}

tria_status tria_build_policy_varlen(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                     int32_t n_policy_heads, int32_t n_seqs, const int64_t* cu_seqlens,
                                     void* sched_host, size_t sched_bytes, size_t* sched_bytes_needed) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  if (n_policy_heads != dims->n_q_heads)
    return fail(TRIA_ERR_INVALID_ARG, "n_policy_heads %d != n_q_heads %d", n_policy_heads, dims->n_q_heads);
  st = check_policy(hi, keep, n_policy_heads);
  if (st != TRIA_OK) return st;
  std::vector<int64_t> nbs;
  int64_t n_units;
  st = varlen_layout(dims, n_seqs, cu_seqlens, nbs, n_units);
  if (st != TRIA_OK) return st;
  const size_t need = TRIA_SCHED_HEADER_BYTES + TRIA_SCHED_UNIT_BYTES * (size_t)n_units + 8 * (size_t)n_seqs;
  if (sched_bytes_needed) *sched_bytes_needed = need;
  if (!sched_host) {
    if (sched_bytes_needed) return ok();
    return fail(TRIA_ERR_INVALID_ARG, "sched_host and sched_bytes_needed are both NULL");
  }
  if (sched_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "schedule needs %zu bytes, got %zu", need, sched_bytes);
  int32_t* out = static_cast<int32_t*>(sched_host);
  schedule_header(out, TRIA_SCHED_VERSION_VARLEN, n_seqs, dims, *std::max_element(nbs.begin(), nbs.end()), n_units);
  int32_t* units = out + TRIA_SCHED_HEADER_BYTES / 4;
  expand_units(nbs, dims->n_q_heads, hi, keep, units);
  int32_t* seqs = units + 8 * n_units;
  for (int32_t i = 0; i < n_seqs; ++i) {
    seqs[2 * i] = (int32_t)cu_seqlens[i];
    seqs[2 * i + 1] = (int32_t)(cu_seqlens[i + 1] - cu_seqlens[i]);
  }
  return ok();
}

// ------------------------------------------------------------------ (2) quantiser
tria_status tria_quantize_qk(const tria_dims* dims, const void* q_bf16, const void* k_bf16, int8_t* q8,
                             uint8_t* q4, float* q8s, float* q4s, int8_t* k8, uint8_t* k4, float* k8s,
                             float* k4s, void* stream) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(q_bf16);
  NONNULL(k_bf16);
  NONNULL(q8);
  NONNULL(q4);
  NONNULL(q8s);
  NONNULL(q4s);
  NONNULL(k8);
  NONNULL(k4);
  NONNULL(k8s);
  NONNULL(k4s);
  return launched(tria::launch_quantize(shape_of(dims), q_bf16, k_bf16, q8, q4, q8s, q4s, k8, k4, k8s, k4s,
                                        static_cast<hipStream_t>(stream)),
                  "quantize launch");
}

tria_status tria_quantize_k(const tria_dims* dims, const void* k_bf16, int8_t* k8, uint8_t* k4, float* k8s,
                            float* k4s, void* stream) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(k_bf16);
  NONNULL(k8);
  NONNULL(k4);
  NONNULL(k8s);
  NONNULL(k4s);
  return launched(tria::launch_quantize(shape_of(dims), nullptr, k_bf16, nullptr, nullptr, nullptr, nullptr, k8, k4,
                                        k8s, k4s, static_cast<hipStream_t>(stream)),
                  "quantize launch");
}

// ------------------------------------------------------------------ (3) prefill
// The kernel addresses a unit's K, V and key-scale rows with 32-bit byte offsets from
// the unit's first row (the widest, a V row, is 2 * head_dim bytes), up to three
// stages of 64 keys past the sequence's last block.
static bool prefill_len_ok(const tria_dims* d) {
  return ((int64_t)d->seq_len + 4 * (int64_t)d->block) * 2 * d->head_dim <= (int64_t)INT32_MAX;
}
// Validation and launch shared by tria_prefill (codes q8 .. q4s) and
// tria_prefill_bf16q (qraw: bf16 Q quantised inside the kernel).
static tria_status prefill_fixed(const tria_dims* dims, const void* sched_dev, size_t sched_bytes, const int8_t* q8,
                                 const uint8_t* q4, const float* q8s, const float* q4s, const void* qraw,
                                 const int8_t* k8, const uint8_t* k4, const float* k8s, const float* k4s,
                                 const void* v_bf16, float sm_scale, float* out, float* lse, void* stream) {
  NONNULL(sched_dev);
  NONNULL(k8);
  NONNULL(k4);
  NONNULL(k8s);
  NONNULL(k4s);
  NONNULL(v_bf16);
  NONNULL(out);
  const int64_t nb = (dims->seq_len + dims->block - 1) / dims->block;
  const int64_t n_units = (int64_t)dims->batch * dims->n_q_heads * nb;
  const size_t need = TRIA_SCHED_HEADER_BYTES + TRIA_SCHED_UNIT_BYTES * (size_t)n_units;
  if (sched_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "schedule for these dims needs %zu bytes, got %zu", need, sched_bytes);
  if (sched_bytes != need)
    return fail(TRIA_ERR_INVALID_ARG, "schedule for these dims is %zu bytes, got %zu", need, sched_bytes);
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return fail(TRIA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  if (!prefill_len_ok(dims))
    return fail(TRIA_ERR_UNSUPPORTED, "prefill supports (seq_len + 4 * block) * 2 * head_dim < 2^31, got seq_len %lld",
                (long long)dims->seq_len);
  const int32_t* header = static_cast<const int32_t*>(sched_dev);
  return launched(tria::launch_prefill(shape_of(dims), header, TRIA_SCHED_VERSION, nb, n_units, nullptr, 0, q8, q4,
                                       q8s, q4s, qraw, k8, k4, k8s, k4s, v_bf16, sm_scale, out, lse,
                                       static_cast<hipStream_t>(stream)),
                  "prefill launch");
}

tria_status tria_prefill(const tria_dims* dims, const void* sched_dev, size_t sched_bytes, const int8_t* q8,
                         const uint8_t* q4, const float* q8s, const float* q4s, const int8_t* k8,
                         const uint8_t* k4, const float* k8s, const float* k4s, const void* v_bf16,
                         float sm_scale, float* out, float* lse, void* stream) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(q8);
  NONNULL(q4);
  NONNULL(q8s);
  NONNULL(q4s);
  return prefill_fixed(dims, sched_dev, sched_bytes, q8, q4, q8s, q4s, nullptr, k8, k4, k8s, k4s, v_bf16, sm_scale,
                       out, lse, stream);
}

tria_status tria_prefill_bf16q(const tria_dims* dims, const void* sched_dev, size_t sched_bytes, const void* q_bf16,
                               const int8_t* k8, const uint8_t* k4, const float* k8s, const float* k4s,
                               const void* v_bf16, float sm_scale, float* out, float* lse, void* stream) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(q_bf16);
  return prefill_fixed(dims, sched_dev, sched_bytes, nullptr, nullptr, nullptr, nullptr, q_bf16, k8, k4, k8s, k4s,
                       v_bf16, sm_scale, out, lse, stream);
}

tria_status tria_prefill_varlen(const tria_dims* dims, int32_t n_seqs, const int64_t* cu_seqlens,
                                const void* sched_dev, size_t sched_bytes, const int8_t* q8, const uint8_t* q4,
                                const float* q8s, const float* q4s, const int8_t* k8, const uint8_t* k4,
                                const float* k8s, const float* k4s, const void* v_bf16, float sm_scale, float* out,
                                float* lse, void* stream) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(sched_dev);
  NONNULL(q8);
  NONNULL(q4);
  NONNULL(q8s);
  NONNULL(q4s);
  NONNULL(k8);
  NONNULL(k4);
  NONNULL(k8s);
  NONNULL(k4s);
  NONNULL(v_bf16);
  NONNULL(out);
  std::vector<int64_t> nbs;
  int64_t n_units;
  st = varlen_layout(dims, n_seqs, cu_seqlens, nbs, n_units);
  if (st != TRIA_OK) return st;
  const size_t need = TRIA_SCHED_HEADER_BYTES + TRIA_SCHED_UNIT_BYTES * (size_t)n_units + 8 * (size_t)n_seqs;
  if (sched_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "schedule for this batch needs %zu bytes, got %zu", need, sched_bytes);
  if (sched_bytes != need)
    return fail(TRIA_ERR_INVALID_ARG, "schedule for this batch is %zu bytes, got %zu", need, sched_bytes);
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return fail(TRIA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  if (!prefill_len_ok(dims))
    return fail(TRIA_ERR_UNSUPPORTED, "prefill supports (seq_len + 4 * block) * 2 * head_dim < 2^31, got seq_len %lld",
                (long long)dims->seq_len);
  const int32_t* header = static_cast<const int32_t*>(sched_dev);
  const int32_t* seqs = header + TRIA_SCHED_HEADER_BYTES / 4 + 8 * n_units;
  return launched(tria::launch_prefill(shape_of(dims), header, TRIA_SCHED_VERSION_VARLEN,
                                       *std::max_element(nbs.begin(), nbs.end()), n_units, seqs, n_seqs, q8, q4, q8s,
                                       q4s, nullptr, k8, k4, k8s, k4s, v_bf16, sm_scale, out, lse,
                                       static_cast<hipStream_t>(stream)),
                  "prefill launch");
}

// ------------------------------------------------------------------ (4) cache
tria_status tria_kv_cache_bytes(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                int32_t n_policy_heads, int64_t ctx_len, size_t* bytes) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(bytes);
  if (ctx_len < 1 || ctx_len > dims->seq_len)
    return fail(TRIA_ERR_INVALID_ARG, "ctx_len %lld outside [1, seq_len=%lld]", (long long)ctx_len,
                (long long)dims->seq_len);
  tria::KvPolicy pol;
  st = kv_policy(dims, hi, keep, n_policy_heads, pol);
  if (st != TRIA_OK) return st;
  *bytes = (size_t)cache_geom(dims, pol, ctx_len).total_bytes;
  return ok();
}

tria_status tria_pack_kv_cache(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                               int32_t n_policy_heads, int64_t ctx_len, const void* k_bf16, const void* v_bf16,
                               void* cache, size_t cache_bytes, void* stream) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(k_bf16);
  NONNULL(v_bf16);
  NONNULL(cache);
  if (ctx_len < 1 || ctx_len > dims->seq_len)
    return fail(TRIA_ERR_INVALID_ARG, "ctx_len %lld outside [1, seq_len=%lld]", (long long)ctx_len,
                (long long)dims->seq_len);
  if ((int64_t)dims->batch * dims->n_kv_heads > 65535)
    return fail(TRIA_ERR_UNSUPPORTED, "batch * n_kv_heads above 65535");
  tria::KvPolicy pol;
  st = kv_policy(dims, hi, keep, n_policy_heads, pol);
  if (st != TRIA_OK) return st;
  const tria::CacheGeom g = cache_geom(dims, pol, ctx_len);
  if ((int64_t)cache_bytes < g.total_bytes)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "cache needs %lld bytes, got %zu", (long long)g.total_bytes, cache_bytes);
  return launched(tria::launch_pack(shape_of(dims), pol, g, k_bf16, v_bf16, cache, nullptr, nullptr, false,
                                    static_cast<hipStream_t>(stream)),
                  "pack launch");
}

tria_status tria_update_kv_cache(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                 int32_t n_policy_heads, int64_t ctx_len, const void* k_bf16, const void* v_bf16,
                                 const void* cache_in, size_t cache_in_bytes, void* cache_out, size_t cache_out_bytes,
                                 void* stream) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(k_bf16);
  NONNULL(v_bf16);
  NONNULL(cache_in);
  NONNULL(cache_out);
  if (ctx_len < 2 || ctx_len > dims->seq_len)
    return fail(TRIA_ERR_INVALID_ARG, "ctx_len %lld outside [2, seq_len=%lld]", (long long)ctx_len,
                (long long)dims->seq_len);
  if ((int64_t)dims->batch * dims->n_kv_heads > 65535)
    return fail(TRIA_ERR_UNSUPPORTED, "batch * n_kv_heads above 65535");
  tria::KvPolicy pol;
  st = kv_policy(dims, hi, keep, n_policy_heads, pol);
  if (st != TRIA_OK) return st;
  const tria::CacheGeom g = cache_geom(dims, pol, ctx_len);
  const tria::CacheGeom go = cache_geom(dims, pol, ctx_len - 1);
  if ((int64_t)cache_in_bytes < go.total_bytes)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "cache_in must hold the %lld-byte cache for ctx_len - 1, got %zu",
                (long long)go.total_bytes, cache_in_bytes);
  if ((int64_t)cache_out_bytes < g.total_bytes)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "cache_out needs %lld bytes, got %zu", (long long)g.total_bytes,
                cache_out_bytes);
  const bool boundary = g.cur_block != go.cur_block;
  const uintptr_t i0 = reinterpret_cast<uintptr_t>(cache_in), o0 = reinterpret_cast<uintptr_t>(cache_out);
  const bool in_place = i0 == o0;
  if (in_place && boundary)
    return fail(TRIA_ERR_INVALID_ARG, "ctx_len - 1 = %lld starts a new block: records move, so cache_out must be "
                "another buffer", (long long)(ctx_len - 1));
  if (!in_place && i0 < o0 + (uintptr_t)g.total_bytes && o0 < i0 + (uintptr_t)go.total_bytes)
    return fail(TRIA_ERR_INVALID_ARG, "cache_in and cache_out overlap without being the same buffer");
  return launched(tria::launch_pack(shape_of(dims), pol, g, k_bf16, v_bf16, cache_out, cache_in, &go, in_place,
                                    static_cast<hipStream_t>(stream)),
                  "cache update launch");
}

// Variable-length batch: per-sequence lengths (host); geometry of the longest.
static tria_status varlen_cache_geom(const tria_dims* dims, const tria::KvPolicy& pol, const int64_t* ctx_lens,
                                     tria::CacheGeom& g) {
  NONNULL(ctx_lens);
  if (dims->batch > tria::kMaxVarlenBatch)
    return fail(TRIA_ERR_UNSUPPORTED, "variable-length caches hold at most %d sequences", tria::kMaxVarlenBatch);
  int64_t longest = 1;
  for (int b = 0; b < dims->batch; ++b) {
    if (ctx_lens[b] < 1 || ctx_lens[b] > dims->seq_len)
      return fail(TRIA_ERR_INVALID_ARG, "ctx_lens[%d] = %lld outside [1, seq_len=%lld]", b, (long long)ctx_lens[b],
                  (long long)dims->seq_len);
    longest = std::max(longest, ctx_lens[b]);
  }
  g = cache_geom(dims, pol, longest);
  int64_t total = g.data_offset;
  for (int b = 0; b < dims->batch; ++b) {
    const int64_t c = (ctx_lens[b] - 1) / dims->block;
    for (int gk = 0; gk < dims->n_kv_heads; ++gk) {
      const Stored s = stored_count(c, pol.hi[gk], pol.keep[gk]);
      total += s.n8 * g.rec8_bytes + s.n4 * g.rec4_bytes;
    }
  }
  g.total_bytes = total;
  g.batch_bytes = 0;  // varies by sequence
  return TRIA_OK;
}

tria_status tria_kv_cache_bytes_varlen(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                       int32_t n_policy_heads, const int64_t* ctx_lens, size_t* bytes) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(bytes);
  tria::KvPolicy pol;
  st = kv_policy(dims, hi, keep, n_policy_heads, pol);
  if (st != TRIA_OK) return st;
  tria::CacheGeom g;
  st = varlen_cache_geom(dims, pol, ctx_lens, g);
  if (st != TRIA_OK) return st;
  *bytes = (size_t)g.total_bytes;
  return ok();
}

tria_status tria_pack_kv_cache_varlen(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                      int32_t n_policy_heads, const int64_t* ctx_lens, const void* k_bf16,
                                      const void* v_bf16, void* cache, size_t cache_bytes, void* stream) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(k_bf16);
  NONNULL(v_bf16);
  NONNULL(cache);
  tria::KvPolicy pol;
  st = kv_policy(dims, hi, keep, n_policy_heads, pol);
  if (st != TRIA_OK) return st;
  tria::CacheGeom g;
  st = varlen_cache_geom(dims, pol, ctx_lens, g);
  if (st != TRIA_OK) return st;
  if ((int64_t)cache_bytes < g.total_bytes)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "cache needs %lld bytes, got %zu", (long long)g.total_bytes, cache_bytes);
  return launched(tria::launch_pack_varlen(shape_of(dims), pol, g, ctx_lens, k_bf16, v_bf16, cache,
                                           static_cast<hipStream_t>(stream)),
                  "pack launch");
}

tria_status tria_check_cache(const tria_dims* dims, const void* cache, size_t cache_bytes, int64_t ctx_len) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(cache);
  const int64_t pairs = (int64_t)dims->batch * dims->n_kv_heads;
  const int64_t dir_end = 64 + 64 * pairs;
  if ((int64_t)cache_bytes < dir_end) return fail(TRIA_ERR_INVALID_ARG, "cache smaller than its directory");
  std::vector<uint8_t> h((size_t)dir_end);
  hipError_t e = hipMemcpy(h.data(), cache, (size_t)dir_end, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(TRIA_ERR_HIP, "reading the cache header: %s", hipGetErrorString(e));
  int32_t hd[8];
  int64_t h64[4];
  std::memcpy(hd, h.data(), 32);
  std::memcpy(h64, h.data() + 32, 32);
  const int64_t c = (ctx_len - 1) / dims->block;
  const int64_t data_off = (dir_end + 255) / 256 * 256;
  if (hd[0] != TRIA_CACHE_MAGIC || hd[1] != TRIA_CACHE_VERSION) return fail(TRIA_ERR_INVALID_ARG, "bad cache magic/version");
  if (hd[2] != dims->batch || hd[3] != dims->n_kv_heads || hd[4] != dims->head_dim || hd[5] != dims->block)
    return fail(TRIA_ERR_INVALID_ARG, "cache shape does not match dims");
  if (h64[0] != ctx_len || hd[7] != c || hd[6] != c + 1) return fail(TRIA_ERR_INVALID_ARG, "cache ctx_len does not match");
  if (h64[1] > (int64_t)cache_bytes || h64[2] != 64 || h64[3] != data_off)
    return fail(TRIA_ERR_INVALID_ARG, "cache sizes/offsets corrupt");
  const int64_t rec8 = 2LL * dims->block * dims->head_dim + 8LL * dims->block;
  const int64_t rec4 = (int64_t)dims->block * dims->head_dim + 8LL * dims->block;
  int64_t expect = data_off;
  for (int64_t p = 0; p < pairs; ++p) {
    int64_t off;
    int32_t f[12];
    std::memcpy(&off, h.data() + 64 + 64 * p, 8);
    std::memcpy(f, h.data() + 64 + 64 * p + 8, 48);
    const int32_t n8 = f[0], n4 = f[1], H = f[2], K = f[3], lo8 = f[4], sink = f[5], lo4 = f[6], hi4 = f[7];
    const Stored s = stored_count(c, H, K);
    const int64_t lo8e = (c - H >= 2) ? c - H : 0;
    if (off != expect || H < 0 || K < H || n8 != s.n8 || n4 != s.n4 || lo8 != lo8e || sink != (lo8e > 0 ? 1 : 0) ||
        (n4 > 0 && (lo4 != std::max<int64_t>(1, c - K) || hi4 != c - H - 1)) || (n4 == 0 && (lo4 != 0 || hi4 != -1)))
      return fail(TRIA_ERR_INVALID_ARG, "directory entry %lld corrupt", (long long)p);
    expect += n8 * rec8 + n4 * rec4;
  }
  if (expect != h64[1]) return fail(TRIA_ERR_INVALID_ARG, "cache total_bytes corrupt");
  return ok();
}

// ------------------------------------------------------------------ (5) decode
tria_status tria_decode_workspace_bytes(const tria_dims* dims, int64_t ctx_len, size_t* bytes) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(bytes);
  if (ctx_len < 1) return fail(TRIA_ERR_INVALID_ARG, "ctx_len must be >= 1");
  *bytes = (size_t)tria::decode_workspace_bytes(shape_of(dims), ctx_len);
  return ok();
}

// The checks tria_decode and tria_decode_noalloc share (all before any HIP call);
// *need: the workspace the call takes.
static tria_status check_decode_call(const tria_dims* dims, const void* cache, size_t cache_bytes, int64_t ctx_len,
                                     const void* q_bf16, float sm_scale, float* out, int64_t* need) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(cache);
  NONNULL(q_bf16);
  NONNULL(out);
  if (ctx_len < 1) return fail(TRIA_ERR_INVALID_ARG, "ctx_len must be >= 1");
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return fail(TRIA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  const int G = dims->n_q_heads / dims->n_kv_heads;
  if (G > 32) return fail(TRIA_ERR_UNSUPPORTED, "more than 32 query heads per KV head");
  if ((int64_t)dims->batch * dims->n_kv_heads > 4096) return fail(TRIA_ERR_UNSUPPORTED, "batch * n_kv_heads above 4096");
  const int64_t dir_end = 64 + 64LL * dims->batch * dims->n_kv_heads;
  if ((int64_t)cache_bytes < dir_end) return fail(TRIA_ERR_BUFFER_TOO_SMALL, "cache smaller than its directory");
  const tria::Shape s = shape_of(dims);
  if (!tria::decode_units_fit(s, ctx_len))
    return fail(TRIA_ERR_UNSUPPORTED, "batch * n_kv_heads * ctx_len too large for one decode call");
  *need = tria::decode_workspace_bytes(s, ctx_len);
  return TRIA_OK;
}

tria_status tria_decode_noalloc(const tria_dims* dims, const void* cache, size_t cache_bytes, int64_t ctx_len,
                                const void* q_bf16, float sm_scale, float* out, void* stream) {
  int64_t need = 0;
  tria_status st = check_decode_call(dims, cache, cache_bytes, ctx_len, q_bf16, sm_scale, out, &need);
  if (st != TRIA_OK) return st;
  if (need > tria::decode_scratch_capacity())
    return fail(TRIA_ERR_UNSUPPORTED,
                "this decode needs %lld bytes of scratch; the entry point that allocates nothing holds %lld "
                "(use tria_decode with a workspace)",
                (long long)need, (long long)tria::decode_scratch_capacity());
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(TRIA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (stream) {
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sd);
    if (e != hipSuccess) return fail(TRIA_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if ((int)sd != cur)
      return fail(TRIA_ERR_INVALID_ARG, "stream belongs to device %d but device %d is current", (int)sd, cur);
  }
  void* ws = nullptr;
  e = tria::decode_scratch(&ws);
  if (e != hipSuccess) return fail(TRIA_ERR_HIP, "decode scratch address: %s", hipGetErrorString(e));
  return launched(tria::launch_decode(shape_of(dims), ctx_len, cache, (int64_t)cache_bytes, q_bf16, sm_scale, out, ws,
                                      false, static_cast<hipStream_t>(stream)),
                  "decode launch");
}

tria_status tria_decode(const tria_dims* dims, const void* cache, size_t cache_bytes, int64_t ctx_len,
                        const void* q_bf16, float sm_scale, float* out, void* workspace, size_t ws_bytes,
                        void* stream) {
  int64_t need = 0;
  tria_status st = check_decode_call(dims, cache, cache_bytes, ctx_len, q_bf16, sm_scale, out, &need);
  if (st != TRIA_OK) return st;
  NONNULL(workspace);
  if ((int64_t)ws_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "decode workspace needs %lld bytes, got %zu", (long long)need, ws_bytes);
  return launched(tria::launch_decode(shape_of(dims), ctx_len, cache, (int64_t)cache_bytes, q_bf16, sm_scale, out,
                                      workspace, false, static_cast<hipStream_t>(stream)),
                  "decode launch");
}

// ------------------------------------------------------------------ (f3) paged cache
static int64_t paged_rmax(const tria_dims* d, int64_t ctx_len) { return (ctx_len - 1) / d->block + 1; }
static int64_t paged_table_bytes_of(const tria_dims* d, int64_t ctx_len) {
  const int64_t P = (int64_t)d->batch * d->n_kv_heads;
  return 64 + 64 * P + 4 * P * paged_rmax(d, ctx_len);
}
static const int32_t kPagedMagic = 0x50564B54;  // "TKVP"

// Stored blocks of one KV head for current block c in record order: {block, 8 or 4}.
static void record_blocks(int64_t c, int64_t hi, int64_t keep, std::vector<std::pair<int64_t, int>>& out) {
  out.clear();
  const int64_t lo8 = (c - hi >= 2) ? c - hi : 0;
  if (lo8 > 0) out.push_back({0, 8});
  for (int64_t kb = lo8; kb <= c; ++kb) out.push_back({kb, 8});
  for (int64_t kb = std::max<int64_t>(1, c - keep); kb <= c - hi - 1; ++kb) out.push_back({kb, 4});
}

tria_status tria_paged_page_bytes(const tria_dims* dims, size_t* bytes) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(bytes);
  *bytes = (size_t)(2LL * dims->block * dims->head_dim + 8LL * dims->block);
  return ok();
}

tria_status tria_paged_table_bytes(const tria_dims* dims, int64_t ctx_len, size_t* bytes) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(bytes);
  if (ctx_len < 1) return fail(TRIA_ERR_INVALID_ARG, "ctx_len must be >= 1");
  *bytes = (size_t)paged_table_bytes_of(dims, ctx_len);
  return ok();
}

// The page table for per-pair current blocks (fixed length: one ctx_len; varlen: each
// batch element's ctx_lens[b], header word 7 = -1, each entry's words 10-11 = its
// ctx_len and words 12-13 its sequence id, seq_ids[b] or 0).  A pair whose length is
// below the old table's, or whose sequence id differs from it, starts afresh (all its
// old pages released): its slot holds a new sequence.
static tria_status build_paged(const tria_dims* dims, const int32_t* hi, const int32_t* keep, int32_t n_policy_heads,
                               const int64_t* ctx_lens, const int64_t* seq_ids, int64_t ctx_len, int64_t n_pages,
                               const void* old_table,
                               size_t old_table_bytes, const int32_t* free_pages, int32_t n_free, void* table,
                               size_t table_bytes, int32_t* n_used, int32_t* released, int32_t released_capacity,
                               int32_t* n_released) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(table);
  NONNULL(n_used);
  NONNULL(n_released);
  const bool varlen = ctx_lens != nullptr;
  const int64_t P = (int64_t)dims->batch * dims->n_kv_heads;
  std::vector<int64_t> ctx_b(dims->batch);
  int64_t cmax = 0;
  for (int b = 0; b < dims->batch; ++b) {
    ctx_b[b] = varlen ? ctx_lens[b] : ctx_len;
    if (ctx_b[b] < 1 || ctx_b[b] > dims->seq_len)
      return fail(TRIA_ERR_INVALID_ARG, "ctx_len %lld (batch element %d) outside [1, seq_len=%lld]",
                  (long long)ctx_b[b], b, (long long)dims->seq_len);
    cmax = std::max(cmax, (ctx_b[b] - 1) / dims->block);
  }
  if (n_pages < 1 || n_pages > INT32_MAX) return fail(TRIA_ERR_INVALID_ARG, "n_pages must be in [1, 2^31 - 1]");
  if (n_free < 0 || (n_free > 0 && !free_pages)) return fail(TRIA_ERR_INVALID_ARG, "free_pages is NULL");
  if (released_capacity < 0 || (released_capacity > 0 && !released))
    return fail(TRIA_ERR_INVALID_ARG, "released is NULL");
  tria::KvPolicy pol;
  st = kv_policy(dims, hi, keep, n_policy_heads, pol);
  if (st != TRIA_OK) return st;
  const int64_t rmax = cmax + 1;
  const int64_t need = 64 + 64 * P + 4 * P * rmax;
  if ((int64_t)table_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "table needs %lld bytes, got %zu", (long long)need, table_bytes);
  // the old table: same kind, shape, policy and pool; pages inside the pool, each once
  std::vector<uint8_t> used(static_cast<size_t>(n_pages), 0);
  int64_t orm = 0, oc_all = 0, octx_all = 0;
  const uint8_t* ot = static_cast<const uint8_t*>(old_table);
  if (ot) {
    if (old_table_bytes < 64) return fail(TRIA_ERR_INVALID_ARG, "old table smaller than its header");
    int32_t h[8];
    int64_t h64[4];
    std::memcpy(h, ot, 32);
    std::memcpy(h64, ot + 32, 32);
    orm = h[6];
    oc_all = h[7];
    octx_all = h64[0];
    const bool okind = varlen ? (h[7] == -1 && h64[0] == 0 && orm >= 1)
                              : (orm == oc_all + 1 && oc_all >= 0 && octx_all >= 1 && (octx_all - 1) / dims->block == oc_all);
    if (h[0] != kPagedMagic || h[1] != 4 || h[2] != dims->batch || h[3] != dims->n_kv_heads ||
        h[4] != dims->head_dim || h[5] != dims->block || !okind || h64[2] != n_pages)
      return fail(TRIA_ERR_INVALID_ARG, "old table header does not match (kind, dims, n_pages)");
    if ((int64_t)old_table_bytes < 64 + 64 * P + 4 * P * orm)
      return fail(TRIA_ERR_INVALID_ARG, "old table smaller than its size");
  }
  std::vector<uint8_t> out(static_cast<size_t>(need), 0);
  std::vector<int32_t> rel;
  int64_t taken = 0;
  std::vector<std::pair<int64_t, int>> nb, ob;
  for (int64_t p = 0; p < P; ++p) {
    const int g = (int)(p % dims->n_kv_heads);
    const int64_t ctx = ctx_b[p / dims->n_kv_heads], c = (ctx - 1) / dims->block;
    const int64_t sid = varlen && seq_ids ? seq_ids[p / dims->n_kv_heads] : 0;
    record_blocks(c, pol.hi[g], pol.keep[g], nb);
    std::vector<int32_t> opages;
    bool fresh = false;
    if (ot) {
      int32_t e[16];
      std::memcpy(e, ot + 64 + 64 * p, 64);
      int64_t octx = octx_all, osid = 0;
      if (varlen) {
        std::memcpy(&octx, ot + 64 + 64 * p + 40, 8);
        std::memcpy(&osid, ot + 64 + 64 * p + 48, 8);
      }
      if (octx < 1 || (octx - 1) / dims->block >= orm)
        return fail(TRIA_ERR_INVALID_ARG, "old table entry %lld corrupt", (long long)p);
      if (e[4] != pol.hi[g] || e[5] != pol.keep[g])
        return fail(TRIA_ERR_INVALID_ARG, "old table entry %lld holds another policy", (long long)p);
      record_blocks((octx - 1) / dims->block, pol.hi[g], pol.keep[g], ob);
      if (e[2] + e[3] != (int64_t)ob.size()) return fail(TRIA_ERR_INVALID_ARG, "old table entry %lld corrupt", (long long)p);
      opages.resize(ob.size());
      std::memcpy(opages.data(), ot + 64 + 64 * P + 4 * (p * orm), 4 * ob.size());
      for (int32_t pg : opages) {
        if (pg < 0 || pg >= n_pages || used[pg]) return fail(TRIA_ERR_INVALID_ARG, "old table page %d invalid", pg);
        used[pg] = 1;
      }
      fresh = ctx < octx || sid != osid;  // a shorter sequence, or another id, is a new one
    } else {
      ob.clear();
    }
    int32_t* pages = reinterpret_cast<int32_t*>(out.data() + 64 + 64 * P + 4 * (p * rmax));
    for (int64_t r = 0; r < rmax; ++r) pages[r] = -1;
    std::vector<char> kept(opages.size(), 0);
    // the old record of each (block, precision), by block
    std::vector<int32_t> old8, old4;
    if (ot && !fresh) {
      for (size_t o = 0; o < ob.size(); ++o) {
        std::vector<int32_t>& m = ob[o].second == 8 ? old8 : old4;
        if ((int64_t)m.size() <= ob[o].first) m.resize(static_cast<size_t>(ob[o].first) + 1, -1);
        m[static_cast<size_t>(ob[o].first)] = (int32_t)o;
      }
    }
    for (size_t r = 0; r < nb.size(); ++r) {
      int32_t pg = -1;
      const std::vector<int32_t>& m = nb[r].second == 8 ? old8 : old4;
      if (nb[r].first < (int64_t)m.size()) {
        const int32_t o = m[static_cast<size_t>(nb[r].first)];
        if (o >= 0 && !kept[o]) {
          pg = opages[o];
          kept[o] = 1;
        }
      }
      if (pg < 0) {
        if (taken < n_free) pg = free_pages[taken];
        ++taken;
      }
      pages[r] = pg;
    }
    for (size_t o = 0; o < opages.size(); ++o)
      if (!kept[o]) rel.push_back(opages[o]);
    int32_t e[16] = {0};
    int64_t n8 = 0;
    for (auto& x : nb) n8 += x.second == 8;
    const int64_t lo8 = (c - pol.hi[g] >= 2) ? c - pol.hi[g] : 0;
    e[2] = (int32_t)n8;
    e[3] = (int32_t)(nb.size() - n8);
    e[4] = pol.hi[g];
    e[5] = pol.keep[g];
    e[6] = (int32_t)lo8;
    e[7] = lo8 > 0 ? 1 : 0;
    e[8] = e[3] > 0 ? (int32_t)std::max<int64_t>(1, c - pol.keep[g]) : 0;
    e[9] = e[3] > 0 ? (int32_t)(c - pol.hi[g] - 1) : -1;
    if (varlen) {
      std::memcpy(&e[10], &ctx, 8);
      std::memcpy(&e[12], &sid, 8);
    }
    std::memcpy(out.data() + 64 + 64 * p, e, 64);
  }
  *n_used = (int32_t)std::min<int64_t>(taken, INT32_MAX);
  *n_released = (int32_t)rel.size();
  if (taken > n_free)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "%lld free pages needed, %d given", (long long)taken, n_free);
  if ((int64_t)rel.size() > released_capacity)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "%zu released pages, capacity %d", rel.size(), released_capacity);
  // the free pages taken: inside the pool and not held by the old table or given twice
  // (a page this update releases is still held: it can be reused from the next call on)
  for (int64_t i = 0; i < taken; ++i) {
    const int32_t pg = free_pages[i];
    if (pg < 0 || pg >= n_pages) return fail(TRIA_ERR_INVALID_ARG, "free page %d outside the pool", pg);
    if (used[pg] == 2) return fail(TRIA_ERR_INVALID_ARG, "free page %d given twice", pg);
    if (used[pg] == 1) return fail(TRIA_ERR_INVALID_ARG, "free page %d is held by the old table", pg);
    used[pg] = 2;
  }
  const int32_t c7 = varlen ? -1 : (int32_t)cmax;
  int32_t h[8] = {kPagedMagic, 4, dims->batch, dims->n_kv_heads, dims->head_dim, dims->block, (int32_t)rmax, c7};
  int64_t h64[4] = {varlen ? 0 : ctx_len, 2LL * dims->block * dims->head_dim + 8LL * dims->block, n_pages, 0};
  std::memcpy(out.data(), h, 32);
  std::memcpy(out.data() + 32, h64, 32);
  std::memcpy(table, out.data(), out.size());
  if (!rel.empty()) std::memcpy(released, rel.data(), 4 * rel.size());
  return ok();
}

tria_status tria_build_paged_table(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                   int32_t n_policy_heads, int64_t ctx_len, int64_t n_pages, const void* old_table,
                                   size_t old_table_bytes, const int32_t* free_pages, int32_t n_free, void* table,
                                   size_t table_bytes, int32_t* n_used, int32_t* released, int32_t released_capacity,
                                   int32_t* n_released) {
  return build_paged(dims, hi, keep, n_policy_heads, nullptr, nullptr, ctx_len, n_pages, old_table, old_table_bytes,
                     free_pages, n_free, table, table_bytes, n_used, released, released_capacity, n_released);
}

tria_status tria_build_paged_table_varlen(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                          int32_t n_policy_heads, const int64_t* ctx_lens, const int64_t* seq_ids,
                                          int64_t n_pages, const void* old_table, size_t old_table_bytes,
                                          const int32_t* free_pages, int32_t n_free, void* table, size_t table_bytes,
                                          int32_t* n_used, int32_t* released, int32_t released_capacity,
                                          int32_t* n_released) {
  if (!ctx_lens) return fail(TRIA_ERR_INVALID_ARG, "ctx_lens is NULL");
  if (dims && dims->batch > tria::kMaxVarlenBatch)
    return fail(TRIA_ERR_UNSUPPORTED, "batch above %d for a variable-length cache", tria::kMaxVarlenBatch);
  return build_paged(dims, hi, keep, n_policy_heads, ctx_lens, seq_ids, 0, n_pages, old_table, old_table_bytes,
                     free_pages, n_free, table, table_bytes, n_used, released, released_capacity, n_released);
}

// ------------------------------------------------------------------ (f4) dynamic block skipping

static tria_status check_skip_call(const tria_dims* dims, int64_t ctx_len, const void* cache, size_t cache_bytes) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(cache);
  if (ctx_len < 1) return fail(TRIA_ERR_INVALID_ARG, "ctx_len must be >= 1");
  if (dims->n_q_heads / dims->n_kv_heads > 32) return fail(TRIA_ERR_UNSUPPORTED, "more than 32 query heads per KV head");
  if ((int64_t)dims->batch * dims->n_kv_heads > 4096) return fail(TRIA_ERR_UNSUPPORTED, "batch * n_kv_heads above 4096");
  const int64_t dir_end = 64 + 64LL * dims->batch * dims->n_kv_heads;
  if ((int64_t)cache_bytes < dir_end) return fail(TRIA_ERR_BUFFER_TOO_SMALL, "cache smaller than its directory");
  const tria::Shape s = shape_of(dims);
  if (!tria::decode_units_fit(s, ctx_len))
    return fail(TRIA_ERR_UNSUPPORTED, "batch * n_kv_heads * ctx_len too large for one decode call");
  const int64_t slots = (int64_t)dims->batch * dims->n_kv_heads * ((ctx_len - 1) / dims->block + 1);
  if (slots > INT32_MAX / 2) return fail(TRIA_ERR_UNSUPPORTED, "too many record slots");
  return TRIA_OK;
}

tria_status tria_block_summaries_bytes(const tria_dims* dims, int64_t ctx_len, size_t* bytes) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(bytes);
  if (ctx_len < 1) return fail(TRIA_ERR_INVALID_ARG, "ctx_len must be >= 1");
  *bytes = (size_t)tria::summaries_bytes(shape_of(dims), ctx_len);
  return ok();
}

tria_status tria_build_block_summaries(const tria_dims* dims, const void* cache, size_t cache_bytes, int64_t ctx_len,
                                       void* summaries, size_t summaries_bytes, void* stream) {
  tria_status st = check_skip_call(dims, ctx_len, cache, cache_bytes);
  if (st != TRIA_OK) return st;
  NONNULL(summaries);
  const int64_t need = tria::summaries_bytes(shape_of(dims), ctx_len);
  if ((int64_t)summaries_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "summaries need %lld bytes, got %zu", (long long)need, summaries_bytes);
  return launched(tria::launch_summaries(shape_of(dims), ctx_len, cache, (int64_t)cache_bytes, summaries,
                                         static_cast<hipStream_t>(stream)),
                  "summaries launch");
}

tria_status tria_skip_masks(const tria_dims* dims, const void* cache, size_t cache_bytes, int64_t ctx_len,
                            const void* summaries, size_t summaries_bytes, const void* q_bf16, const float* thresholds,
                            float sm_scale, uint32_t* masks, size_t masks_bytes, void* stream) {
  tria_status st = check_skip_call(dims, ctx_len, cache, cache_bytes);
  if (st != TRIA_OK) return st;
  NONNULL(summaries);
  NONNULL(q_bf16);
  NONNULL(thresholds);
  NONNULL(masks);
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return fail(TRIA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  const tria::Shape s = shape_of(dims);
  if ((int64_t)summaries_bytes < tria::summaries_bytes(s, ctx_len))
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "summaries smaller than tria_block_summaries_bytes");
  const int64_t need = 4LL * dims->batch * dims->n_kv_heads * ((ctx_len - 1) / dims->block + 1);
  if ((int64_t)masks_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "masks need %lld bytes, got %zu", (long long)need, masks_bytes);
  return launched(tria::launch_skip_masks(s, ctx_len, cache, (int64_t)cache_bytes, summaries, q_bf16, thresholds,
                                          sm_scale, masks, static_cast<hipStream_t>(stream)),
                  "skip masks launch");
}

tria_status tria_decode_skip_workspace_bytes(const tria_dims* dims, int64_t ctx_len, size_t* bytes) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(bytes);
  if (ctx_len < 1) return fail(TRIA_ERR_INVALID_ARG, "ctx_len must be >= 1");
  *bytes = (size_t)tria::skip_workspace_bytes(shape_of(dims), ctx_len);
  return ok();
}

tria_status tria_decode_skip(const tria_dims* dims, const void* cache, size_t cache_bytes, int64_t ctx_len,
                             const void* summaries, size_t summaries_bytes, const void* q_bf16,
                             const float* thresholds, float sm_scale, float* out, void* workspace, size_t ws_bytes,
                             void* stream) {
  tria_status st = check_skip_call(dims, ctx_len, cache, cache_bytes);
  if (st != TRIA_OK) return st;
  NONNULL(summaries);
  NONNULL(q_bf16);
  NONNULL(thresholds);
  NONNULL(out);
  NONNULL(workspace);
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return fail(TRIA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  const tria::Shape s = shape_of(dims);
  if ((int64_t)summaries_bytes < tria::summaries_bytes(s, ctx_len))
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "summaries smaller than tria_block_summaries_bytes");
  const int64_t need = tria::skip_workspace_bytes(s, ctx_len);
  if ((int64_t)ws_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "skip workspace needs %lld bytes, got %zu", (long long)need, ws_bytes);
  return launched(tria::launch_decode_skip(s, ctx_len, cache, (int64_t)cache_bytes, summaries, q_bf16, thresholds,
                                           sm_scale, out, workspace, static_cast<hipStream_t>(stream)),
                  "skip decode launch");
}

tria_status tria_pack_kv_cache_paged(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                     int32_t n_policy_heads, int64_t ctx_len, const void* k_bf16,
                                     const void* v_bf16, const void* table, size_t table_bytes,
                                     const void* old_table, size_t old_table_bytes, void* pool,
                                     size_t pool_bytes, void* stream) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(k_bf16);
  NONNULL(v_bf16);
  NONNULL(table);
  NONNULL(pool);
  if (ctx_len < 1 || ctx_len > dims->seq_len)
    return fail(TRIA_ERR_INVALID_ARG, "ctx_len %lld outside [1, seq_len=%lld]", (long long)ctx_len,
                (long long)dims->seq_len);
  if ((int64_t)dims->batch * dims->n_kv_heads > 65535)
    return fail(TRIA_ERR_UNSUPPORTED, "batch * n_kv_heads above 65535");
  tria::KvPolicy pol;
  st = kv_policy(dims, hi, keep, n_policy_heads, pol);
  if (st != TRIA_OK) return st;
  if ((int64_t)table_bytes < paged_table_bytes_of(dims, ctx_len))
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "table smaller than tria_paged_table_bytes");
  if (old_table && old_table_bytes < 64) return fail(TRIA_ERR_INVALID_ARG, "old table smaller than its header");
  const tria::CacheGeom g = cache_geom(dims, pol, ctx_len);
  if ((int64_t)pool_bytes < g.rec8_bytes) return fail(TRIA_ERR_BUFFER_TOO_SMALL, "pool smaller than one page");
  return launched(tria::launch_pack_paged(shape_of(dims), pol, g, k_bf16, v_bf16, table, (int64_t)table_bytes,
                                          old_table, (int64_t)old_table_bytes, pool, (int64_t)pool_bytes,
                                          static_cast<hipStream_t>(stream)),
                  "paged pack launch");
}

tria_status tria_decode_paged(const tria_dims* dims, const void* table, size_t table_bytes, const void* pool,
                              size_t pool_bytes, int64_t ctx_len, const void* q_bf16, float sm_scale, float* out,
                              void* workspace, size_t ws_bytes, void* stream) {
  tria_status st = check_skip_call(dims, ctx_len, table, table_bytes);
  if (st != TRIA_OK) return st;
  NONNULL(pool);
  NONNULL(q_bf16);
  NONNULL(out);
  NONNULL(workspace);
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return fail(TRIA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  const tria::Shape s = shape_of(dims);
  if ((int64_t)table_bytes < paged_table_bytes_of(dims, ctx_len))
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "table smaller than tria_paged_table_bytes");
  const int64_t need = tria::skip_workspace_bytes(s, ctx_len);
  if ((int64_t)ws_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "workspace needs %lld bytes, got %zu", (long long)need, ws_bytes);
  return launched(tria::launch_decode_paged(s, ctx_len, table, (int64_t)table_bytes, pool, (int64_t)pool_bytes,
                                            q_bf16, sm_scale, out, workspace, false, static_cast<hipStream_t>(stream)),
                  "paged decode launch");
}

tria_status tria_build_block_summaries_paged(const tria_dims* dims, const void* table, size_t table_bytes,
                                             const void* pool, size_t pool_bytes, int64_t ctx_len, void* summaries,
                                             size_t summaries_bytes, void* stream) {
  tria_status st = check_skip_call(dims, ctx_len, table, table_bytes);
  if (st != TRIA_OK) return st;
  NONNULL(pool);
  NONNULL(summaries);
  if ((int64_t)table_bytes < paged_table_bytes_of(dims, ctx_len))
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "table smaller than tria_paged_table_bytes");
  const int64_t need = tria::summaries_bytes(shape_of(dims), ctx_len);
  if ((int64_t)summaries_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "summaries need %lld bytes, got %zu", (long long)need, summaries_bytes);
  return launched(tria::launch_summaries_paged(shape_of(dims), ctx_len, table, (int64_t)table_bytes, summaries, pool,
                                               (int64_t)pool_bytes, false, static_cast<hipStream_t>(stream)),
                  "paged summaries launch");
}

tria_status tria_decode_skip_paged(const tria_dims* dims, const void* table, size_t table_bytes, const void* pool,
                                   size_t pool_bytes, int64_t ctx_len, const void* summaries, size_t summaries_bytes,
                                   const void* q_bf16, const float* thresholds, float sm_scale, float* out,
                                   void* workspace, size_t ws_bytes, void* stream) {
  tria_status st = check_skip_call(dims, ctx_len, table, table_bytes);
  if (st != TRIA_OK) return st;
  NONNULL(pool);
  NONNULL(summaries);
  NONNULL(q_bf16);
  NONNULL(thresholds);
  NONNULL(out);
  NONNULL(workspace);
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return fail(TRIA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  const tria::Shape s = shape_of(dims);
  if ((int64_t)table_bytes < paged_table_bytes_of(dims, ctx_len))
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "table smaller than tria_paged_table_bytes");
  if ((int64_t)summaries_bytes < tria::summaries_bytes(s, ctx_len))
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "summaries smaller than tria_block_summaries_bytes");
  const int64_t need = tria::skip_workspace_bytes(s, ctx_len);
  if ((int64_t)ws_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "skip workspace needs %lld bytes, got %zu", (long long)need, ws_bytes);
  return launched(tria::launch_decode_skip_paged(s, ctx_len, table, (int64_t)table_bytes, summaries, q_bf16,
                                                 thresholds, sm_scale, out, workspace, pool, (int64_t)pool_bytes,
                                                 false, static_cast<hipStream_t>(stream)),
                  "paged skip decode launch");
}

tria_status tria_build_block_summaries_varlen(const tria_dims* dims, const void* cache, size_t cache_bytes,
                                              void* summaries, size_t summaries_bytes, void* stream) {
  tria_status st = check_skip_call(dims, dims ? dims->seq_len : 1, cache, cache_bytes);
  if (st != TRIA_OK) return st;
  NONNULL(summaries);
  const int64_t need = tria::summaries_bytes(shape_of(dims), dims->seq_len);
  if ((int64_t)summaries_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "summaries need %lld bytes, got %zu", (long long)need, summaries_bytes);
  return launched(tria::launch_summaries_paged(shape_of(dims), dims->seq_len, cache, (int64_t)cache_bytes, summaries,
                                               nullptr, 0, true, static_cast<hipStream_t>(stream)),
                  "varlen summaries launch");
}

tria_status tria_decode_skip_varlen(const tria_dims* dims, const void* cache, size_t cache_bytes,
                                    const void* summaries, size_t summaries_bytes, const void* q_bf16,
                                    const float* thresholds, float sm_scale, float* out, void* workspace,
                                    size_t ws_bytes, void* stream) {
  tria_status st = check_skip_call(dims, dims ? dims->seq_len : 1, cache, cache_bytes);
  if (st != TRIA_OK) return st;
  NONNULL(summaries);
  NONNULL(q_bf16);
  NONNULL(thresholds);
  NONNULL(out);
  NONNULL(workspace);
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return fail(TRIA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  const tria::Shape s = shape_of(dims);
  if ((int64_t)summaries_bytes < tria::summaries_bytes(s, dims->seq_len))
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "summaries smaller than tria_block_summaries_bytes(seq_len)");
  const int64_t need = tria::skip_workspace_bytes(s, dims->seq_len);
  if ((int64_t)ws_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "skip workspace needs %lld bytes, got %zu", (long long)need, ws_bytes);
  return launched(tria::launch_decode_skip_paged(s, dims->seq_len, cache, (int64_t)cache_bytes, summaries, q_bf16,
                                                 thresholds, sm_scale, out, workspace, nullptr, 0, true,
                                                 static_cast<hipStream_t>(stream)),
                  "varlen skip decode launch");
}

tria_status tria_build_block_summaries_paged_varlen(const tria_dims* dims, const void* table, size_t table_bytes,
                                                    const void* pool, size_t pool_bytes, void* summaries,
                                                    size_t summaries_bytes, void* stream) {
  tria_status st = check_skip_call(dims, dims ? dims->seq_len : 1, table, table_bytes);
  if (st != TRIA_OK) return st;
  NONNULL(pool);
  NONNULL(summaries);
  const int64_t need = tria::summaries_bytes(shape_of(dims), dims->seq_len);
  if ((int64_t)summaries_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "summaries need %lld bytes, got %zu", (long long)need, summaries_bytes);
  return launched(tria::launch_summaries_paged(shape_of(dims), dims->seq_len, table, (int64_t)table_bytes, summaries,
                                               pool, (int64_t)pool_bytes, true, static_cast<hipStream_t>(stream)),
                  "paged varlen summaries launch");
}

tria_status tria_decode_skip_paged_varlen(const tria_dims* dims, const void* table, size_t table_bytes,
                                          const void* pool, size_t pool_bytes, const void* summaries,
                                          size_t summaries_bytes, const void* q_bf16, const float* thresholds,
                                          float sm_scale, float* out, void* workspace, size_t ws_bytes,
                                          void* stream) {
  tria_status st = check_skip_call(dims, dims ? dims->seq_len : 1, table, table_bytes);
  if (st != TRIA_OK) return st;
  NONNULL(pool);
  NONNULL(summaries);
  NONNULL(q_bf16);
  NONNULL(thresholds);
  NONNULL(out);
  NONNULL(workspace);
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return fail(TRIA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  const tria::Shape s = shape_of(dims);
  if ((int64_t)summaries_bytes < tria::summaries_bytes(s, dims->seq_len))
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "summaries smaller than tria_block_summaries_bytes(seq_len)");
  const int64_t need = tria::skip_workspace_bytes(s, dims->seq_len);
  if ((int64_t)ws_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "skip workspace needs %lld bytes, got %zu", (long long)need, ws_bytes);
  return launched(tria::launch_decode_skip_paged(s, dims->seq_len, table, (int64_t)table_bytes, summaries, q_bf16,
                                                 thresholds, sm_scale, out, workspace, pool, (int64_t)pool_bytes, true,
                                                 static_cast<hipStream_t>(stream)),
                  "paged varlen skip decode launch");
}

tria_status tria_pack_kv_cache_paged_varlen(const tria_dims* dims, const int32_t* hi, const int32_t* keep,
                                            int32_t n_policy_heads, const int64_t* ctx_lens, const void* k_bf16,
                                            const void* v_bf16, const void* table, size_t table_bytes,
                                            const void* old_table, size_t old_table_bytes, void* pool,
                                            size_t pool_bytes, void* stream) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(ctx_lens);
  NONNULL(k_bf16);
  NONNULL(v_bf16);
  NONNULL(table);
  NONNULL(pool);
  if (dims->batch > tria::kMaxVarlenBatch)
    return fail(TRIA_ERR_UNSUPPORTED, "batch above %d for a variable-length cache", tria::kMaxVarlenBatch);
  int64_t cmax = 1;
  for (int b = 0; b < dims->batch; ++b) {
    if (ctx_lens[b] < 1 || ctx_lens[b] > dims->seq_len)
      return fail(TRIA_ERR_INVALID_ARG, "ctx_lens[%d] = %lld outside [1, seq_len=%lld]", b, (long long)ctx_lens[b],
                  (long long)dims->seq_len);
    cmax = std::max(cmax, ctx_lens[b]);
  }
  tria::KvPolicy pol;
  st = kv_policy(dims, hi, keep, n_policy_heads, pol);
  if (st != TRIA_OK) return st;
  if ((int64_t)table_bytes < paged_table_bytes_of(dims, cmax))
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "table smaller than tria_paged_table_bytes(longest ctx_len)");
  if (old_table && old_table_bytes < 64) return fail(TRIA_ERR_INVALID_ARG, "old table smaller than its header");
  const tria::CacheGeom g = cache_geom(dims, pol, cmax);
  if ((int64_t)pool_bytes < g.rec8_bytes) return fail(TRIA_ERR_BUFFER_TOO_SMALL, "pool smaller than one page");
  return launched(tria::launch_pack_paged_varlen(shape_of(dims), pol, g, ctx_lens, k_bf16, v_bf16, table,
                                                 (int64_t)table_bytes, old_table, (int64_t)old_table_bytes, pool,
                                                 (int64_t)pool_bytes, static_cast<hipStream_t>(stream)),
                  "paged varlen pack launch");
}

tria_status tria_decode_paged_varlen(const tria_dims* dims, const void* table, size_t table_bytes, const void* pool,
                                     size_t pool_bytes, const void* q_bf16, float sm_scale, float* out,
                                     void* workspace, size_t ws_bytes, void* stream) {
  tria_status st = check_skip_call(dims, dims ? dims->seq_len : 1, table, table_bytes);
  if (st != TRIA_OK) return st;
  NONNULL(pool);
  NONNULL(q_bf16);
  NONNULL(out);
  NONNULL(workspace);
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return fail(TRIA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  const tria::Shape s = shape_of(dims);
  if ((int64_t)table_bytes < 64 + 64LL * dims->batch * dims->n_kv_heads)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "table smaller than its directory");
  const int64_t need = tria::skip_workspace_bytes(s, dims->seq_len);
  if ((int64_t)ws_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "workspace needs %lld bytes, got %zu", (long long)need, ws_bytes);
  return launched(tria::launch_decode_paged(s, 1, table, (int64_t)table_bytes, pool, (int64_t)pool_bytes, q_bf16,
                                            sm_scale, out, workspace, true, static_cast<hipStream_t>(stream)),
                  "paged varlen decode launch");
}

tria_status tria_decode_varlen(const tria_dims* dims, const void* cache, size_t cache_bytes, const void* q_bf16,
                               float sm_scale, float* out, void* workspace, size_t ws_bytes, void* stream) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(cache);
  NONNULL(q_bf16);
  NONNULL(out);
  NONNULL(workspace);
  if (!(sm_scale > 0.0f) || sm_scale > 1e30f) return fail(TRIA_ERR_INVALID_ARG, "sm_scale must be finite and > 0");
  const int G = dims->n_q_heads / dims->n_kv_heads;
  if (G > 32) return fail(TRIA_ERR_UNSUPPORTED, "more than 32 query heads per KV head");
  if ((int64_t)dims->batch * dims->n_kv_heads > 4096) return fail(TRIA_ERR_UNSUPPORTED, "batch * n_kv_heads above 4096");
  const int64_t dir_end = 64 + 64LL * dims->batch * dims->n_kv_heads;
  if ((int64_t)cache_bytes < dir_end) return fail(TRIA_ERR_BUFFER_TOO_SMALL, "cache smaller than its directory");
  const tria::Shape s = shape_of(dims);
  // sequences hold at most seq_len tokens each: the unit count is bounded with it
  if (!tria::decode_units_fit(s, dims->seq_len))
    return fail(TRIA_ERR_UNSUPPORTED, "batch * n_kv_heads * seq_len too large for one decode call");
  const int64_t need = tria::decode_workspace_bytes(s, dims->seq_len);
  if ((int64_t)ws_bytes < need)
    return fail(TRIA_ERR_BUFFER_TOO_SMALL, "decode workspace needs %lld bytes, got %zu", (long long)need, ws_bytes);
  return launched(tria::launch_decode(s, 1, cache, (int64_t)cache_bytes, q_bf16, sm_scale, out, workspace, true,
                                      static_cast<hipStream_t>(stream)),
                  "decode launch");
}

// ------------------------------------------------------------------ (f2) calibration
static tria_status check_costs(double c8, double c4) {
  if (!(c8 > 0.0) || !(c4 > 0.0) || !std::isfinite(c8) || !std::isfinite(c4))
    return fail(TRIA_ERR_INVALID_ARG, "pair costs must be finite and > 0");
  return TRIA_OK;
}

tria_status tria_policy_cost(const tria_dims* dims, int32_t hi, int32_t keep, double cost_int8, double cost_int4,
                             double* cost) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(cost);
  if (hi < 0 || keep < hi) return fail(TRIA_ERR_INVALID_ARG, "need 0 <= hi (%d) <= keep (%d)", hi, keep);
  st = check_costs(cost_int8, cost_int4);
  if (st != TRIA_OK) return st;
  *cost = policy_cost_of(dims, hi, keep, cost_int8, cost_int4);
  return ok();
}

tria_status tria_allocate_policy(const tria_dims* dims, int32_t n_heads, int32_t max_bound, const double* err,
                                 double cost_int8, double cost_int4, double budget, int32_t* hi_out,
                                 int32_t* keep_out, double* total_cost, double* total_err) {
  tria_status st = check_dims(dims);
  if (st != TRIA_OK) return st;
  NONNULL(err);
  NONNULL(hi_out);
  NONNULL(keep_out);
  if (n_heads < 1) return fail(TRIA_ERR_INVALID_ARG, "n_heads must be >= 1");
  if (max_bound < 0 || max_bound > 65535) return fail(TRIA_ERR_INVALID_ARG, "max_bound must be in [0, 65535]");
  st = check_costs(cost_int8, cost_int4);
  if (st != TRIA_OK) return st;
  if (!std::isfinite(budget)) return fail(TRIA_ERR_INVALID_ARG, "budget must be finite");
  const size_t S = (size_t)max_bound + 1;
  for (size_t h = 0; h < (size_t)n_heads; ++h)
    for (size_t a = 0; a < S; ++a)
      for (size_t k = a; k < S; ++k)
        if (!std::isfinite(err[(h * S + a) * S + k]))
          return fail(TRIA_ERR_INVALID_ARG, "err[%zu][%zu][%zu] is not finite", h, a, k);
  auto E = [&](int h, int a, int k) { return err[((size_t)h * S + a) * S + k]; };
  std::vector<double> ctab(S * S, -1.0);  // cost per (hi, keep): the same for every head
  auto C = [&](int a, int k) {
    double& c = ctab[(size_t)a * S + k];
    if (c < 0.0) c = policy_cost_of(dims, a, k, cost_int8, cost_int4);
    return c;
  };
  std::vector<int> hi(n_heads, 0), kp(n_heads, 0);
  std::vector<unsigned> ver(n_heads, 0);
  double total = 0.0;
  for (int h = 0; h < n_heads; ++h) total += C(0, 0);
  if (total > budget)
    return fail(TRIA_ERR_INVALID_ARG, "budget %.17g is below the protected-only cost %.17g", budget, total);
  // Greedy: every head starts at (0, 0); a step raises one head's keep by one block
  // (move 0: one more block kept, at int4) or its hi by one (move 1: one more block at
  // int8, keep raised with it when equal), choosing the move with the largest error
  // reduction per unit of added cost among those that fit the budget (a reduction at
  // no cost first; ties by head, then move).  Moves that reduce no error are never
  // taken.  Candidates live in a heap; a head's entries are dropped once it moves.
  struct Cand {
    double score;
    int h, move;
    unsigned ver;
  };
  auto worse = [](const Cand& x, const Cand& y) {
    if (x.score != y.score) return x.score < y.score;
    if (x.h != y.h) return x.h > y.h;
    return x.move > y.move;
  };
  std::priority_queue<Cand, std::vector<Cand>, decltype(worse)> heap(worse);
  auto target = [&](int h, int move, int& a, int& k) {
    a = hi[h];
    k = kp[h];
    if (move == 0) {
      if (k >= max_bound) return false;
      ++k;
    } else {
      if (a >= max_bound) return false;
      ++a;
      k = std::max(k, a);
    }
    return true;
  };
  auto push = [&](int h) {
    for (int move = 0; move < 2; ++move) {
      int a, k;
      if (!target(h, move, a, k)) continue;
      const double de = E(h, hi[h], kp[h]) - E(h, a, k);
      if (!(de > 0.0)) continue;
      const double dc = C(a, k) - C(hi[h], kp[h]);
      heap.push(Cand{dc > 0.0 ? de / dc : INFINITY, h, move, ver[h]});
    }
  };
  for (int h = 0; h < n_heads; ++h) push(h);
  while (!heap.empty()) {
    const Cand c = heap.top();
    heap.pop();
    if (c.ver != ver[c.h]) continue;
    int a, k;
    target(c.h, c.move, a, k);
    const double dc = C(a, k) - C(hi[c.h], kp[c.h]);
    if (total + dc > budget) continue;  // stays out of budget: totals only grow
    total += dc;
    hi[c.h] = a;
    kp[c.h] = k;
    ++ver[c.h];
    push(c.h);
  }
  double esum = 0.0;
  for (int h = 0; h < n_heads; ++h) {
    hi_out[h] = hi[h];
    keep_out[h] = kp[h];
    esum += E(h, hi[h], kp[h]);
  }
  if (total_cost) *total_cost = total;
  if (total_err) *total_err = esum;
  return ok();
}

tria_status tria_peak_mfma(int32_t kind, int32_t iters, int32_t* sink, double* work, void* stream) {
  NONNULL(sink);
  NONNULL(work);
  if (kind != 0 && kind != 1) return fail(TRIA_ERR_INVALID_ARG, "kind must be 0 (int8) or 1 (bf16)");
  if (iters < 1) return fail(TRIA_ERR_INVALID_ARG, "iters must be >= 1");
  *work = tria::peak_mfma_work(kind, iters);
  return launched(tria::launch_peak_mfma(kind, iters, sink, static_cast<hipStream_t>(stream)), "peak mfma launch");
}

tria_status tria_peak_read(const void* src, int64_t bytes, int32_t* sink, double* work, void* stream) {
  NONNULL(src);
  NONNULL(sink);
  NONNULL(work);
  const int64_t align = tria::peak_read_align();
  if (bytes <= 0 || bytes % align != 0)
    return fail(TRIA_ERR_INVALID_ARG, "bytes must be a positive multiple of %lld", (long long)align);
  if (bytes / TRIA_PEAK_READ_WAVES > INT32_MAX) return fail(TRIA_ERR_UNSUPPORTED, "bytes too large");
  *work = (double)bytes;
  return launched(tria::launch_peak_read(src, bytes, sink, static_cast<hipStream_t>(stream)), "peak read launch");
}

}  // extern "C"
