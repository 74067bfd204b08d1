// pack.hip - builds the compressed mixed-precision KV cache for one query position.
//
// TriAttention summary page (rit.work), section on calibration: the prepared keys
// and values go to a compressed KV cache so that generation reads less of it; the
// section on infrastructure plans adds that this needs its own cache layout.  For
// query position t = ctx_len - 1 (current block c) and the KV head's (hi, keep),
// the stored blocks are the ones the tile rule keeps for query block c: block 0
// and blocks within hi of c at int8, blocks within keep at int4, nothing else.
// Every K and V row of a stored block is quantised per row at its block's
// precision (same contract as the Q/K quantiser).
//
// Layout (bytes, documented in tria.h): header, one 64-byte directory entry per
// (batch, KV head), then per pair its int8 records and its int4 records.  A record
// is B/32 chunks of 32 tokens, each self-contained: the K codes in the order of the
// decode kernel's matrix operand, the V codes transposed with the tokens in the
// order its bf16 MFMA consumes them, then the chunk's K and V scales.  K and V are
// sequences of 16-byte lane units, so one decode step reads one contiguous chunk
// with full 1 KB loads.
//
// One work group per stored block (grid x = block slot in the pair, y = pair); each
// group computes its record offset from the policy (every batch element has the
// same layout because the policy is per KV head).  V codes go through LDS for the
// transpose.
//
// Update (the cache for ctx_len from the one for ctx_len - 1, same policy and K/V):
// a block's record depends only on its rows and its precision, so a record of a
// block before the new current block that the old layout stored at the same
// precision is reused (left alone in place at an unchanged offset, else copied);
// every other record (the current block, a block demoted from int8 to int4) is
// quantised from the bf16 rows as above.  Within a block nothing moves and only the
// new token's row of the current block changes: in place, one wavefront per pair
// quantises that K and V row and writes its bytes into the record (append kernel).
#include "device_common.h"
#include "kernels.h"

namespace tria {

namespace {

constexpr int kThreads = 256;

struct PackArgs {
  const uint16_t* k;
  const uint16_t* v;
  uint8_t* cache;
  const uint8_t* old;  // update: the cache for ctx_len - 1 (else null), geometry ogeo
  CacheGeom ogeo;
  int only_current;    // update in place within the current block: the new token's row only
  int varlen;          // per-sequence lengths ctxs[b] (the directory is written first)
  int64_t ctxs[kMaxVarlenBatch];
  int64_t n;  // token rows in the K/V source
  int batch, hkv;
  KvPolicy pol;
  CacheGeom geo;
  // paged cache: records go to pool + page * page_bytes by the version-4 table for
  // geo.ctx_len (else null); old_table (or null): the table the pool holds
  const uint8_t* table;
  const uint8_t* old_table;
  int64_t table_bytes, old_table_bytes, pool_pages, page_bytes;
  uint8_t* pool;
};

struct Blocks {  // the stored set of one KV head for current block c
  int lo8, sink, n8, lo4, hi4, n4;
};

__device__ __forceinline__ Blocks stored_blocks(int c, int hi, int keep) {
  Blocks s;
  s.lo8 = (c - hi >= 2) ? c - hi : 0;  // block 0 joins the run when adjacent
  s.sink = s.lo8 > 0 ? 1 : 0;
  s.n8 = c - s.lo8 + 1 + s.sink;
  s.lo4 = c - keep > 1 ? c - keep : 1;
  s.hi4 = c - hi - 1;
  if (s.lo4 > s.hi4) {
    s.lo4 = 0;
    s.hi4 = -1;
  }
  s.n4 = s.hi4 - s.lo4 + 1;
  return s;
}

// token held at position 8q + p of a 32-token chunk in the transposed V layout
__device__ __forceinline__ int feed_token(int q, int p) { return 16 * (p >> 2) + 4 * q + (p & 3); }

// 8 sign-extended int4 codes (bytes) -> 4 packed bytes, low nibble = even element
__device__ __forceinline__ uint32_t pack8_nibbles(uint32_t lo, uint32_t hi) {
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t e = ((i < 2 ? lo : hi) >> (16 * (i & 1))) & 0xFFFFu;  // elements 2i, 2i+1
    r |= ((e & 0xFu) | (((e >> 8) & 0xFu) << 4)) << (8 * i);
  }
  return r;
}

// ctx_len of pair p in a variable-length page table (entry words 10-11).
__device__ __forceinline__ int64_t table_ctx(const uint8_t* table, int p) {
  return *reinterpret_cast<const int64_t*>(table + 64 + 64 * (int64_t)p + 40);
}

// Record slot j of pair `pair` (the whole work group; every early return is uniform).
template <int D, int BLK>
__device__ __forceinline__ void pack_record(const PackArgs& a, int pair, int j) {
  constexpr int TPR = D / 8;
  constexpr int RPP = kThreads / TPR;  // rows per pass
  __shared__ __attribute__((aligned(16))) int8_t kbuf[BLK][D];  // codes (int4: sign-extended bytes)
  __shared__ __attribute__((aligned(16))) int8_t vbuf[BLK][D];
  __shared__ float ksb[BLK], vsb[BLK];

  const int b = pair / a.hkv, g = pair % a.hkv;
  const int64_t ctx = a.varlen ? a.ctxs[b] : a.geo.ctx_len;
  const int c = a.varlen ? (int)((ctx - 1) / BLK) : a.geo.cur_block;
  const Blocks st = stored_blocks(c, a.pol.hi[g], a.pol.keep[g]);
  if (j >= st.n8 + st.n4) return;
  auto pair_offset = [&](const CacheGeom& geo) {
    int64_t off = geo.data_offset + (int64_t)b * geo.batch_bytes;
    for (int gg = 0; gg < g; ++gg) {
      const Blocks o = stored_blocks(geo.cur_block, a.pol.hi[gg], a.pol.keep[gg]);
      off += (int64_t)o.n8 * geo.rec8_bytes + (int64_t)o.n4 * geo.rec4_bytes;
    }
    return off;
  };
  // variable lengths: the pair's offset from the directory (written by the
  // directory kernel before this launch)
  const int64_t pair_off = a.table ? 0
                           : a.varlen ? *reinterpret_cast<const int64_t*>(a.cache + 64 + 64 * (int64_t)pair)
                                      : pair_offset(a.geo);
  const bool is4 = j >= st.n8;
  const int kb = !is4 ? ((st.sink && j == 0) ? 0 : st.lo8 + j - st.sink) : st.lo4 + (j - st.n8);
  const int64_t off = !is4 ? pair_off + (int64_t)j * a.geo.rec8_bytes
                           : pair_off + (int64_t)st.n8 * a.geo.rec8_bytes + (int64_t)(j - st.n8) * a.geo.rec4_bytes;
  uint8_t* rec = a.cache + off;
  const int tid = threadIdx.x;

  if (a.table) {  // paged: the record's page from the table (checked), nothing else written
    const int P = a.batch * a.hkv;
    const int32_t* th = reinterpret_cast<const int32_t*>(a.table);
    const int64_t* th64 = reinterpret_cast<const int64_t*>(a.table);
    const int rmax = th[6];
    // fixed length: one ctx_len in the header; variable length: each entry's own
    const bool kind_ok = a.varlen ? th[7] == -1 && th64[4] == 0 && table_ctx(a.table, pair) == ctx
                                  : th[7] == c && th64[4] == ctx && rmax == c + 1;
    if (th[0] != 0x50564B54 || th[1] != 4 || th[2] != a.batch || th[3] != a.hkv || th[4] != D || th[5] != BLK ||
        !kind_ok || rmax < c + 1 || th64[5] != a.page_bytes || 64 + 64LL * P + 4LL * P * rmax > a.table_bytes)
      return;
    const int32_t* e = th + 16 + 16 * pair;
    if (e[2] != st.n8 || e[3] != st.n4) return;
    const int page = th[16 + 16 * P + pair * rmax + j];
    if (page < 0 || page >= a.pool_pages) return;
    rec = a.pool + (int64_t)page * a.page_bytes;
    if (a.old_table && kb < c) {  // a record the pool already holds at this page
      const int32_t* oh = reinterpret_cast<const int32_t*>(a.old_table);
      const int orm = oh[6];
      const int64_t octx = a.varlen ? table_ctx(a.old_table, pair) : reinterpret_cast<const int64_t*>(a.old_table)[4];
      const int oc = octx >= 1 ? (int)((octx - 1) / BLK) : -1;
      if (oh[0] == 0x50564B54 && oh[1] == 4 && oh[2] == a.batch && oh[3] == a.hkv && oh[4] == D && oh[5] == BLK &&
          (a.varlen ? oh[7] == -1 : oh[7] == oc) && oc >= 0 && oc < orm && octx <= ctx &&
          64 + 64LL * P + 4LL * P * orm <= a.old_table_bytes) {
        const Blocks so = stored_blocks(oc, a.pol.hi[g], a.pol.keep[g]);
        int jo = -1;
        if (!is4) {
          if (kb == 0 && so.sink) jo = 0;
          else if (kb >= so.lo8 && kb <= oc) jo = so.sink + kb - so.lo8;
          if (kb == oc && octx != (int64_t)(oc + 1) * BLK) jo = -1;  // the old current block, not yet full
        } else if (kb >= so.lo4 && kb <= so.hi4) {
          jo = so.n8 + kb - so.lo4;
        }
        if (jo >= 0 && oh[16 + 16 * P + pair * orm + jo] == page) return;
      }
    }
  }

  if (j == 0 && tid == 0 && !a.varlen && !a.table) {
    int32_t* e = reinterpret_cast<int32_t*>(a.cache + 64 + 64 * (int64_t)pair);
    *reinterpret_cast<int64_t*>(e) = pair_off;
    e[2] = st.n8;
    e[3] = st.n4;
    e[4] = a.pol.hi[g];
    e[5] = a.pol.keep[g];
    e[6] = st.lo8;
    e[7] = st.sink;
    e[8] = st.lo4;
    e[9] = st.hi4;
    e[10] = e[11] = e[12] = e[13] = e[14] = e[15] = 0;
    if (pair == 0) {
      int32_t* hd = reinterpret_cast<int32_t*>(a.cache);
      hd[0] = 0x43564B54;  // "TKVC"
      hd[1] = 2;  // format version
      hd[2] = a.batch;
      hd[3] = a.hkv;
      hd[4] = D;
      hd[5] = BLK;
      hd[6] = c + 1;
      hd[7] = c;
      int64_t* h64 = reinterpret_cast<int64_t*>(a.cache);
      h64[4] = a.geo.ctx_len;
      h64[5] = a.geo.total_bytes;
      h64[6] = 64;
      h64[7] = a.geo.data_offset;
    }
  }

  if (pair == 0 && j == 0 && !a.varlen && !a.table) {  // the padding between the directory and the first record
    const int64_t pad0 = 64 + 64LL * a.batch * a.hkv;
    for (int64_t i = pad0 + tid; i < a.geo.data_offset; i += kThreads) a.cache[i] = 0;
  }

  if (a.old != nullptr && kb < c) {  // update: reuse the old record when it has this block and precision
    const Blocks so = stored_blocks(a.ogeo.cur_block, a.pol.hi[g], a.pol.keep[g]);
    int jo = -1;
    if (!is4) {
      if (kb == 0 && so.sink) jo = 0;
      else if (kb >= so.lo8 && kb <= a.ogeo.cur_block) jo = so.sink + kb - so.lo8;
    } else if (kb >= so.lo4 && kb <= so.hi4) {
      jo = so.n8 + kb - so.lo4;
    }
    if (jo >= 0) {
      const int64_t opair = pair_offset(a.ogeo);
      const int64_t ooff = !is4 ? opair + (int64_t)jo * a.ogeo.rec8_bytes
                                : opair + (int64_t)so.n8 * a.ogeo.rec8_bytes + (int64_t)(jo - so.n8) * a.ogeo.rec4_bytes;
      if (a.old == a.cache && ooff == off) return;  // in place, same bytes
      const int64_t n16 = (!is4 ? a.geo.rec8_bytes : a.geo.rec4_bytes) / 16;
      const uint4* src = reinterpret_cast<const uint4*>(a.old + ooff);
      uint4* dst = reinterpret_cast<uint4*>(rec);
      for (int64_t i = tid; i < n16; i += kThreads) dst[i] = src[i];
      return;
    }
  }

  const int64_t src0 = ((int64_t)b * a.hkv + g) * a.n;
  const int part = tid % TPR;
  // int4 codes as sign-extended bytes
  auto widen4 = [](uint32_t w, uint32_t& e0, uint32_t& e1) {
    e0 = e1 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int code = ((int)(w << (28 - 4 * i))) >> 28;
      if (i < 4) e0 |= ((uint32_t)code & 0xFFu) << (8 * i);
      else e1 |= ((uint32_t)code & 0xFFu) << (8 * (i - 4));
    }
  };
#pragma unroll 1
  for (int p = 0; p < BLK / RPP; ++p) {
    const int r = p * RPP + tid / TPR;
    const int64_t tok = (int64_t)kb * BLK + r;
    const bool valid = tok < ctx;
    float xk[8], xv[8];
    uint4 rk = make_uint4(0, 0, 0, 0), rv = make_uint4(0, 0, 0, 0);
    if (valid) {
      rk = *reinterpret_cast<const uint4*>(a.k + (src0 + tok) * D + part * 8);
      rv = *reinterpret_cast<const uint4*>(a.v + (src0 + tok) * D + part * 8);
    }
    bf16x8_to_f32(rk, xk);
    bf16x8_to_f32(rv, xv);
    uint32_t k8w[2], k4w, v8w[2], v4w;
    float ks8, ks4, vs8, vs4;
    quantize8<TPR>(xk, k8w, k4w, ks8, ks4);
    quantize8<TPR>(xv, v8w, v4w, vs8, vs4);
    if (!is4) {
      *reinterpret_cast<uint2*>(&kbuf[r][part * 8]) = make_uint2(k8w[0], k8w[1]);
      *reinterpret_cast<uint2*>(&vbuf[r][part * 8]) = make_uint2(v8w[0], v8w[1]);
    } else {
      uint32_t e0, e1;
      widen4(k4w, e0, e1);
      *reinterpret_cast<uint2*>(&kbuf[r][part * 8]) = make_uint2(e0, e1);
      widen4(v4w, e0, e1);
      *reinterpret_cast<uint2*>(&vbuf[r][part * 8]) = make_uint2(e0, e1);
    }
    if (part == 0) {
      ksb[r] = is4 ? ks4 : ks8;
      vsb[r] = is4 ? vs4 : vs8;
    }
  }
  __syncthreads();
  // the record, chunk by chunk, in 16-byte pieces
  constexpr int KSL = D / 64;
  const int kpart = is4 ? 16 * D : 32 * D;    // bytes of the K (and of the V) part of a chunk
  const int cbytes = 2 * kpart + 256;
  const int npieces = (BLK / 32) * cbytes / 16;
  for (int pc = tid; pc < npieces; pc += kThreads) {
    const int c = pc / (cbytes / 16), o = (pc % (cbytes / 16)) * 16;  // chunk, byte offset in it
    uint32_t w[4];
    if (o < kpart) {
      if (!is4) {
        // unit (s, ks, q, r): dims 64ks + 16q .. +15 of token 32c + 16s + r
        const int u = o / 16;
        const int r = u % 16, q = (u / 16) % 4, kk = (u / 64) % KSL, sub = u / (64 * KSL);
        const uint4 x = *reinterpret_cast<const uint4*>(&kbuf[32 * c + 16 * sub + r][64 * kk + 16 * q]);
        w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
      } else {
        // unit (s, q, r) of 8 * KSL bytes: for each ks, dims 64ks + 16q .. +15 packed
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // the piece's two 8-byte halves
          const int e = o / 8 + h;       // 8-byte index in the K part
          const int u = e / KSL, kk = e % KSL;
          const int r = u % 16, q = (u / 16) % 4, sub = u / 64;
          const uint4 x = *reinterpret_cast<const uint4*>(&kbuf[32 * c + 16 * sub + r][64 * kk + 16 * q]);
          w[2 * h] = pack8_nibbles(x.x, x.y);
          w[2 * h + 1] = pack8_nibbles(x.z, x.w);
        }
      }
    } else if (o < 2 * kpart) {
      // unit (m, q, r): for dim groups dt = per*m .. per*m + per - 1, the 8 positions p
      // of dim 16dt + r (token 32c + feed_token(q, p)); int8: 8 bytes, int4: 4 bytes
      const int u = (o - kpart) / 16;
      const int r = u % 16, q = (u / 16) % 4, m = u / 64;
      const int per = is4 ? 4 : 2;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t >= per) break;
        const int dim = 16 * (per * m + t) + r;
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int pp = 0; pp < 8; ++pp) {
          const uint32_t x = (uint8_t)vbuf[32 * c + feed_token(q, pp)][dim];
          if (pp < 4) lo |= x << (8 * pp);
          else hi |= x << (8 * (pp - 4));
        }
        if (!is4) {
          w[2 * t] = lo;
          w[2 * t + 1] = hi;
        } else {
          w[t] = pack8_nibbles(lo, hi);
        }
      }
    } else {
      // scales: K scales of the chunk's 32 tokens, then V scales
      const int t0 = (o - 2 * kpart) / 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + i;
        w[i] = __float_as_uint(t < 32 ? ksb[32 * c + t] : vsb[32 * c + t - 32]);
      }
    }
    *reinterpret_cast<uint4*>(rec + (int64_t)c * cbytes + o) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <int D, int BLK>
__global__ void __launch_bounds__(kThreads) pack_kernel(PackArgs a) {
  pack_record<D, BLK>(a, blockIdx.y, blockIdx.x);
}

template <int D, int BLK>
__device__ __forceinline__ void append_row(const PackArgs& a, uint8_t* rec, int b, int g, int64_t t, int c, int lane);

// Paged update (an old table given): work group x of pair y writes the pair's new
// records number x, x + gridDim.x, ... in record order, where a record is new unless
// it lies before the current block and the old table maps the same (block,
// precision) to the same page (the test pack_record repeats before writing).  When
// both tables hold the same current block at the same page and the old one is
// shorter, only the rows it lacks are written (work group 0, a wavefront per row).
template <int D, int BLK>
__global__ void __launch_bounds__(kThreads) paged_update_kernel(PackArgs a) {
  __shared__ int tmp[2 * (kThreads / 64)];
  __shared__ int list[kThreads];
  const int pair = blockIdx.y, g = pair % a.hkv, tid = threadIdx.x;
  const int P = a.batch * a.hkv;
  const int64_t ctx = a.varlen ? a.ctxs[pair / a.hkv] : a.geo.ctx_len;
  const int c = (int)((ctx - 1) / BLK);
  const Blocks st = stored_blocks(c, a.pol.hi[g], a.pol.keep[g]);
  const int32_t* th = reinterpret_cast<const int32_t*>(a.table);
  const int32_t* oh = reinterpret_cast<const int32_t*>(a.old_table);
  const int rmax = th[6], orm = oh[6];
  const int64_t octx = a.varlen ? table_ctx(a.old_table, pair) : reinterpret_cast<const int64_t*>(a.old_table)[4];
  const int oc = octx >= 1 ? (int)((octx - 1) / BLK) : -1;
  // both tables of this kind and shape (pack_record checks the new one fully before writing)
  const bool new_ok = th[0] == 0x50564B54 && th[1] == 4 && rmax >= c + 1 && (a.varlen ? th[7] == -1 : th[7] == c) &&
                      64 + 64LL * P + 4LL * P * rmax <= a.table_bytes;
  const bool old_ok = new_ok && oh[0] == 0x50564B54 && oh[1] == 4 && oh[2] == a.batch && oh[3] == a.hkv &&
                      oh[4] == D && oh[5] == BLK && (a.varlen ? oh[7] == -1 : oh[7] == oc) && oc >= 0 && oc < orm &&
                      octx <= ctx && 64 + 64LL * P + 4LL * P * orm <= a.old_table_bytes;
  if (!new_ok) return;
  const Blocks so = stored_blocks(old_ok ? oc : 0, a.pol.hi[g], a.pol.keep[g]);
  const int cur_page = th[16 + 16 * P + pair * rmax + st.n8 - 1];
  const bool same_cur = old_ok && oc == c && so.n8 == st.n8 && octx >= (int64_t)c * BLK + 1 && octx < ctx &&
                        oh[16 + 16 * P + pair * orm + so.n8 - 1] == cur_page && cur_page >= 0 &&
                        cur_page < a.pool_pages && (!a.varlen || table_ctx(a.table, pair) == ctx);
  if (same_cur && blockIdx.x == 0) {
    const int b = pair / a.hkv, wave = tid >> 6, lane = tid & 63;
    uint8_t* rec = a.pool + (int64_t)cur_page * a.page_bytes;
    for (int64_t t = octx + wave; t < ctx; t += kThreads / 64) append_row<D, BLK>(a, rec, b, g, t, c, lane);
  }
  int done = 0;  // new records seen before this chunk
  for (int j0 = 0; j0 < st.n8 + st.n4; j0 += kThreads) {
    const int j = j0 + tid;
    int fresh = 0;
    if (j < st.n8 + st.n4) {
      fresh = 1;
      const bool is4 = j >= st.n8;
      const int kb = !is4 ? ((st.sink && j == 0) ? 0 : st.lo8 + j - st.sink) : st.lo4 + (j - st.n8);
      if (same_cur && kb == c) fresh = 0;  // its new rows are written above
      if (old_ok && kb < c) {
        int jo = -1;
        if (!is4) {
          if (kb == 0 && so.sink) jo = 0;
          else if (kb >= so.lo8 && kb <= oc) jo = so.sink + kb - so.lo8;
          if (kb == oc && octx != (int64_t)(oc + 1) * BLK) jo = -1;  // the old current block, not yet full
        } else if (kb >= so.lo4 && kb <= so.hi4) {
          jo = so.n8 + kb - so.lo4;
        }
        if (jo >= 0 && oh[16 + 16 * P + pair * orm + jo] == th[16 + 16 * P + pair * rmax + j]) fresh = 0;
      }
    }
    // exclusive prefix of the flags over the work group
    const int lane = tid & 63, wave = tid >> 6;
    int incl = fresh;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) tmp[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) {
      before += w < wave ? tmp[w] : 0;
      total += tmp[w];
    }
    if (fresh) list[before + incl - fresh] = j;
    __syncthreads();
    // this work group's share of the chunk's new records
    for (int k = 0; k < total; ++k)
      if ((done + k) % (int)gridDim.x == (int)blockIdx.x) pack_record<D, BLK>(a, pair, list[k]);
    done += total;
    __syncthreads();
  }
}

// Variable-length batch: one work group writes the header (version 3) and every
// pair's directory entry from the per-sequence lengths; each entry also holds its
// sequence's ctx_len (words 10-11).  Offsets are the running sum of the pairs'
// record bytes in (b, g) order.
template <int D, int BLK>
__global__ void __launch_bounds__(kThreads) varlen_directory_kernel(PackArgs a) {
  __shared__ int64_t part[kThreads];
  const int tid = threadIdx.x;
  const int P = a.batch * a.hkv;
  int64_t carry = a.geo.data_offset;
  for (int base = 0; base < P; base += kThreads) {
    const int p = base + tid;
    int64_t bytes = 0;
    Blocks st{};
    int64_t ctx = 1;
    if (p < P) {
      const int b = p / a.hkv, g = p % a.hkv;
      ctx = a.ctxs[b];
      st = stored_blocks((int)((ctx - 1) / BLK), a.pol.hi[g], a.pol.keep[g]);
      bytes = (int64_t)st.n8 * a.geo.rec8_bytes + (int64_t)st.n4 * a.geo.rec4_bytes;
    }
    part[tid] = bytes;
    __syncthreads();
    int64_t before = 0, total = 0;  // exclusive prefix inside this chunk (plain loop: one group)
    for (int i = 0; i < kThreads; ++i) {
      before += i < tid ? part[i] : 0;
      total += part[i];
    }
    if (p < P) {
      const int g = p % a.hkv;
      int32_t* e = reinterpret_cast<int32_t*>(a.cache + 64 + 64 * (int64_t)p);
      *reinterpret_cast<int64_t*>(e) = carry + before;
      e[2] = st.n8;
      e[3] = st.n4;
      e[4] = a.pol.hi[g];
      e[5] = a.pol.keep[g];
      e[6] = st.lo8;
      e[7] = st.sink;
      e[8] = st.lo4;
      e[9] = st.hi4;
      *reinterpret_cast<int64_t*>(e + 10) = ctx;
      e[12] = e[13] = e[14] = e[15] = 0;
    }
    carry += total;
    __syncthreads();
  }
  if (tid == 0) {
    int32_t* hd = reinterpret_cast<int32_t*>(a.cache);
    hd[0] = 0x43564B54;  // "TKVC"
    hd[1] = 3;           // format version: per-pair ctx_len
    hd[2] = a.batch;
    hd[3] = a.hkv;
    hd[4] = D;
    hd[5] = BLK;
    hd[6] = a.geo.cur_block + 1;  // blocks of the longest sequence
    hd[7] = -1;                   // the current block varies by sequence
    int64_t* h64 = reinterpret_cast<int64_t*>(a.cache);
    h64[4] = 0;
    h64[5] = a.geo.total_bytes;
    h64[6] = 64;
    h64[7] = a.geo.data_offset;
  }
  const int64_t pad0 = 64 + 64LL * a.batch * a.hkv;
  for (int64_t i = pad0 + tid; i < a.geo.data_offset; i += kThreads) a.cache[i] = 0;
}

// In place within the current block: token t = ctx_len - 1 (row r of block c, chunk
// r / 32, position tk = r % 32) is the only change.  Lanes [0, TPR) quantise its K
// row, lanes [TPR, 2 TPR) its V row, eight dims each (the quantiser contract of the
// packer); K codes go to their operand-order unit (half of a 16-byte unit), V codes
// byte by byte to their transposed positions, then the two scales and the header's
// ctx_len.  Rows past t are already zero in a cache packed for ctx_len - 1.
// Token t (in current block c) of pair (b, g): its K and V rows quantised at int8 and
// written into the block's int8 record `rec` (one wavefront, lanes 0..63).
template <int D, int BLK>
__device__ __forceinline__ void append_row(const PackArgs& a, uint8_t* rec, int b, int g, int64_t t, int c, int lane) {
  constexpr int TPR = D / 8, KSL = D / 64;
  constexpr int KPART = 32 * D, CBYTES = 2 * KPART + 256;
  const int r = (int)(t - (int64_t)c * BLK), cc = r / 32, tk = r % 32;
  uint8_t* chunk = rec + (int64_t)cc * CBYTES;
  const bool isv = lane >= TPR;
  const int part = lane % TPR;
  const int64_t src = (((int64_t)b * a.hkv + g) * a.n + t) * D + part * 8;
  uint4 raw = make_uint4(0, 0, 0, 0);
  if (lane < 2 * TPR) raw = *reinterpret_cast<const uint4*>((isv ? a.v : a.k) + src);
  float x[8];
  bf16x8_to_f32(raw, x);
  uint32_t w8[2], w4;
  float s8, s4;
  quantize8<TPR>(x, w8, w4, s8, s4);
  if (lane < TPR) {
    // dims 8 part .. +7 = half (part % 2) of unit (s, ks, q, rr) of token 16 s + rr
    const int dim0 = part * 8, ks = dim0 / 64, q = (dim0 % 64) / 16;
    const int u = (((tk / 16) * KSL + ks) * 4 + q) * 16 + tk % 16;
    *reinterpret_cast<uint2*>(chunk + u * 16 + (part % 2) * 8) = make_uint2(w8[0], w8[1]);
    if (part == 0) *reinterpret_cast<float*>(chunk + 2 * KPART + 4 * tk) = s8;
  } else if (lane < 2 * TPR) {
    // byte p of unit (m, qv, rr) holds dim 16 dt + rr (dt = 2m, 2m + 1) of the token
    // at feed position 8 qv + p; for this token qv = (tk % 16) / 4, p = 4 (tk / 16) + tk % 4
    const int qv = (tk % 16) / 4, p = 4 * (tk / 16) + tk % 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int dim = part * 8 + i, dt = dim / 16, rr = dim % 16;
      const int u = ((dt / 2) * 4 + qv) * 16 + rr;
      chunk[KPART + u * 16 + (dt % 2) * 8 + p] = (uint8_t)(w8[i / 4] >> (8 * (i % 4)));
    }
    if (part == 0) *reinterpret_cast<float*>(chunk + 2 * KPART + 4 * (32 + tk)) = s8;
  }
}

template <int D, int BLK>
__global__ void __launch_bounds__(64) append_kernel(PackArgs a) {
  const int pair = blockIdx.x, lane = threadIdx.x;
  const int b = pair / a.hkv, g = pair % a.hkv;
  const int c = a.geo.cur_block;
  int64_t pair_off = a.geo.data_offset + (int64_t)b * a.geo.batch_bytes;
  for (int gg = 0; gg < g; ++gg) {
    const Blocks o = stored_blocks(c, a.pol.hi[gg], a.pol.keep[gg]);
    pair_off += (int64_t)o.n8 * a.geo.rec8_bytes + (int64_t)o.n4 * a.geo.rec4_bytes;
  }
  const Blocks st = stored_blocks(c, a.pol.hi[g], a.pol.keep[g]);
  append_row<D, BLK>(a, a.cache + pair_off + (int64_t)(st.n8 - 1) * a.geo.rec8_bytes, b, g, a.geo.ctx_len - 1, c,
                     lane);
  if (pair == 0 && lane == 0) reinterpret_cast<int64_t*>(a.cache)[4] = a.geo.ctx_len;
}


template <int D, int BLK>
hipError_t launch_t(const PackArgs& a, int max_stored, hipStream_t stream) {
  if (a.only_current) {
    hipLaunchKernelGGL((append_kernel<D, BLK>), dim3(a.batch * a.hkv), dim3(64), 0, stream, a);
    return hipGetLastError();
  }
  if (a.varlen && !a.table) {  // contiguous variable-length cache: its directory first
    hipLaunchKernelGGL((varlen_directory_kernel<D, BLK>), dim3(1), dim3(kThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.table && a.old_table) {  // paged update: only the new records (few per pair)
    hipLaunchKernelGGL((paged_update_kernel<D, BLK>), dim3(max_stored < 4 ? max_stored : 4, a.batch * a.hkv),
                       dim3(kThreads), 0, stream, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((pack_kernel<D, BLK>), dim3(max_stored, a.batch * a.hkv), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack_varlen(const Shape& s, const KvPolicy& pol, const CacheGeom& geo, const int64_t* ctxs,
                              const void* k, const void* v, void* cache, hipStream_t stream) {
  PackArgs a;
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.cache = static_cast<uint8_t*>(cache);
  a.old = nullptr;
  a.ogeo = geo;
  a.only_current = 0;
  a.varlen = 1;
  for (int i = 0; i < kMaxVarlenBatch; ++i) a.ctxs[i] = i < s.batch ? ctxs[i] : 1;
  a.n = s.n;
  a.batch = s.batch;
  a.hkv = s.hkv;
  a.pol = pol;
  a.geo = geo;
  a.table = a.old_table = nullptr;
  a.pool = nullptr;
  a.table_bytes = a.old_table_bytes = a.pool_pages = a.page_bytes = 0;
  const int max_stored = geo.cur_block + 1;
  if (s.d == 128 && s.blk == 128) return launch_t<128, 128>(a, max_stored, stream);
  if (s.d == 128 && s.blk == 64) return launch_t<128, 64>(a, max_stored, stream);
  if (s.d == 64 && s.blk == 128) return launch_t<64, 128>(a, max_stored, stream);
  return launch_t<64, 64>(a, max_stored, stream);
}

hipError_t launch_pack(const Shape& s, const KvPolicy& pol, const CacheGeom& geo, const void* k,
                       const void* v, void* cache, const void* old_cache, const CacheGeom* old_geo,
                       bool only_current, hipStream_t stream) {
  PackArgs a;
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.cache = static_cast<uint8_t*>(cache);
  a.old = static_cast<const uint8_t*>(old_cache);
  a.ogeo = old_geo ? *old_geo : geo;
  a.only_current = only_current ? 1 : 0;
  a.varlen = 0;
  a.n = s.n;
  a.batch = s.batch;
  a.hkv = s.hkv;
  a.pol = pol;
  a.geo = geo;
  a.table = a.old_table = nullptr;
  a.pool = nullptr;
  a.table_bytes = a.old_table_bytes = a.pool_pages = a.page_bytes = 0;
  const int max_stored = geo.cur_block + 1;
  if (s.d == 128 && s.blk == 128) return launch_t<128, 128>(a, max_stored, stream);
  if (s.d == 128 && s.blk == 64) return launch_t<128, 64>(a, max_stored, stream);
  if (s.d == 64 && s.blk == 128) return launch_t<64, 128>(a, max_stored, stream);
  return launch_t<64, 64>(a, max_stored, stream);
}

hipError_t launch_pack_paged(const Shape& s, const KvPolicy& pol, const CacheGeom& geo, const void* k, const void* v,
                             const void* table, int64_t table_bytes, const void* old_table, int64_t old_table_bytes,
                             void* pool, int64_t pool_bytes, hipStream_t stream) {
  PackArgs a;
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.cache = nullptr;
  a.old = nullptr;
  a.ogeo = geo;
  a.only_current = 0;
  a.varlen = 0;
  a.n = s.n;
  a.batch = s.batch;
  a.hkv = s.hkv;
  a.pol = pol;
  a.geo = geo;
  a.table = static_cast<const uint8_t*>(table);
  a.old_table = static_cast<const uint8_t*>(old_table);
  a.table_bytes = table_bytes;
  a.old_table_bytes = old_table ? old_table_bytes : 0;
  a.pool = static_cast<uint8_t*>(pool);
  a.page_bytes = geo.rec8_bytes;
  a.pool_pages = pool_bytes / geo.rec8_bytes;
  const int max_stored = geo.cur_block + 1;
  if (s.d == 128 && s.blk == 128) return launch_t<128, 128>(a, max_stored, stream);
  if (s.d == 128 && s.blk == 64) return launch_t<128, 64>(a, max_stored, stream);
  if (s.d == 64 && s.blk == 128) return launch_t<64, 128>(a, max_stored, stream);
  return launch_t<64, 64>(a, max_stored, stream);
}

hipError_t launch_pack_paged_varlen(const Shape& s, const KvPolicy& pol, const CacheGeom& geo, const int64_t* ctxs,
                                    const void* k, const void* v, const void* table, int64_t table_bytes,
                                    const void* old_table, int64_t old_table_bytes, void* pool, int64_t pool_bytes,
                                    hipStream_t stream) {
  PackArgs a;
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.cache = nullptr;
  a.old = nullptr;
  a.ogeo = geo;
  a.only_current = 0;
  a.varlen = 1;
  for (int i = 0; i < kMaxVarlenBatch; ++i) a.ctxs[i] = i < s.batch ? ctxs[i] : 1;
  a.n = s.n;
  a.batch = s.batch;
  a.hkv = s.hkv;
  a.pol = pol;
  a.geo = geo;
  a.table = static_cast<const uint8_t*>(table);
  a.old_table = static_cast<const uint8_t*>(old_table);
  a.table_bytes = table_bytes;
  a.old_table_bytes = old_table ? old_table_bytes : 0;
  a.pool = static_cast<uint8_t*>(pool);
  a.page_bytes = geo.rec8_bytes;
  a.pool_pages = pool_bytes / geo.rec8_bytes;
  const int max_stored = geo.cur_block + 1;
  if (s.d == 128 && s.blk == 128) return launch_t<128, 128>(a, max_stored, stream);
  if (s.d == 128 && s.blk == 64) return launch_t<128, 64>(a, max_stored, stream);
  if (s.d == 64 && s.blk == 128) return launch_t<64, 128>(a, max_stored, stream);
  return launch_t<64, 64>(a, max_stored, stream);
}

}  // namespace tria
