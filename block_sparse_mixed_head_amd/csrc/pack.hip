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
#include "device_common.h"
#include "kernels.h"

namespace tria {

namespace {

constexpr int kThreads = 256;

struct PackArgs {
  const uint16_t* k;
  const uint16_t* v;
  uint8_t* cache;
  int64_t n;  // token rows in the K/V source
  int batch, hkv;
  KvPolicy pol;
  CacheGeom geo;
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

template <int D, int BLK>
__global__ void __launch_bounds__(kThreads) pack_kernel(PackArgs a) {
  constexpr int TPR = D / 8;
  constexpr int RPP = kThreads / TPR;  // rows per pass
  __shared__ __attribute__((aligned(16))) int8_t kbuf[BLK][D];  // codes (int4: sign-extended bytes)
  __shared__ __attribute__((aligned(16))) int8_t vbuf[BLK][D];
  __shared__ float ksb[BLK], vsb[BLK];

  const int pair = blockIdx.y, j = blockIdx.x;
  const int b = pair / a.hkv, g = pair % a.hkv;
  const int c = a.geo.cur_block;
  const Blocks st = stored_blocks(c, a.pol.hi[g], a.pol.keep[g]);
  if (j >= st.n8 + st.n4) return;
  int64_t pair_off = a.geo.data_offset + (int64_t)b * a.geo.batch_bytes;
  for (int gg = 0; gg < g; ++gg) {
    const Blocks o = stored_blocks(c, a.pol.hi[gg], a.pol.keep[gg]);
    pair_off += (int64_t)o.n8 * a.geo.rec8_bytes + (int64_t)o.n4 * a.geo.rec4_bytes;
  }
  const bool is4 = j >= st.n8;
  const int kb = !is4 ? ((st.sink && j == 0) ? 0 : st.lo8 + j - st.sink) : st.lo4 + (j - st.n8);
  const int64_t off = !is4 ? pair_off + (int64_t)j * a.geo.rec8_bytes
                           : pair_off + (int64_t)st.n8 * a.geo.rec8_bytes + (int64_t)(j - st.n8) * a.geo.rec4_bytes;
  uint8_t* rec = a.cache + off;
  const int tid = threadIdx.x;

  if (j == 0 && tid == 0) {
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

  if (pair == 0 && j == 0) {  // the padding between the directory and the first record
    const int64_t pad0 = 64 + 64LL * a.batch * a.hkv;
    for (int64_t i = pad0 + tid; i < a.geo.data_offset; i += kThreads) a.cache[i] = 0;
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
    const bool valid = tok < a.geo.ctx_len;
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
hipError_t launch_t(const PackArgs& a, int max_stored, hipStream_t stream) {
  hipLaunchKernelGGL((pack_kernel<D, BLK>), dim3(max_stored, a.batch * a.hkv), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const Shape& s, const KvPolicy& pol, const CacheGeom& geo, const void* k,
                       const void* v, void* cache, hipStream_t stream) {
  PackArgs a;
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.cache = static_cast<uint8_t*>(cache);
  a.n = s.n;
  a.batch = s.batch;
  a.hkv = s.hkv;
  a.pol = pol;
  a.geo = geo;
  const int max_stored = geo.cur_block + 1;
  if (s.d == 128 && s.blk == 128) return launch_t<128, 128>(a, max_stored, stream);
  if (s.d == 128 && s.blk == 64) return launch_t<128, 64>(a, max_stored, stream);
  if (s.d == 64 && s.blk == 128) return launch_t<64, 128>(a, max_stored, stream);
  return launch_t<64, 64>(a, max_stored, stream);
}

}  // namespace tria
