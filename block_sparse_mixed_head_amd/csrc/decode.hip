// decode.hip - one-token decode over the compressed mixed-precision KV cache.
//
// TriAttention summary page (rit.work), section on calibration: generation reads
// the compressed cache, so each step reads less data.  Decode reads the whole kept
// cache once per step with about one multiply-add per byte, so it is bound by
// memory bandwidth (llmis.ru chapter 3.5, section 2); the win is fewer bytes.
// For query head h of KV head g at position t = ctx_len - 1:
//   s_j = dot(qc^a, kc_j^a) * sq^a * sk_j * sm_scale      (a = block precision)
//   out = sum_j exp(s_j - max) * sv_j * vc_j / sum_j exp(s_j - max)
//
// gfx950 design (split-KV by bytes, two kernels):
//   * The stored records of all (batch, KV head) pairs form one sequence of
//     32-token steps; an int8 step costs two units (its bytes), an int4 step one.
//     A persistent grid of wavefronts splits the units evenly (wave w owns the
//     steps starting in [U*w/W, U*(w+1)/W)), so every wavefront streams the same
//     number of bytes whatever the policy.  Each work group derives the split from
//     the cache directory itself (prefix sums in LDS); the host needs no knowledge
//     of the policy.
//   * A wavefront serves all G query heads of a KV head at once (G rows padded to
//     16 per MFMA row group), so every cache byte is read exactly once per step,
//     and keeps the next step's loads in flight (register double buffer) while it
//     computes the current one.
//   * q.k: v_mfma_i32_16x16x64_i8 with K codes straight from HBM as the A operand
//     (int4 steps widened to 16*code).  p.v: v_mfma_f32_16x16x32_f16 with the V
//     codes (stored per 32-token chunk, transposed, in the order the MFMA consumes
//     them; a step reads one contiguous chunk with 1 KB lane-contiguous loads) turned
//     into fp16 exactly by byte permutes (a code plus a fixed bias, removed at the
//     end), and the fp32 weight p*sv split into an fp16 high part and an fp16
//     remainder, so the product keeps ~21 mantissa bits.
//   * Online softmax in fp32 (base 2).  Each wavefront writes one partial
//     (m, l, o[d]) per pair it touched; a second kernel merges a pair's partials.
//   * Both kernels validate the cache header and directory before reading any
//     record; on a mismatch nothing is read and the merge writes NaN.
#include <cfloat>
#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "paged_skip.h"

namespace tria {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kGrid = 512;                  // persistent work groups (two per CU)
constexpr int kMaxWaves = kGrid * kWaves;
constexpr int kMaxPairs = 4096;             // directory entries handled in LDS

// workspace: [0,64) header {valid, n_pairs, n_slots, n_waves}; [64, 64 + 8*P) per pair
// {first slot, slot count}; partials from ws_part_offset: [slot][row][D + 4] floats
// (o[0..D), m, l, 0, 0).  Wavefront w writes pair p's partial to slot p + w: the
// wavefronts of consecutive pairs share at most one wavefront, so the slots of
// different (pair, wavefront) are distinct and fewer than W + P.
__host__ __device__ inline int64_t ws_part_offset(int64_t pairs) {
  return (64 + 8 * pairs + 255) / 256 * 256;
}

struct DecArgs {
  const uint8_t* cache;
  const uint16_t* q;
  float* ws;
  float* out;
  int64_t cache_bytes;
  int64_t ctx_len;
  int batch, hq, hkv;
  float c;     // sm_scale * log2(e)
  int varlen;  // version-3 cache: each directory entry holds its sequence's ctx_len
  const int* plan;  // dynamic skipping: per pair {offset, kept and stored counts, mask}, kept lists
  int rmax;         // record slots per pair in the plan's lists
  // paged cache: `cache` is the page table, records at pool + page * page_bytes (list
  // entries hold pages)
  int paged;
  const uint8_t* pool;
  int64_t page_bytes, pool_pages;
};

struct Geo {
  int64_t rec8, rec4, data_offset, total;
  int cur;
};

// A 64-byte header as one load (every field in registers before any test, so the
// tests cost no further memory round trips).
struct Hdr64 {
  int32_t w[16];
  __device__ int64_t q(int i) const { return (int64_t)(((uint64_t)(uint32_t)w[2 * i + 1] << 32) | (uint32_t)w[2 * i]); }
};
// Every word of a loaded header in scalar registers at this point: the loads of all
// sixteen are issued before it and waited for once.  Without it the compiler moves
// the load of a word that only some tests read into the branch of those tests, one
// more memory round trip each.  Called after the other loads of the same round.
__device__ __forceinline__ void pin_hdr(Hdr64& h) {
  asm volatile(""
               : "+s"(h.w[0]), "+s"(h.w[1]), "+s"(h.w[2]), "+s"(h.w[3]), "+s"(h.w[4]), "+s"(h.w[5]), "+s"(h.w[6]),
                 "+s"(h.w[7]), "+s"(h.w[8]), "+s"(h.w[9]), "+s"(h.w[10]), "+s"(h.w[11]), "+s"(h.w[12]),
                 "+s"(h.w[13]), "+s"(h.w[14]), "+s"(h.w[15]));
}

// Validates the global header against the launch; returns false on mismatch.
template <int D, int BLK>
__device__ __forceinline__ bool header_ok_h(const DecArgs& a, const Hdr64& h, Geo& geo) {
  const int32_t* hd = h.w;
  const int64_t h64[8] = {0, 0, 0, 0, h.q(4), h.q(5), h.q(6), h.q(7)};
  geo.rec8 = 2LL * BLK * D + 8LL * BLK;
  geo.rec4 = (int64_t)BLK * D + 8LL * BLK;
  geo.cur = (int)((a.ctx_len - 1) / BLK);
  geo.data_offset = (64 + 64LL * a.batch * a.hkv + 255) / 256 * 256;
  geo.total = h64[5];
  const bool common = hd[0] == 0x43564B54 && hd[2] == a.batch && hd[3] == a.hkv && hd[4] == D && hd[5] == BLK &&
                      geo.total <= a.cache_bytes && h64[6] == 64 && h64[7] == geo.data_offset;
  if (a.varlen) return common && hd[1] == 3 && hd[7] == -1;  // ctx_len per directory entry
  return common && hd[1] == 2 && hd[6] == geo.cur + 1 && hd[7] == geo.cur && h64[4] == a.ctx_len;
}
template <int D, int BLK>
__device__ __forceinline__ bool header_ok(const DecArgs& a, Geo& geo) {
  Hdr64 h = *reinterpret_cast<const Hdr64*>(a.cache);
  pin_hdr(h);
  return header_ok_h<D, BLK>(a, h, geo);
}

// Page table header (version 4) against the launch; geo.total = the table size.  A
// variable-length table (word 7 = -1, header ctx_len 0) holds each pair's ctx_len in its
// entry and rmax (word 6) page slots per pair.
template <int D, int BLK>
__device__ __forceinline__ bool paged_header_h(const DecArgs& a, const Hdr64& h, Geo& geo) {
  geo.rec8 = 2LL * BLK * D + 8LL * BLK;
  geo.rec4 = (int64_t)BLK * D + 8LL * BLK;
  geo.cur = (int)((a.ctx_len - 1) / BLK);
  geo.data_offset = 64 + 64LL * a.batch * a.hkv;
  const int rmax = a.varlen ? h.w[6] : geo.cur + 1;
  geo.total = geo.data_offset + 4LL * a.batch * a.hkv * rmax;
  const bool common = h.w[0] == 0x50564B54 && h.w[1] == 4 && h.w[2] == a.batch && h.w[3] == a.hkv && h.w[4] == D &&
                      h.w[5] == BLK && h.q(5) == geo.rec8 && rmax >= 1 && geo.total <= a.cache_bytes;
  if (a.varlen) return common && h.w[7] == -1 && h.q(4) == 0;
  return common && h.w[6] == geo.cur + 1 && h.w[7] == geo.cur && h.q(4) == a.ctx_len;
}
template <int D, int BLK>
__device__ __forceinline__ bool paged_header_ok(const DecArgs& a, Geo& geo) {
  Hdr64 h = *reinterpret_cast<const Hdr64*>(a.cache);
  pin_hdr(h);
  return paged_header_h<D, BLK>(a, h, geo);
}

// Inclusive prefix sum over the wavefront: DPP row shifts (1, 2, 4, 8) within each
// row of 16 lanes, then the row broadcasts of lane 15 (into rows 1 and 3) and of
// lane 31 (into rows 2 and 3).  Lanes without a source add the old value 0.
__device__ __forceinline__ int wave_scan_incl(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
  return x;
}

// floor(n / d) for 0 <= n < 2^52 and 0 < d < 2^52: the double quotient is within one
// of the exact one (both operands are exact doubles), then corrected by one
// comparison each way with exact 64-bit products.
__device__ __forceinline__ int64_t floor_div(int64_t n, int64_t d) {
  int64_t q = (int64_t)((double)n / (double)d);
  if (q * d > n) --q;
  else if ((q + 1) * d <= n) ++q;
  return q;
}

// Owner of unit u among W wavefronts splitting U units: the largest w with
// floor(U*w/W) <= u.
__device__ __forceinline__ int owner_of(int64_t u, int64_t U, int64_t W) {
  return (int)floor_div((u + 1) * W - 1, U);
}

// Register buffers of one 32-token step.  Lane (lr, kq) holds, for S^T subtile s
// (keys 16s..16s+15 of the step), key 16s + lr's dims [64ks + 16kq, +16) (int4:
// packed), dim 16dt + lr of the keys at feed positions [8kq, +8) for every dim
// group dt, and one of the chunk's 64 scales; the scales reach the lanes that use
// them through LDS.
template <int D>
struct Buf8 {
  v4i k[2][D / 64];
  v4i v[D / 32];  // V units: dim groups 2m, 2m+1 (8 bytes each)
  int sc;         // one dword of the chunk's 64 scales (lane l: K scale l, or V scale l - 32)
};
template <int D>
struct Buf4 {
  v2i k[2][D / 64];
  v4i v[(D + 63) / 64];  // V units: dim groups 4m .. 4m+3 (4 bytes each)
  int sc;
};

template <int D, int BLK, bool IS4>
struct StepIO {
  using Buf = typename std::conditional<IS4, Buf4<D>, Buf8<D>>::type;

  // Cache policy of the record loads: non-temporal.  The cache is streamed once
  // per step; allocating it would evict (and write back) whatever the preceding
  // kernels left dirty in the last-level cache, halving the read rate.
  static constexpr int kNT = 2;
  // Step h (chunk h) of the record at byte `roff` of the run's buffer resource
  // (roff and h wave-uniform).  A chunk holds the K codes in operand order (unit
  // (s, ks, kq, lr) = lane lr + 16kq of MFMA (s, ks)), the V codes as units (dt,
  // kq, lr), then the K and V scales of its 32 tokens: every load below reads a
  // contiguous run with lane l at offset l * size.
  __device__ __forceinline__ static void load(Buf& r, __amdgpu_buffer_rsrc_t rs, int roff, int h, int lr, int kq) {
    constexpr int KS = D / 64;
    constexpr int KPART = IS4 ? 16 * D : 32 * D;  // bytes of the chunk's K (and V) part
    constexpr int CB = 2 * KPART + 256;
    const int co = uni(roff + h * CB);
    const int lane = lr + 16 * kq;
    // region bases in the scalar offset, lane offsets in one register, each load a
    // contiguous 1 KB (int4 K with d = 64: 512 B)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if constexpr (!IS4) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          r.k[s][ks] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + (s * KS + ks) * 1024, co, kNT);
      } else if constexpr (KS == 2) {
        const v4i x = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + s * 1024, co, kNT);
        r.k[s][0] = v2i{x[0], x[1]};
        r.k[s][KS - 1] = v2i{x[2], x[3]};
      } else {
        r.k[s][0] = __builtin_amdgcn_raw_buffer_load_b64(rs, lane * 8 + s * 512, co, kNT);
      }
    }
    const int vo = uni(co + KPART), so = uni(co + 2 * KPART);
#pragma unroll
    for (int m = 0; m < (IS4 ? (D + 63) / 64 : D / 32); ++m)
      r.v[m] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + m * 1024, vo, kNT);
    r.sc = __builtin_amdgcn_raw_buffer_load_b32(rs, lane * 4, so, kNT);
  }
};

template <int D, int RG>
struct SegState {
  float m[RG], l[RG];
  float c[RG];  // bias correction: sum over this lane's keys of bias * p' (see compute_step)
  v4f O[RG][D / 16];
  int k;        // scale exponent of p' (wave-uniform)
};

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// V codes to fp16 MFMA operands, exactly, with a known affine bias: the two's
// complement sign is flipped and the code placed in the low mantissa byte of an
// fp16 with exponent 2^10 (high byte 0x64) by byte permutes:
//   int8 code v -> 1024 + (v + 128)        = 1152 + v
//   int4 code c -> 1024 + 16 (c + 8)       = 1152 + 16 c   (nibble in bits 4..7)
// The bias times the weights' sum is subtracted from O at the end; the 16 of int4
// is folded into its weights.
constexpr float kBias = 1152.0f;
__device__ __forceinline__ v8h v8_to_f16(uint32_t w0, uint32_t w1) {
  const uint32_t magic = 0x64646464u;
  w0 ^= 0x80808080u;
  w1 ^= 0x80808080u;
  const v4i r = {(int)__builtin_amdgcn_perm(magic, w0, 0x04010400u), (int)__builtin_amdgcn_perm(magic, w0, 0x04030402u),
                 (int)__builtin_amdgcn_perm(magic, w1, 0x04010400u), (int)__builtin_amdgcn_perm(magic, w1, 0x04030402u)};
  return __builtin_bit_cast(v8h, r);
}
// 8 packed nibbles (low nibble first) -> 8 fp16 in position order
__device__ __forceinline__ v8h v4_to_f16(uint32_t w) {
  w ^= 0x88888888u;
  const uint32_t e = (w << 4) & 0xF0F0F0F0u, o = w & 0xF0F0F0F0u;  // (c + 8) << 4 per byte: even, odd codes
  // byte j of e and of o into the low bytes of the two halves, high bytes 0x64
  auto pair = [&](uint32_t sel) { return (int)((__builtin_amdgcn_perm(o, e, sel) & 0x00FF00FFu) | 0x64006400u); };
  const v4i r = {pair(0x04040000u), pair(0x05050101u), pair(0x06060202u), pair(0x07070303u)};
  return __builtin_bit_cast(v8h, r);
}

// One 32-token step: scores, online softmax, O^T += V^T . P'^T.  mask_from = the
// step's first key index at or past which keys are masked (>= 32: none).
// With u = S * sk, t = u * a (a > 0 per query row), so the maximum is taken over u
// and a enters the exponent: p = 2^(u * a - m).
template <int D, int RG, bool IS4>
__device__ __forceinline__ void compute_step(const typename std::conditional<IS4, Buf4<D>, Buf8<D>>::type& r,
                                             const v4i (&qop)[RG][D / 64], const float (&ar)[RG], int mask_from,
                                             SegState<D, RG>& st, int kq, float* slot, uint32_t hoff) {
  constexpr int KS = D / 64, ND = D / 16;
  // the step's scales through the wave's LDS slot (one wavefront: in order, no barrier)
  slot[threadIdx.x & 63] = __int_as_float(r.sc);
  float4 skv[2], svv[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    skv[s] = *reinterpret_cast<const float4*>(slot + 16 * s + 4 * kq);
    svv[s] = *reinterpret_cast<const float4*>(slot + 32 + 16 * s + 4 * kq);
  }
  float u[RG][2][4];
  float mt[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      v4i S = {0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        v4i kop;
        if constexpr (IS4) {
          const v2i w = r.k[s][ks];
          kop = unpack16_x16((uint32_t)w[0], (uint32_t)w[1]);
        } else {
          kop = r.k[s][ks];
        }
        S = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop, qop[rg][ks], S, 0, 0, 0);
      }
      const float kv[4] = {skv[s].x, skv[s].y, skv[s].z, skv[s].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) u[rg][s][i] = (float)S[i] * kv[i];
    }
  }
  if (mask_from < 32) {  // only the current block's tail (wave-uniform branch)
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * s + 4 * kq + i >= mask_from) u[rg][s][i] = -INFINITY;
  }
  if (hoff) {  // query rows (bit rg*16 + lr) that skip this block (wave-uniform branch)
    const int lr = threadIdx.x & 15;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
      if ((hoff >> (rg * 16 + lr)) & 1u)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int i = 0; i < 4; ++i) u[rg][s][i] = -INFINITY;
  }
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    float x = fmaxf(fmaxf(u[rg][0][0], u[rg][0][1]), fmaxf(u[rg][0][2], u[rg][0][3]));
    x = fmaxf(x, fmaxf(fmaxf(u[rg][1][0], u[rg][1][1]), fmaxf(u[rg][1][2], u[rg][1][3])));
    mt[rg] = xmax32(xmax16(x)) * ar[rg];  // -inf when the whole step is masked
  }
  bool need = false;
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) need = need || (mt[rg] > st.m[rg]);
  if (__ballot(need)) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      const float mn = fmaxf(st.m[rg], mt[rg]);
      // 0 while m was -inf; a row still without any key (every key so far masked or
      // skipped for it) keeps its zero sums (exp2(-inf - -inf) would be NaN)
      const float f = mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(st.m[rg] - mn);
      st.m[rg] = mn;
      st.l[rg] *= f;
      st.c[rg] *= f;
#pragma unroll
      for (int d = 0; d < ND; ++d) st.O[rg][d] *= f;
    }
  }
  // the weights' scale 2^k keeps p' = p * sv * 2^k (p <= 1) inside fp16: lowered
  // (O and c rescaled exactly) if a step's V scales would take it past 2^14
  {
    float smax = fmaxf(fmaxf(fmaxf(svv[0].x, svv[0].y), fmaxf(svv[0].z, svv[0].w)),
                       fmaxf(fmaxf(svv[1].x, svv[1].y), fmaxf(svv[1].z, svv[1].w)));
    if (__ballot(smax > __builtin_ldexpf(1.0f, 14 - st.k))) {
      const int e = ilogbf(xmax32(xmax16(smax))) + 1;  // 2^e > max scale
      const int kn = 14 - e;
      const float f = __builtin_ldexpf(1.0f, kn - st.k);
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        st.c[rg] *= f;
#pragma unroll
        for (int d = 0; d < ND; ++d) st.O[rg][d] *= f;
      }
      st.k = kn;
    }
  }
  // weights p = 2^(u a - m); p' = p * sv * 2^k (int4: / 16) split into an fp16 high
  // part (rounded toward zero) and the fp16 of the remainder
  const float wsc = __builtin_ldexpf(IS4 ? 1.0f / 16.0f : 1.0f, st.k);
  v8h bhi[RG], blo[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    // m is -inf only while every key seen so far was masked (then u is too)
    const float nm = st.m[rg] == -INFINITY ? 0.0f : -st.m[rg];
    v2h hw[4], lw[4];
    float psum = 0.0f;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float vv[4] = {svv[s].x, svv[s].y, svv[s].z, svv[s].w};
      float pw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(fmaf(u[rg][s][i], ar[rg], nm));
        st.l[rg] += p;
        pw[i] = p * (vv[i] * wsc);
        psum += pw[i];
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const v2h hi = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_pkrtz(pw[2 * h], pw[2 * h + 1]));
        const v2f hf = __builtin_convertvector(hi, v2f);
        hw[2 * s + h] = hi;
        lw[2 * s + h] = __builtin_bit_cast(v2h, __builtin_amdgcn_cvt_pkrtz(pw[2 * h] - hf[0], pw[2 * h + 1] - hf[1]));
      }
    }
    st.c[rg] = fmaf(kBias, psum, st.c[rg]);
    bhi[rg] = __builtin_shufflevector(__builtin_shufflevector(hw[0], hw[1], 0, 1, 2, 3),
                                      __builtin_shufflevector(hw[2], hw[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
    blo[rg] = __builtin_shufflevector(__builtin_shufflevector(lw[0], lw[1], 0, 1, 2, 3),
                                      __builtin_shufflevector(lw[2], lw[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
  }
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) {
    v8h vop;
    if constexpr (IS4)
      vop = v4_to_f16((uint32_t)r.v[dt / 4][dt % 4]);
    else
      vop = dt % 2 == 0 ? v8_to_f16((uint32_t)r.v[dt / 2][0], (uint32_t)r.v[dt / 2][1])
                        : v8_to_f16((uint32_t)r.v[dt / 2][2], (uint32_t)r.v[dt / 2][3]);
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      st.O[rg][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, bhi[rg], st.O[rg][dt], 0, 0, 0);
      st.O[rg][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, blo[rg], st.O[rg][dt], 0, 0, 0);
    }
  }
}

// Subtracts the V-code bias from O (c summed over the four lanes of each query row)
// and restarts c: O then holds only the segment's true partial sums, so fp32 rounding
// stays relative to them however many keys a segment has (once per ring trip).
template <int D, int RG>
__device__ __forceinline__ void fold_bias(SegState<D, RG>& st) {
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const float c = xsum32(xsum16(st.c[rg]));
#pragma unroll
    for (int d = 0; d < D / 16; ++d) st.O[rg][d] -= c;
    st.c[rg] = 0.0f;
  }
}

// Steps [j0, j1) of one precision run of a pair; rec0 = the run's first record.
// A ring of three register buffers keeps the loads of the next two steps in
// flight while a step is computed; `pre` runs once the first loads are issued
// (the segment's query quantisation).  Loads past the run's end fetch nothing,
// so every record byte is read once.
// SKIP: steps count the run's kept records only; kept record i is stored record
// list[i].x (of nstored) and list[i].y has bit r set when query row r keeps it.
template <int D, int BLK, int RG, bool IS4, bool SKIP, class Pre>
__device__ __forceinline__ void run_steps(const uint8_t* rec0, int64_t rec_bytes, int j0, int j1,
                                          const v4i (&qop)[RG][D / 64], const float (&ar)[RG], int mask_jb,
                                          int mask_first, SegState<D, RG>& st, int lr, int kq, float* slot, Pre&& pre,
                                          const int2* list, int64_t stride, uint32_t hfull,
                                          const int32_t* pages = nullptr, int64_t pool_pages = 0) {
  using IO = StepIO<D, BLK, IS4>;
  constexpr int SPB = BLK / 32;
  if (j0 >= j1) return;
  j0 = uni(j0);
  j1 = uni(j1);
  const int rb = uni((int)rec_bytes);
  // keys of step j at or past which keys are masked: only the current block's
  // tail (ctx_len is inside block mask_jb of this run) is masked
  auto mfrom = [&](int j) __attribute__((always_inline)) -> int {
    return j / SPB == mask_jb ? mask_first - 32 * (j % SPB) : 1 << 30;
  };
  if constexpr (SKIP) {
    // record i of the list at rec0 + i * stride; only listed records are loaded (the
    // resource is built per load over the record or, past the window, empty)
    const int64_t base0 = uni64(reinterpret_cast<int64_t>(rec0));
    const int64_t strd = uni64(stride);
    const int lane = threadIdx.x & 63;
    typename IO::Buf A, B, C;
    // windows of up to 64 kept records: lane l holds the window's entry l, read by
    // the whole wavefront with readlane (uniform index, no memory access per step).
    // The first window's entries load together with the query rows, before `pre`.
    // (paged: the entries are the table's page ids, every head keeps every record; a
    // page outside the pool is read as page 0 and poisons the segment's sums with NaN)
    auto window = [&](int w0, int& w1) __attribute__((always_inline)) -> int2 {
      const int r0 = uni(w0 / SPB);
      w1 = uni((r0 + 64) * SPB < j1 ? (r0 + 64) * SPB : j1);
      const int rlast = (w1 - 1) / SPB;
      if (!pages) return r0 + lane <= rlast ? list[r0 + lane] : make_int2(0, 0);
      int pg = r0 + lane <= rlast ? pages[r0 + lane] : 0;
      if (__ballot(pg < 0 || (int64_t)pg >= pool_pages)) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) st.l[rg] = __int_as_float(0x7FC00000);
        pg = pg < 0 || (int64_t)pg >= pool_pages ? 0 : pg;
      }
      return make_int2(pg, (int)hfull);
    };
    int w1f;
    const int2 efirst = window(j0, w1f);
    pre();
    for (int w0 = j0; w0 < j1;) {
      const int r0 = uni(w0 / SPB);
      int w1 = w1f;
      const int2 e = w0 == j0 ? efirst : window(w0, w1);
      auto ld = [&](typename IO::Buf& r, int j) __attribute__((always_inline)) {
        const bool in = j < w1;
        const int rec = in ? __builtin_amdgcn_readlane(e.x, j / SPB - r0) : 0;
        const __amdgpu_buffer_rsrc_t rr = __builtin_amdgcn_make_buffer_rsrc(
            reinterpret_cast<void*>(base0 + (int64_t)rec * strd), (short)0, in ? rb : 0, 0x00020000);
        __builtin_amdgcn_sched_barrier(0);
        IO::load(r, rr, 0, in ? j % SPB : 0, lr, kq);
        __builtin_amdgcn_sched_barrier(0);
      };
      auto hoff = [&](int j) __attribute__((always_inline)) -> uint32_t {
        return hfull & ~(uint32_t)__builtin_amdgcn_readlane(e.y, j / SPB - r0);
      };
      for (int j = w0; j < w1 + 2; j += 3) {
        if (((j / 3) + (blockIdx.x >= gridDim.x / 2)) & 1) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
        ld(A, j);
        if (j - 2 >= w0 && j - 2 < w1) compute_step<D, RG, IS4>(B, qop, ar, mfrom(j - 2), st, kq, slot, hoff(j - 2));
        ld(B, j + 1);
        if (j - 1 >= w0 && j - 1 < w1) compute_step<D, RG, IS4>(C, qop, ar, mfrom(j - 1), st, kq, slot, hoff(j - 1));
        ld(C, j + 2);
        if (j < w1) compute_step<D, RG, IS4>(A, qop, ar, mfrom(j), st, kq, slot, hoff(j));
        fold_bias(st);
      }
      w0 = w1;
    }
    return;
  }
  // the run's records as one buffer resource (dword 3: raw 32-bit data format)
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(uni64(reinterpret_cast<int64_t>(rec0))), (short)0, uni((j1 + SPB - 1) / SPB * rb), 0x00020000);
  // past the run's end, the same loads go through a resource with no records:
  // the hardware range check returns zeros without a memory access, and the
  // loads stay unconditional (a skipped load would make the wait counts unknown)
  const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>(uni64(reinterpret_cast<int64_t>(rec0))), (short)0, 0, 0x00020000);
  typename IO::Buf A, B, C;
  // each step's loads stay together in issue order (sched barriers), so waiting
  // for the oldest buffer never waits for a younger one
  auto ld = [&](typename IO::Buf& r, int j) __attribute__((always_inline)) {
    const bool in = j < j1;
    __builtin_amdgcn_sched_barrier(0);
    IO::load(r, in ? rs : none, in ? (j / SPB) * rb : 0, in ? j % SPB : 0, lr, kq);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Step j is loaded into buffer (j - j0) % 3 and computed two loads later, so
  // two steps are in flight during each compute.  Loads and their uses both sit
  // inside the loop (nothing loaded before it is used in it), which keeps the
  // compiler's wait counts exact; computes outside [j0, j1) are skipped.
  for (int j = j0; j < j1 + 2; j += 3) {
    // The two work groups sharing a CU would otherwise run at fixed relative
    // priority (the older wave issues first), so the second one's waves finish their
    // equal share well after the first one's.  Alternating the issue priority per
    // ring trip, out of phase between the halves of the grid, shares the SIMD fairly.
    if (((j / 3) + (blockIdx.x >= gridDim.x / 2)) & 1) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
    ld(A, j);
    if (j - 2 >= j0 && j - 2 < j1) compute_step<D, RG, IS4>(B, qop, ar, mfrom(j - 2), st, kq, slot, 0u);
    ld(B, j + 1);
    if (j - 1 >= j0 && j - 1 < j1) compute_step<D, RG, IS4>(C, qop, ar, mfrom(j - 1), st, kq, slot, 0u);
    ld(C, j + 2);
    if (j == j0) pre();  // the query quantisation, once the first three steps' loads are in flight
    if (j < j1) compute_step<D, RG, IS4>(A, qop, ar, mfrom(j), st, kq, slot, 0u);
    fold_bias(st);
  }
}

// block_scan of two values at once (same barriers); tmp holds 2 * kWaves ints.
__device__ __forceinline__ int2 block_scan2(int x, int y, int* tmp, int& tx, int& ty) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ix = wave_scan_incl(x), iy = wave_scan_incl(y);
  if (lane == 63) {
    tmp[wave] = ix;
    tmp[kWaves + wave] = iy;
  }
  __syncthreads();
  int bx = 0, by = 0;
  tx = 0;
  ty = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int t = tmp[w], u = tmp[kWaves + w];
    bx += w < wave ? t : 0;
    by += w < wave ? u : 0;
    tx += t;
    ty += u;
  }
  __syncthreads();
  return make_int2(bx + ix - x, by + iy - y);
}

// In-place exclusive prefixes of a[0..P) and b[0..P), a[P], b[P] = totals.
__device__ __forceinline__ void prefix2_lds(int* arr, int* brr, int P, int* tmp) {
  int ca = 0, cb = 0;
  for (int base = 0; base < P; base += kThreads) {
    const int p = base + (int)threadIdx.x;
    int ta, tb;
    const int2 e = block_scan2(p < P ? arr[p] : 0, p < P ? brr[p] : 0, tmp, ta, tb);
    if (p < P) {
      arr[p] = ca + e.x;
      brr[p] = cb + e.y;
    }
    ca += ta;
    cb += tb;
  }
  if (threadIdx.x == 0) {
    arr[P] = ca;
    brr[P] = cb;
  }
  __syncthreads();
}

// SKIP: the per-pair counts, offsets and kept-record lists come from the plan
// written by the skip kernels below (which validated the directory), and the split
// is over the kept records' units.
template <int D, int BLK, int RG, bool SKIP>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(RG == 1 ? 2 : 1, 2)))
decode_split_kernel(DecArgs a) {
  constexpr int KS = D / 64, ND = D / 16, SPB = BLK / 32;
  __shared__ int n8p[kMaxPairs + 1];  // int8 records per pair, then their exclusive prefix
  __shared__ int n4p[kMaxPairs + 1];  // int4 records per pair, then their exclusive prefix
  __shared__ int first[kWaves];      // the pair holding each wavefront's first unit
  __shared__ int mfp[kMaxPairs];     // per pair: keys of the current block below ctx_len (the mask)
  __shared__ int tmp[2 * kWaves];
  __shared__ int bad;
  __shared__ __attribute__((aligned(16))) float scl[kWaves][64];  // per-wave step scales

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, kq = lane >> 4;
  const int G = a.hq / a.hkv;
  const int P = a.batch * a.hkv;
  // the directory entry of pair tid is loaded together with the header (the host
  // checked that the directory lies inside the cache): one memory round trip
  // (SKIP: the plan's pair entry, two vectors)
  // entries from the skip plan, or (plain and paged) the cache directory / table
  const bool from_plan = SKIP && a.plan != nullptr;
  auto entry_ptr = [&](int p) __attribute__((always_inline)) -> const v4i* {
    return from_plan ? reinterpret_cast<const v4i*>(a.plan + 8 * (int64_t)p)
                     : reinterpret_cast<const v4i*>(a.cache + 64 + 64 * (int64_t)p);
  };
  v4i ent[3] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {0, 0, 0, 0}};
  if (tid < P) {
    const v4i* e = entry_ptr(tid);
    ent[0] = e[0];
    ent[1] = e[1];
    if (!from_plan) ent[2] = e[2];
  }
  auto entry = [&](int p, v4i (&x)[3]) __attribute__((always_inline)) {
    if (p == tid) {
      x[0] = ent[0];
      x[1] = ent[1];
      x[2] = ent[2];
    } else {
      const v4i* e = entry_ptr(p);
      x[0] = e[0];
      x[1] = e[1];
      x[2] = from_plan ? v4i{0, 0, 0, 0} : e[2];
    }
  };
  Geo geo;
  Hdr64 hdr = *reinterpret_cast<const Hdr64*>(a.cache);
  pin_hdr(hdr);
  if (!(SKIP && a.paged ? paged_header_h<D, BLK>(a, hdr, geo) : header_ok_h<D, BLK>(a, hdr, geo))) {
    if (blockIdx.x == 0 && tid == 0) reinterpret_cast<int*>(a.ws)[0] = 0;
    return;
  }
  if (tid == 0) bad = 0;
  // page slots per pair of a paged table (variable length: the header's)
  const int prmax = SKIP && a.paged ? (a.varlen ? hdr.w[6] : a.rmax) : 0;
  __syncthreads();
  // ---- directory: record counts per pair, checked
  for (int p = tid; p < P; p += kThreads) {
    v4i e[3];
    entry(p, e);
    if (from_plan) {
      // {offset lo, hi, kept int8, kept int4}, {stored int8, stored int4, mask, ok}
      const int k8 = e[0][2], k4 = e[0][3], n8 = e[1][0], n4 = e[1][1], mf = e[1][2];
      const bool ok = e[1][3] == 1 && k8 >= 1 && k4 >= 0 && k8 <= n8 && k4 <= n4 && mf >= 1 && mf <= BLK;
      if (!ok) bad = 1;
      n8p[p] = ok ? k8 : 0;
      n4p[p] = ok ? k4 : 0;
      mfp[p] = mf;
      continue;
    }
    const int n8 = e[0][2], n4 = e[0][3], lo8 = e[1][2], sink = e[1][3], lo4 = e[2][0];
    // the pair's position: the launch's ctx_len, or (version 3) its own
    const int64_t ctx = a.varlen ? (int64_t)(((uint64_t)(uint32_t)e[2][3] << 32) | (uint32_t)e[2][2]) : a.ctx_len;
    const bool pos_ok = ctx >= 1 && ctx <= (1LL << 40);
    const int cur = pos_ok ? (int)((ctx - 1) / BLK) : 0;
    // the int8 run ends at the current block; int4 records lie below it
    const bool ok = pos_ok && n8 >= 1 && n4 >= 0 && n8 + n4 <= cur + 1 && (sink == 0 || sink == 1) && lo8 >= 0 &&
                    lo8 + (n8 - sink) - 1 == cur && sink == (lo8 > 0 ? 1 : 0) && lo4 >= 0 && lo4 + n4 <= cur + 1 &&
                    (!(SKIP && a.paged) || cur + 1 <= prmax);
    if (!ok) bad = 1;
    n8p[p] = ok ? n8 : 0;
    n4p[p] = ok ? n4 : 0;
    mfp[p] = (int)(ctx - (int64_t)cur * BLK);
  }
  __syncthreads();
  prefix2_lds(n8p, n4p, P, tmp);
  // ---- the split: U units, W wavefronts, W <= U / 2 so that every wavefront's
  // range (>= 2 units) holds at least one step start
  auto units_at = [&](int p) -> int64_t { return (int64_t)SPB * (2 * (int64_t)n8p[p] + n4p[p]); };
  const int64_t U = uni64(units_at(P));
  const int64_t W = (int64_t)gridDim.x * kWaves < U / 2 ? (int64_t)gridDim.x * kWaves : U / 2;
  // wavefront w owns the units [floor(U w / W), floor(U (w + 1) / W))
  int64_t wlo[kWaves];
#pragma unroll
  for (int i = 0; i < kWaves; ++i) wlo[i] = floor_div(U * ((int64_t)blockIdx.x * kWaves + i), W);
  int* wsh = reinterpret_cast<int*>(a.ws);
  // records are contiguous in (b, g) order: check every pair's offset, find the pair
  // holding each of this work group's first units, and (work group 0) publish each
  // pair's slot range: the wavefronts owning its first and last step starts, every
  // one in between owning at least one (W <= U / 2: ranges of >= 2 units)
  for (int p = tid; p < P; p += kThreads) {
    v4i e[3];
    entry(p, e);
    const int64_t off = (int64_t)(((uint64_t)(uint32_t)e[0][1] << 32) | (uint32_t)e[0][0]);
    if (!SKIP && off != geo.data_offset + (int64_t)n8p[p] * geo.rec8 + (int64_t)n4p[p] * geo.rec4) bad = 1;
    const int64_t u0 = units_at(p), u1 = units_at(p + 1);
#pragma unroll
    for (int i = 0; i < kWaves; ++i)
      if (wlo[i] >= u0 && wlo[i] < u1) first[i] = p;
    if (blockIdx.x == 0 && U >= 4) {
      const int64_t last = n4p[p + 1] > n4p[p] ? u1 - 1 : u1 - 2;  // start of the pair's last step
      const int o0 = owner_of(u0, U, W), o1 = owner_of(last, U, W);
      *reinterpret_cast<int2*>(wsh + 16 + 2 * p) = make_int2(o0 + p, o1 - o0 + 1);
    }
  }
  __syncthreads();
  if (bad || U < 4 ||
      (!(SKIP && a.paged) && geo.data_offset + (int64_t)n8p[P] * geo.rec8 + (int64_t)n4p[P] * geo.rec4 > geo.total)) {
    if (blockIdx.x == 0 && tid == 0) wsh[0] = 0;
    return;
  }
  if (blockIdx.x == 0 && tid == 0) {
    wsh[0] = 1;
    wsh[1] = P;
    wsh[2] = (int)W + P;
    wsh[3] = (int)W;
  }
  float* part = a.ws + ws_part_offset(P) / 4;

  // ---- this wavefront's steps
  const int64_t w = (int64_t)blockIdx.x * kWaves + uni(wave);
  if (w >= W) return;
  const int64_t lo = uni64(wlo[wave]), hi = floor_div(U * (w + 1), W);
  int p = uni(first[wave]);
  for (; p < P && uni64(units_at(p)) < hi; ++p) {
    const int64_t u0 = uni64(units_at(p));
    const int n8 = uni(n8p[p + 1] - n8p[p]), n4 = uni(n4p[p + 1] - n4p[p]);
    const int s8 = n8 * SPB, s4 = n4 * SPB;
    // owned int8 steps: start u0 + 2j in [lo, hi); int4 steps: u0 + 2*s8 + j
    auto ceil2 = [](int64_t x) -> int64_t { return x <= 0 ? 0 : (x + 1) >> 1; };
    auto clampn = [](int64_t x, int n) -> int { return x <= 0 ? 0 : (x >= n ? n : (int)x); };
    const int j8a = clampn(ceil2(lo - u0), s8), j8b = clampn(ceil2(hi - u0), s8);
    const int64_t base4 = u0 + 2LL * s8;
    const int j4a = clampn(lo - base4, s4), j4b = clampn(hi - base4, s4);
    if (j8a >= j8b && j4a >= j4b) continue;
    const int slot = p + (int)w;
    const int b = p / a.hkv, gkv = p % a.hkv;
    const uint8_t* rec0 =
        a.cache + geo.data_offset + (int64_t)uni(n8p[p]) * geo.rec8 + (int64_t)uni(n4p[p]) * geo.rec4;
    // SKIP: the pair's records start at its (validated) offset; n8s, n4s records stored
    int n8s = n8;
    const int2* list = nullptr;
    const int32_t* pages = nullptr;
    const uint8_t* rec4 = nullptr;
    int64_t stride8 = geo.rec8, stride4 = geo.rec4;
    if constexpr (SKIP) {
      if (from_plan) {  // kept records from the plan (entries: stored index, or page when paged)
        const int* pe = a.plan + 8 * (int64_t)p;
        rec0 = a.cache + (int64_t)(((uint64_t)(uint32_t)pe[1] << 32) | (uint32_t)pe[0]);
        n8s = uni(pe[4]);
        list = reinterpret_cast<const int2*>(a.plan + 8 * (int64_t)P) + (int64_t)p * a.rmax;
      } else {  // every record, pages from the table
        pages = reinterpret_cast<const int32_t*>(a.cache + 64 + 64LL * P) + (int64_t)p * prmax;
      }
      if (a.paged) {
        rec0 = a.pool;
        stride8 = stride4 = a.page_bytes;
      }
    }
    rec4 = SKIP && a.paged ? rec0 : rec0 + (int64_t)n8s * geo.rec8;
    if constexpr (SKIP) {  // pair-uniform: kept in scalar registers across the pair's steps
      rec0 = reinterpret_cast<const uint8_t*>(uni64(reinterpret_cast<int64_t>(rec0)));
      rec4 = reinterpret_cast<const uint8_t*>(uni64(reinterpret_cast<int64_t>(rec4)));
      list = reinterpret_cast<const int2*>(uni64(reinterpret_cast<int64_t>(list)));
      pages = reinterpret_cast<const int32_t*>(uni64(reinterpret_cast<int64_t>(pages)));
      stride8 = uni64(stride8);
      stride4 = uni64(stride4);
    }
    const uint32_t hfull = G >= 32 ? 0xFFFFFFFFu : (1u << G) - 1u;

    // this pair's G query rows, quantised at both precisions (MFMA B operands)
    v4i q8op[RG][KS], q4op[RG][KS];
    float a8[RG], a4[RG];
    // the raw query rows are loaded first (unconditionally: padding rows re-read a
    // valid row and are zeroed below), so they are the oldest loads in flight
    v4i qraw[RG][KS][2];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int row = rg * 16 + lr < G ? rg * 16 + lr : G - 1;
          qraw[rg][ks][hh] = *reinterpret_cast<const v4i*>(a.q + ((int64_t)b * a.hq + gkv * G + row) * D + ks * 64 +
                                                           kq * 16 + hh * 8);
        }
    auto quantise_q = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        const int row = rg * 16 + lr;
        const bool valid = row < G;
        float x[KS][2][8];
        float amax = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const v4i q4 = valid ? qraw[rg][ks][hh] : v4i{0, 0, 0, 0};
            const uint4 raw = make_uint4((uint32_t)q4[0], (uint32_t)q4[1], (uint32_t)q4[2], (uint32_t)q4[3]);
            bf16x8_to_f32(raw, x[ks][hh]);
#pragma unroll
            for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[ks][hh][i]));
          }
        amax = xmax32(xmax16(amax));
        float sc8 = 0.f, sc4 = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          uint32_t c8a[2], c8b[2], c4a, c4b;
          codes_from_amax(x[ks][0], amax, c8a, c4a, sc8, sc4);
          codes_from_amax(x[ks][1], amax, c8b, c4b, sc8, sc4);
          q8op[rg][ks] = v4i{(int)c8a[0], (int)c8a[1], (int)c8b[0], (int)c8b[1]};
          q4op[rg][ks] = unpack16_x16(c4a, c4b);
        }
        a8[rg] = fmaxf(sc8 * a.c, FLT_MIN);
        a4[rg] = fmaxf(sc4 * a.c * (1.0f / 256.0f), FLT_MIN);
      }
    };

    SegState<D, RG> st;
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      st.m[rg] = -INFINITY;
      st.l[rg] = 0.0f;
      st.c[rg] = 0.0f;
#pragma unroll
      for (int d = 0; d < ND; ++d) st.O[rg][d] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    st.k = 8;
    // the last int8 record is the current block; keys at or past ctx_len are masked
    const int mask_first = uni(mfp[p]);
    const bool has8 = j8a < j8b;
    run_steps<D, BLK, RG, false, SKIP>(rec0, geo.rec8, j8a, j8b, q8op, a8, n8 - 1, mask_first, st, lr, kq,
                                       scl[wave], quantise_q, list, stride8, hfull, pages, a.pool_pages);
    run_steps<D, BLK, RG, true, SKIP>(rec4, geo.rec4, j4a, j4b, q4op, a4, -1, 0, st, lr, kq, scl[wave],
                                      [&]() __attribute__((always_inline)) {
                                        if (!has8) quantise_q();
                                      },
                                      SKIP && list ? list + n8s : nullptr, stride4, hfull, pages ? pages + n8s : nullptr,
                                      a.pool_pages);

    // ---- the wavefront's partial for this pair
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      const float l = xsum32(xsum16(st.l[rg]));
      // O = (accumulated - bias correction) / 2^k (exact scaling)
      const float c = xsum32(xsum16(st.c[rg]));
      const float inv = __builtin_ldexpf(1.0f, -st.k);
      const int row = rg * 16 + lr;
      if (row < G) {
        float* dst = part + ((int64_t)slot * G + row) * (D + 4);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
          *reinterpret_cast<float4*>(dst + dt * 16 + kq * 4) =
              make_float4((st.O[rg][dt][0] - c) * inv, (st.O[rg][dt][1] - c) * inv, (st.O[rg][dt][2] - c) * inv,
                          (st.O[rg][dt][3] - c) * inv);
        if (kq == 0) *reinterpret_cast<float4*>(dst + D) = make_float4(st.m[rg], l, 0.0f, 0.0f);
      }
    }
  }
}

// Merge of the partials of each pair: one work group per (batch, query head), one
// thread per output column.  The pair's slot range and, for the first 32 slots (a
// pair spans about W / P + 1 of them: 17 at 2048 wavefronts and 128 pairs), every
// column value are loaded in two rounds with all loads in flight; thread t also
// takes slot t's (m, l).  Then M = max m, f_i = 2^(m_i - M) through LDS, and
// out = sum_i f_i o_i / sum_i f_i l_i.
template <int D>
__global__ void __launch_bounds__(D) decode_merge_kernel(DecArgs a) {
  constexpr int NW = D / 64, BO = 32;
  __shared__ float fs[D];
  __shared__ float red[2][NW];
  const int bh = blockIdx.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int b = bh / a.hq, h = bh % a.hq;
  const int G = a.hq / a.hkv;
  const int pair = b * a.hkv + h / G, row = h % G;
  const int* wsh = reinterpret_cast<const int*>(a.ws);
  float* dst = a.out + (int64_t)bh * D;
  // header and slot range in one round (the workspace holds them for every pair; the
  // empty asm needs all four at once, so the range load is not moved behind the
  // header test, a second round trip)
  int valid = wsh[0], np = wsh[1];
  int2 range = *reinterpret_cast<const int2*>(wsh + 16 + 2 * pair);
  asm volatile("" : "+s"(valid), "+s"(np), "+s"(range.x), "+s"(range.y));
  const int i0 = range.x, i1 = range.x + range.y;
  if (valid != 1 || np != a.batch * a.hkv) {
    dst[t] = __int_as_float(0x7FC00000);  // NaN: the cache did not validate
    return;
  }
  const float* part = a.ws + ws_part_offset(np) / 4;
  auto rowp = [&](int it) { return part + ((int64_t)it * G + row) * (D + 4); };
  float o = 0.0f, lsum = 0.0f;
  float M = -INFINITY;  // maximum over all slots (first chunk's pass computes it for <= D slots)
  for (int base = i0; base < i1; base += D) {
    const int n = i1 - base < D ? i1 - base : D;
    // slot base + t's (m, l), and the first BO slots' column t, all in flight
    float2 ml = make_float2(-INFINITY, 0.0f);
    if (t < n) ml = *reinterpret_cast<const float2*>(rowp(base + t) + D);
    float oc[BO];
#pragma unroll
    for (int j = 0; j < BO; ++j) oc[j] = rowp(base + (j < n ? j : 0))[t];
    float mx = ml.x;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) mx = fmaxf(mx, __shfl_xor(mx, s));
    if (lane == 0) red[0][wv] = mx;
    __syncthreads();
    mx = red[0][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) mx = fmaxf(mx, red[0][w]);
    // fold the running sums into the new maximum (exact powers of two apart, or 0)
    const float Mn = fmaxf(M, mx);
    const float fo = M == -INFINITY ? 0.0f : exp2f(M - Mn);
    o *= fo;
    lsum *= fo;
    M = Mn;
    const float f = ml.x == -INFINITY ? 0.0f : exp2f(ml.x - M);
    fs[t] = f;
    lsum += t < n ? ml.y * f : 0.0f;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < BO; ++j) o += j < n ? fs[j] * oc[j] : 0.0f;
    for (int j = BO; j < n; ++j) o += fs[j] * rowp(base + j)[t];
    __syncthreads();
  }
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) lsum += __shfl_xor(lsum, s);
  if (lane == 0) red[1][wv] = lsum;
  __syncthreads();
  float l = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) l += red[1][w];
  dst[t] = o / l;
}

// ---- dynamic block skipping (ETA page, rit.work: section on how the model decides
// which part of the context to read).  Per stored record a few statistics of its K
// codes bound every score of the record; a record whose bound is below a query
// head's threshold is skipped for that head, and a record every head of the group
// skips is never read.
//
// Statistics index: a 64-byte header {magic, version 2, pairs, record slots per pair
// (rmax = current block + 1), d, block, current block, 0, cache total bytes (int64)},
// then per (pair, record slot) S = 2d + 16 bytes: lo[d], hi[d] (int8: per-coordinate
// minimum and maximum code over the record's rows), the largest row scale (fp32), the
// stamp (the pair's current block + 1 when the slot was built; 0 for an unused slot),
// and the largest (scale * scale) * |codes|^2 over rows (fp64).  A slot's statistics
// hold while its pair keeps the same current block: the record order, and every record
// before the current one, depend only on it.
constexpr int kSumMagic = 0x4D534254;  // "TBSM"
__host__ __device__ constexpr int sum_stride(int d) { return 2 * d + 16; }

struct SkipArgs {
  const uint8_t* cache;
  int64_t cache_bytes;
  int64_t ctx_len;
  const uint8_t* sums;
  uint8_t* sums_out;
  const uint16_t* q;
  const float* th;
  uint32_t* masks;  // or null: [P][rmax] keep bits per stored record
  int* plan;        // or null: [P][8] pair entries, then [P][rmax] kept {record, mask} lists
  float sm;
  int batch, hq, hkv, rmax;
  // paged cache: `cache` is the page table (fixed length), records in the pool
  int paged;
  int varlen;  // version-3 cache: each pair's ctx_len in its directory entry

  const uint8_t* pool;
  int64_t pool_pages;
};

// The cache header (contiguous) or the page table header (paged) against the launch.
template <int D, int BLK>
__device__ __forceinline__ bool skip_header_h(const SkipArgs& s, const Hdr64& h, Geo& geo) {
  DecArgs a{};
  a.cache = s.cache;
  a.cache_bytes = s.cache_bytes;
  a.ctx_len = s.ctx_len;
  a.batch = s.batch;
  a.hkv = s.hkv;
  a.varlen = s.varlen;
  return s.paged ? paged_header_h<D, BLK>(a, h, geo) : header_ok_h<D, BLK>(a, h, geo);
}
template <int D, int BLK>
__device__ __forceinline__ bool skip_header_ok(const SkipArgs& s, Geo& geo) {
  Hdr64 h = *reinterpret_cast<const Hdr64*>(s.cache);
  pin_hdr(h);
  return skip_header_h<D, BLK>(s, h, geo);
}

// Page slots per pair of a paged table: the index's rmax, or (variable length) the
// table's own (header word 6, checked against the table size by the header test).
__device__ __forceinline__ int table_rmax(const SkipArgs& s) {
  return s.varlen ? reinterpret_cast<const int32_t*>(s.cache)[6] : s.rmax;
}

// Page of record r of pair p in a paged table, or -1 when outside the pool.
__device__ __forceinline__ int page_of(const SkipArgs& s, int p, int r) {
  const int pg =
      reinterpret_cast<const int32_t*>(s.cache + 64 + 64LL * s.batch * s.hkv)[(int64_t)p * table_rmax(s) + r];
  return pg >= 0 && (int64_t)pg < s.pool_pages ? pg : -1;
}

// The index describes this cache's records: same pairs, slots, shape, current block
// and total size (statistics of the current block itself are never used).
template <int D, int BLK>
__device__ __forceinline__ bool sums_ok(const SkipArgs& s, const Hdr64& h, const Geo& geo) {
  return h.w[0] == kSumMagic && h.w[1] == 2 && h.w[2] == s.batch * s.hkv && h.w[3] == s.rmax && h.w[4] == D &&
         h.w[5] == BLK && h.w[6] == (s.varlen ? -1 : geo.cur) && h.q(4) == geo.total;
}

// One work group per (pair, record slot): the record's K codes are staged in LDS
// with 16-byte loads, then per-coordinate ranges (thread per coordinate) and per-row
// norms (256 / BLK threads per row) are reduced.
template <int D, int BLK>
__global__ void __launch_bounds__(kThreads) summaries_kernel(SkipArgs a) {
  constexpr int KS = D / 64, SPB = BLK / 32, NG = kThreads / D, TPT = kThreads / BLK, S = sum_stride(D);
  __shared__ __attribute__((aligned(16))) int8_t kc[BLK * D];  // int4 records use half
  __shared__ int rng[2][NG][D];
  __shared__ double nmw[kWaves];
  __shared__ float smw[kWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = a.batch * a.hkv;
  const int p = blockIdx.x / a.rmax, r = blockIdx.x % a.rmax;
  Geo geo;
  if (!skip_header_ok<D, BLK>(a, geo)) return;
  uint8_t* dst = a.sums_out + 64 + (int64_t)blockIdx.x * S;
  if (blockIdx.x == 0 && tid == 0) {
    int32_t* h = reinterpret_cast<int32_t*>(a.sums_out);
    int64_t* h64 = reinterpret_cast<int64_t*>(a.sums_out);
    h[0] = kSumMagic;
    h[1] = 2;
    h[2] = P;
    h[3] = a.rmax;
    h[4] = D;
    h[5] = BLK;
    h[6] = a.varlen ? -1 : geo.cur;
    h[7] = 0;
    h64[4] = geo.total;
    h64[5] = h64[6] = h64[7] = 0;
  }
  const v4i* e = reinterpret_cast<const v4i*>(a.cache + 64 + 64 * (int64_t)p);
  const v4i e0 = e[0], e2 = e[2];
  const int64_t off = (int64_t)(((uint64_t)(uint32_t)e0[1] << 32) | (uint32_t)e0[0]);
  const int n8 = e0[2], n4 = e0[3];
  // the pair's current block (variable length: from its entry's ctx_len)
  const int64_t pctx = a.varlen ? (int64_t)(((uint64_t)(uint32_t)e2[3] << 32) | (uint32_t)e2[2]) : a.ctx_len;
  if (n8 < 1 || n4 < 0 || n8 + n4 > a.rmax || (a.paged && n8 + n4 > table_rmax(a)) || pctx < 1 ||
      (pctx - 1) / BLK >= a.rmax ||
      (!a.paged && (off < geo.data_offset || off + (int64_t)n8 * geo.rec8 + (int64_t)n4 * geo.rec4 > geo.total)))
    return;
  const int stamp = (int)((pctx - 1) / BLK) + 1;
  if (r >= n8 + n4) {  // unused slot: zeros
    for (int i = tid; i < S / 4; i += kThreads) reinterpret_cast<int*>(dst)[i] = 0;
    return;
  }
  const bool is4 = r >= n8;
  const int pg = a.paged ? page_of(a, p, r) : 0;
  if (pg < 0) return;
  const uint8_t* rec = a.paged ? a.pool + (int64_t)pg * (2LL * BLK * D + 8LL * BLK)
                               : a.cache + off + (is4 ? (int64_t)n8 * geo.rec8 + (int64_t)(r - n8) * geo.rec4
                                                      : (int64_t)r * geo.rec8);
  const int kpart = is4 ? 16 * D : 32 * D, cb = 2 * kpart + 256;
  for (int u = tid; u < SPB * kpart / 16; u += kThreads) {
    const int h = u / (kpart / 16), o = (u % (kpart / 16)) * 16;
    *reinterpret_cast<v4i*>(kc + h * kpart + o) = *reinterpret_cast<const v4i*>(rec + (int64_t)h * cb + o);
  }
  __syncthreads();
  // code of row t, coordinate x in the chunk layout (int8 unit (s, ks, q, r) of 16
  // bytes; int4 unit (s, q, r) of 8 * KS bytes, low nibble = even coordinate)
  auto code = [&](int t, int x) __attribute__((always_inline)) -> int {
    const int h = t / 32, s = (t % 32) / 16, rr = t % 16, ks = x / 64, q = (x % 64) / 16, el = x % 16;
    if (!is4) return kc[h * kpart + ((s * KS + ks) * 4 + q) * 256 + rr * 16 + el];
    const int b = (uint8_t)kc[h * kpart + ((s * 4 + q) * 16 + rr) * 8 * KS + ks * 8 + el / 2];
    const int nib = (b >> (4 * (el & 1))) & 0xF;
    return (nib ^ 8) - 8;
  };
  {
    const int x = tid % D, tg = tid / D;
    int lo = code(tg, x), hi = lo;
    for (int t = tg + NG; t < BLK; t += NG) {
      const int c = code(t, x);
      lo = c < lo ? c : lo;
      hi = c > hi ? c : hi;
    }
    rng[0][tg][x] = lo;
    rng[1][tg][x] = hi;
  }
  double nv;
  float sv;
  {
    const int t = tid / TPT, part = tid % TPT;
    int n2 = 0;
    for (int x = part * (D / TPT); x < (part + 1) * (D / TPT); ++x) {
      const int c = code(t, x);
      n2 += c * c;
    }
#pragma unroll
    for (int o = TPT / 2; o >= 1; o >>= 1) n2 += __shfl_xor(n2, o, TPT);
    sv = *reinterpret_cast<const float*>(rec + (int64_t)(t / 32) * cb + 2 * kpart + (t % 32) * 4);
    nv = ((double)sv * (double)sv) * (double)n2;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const double on = __shfl_xor(nv, o);
    const float os = __shfl_xor(sv, o);
    nv = on > nv ? on : nv;
    sv = os > sv ? os : sv;
  }
  if (lane == 0) {
    nmw[wave] = nv;
    smw[wave] = sv;
  }
  __syncthreads();
  if (tid < D) {
    int lo = rng[0][0][tid], hi = rng[1][0][tid];
#pragma unroll
    for (int g = 1; g < NG; ++g) {
      lo = rng[0][g][tid] < lo ? rng[0][g][tid] : lo;
      hi = rng[1][g][tid] > hi ? rng[1][g][tid] : hi;
    }
    dst[tid] = (uint8_t)(int8_t)lo;
    dst[D + tid] = (uint8_t)(int8_t)hi;
  }
  if (tid == 0) {
    double n = nmw[0];
    float m = smw[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      n = nmw[w] > n ? nmw[w] : n;
      m = smw[w] > m ? smw[w] : m;
    }
    *reinterpret_cast<float*>(dst + 2 * D) = m;
    *reinterpret_cast<int*>(dst + 2 * D + 4) = stamp;
    *reinterpret_cast<double*>(dst + 2 * D + 8) = n;
  }
}

// Exclusive prefix of two values over a work group of NW wavefronts (tmp: 2 * NW ints);
// tx, ty = the totals.
template <int NW>
__device__ __forceinline__ int2 block_scan2_n(int x, int y, int* tmp, int& tx, int& ty) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ix = wave_scan_incl(x), iy = wave_scan_incl(y);
  if (lane == 63) {
    tmp[wave] = ix;
    tmp[NW + wave] = iy;
  }
  __syncthreads();
  int bx = 0, by = 0;
  tx = 0;
  ty = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = tmp[w], u = tmp[NW + w];
    bx += w < wave ? t : 0;
    by += w < wave ? u : 0;
    tx += t;
    ty += u;
  }
  __syncthreads();
  return make_int2(bx + ix - x, by + iy - y);
}

// The plan of one pair per work group of 1024 lanes, one lane per (record slot, query
// head): Gp = G rounded up to a power of two consecutive lanes per record, so a pass
// covers 1024 / Gp records, or the index slots that fit the 72 KB stage in LDS if
// fewer.  Keep bits: for query head h (codes qc, scale sq at the
// record's precision) and threshold th,
//   box  = (t * smax) * max(sum_x max(qc_x lo_x, qc_x hi_x), 0),  t = sm_scale * sq
//   norm = ((t * t) * |qc|^2) * nmax
// and h skips the record iff th > 0 and (box < th or norm < th * th), all in IEEE
// double in this order (bit-reproducible); the first and the current record are
// always kept.  With a plan buffer, the kept records of each run are listed in order
// ({stored index in the run, keep bits}: int8 run from slot 0, int4 run from slot
// n8) and the pair entry {offset lo, hi, kept int8, kept int4, stored int8, stored
// int4, keys of the current block below ctx_len, ok} is written after the
// directory checks of the decode (and that the pair's records start where the
// previous pair's end).  With a masks buffer, the keep bits of every stored record.
constexpr int kPlanThreads = 1024;
constexpr int kPlanStageBytes = 72 * 1024;  // LDS for the index slots of one pass
#pragma clang fp contract(off)
template <int D, int BLK>
__global__ void __launch_bounds__(kPlanThreads) skip_plan_kernel(SkipArgs a) {
  constexpr int TPR = D / 8, S = sum_stride(D), KW = D / 16, NW = kPlanThreads / 64;
  __shared__ __attribute__((aligned(16))) int8_t qc[2][32][D];
  __shared__ float sq[2][32];
  __shared__ int q2[2][32];
  __shared__ float ths[32];
  __shared__ int tmp[2 * NW];
  __shared__ int stale_w[NW];
  // index slots of the current pass, copied from memory with whole-row loads (lanes
  // reading 16 bytes each from a different 272-byte slot pull a cache line per lane
  // per load, several times the slots' bytes)
  constexpr int CHMAX = kPlanStageBytes / S, SWEEPS = (kPlanStageBytes / 16 + kPlanThreads - 1) / kPlanThreads;
  __shared__ __attribute__((aligned(16))) uint8_t stage[CHMAX * S];
  const int tid = threadIdx.x, lane = tid & 63;
  const int G = a.hq / a.hkv, P = a.batch * a.hkv;
  int Gp = 1;
  while (Gp < G) Gp <<= 1;
  const int rpp = kPlanThreads / Gp, h = tid % Gp;
  const int CH = rpp < CHMAX ? rpp : CHMAX;  // slots per pass
  const int p = blockIdx.x, b = p / a.hkv, g = p % a.hkv;
  // every load first, in one round trip: both headers, the directory entries of this
  // pair and the previous one, the query rows, the thresholds and this lane's first
  // index slot (no address depends on a loaded value; all lie inside their buffers)
  const Hdr64 hc = *reinterpret_cast<const Hdr64*>(a.cache);
  const Hdr64 hs = *reinterpret_cast<const Hdr64*>(a.sums);
  const v4i* ep = reinterpret_cast<const v4i*>(a.cache + 64 + 64 * (int64_t)p);
  const v4i e0 = ep[0], e1 = ep[1], e2 = ep[2];
  const v4i f = *reinterpret_cast<const v4i*>(a.cache + 64 + 64 * (int64_t)(p > 0 ? p - 1 : p));
  const int qrow = tid / TPR, qpart = tid % TPR;  // G * TPR <= 512 pieces
  uint4 qraw = make_uint4(0, 0, 0, 0);
  if (qrow < G) qraw = *reinterpret_cast<const uint4*>(a.q + ((int64_t)b * a.hq + g * G + qrow) * D + qpart * 8);
  const float th_own = tid < G ? a.th[(int64_t)b * a.hq + g * G + tid] : 0.0f;
  // slots r0 .. r0 + n - 1 (n <= CH, r0 + n <= rmax): lane t loads 16-byte pieces t,
  // t + 1024, ... of their contiguous bytes, then writes them to the stage
  v4u piece[SWEEPS];
  auto stage_load = [&](int r0, int n) __attribute__((always_inline)) {
    const v4u* src = reinterpret_cast<const v4u*>(a.sums + 64 + ((int64_t)p * a.rmax + r0) * S);
    const int npieces = n * (S / 16);
#pragma unroll
    for (int i = 0; i < SWEEPS; ++i)
      if (tid + i * kPlanThreads < npieces) piece[i] = src[tid + i * kPlanThreads];
    return npieces;
  };
  auto stage_store = [&](int npieces) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SWEEPS; ++i)
      if (tid + i * kPlanThreads < npieces) reinterpret_cast<v4u*>(stage)[tid + i * kPlanThreads] = piece[i];
  };
  // the first pass's slots with the other loads (the record count is not known yet:
  // every slot the pass could use)
  const int first_pieces = stage_load(0, a.rmax < CH ? a.rmax : CH);
  stage_store(first_pieces);
  // ---- checks (uniform)
  DecArgs da{};
  da.cache_bytes = a.cache_bytes;
  da.ctx_len = a.ctx_len;
  da.batch = a.batch;
  da.hkv = a.hkv;
  Geo geo;
  bool ok = skip_header_h<D, BLK>(a, hc, geo) && sums_ok<D, BLK>(a, hs, geo);
  const int64_t off = (int64_t)(((uint64_t)(uint32_t)e0[1] << 32) | (uint32_t)e0[0]);
  const int n8 = e0[2], n4 = e0[3], nrec = n8 + n4;
  // this pair's ctx_len and current block (variable length: from its entry)
  const int64_t pctx = a.varlen ? (int64_t)(((uint64_t)(uint32_t)e2[3] << 32) | (uint32_t)e2[2]) : a.ctx_len;
  const bool pctx_ok = pctx >= 1 && pctx <= (1LL << 40);
  const int cur = pctx_ok ? (int)((pctx - 1) / BLK) : 0;
  ok = ok && pctx_ok;
  {
    const int lo8 = e1[2], sink = e1[3], lo4 = e2[0];
    const int64_t expect = p == 0 ? geo.data_offset
                                  : (int64_t)(((uint64_t)(uint32_t)f[1] << 32) | (uint32_t)f[0]) +
                                        (int64_t)f[2] * geo.rec8 + (int64_t)f[3] * geo.rec4;
    ok = ok && n8 >= 1 && n4 >= 0 && n8 + n4 <= cur + 1 && (sink == 0 || sink == 1) && lo8 >= 0 &&
         lo8 + (n8 - sink) - 1 == cur && sink == (lo8 > 0 ? 1 : 0) && lo4 >= 0 && lo4 + n4 <= cur + 1 &&
         (a.paged || (off == expect && off + (int64_t)n8 * geo.rec8 + (int64_t)n4 * geo.rec4 <= geo.total)) &&
         (a.varlen ? cur + 1 <= a.rmax : cur + 1 == a.rmax) && (!a.paged || cur + 1 <= table_rmax(a));
  }
  {  // every stored record's slot was built for this current block (a variable-length
     // sequence that moved to another block, or restarted in one, leaves stale slots)
    bool stale = false;
    const int staged = a.rmax < CH ? a.rmax : CH;
    __syncthreads();  // the stage written
    if (ok)
      for (int r = tid; r < nrec; r += kPlanThreads)
        stale = stale || (r < staged ? *reinterpret_cast<const int*>(stage + r * S + 2 * D + 4)
                                     : *reinterpret_cast<const int*>(a.sums + 64 + ((int64_t)p * a.rmax + r) * S +
                                                                     2 * D + 4)) != cur + 1;
    // (a block OR through LDS: __syncthreads_or reads the work-group size from the
    // kernel's hidden arguments, one more memory round trip)
    const bool wave_stale = __ballot(stale) != 0;
    if (lane == 0) stale_w[tid >> 6] = wave_stale;
    __syncthreads();
    bool any = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) any = any || stale_w[w] != 0;
    ok = ok && !any;
  }
  int* pe = a.plan ? a.plan + 8 * (int64_t)p : nullptr;
  if (!ok) {
    if (pe && tid < 8) pe[tid] = 0;
    return;
  }
  // ---- the pair's G query rows at both precisions (the decode's quantiser)
  if (tid < 512) {  // whole TPR groups (uniform per group)
    float x[8];
    bf16x8_to_f32(qraw, x);
    uint32_t c8[2], c4;
    float s8, s4;
    quantize8<TPR>(x, c8, c4, s8, s4);
    int n8sq = 0, n4sq = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int v8 = (int8_t)((c8[k / 4] >> (8 * (k % 4))) & 0xFFu);
      const int v4 = (((int)((c4 >> (4 * k)) & 0xFu)) ^ 8) - 8;
      n8sq += v8 * v8;
      n4sq += v4 * v4;
      if (qrow < G) {
        qc[0][qrow][qpart * 8 + k] = (int8_t)v8;
        qc[1][qrow][qpart * 8 + k] = (int8_t)v4;
      }
    }
#pragma unroll
    for (int o = TPR / 2; o >= 1; o >>= 1) {
      n8sq += __shfl_xor(n8sq, o, TPR);
      n4sq += __shfl_xor(n4sq, o, TPR);
    }
    if (qrow < G && qpart == 0) {
      sq[0][qrow] = s8;
      sq[1][qrow] = s4;
      q2[0][qrow] = n8sq;
      q2[1][qrow] = n4sq;
    }
  }
  if (tid < G) ths[tid] = th_own;
  __syncthreads();
  const uint32_t gm = G >= 32 ? 0xFFFFFFFFu : (1u << G) - 1u;
  int2* list = a.plan ? reinterpret_cast<int2*>(a.plan + 8 * (int64_t)P) + (int64_t)p * a.rmax : nullptr;
  int c8 = 0, c4 = 0;
  for (int r0 = 0; r0 < nrec; r0 += CH) {
    if (r0 > 0) {  // the next slots, once every lane has read the previous ones
      __syncthreads();
      stage_store(stage_load(r0, nrec - r0 < CH ? nrec - r0 : CH));
      __syncthreads();
    }
    const int rl = tid / Gp, r = r0 + rl;
    const bool in = rl < CH && r < nrec;
    bool keep = false;
    if (in && h < G) {
      if (r == 0 || r == n8 - 1) {
        keep = true;
      } else {
        const uint8_t* sp = stage + rl * S;
        v4u lo[KW], hi[KW];
#pragma unroll
        for (int w = 0; w < KW; ++w) {
          lo[w] = reinterpret_cast<const v4u*>(sp)[w];
          hi[w] = reinterpret_cast<const v4u*>(sp + D)[w];
        }
        const float smax = *reinterpret_cast<const float*>(sp + 2 * D);
        const double nmax = *reinterpret_cast<const double*>(sp + 2 * D + 8);
        const int pr = r < n8 ? 0 : 1;
        // per byte of q: the bound's coordinate is hi where the code is >= 0, else lo
        const v4u* qv = reinterpret_cast<const v4u*>(&qc[pr][h][0]);
        int box = 0;
#pragma unroll
        for (int w = 0; w < KW; ++w) {
          const v4u qq = qv[w];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t neg = ((qq[i] >> 7) & 0x01010101u) * 0xFFu;
            const uint32_t sel = (lo[w][i] & neg) | (hi[w][i] & ~neg);
            box = __builtin_amdgcn_sdot4((int)qq[i], (int)sel, box, false);
          }
        }
        const double t = (double)a.sm * (double)sq[pr][h];
        const double bound = (t * (double)smax) * (double)(box > 0 ? box : 0);
        const double norm2 = ((t * t) * (double)q2[pr][h]) * nmax;
        const double th = (double)ths[h];
        keep = !(th > 0.0 && (bound < th || norm2 < th * th));
      }
    }
    // the record's keep bits from its Gp lanes (aligned groups inside the wavefront)
    const uint64_t bal = __ballot(keep);
    const uint32_t mk = (uint32_t)(bal >> (lane & ~(Gp - 1))) & gm;
    const bool lead = h == 0 && in;
    if (lead && a.masks) a.masks[(int64_t)p * a.rmax + r] = mk;
    if (list) {
      const int f8 = lead && r < n8 && mk ? 1 : 0, f4 = lead && r >= n8 && mk ? 1 : 0;
      int t8, t4;
      const int2 ex = block_scan2_n<NW>(f8, f4, tmp, t8, t4);
      // (paged: the entry holds the record's page; a page outside the pool is read as
      // page 0 and the pair's sums are poisoned with NaN by its keep bits of 0)
      const int pg = a.paged && (f8 || f4) ? page_of(a, p, r) : 0;
      if (f8) list[c8 + ex.x] = make_int2(a.paged ? (pg < 0 ? 0 : pg) : r, pg < 0 ? 0 : (int)mk);
      if (f4) list[n8 + c4 + ex.y] = make_int2(a.paged ? (pg < 0 ? 0 : pg) : r - n8, pg < 0 ? 0 : (int)mk);
      c8 += t8;
      c4 += t4;
    }
  }
  if (pe && tid == 0) {
    pe[0] = (int)(uint32_t)off;
    pe[1] = (int)(off >> 32);
    pe[2] = c8;
    pe[3] = c4;
    pe[4] = n8;
    pe[5] = n4;
    pe[6] = (int)(pctx - (int64_t)cur * BLK);
    pe[7] = 1;
  }
}
#pragma clang fp contract(on)

// Work groups of the split kernel: kGrid, or fewer when TRIA_DECODE_GRID (1..kGrid) is
// set -- a testing and tuning knob: fewer wavefronts give each one longer segments.
int split_grid() {
  const char* e = getenv("TRIA_DECODE_GRID");
  if (!e) return kGrid;
  const int g = atoi(e);
  return g >= 1 && g <= kGrid ? g : kGrid;
}

template <int D, int BLK, int RG, bool SKIP = false>
hipError_t launch_t(const DecArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<D, BLK, RG, SKIP>), dim3(split_grid()), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.batch * a.hq), dim3(D), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

// Scratch of the decode entry point that allocates nothing: the split kernel's
// partials and slot table live here instead of in a caller workspace.  Each device
// holds its own copy of the array for as long as the process runs.  In host code
// `scratch` names a host-side stand-in, never the device memory: kernels get the
// address hipGetSymbolAddress returns on the device, kept per device below.
namespace {
constexpr int64_t kScratchBytes = 64LL << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};
}  // namespace

int64_t decode_scratch_capacity() { return kScratchBytes; }

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {  // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_dev[dev] = p;
  }
  *ptr = g_scratch_dev[dev];
  return hipSuccess;
}

int64_t decode_workspace_bytes(const Shape& s, int64_t ctx_len) {
  (void)ctx_len;  // the split is by wavefront: at most one partial per wavefront and pair boundary
  const int64_t pairs = (int64_t)s.batch * s.hkv;
  const int G = s.hq / s.hkv;
  return ws_part_offset(pairs) + (kMaxWaves + pairs) * G * (s.d + 4) * 4;
}

bool decode_units_fit(const Shape& s, int64_t ctx_len) {
  const int64_t nb = (ctx_len - 1) / s.blk + 1;
  return (int64_t)s.batch * s.hkv * nb * (s.blk / 32) * 2 < (1LL << 31);
}

hipError_t launch_decode(const Shape& s, int64_t ctx_len, const void* cache, int64_t cache_bytes,
                         const void* q, float sm_scale, float* out, void* workspace, bool varlen,
                         hipStream_t stream) {
  DecArgs a;
  a.cache = static_cast<const uint8_t*>(cache);
  a.q = static_cast<const uint16_t*>(q);
  a.ws = static_cast<float*>(workspace);
  a.out = out;
  a.cache_bytes = cache_bytes;
  a.ctx_len = ctx_len;
  a.batch = s.batch;
  a.hq = s.hq;
  a.hkv = s.hkv;
  a.c = sm_scale * 1.44269504088896340736f;
  a.varlen = varlen ? 1 : 0;
  a.plan = nullptr;
  a.rmax = 0;
  a.paged = 0;
  a.pool = nullptr;
  a.page_bytes = a.pool_pages = 0;
  const int G = s.hq / s.hkv;
  const bool two = G > 16;
  if (s.d == 128 && s.blk == 128) return two ? launch_t<128, 128, 2>(a, stream) : launch_t<128, 128, 1>(a, stream);
  if (s.d == 128 && s.blk == 64) return two ? launch_t<128, 64, 2>(a, stream) : launch_t<128, 64, 1>(a, stream);
  if (s.d == 64 && s.blk == 128) return two ? launch_t<64, 128, 2>(a, stream) : launch_t<64, 128, 1>(a, stream);
  return two ? launch_t<64, 64, 2>(a, stream) : launch_t<64, 64, 1>(a, stream);
}

int64_t summaries_bytes(const Shape& s, int64_t ctx_len) {
  const int64_t rmax = (ctx_len - 1) / s.blk + 1;
  return 64 + (int64_t)s.batch * s.hkv * rmax * sum_stride(s.d);
}

int64_t skip_workspace_bytes(const Shape& s, int64_t ctx_len) {
  const int64_t pairs = (int64_t)s.batch * s.hkv, rmax = (ctx_len - 1) / s.blk + 1;
  const int64_t base = (decode_workspace_bytes(s, ctx_len) + 255) / 256 * 256;
  return base + 32 * pairs + 8 * pairs * rmax;
}

namespace {
SkipArgs skip_args(const Shape& s, int64_t ctx_len, const void* cache, int64_t cache_bytes, const void* sums,
                   const void* q, const float* th, float sm_scale) {
  SkipArgs a{};
  a.cache = static_cast<const uint8_t*>(cache);
  a.cache_bytes = cache_bytes;
  a.ctx_len = ctx_len;
  a.sums = static_cast<const uint8_t*>(sums);
  a.q = static_cast<const uint16_t*>(q);
  a.th = th;
  a.sm = sm_scale;
  a.batch = s.batch;
  a.hq = s.hq;
  a.hkv = s.hkv;
  a.rmax = (int)((ctx_len - 1) / s.blk + 1);
  a.paged = 0;
  a.varlen = 0;
  a.pool = nullptr;
  a.pool_pages = 0;
  return a;
}

template <int D, int BLK>
hipError_t launch_plan(const SkipArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((skip_plan_kernel<D, BLK>), dim3(a.batch * a.hkv), dim3(kPlanThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D, int BLK>
hipError_t launch_skip_t(const SkipArgs& sa, const DecArgs& da, bool two, hipStream_t stream) {
  const hipError_t e = launch_plan<D, BLK>(sa, stream);
  if (e != hipSuccess) return e;
  return two ? launch_t<D, BLK, 2, true>(da, stream) : launch_t<D, BLK, 1, true>(da, stream);
}
}  // namespace

hipError_t launch_decode_paged(const Shape& s, int64_t ctx_len, const void* table, int64_t table_bytes,
                               const void* pool, int64_t pool_bytes, const void* q, float sm_scale, float* out,
                               void* workspace, bool varlen, hipStream_t stream) {
  DecArgs da;
  da.cache = static_cast<const uint8_t*>(table);
  da.q = static_cast<const uint16_t*>(q);
  da.ws = static_cast<float*>(workspace);
  da.out = out;
  da.cache_bytes = table_bytes;
  da.ctx_len = ctx_len;
  da.batch = s.batch;
  da.hq = s.hq;
  da.hkv = s.hkv;
  da.c = sm_scale * 1.44269504088896340736f;
  da.varlen = varlen ? 1 : 0;  // (variable length: ctx_len 1, each pair's from the table)
  da.plan = nullptr;
  da.rmax = (int)((ctx_len - 1) / s.blk + 1);
  da.paged = 1;
  da.pool = static_cast<const uint8_t*>(pool);
  da.page_bytes = 2LL * s.blk * s.d + 8LL * s.blk;
  da.pool_pages = pool_bytes / da.page_bytes;
  const bool two = s.hq / s.hkv > 16;
  if (s.d == 128 && s.blk == 128) return two ? launch_t<128, 128, 2, true>(da, stream) : launch_t<128, 128, 1, true>(da, stream);
  if (s.d == 128) return two ? launch_t<128, 64, 2, true>(da, stream) : launch_t<128, 64, 1, true>(da, stream);
  if (s.blk == 128) return two ? launch_t<64, 128, 2, true>(da, stream) : launch_t<64, 128, 1, true>(da, stream);
  return two ? launch_t<64, 64, 2, true>(da, stream) : launch_t<64, 64, 1, true>(da, stream);
}

hipError_t launch_summaries(const Shape& s, int64_t ctx_len, const void* cache, int64_t cache_bytes, void* sums,
                            hipStream_t stream) {
  return launch_summaries_paged(s, ctx_len, cache, cache_bytes, sums, nullptr, 0, false, stream);
}

hipError_t launch_summaries_paged(const Shape& s, int64_t ctx_len, const void* cache, int64_t cache_bytes, void* sums,
                                  const void* pool, int64_t pool_bytes, bool varlen, hipStream_t stream) {
  SkipArgs a = skip_args(s, ctx_len, cache, cache_bytes, nullptr, nullptr, nullptr, 0.0f);
  a.varlen = varlen ? 1 : 0;
  a.paged = pool ? 1 : 0;
  a.pool = static_cast<const uint8_t*>(pool);
  a.pool_pages = pool ? pool_bytes / (2LL * s.blk * s.d + 8LL * s.blk) : 0;
  a.sums_out = static_cast<uint8_t*>(sums);
  const dim3 grid((unsigned)((int64_t)s.batch * s.hkv * a.rmax));
  if (s.d == 128 && s.blk == 128) hipLaunchKernelGGL((summaries_kernel<128, 128>), grid, dim3(kThreads), 0, stream, a);
  else if (s.d == 128) hipLaunchKernelGGL((summaries_kernel<128, 64>), grid, dim3(kThreads), 0, stream, a);
  else if (s.blk == 128) hipLaunchKernelGGL((summaries_kernel<64, 128>), grid, dim3(kThreads), 0, stream, a);
  else hipLaunchKernelGGL((summaries_kernel<64, 64>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_skip_masks(const Shape& s, int64_t ctx_len, const void* cache, int64_t cache_bytes,
                             const void* sums, const void* q, const float* thresholds, float sm_scale,
                             uint32_t* masks, hipStream_t stream) {
  SkipArgs a = skip_args(s, ctx_len, cache, cache_bytes, sums, q, thresholds, sm_scale);
  a.masks = masks;
  if (s.d == 128 && s.blk == 128) return launch_plan<128, 128>(a, stream);
  if (s.d == 128) return launch_plan<128, 64>(a, stream);
  if (s.blk == 128) return launch_plan<64, 128>(a, stream);
  return launch_plan<64, 64>(a, stream);
}

hipError_t launch_decode_skip(const Shape& s, int64_t ctx_len, const void* cache, int64_t cache_bytes,
                              const void* sums, const void* q, const float* thresholds, float sm_scale, float* out,
                              void* workspace, hipStream_t stream) {
  return launch_decode_skip_paged(s, ctx_len, cache, cache_bytes, sums, q, thresholds, sm_scale, out, workspace,
                                  nullptr, 0, false, stream);
}

hipError_t launch_decode_skip_paged(const Shape& s, int64_t ctx_len, const void* cache, int64_t cache_bytes,
                                    const void* sums, const void* q, const float* thresholds, float sm_scale,
                                    float* out, void* workspace, const void* pool, int64_t pool_bytes, bool varlen,
                                    hipStream_t stream) {
  SkipArgs sa = skip_args(s, ctx_len, cache, cache_bytes, sums, q, thresholds, sm_scale);
  sa.varlen = varlen ? 1 : 0;
  const int64_t page_bytes = 2LL * s.blk * s.d + 8LL * s.blk;
  sa.paged = pool ? 1 : 0;
  sa.pool = static_cast<const uint8_t*>(pool);
  sa.pool_pages = pool ? pool_bytes / page_bytes : 0;
  const int64_t base = (decode_workspace_bytes(s, ctx_len) + 255) / 256 * 256;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  sa.plan = reinterpret_cast<int*>(ws + base);
  sa.masks = nullptr;
  DecArgs da;
  da.cache = static_cast<const uint8_t*>(cache);
  da.q = static_cast<const uint16_t*>(q);
  da.ws = static_cast<float*>(workspace);
  da.out = out;
  da.cache_bytes = cache_bytes;
  da.ctx_len = ctx_len;
  da.batch = s.batch;
  da.hq = s.hq;
  da.hkv = s.hkv;
  da.c = sm_scale * 1.44269504088896340736f;
  da.varlen = sa.varlen;
  da.plan = sa.plan;
  da.rmax = sa.rmax;
  da.paged = sa.paged;
  da.pool = sa.pool;
  da.page_bytes = pool ? page_bytes : 0;
  da.pool_pages = sa.pool_pages;
  const bool two = s.hq / s.hkv > 16;
  if (s.d == 128 && s.blk == 128) return launch_skip_t<128, 128>(sa, da, two, stream);
  if (s.d == 128) return launch_skip_t<128, 64>(sa, da, two, stream);
  if (s.blk == 128) return launch_skip_t<64, 128>(sa, da, two, stream);
  return launch_skip_t<64, 64>(sa, da, two, stream);
}

}  // namespace tria
