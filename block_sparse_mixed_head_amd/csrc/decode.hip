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
// gfx950 design (split-KV, two kernels):
//   * The stored blocks of each (batch, KV head) pair are cut into items of up to
//     kGroupsPerItem 64-token groups.  A persistent grid walks the items; each work
//     group derives the item -> pair map from the cache directory itself (prefix
//     over the directory in LDS), so the host needs no knowledge of the policy.
//   * Each wavefront takes whole 64-token groups and serves all G query heads of
//     the KV head at once (G rows padded to 16 per MFMA row group): every cache
//     byte is read exactly once per step.
//   * q.k: v_mfma_i32_16x16x64_i8 with K codes loaded straight from HBM into
//     registers as the A operand (int4 groups widened to 16*code).
//   * p.v: v_mfma_f32_16x16x32_bf16 with the V codes (stored transposed, in feed
//     order, so each lane loads one 16-byte run) converted to bf16 exactly, and the
//     fp32 weight p*sv split into a bf16 high part and a bf16 remainder, so the
//     product keeps ~16 mantissa bits (fp32-class accuracy, no bf16 rounding of P).
//   * Online softmax in fp32 (base 2); the four wavefronts of a work group merge in
//     LDS; one partial (m, l, o[d]) per item and row goes to the workspace, and a
//     second kernel merges the items of each pair.
//   * The kernels validate the cache header and directory before reading any
//     record; on a mismatch nothing is read and the merge writes NaN.
#include <cfloat>

#include "device_common.h"
#include "kernels.h"

namespace tria {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kGroupsPerItem = 8;  // 64-token groups per work item
constexpr int kMaxPairs = 4096;    // directory entries kept in LDS
constexpr int kMaxGrid = 2048;

// workspace: [0,64) header {valid, n_pairs, total_items}; [64, 64 + 4*(P+1)) item
// prefix per pair; partials from ws_part_offset: [item][row][D + 4] floats
// (o[0..D), m, l, 0, 0).
__host__ __device__ inline int64_t ws_part_offset(int64_t pairs) {
  return (64 + 4 * (pairs + 1) + 255) / 256 * 256;
}

struct DecArgs {
  const uint8_t* cache;
  const uint16_t* q;
  float* ws;
  float* out;
  int64_t cache_bytes;
  int64_t ctx_len;
  int64_t max_items;
  int batch, hq, hkv;
  float c;  // sm_scale * log2(e)
};

struct Geo {
  int64_t rec8, rec4, data_offset, total;
  int cur;
};

// Validates the global header against the launch; returns false on mismatch.
template <int D, int BLK>
__device__ __forceinline__ bool header_ok(const DecArgs& a, Geo& geo) {
  const int32_t* hd = reinterpret_cast<const int32_t*>(a.cache);
  const int64_t* h64 = reinterpret_cast<const int64_t*>(a.cache);
  geo.rec8 = 2LL * BLK * D + 8LL * BLK;
  geo.rec4 = (int64_t)BLK * D + 8LL * BLK;
  geo.cur = (int)((a.ctx_len - 1) / BLK);
  geo.data_offset = (64 + 64LL * a.batch * a.hkv + 255) / 256 * 256;
  geo.total = h64[5];
  return hd[0] == 0x43564B54 && hd[1] == 1 && hd[2] == a.batch && hd[3] == a.hkv && hd[4] == D &&
         hd[5] == BLK && hd[6] == geo.cur + 1 && hd[7] == geo.cur && h64[4] == a.ctx_len &&
         geo.total <= a.cache_bytes && h64[6] == 64 && h64[7] == geo.data_offset;
}

struct Entry {
  int64_t off;
  int n8, n4, lo8, sink, lo4;
};

__device__ __forceinline__ Entry read_entry(const uint8_t* cache, int pair) {
  const int32_t* e = reinterpret_cast<const int32_t*>(cache + 64 + 64 * (int64_t)pair);
  Entry r;
  r.off = *reinterpret_cast<const int64_t*>(e);
  r.n8 = e[2];
  r.n4 = e[3];
  r.lo8 = e[6];
  r.sink = e[7];
  r.lo4 = e[8];
  return r;
}

template <int D, int BLK>
__device__ __forceinline__ bool entry_ok(const Entry& e, const Geo& geo) {
  return e.n8 >= 1 && e.n4 >= 0 && e.n8 + e.n4 <= geo.cur + 1 && e.off >= geo.data_offset &&
         e.off + (int64_t)e.n8 * geo.rec8 + (int64_t)e.n4 * geo.rec4 <= geo.total && e.lo8 >= 0 &&
         e.lo8 <= geo.cur && (e.sink == 0 || e.sink == 1) && e.lo4 >= 0 && e.lo4 + e.n4 <= geo.cur + 1;
}

template <int BLK>
__device__ __forceinline__ int items_of(const Entry& e) {
  const int groups = (e.n8 + e.n4) * (BLK / 64);
  return (groups + kGroupsPerItem - 1) / kGroupsPerItem;
}

// 8 signed bytes -> 8 bf16 (exact: |value| <= 127)
__device__ __forceinline__ v8bf i8x8_to_bf16(uint32_t w0, uint32_t w1) {
  v8bf r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r[i] = (__bf16)(float)(int)(int8_t)(w0 >> (8 * i));
    r[4 + i] = (__bf16)(float)(int)(int8_t)(w1 >> (8 * i));
  }
  return r;
}

// 8 packed nibbles (one dword, low nibble first) -> 8 int8 holding 16*code, in
// position order.
__device__ __forceinline__ v2i nib8_ordered_x16(uint32_t w) {
  const uint32_t e = nib_even_x16(w), o = nib_odd_x16(w);
  v2i r;
  r[0] = (int)__builtin_amdgcn_perm(o, e, 0x05010400u);
  r[1] = (int)__builtin_amdgcn_perm(o, e, 0x07030602u);
  return r;
}

template <int D, int BLK, int RG>
__global__ void __launch_bounds__(kThreads) decode_split_kernel(DecArgs a) {
  constexpr int KS = D / 64, ND = D / 16;
  constexpr int ROWS = 16 * RG;
  __shared__ int pfx[kMaxPairs + 1];
  __shared__ __attribute__((aligned(16))) float mrg[ROWS][D + 4];
  __shared__ int bad;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, kq = lane >> 4;
  const int G = a.hq / a.hkv;
  const int P = a.batch * a.hkv;
  Geo geo;
  if (!header_ok<D, BLK>(a, geo)) {
    if (blockIdx.x == 0 && tid == 0) reinterpret_cast<int*>(a.ws)[0] = 0;
    return;
  }
  // ---- item prefix over the directory (validated), computed by wave 0
  if (tid == 0) bad = 0;
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    for (int base = 0; base < P; base += 64) {
      const int p = base + lane;
      int cnt = 0;
      if (p < P) {
        const Entry e = read_entry(a.cache, p);
        if (!entry_ok<D, BLK>(e, geo)) bad = 1;
        else cnt = items_of<BLK>(e);
      }
      int incl = cnt;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      if (p < P) pfx[p + 1] = carry + incl;
      carry += __shfl(incl, 63);
    }
    if (lane == 0) pfx[0] = 0;
  }
  __syncthreads();
  const int total = pfx[P];
  if (bad || total > a.max_items) {
    if (blockIdx.x == 0 && tid == 0) reinterpret_cast<int*>(a.ws)[0] = 0;
    return;
  }
  if (blockIdx.x == 0 && tid == 0) {
    int* wsh = reinterpret_cast<int*>(a.ws);
    wsh[0] = 1;
    wsh[1] = P;
    wsh[2] = total;
  }
  if (blockIdx.x == 0)
    for (int p = tid; p <= P; p += kThreads) reinterpret_cast<int*>(a.ws)[16 + p] = pfx[p];
  float* part = a.ws + ws_part_offset(P) / 4;

  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    // pair of this item: largest p with pfx[p] <= item
    int lo = 0, hi = P - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pfx[mid] <= item) lo = mid;
      else hi = mid - 1;
    }
    const int pair = lo;
    const int ii = item - pfx[pair];
    const Entry e = read_entry(a.cache, pair);
    const int groups = (e.n8 + e.n4) * (BLK / 64);
    const int g_begin = ii * kGroupsPerItem;
    const int g_end = min(groups, g_begin + kGroupsPerItem);
    const int b = pair / a.hkv, gkv = pair % a.hkv;

    // ---- quantise this pair's G query rows (int8 + int4 codes as MFMA B operands)
    v4i q8op[RG][KS], q4op[RG][KS];
    float a8[RG], a4[RG];
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
          uint4 raw = make_uint4(0, 0, 0, 0);
          if (valid)
            raw = *reinterpret_cast<const uint4*>(a.q + ((int64_t)b * a.hq + gkv * G + row) * D + ks * 64 +
                                                  kq * 16 + hh * 8);
          bf16x8_to_f32(raw, x[ks][hh]);
#pragma unroll
          for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[ks][hh][i]));
        }
      amax = fmaxf(amax, __shfl_xor(amax, 16));
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      float s8 = 0.f, s4 = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint32_t c8a[2], c8b[2], c4a, c4b;
        codes_from_amax(x[ks][0], amax, c8a, c4a, s8, s4);
        codes_from_amax(x[ks][1], amax, c8b, c4b, s8, s4);
        q8op[rg][ks] = v4i{(int)c8a[0], (int)c8a[1], (int)c8b[0], (int)c8b[1]};
        q4op[rg][ks] = unpack16_x16(c4a, c4b);
      }
      a8[rg] = fmaxf(s8 * a.c, FLT_MIN);
      a4[rg] = fmaxf(s4 * a.c * (1.0f / 256.0f), FLT_MIN);
    }

    float m[RG], l[RG];
    v4f O[RG][ND];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      m[rg] = -INFINITY;
      l[rg] = 0.0f;
#pragma unroll
      for (int d = 0; d < ND; ++d) O[rg][d] = v4f{0.f, 0.f, 0.f, 0.f};
    }

    for (int gi = g_begin + wave; gi < g_end; gi += kWaves) {
      const int jblk = gi / (BLK / 64), sub = gi % (BLK / 64);
      const bool is4 = jblk >= e.n8;
      const int kb = !is4 ? ((e.sink && jblk == 0) ? 0 : e.lo8 + jblk - e.sink) : e.lo4 + (jblk - e.n8);
      const uint8_t* rec = a.cache + e.off +
                           (!is4 ? (int64_t)jblk * geo.rec8
                                 : (int64_t)e.n8 * geo.rec8 + (int64_t)(jblk - e.n8) * geo.rec4);
      const int kbytes = is4 ? BLK * D / 2 : BLK * D;
      const float* sk = reinterpret_cast<const float*>(rec + 2 * kbytes) + sub * 64;
      const float* sv = sk + BLK;

      // ---- loads: K codes (A operands), V^T codes, key and value scales
      v4i kop[4][KS];
      uint4 vraw[ND];
      float4 skv[4], svv[4];
      if (!is4) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            kop[s][ks] = *reinterpret_cast<const v4i*>(rec + (int64_t)(sub * 64 + 16 * s + lr) * D + ks * 64 + kq * 16);
#pragma unroll
        for (int d = 0; d < ND; ++d)
          vraw[d] = *reinterpret_cast<const uint4*>(rec + kbytes + (int64_t)(d * 16 + lr) * BLK + sub * 64 + 16 * kq);
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const uint2 p = *reinterpret_cast<const uint2*>(rec + (int64_t)(sub * 64 + 16 * s + lr) * (D / 2) + ks * 32 + kq * 8);
            kop[s][ks] = unpack16_x16(p.x, p.y);
          }
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const uint2 p = *reinterpret_cast<const uint2*>(rec + kbytes + (int64_t)(d * 16 + lr) * (BLK / 2) + (sub * 64 + 16 * kq) / 2);
          const v2i lo = nib8_ordered_x16(p.x), hi = nib8_ordered_x16(p.y);
          vraw[d] = make_uint4((uint32_t)lo[0], (uint32_t)lo[1], (uint32_t)hi[0], (uint32_t)hi[1]);
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        skv[s] = *reinterpret_cast<const float4*>(sk + 16 * s + 4 * kq);
        svv[s] = *reinterpret_cast<const float4*>(sv + 16 * s + 4 * kq);
      }

      // ---- scores (S^T: lane = query row, 4 keys per 16-key subtile)
      float t[RG][4][4];
      float mt[RG];
      const int64_t tok0 = (int64_t)kb * BLK + sub * 64;
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        mt[rg] = -INFINITY;
        const float ar = is4 ? a4[rg] : a8[rg];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          v4i S = {0, 0, 0, 0};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            S = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop[s][ks], is4 ? q4op[rg][ks] : q8op[rg][ks], S, 0, 0, 0);
          const float kv[4] = {skv[s].x, skv[s].y, skv[s].z, skv[s].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x = (float)S[i] * kv[i] * ar;
            if (tok0 + 16 * s + 4 * kq + i >= a.ctx_len) x = -INFINITY;
            t[rg][s][i] = x;
            mt[rg] = fmaxf(mt[rg], x);
          }
        }
        mt[rg] = fmaxf(mt[rg], __shfl_xor(mt[rg], 16));
        mt[rg] = fmaxf(mt[rg], __shfl_xor(mt[rg], 32));
      }
      bool need = false;
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) need = need || (mt[rg] > m[rg]);
      if (__ballot(need)) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          const float mn = fmaxf(m[rg], mt[rg]);
          const float f = exp2f(m[rg] - mn);
          m[rg] = mn;
          l[rg] *= f;
#pragma unroll
          for (int d = 0; d < ND; ++d) O[rg][d] *= f;
        }
      }
      // ---- weights: p = 2^(t - m); p' = p * sv split into bf16 hi + lo
      v8bf bhi[RG][2], blo[RG][2];
      const float vscale = is4 ? (1.0f / 16.0f) : 1.0f;
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const float vv[4] = {svv[s].x, svv[s].y, svv[s].z, svv[s].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            // m is -inf only while every key seen so far was masked (then t is too)
            const float p = exp2f(t[rg][s][i] - (m[rg] == -INFINITY ? 0.0f : m[rg]));
            l[rg] += p;
            const float pw = p * vv[i] * vscale;
            const __bf16 h = (__bf16)pw;
            const __bf16 r = (__bf16)(pw - (float)h);
            bhi[rg][s >> 1][4 * (s & 1) + i] = h;
            blo[rg][s >> 1][4 * (s & 1) + i] = r;
          }
        }
      }
      // ---- O^T += V^T . P'^T
#pragma unroll
      for (int d = 0; d < ND; ++d) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const v8bf vop = t2 == 0 ? i8x8_to_bf16(vraw[d].x, vraw[d].y) : i8x8_to_bf16(vraw[d].z, vraw[d].w);
#pragma unroll
          for (int rg = 0; rg < RG; ++rg) {
            O[rg][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, bhi[rg][t2], O[rg][d], 0, 0, 0);
            O[rg][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, blo[rg][t2], O[rg][d], 0, 0, 0);
          }
        }
      }
    }

    // ---- merge the waves' partials in LDS (sequentially: deterministic)
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
      l[rg] += __shfl_xor(l[rg], 16);
      l[rg] += __shfl_xor(l[rg], 32);
    }
    for (int w = 0; w < kWaves; ++w) {
      __syncthreads();
      if (wave == w) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          const int row = rg * 16 + lr;
          float* dst = &mrg[row][0];
          if (w == 0) {
#pragma unroll
            for (int d = 0; d < ND; ++d) *reinterpret_cast<float4*>(dst + d * 16 + kq * 4) = make_float4(O[rg][d][0], O[rg][d][1], O[rg][d][2], O[rg][d][3]);
            if (kq == 0) {
              dst[D] = m[rg];
              dst[D + 1] = l[rg];
            }
          } else {
            const float m0 = dst[D], l0 = dst[D + 1];
            const float mn = fmaxf(m0, m[rg]);
            const float f0 = (m0 == -INFINITY) ? 0.0f : exp2f(m0 - mn);
            const float f1 = (m[rg] == -INFINITY) ? 0.0f : exp2f(m[rg] - mn);
#pragma unroll
            for (int d = 0; d < ND; ++d) {
              float4 o = *reinterpret_cast<float4*>(dst + d * 16 + kq * 4);
              o.x = o.x * f0 + O[rg][d][0] * f1;
              o.y = o.y * f0 + O[rg][d][1] * f1;
              o.z = o.z * f0 + O[rg][d][2] * f1;
              o.w = o.w * f0 + O[rg][d][3] * f1;
              *reinterpret_cast<float4*>(dst + d * 16 + kq * 4) = o;
            }
            // all four lanes of the row have read m0/l0 before lane kq==0 writes
            __builtin_amdgcn_wave_barrier();
            if (kq == 0) {
              dst[D] = mn;
              dst[D + 1] = l0 * f0 + l[rg] * f1;
            }
          }
        }
      }
    }
    __syncthreads();
    // ---- write the item's partials for the G valid rows
    float* dstp = part + (int64_t)item * G * (D + 4);
    for (int i = tid; i < G * (D + 4); i += kThreads) {
      const int row = i / (D + 4), col = i % (D + 4);
      dstp[i] = col < D + 2 ? mrg[row][col] : 0.0f;
    }
    __syncthreads();  // mrg is reused by the next item
  }
}

// Merge of the items of each pair: one work group per (batch, query head).
template <int D>
__global__ void __launch_bounds__(D) decode_merge_kernel(DecArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.hq, h = bh % a.hq;
  const int G = a.hq / a.hkv;
  const int pair = b * a.hkv + h / G, row = h % G;
  const int* wsh = reinterpret_cast<const int*>(a.ws);
  float* dst = a.out + (int64_t)bh * D;
  if (wsh[0] != 1 || wsh[1] != a.batch * a.hkv) {
    dst[threadIdx.x] = __int_as_float(0x7FC00000);  // NaN: the cache did not validate
    return;
  }
  const int P = wsh[1];
  const int i0 = wsh[16 + pair], i1 = wsh[16 + pair + 1];
  const float* part = a.ws + ws_part_offset(P) / 4;
  float mx = -INFINITY;
  for (int it = i0; it < i1; ++it) mx = fmaxf(mx, part[((int64_t)it * G + row) * (D + 4) + D]);
  float l = 0.0f, o = 0.0f;
  for (int it = i0; it < i1; ++it) {
    const float* p = part + ((int64_t)it * G + row) * (D + 4);
    const float f = p[D] == -INFINITY ? 0.0f : exp2f(p[D] - mx);
    l += p[D + 1] * f;
    o += p[threadIdx.x] * f;
  }
  dst[threadIdx.x] = o / l;
}

template <int D, int BLK, int RG>
hipError_t launch_t(const DecArgs& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<D, BLK, RG>), dim3(grid), dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3(a.batch * a.hq), dim3(D), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int64_t decode_max_items(const Shape& s, int64_t ctx_len) {
  const int64_t nb = (ctx_len - 1) / s.blk + 1;
  const int64_t groups = nb * (s.blk / 64);
  return (int64_t)s.batch * s.hkv * ((groups + kGroupsPerItem - 1) / kGroupsPerItem);
}

int64_t decode_workspace_bytes(const Shape& s, int64_t ctx_len) {
  const int64_t pairs = (int64_t)s.batch * s.hkv;
  const int G = s.hq / s.hkv;
  return ws_part_offset(pairs) + decode_max_items(s, ctx_len) * G * (s.d + 4) * 4;
}

hipError_t launch_decode(const Shape& s, int64_t ctx_len, const void* cache, int64_t cache_bytes,
                         const void* q, float sm_scale, float* out, void* workspace, hipStream_t stream) {
  DecArgs a;
  a.cache = static_cast<const uint8_t*>(cache);
  a.q = static_cast<const uint16_t*>(q);
  a.ws = static_cast<float*>(workspace);
  a.out = out;
  a.cache_bytes = cache_bytes;
  a.ctx_len = ctx_len;
  a.max_items = decode_max_items(s, ctx_len);
  a.batch = s.batch;
  a.hq = s.hq;
  a.hkv = s.hkv;
  a.c = sm_scale * 1.44269504088896340736f;
  const int grid = (int)(a.max_items < kMaxGrid ? a.max_items : kMaxGrid);
  const int G = s.hq / s.hkv;
  const bool two = G > 16;
  if (s.d == 128 && s.blk == 128) return two ? launch_t<128, 128, 2>(a, grid, stream) : launch_t<128, 128, 1>(a, grid, stream);
  if (s.d == 128 && s.blk == 64) return two ? launch_t<128, 64, 2>(a, grid, stream) : launch_t<128, 64, 1>(a, grid, stream);
  if (s.d == 64 && s.blk == 128) return two ? launch_t<64, 128, 2>(a, grid, stream) : launch_t<64, 128, 1>(a, grid, stream);
  return two ? launch_t<64, 64, 2>(a, grid, stream) : launch_t<64, 64, 1>(a, grid, stream);
}

}  // namespace tria
