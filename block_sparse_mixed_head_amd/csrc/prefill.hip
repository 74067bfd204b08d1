// prefill.hip - fused block-sparse, mixed-precision causal attention (prompt stage).
//
// What it computes (TriAttention summary page, rit.work, section on which links can
// be skipped: per-tile skip / 4-bit / 8-bit by distance from the diagonal, block 0
// and the diagonal protected at 8 bits; section on calibration: one fused kernel
// groups the kept blocks by precision and reduces them into one normalised result):
//   t_ij = S_ij * sq_i * sk_j * sm_scale * log2(e),  S_ij = exact integer dot of codes
//   P_ij = bf16(2^(t_ij - M_i)),  M_i an integer >= max_j t_ij
//   out_i = sum_j P_ij V_j / sum_j P_ij
// over the keys of the unit's sink block, int4 range and int8 range.  Skipped tiles
// are never loaded.
//
// gfx950 design.  One work group per (b, h, q-block) unit, BLK/32 waves, each wave
// owns 32 query rows as two 16-row MFMA groups.
//   * Scores are computed transposed, S^T = K . Q^T, with v_mfma_i32_16x16x64_i8:
//     K (A operand) comes from LDS, the Q codes (B operand) stay in registers for
//     the whole unit.  The 16x16 accumulator layout then gives every lane one query
//     row and four keys per 16-key subtile, so row maxima and sums are mostly
//     in-lane (two cross-lane steps).
//   * int4 tiles: both K (once per tile, cooperatively, into LDS) and Q (once per
//     unit, in registers) are widened to int8 as 16*code; gfx950 has no int4 MFMA.
//     The factor 256 is folded into the query-row scale.
//   * Softmax in fp32 with an integer running maximum: rescales are exact powers of
//     two, so rounding P to bf16 commutes with them and the result matches a
//     final-maximum evaluation.  Rescaling is skipped when no row's maximum rose.
//   * O^T = V^T . P^T with v_mfma_f32_16x16x32_bf16: the transposed scores are
//     already the B operand layout (P^T), and V (row-major in LDS) is fed as V^T by
//     ds_read_b64_tr_b16, so V needs no transpose pass.
//   * K and V tiles are staged through LDS with 16-byte coalesced loads; both LDS
//     layouts are XOR-swizzled so the MFMA-operand reads avoid bank conflicts.
#include <cfloat>

#include "device_common.h"
#include "kernels.h"

namespace tria {

namespace {

template <int D, int BLK>
struct Cfg {
  static constexpr int WAVES = BLK / 32;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int KS = D / 64;    // k-steps of 64 int8 per QK MFMA
  static constexpr int KCH = D / 16;   // 16-byte chunks per int8 K row
  static constexpr int VCH = D / 8;    // 16-byte chunks per bf16 V row
  static constexpr int VU = D / 16;    // 32-byte units per bf16 V row
  static constexpr int NS = BLK / 16;  // 16-key subtiles
  static constexpr int NT = BLK / 32;  // 32-key P.V k-steps
  static constexpr int ND = D / 16;    // 16-wide output column groups
  static constexpr int K_BYTES = BLK * D;
  static constexpr int V_BYTES = BLK * D * 2;
  static constexpr int LDS_BYTES = K_BYTES + V_BYTES + BLK * 4;
};

struct Args {
  const int32_t* units;
  const int8_t* q8;
  const uint8_t* q4;
  const float* q8s;
  const float* q4s;
  const int8_t* k8;
  const uint8_t* k4;
  const float* k8s;
  const float* k4s;
  const uint16_t* v;
  float* out;
  float* lse;
  int64_t n;
  int batch, hq, hkv;
  float c;  // sm_scale * log2(e)
};

// byte offset of 16-byte chunk c of K row r in LDS
template <int KCH>
__device__ __forceinline__ int k_off(int r, int c, int D) {
  return r * D + ((c ^ (r & (KCH - 1))) << 4);
}
// byte offset of byte b of V row r in LDS (32-byte units swizzled)
template <int VU>
__device__ __forceinline__ int v_off(int r, int b, int D) {
  return r * 2 * D + ((((b >> 5) ^ (r & (VU - 1)))) << 5) + (b & 31);
}

template <int D, int BLK>
__global__ void __launch_bounds__((Cfg<D, BLK>::THREADS)) prefill_kernel(Args a) {
  using C = Cfg<D, BLK>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS_BYTES];
  uint8_t* k_lds = smem;
  uint8_t* v_lds = smem + C::K_BYTES;
  float* s_lds = reinterpret_cast<float*>(smem + C::K_BYTES + C::V_BYTES);

  const int32_t* u = a.units + 8 * (int64_t)blockIdx.x;
  const int b = u[0], h = u[1], qb = u[2], lo8 = u[3], lo4 = u[4], hi4 = u[5], sink = u[6];
  const int n4 = hi4 - lo4 + 1;
  const int ntiles = u[7];
  {  // a malformed record is skipped rather than allowed to address out of range
    const int64_t nbq = (a.n + BLK - 1) / BLK;
    const bool bad = b < 0 || b >= a.batch || h < 0 || h >= a.hq || qb < 0 || qb >= nbq || lo8 < 0 ||
                     lo8 > qb || sink < 0 || sink > 1 || (sink == 1 && lo8 == 0) || n4 < 0 ||
                     (n4 > 0 && (lo4 < 1 || hi4 >= lo8)) || ntiles != (qb - lo8 + 1) + sink + n4;
    if (bad) return;
  }
  const int g_kv = h / (a.hq / a.hkv);
  const int64_t n = a.n;
  const int64_t qrow0 = ((int64_t)b * a.hq + h) * n;
  const int64_t krow0 = ((int64_t)b * a.hkv + g_kv) * n;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, kq = lane >> 4;

  // ---- per-unit query state: codes as MFMA B operands, scales, softmax state
  v4i q8op[2][C::KS], q4op[2][C::KS];
  float a8[2], a4[2], M[2], lsum[2];
  int rowq[2];  // row index inside the q-block
  v4f O[2][C::ND];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    rowq[g] = wave * 32 + g * 16 + lr;
    const int64_t qi = (int64_t)qb * BLK + rowq[g];
    const bool valid = qi < n;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      v4i z = {0, 0, 0, 0};
      q8op[g][ks] = z;
      q4op[g][ks] = z;
      if (valid) {
        q8op[g][ks] = *reinterpret_cast<const v4i*>(a.q8 + (qrow0 + qi) * D + ks * 64 + kq * 16);
        const uint2 p = *reinterpret_cast<const uint2*>(a.q4 + (qrow0 + qi) * (D / 2) + ks * 32 + kq * 8);
        q4op[g][ks] = unpack16_x16(p.x, p.y);
      }
    }
    const float sq8 = valid ? a.q8s[qrow0 + qi] : 0.0f;
    const float sq4 = valid ? a.q4s[qrow0 + qi] : 0.0f;
    // a row of zeros has scale 0; a tiny positive factor keeps -inf * a = -inf
    a8[g] = fmaxf(sq8 * a.c, FLT_MIN);
    a4[g] = fmaxf(sq4 * a.c * (1.0f / 256.0f), FLT_MIN);
    M[g] = -INFINITY;
    lsum[g] = 0.0f;
#pragma unroll
    for (int d = 0; d < C::ND; ++d) O[g][d] = v4f{0.f, 0.f, 0.f, 0.f};
  }

  for (int it = 0; it < ntiles; ++it) {
    int kb;
    bool is4;
    if (it < sink) {
      kb = 0;
      is4 = false;
    } else if (it < sink + n4) {
      kb = lo4 + (it - sink);
      is4 = true;
    } else {
      kb = lo8 + (it - sink - n4);
      is4 = false;
    }
    const bool diag = (kb == qb);
    const int64_t key0 = (int64_t)kb * BLK;

    __syncthreads();  // previous tile's LDS reads are done
    // ---- stage K (int8, or int4 widened to int8 x16), V (bf16) and key scales.
    // All global loads are issued before the LDS stores.
    constexpr int KIT = BLK * C::KCH / C::THREADS;   // 16-byte K chunks per thread
    constexpr int VIT = BLK * C::VCH / C::THREADS;   // 16-byte V chunks per thread
    uint4 kv[KIT], vv[VIT];
    if (!is4) {
#pragma unroll
      for (int j = 0; j < KIT; ++j) {
        const int i = tid + j * C::THREADS, r = i / C::KCH, c = i % C::KCH;
        kv[j] = make_uint4(0, 0, 0, 0);
        if (key0 + r < n) kv[j] = *reinterpret_cast<const uint4*>(a.k8 + (krow0 + key0 + r) * D + c * 16);
      }
    } else {
#pragma unroll
      for (int j = 0; j < KIT / 2; ++j) {
        const int i = tid + j * C::THREADS, r = i / (C::KCH / 2), c2 = i % (C::KCH / 2);
        kv[j] = make_uint4(0, 0, 0, 0);
        if (key0 + r < n) kv[j] = *reinterpret_cast<const uint4*>(a.k4 + (krow0 + key0 + r) * (D / 2) + c2 * 16);
      }
    }
#pragma unroll
    for (int j = 0; j < VIT; ++j) {
      const int i = tid + j * C::THREADS, r = i / C::VCH, c = i % C::VCH;
      vv[j] = make_uint4(0, 0, 0, 0);
      if (key0 + r < n) vv[j] = *reinterpret_cast<const uint4*>(a.v + (krow0 + key0 + r) * D + c * 8);
    }
    float sc = 0.0f;
    if (tid < BLK && key0 + tid < n) sc = (is4 ? a.k4s : a.k8s)[krow0 + key0 + tid];
    if (!is4) {
#pragma unroll
      for (int j = 0; j < KIT; ++j) {
        const int i = tid + j * C::THREADS, r = i / C::KCH, c = i % C::KCH;
        *reinterpret_cast<uint4*>(k_lds + k_off<C::KCH>(r, c, D)) = kv[j];
      }
    } else {
#pragma unroll
      for (int j = 0; j < KIT / 2; ++j) {
        const int i = tid + j * C::THREADS, r = i / (C::KCH / 2), c2 = i % (C::KCH / 2);
        *reinterpret_cast<v4i*>(k_lds + k_off<C::KCH>(r, 2 * c2, D)) = unpack16_x16(kv[j].x, kv[j].y);
        *reinterpret_cast<v4i*>(k_lds + k_off<C::KCH>(r, 2 * c2 + 1, D)) = unpack16_x16(kv[j].z, kv[j].w);
      }
    }
#pragma unroll
    for (int j = 0; j < VIT; ++j) {
      const int i = tid + j * C::THREADS, r = i / C::VCH, c = i % C::VCH;
      *reinterpret_cast<uint4*>(v_lds + v_off<C::VU>(r, c * 16, D)) = vv[j];
    }
    if (tid < BLK) s_lds[tid] = sc;
    __syncthreads();

    // ---- S^T = K . Q^T (int8 MFMA, exact int32)
    v4i S[2][C::NS];
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      S[0][s] = v4i{0, 0, 0, 0};
      S[1][s] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int r = s * 16 + lr;
        const v4i kop = *reinterpret_cast<const v4i*>(k_lds + k_off<C::KCH>(r, ks * 4 + kq, D));
        const v4i b0 = is4 ? q4op[0][ks] : q8op[0][ks];
        const v4i b1 = is4 ? q4op[1][ks] : q8op[1][ks];
        S[0][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop, b0, S[0][s], 0, 0, 0);
        S[1][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop, b1, S[1][s], 0, 0, 0);
      }
    }

    // ---- softmax: u = S * sk (per key), row max, integer running max, P = 2^(u*a - M)
    float u[2][C::NS][4];
    float mx[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int s = 0; s < C::NS; ++s) {
      const float4 ksc = *reinterpret_cast<const float4*>(s_lds + s * 16 + kq * 4);
      const float kv[4] = {ksc.x, ksc.y, ksc.z, ksc.w};
#pragma unroll
      for (int g = 0; g < 2; ++g) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = (float)S[g][s][i] * kv[i];
          if (diag && (s * 16 + kq * 4 + i > rowq[g])) x = -INFINITY;
          u[g][s][i] = x;
          mx[g] = fmaxf(mx[g], x);
        }
      }
    }
    bool need = false;
    float Mc[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      mx[g] = fmaxf(mx[g], __shfl_xor(mx[g], 16));
      mx[g] = fmaxf(mx[g], __shfl_xor(mx[g], 32));
      const float ag = is4 ? a4[g] : a8[g];
      Mc[g] = ceilf(mx[g] * ag);
      need = need || (Mc[g] > M[g]);
    }
    if (__ballot(need)) {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const float Mn = fmaxf(M[g], Mc[g]);
        const float f = exp2f(M[g] - Mn);  // exact power of two (0 on the first tile)
        M[g] = Mn;
        lsum[g] *= f;
#pragma unroll
        for (int d = 0; d < C::ND; ++d) O[g][d] *= f;
      }
    }
    v8bf pb[2][C::NT];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float ag = is4 ? a4[g] : a8[g];
      const float nM = -M[g];
      const v2bf one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int t = 0; t < C::NT; ++t) {
        v2bf x[4];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int s = 2 * t + half;
          const v2f p01 = {__builtin_amdgcn_exp2f(fmaf(u[g][s][0], ag, nM)),
                           __builtin_amdgcn_exp2f(fmaf(u[g][s][1], ag, nM))};
          const v2f p23 = {__builtin_amdgcn_exp2f(fmaf(u[g][s][2], ag, nM)),
                           __builtin_amdgcn_exp2f(fmaf(u[g][s][3], ag, nM))};
          x[2 * half] = __builtin_convertvector(p01, v2bf);
          x[2 * half + 1] = __builtin_convertvector(p23, v2bf);
          lsum[g] = __builtin_amdgcn_fdot2_f32_bf16(x[2 * half], one, lsum[g], false);
          lsum[g] = __builtin_amdgcn_fdot2_f32_bf16(x[2 * half + 1], one, lsum[g], false);
        }
        // keys 16*(2t) + 4kq + 0..3, then 16*(2t+1) + 4kq + 0..3 (the B operand's k order)
        pb[g][t] = __builtin_shufflevector(__builtin_shufflevector(x[0], x[1], 0, 1, 2, 3),
                                           __builtin_shufflevector(x[2], x[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }

    // ---- O^T += V^T . P^T (bf16 MFMA); V^T operand via transposing LDS reads
#pragma unroll
    for (int t = 0; t < C::NT; ++t) {
      const int r0 = 32 * t + kq * 4 + (lr >> 2);
      const int r1 = r0 + 16;
#pragma unroll
      for (int d = 0; d < C::ND; ++d) {
        const int bcol = d * 32 + (lr & 3) * 8;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4s*)((__attribute__((address_space(3))) uint8_t*)(v_lds) + v_off<C::VU>(r0, bcol, D)));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4s*)((__attribute__((address_space(3))) uint8_t*)(v_lds) + v_off<C::VU>(r1, bcol, D)));
        // whole-vector concatenation (element-wise inserts of the halves have been
        // folded incorrectly by the compiler)
        const v8bf vop = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        O[0][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pb[0][t], O[0][d], 0, 0, 0);
        O[1][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pb[1][t], O[1][d], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: normalise and store (fp32), optional base-2 LSE
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    float l = lsum[g];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int64_t qi = (int64_t)qb * BLK + rowq[g];
    if (qi < n) {
      const float inv = 1.0f / l;
      float* dst = a.out + (qrow0 + qi) * D + kq * 4;
#pragma unroll
      for (int d = 0; d < C::ND; ++d) {
        const v4f o = O[g][d] * inv;
        *reinterpret_cast<float4*>(dst + d * 16) = make_float4(o[0], o[1], o[2], o[3]);
      }
      if (a.lse && kq == 0) a.lse[qrow0 + qi] = M[g] + __log2f(l);
    }
  }
}

template <int D, int BLK>
hipError_t launch_t(const Args& a, int64_t n_units, hipStream_t stream) {
  using C = Cfg<D, BLK>;
  hipLaunchKernelGGL((prefill_kernel<D, BLK>), dim3((unsigned)n_units), dim3(C::THREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const Shape& s, const int32_t* units, int64_t n_units, const int8_t* q8,
                          const uint8_t* q4, const float* q8s, const float* q4s, const int8_t* k8,
                          const uint8_t* k4, const float* k8s, const float* k4s, const void* v,
                          float sm_scale, float* out, float* lse, hipStream_t stream) {
  Args a;
  a.units = units;
  a.q8 = q8;
  a.q4 = q4;
  a.q8s = q8s;
  a.q4s = q4s;
  a.k8 = k8;
  a.k4 = k4;
  a.k8s = k8s;
  a.k4s = k4s;
  a.v = static_cast<const uint16_t*>(v);
  a.out = out;
  a.lse = lse;
  a.n = s.n;
  a.batch = s.batch;
  a.hq = s.hq;
  a.hkv = s.hkv;
  a.c = sm_scale * 1.44269504088896340736f;
  if (n_units == 0) return hipSuccess;
  if (s.d == 128 && s.blk == 128) return launch_t<128, 128>(a, n_units, stream);
  if (s.d == 128 && s.blk == 64) return launch_t<128, 64>(a, n_units, stream);
  if (s.d == 64 && s.blk == 128) return launch_t<64, 128>(a, n_units, stream);
  return launch_t<64, 64>(a, n_units, stream);
}

}  // namespace tria
