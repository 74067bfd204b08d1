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
// gfx950 design.  One work group per (b, h, q-block) unit, BLK/32 wavefronts, each
// owning 32 query rows as two 16-row MFMA groups; the unit's kept key blocks are
// streamed in 64-key stages.
//   * K, V and key scales of a stage go straight from HBM into LDS with
//     global_load_lds_dwordx4 (no staging registers), double-buffered: the next
//     stage's loads are in flight while the current one is computed, one barrier
//     per stage.  Each 1 KB load instruction fills a contiguous LDS range; the XOR
//     swizzles of the LDS layouts are realised by the per-lane global addresses.
//   * Scores are computed transposed, S^T = K . Q^T, with v_mfma_i32_16x16x64_i8:
//     K (A operand) from LDS, the Q codes (B operand) in registers for the whole
//     unit.  The 16x16 accumulator layout gives every lane one query row and four
//     keys per 16-key subtile, so row maxima and sums are in-lane plus two
//     cross-lane steps.
//   * int4 stages: packed K nibbles are read from LDS and widened to int8 as
//     16*code in registers (Q's int4 codes likewise, once per unit); gfx950 has no
//     int4 MFMA.  The factor 256 is folded into the query-row scale.
//   * fp32 softmax with an integer running maximum: rescales are exact powers of
//     two, so rounding P to bf16 commutes with them and the result equals a
//     final-maximum evaluation.  Rescaling is skipped unless some row's max rose.
//     Only the diagonal block's stages carry the causal mask.
//   * O^T = V^T . P^T with v_mfma_f32_16x16x32_bf16: the transposed scores are
//     already the B operand layout, and V (row-major in LDS) is fed as V^T by
//     ds_read_b64_tr_b16, so V needs no transpose pass.
//   * Registers are held to 256 per lane so two work groups share a CU: one
//     group's softmax (VALU) runs while the other's MFMAs and loads proceed.
#include <cfloat>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace tria {

namespace {

template <int D, int BLK>
struct Cfg {
  static constexpr int WAVES = BLK / 32;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int SK = 64;         // keys per stage
  static constexpr int SPT = BLK / SK;  // stages per key block
  static constexpr int KS = D / 64;     // k-steps of 64 int8 per QK MFMA
  static constexpr int KCH = D / 16;    // 16-byte chunks per int8 K row
  static constexpr int K4CH = D / 32;   // 16-byte chunks per packed int4 K row
  static constexpr int VCH = D / 8;     // 16-byte chunks per bf16 V row
  static constexpr int VU = D / 16;     // 32-byte units per bf16 V row
  static constexpr int ND = D / 16;     // 16-wide output column groups
  static constexpr int K_BYTES = SK * D;
  static constexpr int V_BYTES = SK * D * 2;
  static constexpr int STAGE = K_BYTES + V_BYTES + SK * 4;
  static constexpr int Q4_STRIDE = D + 16;       // widened int4 query codes: padded rows
  static constexpr int Q4_BYTES = BLK * Q4_STRIDE;
  static constexpr int LDS_BYTES = 2 * STAGE + Q4_BYTES;  // two stage buffers + query codes
  static constexpr int K8_INSTR = K_BYTES / 1024;   // 1 KB load instructions per stage
  static constexpr int K4_INSTR = K_BYTES / 2048;
  static constexpr int V_INSTR = V_BYTES / 1024;
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

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ void lds_dma16(const void* gsrc, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void* gsrc, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void*)lds_base, 4, 0, 0);
}

// Per-lane byte offsets of the stage loads, relative to the stage's first key row
// (computed once per work group).  Instruction i of a kind fills LDS bytes
// [1024 i, 1024 i + 1024) of its region; lane l supplies the global address of
// the 16 bytes that land at 1024 i + 16 l, which realises the XOR swizzles.
template <int D, int BLK>
struct LoadPlan {
  using C = Cfg<D, BLK>;
  static constexpr int K8N = (C::K8_INSTR + C::WAVES - 1) / C::WAVES;
  static constexpr int K4N = (C::K4_INSTR + C::WAVES - 1) / C::WAVES;
  static constexpr int VN = (C::V_INSTR + C::WAVES - 1) / C::WAVES;
  uint32_t k8[K8N], k4[K4N], v[VN];

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int j = 0; j < K8N; ++j) {
      const int p = (wave + j * C::WAVES) * 64 + lane, r = p / C::KCH, pc = p % C::KCH;
      k8[j] = r * D + ((pc ^ (r & (C::KCH - 1))) << 4);
    }
#pragma unroll
    for (int j = 0; j < K4N; ++j) {
      const int p = (wave + j * C::WAVES) * 64 + lane, r = p / C::K4CH, pc = p % C::K4CH;
      k4[j] = r * (D / 2) + ((pc ^ (r & (C::K4CH - 1))) << 4);
    }
#pragma unroll
    for (int j = 0; j < VN; ++j) {
      const int p = (wave + j * C::WAVES) * 64 + lane, r = p / C::VCH, pc = p % C::VCH;
      v[j] = r * 2 * D + ((2 * ((pc >> 1) ^ (r & (C::VU - 1))) + (pc & 1)) << 4);
    }
  }
};

// A row offset clamped to the last valid row (stages that run past the sequence
// end re-read its last row: finite data that the causal mask discards).
__device__ __forceinline__ uint32_t clamp_row(uint32_t off, uint32_t row_bytes, uint32_t last) {
  const uint32_t r = off / row_bytes;
  return r > last ? off - (r - last) * row_bytes : off;
}

// Issues the loads of one 64-key stage into an LDS buffer.
template <int D, int BLK>
__device__ __forceinline__ void load_stage(const Args& a, const LoadPlan<D, BLK>& lp, uint8_t* buf,
                                           int64_t krow0, int64_t key0, bool is4, int wave, int lane) {
  using C = Cfg<D, BLK>;
  using LP = LoadPlan<D, BLK>;
  const bool tail = key0 + C::SK > a.n;
  const uint32_t last = (uint32_t)(a.n - 1 - key0);  // last valid row relative to key0 (tail only)
  if (!is4) {
    const int8_t* base = a.k8 + (krow0 + key0) * D;
#pragma unroll
    for (int j = 0; j < LP::K8N; ++j) {
      const int i = wave + j * C::WAVES;
      if (i < C::K8_INSTR) lds_dma16(base + (tail ? clamp_row(lp.k8[j], D, last) : lp.k8[j]), buf + i * 1024);
    }
  } else {
    const uint8_t* base = a.k4 + (krow0 + key0) * (D / 2);
#pragma unroll
    for (int j = 0; j < LP::K4N; ++j) {
      const int i = wave + j * C::WAVES;
      if (i < C::K4_INSTR) lds_dma16(base + (tail ? clamp_row(lp.k4[j], D / 2, last) : lp.k4[j]), buf + i * 1024);
    }
  }
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(a.v + (krow0 + key0) * D);
#pragma unroll
  for (int j = 0; j < LP::VN; ++j) {
    const int i = wave + j * C::WAVES;
    if (i < C::V_INSTR) lds_dma16(vbase + (tail ? clamp_row(lp.v[j], 2 * D, last) : lp.v[j]), buf + C::K_BYTES + i * 1024);
  }
  if (wave == C::WAVES - 1) {  // the 64 key scales, one per lane
    const float* sbase = (is4 ? a.k4s : a.k8s) + krow0 + key0;
    const uint32_t r = (tail && (uint32_t)lane > last) ? last : (uint32_t)lane;
    lds_dma4(sbase + r, buf + C::K_BYTES + C::V_BYTES);
  }
}

struct RowState {
  float M, l, a8, a4;
  int row;  // row index inside the q-block
};

// One 64-key stage for one wavefront (32 query rows).  DIAG: the stage lies in the
// diagonal block and keys past a row are masked (key_base = first key of the stage
// relative to the block start).
template <int D, int BLK, bool IS4, bool DIAG, class After>
__device__ __forceinline__ void compute_stage(const uint8_t* buf, int key_base, const float4 (&ksc)[4],
                                              const v4i (&q8op)[2][Cfg<D, BLK>::KS],
                                              const uint8_t* q4lds, RowState (&rs)[2], v4f (&O)[2][Cfg<D, BLK>::ND],
                                              int lr, int kq, After&& after_reads) {
  using C = Cfg<D, BLK>;
  // int4 stages read this wave's query codes (widened to 16*code) from LDS
  v4i q4op[IS4 ? 2 : 1][C::KS];
  if (IS4) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
        q4op[IS4 ? g : 0][ks] = *reinterpret_cast<const v4i*>(q4lds + rs[g].row * C::Q4_STRIDE + ks * 64 + kq * 16);
  }
  const uint8_t* kb = buf;
  const lds_u8* vb = (const lds_u8*)(buf + C::K_BYTES);

  // ---- S^T = K . Q^T
  v4i S[2][4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    S[0][s] = v4i{0, 0, 0, 0};
    S[1][s] = v4i{0, 0, 0, 0};
    const int r = s * 16 + lr;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      v4i kop;
      if (!IS4) {
        const int c = ks * 4 + kq;
        kop = *reinterpret_cast<const v4i*>(kb + r * D + ((c ^ (r & (C::KCH - 1))) << 4));
      } else {
        const int c = 2 * ks + (kq >> 1);
        const uint2 w = *reinterpret_cast<const uint2*>(kb + r * (D / 2) + ((c ^ (r & (C::K4CH - 1))) << 4) + (kq & 1) * 8);
        kop = unpack16_x16(w.x, w.y);
      }
      S[0][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop, IS4 ? q4op[0][ks] : q8op[0][ks], S[0][s], 0, 0, 0);
      S[1][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop, IS4 ? q4op[IS4 ? 1 : 0][ks] : q8op[1][ks], S[1][s], 0, 0, 0);
    }
  }

  __builtin_amdgcn_sched_barrier(0);
  // ---- softmax with the integer running maximum
  float u[2][4][4];
  float mx[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    mx[g] = -INFINITY;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float kv[4] = {ksc[s].x, ksc[s].y, ksc[s].z, ksc[s].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = (float)S[g][s][i] * kv[i];
        if (DIAG && (key_base + s * 16 + kq * 4 + i > rs[g].row)) x = -INFINITY;
        u[g][s][i] = x;
        mx[g] = fmaxf(mx[g], x);
      }
    }
    mx[g] = fmaxf(mx[g], __shfl_xor(mx[g], 16));
    mx[g] = fmaxf(mx[g], __shfl_xor(mx[g], 32));
  }
  // The running maximum M only has to be an integer that keeps 2^(t - M) finite:
  // it is raised (and O, l rescaled by an exact power of two) only when a row's
  // stage maximum exceeds it by more than kSlack, so weights stay below 2^kSlack.
  constexpr float kSlack = 8.0f;
  bool need = false;
  float Mc[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const float ag = IS4 ? rs[g].a4 : rs[g].a8;
    Mc[g] = ceilf(mx[g] * ag);  // -inf when the whole stage is masked for this row
    need = need || (Mc[g] > rs[g].M + kSlack);
  }
  if (__ballot(need)) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float Mn = Mc[g] > rs[g].M + kSlack ? Mc[g] : rs[g].M;
      const float f = exp2f(rs[g].M - Mn);  // exact power of two; 0 on the first stage
      rs[g].M = Mn;
      rs[g].l *= f;
#pragma unroll
      for (int d = 0; d < C::ND; ++d) O[g][d] *= f;
    }
  }
  v8bf pb[2][2];
  const v2bf one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const float ag = IS4 ? rs[g].a4 : rs[g].a8;
    const float nM = -rs[g].M;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      v2bf x[4];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int s = 2 * t + half;
        const v2f p01 = {__builtin_amdgcn_exp2f(fmaf(u[g][s][0], ag, nM)), __builtin_amdgcn_exp2f(fmaf(u[g][s][1], ag, nM))};
        const v2f p23 = {__builtin_amdgcn_exp2f(fmaf(u[g][s][2], ag, nM)), __builtin_amdgcn_exp2f(fmaf(u[g][s][3], ag, nM))};
        x[2 * half] = __builtin_convertvector(p01, v2bf);
        x[2 * half + 1] = __builtin_convertvector(p23, v2bf);
        rs[g].l = __builtin_amdgcn_fdot2_f32_bf16(x[2 * half], one, rs[g].l, false);
        rs[g].l = __builtin_amdgcn_fdot2_f32_bf16(x[2 * half + 1], one, rs[g].l, false);
      }
      // keys 16*(2t) + 4kq + 0..3, then 16*(2t+1) + 4kq + 0..3: the B operand's k order
      pb[g][t] = __builtin_shufflevector(__builtin_shufflevector(x[0], x[1], 0, 1, 2, 3),
                                         __builtin_shufflevector(x[2], x[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
    }
  }

  __builtin_amdgcn_sched_barrier(0);
  // ---- O^T += V^T . P^T
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int r0 = 32 * t + kq * 4 + (lr >> 2);
    const int r1 = r0 + 16;
#pragma unroll
    for (int d = 0; d < C::ND; ++d) {
      const int off0 = r0 * 2 * D + ((d ^ (r0 & (C::VU - 1))) << 5) + (lr & 3) * 8;
      const int off1 = r1 * 2 * D + ((d ^ (r1 & (C::VU - 1))) << 5) + (lr & 3) * 8;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vb + off0));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vb + off1));
      // whole-vector concatenation (element-wise inserts of the halves have been
      // folded incorrectly by the compiler)
      const v8bf vop = __builtin_bit_cast(v8bf, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      O[0][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pb[0][t], O[0][d], 0, 0, 0);
      O[1][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pb[1][t], O[1][d], 0, 0, 0);
    }
  }
  // the last LDS read of the stage is issued: start the caller's next loads while
  // the MFMAs drain
  __builtin_amdgcn_sched_barrier(0);
  after_reads();
}

template <int D, int BLK>
__global__ void __launch_bounds__((Cfg<D, BLK>::THREADS)) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_kernel(Args a) {
  using C = Cfg<D, BLK>;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * C::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t q4lds[C::Q4_BYTES];

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

  // key block and precision of tile t of this unit: sink, int4 range, int8 range
  auto tile_of = [&](int t, bool& is4) -> int {
    if (t < sink) {
      is4 = false;
      return 0;
    }
    if (t < sink + n4) {
      is4 = true;
      return lo4 + (t - sink);
    }
    is4 = false;
    return lo8 + (t - sink - n4);
  };
  const int nstages = ntiles * C::SPT;

  LoadPlan<D, BLK> lp;
  lp.init(wave, lane);
  auto issue = [&](int st, uint8_t* buf) {
    bool is4n;
    const int kbn = tile_of(st / C::SPT, is4n);
    load_stage<D, BLK>(a, lp, buf, krow0, (int64_t)kbn * BLK + (st % C::SPT) * C::SK, is4n, wave, lane);
  };
  // first stage in flight while the query state is set up
  issue(0, smem);

  // int4 query codes of the block, widened once to 16*code, into LDS (rows past the
  // end as zeros); each 16-byte group keeps the order unpack16_x16 gives the keys
#pragma unroll
  for (int i = tid; i < BLK * (D / 16); i += C::THREADS) {
    const int r = i / (D / 16), c = i % (D / 16);
    const int64_t qi = (int64_t)qb * BLK + r;
    uint2 val = make_uint2(0, 0);
    if (qi < n) val = *reinterpret_cast<const uint2*>(a.q4 + (qrow0 + qi) * (D / 2) + c * 8);
    *reinterpret_cast<v4i*>(q4lds + r * C::Q4_STRIDE + c * 16) = unpack16_x16(val.x, val.y);
  }
  v4i q8op[2][C::KS];
  RowState rs[2];
  v4f O[2][C::ND];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    rs[g].row = wave * 32 + g * 16 + lr;
    const int64_t qi = (int64_t)qb * BLK + rs[g].row;
    const bool valid = qi < n;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      q8op[g][ks] = v4i{0, 0, 0, 0};
      if (valid) q8op[g][ks] = *reinterpret_cast<const v4i*>(a.q8 + (qrow0 + qi) * D + ks * 64 + kq * 16);
    }
    const float sq8 = valid ? a.q8s[qrow0 + qi] : 0.0f;
    const float sq4 = valid ? a.q4s[qrow0 + qi] : 0.0f;
    // a row of zeros has scale 0; a tiny positive factor keeps -inf * a = -inf
    rs[g].a8 = fmaxf(sq8 * a.c, FLT_MIN);
    rs[g].a4 = fmaxf(sq4 * a.c * (1.0f / 256.0f), FLT_MIN);
    rs[g].M = -INFINITY;
    rs[g].l = 0.0f;
#pragma unroll
    for (int d = 0; d < C::ND; ++d) O[g][d] = v4f{0.f, 0.f, 0.f, 0.f};
  }

  // One stage: drain this wave's loads, barrier (stage st is in LDS and stage
  // st-1's buffer is free), read the key scales, compute, and issue the next
  // stage's loads after the stage's last LDS read (the compiler cannot tell LDS
  // reads from the loads' LDS writes and would otherwise make the reads wait for
  // them; the other work group on the CU computes while they are in flight).
  // The loads write LDS asynchronously and count as loads, so the barrier alone
  // does not wait for them: each wave drains its own first.
  auto run = [&](auto is4_tag, auto diag_tag, int st) __attribute__((always_inline)) {
    constexpr bool IS4 = decltype(is4_tag)::value, DIAG = decltype(diag_tag)::value;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const uint8_t* buf = smem + (st & 1) * C::STAGE;
    float4 ksc[4];
    const float* sc = reinterpret_cast<const float*>(buf + C::K_BYTES + C::V_BYTES);
#pragma unroll
    for (int s = 0; s < 4; ++s) ksc[s] = *reinterpret_cast<const float4*>(sc + s * 16 + kq * 4);
    auto next = [&]() {
      if (st + 1 < nstages) issue(st + 1, smem + ((st + 1) & 1) * C::STAGE);
    };
    const int key_base = (st % C::SPT) * C::SK;
    // diagonal block: waves whose rows all precede the stage's keys skip it
    if (!DIAG || key_base <= wave * 32 + 31)
      compute_stage<D, BLK, IS4, DIAG>(buf, key_base, ksc, q8op, q4lds, rs, O, lr, kq, next);
    else
      next();
  };
  using T = std::true_type;
  using F = std::false_type;
  // stages by kind, in schedule order: sink block, int4 range, int8 run, diagonal
  // (one loop per kind keeps the accumulators in the same registers)
  int st = 0;
  for (; st < sink * C::SPT; ++st) run(F(), F(), st);
  for (; st < (sink + n4) * C::SPT; ++st) run(T(), F(), st);
  for (; st < (ntiles - 1) * C::SPT; ++st) run(F(), F(), st);
  for (; st < nstages; ++st) run(F(), T(), st);

  // ---- epilogue: normalise and store (fp32), optional base-2 LSE
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    float l = rs[g].l;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int64_t qi = (int64_t)qb * BLK + rs[g].row;
    if (qi < n) {
      const float inv = 1.0f / l;
      float* dst = a.out + (qrow0 + qi) * D + kq * 4;
#pragma unroll
      for (int d = 0; d < C::ND; ++d) {
        const v4f o = O[g][d] * inv;
        *reinterpret_cast<float4*>(dst + d * 16) = make_float4(o[0], o[1], o[2], o[3]);
      }
      if (a.lse && kq == 0) a.lse[qrow0 + qi] = rs[g].M + __log2f(l);
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
