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
//   * Software pipeline per wavefront: iteration s computes the softmax of stage s
//     (VALU) together with the P.V product of stage s-1 (MFMA), then the scores of
//     stage s+1.  A rescale of O (rare: the integer running maximum rises) is applied
//     after stage s-1's product and before stage s's.
//   * K, V and key scales go straight from memory into three-slot LDS rings with
//     buffer_load ... lds (no staging registers), issued two iterations before
//     their use.  These loads are written as inline asm: the compiler then does not
//     treat every later read of a ring as waiting for every load into it; the kernel
//     waits itself, for exactly the loads it needs (the next iteration's stay in
//     flight).  One barrier per stage.  Each 1 KB load instruction
//     fills a contiguous LDS range; the XOR swizzles of the LDS layouts are realised
//     by the per-lane global offsets.  Rows past the sequence end read as zeros
//     through the buffer resource's size (the causal mask discards them).
//   * Scores are computed transposed, S^T = K . Q^T, with v_mfma_i32_16x16x64_i8:
//     K (A operand) from LDS, the block's query codes (B operand) in registers for
//     the whole unit.  The 16x16 accumulator layout gives every lane one query row
//     and four keys per 16-key subtile, so row maxima and sums are in-lane plus two
//     lane swaps.
//   * int4 stages: packed K and Q nibbles are widened to int8 as 16*code in
//     registers; gfx950 has no int4 MFMA.  The factor 256 is folded into the
//     query-row scale.
//   * fp32 softmax with an integer running maximum: rescales are exact powers of
//     two, so rounding P to bf16 commutes with them and the result equals a
//     final-maximum evaluation.
//   * O^T = V^T . P^T with v_mfma_f32_16x16x32_bf16: the transposed scores are
//     already the B operand layout, and V (row-major in LDS) is fed as V^T by
//     ds_read_b64_tr_b16, so V needs no transpose pass.
//   * Wavefronts per SIMD: as many as the LDS rings let share a CU, at most two
//     (256 registers per lane); at head_dim 128 with 64-row blocks that is one.
#include <cfloat>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"
#include "tria.h"

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
  static constexpr int NO = ND + 1;     // output tiles: the ND column groups, then the row sums
  static constexpr int K_BYTES = SK * D;      // one K slot (int8; int4 uses half)
  static constexpr int V_BYTES = SK * D * 2;  // one V slot
  static constexpr int K8_INSTR = K_BYTES / 1024;  // 1 KB load instructions per stage
  static constexpr int K4_INSTR = K_BYTES / 2048;
  static constexpr int V_INSTR = V_BYTES / 1024;
  static constexpr int K8N = K8_INSTR / WAVES;  // per wave
  static constexpr int VN = V_INSTR / WAVES;
  // loads per wave and stage: K pieces, V pieces, key scales
  static constexpr int NPER = K8N + VN + 1;
  // LDS per work group (the three-slot K, V and key-scale rings) and the wavefronts
  // per SIMD it leaves room for (160 KB of LDS and four SIMDs per CU), at most two
  static constexpr int LDS = 3 * (K_BYTES + V_BYTES + SK * 4);
  static constexpr int OCC = (160 * 1024 / LDS) * WAVES / 4 < 2 ? (160 * 1024 / LDS) * WAVES / 4 : 2;
};

struct Args {
  const int32_t* header;  // the schedule's 64-byte header (checked by every work group)
  const int32_t* units;
  const int8_t* q8;
  const uint8_t* q4;
  const float* q8s;
  const float* q4s;
  const uint16_t* qraw;  // bf16 Q [rows][D] when the kernel quantises its own query rows
  const int8_t* k8;
  const uint8_t* k4;
  const float* k8s;
  const float* k4s;
  const uint16_t* v;
  float* out;
  float* lse;
  const int32_t* seqs;  // variable-length batch: {start, length} per sequence, else null
  int64_t n;            // rows per (batch, head): the sequence length, or the packed total
  int batch, hq, hkv;   // batch: the number of sequences when seqs is set
  float c;  // sm_scale * log2(e)
  // what the header must hold: version, block count (the largest one for a
  // variable-length batch), unit count
  int version, nb;
  int64_t n_units;
  int64_t rows_total;  // output rows: batch * hq * n (fixed length) or hq * n (packed)
};

// NaN in output rows [r0, r1) of the flat [rows][D] output and their LSE entries.
template <int D>
__device__ __forceinline__ void poison_rows(const Args& a, int64_t r0, int64_t r1) {
  const float qn = __builtin_nanf("");
  float4* o = reinterpret_cast<float4*>(a.out);
  for (int64_t i = r0 * (D / 4) + threadIdx.x; i < r1 * (D / 4); i += blockDim.x) o[i] = make_float4(qn, qn, qn, qn);
  if (a.lse)
    for (int64_t r = r0 + threadIdx.x; r < r1; r += blockDim.x) a.lse[r] = qn;
}

// The share of every output row that work group i poisons when the schedule header
// does not describe the call: the rows split evenly over the grid, so together the
// work groups cover the whole output.
template <int D>
__device__ __forceinline__ void poison_share(const Args& a) {
  const int64_t per = (a.rows_total + a.n_units - 1) / a.n_units;
  const int64_t r0 = (int64_t)blockIdx.x * per;
  const int64_t r1 = r0 + per < a.rows_total ? r0 + per : a.rows_total;
  if (r0 < r1) poison_rows<D>(a, r0, r1);
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) v4i lds_v4i;
typedef __attribute__((address_space(3))) v2i lds_v2i;
typedef __attribute__((address_space(3))) v4f lds_v4f;

// f(integral_constant<int, J>) for J = 0 .. N-1: array indices stay compile-time
// constants from the start, so per-lane arrays live in registers.
template <int J, int N, class F>
__device__ __forceinline__ void unroll(F&& f) {
  if constexpr (J < N) {
    f(std::integral_constant<int, J>());
    unroll<J + 1, N>(f);
  }
}

// Scheduling pattern for the current region: NDS LDS reads first, then NM times
// {one MFMA, NV vector instructions, NDR LDS reads}: matrix and vector work issue
// interleaved from the same wavefront (in-order issue would otherwise stall the
// vector work behind a burst of MFMAs).
template <int NDS, int NM, int NV, int NDR>
__device__ __forceinline__ void interleave() {
  if constexpr (NDS > 0) __builtin_amdgcn_sched_group_barrier(0x100, NDS, 0);
  unroll<0, NM>([](auto) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
    if constexpr (NDR > 0) __builtin_amdgcn_sched_group_barrier(0x100, NDR, 0);
  });
}

// s_waitcnt immediate: at most vm vector-memory and lgkm LDS/scalar operations of
// this wave still outstanding.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

// buffer_load ... lds: every active lane's 16 (4) bytes at desc base + soff + voff
// go to LDS address lds + 16 (4) * lane.  The range check covers soff + voff: lanes
// at or past the resource's byte count read 0 without a memory access.  The LDS base travels
// in m0, given to the asm as an input operand so the compiler itself loads m0 and
// knows it is in use.  No register result; completion is counted by vmcnt, which
// the caller waits for before the data is read (by any wave).
__device__ __forceinline__ void dma16(v4u desc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(desc), "s"(soff), "{m0}"(lds)
               : "memory");
}
__device__ __forceinline__ void dma4(v4u desc, uint32_t voff, uint32_t soff, uint32_t lds) {
  asm volatile("buffer_load_dword %0, %1, %2 offen lds"
               :
               : "v"(voff), "s"(desc), "s"(soff), "{m0}"(lds)
               : "memory");
}

// Per-lane byte offsets, computed once per work group and held in registers.
//   * Loads: piece j of a kind is the wave's instruction-sized share
//     i = wave + j * WAVES of a stage; it covers LDS bytes [1024 i, 1024 i + 1024)
//     of its slot, and lane l's 16 bytes land at 1024 i + 16 l, so the XOR swizzles
//     of the LDS layouts are realised by the global offsets (relative to the
//     stage's first key row).  Piece j starts 1024 * WAVES * j bytes after piece 0,
//     in LDS and in memory alike: that distance is a whole number of swizzle
//     periods of rows, so one offset per kind serves every piece.
//   * LDS reads: every slot-relative read offset is one of these bases plus a
//     compile-time constant (folded into the instruction's offset field): the
//     swizzle term only depends on bits that the constant parts leave alone.
// The values pass through an empty asm so the compiler treats them as opaque: it
// neither rebuilds them inside the loop nor hoists further derived values into
// registers.
template <int D, int BLK>
struct LaneOffsets {
  using C = Cfg<D, BLK>;
  static constexpr int PIECE_STEP = 1024 * C::WAVES;
  uint32_t gk8, gk4, gv, gs;      // global offsets of piece 0 (int8 K, int4 K, V) and of a key scale
  uint32_t k8[C::KS], k4[C::KS];  // K reads (int8 / packed int4), per k-step
  uint32_t vrow, vx;              // V reads: row part, and the XOR term of the 32-byte unit

  __device__ __forceinline__ void init(int wave, int lane) {
    const int lr = lane & 15, kq = lane >> 4;
    {
      const unsigned p = wave * 64 + lane, pc = p % C::KCH, r = p / C::KCH;
      gk8 = r * D + ((pc ^ (r & (C::KCH - 1))) << 4);
    }
    {  // a wave past the int4 stage size never loads it (empty resource).  Packed rows
       // are D/2 bytes: the chunk swizzle follows row / 4, so the 16 rows one MFMA
       // operand read touches spread over distinct banks (row mod 4 would repeat
       // every four rows)
      const unsigned p = (wave < C::K4_INSTR ? wave : 0) * 64 + lane, pc = p % C::K4CH, r = p / C::K4CH;
      gk4 = r * (D / 2) + ((pc ^ ((r >> 2) & (C::K4CH - 1))) << 4);
    }
    {
      const unsigned p = wave * 64 + lane, pc = p % C::VCH, r = p / C::VCH;
      gv = r * 2 * D + ((2 * ((pc >> 1) ^ (r & (C::VU - 1))) + (pc & 1)) << 4);
    }
    gs = lane * 4;
    // K row s*16 + lr, 16-byte chunk ks*4 + kq (int8) or 2ks + kq/2, half kq%2
    // (int4); s*16 leaves the swizzle terms (row, or row / 4, mod chunks per row)
    // unchanged
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      k8[ks] = lr * D + ((((ks << 2) + kq) ^ (lr & (C::KCH - 1))) << 4);
      k4[ks] = lr * (D / 2) + ((((ks << 1) + (kq >> 1)) ^ ((lr >> 2) & (C::K4CH - 1))) << 4) + (kq & 1) * 8;
    }
    // V row 32t + 16h + 4kq + lr/4, 32-byte unit d at (d ^ (row mod VU)); 32t + 16h
    // leaves the XOR term unchanged
    const int vr = kq * 4 + (lr >> 2);
    vrow = vr * 2 * D + (lr & 3) * 8;
    vx = (vr & (C::VU - 1)) << 5;
    asm volatile("" : "+v"(gk8));
    asm volatile("" : "+v"(gk4));
    asm volatile("" : "+v"(gv));
    asm volatile("" : "+v"(gs));
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      asm volatile("" : "+v"(k8[ks]));
      asm volatile("" : "+v"(k4[ks]));
    }
    asm volatile("" : "+v"(vrow));
    asm volatile("" : "+v"(vx));
  }
};

struct RowState {
  float M, a8, a4;
  int row;  // row index inside the q-block
};

// The block's query codes of the wave's two row groups, for the whole unit: int8 as
// MFMA operands, int4 packed (widened per int4 stage).
template <int D>
struct QCodes {
  v4i q8[2][D / 64];
  v2i q4[2][D / 64];
};

// Scores of one 64-key stage for the wave's 32 rows, S^T = K . Q^T, in two halves
// (16-key subtiles 2*PART and 2*PART + 1).  qop: the query operands of the stage's
// precision (int4 codes widened to 16*code).
template <int D, bool IS4>
__device__ __forceinline__ void qk_operands(const QCodes<D>& q, v4i (&qop)[2][D / 64]) {
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) {
      if constexpr (IS4)
        qop[g][ks] = unpack16_x16(q.q4[g][ks][0], q.q4[g][ks][1]);
      else
        qop[g][ks] = q.q8[g][ks];
    }
}
template <int D, int BLK, bool IS4, int PART>
__device__ __forceinline__ void qk_read(const lds_u8* kb, const LaneOffsets<D, BLK>& lo, v4i (&kop)[2][D / 64]) {
  using C = Cfg<D, BLK>;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const int s = 2 * PART + j;
      if constexpr (!IS4) {
        kop[j][ks] = *(const lds_v4i*)(kb + lo.k8[ks] + s * 16 * D);
      } else {
        const v2i w = *(const lds_v2i*)(kb + lo.k4[ks] + s * 16 * (D / 2));
        kop[j][ks] = unpack16_x16(w[0], w[1]);
      }
    }
}
template <int D, int PART>
__device__ __forceinline__ void qk_mma(const v4i (&kop)[2][D / 64], const v4i (&qop)[2][D / 64], v4i (&S)[2][4]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int s = 2 * PART + j;
    S[0][s] = v4i{0, 0, 0, 0};
    S[1][s] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) {
      S[0][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop[j][ks], qop[0][ks], S[0][s], 0, 0, 0);
      S[1][s] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kop[j][ks], qop[1][ks], S[1][s], 0, 0, 0);
    }
  }
}
template <int D, int BLK, bool IS4, int PART>
__device__ __forceinline__ void qk_part(const lds_u8* kb, const LaneOffsets<D, BLK>& lo, const v4i (&qop)[2][D / 64],
                                        v4i (&S)[2][4]) {
  v4i kop[2][D / 64];
  qk_read<D, BLK, IS4, PART>(kb, lo, kop);
  qk_mma<D, PART>(kop, qop, S);
}
template <int D, int BLK, bool IS4>
__device__ __forceinline__ void qk_stage(const lds_u8* kb, const LaneOffsets<D, BLK>& lo, const QCodes<D>& q,
                                         v4i (&S)[2][4]) {
  v4i qop[2][D / 64];
  qk_operands<D, IS4>(q, qop);
  qk_part<D, BLK, IS4, 0>(kb, lo, qop, S);
  qk_part<D, BLK, IS4, 1>(kb, lo, qop, S);
}

// Key scales of one stage for this lane's keys s*16 + kq*4 + 0..3.
__device__ __forceinline__ void read_key_scales(const lds_f32* sc, int kq, v4f (&ksc)[4]) {
#pragma unroll
  for (int s = 0; s < 4; ++s) ksc[s] = *(const lds_v4f*)(sc + s * 16 + kq * 4);
}

// One group (t, d) of O^T += V^T . P^T: two transposing reads give the V^T operand
// for keys 32t + (16 per half) of column group d.
template <int D, int BLK, int t, int d>
__device__ __forceinline__ v8bf pv_read(const lds_u8* vslot, const LaneOffsets<D, BLK>& lo) {
  const lds_u8* vb = vslot + lo.vrow + (lo.vx ^ (d << 5));
  const v4s lo16 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vb + 32 * t * 2 * D));
  const v4s hi16 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(vb + (32 * t + 16) * 2 * D));
  // whole-vector concatenation (element-wise inserts of the halves have been folded
  // incorrectly by the compiler)
  return __builtin_bit_cast(v8bf, __builtin_shufflevector(lo16, hi16, 0, 1, 2, 3, 4, 5, 6, 7));
}
template <int D, int BLK, int t, int d>
__device__ __forceinline__ void pv_mma(const v8bf& vop, const v8bf (&pb)[2][2], v4f (&O)[2][Cfg<D, BLK>::NO]) {
  O[0][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pb[0][t], O[0][d], 0, 0, 0);
  O[1][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pb[1][t], O[1][d], 0, 0, 0);
}
template <int D, int BLK, int t, int d>
__device__ __forceinline__ void pv_group(const lds_u8* vslot, const LaneOffsets<D, BLK>& lo, const v8bf (&pb)[2][2],
                                         v4f (&O)[2][Cfg<D, BLK>::NO]) {
  pv_mma<D, BLK, t, d>(pv_read<D, BLK, t, d>(vslot, lo), pb, O);
}
// Row sums l += sum_k P[q][k] on the matrix cores: an all-ones A operand in place of
// V^T gives every row of tile ND the sum over the stage's keys of each query's bf16
// weights (the same bf16 values the product uses).
template <int D, int BLK>
__device__ __forceinline__ void pv_rowsum(const v8bf (&pb)[2][2], v4f (&O)[2][Cfg<D, BLK>::NO]) {
  constexpr int ND = Cfg<D, BLK>::ND;
  const v8bf ones = __builtin_bit_cast(v8bf, v4i{0x3F803F80, 0x3F803F80, 0x3F803F80, 0x3F803F80});
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    O[0][ND] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[0][t], O[0][ND], 0, 0, 0);
    O[1][ND] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[1][t], O[1][ND], 0, 0, 0);
  }
}

// Softmax of stage s interleaved with the P.V product of stage s-1.
//
// Softmax with the integer running maximum: M only has to be an integer that keeps
// 2^(t - M) finite; it is raised (and O, l rescaled by an exact power of two) only
// when a row's stage maximum exceeds it by more than kSlack, so weights stay below
// 2^kSlack.  Produces the bf16 weights of stage s in the B operand layout (pcur)
// and the rescale factor per row group (f, 1 when unchanged); returns whether any
// row of the lane rescaled.  is4: an int4 stage; DIAG: a diagonal-block stage, keys
// past a row are masked (key_base = first key of the stage relative to the block
// start).
//
// The product O^T += V^T . P^T of stage s-1 (pprev, V slot vslot) is cut into
// 2*ND groups (t, d) of two transposing LDS reads and two MFMAs, emitted between the
// softmax's first three phases; scheduling barriers bound each region, so the
// compiler overlaps the MFMAs with the softmax's VALU work without hoisting every V
// read.  The product is complete before the new weights exist, so pprev and pcur
// never share registers.  The scores of stage s+1 (K slot kslot, precision QK4)
// are computed in the weights phases 3 and 4, again one half per phase, into S
// (whose stage-s values the scores phases consumed): every phase mixes matrix and
// vector work.  between(k) runs after phase k's region (k = 0, 1, 2): the caller
// spreads its memory-load issues over the iteration with it.
template <int D, int BLK, bool QK4, bool DIAG, bool NEXT, class Between>
__device__ __forceinline__ bool softmax_pv_qk(bool is4, v4i (&S)[2][4], const v4f (&ksc)[4],
                                              int key_base, RowState (&rs)[2], v8bf (&pcur)[2][2], float (&f)[2],
                                              const v8bf (&pprev)[2][2], const lds_u8* vslot,
                                              const LaneOffsets<D, BLK>& lo, v4f (&O)[2][Cfg<D, BLK>::NO], int kq,
                                              const lds_u8* kslot, const QCodes<D>& q, Between&& between) {
  using C = Cfg<D, BLK>;
  constexpr int NG = 2 * C::ND;  // product groups
  constexpr float kSlack = 8.0f;
  // Region k (k = 0, 1, 2) holds product groups [NG k / 3, NG (k + 1) / 3): their V
  // reads come first, then softmax phase k's vector work (pinned to the region),
  // then the MFMAs, which the interleave pattern spreads through the vector work.
  constexpr int NGR = (NG + 2) / 3;  // largest region
  v8bf vop[NGR];
  auto pv_read_part = [&](auto k) __attribute__((always_inline)) {
    constexpr int K = decltype(k)::value;
    unroll<NG * K / 3, NG * (K + 1) / 3>([&](auto idx) __attribute__((always_inline)) {
      constexpr int i = decltype(idx)::value, t = i / C::ND, d = i % C::ND;
      vop[i - NG * K / 3] = pv_read<D, BLK, t, d>(vslot, lo);
    });
  };
  auto pv_part = [&](auto k) __attribute__((always_inline)) {
    constexpr int K = decltype(k)::value;
    constexpr int NGK = NG * (K + 1) / 3 - NG * K / 3;  // groups in this region
    unroll<NG * K / 3, NG * (K + 1) / 3>([&](auto idx) __attribute__((always_inline)) {
      constexpr int i = decltype(idx)::value, t = i / C::ND, d = i % C::ND;
      pv_mma<D, BLK, t, d>(vop[i - NG * K / 3], pprev, O);
    });
    if constexpr (K == 2) pv_rowsum<D, BLK>(pprev, O);
    interleave<0, 2 * NGK + (K == 2 ? 4 : 0), (K < 2 ? 4 : 2), 0>();
    __builtin_amdgcn_sched_barrier(0);
    between(k);
    __builtin_amdgcn_sched_barrier(0);
  };

  float u[2][4][4];
  float mx[2];
  // phases 0, 1: scaled scores and in-lane maxima of row groups 0 and 1
  auto scores = [&](auto gtag) __attribute__((always_inline)) {
    constexpr int g = decltype(gtag)::value;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float kv[4] = {ksc[s][0], ksc[s][1], ksc[s][2], ksc[s][3]};
#pragma unroll
      for (int i = 0; i < 4; ++i) u[g][s][i] = (float)S[g][s][i] * kv[i];
    }
    if constexpr (DIAG) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key_base + s * 16 + kq * 4 + i > rs[g].row) u[g][s][i] = -INFINITY;
    }
    mx[g] = -INFINITY;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx[g] = fmaxf(mx[g], u[g][s][i]);
    // pinned here: the compiler would otherwise move this vector work across the
    // barrier or into other phases, away from the MFMAs it is meant to overlap
#pragma unroll
    for (int s = 0; s < 4; ++s) asm volatile("" : "+v"(u[g][s][0]), "+v"(u[g][s][1]), "+v"(u[g][s][2]), "+v"(u[g][s][3]));
    asm volatile("" : "+v"(mx[g]));
  };
  // Wave priority: raised through regions 0-2 (the P.V product with the scores and
  // the maxima), back to normal for the weights and the next scores: of the two
  // wavefronts sharing a SIMD, the one in these MFMA-dense regions gets the issue
  // slots first (measured: configs 2 / 3 / 5 5% / 1% / 2% faster).
  __builtin_amdgcn_s_setprio(2);
  __builtin_amdgcn_sched_barrier(0);
  pv_read_part(std::integral_constant<int, 0>());
  scores(std::integral_constant<int, 0>());
  pv_part(std::integral_constant<int, 0>());
  pv_read_part(std::integral_constant<int, 1>());
  scores(std::integral_constant<int, 1>());
  pv_part(std::integral_constant<int, 1>());
  pv_read_part(std::integral_constant<int, 2>());
  // phase 2: row maxima across the four lanes of a row, new running maxima
  bool need = false;
  float nM[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const float ag = is4 ? rs[g].a4 : rs[g].a8;
    const float Mc = ceilf(xmax32(xmax16(mx[g])) * ag);  // -inf when the stage is masked for the row
    const bool up = Mc > rs[g].M + kSlack;
    need = need || up;
    const float Mn = up ? Mc : rs[g].M;
    // M - Mn: an integer <= 0 (or -inf on the first stage), so the raw hardware exp2
    // is exact (a factor below 2^-126 only scales away what it multiplies)
    f[g] = up ? __builtin_amdgcn_exp2f(rs[g].M - Mn) : 1.0f;
    rs[g].M = Mn;
    nM[g] = -Mn;
  }
  pv_part(std::integral_constant<int, 2>());
  // phases 3, 4: weights of row groups 0 and 1 in the B operand layout
  auto weights = [&](auto gtag) __attribute__((always_inline)) {
    constexpr int g = decltype(gtag)::value;
    const float ag = is4 ? rs[g].a4 : rs[g].a8;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      v2bf x[4];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int s = 2 * t + half;
        const v2f p01 = {__builtin_amdgcn_exp2f(fmaf(u[g][s][0], ag, nM[g])),
                         __builtin_amdgcn_exp2f(fmaf(u[g][s][1], ag, nM[g]))};
        const v2f p23 = {__builtin_amdgcn_exp2f(fmaf(u[g][s][2], ag, nM[g])),
                         __builtin_amdgcn_exp2f(fmaf(u[g][s][3], ag, nM[g]))};
        x[2 * half] = __builtin_convertvector(p01, v2bf);
        x[2 * half + 1] = __builtin_convertvector(p23, v2bf);
      }
      // keys 16*(2t) + 4kq + 0..3, then 16*(2t+1) + 4kq + 0..3: the B operand's k order
      pcur[g][t] = __builtin_shufflevector(__builtin_shufflevector(x[0], x[1], 0, 1, 2, 3),
                                           __builtin_shufflevector(x[2], x[3], 0, 1, 2, 3), 0, 1, 2, 3, 4, 5, 6, 7);
      asm volatile("" : "+v"(pcur[g][t]));  // pinned to this phase (see scores)
    }
  };
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
  // regions 3, 4: the next stage's K reads, then the weights of one row group, then
  // half of the next stage's score MFMAs, interleaved with the weights
  // (NEXT false: the unit's last stage, which has no next one to score)
  if constexpr (NEXT) {
    v4i qop[2][D / 64];
    qk_operands<D, QK4>(q, qop);
    v4i kop[2][D / 64];
    qk_read<D, BLK, QK4, 0>(kslot, lo, kop);
    weights(std::integral_constant<int, 0>());
    qk_mma<D, 0>(kop, qop, S);
    interleave<0, 4 * C::KS, (QK4 ? 9 : 6), 0>();
    __builtin_amdgcn_sched_barrier(0);
    qk_read<D, BLK, QK4, 1>(kslot, lo, kop);
    weights(std::integral_constant<int, 1>());
    qk_mma<D, 1>(kop, qop, S);
    interleave<0, 4 * C::KS, (QK4 ? 9 : 6), 0>();
  } else {
    weights(std::integral_constant<int, 0>());
    weights(std::integral_constant<int, 1>());
  }
  return need;
}

// O^T += V^T . P^T for one stage (the last one, after the loop).
template <int D, int BLK>
__device__ __forceinline__ void pv_stage(const lds_u8* vslot, const LaneOffsets<D, BLK>& lo, const v8bf (&pb)[2][2],
                                         v4f (&O)[2][Cfg<D, BLK>::NO]) {
  using C = Cfg<D, BLK>;
  unroll<0, 2 * C::ND>([&](auto idx) __attribute__((always_inline)) {
    constexpr int t = decltype(idx)::value / C::ND, d = decltype(idx)::value % C::ND;
    pv_group<D, BLK, t, d>(vslot, lo, pb, O);
  });
  pv_rowsum<D, BLK>(pb, O);
}

// The work group's unit, checked: the schedule's header must describe the call and
// the unit's record must be well formed.  A header that does not describe the call:
// NaN over the work group's even share of all output rows (every work group does
// the same and none computes, so the whole output is NaN).  A malformed record: NaN
// over the rows it names (rows no other unit of a valid list holds), or nothing
// written when it names no rows.  Either way false is returned.
struct Unit {
  int b, h, qb, lo8, lo4, hi4, sink, n4, ntiles, bb;
  int64_t seq0, n;
};
template <int D, int BLK>
__device__ __forceinline__ bool unit_of(const Args& a, Unit& un) {
  // The header's first twelve words and the unit's record in one round trip (the
  // host sized the schedule for n_units records); the empty asm keeps the five
  // scalar loads together here rather than sunk past the header check.
  const v4i* hp = reinterpret_cast<const v4i*>(a.header);
  const v4i* up = reinterpret_cast<const v4i*>(a.units + 8 * (int64_t)blockIdx.x);
  v4i h0 = hp[0], h1 = hp[1], h2 = hp[2], u0 = up[0], u1 = up[1];
  asm volatile("" : "+s"(h0), "+s"(h1), "+s"(h2), "+s"(u0), "+s"(u1));
  const int b = u0[0], h = u0[1], qb = u0[2], lo8 = u0[3], lo4 = u1[0], hi4 = u1[1], sink = u1[2];
  const int n4 = hi4 - lo4 + 1;
  const int ntiles = u1[3];
  {  // a header that does not describe this call: NaN over every output row
    // (compared without short-circuit branches)
    const bool ok = (h0[0] == TRIA_SCHED_MAGIC) & (h0[1] == a.version) & (h0[2] == a.batch) & (h0[3] == a.hq) &
                    (h1[0] == a.hkv) & (h1[1] == D) & (h1[2] == BLK) & (h1[3] == a.nb) &
                    (h2[0] == (int32_t)a.n_units) & (h2[2] == (int32_t)(a.n & 0xFFFFFFFF)) &
                    (h2[3] == (int32_t)(a.n >> 32));
    if (!ok) {
      poison_share<D>(a);
      return false;
    }
  }
  // a variable-length batch packs its sequences along the rows of one batch element:
  // unit b is sequence b, rows [seq0, seq0 + n)
  int64_t seq0 = 0, n = a.n;
  int bb = b;
  if (b >= 0 && b < a.batch && a.seqs) {  // (b checked before the sequence table is read)
    seq0 = a.seqs[2 * b];
    n = a.seqs[2 * b + 1];
    bb = 0;
  }
  {  // a malformed record computes nothing: NaN over the rows it names, if any
    const int64_t nbq = (n + BLK - 1) / BLK;
    const bool rows_ok = b >= 0 && b < a.batch && seq0 >= 0 && n >= 1 && seq0 + n <= a.n && h >= 0 && h < a.hq &&
                         qb >= 0 && qb < nbq;
    const bool bad = !rows_ok || lo8 < 0 || lo8 > qb || sink < 0 || sink > 1 || (sink == 1 && lo8 == 0) || n4 < 0 ||
                     (n4 > 0 && (lo4 < 1 || hi4 != lo8 - 1)) || ntiles != (qb - lo8 + 1) + sink + n4;
    if (bad) {
      if (rows_ok) {
        const int64_t r0 = ((int64_t)bb * a.hq + h) * a.n + seq0 + (int64_t)qb * BLK;
        poison_rows<D>(a, r0, r0 + ((n - (int64_t)qb * BLK) < BLK ? (n - (int64_t)qb * BLK) : BLK));
      }
      return false;
    }
  }
  un = Unit{b, h, qb, lo8, lo4, hi4, sink, n4, ntiles, bb, seq0, n};
  return true;
}

// QRAW: the query rows arrive as bf16 and each work group quantises its own block
// (the rows no other unit reads) in the prologue, with the quantiser's arithmetic
// (the same codes and scales as tria_quantize_qk), instead of reading codes.
template <int D, int BLK, bool QRAW>
__global__ void __launch_bounds__((Cfg<D, BLK>::THREADS))
__attribute__((amdgpu_waves_per_eu(Cfg<D, BLK>::OCC, Cfg<D, BLK>::OCC)))
prefill_kernel(Args a) {
  using C = Cfg<D, BLK>;
  using LO = LaneOffsets<D, BLK>;
  // three-slot rings
  __shared__ __attribute__((aligned(1024))) uint8_t kring_[3 * C::K_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vring_[3 * C::V_BYTES];
  __shared__ __attribute__((aligned(16))) float sring_[3 * C::SK];
  static_assert(sizeof(kring_) + sizeof(vring_) + sizeof(sring_) == C::LDS, "LDS budget");
  lds_u8* const kring = (lds_u8*)kring_;
  lds_u8* const vring = (lds_u8*)vring_;
  lds_f32* const sring = (lds_f32*)sring_;
  auto kslot = [&](int r) __attribute__((always_inline)) { return kring + r * C::K_BYTES; };
  auto vslot = [&](int r) __attribute__((always_inline)) { return vring + r * C::V_BYTES; };
  auto sslot = [&](int r) __attribute__((always_inline)) { return sring + r * C::SK; };
  auto lds_addr = [](const void __attribute__((address_space(3)))* p) __attribute__((always_inline)) {
    return (uint32_t)uni((int)(uint32_t)(uintptr_t)p);
  };

  Unit un;
  if (!unit_of<D, BLK>(a, un)) return;
  const int h = un.h, qb = un.qb, lo8 = un.lo8, lo4 = un.lo4, sink = un.sink, n4 = un.n4, ntiles = un.ntiles;
  const int64_t seq0 = un.seq0, n = un.n;
  const int g_kv = h / (a.hq / a.hkv);
  const int64_t qrow0 = ((int64_t)un.bb * a.hq + h) * a.n + seq0;
  const int64_t krow0 = ((int64_t)un.bb * a.hkv + g_kv) * a.n + seq0;

  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6), lane = tid & 63;
  const int lr = lane & 15, kq = lane >> 4;

  // stage kinds, in schedule order: sink block, int4 range, int8 run, diagonal block
  const int nstages = ntiles * C::SPT;
  const int e_sink = sink * C::SPT, e_int4 = (sink + n4) * C::SPT, e_int8 = (ntiles - 1) * C::SPT;
  auto is4_of = [&](int st) __attribute__((always_inline)) { return st >= e_sink && st < e_int4; };

  LO lo;
  lo.init(wave, lane);

  // Loads of stage st's K pieces and key scales into a K slot and a scale slot, and
  // of stage st's V pieces into a V slot.  Each issues a fixed number of load
  // instructions (K8N + 1, VN) whatever the stage, so the waits can count them: a
  // stage past the last one, or a K piece past the int4 stage size, reads through an
  // empty resource.  Resources and offsets are chosen by value, never by branching.
  // The resources start at the unit's rows (per-unit words: the low 32 bits of the
  // base and its high 16); a stage passes its first key's byte offset as the scalar
  // offset and ends the resource at its last row inside the sequence (byte count =
  // that offset + its rows' bytes), so rows past the end read as zero.  Byte offsets
  // are 32-bit (the host guarantees (seq_len + 4 * block) * 2 * head_dim < 2^31,
  // which covers the three stages issued past the last one): a stage's addresses
  // cost a few scalar instructions.
  const uint64_t k8u = uni64(reinterpret_cast<int64_t>(a.k8 + krow0 * D));
  const uint64_t k4u = uni64(reinterpret_cast<int64_t>(a.k4 + krow0 * (D / 2)));
  const uint64_t vu = uni64(reinterpret_cast<int64_t>(a.v + krow0 * D));
  const uint64_t s8u = uni64(reinterpret_cast<int64_t>(a.k8s + krow0));
  const uint64_t s4u = uni64(reinterpret_cast<int64_t>(a.k4s + krow0));
  auto w0_of = [](uint64_t p) __attribute__((always_inline)) { return (uint32_t)p; };
  auto w1_of = [](uint64_t p) __attribute__((always_inline)) { return (uint32_t)(p >> 32) & 0xffffu; };
  auto rsrc = [](uint32_t w0, uint32_t w1, int bytes) __attribute__((always_inline)) {
    return v4u{(uint32_t)uni((int)w0), (uint32_t)uni((int)w1), (uint32_t)uni(bytes), 0x00020000u};
  };
  const int n32 = (int)n;
  // The stages' first keys: the sink block's stages start at key 0; from stage e_sink
  // on the keys are consecutive (the int4 range ends where the int8 run begins), so
  // key0 = st * SK + key_off there.  PAST: st >= e_sink is known (every stage issued
  // inside the loop, s + 3 >= 3 >= e_sink).
  const int key_off = ((n4 > 0 ? lo4 : lo8) * C::SPT - e_sink) * C::SK;
  auto key0_of = [&](int st, auto past_tag) __attribute__((always_inline)) -> int {
    if constexpr (decltype(past_tag)::value)
      return st * C::SK + key_off;
    else
      return st * C::SK + (st < e_sink ? 0 : key_off);
  };
  // rows of the stage inside the sequence (0 for a stage past the last one)
  auto rows_of = [&](bool valid, int key0) __attribute__((always_inline)) {
    // clamp(n - key0, 0, SK) on the scalar unit: as plain min/max the compiler forms
    // a v_med3_i32 and moves the result back with v_readfirstlane
    int rows;
    asm("s_sub_i32 %0, %1, %2\n\ts_max_i32 %0, %0, 0\n\ts_min_i32 %0, %0, %3"
        : "=&s"(rows) : "s"(n32), "s"(key0), "i"(C::SK) : "scc");
    return valid ? rows : 0;
  };
  constexpr int LOG2D = D == 128 ? 7 : 6;
  static_assert((1 << LOG2D) == D, "head_dim 64 or 128");
  // issue_k returns the stage's {first key, rows}; the V loads of the same stage,
  // issued two iterations later, take them from there
  auto issue_k = [&](int st, lds_u8* kd, lds_f32* sd, auto past_tag) __attribute__((always_inline)) {
    constexpr bool PAST = decltype(past_tag)::value;
    const bool valid = st < nstages;
    const bool is4 = PAST ? st < e_int4 : is4_of(st);
    const int key0 = key0_of(st, past_tag);
    const int rows = rows_of(valid, key0);
    // resource words chosen by value.  At d = 64 the compiler turns plain selects of
    // several words into a lookup table in scratch memory, loaded in every
    // iteration, so there the choice is mask arithmetic; at d = 128 plain selects
    // give fewer instructions.
    const uint32_t m4 = D == 64 ? (uint32_t)uni(is4 ? -1 : 0) : 0u;
    auto pick = [&](uint32_t w8, uint32_t w4) __attribute__((always_inline)) -> uint32_t {
      return D == 64 ? w8 ^ ((w8 ^ w4) & m4) : (is4 ? w4 : w8);
    };
    const int sh = is4 ? LOG2D - 1 : LOG2D;  // log2 of the K row bytes
    const uint32_t kw0 = pick(w0_of(k8u), w0_of(k4u)), kw1 = pick(w1_of(k8u), w1_of(k4u));
    // a stage with no rows (past the last) gets an empty resource: no lane in range
    // whatever the offset
    const int ksoff = key0 << sh;
    const int kend = rows > 0 ? ksoff + (rows << sh) : 0;
    const uint32_t off = lo.gk8 ^ ((lo.gk8 ^ lo.gk4) & (is4 ? ~0u : 0u));
#pragma unroll
    for (int j = 0; j < C::K8N; ++j) {
      const bool skip = is4 && wave + j * C::WAVES >= C::K4_INSTR;
      dma16(rsrc(kw0, kw1, skip ? 0 : kend), off + j * LO::PIECE_STEP, (uint32_t)ksoff,
            lds_addr(kd + (wave + j * C::WAVES) * 1024));
    }
    const uint32_t sw0 = pick(w0_of(s8u), w0_of(s4u)), sw1 = pick(w1_of(s8u), w1_of(s4u));
    dma4(rsrc(sw0, sw1, rows > 0 ? (key0 + rows) * 4 : 0), lo.gs, (uint32_t)(key0 * 4), lds_addr(sd));
    return make_int2(key0, rows);
  };
  auto issue_v = [&](int2 kr, lds_u8* vd) __attribute__((always_inline)) {
    const v4u rv = rsrc(w0_of(vu), w1_of(vu), kr.y > 0 ? (kr.x + kr.y) * 2 * D : 0);
    const uint32_t vsoff = (uint32_t)(kr.x * 2 * D);
#pragma unroll
    for (int j = 0; j < C::VN; ++j)
      dma16(rv, lo.gv + j * LO::PIECE_STEP, vsoff, lds_addr(vd + (wave + j * C::WAVES) * 1024));
  };

  // ---- prologue: K and scales of stages 0..2, V of stage 0; V slot 2 (read with
  // zero weights by the first iteration, as "stage -1") cleared
  // {first key, rows} of stages s + 1 and s + 2 for iteration s (from their K loads)
  using T = std::true_type;
  using F = std::false_type;
  const int2 kr0 = issue_k(0, kslot(0), sslot(0), F());
  int2 kr_next = issue_k(1, kslot(1), sslot(1), F());
  int2 kr_next2 = issue_k(2, kslot(2), sslot(2), F());
  issue_v(kr0, vslot(0));
  for (int i = tid; i < C::V_BYTES / 16; i += C::THREADS) *(lds_v4i*)(vslot(2) + i * 16) = v4i{0, 0, 0, 0};

  // the block's query codes (rows past the end as zeros)
  QCodes<D> q;
  RowState rs[2];
  v4f O[2][C::NO];
  // QRAW: every bf16 load of both row groups is issued before any is used, each from
  // a row inside the sequence (a row past the end re-reads row n - 1 and is zeroed
  // after it lands).  A load under a per-lane condition would be followed by a write
  // of zeros to its destination register on the other lanes, which must wait for the
  // load: one memory round trip per load.  Lane (lr, kq) holds columns 64 ks + 16 kq
  // .. + 15 of its row, as the codes' operand layout below wants.
  uint4 qw[QRAW ? 2 : 1][C::KS][2];
  if constexpr (QRAW) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int64_t qi = (int64_t)qb * BLK + wave * 32 + g * 16 + lr;
      const int64_t qr = qi < n ? qi : n - 1;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          qw[g][ks][hh] = *reinterpret_cast<const uint4*>(a.qraw + (qrow0 + qr) * D + ks * 64 + kq * 16 + hh * 8);
    }
  }
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    rs[g].row = wave * 32 + g * 16 + lr;
    const int64_t qi = (int64_t)qb * BLK + rs[g].row;
    const bool valid = qi < n;
    float sq8, sq4;
    if constexpr (QRAW) {
      // the row's other columns sit in lanes lr + 16 kq' (lane distances 16 and 32),
      // so the row maximum is two lane swaps away
      float x[C::KS][2][8];
      float amax = 0.0f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint4 w = valid ? qw[g][ks][hh] : make_uint4(0u, 0u, 0u, 0u);
          bf16x8_to_f32(w, x[ks][hh]);
#pragma unroll
          for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[ks][hh][i]));
        }
      amax = xmax32(xmax16(amax));
      sq8 = 0.0f;
      sq4 = 0.0f;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        uint32_t c8a[2], c8b[2], c4a, c4b;
        codes_from_amax(x[ks][0], amax, c8a, c4a, sq8, sq4);
        codes_from_amax(x[ks][1], amax, c8b, c4b, sq8, sq4);
        q.q8[g][ks] = v4i{(int)c8a[0], (int)c8a[1], (int)c8b[0], (int)c8b[1]};
        q.q4[g][ks] = v2i{(int)c4a, (int)c4b};
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        q.q8[g][ks] = valid ? *reinterpret_cast<const v4i*>(a.q8 + (qrow0 + qi) * D + ks * 64 + kq * 16) : v4i{0, 0, 0, 0};
        q.q4[g][ks] = valid ? *reinterpret_cast<const v2i*>(a.q4 + (qrow0 + qi) * (D / 2) + ks * 32 + kq * 8) : v2i{0, 0};
      }
      sq8 = valid ? a.q8s[qrow0 + qi] : 0.0f;
      sq4 = valid ? a.q4s[qrow0 + qi] : 0.0f;
    }
    // a row of zeros has scale 0; a tiny positive factor keeps -inf * a = -inf
    rs[g].a8 = fmaxf(sq8 * a.c, FLT_MIN);
    rs[g].a4 = fmaxf(sq4 * a.c * (1.0f / 256.0f), FLT_MIN);
    rs[g].M = -INFINITY;
#pragma unroll
    for (int d = 0; d < C::NO; ++d) O[g][d] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));  // every load above complete
  __syncthreads();

  v4i S[2][4];
  v4f ksc[4];
  v8bf pprev[2][2];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int t = 0; t < 2; ++t) pprev[g][t] = __builtin_bit_cast(v8bf, v4i{0, 0, 0, 0});
  if (is4_of(0))
    qk_stage<D, BLK, true>(kslot(0), lo, q, S);
  else
    qk_stage<D, BLK, false>(kslot(0), lo, q, S);
  read_key_scales(sslot(0), kq, ksc);

  // ---- iteration s (slot index R = s mod 3):
  //   wait for this wave's loads of K(s+1), V(s-1) (issued two iterations ago; the
  //   previous iteration's stay in flight) and for its reads of scales(s); barrier;
  //   issue K(s+3), scales(s+3) into slot R and V(s+1) into slot R+1 (their previous
  //   contents were last read before the barrier); softmax(s) with the product of
  //   s-1 (V slot R+2); the scores of s+1 (K slot R+1) and the scales of s+1.
  int R = 0;
  auto iter = [&](int s, auto qk4_tag, auto diag_tag, auto next_tag) __attribute__((always_inline)) {
    constexpr bool QK4 = decltype(qk4_tag)::value;  // precision of stage s+1
    constexpr bool DIAG = decltype(diag_tag)::value;  // stage s in the diagonal block
    constexpr bool NEXT = decltype(next_tag)::value;  // a stage s+1 exists
    const int R1 = R == 2 ? 0 : R + 1, R2 = R == 0 ? 2 : R - 1;
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(C::NPER, 0));
    __builtin_amdgcn_s_barrier();
    v8bf pcur[2][2];
    float f[2];
    // the loads of K(s+3) and scales(s+3), then of V(s+1), are issued between the
    // softmax phases rather than all at once after the barrier, when every wave of
    // the CU would queue them together.
    int2 kr3;
    auto between = [&](auto k) __attribute__((always_inline)) {
      if constexpr (decltype(k)::value == 0) kr3 = issue_k(s + 3, kslot(R), sslot(R), T());
      if constexpr (decltype(k)::value == 1) {
        issue_v(kr_next, vslot(R1));
        kr_next = kr_next2;
        kr_next2 = kr3;
      }
    };
    const bool is4 = is4_of(s);
    const int key_base = (s % C::SPT) * C::SK;
    // the V read bases per column group (vx ^ 32d) are rebuilt in every iteration
    // (one XOR each) rather than hoisted out of the loop into registers
    LO lo_it = lo;
    asm volatile("" : "+v"(lo_it.vx));
    const bool need = softmax_pv_qk<D, BLK, QK4, DIAG, NEXT>(is4, S, ksc, key_base, rs, pcur, f, pprev, vslot(R2), lo_it, O,
                                                 kq, kslot(R1), q, between);
    // the rescale of O applies to the products of stages up to s-1 (complete) and
    // precedes the product of stage s (next iteration)
    if (__ballot(need)) {
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int d = 0; d < C::NO; ++d) O[g][d] *= f[g];
    }
    read_key_scales(sslot(R1), kq, ksc);
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int t = 0; t < 2; ++t) pprev[g][t] = pcur[g][t];
    R = R1;
  };
  // Four loops, so that each body has one precision for the scores of stage s+1 and
  // one masking mode (two variants in one body would sit under branches, which
  // split its scheduling regions and double its register needs): s+1 is an int4
  // stage exactly for s in [b1, b2), and stages from e_int8 on are diagonal; the
  // last stage, which has no next one to score, runs on its own.
  const int b1 = n4 > 0 ? (e_sink > 0 ? e_sink - 1 : 0) : 0;
  const int b2 = n4 > 0 ? e_int4 - 1 : 0;
  int s = 0;
  for (; s < (b1 < e_int8 ? b1 : e_int8); ++s) iter(s, F(), F(), T());
  for (; s < b2; ++s) iter(s, T(), F(), T());
  for (; s < e_int8; ++s) iter(s, F(), F(), T());
  for (; s < nstages - 1; ++s) iter(s, F(), T(), T());
  iter(s, F(), T(), F());  // the last stage: nothing left to score
  ++s;
  // product of the last stage, from V slot (nstages - 1) mod 3, whose loads were
  // issued in the last iteration but one
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  __syncthreads();
  pv_stage<D, BLK>(vslot((nstages - 1) % 3), lo, pprev, O);

  // ---- epilogue: normalise and store (fp32), optional base-2 LSE
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const float l = O[g][C::ND][0];  // the row sum (every row of the sums tile)
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
  if (a.qraw)
    hipLaunchKernelGGL((prefill_kernel<D, BLK, true>), dim3((unsigned)n_units), dim3(C::THREADS), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_kernel<D, BLK, false>), dim3((unsigned)n_units), dim3(C::THREADS), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const Shape& s, const int32_t* header, int version, int64_t nb, int64_t n_units,
                          const int32_t* seqs, int n_seqs, const int8_t* q8, const uint8_t* q4, const float* q8s,
                          const float* q4s, const void* qraw, const int8_t* k8, const uint8_t* k4, const float* k8s,
                          const float* k4s, const void* v, float sm_scale, float* out, float* lse, hipStream_t stream) {
  Args a;
  a.header = header;
  a.units = header + TRIA_SCHED_HEADER_BYTES / 4;
  a.version = version;
  a.nb = (int)nb;
  a.n_units = n_units;
  a.rows_total = (int64_t)(seqs ? 1 : s.batch) * s.hq * s.n;
  a.seqs = seqs;
  a.q8 = q8;
  a.q4 = q4;
  a.q8s = q8s;
  a.q4s = q4s;
  a.qraw = static_cast<const uint16_t*>(qraw);
  a.k8 = k8;
  a.k4 = k4;
  a.k8s = k8s;
  a.k4s = k4s;
  a.v = static_cast<const uint16_t*>(v);
  a.out = out;
  a.lse = lse;
  a.n = s.n;
  a.batch = seqs ? n_seqs : s.batch;
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
