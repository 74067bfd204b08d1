// peaks.hip - measured ceilings for the roofline report (measurement helpers, not
// part of the method).
//
// The benchmark quotes its fractions against MI355X's published peaks.  These loops
// measure what the part sustains for the same instructions, so the fractions can
// also be read against measured ceilings:
//   * an MFMA issue loop for each contraction the prefill kernel uses
//     (v_mfma_i32_16x16x64_i8 and v_mfma_f32_16x16x32_bf16): every wavefront keeps
//     eight independent accumulators, two wavefronts per SIMD, no memory traffic;
//   * a streaming read with the decode kernel's access pattern: each wavefront reads
//     one contiguous range with 1 KB non-temporal loads, eight in flight.
#include "device_common.h"
#include "kernels.h"

namespace tria {

namespace {

constexpr int kThreads = 256;           // four wavefronts
constexpr int kMfmaBlocks = 512;        // two work groups per CU: two wavefronts per SIMD
constexpr int kChains = 8;              // independent accumulators per wavefront
constexpr int kReadWaves = 8192;        // wavefronts of the streaming read
constexpr int kReadUnroll = 8;          // 1 KB loads in flight per wavefront
constexpr int kReadChunk = 1024;        // bytes per wavefront load

typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));

// Eight accumulators as separate variables, each with its own A operand (so no two
// chains are provably equal and each keeps one aligned register tuple).
#define TRIA_CHAINS(X) X(0) X(1) X(2) X(3) X(4) X(5) X(6) X(7)
template <bool BF16>
__global__ void __launch_bounds__(kThreads) mfma_loop_kernel(int iters, int* sink) {
  const int lane = threadIdx.x & 63;
  const v4i b = {lane ^ 5, 2, lane + 11, lane};
  int x = 0;
  if constexpr (!BF16) {
#define DECL(c) const v4i a##c = {lane + c, 3 * lane, 7 - c, lane ^ c}; v4i acc##c = {0, 0, 0, 0};
    TRIA_CHAINS(DECL)
#undef DECL
    for (int it = 0; it < iters; ++it) {
#define STEP(c) acc##c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a##c, b, acc##c, 0, 0, 0);
      TRIA_CHAINS(STEP)
#undef STEP
    }
#define RED(c) x ^= acc##c[0] ^ acc##c[1] ^ acc##c[2] ^ acc##c[3];
    TRIA_CHAINS(RED)
#undef RED
  } else {
    // small finite bf16 operands (bit patterns 0x3C00..0x3CFF: values near 2^-7)
    const v8bf_t bb = __builtin_bit_cast(v8bf_t, (b & 0x00FF00FF) | 0x3C003C00);
#define DECL(c)                                                                                  \
  const v8bf_t a##c = __builtin_bit_cast(v8bf_t, (v4i{lane + c, 3 * lane, 7 - c, lane ^ c} & 0x00FF00FF) | 0x3C003C00); \
  v4f acc##c = {0.f, 0.f, 0.f, 0.f};
    TRIA_CHAINS(DECL)
#undef DECL
    for (int it = 0; it < iters; ++it) {
#define STEP(c) acc##c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a##c, bb, acc##c, 0, 0, 0);
      TRIA_CHAINS(STEP)
#undef STEP
    }
#define RED(c) x ^= __float_as_int(acc##c[0]) ^ __float_as_int(acc##c[1]) ^ __float_as_int(acc##c[2]) ^ __float_as_int(acc##c[3]);
    TRIA_CHAINS(RED)
#undef RED
  }
  // every lane's result feeds the stored value, so no lane's work is dead
  x ^= __shfl_xor(x, 1);
  x ^= __shfl_xor(x, 2);
  if (lane == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = x;
}
#undef TRIA_CHAINS

// Wavefront w reads bytes [w * per_wave, (w + 1) * per_wave) of src.
__global__ void __launch_bounds__(kThreads) stream_read_kernel(const uint8_t* src, int per_wave, int* sink) {
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(src + uni64(w * per_wave), per_wave);
  v4i acc = {0, 0, 0, 0};
  for (int i0 = 0; i0 < per_wave; i0 += kReadUnroll * kReadChunk) {
    v4i x[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u)
      x[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + u * kReadChunk, uni(i0), 2 /* nt */);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= x[u];
  }
  int y = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  y ^= __shfl_xor(y, 1);
  y ^= __shfl_xor(y, 2);
  if (lane == 0) sink[w] = y;
}

}  // namespace

double peak_mfma_work(int kind, int iters) {
  const double per_mfma = kind == 0 ? 2.0 * 16 * 16 * 64 : 2.0 * 16 * 16 * 32;
  return per_mfma * kChains * (double)iters * kMfmaBlocks * (kThreads / 64);
}

hipError_t launch_peak_mfma(int kind, int iters, int* sink, hipStream_t stream) {
  if (kind == 0)
    hipLaunchKernelGGL(mfma_loop_kernel<false>, dim3(kMfmaBlocks), dim3(kThreads), 0, stream, iters, sink);
  else
    hipLaunchKernelGGL(mfma_loop_kernel<true>, dim3(kMfmaBlocks), dim3(kThreads), 0, stream, iters, sink);
  return hipGetLastError();
}

int64_t peak_read_align() { return (int64_t)kReadWaves * kReadUnroll * kReadChunk; }

hipError_t launch_peak_read(const void* src, int64_t bytes, int* sink, hipStream_t stream) {
  const int per_wave = (int)(bytes / kReadWaves);
  hipLaunchKernelGGL(stream_read_kernel, dim3(kReadWaves / (kThreads / 64)), dim3(kThreads), 0, stream,
                     static_cast<const uint8_t*>(src), per_wave, sink);
  return hipGetLastError();
}

}  // namespace tria
