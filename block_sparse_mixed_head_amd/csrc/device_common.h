// device_common.h - small gfx950 helpers shared by the library's kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tria {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Signed 4-bit codes, packed two per byte (low nibble = even element), widened to
// int8 as 16 * code: the nibble lands in the top half of its byte, so two's
// complement gives the sign for free.  The products of two widened codes carry a
// factor 256 that the callers fold into their fp32 scale (an exact power of two).
// Output order for one packed dword w: even nibbles, then odd nibbles; any order
// works for dot products as long as both operands use the same one.
__device__ __forceinline__ uint32_t nib_even_x16(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t nib_odd_x16(uint32_t w) { return w & 0xF0F0F0F0u; }

// 16 packed nibbles (8 bytes) -> 16 int8 (x16) as one MFMA operand.
__device__ __forceinline__ v4i unpack16_x16(uint32_t w0, uint32_t w1) {
  v4i r;
  r[0] = (int)nib_even_x16(w0);
  r[1] = (int)nib_odd_x16(w0);
  r[2] = (int)nib_even_x16(w1);
  r[3] = (int)nib_odd_x16(w1);
  return r;
}

}  // namespace tria

namespace tria {

// One row of the per-row symmetric quantiser, held by TPR consecutive lanes with
// eight values each (TPR = d / 8, an aligned power-of-two group of a wavefront).
// scale = amax / qmax, r = qmax / amax (IEEE divisions), code = clamp(rint(x * r)).
// Returns the scales; codes8 gets eight int8 codes (two dwords), codes4 eight
// packed int4 codes (one dword, low nibble = even element).
#pragma clang fp contract(off)
// Codes of eight values given the row's amax (see quantize8).
__device__ __forceinline__ void codes_from_amax(const float x[8], float amax, uint32_t codes8[2],
                                                uint32_t& codes4, float& s8, float& s4) {
  float r8 = 0.0f, r4 = 0.0f;
  s8 = 0.0f;
  s4 = 0.0f;
  if (amax > 0.0f) {
    s8 = amax / 127.0f;
    r8 = 127.0f / amax;
    s4 = amax / 7.0f;
    r4 = 7.0f / amax;
  }
  codes8[0] = codes8[1] = 0u;
  codes4 = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = fminf(fmaxf(__builtin_rintf(x[i] * r8), -127.0f), 127.0f);
    const float b = fminf(fmaxf(__builtin_rintf(x[i] * r4), -7.0f), 7.0f);
    codes8[i / 4] |= ((uint32_t)(int)a & 0xFFu) << (8 * (i % 4));
    codes4 |= ((uint32_t)(int)b & 0xFu) << (4 * i);
  }
}

template <int TPR>
__device__ __forceinline__ void quantize8(const float x[8], uint32_t codes8[2], uint32_t& codes4,
                                          float& s8, float& s4) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, TPR));
  codes_from_amax(x, amax, codes8, codes4, s8, s4);
}
#pragma clang fp contract(on)

// Maximum / sum over lanes l and l ^ 16, l ^ 32 (gfx950 lane-swap instructions:
// VALU, no LDS round trip).
// max(a, b) for non-NaN operands as one v_max_f32: fmaxf would first quiet both
// operands (they come from lane permutes, which the compiler cannot prove canonical)
__device__ __forceinline__ float max_nonan(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float xmax16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nonan(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xmax32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max_nonan(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xsum16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xsum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave-uniform copies (scalar registers): bases built from them keep loads in the
// scalar-base + lane-offset form, with no per-lane address arithmetic.
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uni64(int64_t x) {
  return (int64_t)(((uint64_t)(uint32_t)uni((int)(x >> 32)) << 32) | (uint32_t)uni((int)x));
}

// Buffer resource over [base, base + bytes): loads at offsets past the end return 0
// without touching memory (gfx950 descriptor word 3 for raw 32-bit data).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(uni64(reinterpret_cast<int64_t>(base))),
                                           (short)0, uni(bytes), 0x00020000);
}

__device__ __forceinline__ void bf16x8_to_f32(uint4 raw, float x[8]) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_bits_to_f32(w[i] & 0xFFFFu);
    x[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
}

}  // namespace tria
