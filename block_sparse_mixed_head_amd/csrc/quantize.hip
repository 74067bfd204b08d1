// quantize.hip - per-row symmetric int8 / int4 quantisation of Q and K.
//
// TriAttention summary page (rit.work), section on which links can be skipped:
// a kept tile is computed at 8 or at 4 bits.  Each row (d values of one token of
// one head) gets its own fp32 scale: scale = amax / qmax and
// code = clamp(rint(x * (qmax / amax)), -qmax, qmax), qmax = 127 or 7.
//
// Memory-bound: one 16-byte load of eight bf16 per lane, d/8 lanes per row (an
// aligned group of a wavefront, reduced with cross-lane shuffles), 8 bytes of int8
// codes, 4 bytes of packed int4 codes and two scales out.  Q and K rows share one
// launch (grid over both tensors' rows).  Division is IEEE-correct (the hipcc
// default) and nothing here is contracted into an FMA, so the codes are bit-exact
// with any correctly rounded implementation of the same formula.
#include "device_common.h"
#include "kernels.h"

namespace tria {

namespace {

constexpr int kThreads = 256;

struct RowOut {
  int8_t* c8;
  uint8_t* c4;
  float* s8;
  float* s4;
};

template <int D>
__global__ void __launch_bounds__(kThreads) quantize_rows_kernel(const uint16_t* __restrict__ q,
                                                                 const uint16_t* __restrict__ k,
                                                                 int64_t q_rows, int64_t k_rows,
                                                                 RowOut qo, RowOut ko) {
  constexpr int TPR = D / 8;  // lanes per row
  const int64_t row = (int64_t)blockIdx.x * (kThreads / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  const bool is_q = row < q_rows;
  const int64_t r = is_q ? row : row - q_rows;
  if (!is_q && r >= k_rows) return;  // whole row groups leave together
  const uint16_t* src = (is_q ? q : k) + r * D + part * 8;
  const RowOut o = is_q ? qo : ko;

  float x[8];
  bf16x8_to_f32(*reinterpret_cast<const uint4*>(src), x);
  uint32_t c8w[2], c4w;
  float s8, s4;
  quantize8<TPR>(x, c8w, c4w, s8, s4);
  *reinterpret_cast<uint2*>(o.c8 + r * D + part * 8) = make_uint2(c8w[0], c8w[1]);
  *reinterpret_cast<uint32_t*>(o.c4 + r * (D / 2) + part * 4) = c4w;
  if (part == 0) {
    o.s8[r] = s8;
    o.s4[r] = s4;
  }
}

}  // namespace

hipError_t launch_quantize(const Shape& s, const void* q, const void* k, int8_t* q8, uint8_t* q4,
                           float* q8s, float* q4s, int8_t* k8, uint8_t* k4, float* k8s, float* k4s,
                           hipStream_t stream) {
  const int64_t q_rows = q ? (int64_t)s.batch * s.hq * s.n : 0;  // (no Q: K rows only)
  const int64_t k_rows = (int64_t)s.batch * s.hkv * s.n;
  const int64_t rows = q_rows + k_rows;
  const int rows_per_block = kThreads / (s.d / 8);
  const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  RowOut qo{q8, q4, q8s, q4s}, ko{k8, k4, k8s, k4s};
  const uint16_t* qp = static_cast<const uint16_t*>(q);
  const uint16_t* kp = static_cast<const uint16_t*>(k);
  if (s.d == 128)
    hipLaunchKernelGGL(quantize_rows_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       qp, kp, q_rows, k_rows, qo, ko);
  else
    hipLaunchKernelGGL(quantize_rows_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       qp, kp, q_rows, k_rows, qo, ko);
  return hipGetLastError();
}

}  // namespace tria
