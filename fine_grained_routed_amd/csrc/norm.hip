// RMSNorm of the block's residual stream, the input of the FFN:
//   u[t, c] = x[t, c] / sqrt(mean_c' x[t, c']^2 + eps) * gamma[c]
//
// Source: "Shared Expert" page on DeepSeek-V3 (How it works: the FFN input u_t
// is already RMS-normalised; Watch-outs: the shared experts sit behind the
// block's ffn_norm like the routed ones).  The norm's formula (mean of squares
// plus eps under the square root, per-channel gain) is the standard RMSNorm;
// the pages name it without writing it out.
//
// One work-group per token row.  The sum of squares, the scale and the
// products are fp64 (each square of a bf16 or fp32 value is exact in fp64), the
// reduction order is fixed (per-thread strided sums, a butterfly inside each
// wave, then the four wave sums in order), and every output is rounded once to
// the stored dtype.  The row is read twice; the second read hits L2.
#include "common.h"

#define RN_THREADS 256

// fp64 -> bf16, rounded once to nearest with ties to even.  The value is first
// rounded to fp32 toward zero with an inexact result marked in the last bit
// (round to odd); fp32 keeps 16 more significant bits than bf16, so rounding
// that fp32 to nearest-even bf16 then gives the correctly rounded bf16 of the
// fp64 value (Boldo and Melquiond, "When double rounding is odd", 2005).
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
  if (v != v) return 0x7fc0;
  const float f = __double2float_rz(v);
  uint32_t b = __float_as_uint(f);
  if ((double)f != v) b |= 1u;
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// the 8 elements of x at [i, i + 8)
template <bool BF16>
__device__ __forceinline__ void load8(const void *x, int64_t i, double v[8]) {
  if (BF16) {
    const uint4 q = *(const uint4 *)((const uint16_t *)x + i);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = (double)bf16_to_f32((uint16_t)w[j]);
      v[2 * j + 1] = (double)bf16_to_f32((uint16_t)(w[j] >> 16));
    }
  } else {
    const float4 a = *(const float4 *)((const float *)x + i);
    const float4 b = *(const float4 *)((const float *)x + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <bool BF16>
__global__ __launch_bounds__(RN_THREADS) void rmsnorm_kernel(const void *__restrict__ x,
                                                             const float *__restrict__ gamma, double eps, int d,
                                                             void *__restrict__ u) {
  const int64_t row = (int64_t)blockIdx.x * d;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  double s = 0.0;
  for (int c = tid * 8; c < d; c += RN_THREADS * 8) {
    double v[8];
    load8<BF16>(x, row + c, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) s = fma(v[j], v[j], s);
  }
  s = wave_sum_f64(s);  // every lane holds the same sum (each step adds the same pair)
  __shared__ double part[RN_THREADS / 64];
  if (lane == 0) part[wv] = s;
  __syncthreads();
  const double ms = ((part[0] + part[1]) + (part[2] + part[3])) / (double)d;
  const double r = 1.0 / sqrt(ms + eps);
  for (int c = tid * 8; c < d; c += RN_THREADS * 8) {
    double v[8];
    load8<BF16>(x, row + c, v);
    const float4 g0 = *(const float4 *)(gamma + c), g1 = *(const float4 *)(gamma + c + 4);
    const double g[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    if (BF16) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = (uint32_t)f64_to_bf16_rne(v[2 * j] * r * g[2 * j]) |
               ((uint32_t)f64_to_bf16_rne(v[2 * j + 1] * r * g[2 * j + 1]) << 16);
      *(uint4 *)((uint16_t *)u + row + c) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = (float)(v[j] * r * g[j]);
      *(float4 *)((float *)u + row + c) = make_float4(o[0], o[1], o[2], o[3]);
      *(float4 *)((float *)u + row + c + 4) = make_float4(o[4], o[5], o[6], o[7]);
    }
  }
}

hipError_t launch_rmsnorm(const moe_dims &dm, int64_t T, const void *x, const float *gamma, double eps, void *u,
                          hipStream_t st) {
  if (dm.dtype == MOE_BF16)
    rmsnorm_kernel<true><<<dim3((unsigned)T), RN_THREADS, 0, st>>>(x, gamma, eps, dm.d_model, u);
  else
    rmsnorm_kernel<false><<<dim3((unsigned)T), RN_THREADS, 0, st>>>(x, gamma, eps, dm.d_model, u);
  return hipGetLastError();
}
