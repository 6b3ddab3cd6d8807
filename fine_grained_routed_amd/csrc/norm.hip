// RMSNorm of the block's residual stream, the input of the FFN:
//   u[t, c] = x[t, c] / sqrt(mean_c' x[t, c']^2 + eps) * gamma[c]
//
// Source: "Shared Expert" page on DeepSeek-V3 (How it works: the FFN input u_t
// is already RMS-normalised; Watch-outs: the shared experts sit behind the
// block's ffn_norm like the routed ones).  The norm's formula (mean of squares
// plus eps under the square root, per-channel gain) is the standard RMSNorm;
// the pages name it without writing it out.
//
// One wave per token row.  The sum of squares, the scale and the products are
// fp64 (each square of a bf16 or fp32 value is exact in fp64), the reduction
// order is fixed (per-lane sums in chunk order, then a butterfly inside the
// wave), and every output is rounded once to the stored dtype.  The row is
// read once and kept in registers.
#include "common.h"

#define RN_THREADS 256

// fp64 -> bf16, rounded once to nearest with ties to even.  The value is first
// rounded to fp32 toward zero with an inexact result marked in the last bit
// (round to odd); fp32 keeps 16 more significant bits than bf16, so rounding
// that fp32 to nearest-even bf16 then gives the correctly rounded bf16 of the
// fp64 value (Boldo and Melquiond, "When double rounding is odd", 2005).  The
// toward-zero step is derived from the hardware's nearest-even conversion:
// about a third of the instructions of the library's toward-zero conversion,
// which made this kernel VALU-bound (0.124 against 0.159 ms at DeepSeek-V3
// prefill, identical bits).
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
  if (v != v) return 0x7fc0;
  const float f = (float)v;  // the hardware conversion, to nearest even
  const double back = (double)f;
  uint32_t b = __float_as_uint(f);
  if (back != v) {
    // inexact: where the nearest value lies beyond v, the one toward zero is
    // the adjacent encoding (also across the subnormal boundary, and from
    // infinity to the largest finite value); then mark the last bit
    if (fabs(back) > fabs(v)) b -= 1u;
    b |= 1u;
  }
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// Raw bits of 8 consecutive elements (one 16-byte load for bf16, two for fp32).
template <bool BF16>
struct Chunk {
  uint4 q[BF16 ? 1 : 2];
};

template <bool BF16>
__device__ __forceinline__ void load_chunk(const void *x, int64_t i, Chunk<BF16> &c) {
  if (BF16) {
    c.q[0] = *(const uint4 *)((const uint16_t *)x + i);
  } else {
    c.q[0] = *(const uint4 *)((const float *)x + i);
    c.q[BF16 ? 0 : 1] = *(const uint4 *)((const float *)x + i + 4);
  }
}

template <bool BF16>
__device__ __forceinline__ void widen(const Chunk<BF16> &c, double v[8]) {
  if (BF16) {
    const uint32_t w[4] = {c.q[0].x, c.q[0].y, c.q[0].z, c.q[0].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = (double)bf16_to_f32((uint16_t)w[j]);
      v[2 * j + 1] = (double)bf16_to_f32((uint16_t)(w[j] >> 16));
    }
  } else {
    const uint4 a = c.q[0], b = c.q[BF16 ? 0 : 1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (double)__uint_as_float(w[j]);
  }
}

// One wave per row.  The row is walked in segments of NCH * 512 elements;
// lane l holds chunks l, l + 64, ... of a segment (8 elements each), all
// loaded before the first use so the segment is in flight at once.  A row of
// one segment stays in registers for the scaling pass; longer rows are read
// again segment by segment (from L2).
template <bool BF16, int NCH>
__global__ __launch_bounds__(RN_THREADS) void rmsnorm_kernel(const void *__restrict__ x,
                                                             const float *__restrict__ gamma, double eps, int d,
                                                             int64_t T, void *__restrict__ u) {
  constexpr int SEG = NCH * 64 * 8;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (RN_THREADS / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const int64_t row = t * d;
  const int nseg = (d + SEG - 1) / SEG;
  Chunk<BF16> ch[NCH];
  double s = 0.0;
  for (int sg = 0; sg < nseg; ++sg) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = sg * SEG + (lane + i * 64) * 8;
      if (c < d) load_chunk<BF16>(x, row + c, ch[i]);
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      if (sg * SEG + (lane + i * 64) * 8 < d) {
        double v[8];
        widen<BF16>(ch[i], v);
#pragma unroll
        for (int j = 0; j < 8; ++j) s = fma(v[j], v[j], s);
      }
    }
  }
  s = wave_sum_f64(s);  // every lane holds the same sum (each step adds the same pair)
  const double r = 1.0 / sqrt(s / (double)d + eps);
  for (int sg = 0; sg < nseg; ++sg) {
    if (nseg > 1) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int c = sg * SEG + (lane + i * 64) * 8;
        if (c < d) load_chunk<BF16>(x, row + c, ch[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = sg * SEG + (lane + i * 64) * 8;
      if (c >= d) continue;
      double v[8];
      widen<BF16>(ch[i], v);
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
}

template <bool BF16>
static void launch_rmsnorm_t(const moe_dims &dm, int64_t T, const void *x, const float *gamma, double eps, void *u,
                             hipStream_t st) {
  const int need = (dm.d_model + 511) / 512;  // chunks per lane for a single segment
  const dim3 g((unsigned)((T + RN_THREADS / 64 - 1) / (RN_THREADS / 64)));
  const int d = dm.d_model;
  // at most 16 (bf16) or 8 (fp32) chunks per lane, so the segment fits in registers
  if (need <= 2) rmsnorm_kernel<BF16, 2><<<g, RN_THREADS, 0, st>>>(x, gamma, eps, d, T, u);
  else if (need <= 4) rmsnorm_kernel<BF16, 4><<<g, RN_THREADS, 0, st>>>(x, gamma, eps, d, T, u);
  else if (need <= 8 || !BF16) rmsnorm_kernel<BF16, 8><<<g, RN_THREADS, 0, st>>>(x, gamma, eps, d, T, u);
  else rmsnorm_kernel<BF16, 16><<<g, RN_THREADS, 0, st>>>(x, gamma, eps, d, T, u);
}

hipError_t launch_rmsnorm(const moe_dims &dm, int64_t T, const void *x, const float *gamma, double eps, void *u,
                          hipStream_t st) {
  if (dm.dtype == MOE_BF16)
    launch_rmsnorm_t<true>(dm, T, x, gamma, eps, u, st);
  else
    launch_rmsnorm_t<false>(dm, T, x, gamma, eps, u, st);
  return hipGetLastError();
}
