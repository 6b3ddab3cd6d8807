// Router: logits l[t,e] = u[t,:] . w_router[e,:] (+ b_e), with a per-logit error bound.
//
// Source: "What is an 'expert', really?" (panel 2: a linear layer scores the
// experts); "Shared Expert" (How it works: the N_r centroids).  The ranking
// key is the exact real logit of the stored inputs; the logits computed here
// are approximations with a rigorous bound, which the top-k kernel uses to
// decide when a comparison must be settled exactly.
//
// bf16 inputs: bf16 x bf16 products are exact in fp32; the matrix cores sum
// chunks of ROUTER_CHUNK products in fp32 and the chunk sums are added in
// fp64.  Error bound per logit (any summation order inside the chunk, unit
// roundoff taken as 2^-22, twice truncation's 2^-23):
//     |L - l| <= (CHUNK * 2^-22 + (d / CHUNK + 2) * 2^-52) * ||u_t|| ||c_e|| + 2^-50 |L| + d 2^-120
// using sum |u_i c_ei| <= ||u_t|| ||c_e|| (Cauchy-Schwarz).  For small token
// counts the reduction is split into S slices of whole chunks whose fp64
// partial sums are added in slice order afterwards: every logit then passes
// through at most d / CHUNK / S + S fp64 additions, never more than the
// d / CHUNK + 2 the bound allows for.
// fp32 inputs: products are exact in fp64 and summed in fp64:
//     |L - l| <= (d + 2) * 2^-52 * ||u_t|| ||c_e|| + 2^-50 |L| + d 2^-120.
#include "common.h"

#define ROUTER_CHUNK 64
#define RT_BM 64
#define RT_BN 64
#define RT_BK 64
#define RT_LDS_STRIDE (RT_BK + 8)  // bf16 elements per LDS row (16-byte pad)

// ------------------------------------------------------------------ row norms
// out[r] = sum_i x[r,i]^2 in fp64 (one wave per row), or its square root (ROOT).
template <bool BF16, bool ROOT = false>
__global__ __launch_bounds__(256) void row_norm2_kernel(const void *__restrict__ x, int64_t rows, int d,
                                                        double *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  double s = 0.0;
  if (BF16) {
    const uint16_t *p = (const uint16_t *)x + r * d;
    for (int i = lane * 8; i < d; i += 512) {
      uint4 v = *(const uint4 *)(p + i);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        double a = (double)__uint_as_float(w4[q] << 16);
        double b = (double)__uint_as_float(w4[q] & 0xffff0000u);
        s += a * a + b * b;
      }
    }
  } else {
    const float *p = (const float *)x + r * d;
    for (int i = lane; i < d; i += 64) {
      double a = (double)p[i];
      s += a * a;
    }
  }
  s = wave_sum_f64(s);
  if (lane == 0) out[r] = ROOT ? sqrt(s) : s;
}

// -------------------------------------------------------- bf16 logits (MFMA)
// Work-group tile: 64 tokens x 64 experts, 4 waves in a 2 x 2 grid, each wave
// 32 x 32 = 2 x 2 MFMA 16x16x32 tiles.
// blockIdx.z selects a slice of kps k-tiles; with one slice the logits (bias
// added) are written, otherwise slice s writes its fp64 partial sums to
// logits + s * T * E and router_reduce_kernel adds them.
__global__ __launch_bounds__(256) void router_logits_bf16_kernel(const uint16_t *__restrict__ u,
                                                                 const uint16_t *__restrict__ w,
                                                                 const float *__restrict__ bias, int64_t T,
                                                                 int E, int d, int kps, double *__restrict__ logits) {
  __shared__ __attribute__((aligned(16))) uint16_t As[RT_BM * RT_LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[RT_BN * RT_LDS_STRIDE];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int64_t t0 = (int64_t)blockIdx.x * RT_BM;
  const int e0 = blockIdx.y * RT_BN;

  f32x4_t acc[2][2];
  double acc64[2][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) acc64[i][j][r] = 0.0;
    }

  // each thread moves 2 chunks of 16 bytes of A and of B per k-tile
  const uint16_t *ap[2];
  const uint16_t *bp[2];
  bool aok[2], bok[2];
  int lrow[2], lcol[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = tid + 256 * q;
    lrow[q] = c >> 3;
    lcol[q] = (c & 7) * 8;
    aok[q] = t0 + lrow[q] < T;
    bok[q] = e0 + lrow[q] < E;
    ap[q] = u + (aok[q] ? (t0 + lrow[q]) : 0) * (int64_t)d + lcol[q];
    bp[q] = w + (int64_t)(bok[q] ? (e0 + lrow[q]) : 0) * d + lcol[q];
  }
  const int nk = d / RT_BK;
  const int kt0 = blockIdx.z * kps, kt1 = min(nk, kt0 + kps);
  const int chunk_tiles = ROUTER_CHUNK / RT_BK;
  // the next k-tile's loads are in flight while the current one is multiplied
  uint4 av[2], bv[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    av[q] = keep_or_zero(aok[q], *(const uint4 *)(ap[q] + kt0 * RT_BK));  // pointers clamped in bounds
    bv[q] = keep_or_zero(bok[q], *(const uint4 *)(bp[q] + kt0 * RT_BK));
  }
  for (int kt = kt0; kt < kt1; ++kt) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      *(uint4 *)&As[lrow[q] * RT_LDS_STRIDE + lcol[q]] = av[q];
      *(uint4 *)&Bs[lrow[q] * RT_LDS_STRIDE + lcol[q]] = bv[q];
    }
    __syncthreads();
    const int kn = min(kt + 1, kt1 - 1);  // the last trip re-loads its own tile (in bounds, unused)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      av[q] = keep_or_zero(aok[q], *(const uint4 *)(ap[q] + kn * RT_BK));
      bv[q] = keep_or_zero(bok[q], *(const uint4 *)(bp[q] + kn * RT_BK));
    }
#pragma unroll
    for (int kk = 0; kk < RT_BK / 32; ++kk) {
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = as_bf16x8(*(const uint4 *)&As[(wm * 32 + i * 16 + (lane & 15)) * RT_LDS_STRIDE + kk * 32 +
                                             (lane >> 4) * 8]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = as_bf16x8(*(const uint4 *)&Bs[(wn * 32 + j * 16 + (lane & 15)) * RT_LDS_STRIDE + kk * 32 +
                                             (lane >> 4) * 8]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if ((kt + 1) % chunk_tiles == 0 || kt + 1 == kt1) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc64[i][j][r] += (double)acc[i][j][r];
          acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
  }
  // D layout of a 16x16 tile: lane holds rows 4*(lane/16)+r, column lane%16
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + wn * 32 + j * 16 + (lane & 15);
      if (e >= E) continue;
      const bool whole = gridDim.z == 1;
      const double b = (whole && bias) ? (double)bias[e] : 0.0;
      double *dst = logits + (whole ? 0 : (int64_t)blockIdx.z * T * E);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + wm * 32 + i * 16 + (lane >> 4) * 4 + r;
        if (t < T) dst[t * E + e] = acc64[i][j][r] + b;
      }
    }
}

// logits[t, e] = sum over slices s = 0, 1, ... of part[s][t][e] (in this
// order) + b_e.
__global__ __launch_bounds__(256) void router_reduce_kernel(const double *__restrict__ part, int S, int64_t n, int E,
                                                            const float *__restrict__ bias, double *__restrict__ logits) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  // loads in batches of 8 (in flight together), additions in slice order
  double s = 0.0;
  for (int k0 = 0; k0 < S; k0 += 8) {
    double v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = k0 + q < S ? part[(int64_t)(k0 + q) * n + i] : 0.0;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (k0 + q < S) s = (k0 + q == 0) ? v[q] : s + v[q];
  }
  logits[i] = s + (bias ? (double)bias[i % E] : 0.0);
}

// ------------------------------------------------------ fp32 logits (fp64 VALU)
// 16 tokens x 16 experts per work-group, one logit per thread, exact products.
__global__ __launch_bounds__(256) void router_logits_f32_kernel(const float *__restrict__ u,
                                                                const float *__restrict__ w,
                                                                const float *__restrict__ bias, int64_t T,
                                                                int E, int d, double *__restrict__ logits) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t t = (int64_t)blockIdx.x * 16 + ty;
  const int e = blockIdx.y * 16 + tx;
  double acc = 0.0;
  for (int k0 = 0; k0 < d; k0 += 64) {
    for (int c = threadIdx.x; c < 16 * 64; c += 256) {
      const int r = c >> 6, col = c & 63;
      const int64_t tr = (int64_t)blockIdx.x * 16 + r;
      const int er = blockIdx.y * 16 + r;
      As[r][col] = tr < T ? u[tr * d + k0 + col] : 0.f;
      Bs[r][col] = er < E ? w[(int64_t)er * d + k0 + col] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 64; ++kk) acc += (double)As[ty][kk] * (double)Bs[tx][kk];
    __syncthreads();
  }
  if (t < T && e < E) logits[t * E + e] = acc + (bias ? (double)bias[e] : 0.0);
}

hipError_t launch_router_logits(const moe_dims &dm, int64_t T, const void *u, const void *w_router,
                                const float *bias, const WsLayout &L, char *ws, hipStream_t st) {
  const int E = dm.n_routed, d = dm.d_model;
  double *logits = (double *)(ws + L.logits);
  double *un2 = (double *)(ws + L.unorm2);
  double *wn = (double *)(ws + L.wnorm);
  if (dm.dtype == MOE_BF16) {
    row_norm2_kernel<true><<<dim3((unsigned)((T + 3) / 4)), 256, 0, st>>>(u, T, d, un2);
    row_norm2_kernel<true, true><<<dim3((unsigned)((E + 3) / 4)), 256, 0, st>>>(w_router, E, d, wn);
    const int nk = d / RT_BK;
    const int S = router_splits(dm, T);
    const int kps = (nk + S - 1) / S;
    dim3 grid((unsigned)((T + RT_BM - 1) / RT_BM), (unsigned)((E + RT_BN - 1) / RT_BN), (unsigned)S);
    double *part = S > 1 ? (double *)(ws + L.logit_part) : logits;
    router_logits_bf16_kernel<<<grid, 256, 0, st>>>((const uint16_t *)u, (const uint16_t *)w_router, bias, T, E, d,
                                                    kps, part);
    if (S > 1) {
      const int64_t n = T * E;
      router_reduce_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(part, S, n, E, bias, logits);
    }
  } else {
    row_norm2_kernel<false><<<dim3((unsigned)((T + 3) / 4)), 256, 0, st>>>(u, T, d, un2);
    row_norm2_kernel<false, true><<<dim3((unsigned)((E + 3) / 4)), 256, 0, st>>>(w_router, E, d, wn);
    dim3 grid((unsigned)((T + 15) / 16), (unsigned)((E + 15) / 16));
    router_logits_f32_kernel<<<grid, 256, 0, st>>>((const float *)u, (const float *)w_router, bias, T, E, d, logits);
  }
  return hipGetLastError();
}

// Coefficient of ||u|| ||c|| in the logit error bound (see the file header).
double router_bound_coeff(const moe_dims &dm) {
  const double d = dm.d_model;
  if (dm.dtype == MOE_BF16) return ROUTER_CHUNK * 0x1p-22 + (d / ROUTER_CHUNK + 2.0) * 0x1p-52;
  return (d + 2.0) * 0x1p-52;
}
