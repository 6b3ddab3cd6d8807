// Combine: out[t,:] = y_shared[t,:] + sum_{j<k} w[t,j] * y_rows[token_row[t,j], :]
// accumulated in fp32 in slot order (start from 0 when there is no shared term),
// then, for the pre-norm block, plus the raw block input x[t,:].
//
// Source: "Shared Expert" (How it works: the shared output is added to the
// scatter-sum of routed expert outputs, and eq. 12's residual is added at
// block level; Overview and Watch-outs: coefficient exactly 1, no gate and no
// 1/N_s; Official code: no residual inside MoE.forward).  The scatter-sum is
// done as a gather per token so that the order of the additions is fixed and
// the result deterministic.  Slots dropped for capacity (token_row -1) add
// nothing.
#include "common.h"

#define CB_MAXK 16

// Y rows, Y_sh and the fp32 output are each touched once: non-temporal
// accesses keep them from displacing other lines (measured 0.885 ms against
// 0.963 ms at DeepSeek-V3 prefill).  One work-group of 512 threads per token
// (0.86 ms against 0.88 with 256).  Each thread owns NC float4 columns
// 2048 apart and issues the loads of all of them (every slot and the shared
// row) before its first addition, so a token's row is fetched in one round
// trip instead of one per 2048 columns: 0.78 ms against 0.86 at DeepSeek-V3
// prefill (6.0 TB/s), with 448, 384 and 1024 threads no better.  Top-k above
// 9 keeps two chunks in flight, which fits the registers without spilling.
// Rows of at most 2048 columns have a single chunk: they take NC = 1, since
// registers held for absent chunks only cut occupancy (at d = 2048 the
// four-chunk kernel took 0.12 against 0.094 ms, at d = 128 three times as long).
__device__ __forceinline__ float4 load_once(const float *p) {
  const f32x4_t v = __builtin_nontemporal_load((const f32x4_t *)p);
  return make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store_once(float4 a, float *p) {
  const f32x4_t v = {a.x, a.y, a.z, a.w};
  __builtin_nontemporal_store(v, (f32x4_t *)p);
}

// KM: top_k rounded up to 0, 1, 2, 4, 8 or 16 (slots j >= k are predicated off;
// 0 = dense layer, shared term only).  RES: 0 no residual, 1 fp32, 2 bf16 x.
// WIDE: rows of more than 2048 columns (several chunks per thread).
template <bool OUT_BF16, int KM, int RES, bool WIDE>
__global__ __launch_bounds__(512) void combine_kernel(const float *__restrict__ y_rows, const float *__restrict__ y_sh,
                                                      const float *__restrict__ topk_w,
                                                      const int32_t *__restrict__ token_row,
                                                      const void *__restrict__ resid, int64_t T, int d, int k,
                                                      void *__restrict__ out) {
  const int64_t t = blockIdx.x;
  __shared__ int64_t rows[CB_MAXK];
  __shared__ float gw[CB_MAXK];
  if (KM > 0 && threadIdx.x < CB_MAXK) {
    const bool slot = (int)threadIdx.x < k;
    rows[threadIdx.x] = slot ? (int64_t)token_row[t * k + threadIdx.x] : -1;
    gw[threadIdx.x] = slot ? topk_w[t * k + threadIdx.x] : 0.f;
  }
  __syncthreads();
  const int64_t R = T * k;
  constexpr int NC = !WIDE ? 1 : (KM + 1) * 4 <= 40 ? 4 : 2;  // float4 chunks per thread per pass
  for (int c0 = threadIdx.x * 4; c0 < d; c0 += 512 * 4 * NC) {
    float4 y[NC][KM > 0 ? KM : 1];
    float4 acc[NC];
    float4 xf[RES == 1 ? NC : 1];  // the residual row's chunks, loaded with the rest
    uint2 xb[RES == 2 ? NC : 1];
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const int c = c0 + cc * 2048;
      if (c < d) {
#pragma unroll
        for (int j = 0; j < KM; ++j) {
          const int64_t r = rows[j];        // -1 past the token's k slots or for a dropped pair
          const bool ok = r >= 0 && r < R;  // an invalid row contributes nothing
          const float4 v = load_once(y_rows + (ok ? r : 0) * d + c);
          y[cc][j] = make_float4(ok ? v.x : 0.f, ok ? v.y : 0.f, ok ? v.z : 0.f, ok ? v.w : 0.f);
        }
        acc[cc] = y_sh ? load_once(y_sh + t * d + c) : make_float4(0.f, 0.f, 0.f, 0.f);
        if (RES == 1) xf[cc] = *(const float4 *)((const float *)resid + t * d + c);
        if (RES == 2) xb[cc] = *(const uint2 *)((const uint16_t *)resid + t * d + c);
      }
    }
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      const int c = c0 + cc * 2048;
      if (c >= d) continue;
      float4 a = acc[cc];
#pragma unroll
      for (int j = 0; j < KM; ++j) {
        if (j < k) {
          const float g = gw[j];
          a.x = fmaf(g, y[cc][j].x, a.x);
          a.y = fmaf(g, y[cc][j].y, a.y);
          a.z = fmaf(g, y[cc][j].z, a.z);
          a.w = fmaf(g, y[cc][j].w, a.w);
        }
      }
      if (RES == 1) {
        const float4 x = xf[cc];
        a = make_float4(x.x + a.x, x.y + a.y, x.z + a.z, x.w + a.w);
      } else if (RES == 2) {
        const uint2 x = xb[cc];
        a.x = bf16_to_f32((uint16_t)x.x) + a.x;
        a.y = bf16_to_f32((uint16_t)(x.x >> 16)) + a.y;
        a.z = bf16_to_f32((uint16_t)x.y) + a.z;
        a.w = bf16_to_f32((uint16_t)(x.y >> 16)) + a.w;
      }
      if (OUT_BF16) {
        uint16_t *o = (uint16_t *)out + t * d + c;
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(a.x) | ((uint32_t)f32_to_bf16(a.y) << 16);
        pk.y = (uint32_t)f32_to_bf16(a.z) | ((uint32_t)f32_to_bf16(a.w) << 16);
        *(uint2 *)o = pk;
      } else {
        store_once(a, (float *)out + t * d + c);
      }
    }
  }
}

struct CombineCall {
  const float *y_rows, *y_sh, *topk_w;
  const int32_t *token_row;
  const void *resid;
  void *out;
};

template <bool OUT_BF16, int KM, int RES>
static void launch_combine_k(const moe_dims &dm, int64_t T, const CombineCall &c, hipStream_t st) {
  if (dm.d_model > 2048)
    combine_kernel<OUT_BF16, KM, RES, true><<<dim3((unsigned)T), 512, 0, st>>>(c.y_rows, c.y_sh, c.topk_w, c.token_row,
                                                                               c.resid, T, dm.d_model, dm.top_k, c.out);
  else
    combine_kernel<OUT_BF16, KM, RES, false><<<dim3((unsigned)T), 512, 0, st>>>(
        c.y_rows, c.y_sh, c.topk_w, c.token_row, c.resid, T, dm.d_model, dm.top_k, c.out);
}

template <bool OUT_BF16, int RES>
static void launch_combine_r(const moe_dims &dm, int64_t T, const CombineCall &c, hipStream_t st) {
  const int k = dm.top_k;
  if (k <= 0) launch_combine_k<OUT_BF16, 0, RES>(dm, T, c, st);
  else if (k <= 1) launch_combine_k<OUT_BF16, 1, RES>(dm, T, c, st);
  else if (k <= 2) launch_combine_k<OUT_BF16, 2, RES>(dm, T, c, st);
  else if (k <= 4) launch_combine_k<OUT_BF16, 4, RES>(dm, T, c, st);
  else if (k <= 8) launch_combine_k<OUT_BF16, 8, RES>(dm, T, c, st);
  else launch_combine_k<OUT_BF16, CB_MAXK, RES>(dm, T, c, st);
}

template <bool OUT_BF16>
static void launch_combine_t(const moe_dims &dm, int64_t T, const CombineCall &c, hipStream_t st) {
  if (!c.resid) launch_combine_r<OUT_BF16, 0>(dm, T, c, st);
  else if (dm.dtype == MOE_BF16) launch_combine_r<OUT_BF16, 2>(dm, T, c, st);
  else launch_combine_r<OUT_BF16, 1>(dm, T, c, st);
}

hipError_t launch_combine(const moe_dims &dm, int64_t T, const float *y_rows, const float *y_sh, const float *topk_w,
                          const int32_t *token_row, const void *resid, void *out, hipStream_t st) {
  const CombineCall c{y_rows, y_sh, topk_w, token_row, resid, out};
  if (dm.out_dtype == MOE_BF16)
    launch_combine_t<true>(dm, T, c, st);
  else
    launch_combine_t<false>(dm, T, c, st);
  return hipGetLastError();
}
