// Combine: out[t,:] = y_shared[t,:] + sum_{j<k} w[t,j] * y_rows[token_row[t,j], :]
// accumulated in fp32 in slot order (start from 0 when there is no shared term).
//
// Source: "Shared Expert" (How it works: the shared output is added to the
// scatter-sum of routed expert outputs; Overview and Watch-outs: coefficient
// exactly 1, no gate and no 1/N_s; Official code: no residual inside the
// layer).  The scatter-sum is done as a gather per token so that the order of
// the additions is fixed and the result deterministic.
#include "common.h"

#define CB_MAXK 16

// KM: top_k rounded up to 1, 2, 4, 8 or 16 (slots j >= k are predicated off)
template <bool OUT_BF16, int KM>
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y_rows, const float *__restrict__ y_sh,
                                                      const float *__restrict__ topk_w,
                                                      const int32_t *__restrict__ token_row, int64_t T, int d, int k,
                                                      void *__restrict__ out) {
  const int64_t t = blockIdx.x;
  __shared__ int64_t rows[CB_MAXK];
  __shared__ float gw[CB_MAXK];
  if (threadIdx.x < CB_MAXK) {
    const bool slot = (int)threadIdx.x < k;
    rows[threadIdx.x] = slot ? (int64_t)token_row[t * k + threadIdx.x] : -1;
    gw[threadIdx.x] = slot ? topk_w[t * k + threadIdx.x] : 0.f;
  }
  __syncthreads();
  const int64_t R = T * k;
  for (int c = threadIdx.x * 4; c < d; c += 256 * 4) {
    // every row of the token is loaded before the first addition, so the k
    // loads are in flight together; the additions then run in slot order
    float4 y[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      const int64_t r = rows[j];        // -1 past the token's k slots
      const bool ok = r >= 0 && r < R;  // an invalid caller row contributes nothing
      const float4 v = *(const float4 *)(y_rows + (ok ? r : 0) * d + c);
      y[j] = make_float4(ok ? v.x : 0.f, ok ? v.y : 0.f, ok ? v.z : 0.f, ok ? v.w : 0.f);
    }
    float4 acc = y_sh ? *(const float4 *)(y_sh + t * d + c) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j < k) {
        const float g = gw[j];
        acc.x = fmaf(g, y[j].x, acc.x);
        acc.y = fmaf(g, y[j].y, acc.y);
        acc.z = fmaf(g, y[j].z, acc.z);
        acc.w = fmaf(g, y[j].w, acc.w);
      }
    }
    if (OUT_BF16) {
      uint16_t *o = (uint16_t *)out + t * d + c;
      uint2 pk;
      pk.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
      pk.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
      *(uint2 *)o = pk;
    } else {
      *(float4 *)((float *)out + t * d + c) = acc;
    }
  }
}

template <bool OUT_BF16, int KM>
static void launch_combine_k(const moe_dims &dm, int64_t T, const float *y_rows, const float *y_sh,
                             const float *topk_w, const int32_t *token_row, void *out, hipStream_t st) {
  combine_kernel<OUT_BF16, KM><<<dim3((unsigned)T), 256, 0, st>>>(y_rows, y_sh, topk_w, token_row, T, dm.d_model,
                                                                  dm.top_k, out);
}

template <bool OUT_BF16>
static void launch_combine_t(const moe_dims &dm, int64_t T, const float *y_rows, const float *y_sh,
                             const float *topk_w, const int32_t *token_row, void *out, hipStream_t st) {
  const int k = dm.top_k;
  if (k <= 1) launch_combine_k<OUT_BF16, 1>(dm, T, y_rows, y_sh, topk_w, token_row, out, st);
  else if (k <= 2) launch_combine_k<OUT_BF16, 2>(dm, T, y_rows, y_sh, topk_w, token_row, out, st);
  else if (k <= 4) launch_combine_k<OUT_BF16, 4>(dm, T, y_rows, y_sh, topk_w, token_row, out, st);
  else if (k <= 8) launch_combine_k<OUT_BF16, 8>(dm, T, y_rows, y_sh, topk_w, token_row, out, st);
  else launch_combine_k<OUT_BF16, CB_MAXK>(dm, T, y_rows, y_sh, topk_w, token_row, out, st);
}

hipError_t launch_combine(const moe_dims &dm, int64_t T, const float *y_rows, const float *y_sh, const float *topk_w,
                          const int32_t *token_row, void *out, hipStream_t st) {
  if (dm.out_dtype == MOE_BF16)
    launch_combine_t<true>(dm, T, y_rows, y_sh, topk_w, token_row, out, st);
  else
    launch_combine_t<false>(dm, T, y_rows, y_sh, topk_w, token_row, out, st);
  return hipGetLastError();
}
