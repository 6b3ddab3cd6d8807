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

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ y_rows, const float *__restrict__ y_sh,
                                                      const float *__restrict__ topk_w,
                                                      const int32_t *__restrict__ token_row, int64_t T, int d, int k,
                                                      void *__restrict__ out) {
  const int64_t t = blockIdx.x;
  __shared__ int64_t rows[CB_MAXK];
  __shared__ float gw[CB_MAXK];
  if (threadIdx.x < k) {
    rows[threadIdx.x] = (int64_t)token_row[t * k + threadIdx.x];
    gw[threadIdx.x] = topk_w[t * k + threadIdx.x];
  }
  __syncthreads();
  for (int c = threadIdx.x * 4; c < d; c += 256 * 4) {
    float4 acc = y_sh ? *(const float4 *)(y_sh + t * d + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      if (rows[j] < 0 || rows[j] >= T * k) continue;  // invalid caller row: no contribution
      const float4 y = *(const float4 *)(y_rows + rows[j] * d + c);
      const float g = gw[j];
      acc.x = fmaf(g, y.x, acc.x);
      acc.y = fmaf(g, y.y, acc.y);
      acc.z = fmaf(g, y.z, acc.z);
      acc.w = fmaf(g, y.w, acc.w);
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

hipError_t launch_combine(const moe_dims &dm, int64_t T, const float *y_rows, const float *y_sh, const float *topk_w,
                          const int32_t *token_row, void *out, hipStream_t st) {
  if (dm.out_dtype == MOE_BF16)
    combine_kernel<true><<<dim3((unsigned)T), 256, 0, st>>>(y_rows, y_sh, topk_w, token_row, T, dm.d_model,
                                                            dm.top_k, out);
  else
    combine_kernel<false><<<dim3((unsigned)T), 256, 0, st>>>(y_rows, y_sh, topk_w, token_row, T, dm.d_model,
                                                             dm.top_k, out);
  return hipGetLastError();
}
