// Grouped expert GEMMs in fp32 (fp32 workloads; plain VALU FMA, fp32 accumulate).
//
// Same grouping and tile scheduling as the bf16 path (routed groups from the
// permutation, the shared MLP as group N_r over all tokens), with 32-row
// tiles: at the small batches of the fp32 workloads the tiles cannot fill the
// chip, and each thread's serial chain of FMAs sets a tile's time, so tiles of
// half the height give twice the work-groups and half the chain (the tiny
// layer: gate/up 12.8 against 16.6 us, the layer 0.055 against 0.061 ms;
// 16-row tiles were no faster).  Source: "Shared Expert" (How it works: SwiGLU; Official code: fused
// shared MLP of width N_s*f on the full batch).
#include <algorithm>

#include "common.h"

#define F_BM 32
#define F_RM (F_BM / 16)  // rows per thread
#define F_BN 64
#define F_BK 16
#define F_BM_IDX 1  // moe_bm_of(1) == 32

struct GemmArgsF {
  const float *A, *A_sh;
  const int32_t *row_token, *offsets, *tile_off;
  const float *B1, *B3, *B1s, *B3s;
  float *C, *C_sh;
  int64_t T;
  int E, K, K_sh, N, N_sh, has_shared, nt_r, nt_s;
};

template <bool GATEUP>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(GemmArgsF a) {
  __shared__ float As[F_BM][F_BK + 1];
  __shared__ float Bs[F_BN][F_BK + 1];
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int mt_r = a.tile_off[a.E];
  const int mt_s = a.tile_off[a.E + 1] - mt_r;
  const int64_t tiles_r = (int64_t)mt_r * a.nt_r;
  const int64_t total = tiles_r + (int64_t)mt_s * a.nt_s;
  const int64_t tile = blockIdx.x;
  if (tile >= total) return;
  bool shared;
  int g, nt, K, N, valid;
  int64_t rb;
  if (tile < tiles_r) {
    shared = false;
    const int mt = (int)(tile / a.nt_r);
    nt = (int)(tile % a.nt_r);
    int lo = 0, hi = a.E - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.tile_off[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    g = lo;
    const int m0 = (mt - a.tile_off[g]) * F_BM;
    valid = min(F_BM, a.offsets[g + 1] - a.offsets[g] - m0);
    rb = (int64_t)a.offsets[g] + m0;
    K = a.K;
    N = a.N;
  } else {
    shared = true;
    const int64_t ts = tile - tiles_r;
    const int mt = (int)(ts / a.nt_s);
    nt = (int)(ts % a.nt_s);
    g = a.E;
    rb = (int64_t)mt * F_BM;
    valid = (int)min((int64_t)F_BM, a.T - rb);
    K = a.K_sh;
    N = a.N_sh;
  }
  const float *Abase = shared ? a.A_sh : a.A;
  // loader: F_RM A and 4 B elements per thread per k-tile
  const float *ap[4];
  const float *bp[4];
  bool bok[4];
  int lr[4], lc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = tid + 256 * q;
    lr[q] = c >> 4;
    lc[q] = c & 15;
    const int r = min(lr[q] % F_BM, valid - 1);
    const int64_t arow = (GATEUP && !shared) ? (int64_t)a.row_token[rb + r] : rb + r;
    ap[q] = Abase + arow * K + lc[q];
    int n;
    const float *bw;
    if (GATEUP) {
      const int half = lr[q] >> 5;
      n = nt * (F_BN / 2) + (lr[q] & 31);
      bw = shared ? (half ? a.B3s : a.B1s) : ((half ? a.B3 : a.B1) + (int64_t)g * N * K);
    } else {
      n = nt * F_BN + lr[q];
      bw = shared ? a.B1s : (a.B1 + (int64_t)g * N * K);
    }
    bok[q] = n < N;
    bp[q] = bw + (int64_t)(bok[q] ? n : 0) * K + lc[q];
  }
  int bcol[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) bcol[j] = GATEUP ? ((j >> 1) * 32 + tx * 2 + (j & 1)) : (tx * 4 + j);
  float acc[F_RM][4] = {};
  // the next k-tile's elements are loaded into registers while the current
  // one is multiplied (the same additions in the same order)
  float na[4], nb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    na[q] = q < F_RM ? ap[q][0] : 0.f;
    nb[q] = bok[q] ? bp[q][0] : 0.f;
  }
  for (int k0 = 0; k0 < K; k0 += F_BK) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (q < F_RM) As[lr[q]][lc[q]] = na[q];
      Bs[lr[q]][lc[q]] = nb[q];
    }
    __syncthreads();
    if (k0 + F_BK < K) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        na[q] = q < F_RM ? ap[q][k0 + F_BK] : 0.f;
        nb[q] = bok[q] ? bp[q][k0 + F_BK] : 0.f;
      }
    }
#pragma unroll
    for (int kk = 0; kk < F_BK; ++kk) {
      float av[F_RM], bv[4];
#pragma unroll
      for (int i = 0; i < F_RM; ++i) av[i] = As[ty * F_RM + i][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[bcol[j]][kk];
#pragma unroll
      for (int i = 0; i < F_RM; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  float *C = shared ? a.C_sh : a.C;
#pragma unroll
  for (int i = 0; i < F_RM; ++i) {
    const int row = ty * F_RM + i;
    if (row >= valid) continue;
    if (GATEUP) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = nt * (F_BN / 2) + tx * 2 + j;
        if (n < N) {
          const float gt = acc[i][j];
          C[(rb + row) * N + n] = gt / (1.0f + expf(-gt)) * acc[i][j + 2];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = nt * F_BN + tx * 4 + j;
        if (n < N) C[(rb + row) * N + n] = acc[i][j];
      }
    }
  }
}

// Work-groups of each launch below: 64-row tiles times column tiles.
static void f32_grids(const moe_dims &dm, int64_t T, int64_t *grid1, int64_t *grid2) {
  const int E = dm.n_routed, d = dm.d_model, f = dm.d_ff, fs = dm.d_ff_shared;
  const int64_t R = T * dm.top_k;
  const int64_t mtb = (R + F_BM - 1) / F_BM + std::min<int64_t>(E, R);
  const int64_t mts = fs > 0 ? (T + F_BM - 1) / F_BM : 0;
  *grid1 = mtb * ((f + F_BN / 2 - 1) / (F_BN / 2)) + mts * (fs > 0 ? (fs + F_BN / 2 - 1) / (F_BN / 2) : 1);
  *grid2 = (mtb + mts) * ((d + F_BN - 1) / F_BN);
}

int64_t ffn_f32_max_workgroups(const moe_dims &dm, int64_t T) {
  int64_t g1, g2;
  f32_grids(dm, T, &g1, &g2);
  return std::max(g1, g2);
}

hipError_t launch_ffn_f32(const moe_dims &dm, int64_t T, const void *u, const moe_weights &w, const int32_t *offsets,
                          const int32_t *row_token, float *y_rows, float *y_sh, const WsLayout &L, char *ws,
                          hipStream_t st, hipEvent_t ev_mid) {
  const int E = dm.n_routed, d = dm.d_model, f = dm.d_ff, fs = dm.d_ff_shared;
  const int64_t R = T * dm.top_k;
  const int hs = fs > 0 ? 1 : 0;
  const int32_t *tile_off = (const int32_t *)(ws + L.tile_off) + F_BM_IDX * (E + 2);
  float *H = (float *)(ws + L.h);
  float *Hs = (float *)(ws + L.h_sh);
  const int64_t mtb = (R + F_BM - 1) / F_BM + std::min<int64_t>(E, R);
  const int64_t mts = hs ? (T + F_BM - 1) / F_BM : 0;
  GemmArgsF g1{(const float *)u, (const float *)u, row_token, offsets, tile_off, (const float *)w.w1,
               (const float *)w.w3, (const float *)w.w1s, (const float *)w.w3s, H, Hs, T, E, d, d, f, fs, hs,
               (f + F_BN / 2 - 1) / (F_BN / 2), hs ? (fs + F_BN / 2 - 1) / (F_BN / 2) : 1};
  int64_t grid1, grid2;
  f32_grids(dm, T, &grid1, &grid2);
  grouped_gemm_f32_kernel<true><<<dim3((unsigned)grid1), 256, 0, st>>>(g1);
  if (ev_mid) (void)hipEventRecord(ev_mid, st);
  GemmArgsF g2{H, Hs, nullptr, offsets, tile_off, (const float *)w.w2, nullptr, (const float *)w.w2s, nullptr,
               y_rows, y_sh, T, E, f, fs, d, d, hs, (d + F_BN - 1) / F_BN, (d + F_BN - 1) / F_BN};
  grouped_gemm_f32_kernel<false><<<dim3((unsigned)grid2), 256, 0, st>>>(g2);
  return hipGetLastError();
}
