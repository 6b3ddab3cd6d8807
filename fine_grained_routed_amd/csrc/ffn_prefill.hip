// Grouped expert GEMMs on bf16 matrix cores (prefill path).
//
// Source: "Shared Expert" (How it works: SwiGLU expert W2(SiLU(W1 u) * W3 u);
// Official code: the N_s shared experts form one MLP of width N_s*f applied to
// the full token batch and added with coefficient 1); "Shared and
// fine-grained experts" (Researcher level, Systems limits: many small experts
// are run as grouped GEMMs).
//
// Groups 0..N_r-1 are the routed experts: group g owns the permuted rows
// offsets[g]..offsets[g+1]-1.  Group N_r is the shared MLP over all T tokens
// in token order (it is treated as one more expert every token enters).
//
// gate/up: H[r, n] = SiLU(sum_i A[r,i] W1_g[n,i]) * (sum_i A[r,i] W3_g[n,i]),
//          A[r,:] = u[row_token[r], :]  (u[r,:] for the shared group), H in bf16
// down:    Y[r, n] = sum_i H[r,i] W2_g[n,i], fp32
//
// Tiles: 128 rows x 128 columns x 64 deep, 4 waves in a 2 x 2 grid, each wave
// 64 x 64 as 4 x 4 MFMA 16x16x32 tiles; for gate/up the 128 B-columns are 64
// gate columns followed by the same 64 up columns so that each lane holds the
// gate and up accumulators of the same output element.  LDS double buffer,
// register-staged global loads.  The grid covers an upper bound of the tile
// count; each work-group reads the device-side tile prefixes, so no host sync
// is needed.  Work-groups are remapped so that each XCD (8 per chip, dispatched
// round-robin) walks a contiguous range of tiles: consecutive tiles share an
// expert's A rows and weight panels, which then stay in that XCD's L2.
#include <algorithm>

#include "common.h"

#define PF_BM 128
#define PF_BN 128
#define PF_BK 64
#define PF_LDS (PF_BK + 8)  // padded row, bf16 elements
#define PF_BM_IDX 3         // moe_bm_of(3) == 128

struct GemmArgs {
  const uint16_t *A;         // gate/up: u [T, d]; down: H [R, f]
  const uint16_t *A_sh;      // gate/up: u;       down: H_sh [T, f_s]
  const int32_t *row_token;  // gate/up: permuted row -> token; down: unused
  const int32_t *offsets;    // [E + 1]
  const int32_t *tile_off;   // [E + 2] m-tile prefix for BM = 128
  const uint16_t *B1, *B3;   // routed: gate/up W1, W3 [E, N, K]; down W2 [E, N, K] (B3 unused)
  const uint16_t *B1s, *B3s; // shared
  void *C, *C_sh;            // gate/up: H bf16 [R, f], H_sh [T, f_s]; down: Y f32 [R, d], Y_sh [T, d]
  int64_t T;
  int E, K, K_sh, N, N_sh, has_shared;
  int nt_r, nt_s;            // n-tiles of a routed / the shared group
};

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

template <bool GATEUP>
__global__ __launch_bounds__(256, 2) void grouped_gemm_bf16_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][PF_BM * PF_LDS];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][PF_BN * PF_LDS];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;

  // ---- tile lookup (XCD-contiguous order)
  const int mt_r = a.tile_off[a.E];
  const int mt_s = a.tile_off[a.E + 1] - mt_r;
  const int64_t tiles_r = (int64_t)mt_r * a.nt_r;
  const int64_t total = tiles_r + (int64_t)mt_s * a.nt_s;
  const int64_t per = (total + 7) / 8;
  const int64_t slot = blockIdx.x >> 3;
  if (slot >= per) return;
  const int64_t tile = (int64_t)(blockIdx.x & 7) * per + slot;
  if (tile >= total) return;

  bool shared;
  int g, nt, K, N, valid;
  int64_t rb;  // first row of this tile in the group's row space
  if (tile < tiles_r) {
    shared = false;
    const int mt = (int)(tile / a.nt_r);
    nt = (int)(tile % a.nt_r);
    int lo = 0, hi = a.E - 1;  // largest g with tile_off[g] <= mt
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.tile_off[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    g = lo;
    const int m0 = (mt - a.tile_off[g]) * PF_BM;
    const int cnt = a.offsets[g + 1] - a.offsets[g];
    valid = min(PF_BM, cnt - m0);
    rb = (int64_t)a.offsets[g] + m0;
    K = a.K;
    N = a.N;
  } else {
    shared = true;
    const int64_t ts = tile - tiles_r;
    const int mt = (int)(ts / a.nt_s);
    nt = (int)(ts % a.nt_s);
    g = a.E;
    rb = (int64_t)mt * PF_BM;
    valid = (int)min((int64_t)PF_BM, a.T - rb);
    K = a.K_sh;
    N = a.N_sh;
  }

  // ---- per-thread global source pointers: 4 chunks of 16 B of A and of B
  const uint16_t *ap[4];
  const uint16_t *bp[4];
  bool bok[4];
  int lrow[4], lcol[4];
  const uint16_t *Abase = shared ? a.A_sh : a.A;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = tid + 256 * q;
    lrow[q] = c >> 3;
    lcol[q] = (c & 7) * 8;
    const int r = min(lrow[q], valid - 1);  // rows past the group are clamped, never stored
    int64_t arow;
    if (GATEUP && !shared) arow = a.row_token[rb + r];
    else arow = rb + r;
    ap[q] = Abase + arow * (int64_t)K + lcol[q];
    int n;
    const uint16_t *bw;
    if (GATEUP) {
      const int half = lrow[q] >> 6;  // 0: gate rows, 1: up rows
      n = nt * (PF_BN / 2) + (lrow[q] & 63);
      bw = shared ? (half ? a.B3s : a.B1s) : ((half ? a.B3 : a.B1) + (int64_t)g * N * K);
    } else {
      n = nt * PF_BN + lrow[q];
      bw = shared ? a.B1s : (a.B1 + (int64_t)g * N * K);
    }
    bok[q] = n < N;
    bp[q] = bw + (int64_t)(bok[q] ? n : 0) * K + lcol[q];
  }

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 ra[4], rbv[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    ra[q] = *(const uint4 *)(ap[q]);
    rbv[q] = keep_or_zero(bok[q], *(const uint4 *)(bp[q]));  // bp is clamped in bounds
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    *(uint4 *)&As[0][lrow[q] * PF_LDS + lcol[q]] = ra[q];
    *(uint4 *)&Bs[0][lrow[q] * PF_LDS + lcol[q]] = rbv[q];
  }
  __syncthreads();

  // B-row base of each wave column tile
  int brow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) brow[j] = GATEUP ? ((j >> 1) * 64 + wn * 32 + (j & 1) * 16) : (wn * 64 + j * 16);

  const int nk = K / PF_BK;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    // prefetch the next k-tile (the last iteration re-reads the current one;
    // its copy lands in the idle buffer and is never read)
    const int kn = min(kt + 1, nk - 1) * PF_BK;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ra[q] = *(const uint4 *)(ap[q] + kn);
      rbv[q] = keep_or_zero(bok[q], *(const uint4 *)(bp[q] + kn));
    }
#pragma unroll
    for (int kk = 0; kk < PF_BK / 32; ++kk) {
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = as_bf16x8(*(const uint4 *)&As[cur][(wm * 64 + i * 16 + (lane & 15)) * PF_LDS + kk * 32 + (lane >> 4) * 8]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = as_bf16x8(*(const uint4 *)&Bs[cur][(brow[j] + (lane & 15)) * PF_LDS + kk * 32 + (lane >> 4) * 8]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *(uint4 *)&As[cur ^ 1][lrow[q] * PF_LDS + lcol[q]] = ra[q];
      *(uint4 *)&Bs[cur ^ 1][lrow[q] * PF_LDS + lcol[q]] = rbv[q];
    }
    __syncthreads();
  }

  // ---- epilogue; D layout: lane holds rows 4*(lane/16)+r of column lane%16
  if (GATEUP) {
    uint16_t *C = (uint16_t *)(shared ? a.C_sh : a.C);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = nt * (PF_BN / 2) + wn * 32 + j * 16 + (lane & 15);
        if (n >= N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = wm * 64 + i * 16 + (lane >> 4) * 4 + r;
          if (row < valid) {
            const float h = silu_f(acc[i][j][r]) * acc[i][j + 2][r];
            C[(rb + row) * (int64_t)N + n] = f32_to_bf16(h);
          }
        }
      }
  } else {
    float *C = (float *)(shared ? a.C_sh : a.C);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = nt * PF_BN + wn * 64 + j * 16 + (lane & 15);
        if (n >= N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = wm * 64 + i * 16 + (lane >> 4) * 4 + r;
          if (row < valid) C[(rb + row) * (int64_t)N + n] = acc[i][j][r];
        }
      }
  }
}

// Upper bound of the number of 128-row m-tiles over the routed groups.
static int64_t mtile_bound(int64_t R, int E) { return (R + PF_BM - 1) / PF_BM + (int64_t)std::min<int64_t>(E, R); }

hipError_t launch_ffn_prefill_bf16(const moe_dims &dm, int64_t T, const void *u, const moe_weights &w,
                                   const int32_t *offsets, const int32_t *row_token, float *y_rows, float *y_sh,
                                   const WsLayout &L, char *ws, hipStream_t st, hipEvent_t ev_mid) {
  const int E = dm.n_routed, d = dm.d_model, f = dm.d_ff, fs = dm.d_ff_shared;
  const int64_t R = T * dm.top_k;
  const int hs = fs > 0 ? 1 : 0;
  const int32_t *tile_off = (const int32_t *)(ws + L.tile_off) + PF_BM_IDX * (E + 2);
  uint16_t *H = (uint16_t *)(ws + L.h);
  uint16_t *Hs = (uint16_t *)(ws + L.h_sh);
  const int64_t mt_sh = hs ? (T + PF_BM - 1) / PF_BM : 0;

  GemmArgs g1{};
  g1.A = (const uint16_t *)u;
  g1.A_sh = (const uint16_t *)u;
  g1.row_token = row_token;
  g1.offsets = offsets;
  g1.tile_off = tile_off;
  g1.B1 = (const uint16_t *)w.w1;
  g1.B3 = (const uint16_t *)w.w3;
  g1.B1s = (const uint16_t *)w.w1s;
  g1.B3s = (const uint16_t *)w.w3s;
  g1.C = H;
  g1.C_sh = Hs;
  g1.T = T;
  g1.E = E;
  g1.K = d;
  g1.K_sh = d;
  g1.N = f;
  g1.N_sh = fs;
  g1.has_shared = hs;
  g1.nt_r = (f + PF_BN / 2 - 1) / (PF_BN / 2);
  g1.nt_s = hs ? (fs + PF_BN / 2 - 1) / (PF_BN / 2) : 1;
  int64_t grid1 = mtile_bound(R, E) * g1.nt_r + mt_sh * g1.nt_s;
  grid1 = ((grid1 + 7) / 8) * 8;
  grouped_gemm_bf16_kernel<true><<<dim3((unsigned)grid1), 256, 0, st>>>(g1);
  if (ev_mid) (void)hipEventRecord(ev_mid, st);

  GemmArgs g2{};
  g2.A = H;
  g2.A_sh = Hs;
  g2.row_token = nullptr;
  g2.offsets = offsets;
  g2.tile_off = tile_off;
  g2.B1 = (const uint16_t *)w.w2;
  g2.B1s = (const uint16_t *)w.w2s;
  g2.C = y_rows;
  g2.C_sh = y_sh;
  g2.T = T;
  g2.E = E;
  g2.K = f;
  g2.K_sh = fs;
  g2.N = d;
  g2.N_sh = d;
  g2.has_shared = hs;
  g2.nt_r = (d + PF_BN - 1) / PF_BN;
  g2.nt_s = g2.nt_r;
  int64_t grid2 = mtile_bound(R, E) * g2.nt_r + mt_sh * g2.nt_s;
  grid2 = ((grid2 + 7) / 8) * 8;
  grouped_gemm_bf16_kernel<false><<<dim3((unsigned)grid2), 256, 0, st>>>(g2);
  return hipGetLastError();
}
