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
// Tiles: up to 256 rows x 256 B-columns x 64 deep per work-group; B-columns
// are 128 gate + the same 128 up columns (gate/up) or 256 output columns
// (down).  4 waves split the columns (1 x 4): each wave owns all 256 rows and
// 64 B-columns as 8 x 2 tiles of the 32x32x16 bf16 matrix-core instruction,
// 256 fp32 accumulators per lane.  A wave skips the 32-row sub-tiles past the
// group's last row, so a ragged tail costs in proportion to its rows.  Both
// operands are K-contiguous; LDS rows of 64 bf16 hold their 16-byte chunks
// XOR-swizzled by (row % 8) so that the 16-byte fragment reads of 8
// consecutive rows hit distinct banks.  Two LDS stages (128 KB) filled by
// direct global-to-LDS loads (global_load_lds_dwordx4: each lane's 16 bytes
// land at LDS base + 16 * lane, so the swizzle is applied by choosing which
// global chunk each lane fetches): the next k-tile streams into the idle
// stage while the current one is multiplied, with no staging registers.
// Rows past the group and columns past N read clamped in-bounds addresses;
// their products only reach outputs that are never stored.  One work-group
// per CU.
//
// The grid covers an upper bound of the tile count; each work-group reads the
// device-side tile prefixes (256-row tiles), so no host sync is needed.
// Work-groups are remapped so that each XCD (8 per chip, dispatched
// round-robin) walks a contiguous range of tiles, column tiles fastest: the
// 32 CUs of an XCD then work on one expert at a time, sharing its token rows
// and weight panels in that XCD's L2.
#include <algorithm>

#include "common.h"

#define PF_BM 256
#define PF_BN 256   // B rows per tile (gate/up: 128 gate + 128 up)
#define PF_BK 64
#define PF_BM_IDX 4  // moe_bm_of(4) == 256
#define PF_MT 8      // 32-row sub-tiles per tile
#define PF_LOADS 8   // 16-byte chunks per lane per operand per k-tile (8 rows per wave instruction)

struct GemmArgs {
  const uint16_t *A;         // gate/up: u [T, d]; down: H [R, f]
  const uint16_t *A_sh;      // gate/up: u;       down: H_sh [T, f_s]
  const int32_t *row_token;  // gate/up: permuted row -> token; down: unused
  const int32_t *offsets;    // [E + 1]
  const int32_t *tile_off;   // [E + 2] 256-row tile prefix (shared appended)
  const uint16_t *B1, *B3;   // routed: gate/up W1, W3 [E, N, K]; down W2 [E, N, K] (B3 unused)
  const uint16_t *B1s, *B3s; // shared
  void *C, *C_sh;            // gate/up: H bf16 [R, f], H_sh [T, f_s]; down: Y f32 [R, d], Y_sh [T, d]
  int64_t T;
  int E, K, K_sh, N, N_sh, has_shared;
  int nt_r, nt_s;            // column tiles of a routed / the shared group
};

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// element offset of 16-byte chunk c of LDS row r (rows of 64 bf16)
__device__ __forceinline__ int lds_off(int r, int c) { return r * PF_BK + ((c ^ (r & 7)) << 3); }

// 16 bytes per lane from global memory straight into LDS at dst + 16 * lane
__device__ __forceinline__ void dma16(const uint16_t *src, uint16_t *dst) {
  __builtin_amdgcn_global_load_lds((const void *)src, (lds_void_t *)dst, 16, 0, 0);
}

__device__ __forceinline__ void wait_dma_and_sync() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// LDS stages: four distinct objects, so that the compiler can tell the stage
// being filled by DMA from the stage being read.
__shared__ __attribute__((aligned(16))) uint16_t g_As0[PF_BM * PF_BK];
__shared__ __attribute__((aligned(16))) uint16_t g_As1[PF_BM * PF_BK];
__shared__ __attribute__((aligned(16))) uint16_t g_Bs0[PF_BN * PF_BK];
__shared__ __attribute__((aligned(16))) uint16_t g_Bs1[PF_BN * PF_BK];

template <int ST>
__device__ __forceinline__ uint16_t *stage_a() { return ST == 0 ? g_As0 : g_As1; }
template <int ST>
__device__ __forceinline__ uint16_t *stage_b() { return ST == 0 ? g_Bs0 : g_Bs1; }

// Issue the DMA of the k-tile starting at k0 into stage ST.  Wave w fills LDS
// rows 64w + 8q .. 64w + 8q + 7 (q < 8) of each operand; lane l writes row
// 64w + 8q + l/8, slot l%8, which holds global chunk (l%8) ^ (l/8).
template <int MTV, int ST>
__device__ __forceinline__ void issue_tile(const uint16_t *const (&ap)[PF_LOADS],
                                           const uint16_t *const (&bp)[PF_LOADS], int k0) {
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int q = 0; q < PF_LOADS; ++q) {
    if (64 * wv + 8 * q < 32 * MTV) dma16(ap[q] + k0, stage_a<ST>() + (64 * wv + 8 * q) * PF_BK);
    dma16(bp[q] + k0, stage_b<ST>() + (64 * wv + 8 * q) * PF_BK);
  }
}

struct Frags {
  bf16x8_t b0, b1;
};

// One k-tile: multiply stage ST while the next tile streams into the other
// stage.  Fragments of 16-deep step ks+1 are read while step ks multiplies.
template <int MTV, int ST>
__device__ __forceinline__ void k_step(const uint16_t *const (&ap)[PF_LOADS], const uint16_t *const (&bp)[PF_LOADS],
                                       int brow0, int brow1, int k_next, bool has_next,
                                       f32x16_t (&acc)[PF_MT][2]) {
  if (has_next) issue_tile<MTV, 1 - ST>(ap, bp, k_next);
  const uint16_t *As = stage_a<ST>();
  const uint16_t *Bs = stage_b<ST>();
  const int lane = threadIdx.x & 63;
  const int frow = lane & 31;    // fragment row inside a 32-row tile
  const int fchunk = lane >> 5;  // 0/1: first/second 8 of a 16-deep step
  bf16x8_t b0 = as_bf16x8(*(const uint4 *)&Bs[lds_off(brow0 + frow, fchunk)]);
  bf16x8_t b1 = as_bf16x8(*(const uint4 *)&Bs[lds_off(brow1 + frow, fchunk)]);
  bf16x8_t av[MTV];
#pragma unroll
  for (int i = 0; i < MTV; ++i) av[i] = as_bf16x8(*(const uint4 *)&As[lds_off(i * 32 + frow, fchunk)]);
#pragma unroll
  for (int ks = 0; ks < PF_BK / 16; ++ks) {
    bf16x8_t nb0, nb1, nav[MTV];
    if (ks + 1 < PF_BK / 16) {
      const int ch = (ks + 1) * 2 + fchunk;
      nb0 = as_bf16x8(*(const uint4 *)&Bs[lds_off(brow0 + frow, ch)]);
      nb1 = as_bf16x8(*(const uint4 *)&Bs[lds_off(brow1 + frow, ch)]);
#pragma unroll
      for (int i = 0; i < MTV; ++i) nav[i] = as_bf16x8(*(const uint4 *)&As[lds_off(i * 32 + frow, ch)]);
    }
#pragma unroll
    for (int i = 0; i < MTV; ++i) {
      acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], b0, acc[i][0], 0, 0, 0);
      acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], b1, acc[i][1], 0, 0, 0);
    }
    if (ks + 1 < PF_BK / 16) {
      b0 = nb0;
      b1 = nb1;
#pragma unroll
      for (int i = 0; i < MTV; ++i) av[i] = nav[i];
    }
  }
  // Schedule: the first step's fragment reads, then for every step its MFMAs
  // in pairs, each pair followed by one fragment read of the next step.
  __builtin_amdgcn_sched_group_barrier(0x100, 2 + MTV, 0);
#pragma unroll
  for (int ks = 0; ks < PF_BK / 16; ++ks) {
#pragma unroll
    for (int i = 0; i < MTV; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (ks + 1 < PF_BK / 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if (ks + 1 < PF_BK / 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  wait_dma_and_sync();
}

// The k loop of one tile with MTV valid 32-row sub-tiles (compile-time, so
// the body is straight-line).
template <int MTV>
__device__ __forceinline__ void k_loop(const uint16_t *const (&ap)[PF_LOADS], const uint16_t *const (&bp)[PF_LOADS],
                                       int brow0, int brow1, int K, f32x16_t (&acc)[PF_MT][2]) {
  const int nk = K / PF_BK;
  issue_tile<MTV, 0>(ap, bp, 0);
  wait_dma_and_sync();
  for (int kt = 0; kt < nk; kt += 2) {
    k_step<MTV, 0>(ap, bp, brow0, brow1, (kt + 1) * PF_BK, kt + 1 < nk, acc);
    if (kt + 1 < nk) k_step<MTV, 1>(ap, bp, brow0, brow1, (kt + 2) * PF_BK, kt + 2 < nk, acc);
  }
}

template <bool GATEUP>
__global__ __launch_bounds__(256, 1) void grouped_gemm_bf16_kernel(GemmArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  // ---- tile lookup (XCD-contiguous order, column tiles fastest)
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
    valid = min(PF_BM, a.offsets[g + 1] - a.offsets[g] - m0);
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
  const int mtv = (valid + 31) >> 5;  // 32-row sub-tiles holding rows of this group

  // ---- DMA sources: lane l of wave w fetches, for q < 8, row 64w + 8q + l/8,
  // chunk (l%8) ^ (l/8) of each operand
  const int lrow = 64 * wv + (lane >> 3);
  const int lchunk = (lane & 7) ^ ((lane >> 3) & 7);
  const uint16_t *ap[PF_LOADS];
  const uint16_t *bp[PF_LOADS];
  const uint16_t *Abase = shared ? a.A_sh : a.A;
#pragma unroll
  for (int q = 0; q < PF_LOADS; ++q) {
    const int row = lrow + 8 * q;
    const int r = min(row, valid - 1);  // clamped: rows past the group are never stored
    const int64_t arow = (GATEUP && !shared) ? (int64_t)a.row_token[rb + r] : rb + r;
    ap[q] = Abase + arow * K + lchunk * 8;
    int n;
    const uint16_t *bw;
    if (GATEUP) {
      n = nt * (PF_BN / 2) + (row & (PF_BN / 2 - 1));
      const bool up = row >= PF_BN / 2;
      bw = shared ? (up ? a.B3s : a.B1s) : ((up ? a.B3 : a.B1) + (int64_t)g * N * K);
    } else {
      n = nt * PF_BN + row;
      bw = shared ? a.B1s : (a.B1 + (int64_t)g * N * K);
    }
    bp[q] = bw + (int64_t)min(n, N - 1) * K + lchunk * 8;  // clamped: columns >= N are never stored
  }

  // B rows of the wave's two 32-column tiles
  const int brow0 = GATEUP ? wv * 32 : wv * 64;
  const int brow1 = GATEUP ? PF_BN / 2 + wv * 32 : wv * 64 + 32;

  f32x16_t acc[PF_MT][2];
#pragma unroll
  for (int i = 0; i < PF_MT; ++i) {
    acc[i][0] = f32x16_t{};
    acc[i][1] = f32x16_t{};
  }

  switch (mtv) {  // branch-free main loop per count of valid 32-row sub-tiles
    case 8: k_loop<8>(ap, bp, brow0, brow1, K, acc); break;
    case 7: k_loop<7>(ap, bp, brow0, brow1, K, acc); break;
    case 6: k_loop<6>(ap, bp, brow0, brow1, K, acc); break;
    case 5: k_loop<5>(ap, bp, brow0, brow1, K, acc); break;
    case 4: k_loop<4>(ap, bp, brow0, brow1, K, acc); break;
    case 3: k_loop<3>(ap, bp, brow0, brow1, K, acc); break;
    case 2: k_loop<2>(ap, bp, brow0, brow1, K, acc); break;
    default: k_loop<1>(ap, bp, brow0, brow1, K, acc); break;
  }

  // ---- epilogue; 32x32 D layout: lane holds rows 8*(r/4) + 4*(lane/32) + r%4 of column lane%32
  const int col = lane & 31;
  if (GATEUP) {
    uint16_t *C = (uint16_t *)(shared ? a.C_sh : a.C);
    const int n = nt * (PF_BN / 2) + wv * 32 + col;
    if (n < N) {
#pragma unroll
      for (int i = 0; i < PF_MT; ++i) {
        if (i >= mtv) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < valid) C[(rb + row) * (int64_t)N + n] = f32_to_bf16(silu_f(acc[i][0][r]) * acc[i][1][r]);
        }
      }
    }
  } else {
    float *C = (float *)(shared ? a.C_sh : a.C);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = nt * PF_BN + wv * 64 + j * 32 + col;
      if (n >= N) continue;
#pragma unroll
      for (int i = 0; i < PF_MT; ++i) {
        if (i >= mtv) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          if (row < valid) C[(rb + row) * (int64_t)N + n] = acc[i][j][r];
        }
      }
    }
  }
}

// Upper bound of the number of 256-row m-tiles over the routed groups.
static int64_t mtile_bound(int64_t R, int E) { return (R + PF_BM - 1) / PF_BM + std::min<int64_t>(E, R); }

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
