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
// XOR-swizzled per row so that fragment reads are free of bank conflicts.
// LDS is filled by direct global-to-LDS loads (global_load_lds_dwordx4: each
// lane's 16 bytes land at LDS base + 16 * lane, so the swizzle is applied by
// choosing which global chunk each lane fetches), with no staging registers;
// every row segment fetched is a whole 128-byte line.  The token-row tile is
// fetched one k-tile ahead (it is shared by all column tiles of the XCD and
// mostly hits in L2) and the weight tile two k-tiles ahead.  The barrier that
// publishes tile j + 1 sits before the last 16-deep step of tile j, so the
// first fragment reads of tile j + 1 overlap the last MFMAs of tile j.
// One work-group per CU.
//
// The grid covers an upper bound of the tile count; each work-group reads the
// device-side tile prefixes (256-row tiles), so no host sync is needed.
// Work-groups are dispatched round-robin over the 8 XCDs, so work-group i is
// remapped to tile (i % 8) * ceil(total / 8) + i / 8: each XCD walks a
// contiguous range of the tile order described in the kernel, and the 32 CUs
// of an XCD work on one expert at a time, sharing its token rows and weight
// panels in that XCD's L2.
#include <algorithm>

#include "common.h"

#define PF_BM 256
#define PF_BN 256    // B rows per tile (gate/up: 128 gate + 128 up)
#define PF_BK 64
#define PF_BM_IDX 4  // moe_bm_of(4) == 256
#define PF_MT 8      // 32-row sub-tiles per tile
#define PF_GM 8      // m-tiles per ordering block (routed experts)
#define PF_GM_SH 4   // m-tiles per ordering block (shared group)
#define PF_LOADS 8   // DMA instructions per wave per operand per k-tile (8 rows of 128 B each)

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

// LDS rows of 64 bf16 hold eight 16-byte chunks; chunk c of row r sits in slot
// c ^ swz(r).  swz is one-to-one on any 8 consecutive rows and on any 8 rows
// of one parity among 16 consecutive rows, so the 16-byte fragment reads of 8
// (or 16) consecutive rows fall on distinct banks whether the LDS serves 8
// lanes over 32 banks or 16 lanes over 64 banks per cycle.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// element offset of 16-byte chunk c of LDS row r
__device__ __forceinline__ int lds_off(int r, int c) { return r * PF_BK + ((c ^ swz(r)) << 3); }

// 16 bytes per lane from global memory straight into LDS at dst + 16 * lane
__device__ __forceinline__ void dma16(const uint16_t *src, uint16_t *dst) {
  __builtin_amdgcn_global_load_lds((const void *)src, (lds_void_t *)dst, 16, 0, 0);
}

// Publish LDS to the work-group: this wave's LDS reads are complete and at
// most one k-tile of B DMA (8 instructions) is still in flight, then the
// work-group barrier.  Written out rather than __syncthreads(), whose release
// fence would also wait for every DMA in flight and so drain the prefetch.
__device__ __forceinline__ void publish() {
  // s_waitcnt immediate (gfx9 layout: vmcnt [3:0] and [15:14], expcnt [6:4],
  // lgkmcnt [11:8]): vmcnt 8, expcnt 7, lgkmcnt 0.  The builtin, unlike
  // inline asm, is visible to the compiler's own wait tracking, which then
  // knows that older DMA into a stage has landed.
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0078);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS: the token-row tile rotates over 2 stages, the weight tile over 3
// (5 x 32 KB = 160 KB).  Separate objects, so that the compiler can tell a
// stage being filled by DMA from a stage being read.
__shared__ __attribute__((aligned(16))) uint16_t g_As0[PF_BM * PF_BK];
__shared__ __attribute__((aligned(16))) uint16_t g_As1[PF_BM * PF_BK];
__shared__ __attribute__((aligned(16))) uint16_t g_Bs0[PF_BN * PF_BK];
__shared__ __attribute__((aligned(16))) uint16_t g_Bs1[PF_BN * PF_BK];
__shared__ __attribute__((aligned(16))) uint16_t g_Bs2[PF_BN * PF_BK];

template <int SA>
__device__ __forceinline__ uint16_t *stage_a() { return SA == 0 ? g_As0 : g_As1; }
template <int SB>
__device__ __forceinline__ uint16_t *stage_b() { return SB == 0 ? g_Bs0 : SB == 1 ? g_Bs1 : g_Bs2; }

// DMA of one operand's k-tile at k0.  Wave w fills LDS rows 64w + 8q ..
// 64w + 8q + 7 (q < 8); lane l writes row 64w + 8q + l/8, slot l%8, which
// holds global chunk (l%8) ^ swz(row) (the per-q chunk is folded into src[q]).
__device__ __forceinline__ void issue_op(const uint16_t *const (&src)[PF_LOADS], uint16_t *stage, int k0) {
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int q = 0; q < PF_LOADS; ++q) dma16(src[q] + k0, stage + (64 * wv + 8 * q) * PF_BK);
}

// Fragments of one 16-deep step: two B column tiles and MTV A row tiles.
template <int MTV>
struct Frags {
  bf16x8_t b0, b1, a[MTV];
};

template <int MTV, int SA, int SB>
__device__ __forceinline__ void read_frags(Frags<MTV> &f, int brow0, int brow1, int step) {
  const uint16_t *As = stage_a<SA>();
  const uint16_t *Bs = stage_b<SB>();
  const int lane = threadIdx.x & 63;
  const int frow = lane & 31;             // fragment row inside a 32-row tile
  const int ch = step * 2 + (lane >> 5);  // chunk: first/second 8 of the 16-deep step
  f.b0 = as_bf16x8(*(const uint4 *)&Bs[lds_off(brow0 + frow, ch)]);
  f.b1 = as_bf16x8(*(const uint4 *)&Bs[lds_off(brow1 + frow, ch)]);
#pragma unroll
  for (int i = 0; i < MTV; ++i) f.a[i] = as_bf16x8(*(const uint4 *)&As[lds_off(i * 32 + frow, ch)]);
}

template <int MTV>
__device__ __forceinline__ void mfma_step(const Frags<MTV> &f, f32x16_t (&acc)[PF_MT][2]) {
#pragma unroll
  for (int i = 0; i < MTV; ++i) {
    acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b0, acc[i][0], 0, 0, 0);
    acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b1, acc[i][1], 0, 0, 0);
  }
}

// MFMAs of one step in pairs, each pair followed by one fragment read of the next step
template <int MTV>
__device__ __forceinline__ void interleave_hint() {
#pragma unroll
  for (int i = 0; i < MTV; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
}

// One k-tile j, its token rows in A-stage SA (= j % 2) and weights in B-stage
// SB (= j % 3).  f0 holds its step-0 fragments on entry and the next tile's
// step-0 fragments on exit.  Every iteration issues exactly one A tile (j + 1)
// and one B tile (j + 2) of DMA, past the end re-fetching the last tile into
// a stage nobody reads again, so the count of DMA in flight is the same on
// every path and one constant wait publishes tile j + 1.
template <int MTV, int SA, int SB>
__device__ __forceinline__ void k_iter(const uint16_t *const (&ap)[PF_LOADS], const uint16_t *const (&bp)[PF_LOADS],
                                       int brow0, int brow1, int j, int nk, Frags<MTV> &f0, Frags<MTV> &f1,
                                       f32x16_t (&acc)[PF_MT][2]) {
  // stages of tile j - 1 (read completely before the previous barrier)
  issue_op(ap, stage_a<SA ^ 1>(), min(j + 1, nk - 1) * PF_BK);
  issue_op(bp, stage_b<(SB + 2) % 3>(), min(j + 2, nk - 1) * PF_BK);
  read_frags<MTV, SA, SB>(f1, brow0, brow1, 1);
  mfma_step<MTV>(f0, acc);
  interleave_hint<MTV>();
  read_frags<MTV, SA, SB>(f0, brow0, brow1, 2);
  mfma_step<MTV>(f1, acc);
  interleave_hint<MTV>();
  read_frags<MTV, SA, SB>(f1, brow0, brow1, 3);
  mfma_step<MTV>(f0, acc);
  interleave_hint<MTV>();
  // publish tile j + 1 (A issued last iteration... this one; B two iterations ago)
  publish();
  // step-0 fragments of tile j + 1 (after the last tile this reads stages
  // whose values are never used; reading LDS is always in bounds)
  read_frags<MTV, SA ^ 1, (SB + 1) % 3>(f0, brow0, brow1, 0);
  mfma_step<MTV>(f1, acc);
  interleave_hint<MTV>();
}

// The k loop of one tile with MTV valid 32-row sub-tiles (compile-time, so
// the body is straight-line).
template <int MTV>
__device__ __forceinline__ void k_loop(const uint16_t *const (&ap)[PF_LOADS], const uint16_t *const (&bp)[PF_LOADS],
                                       int brow0, int brow1, int K, f32x16_t (&acc)[PF_MT][2]) {
  const int nk = K / PF_BK;
  issue_op(ap, stage_a<0>(), 0);
  issue_op(bp, stage_b<0>(), 0);
  issue_op(bp, stage_b<1>(), min(1, nk - 1) * PF_BK);
  publish();  // tile 0 landed; B tile 1 may be in flight
  Frags<MTV> f0, f1;
  read_frags<MTV, 0, 0>(f0, brow0, brow1, 0);
  // six k-tiles per trip (the stage pattern repeats every lcm(2, 3) tiles);
  // whole trips are unconditional, the remainder follows
  int j = 0;
  for (; j + 6 <= nk; j += 6) {
    k_iter<MTV, 0, 0>(ap, bp, brow0, brow1, j, nk, f0, f1, acc);
    k_iter<MTV, 1, 1>(ap, bp, brow0, brow1, j + 1, nk, f0, f1, acc);
    k_iter<MTV, 0, 2>(ap, bp, brow0, brow1, j + 2, nk, f0, f1, acc);
    k_iter<MTV, 1, 0>(ap, bp, brow0, brow1, j + 3, nk, f0, f1, acc);
    k_iter<MTV, 0, 1>(ap, bp, brow0, brow1, j + 4, nk, f0, f1, acc);
    k_iter<MTV, 1, 2>(ap, bp, brow0, brow1, j + 5, nk, f0, f1, acc);
  }
  if (j < nk) k_iter<MTV, 0, 0>(ap, bp, brow0, brow1, j, nk, f0, f1, acc);
  if (j + 1 < nk) k_iter<MTV, 1, 1>(ap, bp, brow0, brow1, j + 1, nk, f0, f1, acc);
  if (j + 2 < nk) k_iter<MTV, 0, 2>(ap, bp, brow0, brow1, j + 2, nk, f0, f1, acc);
  if (j + 3 < nk) k_iter<MTV, 1, 0>(ap, bp, brow0, brow1, j + 3, nk, f0, f1, acc);
  if (j + 4 < nk) k_iter<MTV, 0, 1>(ap, bp, brow0, brow1, j + 4, nk, f0, f1, acc);
  // the trailing re-fetches must land before the work-group can exit
  __builtin_amdgcn_s_waitcnt(0x0070);
}

template <bool GATEUP>
__global__ __launch_bounds__(256, 1) void grouped_gemm_bf16_kernel(GemmArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  // ---- tile lookup.  Order: group by group; inside a group, blocks of up to
  // PF_GM m-tiles (PF_GM_SH for the shared group), and inside a block the
  // m-tiles fastest, so the tiles that share a weight panel (all m-tiles of an
  // expert, its ragged tail included) run at the same time and share it in
  // L2, while neighbouring column tiles share the token rows.  Each XCD walks
  // a contiguous range of this order.
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
  int mt, mt_g, ntiles, gm;
  int64_t q;   // index of the tile inside its group
  if (tile < tiles_r) {
    shared = false;
    const int key = (int)(tile / a.nt_r);  // expert g owns keys tile_off[g] .. tile_off[g+1]-1
    int lo = 0, hi = a.E - 1;              // largest g with tile_off[g] <= key
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.tile_off[mid] <= key) lo = mid; else hi = mid - 1;
    }
    g = lo;
    q = tile - (int64_t)a.nt_r * a.tile_off[g];
    mt_g = a.tile_off[g + 1] - a.tile_off[g];
    ntiles = a.nt_r;
    gm = PF_GM;
    K = a.K;
    N = a.N;
  } else {
    shared = true;
    g = a.E;
    q = tile - tiles_r;
    mt_g = mt_s;
    ntiles = a.nt_s;
    gm = PF_GM_SH;
    K = a.K_sh;
    N = a.N_sh;
  }
  {
    const int64_t blk = q / ((int64_t)gm * ntiles);       // full blocks of gm m-tiles before
    const int in_blk = (int)(q - blk * gm * ntiles);
    const int bsize = min(gm, mt_g - (int)blk * gm);       // m-tiles in this block
    nt = in_blk / bsize;
    mt = (int)blk * gm + in_blk % bsize;
  }
  if (!shared) {
    const int m0 = mt * PF_BM;
    valid = min(PF_BM, a.offsets[g + 1] - a.offsets[g] - m0);
    rb = (int64_t)a.offsets[g] + m0;
  } else {
    rb = (int64_t)mt * PF_BM;
    valid = (int)min((int64_t)PF_BM, a.T - rb);
  }
  const int mtv = (valid + 31) >> 5;  // 32-row sub-tiles holding rows of this group

  // ---- DMA sources: lane l of wave w fetches, for q < 8, row 64w + 8q + l/8,
  // chunk (l%8) ^ swz(row) = (l%8) ^ ((l/8) ^ q) of each operand
  const int lrow = 64 * wv + (lane >> 3);
  const uint16_t *ap[PF_LOADS];
  const uint16_t *bp[PF_LOADS];
  const uint16_t *Abase = shared ? a.A_sh : a.A;
#pragma unroll
  for (int q = 0; q < PF_LOADS; ++q) {
    const int row = lrow + 8 * q;
    const int lchunk = (lane & 7) ^ swz(row);
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

  // branch-free main loop per count of valid 32-row sub-tiles, rounded up to
  // one of 1, 2, 4, 6, 8 (the extra sub-tiles multiply rows that are never stored)
  if (mtv > 6) k_loop<8>(ap, bp, brow0, brow1, K, acc);
  else if (mtv > 4) k_loop<6>(ap, bp, brow0, brow1, K, acc);
  else if (mtv > 2) k_loop<4>(ap, bp, brow0, brow1, K, acc);
  else if (mtv > 1) k_loop<2>(ap, bp, brow0, brow1, K, acc);
  else k_loop<1>(ap, bp, brow0, brow1, K, acc);

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
