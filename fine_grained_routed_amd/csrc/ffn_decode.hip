// Decode path: expert FFNs for small token counts as HBM weight streaming.
//
// Source: "Shared and fine-grained experts", Developer level, 'Why not go finer
// still' (with few tokens per expert, the expert GEMMs are small and their
// time goes to reading weights from memory); Researcher level, Systems limits
// (grouped kernels over many small experts).  "Shared Expert" (How it works): the
// shared MLP runs on every token; here it is one more group.
//
// Work items are (16-row tile, column slice) pairs over the device-side tile
// list of the permutation (16-row tiles; the shared group appended), so
// experts that received no token have no tile and cost nothing.  Each of the
// 4 waves of a work-group owns 16 * NT output columns and walks the whole reduction
// depth, loading the weight fragments of 16x16x32 matrix-core steps straight
// from HBM into registers (no LDS: each weight element is used by this wave
// only); the 16 token rows are re-read from L2.
// An expert's weights are streamed once per 16 of its rows (once for nearly
// every expert at decode sizes; the tiles of one expert run together, so
// repeats mostly hit L2).  Each wave issues the loads of DK_UNROLL steps
// before their MFMAs.
//
// gate/up: H[r, n] = SiLU(A[r,:] . W1_g[n,:]) * (A[r,:] . W3_g[n,:]), bf16 out
// down:    Y[r, n] = H[r,:] . W2_g[n,:], fp32 out
#include <algorithm>

#include "common.h"

#define DK_BM 16                               // rows per tile (one MFMA row tile)
#define DK_BM_IDX 0                            // moe_bm_of(0) == 16
#define DK_WAVES 4
// 16-column MFMA tiles per wave and 32-deep steps per load batch.  gate/up
// streams two weights over the long model dimension; the down projection
// reduces over the short expert width and keeps more of its single weight in
// flight per column (measured at DeepSeek-V3 decode: 1.06 ms against 1.17 ms
// with the gate/up shape).
#ifndef DK_GU_NT
#define DK_GU_NT 2
#endif
#ifndef DK_GU_U
#define DK_GU_U 4
#endif
#ifndef DK_NARROW_WGS
#define DK_NARROW_WGS 3072  // gate/up work-group bound below which 1-tile, 8-step waves are used
#endif
#ifndef DK_DN_NT
#define DK_DN_NT 1
#endif
#ifndef DK_DN_U
#define DK_DN_U 8
#endif
constexpr int dk_cols(int nt) { return 16 * nt * DK_WAVES; }  // columns per work-group

struct DecodeArgs {
  const uint16_t *A, *A_sh;      // gate/up: u [T, d] (gathered); down: H [R, f], H_sh [T, f_s]
  const int32_t *row_token;      // gate/up routed rows -> token
  const int32_t *offsets;        // [E + 1]
  const int32_t *tile_off;       // [E + 2] 16-row tile prefix (shared appended)
  const uint16_t *B1, *B3;       // routed weights [E, N, K] (B3: up, gate/up only)
  const uint16_t *B1s, *B3s;     // shared weights [N_sh, K_sh]
  void *C, *C_sh;                // gate/up: H / H_sh bf16; down: Y / Y_sh fp32
  int64_t T;
  int E, K, K_sh, N, N_sh;
  int ns_r, ns_s;                // column slices of a routed / the shared group
};


// Weight fragments in the matrix-core layout (lane l: row l & 15, 16-byte
// chunk l / 16 of a 32-deep step) are ordinary cached loads: each 128-byte
// line of a weight row is then requested as two 64-byte halves by two
// instructions, and with non-temporal loads the second half often misses L2
// again (measured: 1.7x the weight bytes fetched); cached, it hits.
__device__ __forceinline__ uint4 dk_load(const uint16_t *p) { return *(const uint4 *)p; }

// Whole-line weight loads: for each pair of 32-deep steps (a
// 64-deep window, 128 bytes of every weight row) and each 16-column tile, two
// non-temporal loads each cover 8 complete rows: lane l of load i reads row
// 8 i + (l & 7) of the tile, 16-byte chunk 4 * bit3(l) + l / 16 of the window.
// Swapping the two registers between lanes l and l ^ 8 (within 16-lane rows)
// where bit 3 of the lane is set then gives each step's operand in the
// matrix-core layout (row l & 15, chunk l / 16 of the step): step u takes the
// values that lanes with bit 3 == u loaded.  Every line is fetched once, so
// these loads are non-temporal: at DeepSeek-V3 decode the routed gate/up runs
// at 6.7 TB/s this way against 6.0 with cached half-line loads.  (The dense
// four-wave kernel keeps cached loads: its row blocks share weight lines, and
// holding raw and exchanged registers cost it occupancy.)
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_t dk_load_nt(const uint16_t *p) {
  return __builtin_nontemporal_load((const u32x4_t *)p);
}
__device__ __forceinline__ unsigned dk_xor8(unsigned v) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xf, 0xf, false);  // row_ror:8 == lane ^ 8 in 16
}
__device__ __forceinline__ void dk_lines_to_steps(const u32x4_t &r0, const u32x4_t &r1, bool hi, uint4 &s0,
                                                  uint4 &s1) {
  unsigned o0[4], o1[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const unsigned x0 = dk_xor8(r0[c]), x1 = dk_xor8(r1[c]);
    o0[c] = hi ? x1 : r0[c];
    o1[c] = hi ? r1[c] : x0;
  }
  s0 = make_uint4(o0[0], o0[1], o0[2], o0[3]);
  s1 = make_uint4(o1[0], o1[1], o1[2], o1[3]);
}

template <bool GATEUP, int DK_NT, int DK_UNROLL>
__global__ __launch_bounds__(256) void decode_ffn_kernel(DecodeArgs a) {
  constexpr int DK_COLS = dk_cols(DK_NT);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  // ---- tile lookup: (16-row tile, column slice), routed tiles first
  const int mt_r = a.tile_off[a.E];
  const int mt_s = a.tile_off[a.E + 1] - mt_r;
  const int64_t tiles_r = (int64_t)mt_r * a.ns_r;
  const int64_t tile = blockIdx.x;
  if (tile >= tiles_r + (int64_t)mt_s * a.ns_s) return;
  bool shared;
  int g, slice, K, N, valid;
  int64_t rb;
  if (tile < tiles_r) {
    shared = false;
    const int mt = (int)(tile / a.ns_r);
    slice = (int)(tile % a.ns_r);
    int lo = 0, hi = a.E - 1;  // largest g with tile_off[g] <= mt
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.tile_off[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    g = lo;
    const int m0 = (mt - a.tile_off[g]) * DK_BM;
    valid = min(DK_BM, a.offsets[g + 1] - a.offsets[g] - m0);
    rb = (int64_t)a.offsets[g] + m0;
    K = a.K;
    N = a.N;
  } else {
    shared = true;
    const int64_t ts = tile - tiles_r;
    const int mt = (int)(ts / a.ns_s);
    slice = (int)(ts % a.ns_s);
    g = a.E;
    rb = (int64_t)mt * DK_BM;
    valid = (int)min((int64_t)DK_BM, a.T - rb);
    K = a.K_sh;
    N = a.N_sh;
  }
  const int n0 = slice * DK_COLS + wv * (16 * DK_NT);
  if (n0 >= N) return;
  const int kofs = (lane >> 4) * 8;  // this lane's 8-element slice of a 32-deep step

  // A: this lane's row of the tile (padded rows repeat a valid row, never stored)
  const int r = min(lane & 15, valid - 1);
  const int64_t arow = (GATEUP && !shared) ? (int64_t)a.row_token[rb + r] : rb + r;
  const uint16_t *ap = (shared ? a.A_sh : a.A) + arow * K + kofs;
  // B: this lane's weight row in each of the wave's column tiles
  const uint16_t *w1 = shared ? a.B1s : a.B1 + (int64_t)g * N * K;
  const uint16_t *w3 = GATEUP ? (shared ? a.B3s : a.B3 + (int64_t)g * N * K) : nullptr;
  const uint16_t *p1[DK_NT];
  const uint16_t *p3[DK_NT];
#pragma unroll
  for (int j = 0; j < DK_NT; ++j) {
    const int n = min(n0 + j * 16 + (lane & 15), N - 1);  // clamped; columns >= N are never stored
    p1[j] = w1 + (int64_t)n * K + kofs;
    p3[j] = GATEUP ? w3 + (int64_t)n * K + kofs : nullptr;
  }
  f32x4_t acc1[DK_NT], acc3[DK_NT];
#pragma unroll
  for (int j = 0; j < DK_NT; ++j) {
    acc1[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc3[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  static_assert(DK_UNROLL % 2 == 0, "whole-line loads go by pairs of steps");
  const bool hi8 = (lane & 8) != 0;
  const uint16_t *q1[DK_NT][2];
  const uint16_t *q3[DK_NT][2];
#pragma unroll
  for (int j = 0; j < DK_NT; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int n = min(n0 + j * 16 + 8 * i + (lane & 7), N - 1);  // clamped; columns >= N are never stored
      const int ch = 4 * ((lane >> 3) & 1) + (lane >> 4);
      q1[j][i] = w1 + (int64_t)n * K + 8 * ch;
      q3[j][i] = GATEUP ? w3 + (int64_t)n * K + 8 * ch : nullptr;
    }
  // main loop: DK_UNROLL steps per batch, every load of a batch issued before
  // the first use; remainder: single 32-deep steps
  const int kmain = K - K % (32 * DK_UNROLL);
  for (int k0 = 0; k0 < kmain; k0 += 32 * DK_UNROLL) {
    uint4 av[DK_UNROLL], b1[DK_UNROLL][DK_NT], b3[DK_UNROLL][DK_NT];
    u32x4_t l1[DK_UNROLL][DK_NT], l3[DK_UNROLL][DK_NT];  // [2 x pair + i][j]
#pragma unroll
    for (int s = 0; s < DK_UNROLL; ++s) av[s] = *(const uint4 *)(ap + k0 + 32 * s);
#pragma unroll
    for (int s2 = 0; s2 < DK_UNROLL; s2 += 2)
#pragma unroll
      for (int j = 0; j < DK_NT; ++j)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          l1[s2 + i][j] = dk_load_nt(q1[j][i] + k0 + 32 * s2);
          if (GATEUP) l3[s2 + i][j] = dk_load_nt(q3[j][i] + k0 + 32 * s2);
        }
#pragma unroll
    for (int s2 = 0; s2 < DK_UNROLL; s2 += 2)
#pragma unroll
      for (int j = 0; j < DK_NT; ++j) {
        dk_lines_to_steps(l1[s2][j], l1[s2 + 1][j], hi8, b1[s2][j], b1[s2 + 1][j]);
        if (GATEUP) dk_lines_to_steps(l3[s2][j], l3[s2 + 1][j], hi8, b3[s2][j], b3[s2 + 1][j]);
      }
#pragma unroll
    for (int s = 0; s < DK_UNROLL; ++s) {
      const bf16x8_t a8 = as_bf16x8(av[s]);
#pragma unroll
      for (int j = 0; j < DK_NT; ++j) {
        acc1[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, as_bf16x8(b1[s][j]), acc1[j], 0, 0, 0);
        if (GATEUP) acc3[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, as_bf16x8(b3[s][j]), acc3[j], 0, 0, 0);
      }
    }
    // keep every load of the batch ahead of its MFMAs (the scheduler would
    // otherwise interleave them and hold only a few loads in flight)
    __builtin_amdgcn_sched_group_barrier(0x020, DK_UNROLL * (1 + DK_NT * (GATEUP ? 2 : 1)), 0);
    __builtin_amdgcn_sched_group_barrier(0x008, DK_UNROLL * DK_NT * (GATEUP ? 2 : 1), 0);
  }
  for (int k0 = kmain; k0 < K; k0 += 32) {
    const bf16x8_t a8 = as_bf16x8(*(const uint4 *)(ap + k0));
#pragma unroll
    for (int j = 0; j < DK_NT; ++j) {
      acc1[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, as_bf16x8(dk_load(p1[j] + k0)), acc1[j], 0, 0, 0);
      if (GATEUP)
        acc3[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, as_bf16x8(dk_load(p3[j] + k0)), acc3[j], 0, 0, 0);
    }
  }
  // ---- epilogue: lane holds rows 4*(lane/16)+q of column lane%16 of each tile
#pragma unroll
  for (int j = 0; j < DK_NT; ++j) {
    const int n = n0 + j * 16 + (lane & 15);
    if (n >= N) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = (lane >> 4) * 4 + q;
      if (row >= valid) continue;
      if (GATEUP) {
        uint16_t *C = (uint16_t *)(shared ? a.C_sh : a.C);
        C[(rb + row) * N + n] = (uint16_t)pack_bf16x2(silu_fast(acc1[j][q]) * acc3[j][q], 0.0f);
      } else {
        float *C = (float *)(shared ? a.C_sh : a.C);
        C[(rb + row) * N + n] = acc1[j][q];
      }
    }
  }
}

// ------------------------------------------------------- dense layers (no routed experts)
// The dense prefix layers' FFN streams one weight set for all T tokens, so a
// work-group takes every row of a pass (up to 4 x 16 rows, so one weight
// fragment feeds all of them), 64 NT output columns (4 waves of NT 16-column
// tiles) and one of S slices of the reduction (S is chosen per pass so that
// slices x column groups x row blocks come to a set number of work-groups,
// enough to fill the chip at decode sizes).  The token rows of each batch
// (32 UL deep) are staged once into LDS for the four
// waves (double-buffered, chunks XOR-swizzled per row so the fragment reads
// are free of bank conflicts); each wave streams its own weight fragments
// into registers one batch ahead.  Each slice writes fp32 partial sums
// P[s][row][col]; a second kernel adds the S partials in slice order (fixed,
// so the result is deterministic) and applies SiLU(gate) * up (bf16 H) or
// writes Y.  Gate/up partials hold the gate columns at [0, N) and the up
// columns at [N, 2N).  K is a multiple of the batch depth.
template <bool GATEUP, int MT, int NT, int UL>
__global__ __launch_bounds__(256) void dense_decode_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ W1,
                                                           const uint16_t *__restrict__ W3, int rows, int K, int N,
                                                           int ksl, float *__restrict__ P) {
  constexpr int BK = 32 * UL;      // batch depth
  constexpr int CPR = BK / 8;      // 16-byte chunks per token row of a batch
  constexpr int CPT = 64 * CPR / 256;  // chunks each thread moves per batch
  static_assert(UL % 2 == 0, "the slot swizzle needs whole groups of 8 chunks per row");
  __shared__ __attribute__((aligned(16))) uint4 As[2][64 * CPR];  // [buffer][row * CPR + slot]
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int n0 = blockIdx.x * 64 * NT + wv * 16 * NT;
  const int s = blockIdx.y;
  const int r0 = blockIdx.z * 64;
  const int k_begin = s * ksl, k_end = min(K, k_begin + ksl);
  const int nb = max(0, (k_end - k_begin) / BK);  // batches (a slice past K has none)
  // cooperative token-tile load: thread tid moves chunks tid + 256 q of the
  // 64 x CPR chunks of a batch (row c / CPR, chunk c % CPR); the low three
  // bits of a chunk's slot are XORed with the row's
  const uint16_t *ag[CPT];
  int aslot[CPT];
#pragma unroll
  for (int q = 0; q < CPT; ++q) {
    const int c = tid + 256 * q, row = c / CPR, ch = c % CPR;
    ag[q] = A + (int64_t)min(r0 + row, rows - 1) * K + k_begin + ch * 8;  // clamped: rows past the pass are never stored
    aslot[q] = row * CPR + (ch ^ (row & 7));
  }
  // the wave's weight rows
  const int kofs = (lane >> 4) * 8;  // this lane's 8-element slice of a 32-deep step
  const uint16_t *p1[NT];
  const uint16_t *p3[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int n = min(n0 + 16 * j + (lane & 15), N - 1);  // clamped: columns >= N are never stored
    p1[j] = W1 + (int64_t)n * K + k_begin + kofs;
    p3[j] = GATEUP ? W3 + (int64_t)n * K + k_begin + kofs : nullptr;
  }
  f32x4_t acc1[MT][NT], acc3[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      acc1[m][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc3[m][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  uint4 ar[CPT];  // the next batch's token chunks of this thread
  uint4 bc1[UL][NT], bc3[UL][NT], bn1[UL][NT], bn3[UL][NT];
#pragma unroll
  for (int q = 0; q < CPT; ++q) ar[q] = make_uint4(0u, 0u, 0u, 0u);
  if (nb > 0) {
#pragma unroll
    for (int q = 0; q < CPT; ++q) ar[q] = *(const uint4 *)ag[q];
#pragma unroll
    for (int u = 0; u < UL; ++u)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        bc1[u][j] = dk_load(p1[j] + 32 * u);
        bc3[u][j] = GATEUP ? dk_load(p3[j] + 32 * u) : bc1[u][j];
      }
  }
  for (int b = 0; b < nb; ++b) {
    uint4 *buf = As[b & 1];
#pragma unroll
    for (int q = 0; q < CPT; ++q) buf[aslot[q]] = ar[q];
    __syncthreads();  // batch b's token tile is in LDS (and batch b's weights in registers)
    const int bn = min(b + 1, nb - 1);  // the last batch re-loads its own data (in bounds, unused)
#pragma unroll
    for (int q = 0; q < CPT; ++q) ar[q] = *(const uint4 *)(ag[q] + bn * BK);
#pragma unroll
    for (int u = 0; u < UL; ++u)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        bn1[u][j] = dk_load(p1[j] + bn * BK + 32 * u);
        bn3[u][j] = GATEUP ? dk_load(p3[j] + bn * BK + 32 * u) : bn1[u][j];
      }
#pragma unroll
    for (int u = 0; u < UL; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const int row = 16 * m + (lane & 15), ch = 4 * u + (lane >> 4);
        const bf16x8_t a8 = as_bf16x8(buf[row * CPR + (ch ^ (row & 7))]);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          acc1[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, as_bf16x8(bc1[u][j]), acc1[m][j], 0, 0, 0);
          if (GATEUP)
            acc3[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, as_bf16x8(bc3[u][j]), acc3[m][j], 0, 0, 0);
        }
      }
#pragma unroll
    for (int u = 0; u < UL; ++u)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        bc1[u][j] = bn1[u][j];
        bc3[u][j] = bn3[u][j];
      }
  }
  // lane holds rows 4 * (lane / 16) + q of column lane % 16 of each 16 x 16 tile
  const int pw = GATEUP ? 2 * N : N;  // partial row width
  float *ps = P + (int64_t)s * rows * pw;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int col = n0 + 16 * j + (lane & 15);
    if (col >= N) continue;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = r0 + 16 * m + (lane >> 4) * 4 + q;
        if (row >= rows) continue;
        ps[(int64_t)row * pw + col] = acc1[m][j][q];
        if (GATEUP) ps[(int64_t)row * pw + N + col] = acc3[m][j][q];
      }
  }
}

// Small passes (under 48 rows): single-wave work-groups, each with every row
// of the pass for NT 16-column tiles, re-reading the token fragments from L2
// (as many bytes as its weight fragments); staging them in LDS does not pay
// for its barriers at this size.
#define DD_U 2  // 32-deep steps per load batch

template <bool GATEUP, int MT, int NT>
__global__ __launch_bounds__(64) void dense_decode_wave_kernel(const uint16_t *__restrict__ A, const uint16_t *__restrict__ W1,
                                                          const uint16_t *__restrict__ W3, int rows, int K, int N,
                                                          int ksl, float *__restrict__ P) {
  const int lane = threadIdx.x;
  const int n0 = blockIdx.x * 16 * NT;
  const int s = blockIdx.y;
  const int r0 = blockIdx.z * 64;
  const int k_begin = s * ksl, k_end = min(K, k_begin + ksl);
  const int kofs = (lane >> 4) * 8;  // this lane's 8-element slice of a 32-deep step
  const uint16_t *ap[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) ap[m] = A + (int64_t)min(r0 + 16 * m + (lane & 15), rows - 1) * K + kofs;
  const uint16_t *p1[NT];
  const uint16_t *p3[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int n = min(n0 + 16 * j + (lane & 15), N - 1);  // clamped: columns >= N are never stored
    p1[j] = W1 + (int64_t)n * K + kofs;
    p3[j] = GATEUP ? W3 + (int64_t)n * K + kofs : nullptr;
  }
  f32x4_t acc1[MT][NT], acc3[MT][NT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      acc1[m][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc3[m][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
  // whole-line weight loads by pairs of 32-deep steps (lane layout as in dk_lines_to_steps)
  static_assert(DD_U == 2, "one pair of steps per batch");
  const bool hi8 = (lane & 8) != 0;
  const uint16_t *q1[NT][2];
  const uint16_t *q3[NT][2];
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int n = min(n0 + 16 * j + 8 * i + (lane & 7), N - 1);  // clamped: columns >= N are never stored
      const int ch = 4 * ((lane >> 3) & 1) + (lane >> 4);
      q1[j][i] = W1 + (int64_t)n * K + 8 * ch;
      q3[j][i] = GATEUP ? W3 + (int64_t)n * K + 8 * ch : nullptr;
    }
  int k0 = k_begin;
  for (; k0 + 32 * DD_U <= k_end; k0 += 32 * DD_U) {
    uint4 av[DD_U][MT], b1[DD_U][NT], b3[DD_U][NT];
    u32x4_t l1[2][NT], l3[2][NT];
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        l1[i][j] = dk_load_nt(q1[j][i] + k0);
        if (GATEUP) l3[i][j] = dk_load_nt(q3[j][i] + k0);
      }
#pragma unroll
    for (int u = 0; u < DD_U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m) av[u][m] = *(const uint4 *)(ap[m] + k0 + 32 * u);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      dk_lines_to_steps(l1[0][j], l1[1][j], hi8, b1[0][j], b1[1][j]);
      if (GATEUP) dk_lines_to_steps(l3[0][j], l3[1][j], hi8, b3[0][j], b3[1][j]);
    }
#pragma unroll
    for (int u = 0; u < DD_U; ++u)
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const bf16x8_t a8 = as_bf16x8(av[u][m]);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          acc1[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, as_bf16x8(b1[u][j]), acc1[m][j], 0, 0, 0);
          if (GATEUP)
            acc3[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, as_bf16x8(b3[u][j]), acc3[m][j], 0, 0, 0);
        }
      }
    // keep every load of the batch ahead of its MFMAs
    __builtin_amdgcn_sched_group_barrier(0x020, DD_U * (MT + NT * (GATEUP ? 2 : 1)), 0);
    __builtin_amdgcn_sched_group_barrier(0x008, DD_U * MT * NT * (GATEUP ? 2 : 1), 0);
  }
  for (; k0 < k_end; k0 += 32) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint4 b1v = dk_load(p1[j] + k0);
      const uint4 b3v = GATEUP ? dk_load(p3[j] + k0) : b1v;
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const bf16x8_t a8 = as_bf16x8(*(const uint4 *)(ap[m] + k0));
        acc1[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, as_bf16x8(b1v), acc1[m][j], 0, 0, 0);
        if (GATEUP) acc3[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a8, as_bf16x8(b3v), acc3[m][j], 0, 0, 0);
      }
    }
  }
  // lane holds rows 4 * (lane / 16) + q of column lane % 16 of each 16 x 16 tile
  const int pw = GATEUP ? 2 * N : N;  // partial row width
  float *ps = P + (int64_t)s * rows * pw;
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int col = n0 + 16 * j + (lane & 15);
    if (col >= N) continue;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = r0 + 16 * m + (lane >> 4) * 4 + q;
        if (row >= rows) continue;
        ps[(int64_t)row * pw + col] = acc1[m][j][q];
        if (GATEUP) ps[(int64_t)row * pw + N + col] = acc3[m][j][q];
      }
  }
}

// Sum of the S partials in slice order; gate/up: H = SiLU(gate) * up in bf16,
// down: Y in fp32.  Four consecutive columns per thread.
template <bool GATEUP>
__global__ __launch_bounds__(256) void dense_reduce_kernel(const float *__restrict__ P, int S, int rows, int N,
                                                           void *__restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= (int64_t)rows * N) return;
  const int64_t row = i / N;
  const int col = (int)(i % N);
  const int pw = GATEUP ? 2 * N : N;
  float4 g = make_float4(0.f, 0.f, 0.f, 0.f), u = g;
  for (int s = 0; s < S; ++s) {
    const float *ps = P + ((int64_t)s * rows + row) * pw + col;
    const float4 a = *(const float4 *)ps;
    g = make_float4(g.x + a.x, g.y + a.y, g.z + a.z, g.w + a.w);
    if (GATEUP) {
      const float4 b = *(const float4 *)(ps + N);
      u = make_float4(u.x + b.x, u.y + b.y, u.z + b.z, u.w + b.w);
    }
  }
  if (GATEUP) {
    uint2 pk;
    pk.x = pack_bf16x2(silu_fast(g.x) * u.x, silu_fast(g.y) * u.y);
    pk.y = pack_bf16x2(silu_fast(g.z) * u.z, silu_fast(g.w) * u.w);
    *(uint2 *)((uint16_t *)out + row * N + col) = pk;
  } else {
    *(float4 *)((float *)out + row * N + col) = g;
  }
}

// NT, UL: the four-wave kernel's column tiles per wave and batch depth; NTW:
// the single-wave kernel's column tiles
template <bool GATEUP, int NT, int UL, int NTW>
static void launch_dense_pass(const uint16_t *A, const uint16_t *W1, const uint16_t *W3, int rows, int K, int N,
                              float *P, void *out, hipStream_t st) {
  const int mt = (std::min(rows, 64) + 15) / 16;  // 16-row blocks of a full 64-row group
  const int S = moe_dd_splits(GATEUP, N, rows);
  if (moe_dd_four_wave(rows)) {
    // k per slice: whole batches (K is a multiple of 64; a slice past K adds zeros)
    const dim3 grid((unsigned)((N + 64 * NT - 1) / (64 * NT)), (unsigned)S, (unsigned)((rows + 63) / 64));
    if (K % (32 * UL) == 0) {
      constexpr int BK = 32 * UL;
      const int ksl = ((K / BK + S - 1) / S) * BK;
      if (mt >= 4) dense_decode_kernel<GATEUP, 4, NT, UL><<<grid, 256, 0, st>>>(A, W1, W3, rows, K, N, ksl, P);
      else dense_decode_kernel<GATEUP, 3, NT, UL><<<grid, 256, 0, st>>>(A, W1, W3, rows, K, N, ksl, P);
    } else {
      const int ksl = ((K / 64 + S - 1) / S) * 64;
      if (mt >= 4) dense_decode_kernel<GATEUP, 4, NT, 2><<<grid, 256, 0, st>>>(A, W1, W3, rows, K, N, ksl, P);
      else dense_decode_kernel<GATEUP, 3, NT, 2><<<grid, 256, 0, st>>>(A, W1, W3, rows, K, N, ksl, P);
    }
  } else {
    const int ksl = ((K / 64 + S - 1) / S) * 64;  // k per slice, whole 128-byte lines (a slice past K adds zeros)
    const dim3 grid((unsigned)((N + 16 * NTW - 1) / (16 * NTW)), (unsigned)S, 1);
    if (mt == 2) dense_decode_wave_kernel<GATEUP, 2, NTW><<<grid, 64, 0, st>>>(A, W1, W3, rows, K, N, ksl, P);
    else dense_decode_wave_kernel<GATEUP, 1, NTW><<<grid, 64, 0, st>>>(A, W1, W3, rows, K, N, ksl, P);
  }
  const int64_t n4 = (int64_t)rows * N / 4;
  dense_reduce_kernel<GATEUP><<<dim3((unsigned)((n4 + 255) / 256)), 256, 0, st>>>(P, S, rows, N, out);
}

// The dense layer on the decode path, in passes of up to MOE_DD_ROWS rows.
static hipError_t launch_dense_decode(const moe_dims &dm, int64_t T, const void *u, const moe_weights &w, float *y_sh,
                                      const WsLayout &L, char *ws, hipStream_t st, hipEvent_t ev_mid) {
  const int d = dm.d_model, fs = dm.d_ff_shared;
  uint16_t *Hs = (uint16_t *)(ws + L.h_sh);
  float *P = (float *)(ws + L.dense_part);
  for (int64_t r0 = 0; r0 < T; r0 += MOE_DD_ROWS) {
    const int rows = (int)std::min<int64_t>(MOE_DD_ROWS, T - r0);
    launch_dense_pass<true, MOE_DD_NT_GU, MOE_DD_UL_GU, 2>((const uint16_t *)u + r0 * d, (const uint16_t *)w.w1s,
                                                          (const uint16_t *)w.w3s, rows, d, fs, P, Hs + r0 * fs, st);
    if (ev_mid && r0 + MOE_DD_ROWS >= T) (void)hipEventRecord(ev_mid, st);
    launch_dense_pass<false, MOE_DD_NT_DN, MOE_DD_UL_DN, 2>(Hs + r0 * fs, (const uint16_t *)w.w2s, nullptr, rows, fs, d,
                                                            P, y_sh + r0 * d, st);
  }
  return hipGetLastError();
}

static int64_t dk_mtile_bound(int64_t R, int E) { return (R + DK_BM - 1) / DK_BM + std::min<int64_t>(E, R); }

// Column width of a gate/up work-group: batches with few row tiles (the
// smallest batches) take narrower column slices with deeper load batches,
// which gives twice the work-groups (DeepSeek-V3 T=16: gate/up 0.89 ms
// against 0.94).
static bool dk_narrow(const moe_dims &dm, int64_t T) {
  const int64_t R = T * dm.top_k;
  return dk_mtile_bound(R, dm.n_routed) * ((dm.d_ff + dk_cols(DK_GU_NT) - 1) / dk_cols(DK_GU_NT)) < DK_NARROW_WGS;
}

// Work-groups of the routed layer's two launches.
static void dk_grids(const moe_dims &dm, int64_t T, int64_t *grid1, int64_t *grid2) {
  const int E = dm.n_routed, d = dm.d_model, f = dm.d_ff, fs = dm.d_ff_shared;
  const int64_t R = T * dm.top_k;
  const int64_t mt_sh = fs > 0 ? (T + DK_BM - 1) / DK_BM : 0;
  const int c1 = dk_narrow(dm, T) ? dk_cols(1) : dk_cols(DK_GU_NT);
  *grid1 = dk_mtile_bound(R, E) * ((f + c1 - 1) / c1) + mt_sh * (fs > 0 ? (fs + c1 - 1) / c1 : 1);
  constexpr int c2 = dk_cols(DK_DN_NT);
  *grid2 = (dk_mtile_bound(R, E) + mt_sh) * ((d + c2 - 1) / c2);
}

int64_t ffn_decode_max_workgroups(const moe_dims &dm, int64_t T) {
  if (dm.n_routed == 0) {
    // dense layer: passes of at most MOE_DD_ROWS rows; the pass kernels' 2-D/3-D
    // grids are small in every dimension, the 1-D reduction of a pass with N
    // output columns takes rows * N / 4 / 256 work-groups
    const int64_t rows = std::min<int64_t>(T, MOE_DD_ROWS);
    const int64_t n = std::max<int64_t>(dm.d_ff_shared, dm.d_model);
    return (rows * n / 4 + 255) / 256;
  }
  int64_t g1, g2;
  dk_grids(dm, T, &g1, &g2);
  return std::max(g1, g2);
}

hipError_t launch_ffn_decode(const moe_dims &dm, int64_t T, const void *u, const moe_weights &w,
                             const int32_t *counts, const int32_t *offsets, const int32_t *row_token,
                             float *y_rows, float *y_sh, const WsLayout &L, char *ws, hipStream_t st,
                             hipEvent_t ev_mid) {
  (void)counts;
  if (dm.n_routed == 0) return launch_dense_decode(dm, T, u, w, y_sh, L, ws, st, ev_mid);
  const int E = dm.n_routed, d = dm.d_model, f = dm.d_ff, fs = dm.d_ff_shared;
  const int hs = fs > 0 ? 1 : 0;
  const int64_t R = T * dm.top_k;
  const int32_t *tile_off = (const int32_t *)(ws + L.tile_off) + DK_BM_IDX * (E + 2);
  uint16_t *H = (uint16_t *)(ws + L.h);
  uint16_t *Hs = (uint16_t *)(ws + L.h_sh);
  const int64_t mt_sh = hs ? (T + DK_BM - 1) / DK_BM : 0;

  DecodeArgs g1{};
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
  const bool narrow = dk_narrow(dm, T);
  const int c1 = narrow ? dk_cols(1) : dk_cols(DK_GU_NT);
  g1.ns_r = (f + c1 - 1) / c1;
  g1.ns_s = hs ? (fs + c1 - 1) / c1 : 1;
  int64_t grid1, grid2;
  dk_grids(dm, T, &grid1, &grid2);
  if (narrow) decode_ffn_kernel<true, 1, 8><<<dim3((unsigned)grid1), 256, 0, st>>>(g1);
  else decode_ffn_kernel<true, DK_GU_NT, DK_GU_U><<<dim3((unsigned)grid1), 256, 0, st>>>(g1);
  if (ev_mid) (void)hipEventRecord(ev_mid, st);

  DecodeArgs g2{};
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
  constexpr int c2 = dk_cols(DK_DN_NT);
  g2.ns_r = (d + c2 - 1) / c2;
  g2.ns_s = g2.ns_r;
  decode_ffn_kernel<false, DK_DN_NT, DK_DN_U><<<dim3((unsigned)grid2), 256, 0, st>>>(g2);
  return hipGetLastError();
}
