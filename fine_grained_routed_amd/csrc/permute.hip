// Permutation: group the T*k (token, slot) pairs by expert, tokens ascending
// inside each group, deterministically.
//
// Source: "Shared Expert" (How it works: routed expert outputs are
// scatter-summed back to tokens); the grouping is what lets each expert run
// as one GEMM over its tokens ("Shared and fine-grained experts", Researcher
// level, Systems limits: grouped GEMM kernels).
//
// Three launches, no atomics on the global result:
//   1. per block of 256 tokens, an LDS bitmap per expert (bit i = token i of the
//      block chose the expert); its popcount is the block's count per expert;
//   2. one work-group: per-expert totals, the seats each expert keeps (all of
//      its pairs, or at most the capacity), the exclusive scan of the kept
//      counts over experts (offsets), and each block's first rank per expert;
//   3. per block, rebuild the bitmap; a token's rank inside its expert group is
//      the popcount of the bits below it, so rows follow token order, and a
//      pair whose rank reaches the capacity is dropped (token_row -1).
// The capacity rule is "What is an 'expert', really?" (glossary: capacity
// factor / token dropping: a seat limit per expert, overflow skipped), read as
// "each expert keeps its first seats in token order".
#include "common.h"

#define PERM_WORDS (MOE_PERM_BLOCK / 64)

// The k expert indices of token t, all loads issued before the first use
// (slots j >= k hold -1, never read).
__device__ __forceinline__ void load_slots(const int32_t *__restrict__ idx, int64_t t, int k,
                                           int (&ev)[MOE_MAX_TOPK]) {
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) ev[j] = j < k ? idx[t * k + j] : -1;
}

// Set bits of an expert's block bitmap below bit i: the tokens of the block
// before token i that chose the expert.
__device__ __forceinline__ int bits_below(const unsigned long long *row, int i) {
  const int w = i >> 6;
  int n = 0;
#pragma unroll
  for (int q = 0; q < PERM_WORDS; ++q)
    if (q < w) n += __popcll(row[q]);
  return n + __popcll((i & 63) ? (row[w] & ((1ull << (i & 63)) - 1ull)) : 0ull);
}

// Sets token i's bit in the bitmap of each expert among its k slots (ev);
// an index out of range or a repeated expert is flagged in diag (if given).
__device__ __forceinline__ void mark_slots(unsigned long long *bm, const int (&ev)[MOE_MAX_TOPK], int i, int E, int k,
                                           DiagWords *diag) {
  const unsigned long long bit = 1ull << (i & 63);
  // every atomic is issued before the first result is looked at (an out of
  // range index ORs 0 into expert 0's word, a no-op)
  unsigned long long old[MOE_MAX_TOPK];
  bool bad = false;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    const int e = ev[j];
    const bool ok = e >= 0 && e < E;
    old[j] = j < k ? atomicOr(&bm[(ok ? e : 0) * PERM_WORDS + (i >> 6)], ok ? bit : 0ull) : 0ull;
    bad |= j < k && !ok;
  }
  unsigned long long seen = 0;  // token i's bit was already set in one of its experts' bitmaps
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    const int e = ev[j];
    if (j < k && e >= 0 && e < E) seen |= old[j] & bit;
  }
  if (diag && (seen || bad)) atomicOr(&diag->flags, (seen ? MOE_DIAG_DUPLICATE : 0u) | (bad ? MOE_DIAG_BAD_INDEX : 0u));
}

// Bit i of word (i / 64) of expert e's bitmap: token i of the block (thread
// i, whose slots are ev when it has a token) chose e.
__device__ __forceinline__ void build_bitmap(unsigned long long *bm, const int (&ev)[MOE_MAX_TOPK], bool has_token,
                                             int E, int k, DiagWords *diag) {
  for (int i = threadIdx.x; i < E * PERM_WORDS; i += blockDim.x) bm[i] = 0ull;
  __syncthreads();
  if (has_token) mark_slots(bm, ev, threadIdx.x, E, k, diag);
  __syncthreads();
}

__global__ __launch_bounds__(MOE_PERM_BLOCK) void perm_hist_kernel(const int32_t *__restrict__ idx, int64_t T, int E,
                                                                   int k, int32_t *__restrict__ blk_hist,
                                                                   DiagWords *diag) {
  extern __shared__ unsigned long long bm[];
  const int64_t t = (int64_t)blockIdx.x * MOE_PERM_BLOCK + threadIdx.x;
  int ev[MOE_MAX_TOPK];
  load_slots(idx, t, t < T ? k : 0, ev);
  build_bitmap(bm, ev, t < T, E, k, diag);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int q = 0; q < PERM_WORDS; ++q) c += __popcll(bm[e * PERM_WORDS + q]);
    blk_hist[(int64_t)blockIdx.x * E + e] = c;
  }
}

// Inclusive scan over the 64 lanes of a wave with DPP: shifts by 1, 2, 4 and
// 8 inside each row of 16 lanes (lanes shifted in from outside the row read
// 0), then row 0's total added to row 1 and row 2's to row 3 (the broadcast
// of lane 15 of each row), then the total of rows 0-1 added to rows 2 and 3
// (the broadcast of lane 31).  Every lane of the wave must be active.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return x;
}

// Exclusive scans of the N values v[n] over the work-group (blockDim.x a
// multiple of 64, at most 1024): excl[n] is this thread's prefix, total[n]
// the sum.  Each wave scans in registers (DPP), the wave totals meet in
// LDS (sh: 16 N ints, value-major) behind one barrier, and a second barrier
// frees sh.  Integer sums: the result does not depend on the order.
template <int N>
__device__ __forceinline__ void block_scan_n(const int (&v)[N], int (&excl)[N], int (&total)[N], int *sh) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
  int incl[N];
#pragma unroll
  for (int n = 0; n < N; ++n) incl[n] = wave_incl_scan(v[n]);
  if (lane == 63)
#pragma unroll
    for (int n = 0; n < N; ++n) sh[n * 16 + wv] = incl[n];
  __syncthreads();
  // every wave then scans the wave totals itself: lane l < 16 holds wave l's
  // (0 past the last wave), an inclusive scan over the 16 lanes of DPP row 0
  // (shifts 1, 2, 4, 8), and the wave reads its prefix and the total from
  // lanes wv - 1 and 15
  const int l16 = lane & 15;
  const int wvs = __builtin_amdgcn_readfirstlane(wv);
  int x[N];
#pragma unroll
  for (int n = 0; n < N; ++n) x[n] = sh[n * 16 + l16];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    int sc = l16 < nw ? x[n] : 0;
    sc += __builtin_amdgcn_update_dpp(0, sc, 0x111, 0xf, 0xf, true);  // row_shr:1
    sc += __builtin_amdgcn_update_dpp(0, sc, 0x112, 0xf, 0xf, true);  // row_shr:2
    sc += __builtin_amdgcn_update_dpp(0, sc, 0x114, 0xf, 0xf, true);  // row_shr:4
    sc += __builtin_amdgcn_update_dpp(0, sc, 0x118, 0xf, 0xf, true);  // row_shr:8
    const int pre = wvs > 0 ? __builtin_amdgcn_readlane(sc, wvs - 1) : 0;
    excl[n] = pre + incl[n] - v[n];
    total[n] = __builtin_amdgcn_readlane(sc, 15);
  }
  __syncthreads();
}

// single-value form: returns the exclusive prefix, the total in *total
__device__ __forceinline__ int block_exclusive_scan(int v, int *sh, int *total) {
  const int vv[1] = {v};
  int ex[1], tot[1];
  block_scan_n<1>(vv, ex, tot, sh);
  *total = tot[0];
  return ex[0];
}

// cap: seats per expert, 0 = no limit
__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t *__restrict__ blk_hist, int64_t nblk, int E, int cap,
                                                         int32_t *__restrict__ counts, int32_t *__restrict__ offsets) {
  __shared__ __attribute__((aligned(16))) int sh[16];
  const int e = threadIdx.x;
  int tot = 0;
  if (e < E) {
    // 16 blocks' counts loaded at a time, then replaced by the expert's pairs
    // in earlier blocks (the block's first rank)
    for (int64_t b0 = 0; b0 < nblk; b0 += 16) {
      int c[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) c[q] = b0 + q < nblk ? blk_hist[(b0 + q) * E + e] : 0;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        if (b0 + q < nblk) blk_hist[(b0 + q) * E + e] = tot;
        tot += c[q];
      }
    }
  }
  const int seats = (cap > 0 && tot > cap) ? cap : tot;
  int all;
  const int off = block_exclusive_scan(e < E ? seats : 0, sh, &all);
  if (e < E) {
    counts[e] = seats;
    offsets[e] = off;
  }
  if (e == 0) offsets[E] = all;
}

__global__ __launch_bounds__(MOE_PERM_BLOCK) void perm_scatter_kernel(const int32_t *__restrict__ idx, int64_t T,
                                                                      int E, int k, int cap,
                                                                      const int32_t *__restrict__ blk_base,
                                                                      const int32_t *__restrict__ offsets,
                                                                      int32_t *__restrict__ row_token,
                                                                      int32_t *__restrict__ token_row) {
  extern __shared__ unsigned long long bm[];
  const int i = threadIdx.x;
  const int64_t t = (int64_t)blockIdx.x * MOE_PERM_BLOCK + i;
  int ev[MOE_MAX_TOPK];
  load_slots(idx, t, t < T ? k : 0, ev);
  build_bitmap(bm, ev, t < T, E, k, nullptr);
  if (t >= T) return;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (j < k) {
      const int e = ev[j];
      int r = -1;  // dropped: invalid index or no seat left
      if (e >= 0 && e < E) {
        // rank among all of the expert's pairs: the block's first rank plus
        // the bits below this token's
        int rank = blk_base[(int64_t)blockIdx.x * E + e] + bits_below(bm + e * PERM_WORDS, i);
        if (!(cap > 0 && rank >= cap)) r = offsets[e] + rank;
      }
      token_row[t * k + j] = r;
      if (r >= 0) row_token[r] = (int32_t)t;
    }
  }
}

// The whole permutation for T <= MOE_PERM_BLOCK tokens (one block) in one
// work-group of 1024 threads, and, when tile_off is given, the GEMM tile
// prefixes too: at decode sizes the four launches cost more than their work.
// Same results as the three kernels above and tile_offsets_kernel below.
__global__ __launch_bounds__(1024) void perm_small_kernel(const int32_t *__restrict__ idx, int64_t T, int E, int k,
                                                          int cap, int has_shared, int32_t *__restrict__ counts,
                                                          int32_t *__restrict__ offsets,
                                                          int32_t *__restrict__ row_token,
                                                          int32_t *__restrict__ token_row,
                                                          int32_t *__restrict__ tile_off, DiagWords *diag) {
  extern __shared__ unsigned long long bm[];  // [E][PERM_WORDS] bitmap, then int[E] group starts
  int *start = (int *)(bm + E * PERM_WORDS);
  __shared__ __attribute__((aligned(16))) int sh[16 * (1 + MOE_N_BM)];
  const int tid = threadIdx.x;
  for (int i = tid; i < E * PERM_WORDS; i += 1024) bm[i] = 0ull;
  int ev[MOE_MAX_TOPK];
  load_slots(idx, tid, tid < T ? k : 0, ev);
  __syncthreads();
  if (tid < T) mark_slots(bm, ev, tid, E, k, diag);
  __syncthreads();
  int tot = 0;
  if (tid < E) {
#pragma unroll
    for (int q = 0; q < PERM_WORDS; ++q) tot += __popcll(bm[tid * PERM_WORDS + q]);
  }
  const int seats = (cap > 0 && tot > cap) ? cap : tot;
  // one scan for the row offsets and every tile height's m-tile prefixes
  int v[1 + MOE_N_BM], ex[1 + MOE_N_BM], all[1 + MOE_N_BM];
  v[0] = tid < E ? seats : 0;
#pragma unroll
  for (int b = 0; b < MOE_N_BM; ++b) v[1 + b] = tid < E ? (seats + moe_bm_of(b) - 1) / moe_bm_of(b) : 0;
  block_scan_n<1 + MOE_N_BM>(v, ex, all, sh);
  if (tid < E) {
    counts[tid] = seats;
    offsets[tid] = ex[0];
    start[tid] = ex[0];
  }
  if (tid == 0) offsets[E] = all[0];
  if (tile_off) {
#pragma unroll
    for (int b = 0; b < MOE_N_BM; ++b) {
      const int bmh = moe_bm_of(b);
      int32_t *to = tile_off + b * (E + 2);
      if (tid < E) to[tid] = ex[1 + b];
      if (tid == 0) {
        to[E] = all[1 + b];
        to[E + 1] = all[1 + b] + (has_shared ? (int)((T + bmh - 1) / bmh) : 0);
      }
    }
  }
  __syncthreads();
  if (tid < T) {
    const int w = tid >> 6;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k) {
        const int e = ev[j];
        int r = -1;  // dropped: invalid index or no seat left
        if (e >= 0 && e < E) {
          const int rank = bits_below(bm + e * PERM_WORDS, tid);
          if (!(cap > 0 && rank >= cap)) r = start[e] + rank;
        }
        token_row[(int64_t)tid * k + j] = r;
        if (r >= 0) row_token[r] = tid;
      }
    }
  }
}

// Permutation of T <= MOE_PERM_BLOCK tokens in one launch; tile_off (or NULL)
// receives the tile prefixes as launch_tile_offsets would.
hipError_t launch_permute_small(const moe_dims &dm, int64_t T, const int32_t *topk_idx, int32_t *counts,
                                int32_t *offsets, int32_t *row_token, int32_t *token_row, int32_t *tile_off,
                                const WsLayout &L, char *ws, hipStream_t st) {
  const int E = dm.n_routed;
  const size_t lds = (size_t)E * PERM_WORDS * sizeof(unsigned long long) + (size_t)E * sizeof(int);
  perm_small_kernel<<<1, 1024, lds, st>>>(topk_idx, T, E, dm.top_k, dm.capacity, dm.d_ff_shared > 0 ? 1 : 0, counts,
                                          offsets, row_token, token_row, tile_off, (DiagWords *)(ws + L.diag));
  return hipGetLastError();
}

hipError_t launch_permute(const moe_dims &dm, int64_t T, const int32_t *topk_idx, int32_t *counts, int32_t *offsets,
                          int32_t *row_token, int32_t *token_row, const WsLayout &L, char *ws, hipStream_t st) {
  if (T <= MOE_PERM_BLOCK)
    return launch_permute_small(dm, T, topk_idx, counts, offsets, row_token, token_row, nullptr, L, ws, st);
  const int E = dm.n_routed, k = dm.top_k;
  const int64_t nblk = (T + MOE_PERM_BLOCK - 1) / MOE_PERM_BLOCK;
  int32_t *blk = (int32_t *)(ws + L.blk);
  DiagWords *diag = (DiagWords *)(ws + L.diag);
  const size_t lds = (size_t)E * PERM_WORDS * sizeof(unsigned long long);
  perm_hist_kernel<<<dim3((unsigned)nblk), MOE_PERM_BLOCK, lds, st>>>(topk_idx, T, E, k, blk, diag);
  perm_scan_kernel<<<1, 1024, 0, st>>>(blk, nblk, E, dm.capacity, counts, offsets);
  perm_scatter_kernel<<<dim3((unsigned)nblk), MOE_PERM_BLOCK, lds, st>>>(topk_idx, T, E, k, dm.capacity, blk,
                                                                          offsets, row_token, token_row);
  return hipGetLastError();
}

// ------------------------------------------------------------- GEMM tile prefixes
// tile_off[b][g] = sum_{g' < g} ceil(rows_g' / BM_b) for the routed groups
// g <= E, and tile_off[b][E+1] adds the shared group's ceil(T / BM_b) m-tiles.
__global__ __launch_bounds__(1024) void tile_offsets_kernel(const int32_t *__restrict__ counts, int E, int64_t T,
                                                            int has_shared, int32_t *__restrict__ tile_off) {
  __shared__ __attribute__((aligned(16))) int sh[16 * MOE_N_BM];
  const int e = threadIdx.x;
  const int c = e < E ? counts[e] : 0;
  int v[MOE_N_BM], ex[MOE_N_BM], all[MOE_N_BM];
#pragma unroll
  for (int b = 0; b < MOE_N_BM; ++b) v[b] = e < E ? (c + moe_bm_of(b) - 1) / moe_bm_of(b) : 0;
  block_scan_n<MOE_N_BM>(v, ex, all, sh);
#pragma unroll
  for (int b = 0; b < MOE_N_BM; ++b) {
    const int bm = moe_bm_of(b);
    int32_t *to = tile_off + b * (E + 2);
    if (e < E) to[e] = ex[b];
    if (e == 0) {
      to[E] = all[b];
      to[E + 1] = all[b] + (has_shared ? (int)((T + bm - 1) / bm) : 0);
    }
  }
}

hipError_t launch_tile_offsets(const moe_dims &dm, int64_t T, const int32_t *counts, const WsLayout &L, char *ws,
                               hipStream_t st) {
  tile_offsets_kernel<<<1, 1024, 0, st>>>(counts, dm.n_routed, T, dm.d_ff_shared > 0 ? 1 : 0,
                                          (int32_t *)(ws + L.tile_off));
  return hipGetLastError();
}
