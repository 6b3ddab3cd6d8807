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

__device__ __forceinline__ void build_bitmap(unsigned long long *bm, const int32_t *__restrict__ idx, int64_t T,
                                             int E, int k, int64_t blk, DiagWords *diag) {
  for (int i = threadIdx.x; i < E * PERM_WORDS; i += blockDim.x) bm[i] = 0ull;
  __syncthreads();
  const int i = threadIdx.x;
  const int64_t t = blk * MOE_PERM_BLOCK + i;
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[t * k + j];
      if (e < 0 || e >= E) {
        if (diag) atomicOr(&diag->flags, MOE_DIAG_BAD_INDEX);
        continue;
      }
      const unsigned long long bit = 1ull << (i & 63);
      const unsigned long long old = atomicOr(&bm[e * PERM_WORDS + (i >> 6)], bit);
      if ((old & bit) && diag) atomicOr(&diag->flags, MOE_DIAG_DUPLICATE);
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(MOE_PERM_BLOCK) void perm_hist_kernel(const int32_t *__restrict__ idx, int64_t T, int E,
                                                                   int k, int32_t *__restrict__ blk_hist,
                                                                   DiagWords *diag) {
  extern __shared__ unsigned long long bm[];
  build_bitmap(bm, idx, T, E, k, blockIdx.x, diag);
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    int c = 0;
#pragma unroll
    for (int q = 0; q < PERM_WORDS; ++q) c += __popcll(bm[e * PERM_WORDS + q]);
    blk_hist[(int64_t)blockIdx.x * E + e] = c;
  }
}

// Exclusive scan of v over the work-group (blockDim.x == 1024), returns the
// exclusive prefix of this thread and writes the total to *total.
__device__ int block_exclusive_scan(int v, int *sh, int *total) {
  const int tid = threadIdx.x;
  sh[tid] = v;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    int add = tid >= o ? sh[tid - o] : 0;
    __syncthreads();
    sh[tid] += add;
    __syncthreads();
  }
  const int incl = sh[tid];
  *total = sh[1023];
  __syncthreads();
  return incl - v;
}

// cap: seats per expert, 0 = no limit
__global__ __launch_bounds__(1024) void perm_scan_kernel(int32_t *__restrict__ blk_hist, int64_t nblk, int E, int cap,
                                                         int32_t *__restrict__ counts, int32_t *__restrict__ offsets) {
  __shared__ int sh[1024];
  const int e = threadIdx.x;
  int tot = 0;
  if (e < E) {
    for (int64_t b = 0; b < nblk; ++b) {
      const int c = blk_hist[b * E + e];
      blk_hist[b * E + e] = tot;  // the expert's pairs in earlier blocks: the block's first rank
      tot += c;
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
  build_bitmap(bm, idx, T, E, k, blockIdx.x, nullptr);
  const int i = threadIdx.x;
  const int64_t t = (int64_t)blockIdx.x * MOE_PERM_BLOCK + i;
  if (t >= T) return;
  for (int j = 0; j < k; ++j) {
    const int e = idx[t * k + j];
    if (e < 0 || e >= E) {
      token_row[t * k + j] = -1;
      continue;
    }
    const unsigned long long *row = bm + e * PERM_WORDS;
    int rank = 0;
    const int w = i >> 6;
#pragma unroll
    for (int q = 0; q < PERM_WORDS; ++q)
      if (q < w) rank += __popcll(row[q]);
    const unsigned long long below = (i & 63) ? (row[w] & ((1ull << (i & 63)) - 1ull)) : 0ull;
    rank += __popcll(below);
    rank += blk_base[(int64_t)blockIdx.x * E + e];  // rank among all of the expert's pairs
    if (cap > 0 && rank >= cap) {
      token_row[t * k + j] = -1;  // no seat left
      continue;
    }
    const int r = offsets[e] + rank;
    token_row[t * k + j] = r;
    row_token[r] = (int32_t)t;
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
  __shared__ int sh[1024];
  const int tid = threadIdx.x;
  for (int i = tid; i < E * PERM_WORDS; i += 1024) bm[i] = 0ull;
  __syncthreads();
  if (tid < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[(int64_t)tid * k + j];
      if (e < 0 || e >= E) {
        atomicOr(&diag->flags, MOE_DIAG_BAD_INDEX);
        continue;
      }
      const unsigned long long bit = 1ull << (tid & 63);
      const unsigned long long old = atomicOr(&bm[e * PERM_WORDS + (tid >> 6)], bit);
      if (old & bit) atomicOr(&diag->flags, MOE_DIAG_DUPLICATE);
    }
  }
  __syncthreads();
  int tot = 0;
  if (tid < E) {
#pragma unroll
    for (int q = 0; q < PERM_WORDS; ++q) tot += __popcll(bm[tid * PERM_WORDS + q]);
  }
  const int seats = (cap > 0 && tot > cap) ? cap : tot;
  int all;
  const int off = block_exclusive_scan(tid < E ? seats : 0, sh, &all);
  if (tid < E) {
    counts[tid] = seats;
    offsets[tid] = off;
    start[tid] = off;
  }
  if (tid == 0) offsets[E] = all;
  if (tile_off) {
    for (int b = 0; b < MOE_N_BM; ++b) {
      const int bmh = moe_bm_of(b);
      int tiles;
      const int toff = block_exclusive_scan(tid < E ? (seats + bmh - 1) / bmh : 0, sh, &tiles);
      int32_t *to = tile_off + b * (E + 2);
      if (tid < E) to[tid] = toff;
      if (tid == 0) {
        to[E] = tiles;
        to[E + 1] = tiles + (has_shared ? (int)((T + bmh - 1) / bmh) : 0);
      }
    }
  }
  __syncthreads();
  if (tid < T) {
    const int w = tid >> 6;
    for (int j = 0; j < k; ++j) {
      const int e = idx[(int64_t)tid * k + j];
      if (e < 0 || e >= E) {
        token_row[(int64_t)tid * k + j] = -1;
        continue;
      }
      const unsigned long long *row = bm + e * PERM_WORDS;
      int rank = 0;
#pragma unroll
      for (int q = 0; q < PERM_WORDS; ++q)
        if (q < w) rank += __popcll(row[q]);
      rank += __popcll((tid & 63) ? (row[w] & ((1ull << (tid & 63)) - 1ull)) : 0ull);
      if (cap > 0 && rank >= cap) {
        token_row[(int64_t)tid * k + j] = -1;  // no seat left
        continue;
      }
      const int r = start[e] + rank;
      token_row[(int64_t)tid * k + j] = r;
      row_token[r] = tid;
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
  __shared__ int sh[1024];
  const int e = threadIdx.x;
  const int c = e < E ? counts[e] : 0;
  for (int b = 0; b < MOE_N_BM; ++b) {
    const int bm = moe_bm_of(b);
    int all;
    const int off = block_exclusive_scan(e < E ? (c + bm - 1) / bm : 0, sh, &all);
    int32_t *to = tile_off + b * (E + 2);
    if (e < E) to[e] = off;
    if (e == 0) {
      to[E] = all;
      to[E + 1] = all + (has_shared ? (int)((T + bm - 1) / bm) : 0);
    }
  }
}

hipError_t launch_tile_offsets(const moe_dims &dm, int64_t T, const int32_t *counts, const WsLayout &L, char *ws,
                               hipStream_t st) {
  tile_offsets_kernel<<<1, 1024, 0, st>>>(counts, dm.n_routed, T, dm.d_ff_shared > 0 ? 1 : 0,
                                          (int32_t *)(ws + L.tile_off));
  return hipGetLastError();
}
