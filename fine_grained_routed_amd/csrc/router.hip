// Router: logits l[t,e] = u[t,:] . w_router[e,:] (+ b_e), with a per-logit error bound.
//
// Source: "What is an 'expert', really?" (panel 2: a linear layer scores the
// experts); "Shared Expert" (How it works: the N_r centroids).  The ranking
// key is the exact real logit of the stored inputs; the logits computed here
// are approximations with a rigorous bound, which the top-k kernel uses to
// decide when a comparison must be settled exactly.
//
// bf16 inputs: bf16 x bf16 products are exact in fp32; the matrix cores sum
// chunks of ROUTER_CHUNK products in fp32 and the chunk sums are added in
// fp64.  Error bound per logit (any summation order inside the chunk, unit
// roundoff taken as 2^-22, twice truncation's 2^-23):
//     |L - l| <= (CHUNK * 2^-22 + (d / CHUNK + 2) * 2^-52) * ||u_t|| ||c_e|| + 2^-50 |L| + d 2^-120
// using sum |u_i c_ei| <= ||u_t|| ||c_e|| (Cauchy-Schwarz).  For small token
// counts the reduction is split into S slices of whole chunks whose fp64
// partial sums are added in slice order afterwards: every logit then passes
// through at most d / CHUNK / S + S fp64 additions, never more than the
// d / CHUNK + 2 the bound allows for.
// fp32 inputs: products are exact in fp64 and summed in fp64:
//     |L - l| <= (d + 2) * 2^-52 * ||u_t|| ||c_e|| + 2^-50 |L| + d 2^-120.
#include "common.h"

#define ROUTER_CHUNK 64
#define RT_BM 64
#define RT_BN 64
#define RT_BK 64
#define RT_LDS_STRIDE (RT_BK + 8)  // bf16 elements per LDS row (16-byte pad)

// sum of the squares of 8 bf16 values, in fp64 (each square exact)
__device__ __forceinline__ double sumsq_bf16x8(const uint4 &v) {
  const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
  double s = 0.0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const double lo = (double)__uint_as_float(w4[q] << 16), hi = (double)__uint_as_float(w4[q] & 0xffff0000u);
    s = fma(lo, lo, s);
    s = fma(hi, hi, s);
  }
  return s;
}

// -------------------------------------------------------- bf16 logits (MFMA)
// Work-group tile: 64 tokens x 64 experts, 4 waves in a 2 x 2 grid, each wave
// 32 x 32 = 2 x 2 MFMA 16x16x32 tiles.
// blockIdx.z selects a slice of kps k-tiles; with one slice the logits (bias
// added) are written, otherwise slice s writes its fp64 partial sums to
// logits + s * T * E and router_reduce_kernel adds them.  The squared norms
// come out of the same loads: work-groups of the first expert tile sum their
// token rows' squares, those of the first token tile their router rows'; with
// one slice they write ||u_t||^2 to un2 and ||c_e|| to cn, otherwise slice s
// writes its partial sums to un2 + s * T and cn + s * E for the reduction.
// clear (or NULL): the diagnostics header, zeroed by the first work-group.
__global__ __launch_bounds__(256) void router_logits_bf16_kernel(const uint16_t *__restrict__ u,
                                                                 const uint16_t *__restrict__ w,
                                                                 const float *__restrict__ bias, int64_t T,
                                                                 int E, int d, int kps, double *__restrict__ logits,
                                                                 double *__restrict__ un2, double *__restrict__ cn,
                                                                 DiagWords *clear) {
  if (clear && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0) *clear = DiagWords{};
  __shared__ __attribute__((aligned(16))) uint16_t As[RT_BM * RT_LDS_STRIDE];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[RT_BN * RT_LDS_STRIDE];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int64_t t0 = (int64_t)blockIdx.x * RT_BM;
  const int e0 = blockIdx.y * RT_BN;

  f32x4_t acc[2][2];
  double acc64[2][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int r = 0; r < 4; ++r) acc64[i][j][r] = 0.0;
    }

  // each thread moves 2 chunks of 16 bytes of A and of B per k-tile
  const uint16_t *ap[2];
  const uint16_t *bp[2];
  bool aok[2], bok[2];
  int lrow[2], lcol[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int c = tid + 256 * q;
    lrow[q] = c >> 3;
    lcol[q] = (c & 7) * 8;
    aok[q] = t0 + lrow[q] < T;
    bok[q] = e0 + lrow[q] < E;
    ap[q] = u + (aok[q] ? (t0 + lrow[q]) : 0) * (int64_t)d + lcol[q];
    bp[q] = w + (int64_t)(bok[q] ? (e0 + lrow[q]) : 0) * d + lcol[q];
  }
  const int nk = d / RT_BK;
  const int kt0 = blockIdx.z * kps, kt1 = min(nk, kt0 + kps);
  const int chunk_tiles = ROUTER_CHUNK / RT_BK;
  // the next k-tile's loads are in flight while the current one is multiplied
  uint4 av[2], bv[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    av[q] = keep_or_zero(aok[q], *(const uint4 *)(ap[q] + kt0 * RT_BK));  // pointers clamped in bounds
    bv[q] = keep_or_zero(bok[q], *(const uint4 *)(bp[q] + kt0 * RT_BK));
  }
  const bool unorm = blockIdx.y == 0, cnorm = blockIdx.x == 0;
  double usq[2] = {0.0, 0.0}, csq[2] = {0.0, 0.0};  // this thread's squares of its two chunk rows
  for (int kt = kt0; kt < kt1; ++kt) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      *(uint4 *)&As[lrow[q] * RT_LDS_STRIDE + lcol[q]] = av[q];
      *(uint4 *)&Bs[lrow[q] * RT_LDS_STRIDE + lcol[q]] = bv[q];
      if (unorm) usq[q] += sumsq_bf16x8(av[q]);
      if (cnorm) csq[q] += sumsq_bf16x8(bv[q]);
    }
    __syncthreads();
    const int kn = min(kt + 1, kt1 - 1);  // the last trip re-loads its own tile (in bounds, unused)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      av[q] = keep_or_zero(aok[q], *(const uint4 *)(ap[q] + kn * RT_BK));
      bv[q] = keep_or_zero(bok[q], *(const uint4 *)(bp[q] + kn * RT_BK));
    }
#pragma unroll
    for (int kk = 0; kk < RT_BK / 32; ++kk) {
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = as_bf16x8(*(const uint4 *)&As[(wm * 32 + i * 16 + (lane & 15)) * RT_LDS_STRIDE + kk * 32 +
                                             (lane >> 4) * 8]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = as_bf16x8(*(const uint4 *)&Bs[(wn * 32 + j * 16 + (lane & 15)) * RT_LDS_STRIDE + kk * 32 +
                                             (lane >> 4) * 8]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if ((kt + 1) % chunk_tiles == 0 || kt + 1 == kt1) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc64[i][j][r] += (double)acc[i][j][r];
          acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    }
  }
  // norms: the 8 threads of a chunk row are consecutive lanes; their sums
  // are added in a fixed butterfly order
  const bool whole = gridDim.z == 1;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    double su = usq[q], sc = csq[q];
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      su += __shfl_xor(su, o, 64);
      sc += __shfl_xor(sc, o, 64);
    }
    if (lcol[q] == 0) {
      const int64_t t = t0 + lrow[q];
      const int e = e0 + lrow[q];
      if (unorm && t < T) un2[(whole ? 0 : (int64_t)blockIdx.z * T) + t] = su;
      if (cnorm && e < E) cn[(whole ? 0 : (int64_t)blockIdx.z * E) + e] = whole ? sqrt(sc) : sc;
    }
  }
  // D layout of a 16x16 tile: lane holds rows 4*(lane/16)+r, column lane%16
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + wn * 32 + j * 16 + (lane & 15);
      if (e >= E) continue;
      const double b = (whole && bias) ? (double)bias[e] : 0.0;
      double *dst = logits + (whole ? 0 : (int64_t)blockIdx.z * T * E);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t t = t0 + wm * 32 + i * 16 + (lane >> 4) * 4 + r;
        if (t < T) dst[t * E + e] = acc64[i][j][r] + b;
      }
    }
}

// ------------------------------------- bf16 logits, wide tiles (N_r >= 192)
// Work-group tile: 64 tokens x 256 experts, so the token rows are read once
// per 256 experts (the 64 x 64 kernel above reads them once per 64).  Tiles of
// 64-deep k travel memory -> LDS by direct DMA (no staging registers) in a ring
// of 3 stages, 2 k-tiles ahead; LDS rows of 64 bf16 hold their 16-byte chunks
// XOR-swizzled (swz).  Eight waves, two per SIMD, so that one wave's fp64
// additions overlap the other's matrix-core work: wave w owns experts
// 32 w .. 32 w + 31 of the tile for all 64 tokens, two tiles of the 32x32x16
// bf16 matrix-core instruction with the expert fragment as the first operand,
// so lane l accumulates token l % 32 and, in register 4 q + c, expert
// 8 q + 4 (l / 32) + c of each 32 x 32 tile.  The fp32 chunk sums (one 64-deep
// k-tile: ROUTER_CHUNK products) are added into fp64 after every k-tile, in k
// order, as the 64 x 64 kernel does, so the same error bound holds.  The
// kernel serves token counts whose wide tiles fill the chip by themselves (no
// split-K), and it also writes each token's squared norm (work-groups of the
// first expert block, from the token tiles in LDS) and the router rows' norms
// (work-group (b, y) takes expert rows y * 256 + 8 b + w,
// y * 256 + 8 (b + gridDim.x) + w, ... from memory).
#define RW_BM 64
#define RW_BN 256
#define RW_WAVES 8
#define RW_MIN_EXPERTS 192  // the wide tiles serve layers with at least this many routed experts
#define RW_MIN_TILES 256    // ... and token counts with at least this many wide tiles

template <int S>
__device__ __forceinline__ uint16_t *rw_stage_a();
template <int S>
__device__ __forceinline__ uint16_t *rw_stage_b();
__shared__ __attribute__((aligned(16))) uint16_t rw_A0[RW_BM * RT_BK];
__shared__ __attribute__((aligned(16))) uint16_t rw_A1[RW_BM * RT_BK];
__shared__ __attribute__((aligned(16))) uint16_t rw_A2[RW_BM * RT_BK];
__shared__ __attribute__((aligned(16))) uint16_t rw_B0[RW_BN * RT_BK];
__shared__ __attribute__((aligned(16))) uint16_t rw_B1[RW_BN * RT_BK];
__shared__ __attribute__((aligned(16))) uint16_t rw_B2[RW_BN * RT_BK];
template <> __device__ __forceinline__ uint16_t *rw_stage_a<0>() { return rw_A0; }
template <> __device__ __forceinline__ uint16_t *rw_stage_a<1>() { return rw_A1; }
template <> __device__ __forceinline__ uint16_t *rw_stage_a<2>() { return rw_A2; }
template <> __device__ __forceinline__ uint16_t *rw_stage_b<0>() { return rw_B0; }
template <> __device__ __forceinline__ uint16_t *rw_stage_b<1>() { return rw_B1; }
template <> __device__ __forceinline__ uint16_t *rw_stage_b<2>() { return rw_B2; }

struct RwArgs {
  const uint16_t *u, *w;
  const float *bias;
  int64_t T;
  int E, d;
  double *logits;    // [T, E]
  double *unorm2;    // [T] squared token norms
  double *wnorm;     // [E] router row norms
  DiagWords *clear;  // the diagnostics header, zeroed by the first work-group (or NULL)
};

// DMA of k-tile kt into stage S: lane l of wave w fills LDS row 8 w + l / 8 of
// the A stage and rows 64 q + 8 w + l / 8 (q < 4) of the B stage, each with
// global chunk (l % 8) ^ swz(row) of that row: five instructions per wave.
// The rows were clamped into the matrix when the offsets were made (rows past
// T or E are loaded, never stored).
template <int S>
__device__ __forceinline__ void rw_issue(const __amdgpu_buffer_rsrc_t &ra, const __amdgpu_buffer_rsrc_t &rb,
                                         uint32_t aoff, const uint32_t (&boff)[4], int kt) {
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ko = kt * RT_BK * 2;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t *)(rw_stage_a<S>() + 8 * wv * RT_BK), 16, (int)aoff, ko,
                                           0, 0);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t *)(rw_stage_b<S>() + (64 * q + 8 * wv) * RT_BK), 16,
                                             (int)boff[q], ko, 0, 0);
}

// element offset of 16-byte chunk c of row r in a stage
__device__ __forceinline__ int rw_off(int r, int c) { return r * RT_BK + ((c ^ swz(r)) << 3); }

// One k-tile from stage S: 4 steps of 16, each one expert fragment x 2 token
// fragments; with NORM, this wave also adds the squares of its chunk (lane l:
// token 8 w + l / 8, elements 8 (l % 8) .. + 7) to nrm.
template <int S, bool NORM>
__device__ __forceinline__ void rw_compute(f32x16_t (&acc)[2], double &nrm) {
  const uint16_t *As = rw_stage_a<S>();
  const uint16_t *Bs = rw_stage_b<S>();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    const int ch = st * 2 + (lane >> 5);
    bf16x8_t a[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) a[i] = as_bf16x8(*(const uint4 *)&As[rw_off(32 * i + (lane & 31), ch)]);
    const bf16x8_t b = as_bf16x8(*(const uint4 *)&Bs[rw_off(32 * wv + (lane & 31), ch)]);
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a[i], acc[i], 0, 0, 0);
  }
  if (NORM) {
    const uint4 v = *(const uint4 *)&As[rw_off(8 * wv + (lane >> 3), lane & 7)];
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double lo = (double)__uint_as_float(w4[q] << 16), hi = (double)__uint_as_float(w4[q] & 0xffff0000u);
      nrm = fma(lo, lo, nrm);
      nrm = fma(hi, hi, nrm);
    }
  }
}

// fp32 chunk sums into the fp64 totals (in k order); the chunk accumulators restart
__device__ __forceinline__ void rw_flush(f32x16_t (&acc)[2], double (&acc64)[2][16]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc64[i][r] += (double)acc[i][r];
    acc[i] = f32x16_t{};
  }
}

// k-tile j from stage S = j % 3: wait until it has landed (the 5 DMA
// instructions of k-tile j + 1 may still be in flight) and every wave is past
// its reads of k-tile j - 1, refill that stage with k-tile j + 2, then the
// MFMAs and the flush.  Every trip issues its DMA, the last two re-loading the
// final k-tile into stages nothing reads again: with no DMA left out on any
// path, the compiler's per-stage tracking of pending LDS writes stays exact
// and it inserts no waits of its own before the fragment reads.
template <int S, bool NORM>
__device__ __forceinline__ void rw_iter(const __amdgpu_buffer_rsrc_t &ra, const __amdgpu_buffer_rsrc_t &rb,
                                        uint32_t aoff, const uint32_t (&boff)[4], int j, int n,
                                        f32x16_t (&acc)[2], double (&acc64)[2][16], double &nrm) {
  publish<5>();
  rw_issue<(S + 2) % 3>(ra, rb, aoff, boff, min(j + 2, n - 1));
  rw_compute<S, NORM>(acc, nrm);
  rw_flush(acc, acc64);
}

template <bool NORM>
__device__ __forceinline__ void rw_loop(const __amdgpu_buffer_rsrc_t &ra, const __amdgpu_buffer_rsrc_t &rb,
                                        uint32_t aoff, const uint32_t (&boff)[4], int n, double (&acc64)[2][16],
                                        double &nrm) {
  f32x16_t acc[2] = {f32x16_t{}, f32x16_t{}};
  rw_issue<0>(ra, rb, aoff, boff, 0);
  rw_issue<1>(ra, rb, aoff, boff, min(1, n - 1));
  int j = 0;
  for (; j + 3 <= n; j += 3) {
    rw_iter<0, NORM>(ra, rb, aoff, boff, j, n, acc, acc64, nrm);
    rw_iter<1, NORM>(ra, rb, aoff, boff, j + 1, n, acc, acc64, nrm);
    rw_iter<2, NORM>(ra, rb, aoff, boff, j + 2, n, acc, acc64, nrm);
  }
  // each remaining trip is reached only through the one before it, so every
  // path into a trip carries the same DMA history
  if (j < n) {
    rw_iter<0, NORM>(ra, rb, aoff, boff, j, n, acc, acc64, nrm);
    if (j + 1 < n) rw_iter<1, NORM>(ra, rb, aoff, boff, j + 1, n, acc, acc64, nrm);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the re-loads land before the work-group ends
}

__global__ __launch_bounds__(64 * RW_WAVES, 1) void router_logits_wide_kernel(RwArgs a) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  if (a.clear && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *a.clear = DiagWords{};
  const int64_t t0 = (int64_t)blockIdx.x * RW_BM;
  const int e0 = blockIdx.y * RW_BN;
  const int n = a.d / RT_BK;
  // buffer resources over the tile's 64 token rows and 256 router rows, so
  // that the 32-bit offsets never exceed them (rows clamped into the matrix)
  const int64_t tr = min((int64_t)RW_BM, a.T - t0);
  const int er = min(RW_BN, a.E - e0);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.u + t0 * a.d, (uint64_t)tr * a.d * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.w + (int64_t)e0 * a.d, (uint64_t)er * a.d * 2);
  const int arow = 8 * wv + (lane >> 3);
  const uint32_t aoff = (uint32_t)(min((int64_t)arow, tr - 1) * a.d * 2 + (((lane & 7) ^ swz(arow)) << 4));
  uint32_t boff[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 64 * q + 8 * wv + (lane >> 3);
    boff[q] = (uint32_t)((int64_t)min(row, er - 1) * a.d * 2 + (((lane & 7) ^ swz(row)) << 4));
  }
  double acc64[2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc64[i][r] = 0.0;
  double nrm = 0.0;
  const bool norms = blockIdx.y == 0;
  if (norms) rw_loop<true>(ra, rb, aoff, boff, n, acc64, nrm);
  else rw_loop<false>(ra, rb, aoff, boff, n, acc64, nrm);

  // logits (bias added): lane l, tile i, registers 4 q .. 4 q + 3: token
  // 32 i + l % 32, experts e .. e + 3 with e = 32 w + 8 q + 4 (l / 32) of the
  // tile, 32 contiguous bytes of the token's row
  const bool vec = (a.E & 1) == 0;  // rows of even length keep e (a multiple of 4) 16-byte aligned
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t t = t0 + 32 * i + (lane & 31);
    if (t >= a.T) continue;
    double *row = a.logits + t * a.E;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = e0 + 32 * wv + 8 * q + 4 * (lane >> 5);
      double v[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        v[c] = acc64[i][4 * q + c] + ((a.bias && e + c < a.E) ? (double)a.bias[e + c] : 0.0);
      if (vec && e + 3 < a.E) {
        *(double2 *)(row + e) = make_double2(v[0], v[1]);
        *(double2 *)(row + e + 2) = make_double2(v[2], v[3]);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (e + c < a.E) row[e + c] = v[c];
      }
    }
  }
  if (norms) {
    nrm += __shfl_xor(nrm, 1, 64);
    nrm += __shfl_xor(nrm, 2, 64);
    nrm += __shfl_xor(nrm, 4, 64);
    const int64_t t = t0 + 8 * wv + (lane >> 3);
    if ((lane & 7) == 0 && t < a.T) a.unorm2[t] = nrm;
  }
  // router row norms: rows e0 + 8 b + w, e0 + 8 (b + gridDim.x) + w, ... of
  // this expert block, one wave each
  for (int e = e0 + (int)blockIdx.x * RW_WAVES + wv; e < e0 + er; e += (int)gridDim.x * RW_WAVES) {
    double s2 = 0.0;
    const uint16_t *p = a.w + (int64_t)e * a.d;
    for (int i = lane * 8; i < a.d; i += 512) {
      const uint4 v = *(const uint4 *)(p + i);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const double lo = (double)__uint_as_float(w4[q] << 16), hi = (double)__uint_as_float(w4[q] & 0xffff0000u);
        s2 += lo * lo + hi * hi;
      }
    }
    s2 = wave_sum_f64(s2);
    if (lane == 0) a.wnorm[e] = sqrt(s2);
  }
}

// Sum over slices z = 0, 1, ..., S - 1 (in this order) of p[z * stride + i],
// the loads in batches of 8 that are in flight together.
__device__ __forceinline__ double slice_sum(const double *__restrict__ p, int S, int64_t stride, int64_t i) {
  double s = 0.0;
  for (int k0 = 0; k0 < S; k0 += 8) {
    double v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = k0 + q < S ? p[(int64_t)(k0 + q) * stride + i] : 0.0;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (k0 + q < S) s = (k0 + q == 0) ? v[q] : s + v[q];
  }
  return s;
}

// Thread i < n = T * E: logits[i] = the slices' partial sums of logit i + b_e;
// the next T threads: un2[t] = the slices' partial squared token norms; the
// next E: wn[e] = the square root of the slices' partial squared row norms.
__global__ __launch_bounds__(256) void router_reduce_kernel(const double *__restrict__ part, int S, int64_t n, int E,
                                                            const float *__restrict__ bias, double *__restrict__ logits,
                                                            int64_t T, const double *__restrict__ un2p,
                                                            const double *__restrict__ wnp, double *__restrict__ un2,
                                                            double *__restrict__ wn) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) {
    logits[i] = slice_sum(part, S, n, i) + (bias ? (double)bias[i % E] : 0.0);
  } else if (i < n + T) {
    un2[i - n] = slice_sum(un2p, S, T, i - n);
  } else if (i < n + T + E) {
    wn[i - n - T] = sqrt(slice_sum(wnp, S, E, i - n - T));
  }
}

// ------------------------------------------------------ fp32 logits (fp64 VALU)
// 16 tokens x 16 experts per work-group, one logit per thread, exact products.
__global__ __launch_bounds__(256) void router_logits_f32_kernel(const float *__restrict__ u,
                                                                const float *__restrict__ w,
                                                                const float *__restrict__ bias, int64_t T,
                                                                int E, int d, double *__restrict__ logits,
                                                                double *__restrict__ un2, double *__restrict__ wn,
                                                                DiagWords *clear) {
  __shared__ float As[16][65];
  __shared__ float Bs[16][65];
  if (clear && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *clear = DiagWords{};
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t t = (int64_t)blockIdx.x * 16 + ty;
  const int e = blockIdx.y * 16 + tx;
  // the squared norms from the same loads: lane l of wave w loads column l of
  // rows w, w + 4, w + 8, w + 12; the first expert tile's work-groups sum the
  // token rows, the first token tile's the router rows
  const bool unorm = blockIdx.y == 0, cnorm = blockIdx.x == 0;
  double usq[4] = {0.0, 0.0, 0.0, 0.0}, csq[4] = {0.0, 0.0, 0.0, 0.0};
  double acc = 0.0;
  // the next k-tile's elements are loaded while the current one is summed
  // (the same additions in the same order)
  float na[4], nb[4];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wv + 4 * i;
      const int64_t tr = (int64_t)blockIdx.x * 16 + r;
      const int er = blockIdx.y * 16 + r;
      na[i] = tr < T ? u[tr * d + k0 + lane] : 0.f;
      nb[i] = er < E ? w[(int64_t)er * d + k0 + lane] : 0.f;
    }
  };
  load(0);
  for (int k0 = 0; k0 < d; k0 += 64) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wv + 4 * i;
      As[r][lane] = na[i];
      Bs[r][lane] = nb[i];
      if (unorm) usq[i] = fma((double)na[i], (double)na[i], usq[i]);
      if (cnorm) csq[i] = fma((double)nb[i], (double)nb[i], csq[i]);
    }
    __syncthreads();
    if (k0 + 64 < d) load(k0 + 64);
#pragma unroll 8
    for (int kk = 0; kk < 64; ++kk) acc += (double)As[ty][kk] * (double)Bs[tx][kk];
    __syncthreads();
  }
  if (t < T && e < E) logits[t * E + e] = acc + (bias ? (double)bias[e] : 0.0);
  if (unorm || cnorm) {  // only the first row and column of work-groups hold norms
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wv + 4 * i;
      const double su = dpp_wave_sum_f64(usq[i]), sc = dpp_wave_sum_f64(csq[i]);
      const int64_t tr = (int64_t)blockIdx.x * 16 + r;
      const int er = blockIdx.y * 16 + r;
      if (lane == 0 && unorm && tr < T) un2[tr] = su;
      if (lane == 0 && cnorm && er < E) wn[er] = sqrt(sc);
    }
  }
}

hipError_t launch_router_logits(const moe_dims &dm, int64_t T, const void *u, const void *w_router,
                                const float *bias, const WsLayout &L, char *ws, bool clear_diag, hipStream_t st) {
  const int E = dm.n_routed, d = dm.d_model;
  double *logits = (double *)(ws + L.logits);
  double *un2 = (double *)(ws + L.unorm2);
  double *wn = (double *)(ws + L.wnorm);
  DiagWords *clear = clear_diag ? (DiagWords *)(ws + L.diag) : nullptr;
  if (dm.dtype == MOE_BF16) {
    const int nk = d / RT_BK;
    const int S = router_splits(dm, T);
    const int kps = (nk + S - 1) / S;
    const int64_t wide_tiles = ((T + RW_BM - 1) / RW_BM) * ((E + RW_BN - 1) / RW_BN);
    if (E >= RW_MIN_EXPERTS && wide_tiles >= RW_MIN_TILES) {
      // wide tiles fill the chip without split-K; the norms come out of the same kernel
      RwArgs ra{(const uint16_t *)u, (const uint16_t *)w_router, bias, T, E, d, logits, un2, wn, clear};
      dim3 grid((unsigned)((T + RW_BM - 1) / RW_BM), (unsigned)((E + RW_BN - 1) / RW_BN));
      router_logits_wide_kernel<<<grid, 64 * RW_WAVES, 0, st>>>(ra);
      return hipGetLastError();
    }
    dim3 grid((unsigned)((T + RT_BM - 1) / RT_BM), (unsigned)((E + RT_BN - 1) / RT_BN), (unsigned)S);
    if (S == 1) {
      router_logits_bf16_kernel<<<grid, 256, 0, st>>>((const uint16_t *)u, (const uint16_t *)w_router, bias, T, E, d,
                                                      kps, logits, un2, wn, clear);
    } else {
      double *part = (double *)(ws + L.logit_part);
      double *un2p = (double *)(ws + L.norm_part), *wnp = un2p + (size_t)S * T;
      router_logits_bf16_kernel<<<grid, 256, 0, st>>>((const uint16_t *)u, (const uint16_t *)w_router, bias, T, E, d,
                                                      kps, part, un2p, wnp, clear);
      const int64_t n = T * E, threads = n + T + E;
      router_reduce_kernel<<<dim3((unsigned)((threads + 255) / 256)), 256, 0, st>>>(part, S, n, E, bias, logits, T,
                                                                                   un2p, wnp, un2, wn);
    }
  } else {
    dim3 grid((unsigned)((T + 15) / 16), (unsigned)((E + 15) / 16));
    router_logits_f32_kernel<<<grid, 256, 0, st>>>((const float *)u, (const float *)w_router, bias, T, E, d, logits,
                                                   un2, wn, clear);
  }
  return hipGetLastError();
}

// Coefficient of ||u|| ||c|| in the logit error bound (see the file header).
double router_bound_coeff(const moe_dims &dm) {
  const double d = dm.d_model;
  if (dm.dtype == MOE_BF16) return ROUTER_CHUNK * 0x1p-22 + (d / ROUTER_CHUNK + 2.0) * 0x1p-52;
  return (d + 2.0) * 0x1p-52;
}
