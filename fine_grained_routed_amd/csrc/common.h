// Device and host helpers shared by the library's HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

#define MOE_WAVE 64

// ----------------------------------------------------------------- bf16 helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// fp32 -> bf16, round to nearest even (NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// two fp32 -> packed bf16 pair (lo in bits 0..15), round to nearest even, by
// the hardware conversion
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// SiLU(g) = g * sigmoid(g) with the hardware exponential and reciprocal (a few
// ulp of fp32, far below the bf16 rounding that follows)
__device__ __forceinline__ float silu_fast(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  union { uint4 u; bf16x8_t b; } c;
  c.u = v;
  return c.b;
}

// keep v when ok, else zeros (component-wise, so it stays in registers)
__device__ __forceinline__ uint4 keep_or_zero(bool ok, uint4 v) {
  const uint32_t m = ok ? 0xffffffffu : 0u;
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// ------------------------------------------------- direct-to-LDS DMA helpers
// (used by the tiled matrix-core kernels: the prefill grouped GEMMs and the
// router logits)
typedef __attribute__((address_space(3))) void lds_void_t;

// LDS rows of 64 bf16 hold eight 16-byte chunks; chunk c of row r sits in slot
// c ^ swz(r).  swz is one-to-one on any 8 consecutive rows and on any 8 rows
// of one parity among 16 consecutive rows, so the 16-byte fragment reads of 8
// (or 16) consecutive rows fall on distinct banks whether the LDS serves 8
// lanes over 32 banks or 16 lanes over 64 banks per cycle.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Buffer resource over `bytes` bytes at `base` (raw buffer: no stride, 32-bit
// data format), the form the buffer-to-LDS loads address memory through.
// Accesses past `bytes` read zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0,
                                           (int)(uint32_t)min(bytes, (uint64_t)0xffffffffu), 0x00020000);
}

// s_waitcnt immediate (gfx9 layout: vmcnt [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8]) for "at most vm vector-memory operations outstanding, LDS
// and scalar loads complete".  The builtin, unlike inline asm, is visible to
// the compiler's own wait tracking, which then knows that older DMA into a
// stage has landed.
constexpr int waitcnt_vm(int vm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4); }

// Publish LDS to the work-group: this wave's LDS reads are complete and at
// most `vm` DMA instructions are still in flight, then the work-group barrier.
// Written out rather than __syncthreads(), whose release fence would also
// wait for every DMA in flight and so drain the prefetch.
template <int VM>
__device__ __forceinline__ void publish() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(VM));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------ wave reductions
// Wave-wide fp64 max and sum, uniform: four DPP steps (lane i meets lanes
// i ^ 1, i ^ 2, then its mirror in 8 and in 16) leave every row of 16 lanes
// holding its row's result; two row broadcasts then fold row 0 into row 1,
// row 2 into row 3 and row 1 into row 3, and lane 63's value is the result.
// The order of the additions is fixed, so the sum is reproducible.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double old, double v) {
  const long long o = __double_as_longlong(old), b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp((int)o, (int)b, CTRL, ROWS, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp((int)(o >> 32), (int)(b >> 32), CTRL, ROWS, 0xf, false);
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, l), hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}
#define DPP_XOR1 0xB1       // quad_perm [1, 0, 3, 2]
#define DPP_XOR2 0x4E       // quad_perm [2, 3, 0, 1]
#define DPP_HALF_MIRROR 0x141
#define DPP_MIRROR 0x140
#define DPP_BCAST15 0x142   // lane 15 of each row into the next row
#define DPP_BCAST31 0x143   // lane 31 into rows 2 and 3
__device__ __forceinline__ double dpp_wave_max_f64(double v) {
  v = fmax(v, dpp_f64<DPP_XOR1, 0xf>(v, v));
  v = fmax(v, dpp_f64<DPP_XOR2, 0xf>(v, v));
  v = fmax(v, dpp_f64<DPP_HALF_MIRROR, 0xf>(v, v));
  v = fmax(v, dpp_f64<DPP_MIRROR, 0xf>(v, v));
  v = fmax(v, dpp_f64<DPP_BCAST15, 0xa>(v, v));  // rows outside the mask keep v
  v = fmax(v, dpp_f64<DPP_BCAST31, 0xc>(v, v));
  return readlane_f64(v, 63);
}
__device__ __forceinline__ double dpp_wave_sum_f64(double v) {
  v += dpp_f64<DPP_XOR1, 0xf>(0.0, v);
  v += dpp_f64<DPP_XOR2, 0xf>(0.0, v);
  v += dpp_f64<DPP_HALF_MIRROR, 0xf>(0.0, v);
  v += dpp_f64<DPP_MIRROR, 0xf>(0.0, v);
  v += dpp_f64<DPP_BCAST15, 0xa>(0.0, v);  // rows outside the mask add 0
  v += dpp_f64<DPP_BCAST31, 0xc>(0.0, v);
  return readlane_f64(v, 63);
}

__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_max_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ long long wave_sum_i64(long long v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------- workspace layout
// The diagnostics header sits at offset 0 of every workspace.
#define MOE_DIAG_UNRESOLVED 1u
#define MOE_DIAG_BAD_INDEX 2u
#define MOE_DIAG_DUPLICATE 4u

struct DiagWords {
  uint32_t flags;
  uint32_t tokens_exact;
  uint32_t exact_keys;
  uint32_t refinements;
  uint32_t deferred;  // tokens the first top-k kernel left to the second (not part of moe_diag)
};

// Up to this many tokens the cooperative top-k kernel takes every token;
// above it, the wavefront-per-token kernel first settles the clear ones and
// lists the rest (int32 [T] in the workspace).
#define MOE_TOPK_COOP_ALL 1024

// M-tile heights for which the permutation writes per-expert tile prefixes.
#define MOE_N_BM 5
__host__ __device__ constexpr int moe_bm_of(int i) { return 16 << i; }  // 16 32 64 128 256

// Largest top-k a layer may have (kernels hold a token's slots in registers).
#define MOE_MAX_TOPK 16

// Tokens per call (keeps the per-token dispatches under 2^32 work-items).
#define MOE_MAX_TOKENS (1 << 22)

// Routing block: tokens per permutation work-group.
#define MOE_PERM_BLOCK 256

// Slices of the router reduction (bf16): enough work-groups of 64 x 64
// logits to fill the chip, each slice at least 2 k-tiles of 64 and none
// empty: with kps = ceil(nk / S) k-tiles per slice, (S - 1) * kps < nk.
static inline int router_splits(const moe_dims &dm, int64_t T) {
  if (dm.dtype != MOE_BF16 || T <= 0 || dm.n_routed <= 0) return 1;
  const int64_t nk = dm.d_model / 64;
  const int64_t tiles = ((T + 63) / 64) * ((dm.n_routed + 63) / 64);
  const int64_t want = 256 / tiles;
  const int64_t cap = nk / 2;
  int64_t s = want < cap ? want : cap;
  if (s <= 1) return 1;
  const int64_t kps = (nk + s - 1) / s;
  return (int)((nk + kps - 1) / kps);
}

struct WsLayout {
  size_t diag;        // DiagWords
  size_t logits;      // double [T, N_r]
  size_t logit_part;  // double [S, T, N_r] router partial sums (S = router_splits > 1 only)
  size_t norm_part;   // double [S, T] then [S, N_r]: the slices' partial squared norms (S > 1 only)
  size_t unorm2;      // double [T]   squared 2-norm of each token row
  size_t wnorm;       // double [N_r] 2-norm of each router row
  size_t blk;         // int32  [nblk, N_r] per-block histograms, then bases
  size_t tile_off;    // int32  [MOE_N_BM, N_r + 2] per-expert m-tile prefixes (+ shared)
  size_t h;           // bf16 or f32 [R, f] routed hidden activations
  size_t h_sh;        // bf16 or f32 [T, f_s] shared hidden activations
  size_t topk_idx;    // int32 [T, k]  (layer forward only)
  size_t topk_w;      // f32   [T, k]
  size_t topk_list;   // int32 [T]     tokens left to the cooperative top-k kernel (T > MOE_TOPK_COOP_ALL only)
  size_t counts;      // int32 [N_r]
  size_t offsets;     // int32 [N_r + 1]
  size_t row_token;   // int32 [R]
  size_t token_row;   // int32 [T, k]
  size_t y_rows;      // f32 [R, d]
  size_t y_sh;        // f32 [T, d]
  size_t u_norm;      // dtype [T, d] RMS-normalised input (block forward only)
  size_t dense_part;  // f32 split-reduction partials of the dense decode path (dense bf16 layers only)
  size_t total;
};

// Dense decode path: rows per pass; tile widths and reduction slices.
#define MOE_DD_ROWS 256
#ifndef MOE_DD_SPLIT_GU
#define MOE_DD_SPLIT_GU 4  // reduction slices of the single-wave kernel (passes under 33 rows), gate/up
#endif
#ifndef MOE_DD_SPLIT_DN
#define MOE_DD_SPLIT_DN 8  // the same for the down pass
#endif
#define MOE_DD_SPLIT_MAX 8
#ifndef MOE_DD_WG_GU
#define MOE_DD_WG_GU 1152  // work-groups the four-wave kernel aims at (slices x column groups x row blocks), gate/up
#endif
#ifndef MOE_DD_WG_DN
#define MOE_DD_WG_DN 448  // the same for the down pass
#endif
#ifndef MOE_DD_NT_GU
#define MOE_DD_NT_GU 1  // 16-column tiles per wave of the four-wave kernel, gate/up (each of gate and up)
#endif
#ifndef MOE_DD_NT_DN
#define MOE_DD_NT_DN 2  // the same for the down pass
#endif
#ifndef MOE_DD_UL_GU
#define MOE_DD_UL_GU 4  // 32-deep steps per batch of the four-wave dense decode kernel (gate/up)
#endif
#ifndef MOE_DD_UL_DN
#define MOE_DD_UL_DN 2  // the same for the down pass
#endif

static inline size_t moe_align(size_t x) { return (x + 255) & ~(size_t)255; }

// Whether a dense decode pass of `rows` rows runs the four-wave kernel (three
// or more 16-row blocks) rather than the single-wave one.
static inline bool moe_dd_four_wave(int rows) { return ((rows < 64 ? rows : 64) + 15) / 16 >= 3; }

// Reduction slices of a dense decode pass of `rows` rows with N output
// columns: the four-wave kernel takes as many as give about MOE_DD_WG_*
// work-groups in all (1 to MOE_DD_SPLIT_MAX), the single-wave kernel a fixed
// count.
static inline int moe_dd_splits(bool gateup, int64_t N, int rows) {
  if (!moe_dd_four_wave(rows)) return gateup ? MOE_DD_SPLIT_GU : MOE_DD_SPLIT_DN;
  const int64_t cols = 64 * (gateup ? MOE_DD_NT_GU : MOE_DD_NT_DN);
  const int64_t wg = (N + cols - 1) / cols * ((rows + 63) / 64);
  if (wg <= 0) return 1;
  const int64_t target = gateup ? MOE_DD_WG_GU : MOE_DD_WG_DN;
  const int64_t s = (target + wg / 2) / wg;
  return (int)(s < 1 ? 1 : s > MOE_DD_SPLIT_MAX ? MOE_DD_SPLIT_MAX : s);
}

static inline WsLayout moe_ws_layout(const moe_dims &dm, int64_t T) {
  WsLayout L;
  const size_t E = (size_t)dm.n_routed, k = (size_t)dm.top_k, d = (size_t)dm.d_model;
  const size_t R = (size_t)T * k, f = (size_t)dm.d_ff, fs = (size_t)dm.d_ff_shared;
  const size_t hbytes = dm.dtype == MOE_BF16 ? 2 : 4;
  const size_t nblk = ((size_t)T + MOE_PERM_BLOCK - 1) / MOE_PERM_BLOCK;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = moe_align(o + bytes); return at; };
  L.diag = take(256);
  L.logits = take((size_t)T * E * 8);
  const int S = router_splits(dm, T);
  L.logit_part = take(S > 1 ? (size_t)S * T * E * 8 : 0);
  L.norm_part = take(S > 1 ? (size_t)S * ((size_t)T + E) * 8 : 0);
  L.unorm2 = take((size_t)T * 8);
  L.wnorm = take(E * 8);
  L.blk = take(nblk * E * 4);
  L.tile_off = take((size_t)MOE_N_BM * (E + 2) * 4);
  L.h = take(R * f * hbytes);
  L.h_sh = take((size_t)T * fs * hbytes);
  L.topk_idx = take(R * 4);
  L.topk_w = take(R * 4);
  L.topk_list = take(T > MOE_TOPK_COOP_ALL && E > 0 ? (size_t)T * 4 : 0);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.row_token = take(R * 4);
  L.token_row = take(R * 4);
  L.y_rows = take(R * d * 4);
  L.y_sh = take((size_t)T * d * 4);
  L.u_norm = take((size_t)T * d * hbytes);
  {  // the partials of the largest pass: a full one, or the last (shorter) one
    size_t need = 0;
    const int64_t cand[2] = {T < MOE_DD_ROWS ? T : MOE_DD_ROWS, T % MOE_DD_ROWS};
    for (int64_t r : cand) {
      if (r <= 0 || E != 0 || dm.dtype != MOE_BF16) continue;
      const size_t gu = (size_t)moe_dd_splits(true, (int64_t)fs, (int)r) * r * 2 * fs;
      const size_t dn = (size_t)moe_dd_splits(false, (int64_t)d, (int)r) * r * d;
      need = need > gu ? need : gu;
      need = need > dn ? need : dn;
    }
    L.dense_part = take(E == 0 && dm.dtype == MOE_BF16 ? 4 * need : 0);
  }
  L.total = o;
  return L;
}

// ------------------------------------------------------ kernel launch wrappers
// Implemented in the per-stage sources; all enqueue on `st` and return the
// launch status.
hipError_t launch_diag_clear(void *ws, hipStream_t st);
// clear_diag: the first kernel also zeroes the diagnostics header (saving a launch).
hipError_t launch_router_logits(const moe_dims &dm, int64_t T, const void *u, const void *w_router,
                                const float *bias, const WsLayout &L, char *ws, bool clear_diag, hipStream_t st);
hipError_t launch_topk(const moe_dims &dm, int64_t T, const void *u, const void *w_router, const float *bias,
                       int32_t *topk_idx, float *topk_w, const WsLayout &L, char *ws, hipStream_t st);
hipError_t launch_permute(const moe_dims &dm, int64_t T, const int32_t *topk_idx, int32_t *counts,
                          int32_t *offsets, int32_t *row_token, int32_t *token_row, const WsLayout &L,
                          char *ws, hipStream_t st);
hipError_t launch_tile_offsets(const moe_dims &dm, int64_t T, const int32_t *counts, const WsLayout &L,
                               char *ws, hipStream_t st);
// T <= MOE_PERM_BLOCK: the permutation and (tile_off non-NULL) the tile prefixes in one launch
hipError_t launch_permute_small(const moe_dims &dm, int64_t T, const int32_t *topk_idx, int32_t *counts,
                                int32_t *offsets, int32_t *row_token, int32_t *token_row, int32_t *tile_off,
                                const WsLayout &L, char *ws, hipStream_t st);
hipError_t launch_ffn_f32(const moe_dims &dm, int64_t T, const void *u, const moe_weights &w, const int32_t *offsets,
                          const int32_t *row_token, float *y_rows, float *y_sh, const WsLayout &L, char *ws,
                          hipStream_t st, hipEvent_t ev_mid);
hipError_t launch_ffn_prefill_bf16(const moe_dims &dm, int64_t T, const void *u, const moe_weights &w,
                                   const int32_t *offsets, const int32_t *row_token, float *y_rows, float *y_sh,
                                   const WsLayout &L, char *ws, hipStream_t st, hipEvent_t ev_mid);
hipError_t launch_ffn_decode(const moe_dims &dm, int64_t T, const void *u, const moe_weights &w,
                             const int32_t *counts, const int32_t *offsets, const int32_t *row_token,
                             float *y_rows, float *y_sh, const WsLayout &L, char *ws, hipStream_t st,
                             hipEvent_t ev_mid);
// The largest 1-D grid, in work-groups of 256, that each expert-FFN launcher
// would dispatch for T tokens (the host checks it before enqueueing).
int64_t ffn_prefill_max_workgroups(const moe_dims &dm, int64_t T);
int64_t ffn_decode_max_workgroups(const moe_dims &dm, int64_t T);
int64_t ffn_f32_max_workgroups(const moe_dims &dm, int64_t T);
// resid: NULL, or the block's raw input x [T, d] in dm.dtype, added last
hipError_t launch_combine(const moe_dims &dm, int64_t T, const float *y_rows, const float *y_sh,
                          const float *topk_w, const int32_t *token_row, const void *resid, void *out,
                          hipStream_t st);
hipError_t launch_rmsnorm(const moe_dims &dm, int64_t T, const void *x, const float *gamma, double eps, void *u,
                          hipStream_t st);
