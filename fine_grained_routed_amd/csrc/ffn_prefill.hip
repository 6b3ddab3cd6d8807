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
// (down).  4 waves in a 2 x 2 layout: each wave owns 128 rows and 128
// B-columns (gate/up: 64 gate + the matching 64 up columns) as 4 x 4 tiles
// of the 32x32x16 bf16 matrix-core instruction, 256 fp32 accumulators per
// lane; per 16-deep step a wave reads 8 fragments from LDS for 16
// instructions, and issues the next step's 8 reads under the first 8 of them.
// A wave skips the 32-row sub-tiles past the group's last row, so a ragged
// tail costs in proportion to its rows.  Both
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
// Work-groups are dispatched round-robin over the 8 XCDs.  The tile order
// (described in the kernel) is cut into chunks of CH consecutive tiles (64 for
// gate/up, 32 for down), dealt to the XCDs in turn: work-group i, the (i / 8)-th
// of XCD i % 8, takes tile (((i / 8) / CH) * 8 + i % 8) * CH + (i / 8) % CH.  The
// 32 CUs of an XCD work through one chunk at a time, mostly one expert,
// sharing its token rows and weight panels in that XCD's L2, and every XCD
// receives an even share of full and ragged tiles.
#include <algorithm>
#include <utility>

#include "common.h"

#define PF_BM 256
#define PF_BN 256    // B rows per tile (gate/up: 128 gate + 128 up)
#define PF_BK 64
#define PF_BM_IDX 4  // moe_bm_of(4) == 256
#define PF_WM 4      // 32-row sub-tiles per wave (2 x 2 waves over 8 sub-tiles)
#define PF_GM 8      // m-tiles per ordering block (routed experts)
#define PF_CHUNK_GU 64  // consecutive tiles dealt to one XCD (gate/up)
#define PF_CHUNK_DN 32  // consecutive tiles dealt to one XCD (down; 3.22 against 3.73 ms for the dense layer's)
#define PF_GM_SH 4   // m-tiles per ordering block (shared group)
#define PF_LOADS 8   // DMA instructions per wave per operand per k-tile (8 rows of 128 B each)
#define PF_NT 2      // cache-policy bits of a non-temporal load

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
  int64_t rows_a, rows_a_sh;  // rows of A and A_sh (bounds of their buffer resources)
  int E, K, K_sh, N, N_sh, has_shared;
  int bnt;                   // single-m-tile experts' weights by non-temporal DMA
  int nt_r, nt_s;            // column tiles of a routed / the shared group
  int mt_s;                  // m-tiles of the shared group (0 without one)
};

// element offset of 16-byte chunk c of LDS row r
__device__ __forceinline__ int lds_off(int r, int c) { return r * PF_BK + ((c ^ swz(r)) << 3); }

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

// One operand's DMA sources: a buffer resource over the matrix the wave's
// rows come from and each lane's byte offset for its 8 row segments.
struct Operand {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t off[PF_LOADS];
};

// DMA of one operand's k-tile kt, 16 bytes per lane straight from memory into
// LDS at stage row 64w + 8q (lane l lands at +16 l): wave w fills LDS rows
// 64w + 8q .. 64w + 8q + 7 (q < 8); lane l writes row 64w + 8q + l/8, slot
// l%8, which holds global chunk (l%8) ^ swz(row) (folded into the offsets).
// The k-tile's position is the scalar offset, so advancing costs one add.
// The immediate offset applies to both the memory and the LDS address, so
// row group q is reached as LDS base + (q % 4) KB through the immediate, with
// the memory offset stored less that amount: a wave needs two LDS bases per
// stage instead of eight.
// AUX: the loads' cache policy (0 cached, PF_NT non-temporal).
template <int Q, int AUX>
__device__ __forceinline__ void dma_group(const Operand &op, uint16_t *wstage, int koff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(op.rsrc, (lds_void_t *)(wstage + 8 * (Q & ~3) * PF_BK), 16, (int)op.off[Q],
                                           koff, (Q & 3) * 1024, AUX);
}

template <int Q0, int AUX, int... Qs>
__device__ __forceinline__ void issue_groups(const Operand &op, uint16_t *wstage, int koff,
                                             std::integer_sequence<int, Qs...>) {
  (dma_group<Q0 + Qs, AUX>(op, wstage, koff), ...);
}

template <int Q0 = 0, int Q1 = PF_LOADS, int AUX = 0>
__device__ __forceinline__ void issue_op(const Operand &op, uint16_t *stage, int kt) {
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  issue_groups<Q0, AUX>(op, stage + 64 * wv * PF_BK, kt * (PF_BK * 2), std::make_integer_sequence<int, Q1 - Q0>{});
}

// Fragments of one 16-deep step: MW A row tiles and four B column tiles.
template <int MW>
struct Frags {
  bf16x8_t a[PF_WM], b[4];
};

// Fragment rows of the wave's tiles inside the LDS stages.
struct WaveRows {
  int a0;     // first A row of the wave (0 or 128)
  int b[4];   // first B row of each column tile
};

// Reads in the order the next step consumes them: a0, the four B tiles, a1..
template <int MW, int SA, int SB>
__device__ __forceinline__ void read_frags(Frags<MW> &f, const WaveRows &w, int step) {
  const uint16_t *As = stage_a<SA>();
  const uint16_t *Bs = stage_b<SB>();
  const int lane = threadIdx.x & 63;
  const int frow = lane & 31;             // fragment row inside a 32-row tile
  const int ch = step * 2 + (lane >> 5);  // chunk: first/second 8 of the 16-deep step
  if (MW > 0) f.a[0] = as_bf16x8(*(const uint4 *)&As[lds_off(w.a0 + frow, ch)]);
#pragma unroll
  for (int j = 0; j < 4; ++j) f.b[j] = as_bf16x8(*(const uint4 *)&Bs[lds_off(w.b[j] + frow, ch)]);
#pragma unroll
  for (int i = 1; i < MW; ++i) f.a[i] = as_bf16x8(*(const uint4 *)&As[lds_off(w.a0 + i * 32 + frow, ch)]);
}

// The weight fragment is the first operand, so each accumulator holds the
// transposed product: a lane owns one token row (lane % 32) and, per group of
// four registers, four consecutive output columns, which the epilogue stores
// as one vector.
template <int MW>
__device__ __forceinline__ void mfma_step(const Frags<MW> &f, f32x16_t (&acc)[PF_WM][4]) {
#pragma unroll
  for (int i = 0; i < MW; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

// One fragment read after each of the step's first MFMAs, so that every read
// of the next step is issued early and has the remaining MFMAs to land; the
// step's share of weight-tile DMA (ND instructions) goes under the rest.
template <int MW, int ND>
__device__ __forceinline__ void interleave_hint() {
  constexpr int nm = 4 * MW, nr = MW > 0 ? 4 + MW : 0;
#pragma unroll
  for (int t = 0; t < nr; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
#pragma unroll
  for (int t = 0; t < ND; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
  if (nm > nr + ND) __builtin_amdgcn_sched_group_barrier(0x008, nm - nr - ND, 0);
}

// MFMAs of step 3 after the barrier: the step-0 fragment reads of the next
// tile go under the first MFMAs, the token-tile DMA under the rest.
template <int MW>
__device__ __forceinline__ void post_barrier_hint() {
  constexpr int nm = 4 * MW, nr = MW > 0 ? 4 + MW : 0;
#pragma unroll
  for (int t = 0; t < nr; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
#pragma unroll
  for (int t = nr; t < nm; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
}

// One k-tile j, its token rows in A-stage SA (= j % 2) and weights in B-stage
// SB (= j % 3).  f0 holds its step-0 fragments on entry and the next tile's
// step-0 fragments on exit.  DMA is spread over the iteration so that the
// memory pipeline never holds a burst: the weight tile j + 2 goes into the
// B stage of tile j - 1 under steps 0-2 (3 + 3 + 2 instructions), and after
// the barrier that publishes tile j + 1 the token tile j + 2 goes into the A
// stage of tile j, now free.  Past the end the last tile is re-fetched into
// stages nobody reads again, so every iteration issues the same DMA and one
// constant wait publishes the next tile: when it runs, only the weight tile
// issued in this iteration may be in flight.  A wave without token-tile DMA
// (adma false: its rows are past the tile's valid sub-tiles) issues the weight
// DMA alone, and the same wait still leaves only that tile in flight.
template <int MW, int SA, int SB, int BAUX>
__device__ __forceinline__ void k_iter(const Operand &A, const Operand &B, const WaveRows &w, int j, int nk,
                                       Frags<MW> &f0, Frags<MW> &f1, f32x16_t (&acc)[PF_WM][4], bool adma) {
  const int kb = min(j + 2, nk - 1);
  if (MW > 0) read_frags<MW, SA, SB>(f1, w, 1);
  issue_op<0, 3, BAUX>(B, stage_b<(SB + 2) % 3>(), kb);
  if (MW > 0) {
    mfma_step<MW>(f0, acc);
    interleave_hint<MW, 3>();
    read_frags<MW, SA, SB>(f0, w, 2);
  }
  issue_op<3, 6, BAUX>(B, stage_b<(SB + 2) % 3>(), kb);
  if (MW > 0) {
    mfma_step<MW>(f1, acc);
    interleave_hint<MW, 3>();
    read_frags<MW, SA, SB>(f1, w, 3);
  }
  issue_op<6, 8, BAUX>(B, stage_b<(SB + 2) % 3>(), kb);
  if (MW > 0) {
    mfma_step<MW>(f0, acc);
    interleave_hint<MW, 2>();
  }
  publish<PF_LOADS>();  // A and B tiles j + 1 landed
  // step-0 fragments of tile j + 1 (after the last tile this reads stages
  // whose values are never used; reading LDS is always in bounds)
  if (MW > 0) read_frags<MW, SA ^ 1, (SB + 1) % 3>(f0, w, 0);
  if (adma) issue_op(A, stage_a<SA>(), min(j + 2, nk - 1));
  if (MW > 0) {
    mfma_step<MW>(f1, acc);
    post_barrier_hint<MW>();
  }
}

// The k loop of one tile for a wave with MW valid 32-row sub-tiles
// (compile-time, so the body is straight-line).  Every wave of the
// work-group, whatever its MW, issues the same weight-tile DMA and barriers;
// token-tile DMA only when some of its 64 rows are read (adma).
template <int MW, int BAUX>
__device__ __forceinline__ void k_loop(const Operand &A, const Operand &B, const WaveRows &w, int K,
                                       f32x16_t (&acc)[PF_WM][4], bool adma) {
  const int nk = K / PF_BK;
  // prologue: A tiles 0, 1 and B tiles 0, 1 (clamped), issued in the order the
  // loop's constant wait assumes
  if (adma) issue_op(A, stage_a<0>(), 0);
  issue_op<0, PF_LOADS, BAUX>(B, stage_b<0>(), 0);
  issue_op<0, PF_LOADS, BAUX>(B, stage_b<1>(), min(1, nk - 1));
  if (adma) issue_op(A, stage_a<1>(), min(1, nk - 1));
  // A0 and B0 landed (a wave without token DMA has only B1 left in flight)
  if (adma) publish<2 * PF_LOADS>();
  else publish<PF_LOADS>();
  Frags<MW> f0, f1;
  if (MW > 0) read_frags<MW, 0, 0>(f0, w, 0);
  // six k-tiles per trip (the stage pattern repeats every lcm(2, 3) tiles);
  // whole trips are unconditional, the remainder follows
  int j = 0;
  for (; j + 6 <= nk; j += 6) {
    k_iter<MW, 0, 0, BAUX>(A, B, w, j, nk, f0, f1, acc, adma);
    k_iter<MW, 1, 1, BAUX>(A, B, w, j + 1, nk, f0, f1, acc, adma);
    k_iter<MW, 0, 2, BAUX>(A, B, w, j + 2, nk, f0, f1, acc, adma);
    k_iter<MW, 1, 0, BAUX>(A, B, w, j + 3, nk, f0, f1, acc, adma);
    k_iter<MW, 0, 1, BAUX>(A, B, w, j + 4, nk, f0, f1, acc, adma);
    k_iter<MW, 1, 2, BAUX>(A, B, w, j + 5, nk, f0, f1, acc, adma);
  }
  if (j < nk) k_iter<MW, 0, 0, BAUX>(A, B, w, j, nk, f0, f1, acc, adma);
  if (j + 1 < nk) k_iter<MW, 1, 1, BAUX>(A, B, w, j + 1, nk, f0, f1, acc, adma);
  if (j + 2 < nk) k_iter<MW, 0, 2, BAUX>(A, B, w, j + 2, nk, f0, f1, acc, adma);
  if (j + 3 < nk) k_iter<MW, 1, 0, BAUX>(A, B, w, j + 3, nk, f0, f1, acc, adma);
  if (j + 4 < nk) k_iter<MW, 0, 1, BAUX>(A, B, w, j + 4, nk, f0, f1, acc, adma);
  // the trailing re-fetches must land before the work-group can exit
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
}

// Sixteen 16-byte LDS reads at addr + off[k] issued back to back, then one
// wait: the epilogue's read-backs travel together instead of one LDS round
// trip per output store (the compiler would otherwise place each read next to
// its store).  The wait is inside the same statement, so no result register
// is used or reused before its read has landed.
#define PF_LDS16_OFFS(S, B) "i"((B) + 0 * (S)), "i"((B) + 1 * (S)), "i"((B) + 2 * (S)), "i"((B) + 3 * (S))
#define PF_LDS_READ16(v, addr, SI, SJ)                                                                         \
  asm volatile(                                                                                              \
      "ds_read_b128 %0, %16 offset:%17\n\tds_read_b128 %1, %16 offset:%18\n\t"                           \
      "ds_read_b128 %2, %16 offset:%19\n\tds_read_b128 %3, %16 offset:%20\n\t"                           \
      "ds_read_b128 %4, %16 offset:%21\n\tds_read_b128 %5, %16 offset:%22\n\t"                           \
      "ds_read_b128 %6, %16 offset:%23\n\tds_read_b128 %7, %16 offset:%24\n\t"                           \
      "ds_read_b128 %8, %16 offset:%25\n\tds_read_b128 %9, %16 offset:%26\n\t"                           \
      "ds_read_b128 %10, %16 offset:%27\n\tds_read_b128 %11, %16 offset:%28\n\t"                         \
      "ds_read_b128 %12, %16 offset:%29\n\tds_read_b128 %13, %16 offset:%30\n\t"                         \
      "ds_read_b128 %14, %16 offset:%31\n\tds_read_b128 %15, %16 offset:%32\n\t"                         \
      "s_waitcnt lgkmcnt(0)"                                                                                 \
      : "=v"(v[0]), "=v"(v[1]), "=v"(v[2]), "=v"(v[3]), "=v"(v[4]), "=v"(v[5]), "=v"(v[6]), "=v"(v[7]),      \
        "=v"(v[8]), "=v"(v[9]), "=v"(v[10]), "=v"(v[11]), "=v"(v[12]), "=v"(v[13]), "=v"(v[14]), "=v"(v[15]) \
      : "v"(addr), PF_LDS16_OFFS(SJ, 0), PF_LDS16_OFFS(SJ, SI), PF_LDS16_OFFS(SJ, 2 * (SI)),                 \
        PF_LDS16_OFFS(SJ, 3 * (SI))                                                                          \
      : "memory")

template <bool GATEUP>
__global__ __launch_bounds__(256, 1) void grouped_gemm_bf16_kernel(GemmArgs a) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;

  // ---- tile lookup.  Order: group by group; inside a group, blocks of up to
  // PF_GM m-tiles (PF_GM_SH for the shared group), and inside a block the
  // m-tiles fastest, so the tiles that share a weight panel (all m-tiles of an
  // expert, its ragged tail included) run at the same time and share it in
  // L2, while neighbouring column tiles share the token rows.  Each XCD walks
  // a contiguous range of this order.
  // All tile indices are below 2^24 (the host bounds the grid), so the
  // decoding below runs in 32-bit arithmetic.
  const uint32_t tiles_r = (uint32_t)a.tile_off[a.E] * (uint32_t)a.nt_r;
  const uint32_t total = tiles_r + (uint32_t)a.mt_s * (uint32_t)a.nt_s;
  constexpr uint32_t CH = GATEUP ? PF_CHUNK_GU : PF_CHUNK_DN;
  const uint32_t slot = blockIdx.x >> 3;
  const uint32_t tile = ((slot / CH) * 8 + (blockIdx.x & 7)) * CH + slot % CH;
  if (tile >= total) return;

  bool shared;
  int g, nt, K, N, valid;
  int64_t rb;  // first row of this tile in the group's row space
  int mt, mt_g, gm, rows, row0;
  uint32_t q, ntiles;  // q: index of the tile inside its group
  if (tile < tiles_r) {
    shared = false;
    const int key = (int)(tile / (uint32_t)a.nt_r);  // expert g owns keys tile_off[g] .. tile_off[g+1]-1
    int lo = 0, hi = a.E - 1;                       // largest g with tile_off[g] <= key
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.tile_off[mid] <= key) lo = mid; else hi = mid - 1;
    }
    g = lo;
    const int k0 = a.tile_off[g];
    q = tile - (uint32_t)a.nt_r * (uint32_t)k0;
    mt_g = a.tile_off[g + 1] - k0;
    ntiles = a.nt_r;
    gm = PF_GM;
    K = a.K;
    N = a.N;
    row0 = a.offsets[g];
    rows = a.offsets[g + 1] - row0;
  } else {
    shared = true;
    g = a.E;
    q = tile - tiles_r;
    mt_g = a.mt_s;
    ntiles = a.nt_s;
    gm = PF_GM_SH;
    K = a.K_sh;
    N = a.N_sh;
    row0 = 0;
    rows = (int)a.T;
  }
  {
    const uint32_t per = (uint32_t)gm * ntiles;       // tiles in a full block of gm m-tiles
    const uint32_t blk = q / per;
    const uint32_t in_blk = q - blk * per;
    const uint32_t bsize = (uint32_t)min(gm, mt_g - (int)blk * gm);  // m-tiles in this block
    const uint32_t n = in_blk / bsize;
    nt = (int)n;
    mt = (int)(blk * gm + (in_blk - n * bsize));
  }
  // the group's rows are cut into its mt_g tiles as evenly as possible (all
  // of them at most 256 rows; the first rows % mt_g tiles take one row more),
  // so a group slightly over a multiple of 256 rows gets tiles of nearly
  // equal size rather than a nearly empty last tile
  {
    const int base = rows / mt_g, rem = rows - base * mt_g;
    valid = base + (mt < rem ? 1 : 0);
    rb = (int64_t)row0 + (int64_t)mt * base + min(mt, rem);
  }
  const int wm = wv >> 1, wn = wv & 1;  // 2 x 2 wave layout
  // the tile's 32-row sub-tiles, split as evenly as possible between the two
  // wave rows (the first takes the odd one): mw of them from row a0 on
  const int ns = (valid + 31) >> 5;
  const int mw0 = (ns + 1) >> 1;
  const int mw = wm == 0 ? mw0 : ns - mw0;
  const int a0 = wm == 0 ? 0 : 32 * mw0;

  // ---- DMA sources: lane l of wave w fetches, for q < 8, row 64w + 8q + l/8,
  // chunk (l%8) ^ swz(row) = (l%8) ^ ((l/8) ^ q) of each operand.  Byte
  // offsets fit in 32 bits (the host checks the operand sizes).
  const int wvu = __builtin_amdgcn_readfirstlane(wv);
  const int lrow = 64 * wv + (lane >> 3);
  Operand A, B;
  A.rsrc = shared ? make_rsrc(a.A_sh, (uint64_t)a.rows_a_sh * K * 2) : make_rsrc(a.A, (uint64_t)a.rows_a * K * 2);
  {
    const uint64_t wbytes = (uint64_t)N * K * 2;  // one expert's matrix
    const uint16_t *bw;
    if (GATEUP) {
      // waves 0, 1 fetch gate rows (W1), waves 2, 3 the same rows of up (W3)
      const bool up = wvu >= 2;
      bw = shared ? (up ? a.B3s : a.B1s) : ((up ? a.B3 : a.B1) + (int64_t)g * N * K);
    } else {
      bw = shared ? a.B1s : (a.B1 + (int64_t)g * N * K);
    }
    B.rsrc = make_rsrc(bw, wbytes);
  }
#pragma unroll
  for (int q = 0; q < PF_LOADS; ++q) {
    const int row = lrow + 8 * q;
    const int lchunk = (lane & 7) ^ swz(row);
    const int r = min(row, valid - 1);  // clamped: rows past the group are never stored
    const int64_t arow = (GATEUP && !shared) ? (int64_t)a.row_token[rb + r] : rb + r;
    // offsets are stored less the immediate offset issue_op adds (see there)
    A.off[q] = (uint32_t)(arow * K * 2 + lchunk * 16 - (q & 3) * 1024);
    const int n = GATEUP ? nt * (PF_BN / 2) + (row & (PF_BN / 2 - 1)) : nt * PF_BN + row;
    B.off[q] = (uint32_t)((int64_t)min(n, N - 1) * K * 2 + lchunk * 16 - (q & 3) * 1024);  // clamped: columns >= N are never stored
  }

  // LDS rows of the wave's A sub-tiles and B column tiles (gate/up: tiles 0, 1
  // are gate columns, 2, 3 the same columns of up)
  WaveRows w;
  w.a0 = a0;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    w.b[j] = GATEUP ? (j >> 1) * (PF_BN / 2) + wn * 64 + (j & 1) * 32 : wn * 128 + j * 32;

  f32x16_t acc[PF_WM][4];
#pragma unroll
  for (int i = 0; i < PF_WM; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

  // a wave whose 64 token-tile rows all lie past the tile's valid sub-tiles
  // skips their DMA: nobody reads those LDS rows
  const bool adma = 64 * wvu < 32 * ns;
  // branch-free main loop per count of valid sub-tiles of this wave
  // an expert with a single m-tile reads each of its weight lines once: those
  // stream non-temporally (gate/up only; see launch_ffn_prefill_bf16)
  if (a.bnt && !shared && mt_g == 1) {
    if (mw == 4) k_loop<4, PF_NT>(A, B, w, K, acc, adma);
    else if (mw == 3) k_loop<3, PF_NT>(A, B, w, K, acc, adma);
    else if (mw == 2) k_loop<2, PF_NT>(A, B, w, K, acc, adma);
    else if (mw == 1) k_loop<1, PF_NT>(A, B, w, K, acc, adma);
    else k_loop<0, PF_NT>(A, B, w, K, acc, adma);
  } else {
    if (mw == 4) k_loop<4, 0>(A, B, w, K, acc, adma);
    else if (mw == 3) k_loop<3, 0>(A, B, w, K, acc, adma);
    else if (mw == 2) k_loop<2, 0>(A, B, w, K, acc, adma);
    else if (mw == 1) k_loop<1, 0>(A, B, w, K, acc, adma);
    else k_loop<0, 0>(A, B, w, K, acc, adma);
  }

  // ---- epilogue.  32x32 accumulator layout (transposed product): register
  // 4q + c of lane l holds token row l % 32 of the sub-tile and output column
  // 8q + 4 (l / 32) + c of the column tile.  The fp32 output of the down
  // projection goes through a private LDS slice of the wave, one 32-row
  // sub-tile at a time (rows padded by 16 bytes), and leaves as whole 512-byte
  // rows; the smaller bf16 output is stored directly.  First every wave's DMA
  // has landed and every fragment read is done, so all stages are free.
  publish<0>();  // every wave's DMA has landed and every fragment read is done: all stages are free
  char *stg = (char *)(wv == 0 ? g_As0 : wv == 1 ? g_Bs0 : wv == 2 ? g_Bs1 : g_Bs2);
  const int mrow = lane & 31;
  const int cgrp = 4 * (lane >> 5);
  if (GATEUP) {
    // H: the wave's 64 bf16 columns (j = 0, 1) of each 32-row sub-tile, one
    // 128-byte line per row, turned around in the wave's stage and stored 8
    // rows per instruction
    constexpr int RS = 144;
    uint16_t *C = (uint16_t *)(shared ? a.C_sh : a.C);
    const int nb = nt * (PF_BN / 2) + wn * 64;
    if (nb < N) {  // N is a multiple of 64: the wave's 64 columns are all in or all out
#pragma unroll
      for (int i = 0; i < PF_WM; ++i) {
        if (i >= mw) continue;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float h[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) h[c] = silu_fast(acc[i][j][4 * q + c]) * acc[i][j + 2][4 * q + c];
            *(uint2 *)(stg + (i * 32 + mrow) * RS + (32 * j + 8 * q + cgrp) * 2) =
                make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
          }
      }
      __builtin_amdgcn_wave_barrier();
      // read-back k = 4 i + sg: rows 8 sg + lane / 8 of sub-tile i (past the
      // valid sub-tiles it reads unused rows of the stage, never stored)
      uint4 v[16];
      PF_LDS_READ16(v, (uint32_t)(uintptr_t)(stg + (lane >> 3) * RS + (lane & 7) * 16), 32 * RS, 8 * RS);
#pragma unroll
      for (int i = 0; i < PF_WM; ++i)
#pragma unroll
        for (int sg = 0; sg < 4; ++sg) {
          const int row = w.a0 + i * 32 + 8 * sg + (lane >> 3);
          if (i < mw && row < valid) *(uint4 *)(C + (rb + row) * (int64_t)N + nb + (lane & 7) * 8) = v[4 * i + sg];
        }
    }
  } else {
    // Y: 128 fp32 columns (512 bytes) per row of the wave; all 16 read-backs
    // of a sub-tile are issued before its stores
    constexpr int RS = 528;
    float *C = (float *)(shared ? a.C_sh : a.C);
    const int nb = nt * PF_BN + wn * 128;
#pragma unroll
    for (int i = 0; i < PF_WM; ++i) {
      if (i >= mw) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *(float4 *)(stg + mrow * RS + (32 * j + 8 * q + cgrp) * 4) =
              make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      __builtin_amdgcn_wave_barrier();
      const int col = nb + (lane & 31) * 4;  // 32 lanes per 512-byte row
      // read-back t: rows 2 t + lane / 32
      uint4 v[16];
      PF_LDS_READ16(v, (uint32_t)(uintptr_t)(stg + (lane >> 5) * RS + (lane & 31) * 16), 8 * RS, 2 * RS);
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int row = w.a0 + i * 32 + (lane >> 5) + 2 * t;
        if (col < N && row < valid) *(uint4 *)(C + (rb + row) * (int64_t)N + col) = v[t];
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// Upper bound of the number of 256-row m-tiles over the routed groups.
static int64_t mtile_bound(int64_t R, int E) { return (R + PF_BM - 1) / PF_BM + std::min<int64_t>(E, R); }

// Work-groups covering `tiles` under the chunked XCD deal: whole rounds of 8
// chunks, so that every tile index below `tiles` has a work-group.
static int64_t pf_grid(int64_t tiles, int chunk) {
  const int64_t round = 8 * (int64_t)chunk;
  return (tiles + round - 1) / round * round;
}

// Work-groups of the two launches below (the larger is checked on the host).
static void pf_grids(const moe_dims &dm, int64_t T, int64_t *grid1, int64_t *grid2) {
  const int E = dm.n_routed, d = dm.d_model, f = dm.d_ff, fs = dm.d_ff_shared;
  const int64_t R = T * dm.top_k;
  const int64_t mt_sh = fs > 0 ? (T + PF_BM - 1) / PF_BM : 0;
  const int64_t nt1_r = (f + PF_BN / 2 - 1) / (PF_BN / 2), nt1_s = fs > 0 ? (fs + PF_BN / 2 - 1) / (PF_BN / 2) : 1;
  const int64_t nt2 = (d + PF_BN - 1) / PF_BN;
  *grid1 = pf_grid(mtile_bound(R, E) * nt1_r + mt_sh * nt1_s, PF_CHUNK_GU);
  *grid2 = pf_grid(mtile_bound(R, E) * nt2 + mt_sh * nt2, PF_CHUNK_DN);
}

int64_t ffn_prefill_max_workgroups(const moe_dims &dm, int64_t T) {
  int64_t g1, g2;
  pf_grids(dm, T, &g1, &g2);
  return std::max(g1, g2);
}

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
  g1.rows_a = T;
  g1.rows_a_sh = T;
  g1.E = E;
  g1.K = d;
  g1.K_sh = d;
  g1.N = f;
  g1.N_sh = fs;
  g1.has_shared = hs;
  g1.nt_r = (f + PF_BN / 2 - 1) / (PF_BN / 2);
  g1.nt_s = hs ? (fs + PF_BN / 2 - 1) / (PF_BN / 2) : 1;
  g1.mt_s = (int)mt_sh;
  // routed experts with a single m-tile read each gate/up weight line once, so
  // their tiles stream the weights non-temporally (DeepSeek-V3 gate/up 8%
  // faster at T = 512-1024, 5.5% at 2048, 1.7% at 4096); the down projection
  // measured 4-6% slower this way from T = 1024 up and stays cached
  g1.bnt = E > 0 ? 1 : 0;
  int64_t grid1, grid2;
  pf_grids(dm, T, &grid1, &grid2);
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
  g2.rows_a = R;
  g2.rows_a_sh = T;
  g2.E = E;
  g2.K = f;
  g2.K_sh = fs;
  g2.N = d;
  g2.N_sh = d;
  g2.has_shared = hs;
  g2.nt_r = (d + PF_BN - 1) / PF_BN;
  g2.nt_s = g2.nt_r;
  g2.mt_s = (int)mt_sh;
  g2.bnt = 0;
  grouped_gemm_bf16_kernel<false><<<dim3((unsigned)grid2), 256, 0, st>>>(g2);
  return hipGetLastError();
}
