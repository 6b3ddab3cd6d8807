// Softmax over all routed experts + per-token top-k with exact ranking.
//
// Source: "What is an 'expert', really?" (glossary: the router keeps the top-k;
// softmax turns raw scores into blend weights that add to 1).  The selection
// key is the exact real logit of the stored inputs; ties go to the lower
// expert index; slot j holds the (j+1)-th largest key.  The kept weights are
// the full-softmax probabilities (not renormalised over the k kept experts).
//
// Each of the k rounds picks the largest remaining key.  With computed
// logits L_e and bounds B_e (router.hip), let m be the largest lower bound
// L_e - B_e among the remaining experts; only experts with L_e + B_e >= m can
// hold the maximum.  When that set has one member it is the winner.
// Otherwise its members' logits are recomputed in fp64 (exact products, fp64
// sums; bound ~(d/64 + 8) 2^-52 ||u|| ||c||) and written back in place with
// their tighter bounds, and the round is re-decided.  Members are visited
// lowest index first.  Members whose fp64 intervals still overlap are
// compared exactly: each key becomes a 256-bit
// fixed-point sum of its exact products (bf16 x bf16 and fp32 x fp32 products
// are exact in fp64) and the largest wins, ties to the lower index.  A product
// that falls below the fixed-point window (a dynamic range above ~2^200 inside
// one token) raises a diagnostics flag instead of being dropped silently.
//
// Group-limited routing ("Shared and fine-grained experts": node-limited
// routing caps the machines a token's experts live on, DeepSeek-V3's n_group 8
// and topk_group 4).  Read as: experts form contiguous groups of G, a group
// scores its best expert, the token keeps its topk_group best groups (ties to
// the lower group) and takes its top-k among their experts.  The rounds above
// walk the experts in exact descending key order, so the first topk_group
// groups that walk meets are exactly the kept groups: from the round that
// meets the last of them on, every other group's experts leave the candidate
// set, and every winner is a kept expert.
//
// Two kernels.  The first gives each token one wavefront and settles every
// token whose k rounds all have a single member; a token that needs more is
// appended to a list and left to the second, which runs the full procedure
// with one wavefront per listed token.  Batches of up to MOE_TOPK_COOP_ALL
// tokens skip the first kernel: the second then gives every token a
// work-group of four wavefronts that all hold the token's logits and take the
// same decisions, and a refinement splits every member's fp64 dot product
// over the four, which exchange partial sums through LDS, so that its latency
// is about a quarter of one wavefront's.  A refinement pass takes up to
// several members at once, so their loads are in flight together.
#include "common.h"

double router_bound_coeff(const moe_dims &dm);

#define TOPK_TOKENS_PER_WG 4   // first kernel: one wavefront per token
#define TOPK_MEMBERS_1 2       // members per refinement pass, one wavefront per token
#define TOPK_MEMBERS_4 4       // ... four wavefronts per token
#define TOPK_DOT_BATCH 4       // 16-byte chunks of a row in flight per lane (second kernel)
#define TOPK_FAST_BATCH 2      // ... in the first kernel, whose registers set its occupancy
#define TOPK_LIST_WGS 64       // work-groups of the second kernel over the (usually short) list
#define EXACT_LIMBS 8  // radix 2^32 digits held in int64 (carry headroom)

template <bool BF16>
__device__ __forceinline__ double load_elem(const void *p, int64_t i) {
  if (BF16) return (double)bf16_to_f32(((const uint16_t *)p)[i]);
  return (double)((const float *)p)[i];
}

// floor(log2|x|) of a finite non-zero double; a very small sentinel for zero
__device__ __forceinline__ int exponent_of(double x) {
  if (x == 0.0) return -100000;
  const unsigned long long b = (unsigned long long)__double_as_longlong(x);
  const int ex = (int)((b >> 52) & 0x7ff);
  if (ex == 0) return -1075;  // subnormal: below every value used here
  return ex - 1023;
}

// acc += p exactly as a multiple of 2^E0 (p = mant * 2^lsb).  Sets *bad when a
// non-zero bit of p falls below 2^E0 or above the window.
__device__ __forceinline__ void exact_add(long long (&acc)[EXACT_LIMBS], double p, int E0, unsigned &bad) {
  if (p == 0.0) return;
  const unsigned long long bits = (unsigned long long)__double_as_longlong(p);
  const bool neg = (bits >> 63) != 0;
  int ex = (int)((bits >> 52) & 0x7ff);
  unsigned long long mant = bits & 0xfffffffffffffull;
  if (ex == 0) ex = 1; else mant |= 1ull << 52;
  int sh = (ex - 1075) - E0;
  if (sh < 0) {
    if (sh <= -64) { bad = 1u; return; }
    if (mant & ((1ull << (-sh)) - 1ull)) bad = 1u;
    mant >>= -sh;
    sh = 0;
  }
  const int li = sh >> 5, off = sh & 31;
  if (li > EXACT_LIMBS - 3) { bad = 1u; return; }
  const long long d0 = (long long)((mant << off) & 0xffffffffull);
  const unsigned long long rem = off ? (mant >> (32 - off)) : (mant >> 32);
  const long long d1 = (long long)(rem & 0xffffffffull);
  const long long d2 = (long long)(rem >> 32);
#pragma unroll
  for (int q = 0; q < EXACT_LIMBS; ++q) {
    long long v = (q == li ? d0 : 0) + (q == li + 1 ? d1 : 0) + (q == li + 2 ? d2 : 0);
    acc[q] += neg ? -v : v;
  }
}

// sign of (a - b) for two fixed-point sums on the same window
__device__ __forceinline__ int exact_cmp(const long long (&a)[EXACT_LIMBS], const long long (&b)[EXACT_LIMBS]) {
  long long dlt[EXACT_LIMBS];
#pragma unroll
  for (int q = 0; q < EXACT_LIMBS; ++q) dlt[q] = a[q] - b[q];
#pragma unroll
  for (int q = 0; q < EXACT_LIMBS - 1; ++q) {
    const long long c = dlt[q] >> 32;  // floor division
    dlt[q] -= c * (1ll << 32);
    dlt[q + 1] += c;
  }
  if (dlt[EXACT_LIMBS - 1] != 0) return dlt[EXACT_LIMBS - 1] > 0 ? 1 : -1;
  long long any = 0;
#pragma unroll
  for (int q = 0; q < EXACT_LIMBS - 1; ++q) any |= dlt[q];
  return any != 0 ? 1 : 0;
}

// Wave-cooperative exact key of expert e for the token row urow (uniform result).
template <bool BF16>
__device__ void exact_key(const void *urow, const void *w, const float *bias, int e, int d, int E0,
                          long long (&key)[EXACT_LIMBS], unsigned &bad) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < EXACT_LIMBS; ++q) key[q] = 0;
  for (int i = lane; i < d; i += 64) {
    const double p = load_elem<BF16>(urow, i) * load_elem<BF16>(w, (int64_t)e * d + i);
    exact_add(key, p, E0, bad);
  }
  if (bias && lane == 0) exact_add(key, (double)bias[e], E0, bad);
#pragma unroll
  for (int q = 0; q < EXACT_LIMBS; ++q) key[q] = wave_sum_i64(key[q]);
}

// fp64 logits of up to M experts es[0..m) for the token row urow,
// by the NW wavefronts (1 or 4) that hold the token (uniform results in every
// lane of each): exact products, fp64 sums.  16-byte chunk c of a row (8 bf16
// or 4 fp32 elements) goes to lane c % 64 of wave (c / 64) % NW; a lane adds
// its chunks in order, the wave sums its lanes and, with four waves, the wave
// sums are added in wave order through LDS (part), then the bias.  A term
// passes through at most 8 ceil(d / (512 NW)) + 9 additions, inside the
// (d / 64 + 8) 2^-52 bound's allowance (which counts 2^-53 per addition
// twice over) for every d >= 64.
template <bool BF16, int NW, int M, int DOT_BATCH>
__device__ void coop_dots(const void *urow, const void *w, const float *bias, const int (&es)[M], int m, int d,
                          double (*part)[M], double (&out)[M]) {
  const int lane = threadIdx.x & 63, wv = NW == 1 ? 0 : threadIdx.x >> 6;
  const int nc = BF16 ? d / 8 : d / 4;  // 16-byte chunks per row
  const uint4 *up = (const uint4 *)urow;
  double acc[M];
#pragma unroll
  for (int q = 0; q < M; ++q) acc[q] = 0.0;
  for (int c0 = 64 * wv + lane; c0 < nc; c0 += 64 * NW * DOT_BATCH) {
    uint4 a[DOT_BATCH];
#pragma unroll
    for (int i = 0; i < DOT_BATCH; ++i) {
      const int c = c0 + 64 * NW * i;
      a[i] = c < nc ? up[c] : make_uint4(0, 0, 0, 0);  // zero chunks add exact zeros
    }
#pragma unroll
    for (int q = 0; q < M; ++q) {
      if (q >= m) continue;
      const uint4 *wp = BF16 ? (const uint4 *)((const uint16_t *)w + (int64_t)es[q] * d)
                             : (const uint4 *)((const float *)w + (int64_t)es[q] * d);
      uint4 b[DOT_BATCH];
#pragma unroll
      for (int i = 0; i < DOT_BATCH; ++i) {
        const int c = c0 + 64 * NW * i;
        b[i] = c < nc ? wp[c] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < DOT_BATCH; ++i) {
        const uint32_t av[4] = {a[i].x, a[i].y, a[i].z, a[i].w}, bv[4] = {b[i].x, b[i].y, b[i].z, b[i].w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          if (BF16) {
            acc[q] = fma((double)__uint_as_float(av[h] << 16), (double)__uint_as_float(bv[h] << 16), acc[q]);
            acc[q] = fma((double)__uint_as_float(av[h] & 0xffff0000u), (double)__uint_as_float(bv[h] & 0xffff0000u),
                         acc[q]);
          } else {
            acc[q] = fma((double)__uint_as_float(av[h]), (double)__uint_as_float(bv[h]), acc[q]);
          }
        }
      }
    }
  }
  if (NW == 1) {
#pragma unroll
    for (int q = 0; q < M; ++q) {
      out[q] = dpp_wave_sum_f64(acc[q]);
      if (q < m && bias) out[q] += (double)bias[es[q]];
    }
    return;
  }
#pragma unroll
  for (int q = 0; q < M; ++q) {
    const double v = dpp_wave_sum_f64(acc[q]);
    if (q < m && lane == 0) part[wv][q] = v;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < M; ++q) {
    out[q] = (part[0][q] + part[1][q]) + (part[2][q] + part[3][q]);
    if (q < m && bias) out[q] += (double)bias[es[q]];
  }
  __syncthreads();  // part is free again
}

// Lowest expert index among the set bits of `bits` (bit s of lane l = expert
// l + 64 s) over the wave, or a large value when no bit is set: one ballot
// per register slot.
template <int S>
__device__ __forceinline__ int lowest_expert(unsigned bits) {
  int r = 0x7fffffff;
#pragma unroll
  for (int s = S - 1; s >= 0; --s) {
    const unsigned long long b = __ballot((bits >> s) & 1u);
    if (b) r = (__ffsll((long long)b) - 1) + 64 * s;
  }
  return r;
}

struct TopkArgs {
  const double *logits, *un2, *wn;
  const float *bias;
  const void *u, *w;
  int64_t T;
  int E, d, k;
  double c1;           // first-level bound coefficient (router.hip)
  int G, topk_group;   // group size (0: not group-limited) and groups kept
  int32_t *idx_out;
  float *w_out;
  DiagWords *diag;
  int32_t *list;       // tokens left to the cooperative kernel
};

// A token's state (expert e lives in lane e % 64, register slot e / 64): its
// logit L, the interval [lo, hi] = [L - B, L + B] around it (both -inf once
// the expert has left the candidates, and for slots past N_r), the round
// that took it (rank, -1 if none), the softmax statistics and the groups
// met so far.
template <int S>
struct TokenState {
  double L[S], lo[S], hi[S];
  int rank[S];
  double mx, sum, su;
  unsigned long long kept;
  int nkept;
};

template <int S>
__device__ __forceinline__ void token_setup(const TopkArgs &a, int64_t t, TokenState<S> &z) {
  const int lane = threadIdx.x & 63;
  const double NEG = -__builtin_huge_val();
  z.kept = 0;
  z.nkept = 0;
  // every load issued before any is used (indices clamped into the rows)
  double lg[S], cn[S];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e = min(lane + 64 * s, a.E - 1);
    lg[s] = a.logits[t * a.E + e];
    cn[s] = a.wn[e];
  }
  z.su = sqrt(a.un2[t]);  // ||u_t||; wn[e] = ||c_e|| (the (1 + 2^-30) factor covers their rounding)
  double mx = NEG;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    z.rank[s] = -1;
    if (lane + 64 * s < a.E) {
      const double B = a.c1 * z.su * cn[s] * (1.0 + 0x1p-30) + 0x1p-50 * fabs(lg[s]) + a.d * 0x1p-120;
      z.L[s] = lg[s];
      z.lo[s] = lg[s] - B;
      z.hi[s] = lg[s] + B;
      mx = fmax(mx, lg[s]);
    } else {
      z.L[s] = z.lo[s] = z.hi[s] = NEG;
    }
  }
  // softmax statistics over all experts (fp64)
  z.mx = dpp_wave_max_f64(mx);
  double sum = 0.0;
#pragma unroll
  for (int s = 0; s < S; ++s)
    if (lane + 64 * s < a.E) sum += (double)expf((float)(z.L[s] - z.mx));
  z.sum = dpp_wave_sum_f64(sum);
}

// The round's members, the candidates whose interval reaches the largest
// lower bound, as this lane's slot bits; the winner (uniform) when there is
// a single member, else -1.  One ballot per slot: the count and the winner
// come out of the scalar unit.
template <int S>
__device__ __forceinline__ int round_members(const TokenState<S> &z, unsigned &member) {
  double m = z.lo[0];
#pragma unroll
  for (int s = 1; s < S; ++s) m = fmax(m, z.lo[s]);
  m = dpp_wave_max_f64(m);
  unsigned long long bal[S];
  int cnt = 0;
  member = 0;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const bool in = z.hi[s] >= m;
    bal[s] = __ballot(in);
    member |= in ? 1u << s : 0u;
    cnt += __popcll(bal[s]);
  }
  if (cnt != 1) return -1;
  int win = -1;
#pragma unroll
  for (int s = S - 1; s >= 0; --s)
    if (bal[s]) win = (__ffsll((long long)bal[s]) - 1) + 64 * s;
  return win;
}

// Round j's winner leaves the candidates; with group limits, its group is
// kept (it is one of the first topk_group met) and once topk_group groups are
// met every other group's experts leave too.
template <int S>
__device__ __forceinline__ void take_winner(const TopkArgs &a, TokenState<S> &z, int j, int win) {
  const int lane = threadIdx.x & 63;
  const double NEG = -__builtin_huge_val();
  if (a.G > 0) {
    const int g = win / a.G;
    if (!((z.kept >> g) & 1ull)) {
      z.kept |= 1ull << g;
      if (++z.nkept == a.topk_group) {
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const int e = lane + 64 * s;
          if (e < a.E && !((z.kept >> (e / a.G)) & 1ull)) z.lo[s] = z.hi[s] = NEG;
        }
      }
    }
  }
#pragma unroll
  for (int s = 0; s < S; ++s)
    if (s == (win >> 6) && lane == (win & 63)) {
      z.lo[s] = z.hi[s] = NEG;
      z.rank[s] = j;
    }
}

// Every taken expert's lane writes its slot: the index and the full-softmax
// probability (of its logit as it stands, fp64 where refined).
template <int S>
__device__ __forceinline__ void emit_slots(const TopkArgs &a, const TokenState<S> &z, int64_t t) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int s = 0; s < S; ++s)
    if (z.rank[s] >= 0) {
      a.idx_out[t * a.k + z.rank[s]] = lane + 64 * s;
      a.w_out[t * a.k + z.rank[s]] = (float)((double)expf((float)(z.L[s] - z.mx)) / z.sum);
    }
}

// Level 2 for the members in need (this lane's slot bits): their fp64 logits,
// lowest index first, M per pass, written back in place with the tighter
// fp64 bound.  Marks them in refined.
template <int S, bool BF16, int NW, int M, int DB>
__device__ __forceinline__ void refine_members(const TopkArgs &a, TokenState<S> &z, const void *urow, unsigned need,
                                               unsigned &refined, double (*part)[M]) {
  const int lane = threadIdx.x & 63;
  const int d = a.d;
  const double c64 = (d / 64 + 8) * 0x1p-52;  // fp64 refinement bound coefficient
  for (;;) {
    int es[M];
    int m = 0;
#pragma unroll
    for (int q = 0; q < M; ++q) {
      es[q] = lowest_expert<S>(need);
      if (es[q] != 0x7fffffff) {
        if ((es[q] & 63) == lane) need &= ~(1u << (es[q] >> 6));
        ++m;
      }
    }
    if (m == 0) break;
    double l64[M];
    coop_dots<BF16, NW, M, DB>(urow, a.w, a.bias, es, m, d, part, l64);
    for (int q = 0; q < M; ++q) {
      const int e = es[q];
#pragma unroll
      for (int s = 0; s < S; ++s)
        if (q < m && e == lane + 64 * s) {
          const double b64 = c64 * z.su * a.wn[e] * (1.0 + 0x1p-30) + 0x1p-51 * fabs(l64[q]) + d * 0x1p-120;
          z.L[s] = l64[q];
          z.lo[s] = l64[q] - b64;
          z.hi[s] = l64[q] + b64;
          refined |= 1u << s;
        }
    }
  }
}

// Level 3: the exact tournament over the members (this lane's slot bits), in
// ascending expert order, ties to the lower index; returns the winner
// (uniform).  eu caches the largest exponent of the token's elements.  Kept
// out of line: it is rare, and its fixed-point registers would otherwise
// count against the occupancy of the common path.
template <int S, bool BF16>
__device__ __attribute__((noinline)) int exact_tournament(const void *urow, const void *w, const float *bias,
                                                          unsigned member, int d, int &eu, unsigned &bad) {
  const int lane = threadIdx.x & 63;
  if (eu == -100000) {
    int mm = -100000;
    for (int i = lane; i < d; i += 64) mm = max(mm, exponent_of(load_elem<BF16>(urow, i)));
    eu = wave_max_i32(mm);
  }
  int ew = -100000, eb = -100000;
  for (unsigned rest = member;;) {
    const int e = lowest_expert<S>(rest);
    if (e == 0x7fffffff) break;
    for (int i = lane; i < d; i += 64) ew = max(ew, exponent_of(load_elem<BF16>(w, (int64_t)e * d + i)));
    if (bias) eb = max(eb, exponent_of((double)bias[e]));
    if ((e & 63) == lane) rest &= ~(1u << (e >> 6));
  }
  ew = wave_max_i32(ew);
  eb = __builtin_amdgcn_readfirstlane(eb);
  int lg = 1;
  while ((1 << lg) < d + 2) ++lg;
  const int top = max(eu + ew + 2, eb + 1) + lg + 1;
  const int E0 = __builtin_amdgcn_readfirstlane(top - 240);
  long long best[EXACT_LIMBS];
  long long cur[EXACT_LIMBS];
  int exact_win = -1;
#pragma unroll
  for (int q = 0; q < EXACT_LIMBS; ++q) best[q] = 0;
  for (unsigned rest = member;;) {  // ascending expert order
    const int e = lowest_expert<S>(rest);
    if (e == 0x7fffffff) break;
    if ((e & 63) == lane) rest &= ~(1u << (e >> 6));
    exact_key<BF16>(urow, w, bias, e, d, E0, cur, bad);
    // keys are wave sums: make their uniformity explicit before comparing
    int better = 0;
    if (exact_win >= 0) better = exact_cmp(cur, best) > 0 ? 1 : 0;
    better = __builtin_amdgcn_readfirstlane(better);
    if (exact_win < 0 || better) {
      exact_win = e;
#pragma unroll
      for (int q = 0; q < EXACT_LIMBS; ++q) best[q] = cur[q];
    }
  }
  return __builtin_amdgcn_readfirstlane(exact_win);
}

// First kernel: one wavefront per token, levels 1 and 2.  A token whose
// rounds all settle with fp64 refinement at most is finished here (its
// diagnostics counted here); a round that needs the exact level sends the
// token to the list, and the second kernel takes it from the start.
template <int S, bool BF16>
__global__ __launch_bounds__(256) void topk_fast_kernel(TopkArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * TOPK_TOKENS_PER_WG + (threadIdx.x >> 6);
  if (t >= a.T) return;
  TokenState<S> z;
  token_setup<S>(a, t, z);
  const void *urow = BF16 ? (const void *)((const uint16_t *)a.u + t * a.d) : (const void *)((const float *)a.u + t * a.d);
  unsigned refined = 0, passes = 0;
  for (int j = 0; j < a.k; ++j) {
    int win;
    for (;;) {
      unsigned member;
      win = round_members<S>(z, member);
      if (win >= 0) break;
      const unsigned need = member & ~refined;
      if (!__ballot(need != 0u)) {  // the exact level: left to the second kernel
        if (lane == 0) a.list[atomicAdd(&a.diag->deferred, 1u)] = (int32_t)t;
        return;
      }
      refine_members<S, BF16, 1, TOPK_MEMBERS_1, TOPK_FAST_BATCH>(a, z, urow, need, refined, nullptr);
      ++passes;
    }
    take_winner<S>(a, z, j, win);
  }
  emit_slots<S>(a, z, t);
  if (lane == 0 && passes) {
    atomicAdd(&a.diag->tokens_exact, 1u);
    atomicAdd(&a.diag->refinements, passes);
  }
}

// Second kernel: the full procedure for the listed tokens (LIST) or for
// tokens 0 .. T - 1, with NW wavefronts per token: one (four tokens per
// work-group, each wave on its own) or four.  Four waves load the same
// logits and take the same decisions, so their control flow agrees and they
// meet at every barrier; fp64 refinements split the work over the four
// (coop_dots), the exact level runs in each wave, and wave 0 writes the slots
// and diagnostics.
template <int S, bool BF16, bool LIST, int NW>
__global__ __launch_bounds__(256) void topk_coop_kernel(TopkArgs a) {
  constexpr int M = NW == 1 ? TOPK_MEMBERS_1 : TOPK_MEMBERS_4;  // members per refinement pass
  __shared__ double part[4][M];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const bool lead = NW == 1 || wv == 0;  // writes the slots and diagnostics
  const int64_t n = LIST ? (int64_t)(*(volatile const uint32_t *)&a.diag->deferred) : a.T;
  const int d = a.d;
  const int per = 4 / NW;                     // tokens per work-group
  for (int64_t i = (int64_t)blockIdx.x * per + (NW == 1 ? wv : 0); i < n; i += (int64_t)gridDim.x * per) {
    const int64_t t = LIST ? (int64_t)a.list[i] : i;
    TokenState<S> z;
    token_setup<S>(a, t, z);
    const void *urow = BF16 ? (const void *)((const uint16_t *)a.u + t * d) : (const void *)((const float *)a.u + t * d);
    bool token_exact = false;
    unsigned bad = 0;
    int eu = -100000;     // max exponent of |u_t,i|, computed on first need
    unsigned refined = 0;  // slots whose L/B hold fp64 values
    for (int j = 0; j < a.k; ++j) {
      int win = -1;
      for (;;) {
        unsigned member;
        win = round_members<S>(z, member);
        if (win >= 0) break;
        token_exact = true;
        unsigned need = member & ~refined;
        if (__ballot(need != 0u)) {
          // level 2
          refine_members<S, BF16, NW, M, TOPK_DOT_BATCH>(a, z, urow, need, refined, part);
          if (lead && lane == 0) atomicAdd(&a.diag->refinements, 1u);
          continue;  // re-decide the round with the tighter intervals
        }
        // level 3: exact tournament over the (all refined) members
        win = exact_tournament<S, BF16>(urow, a.w, a.bias, member, d, eu, bad);
        const int cnt = wave_sum_i32(__popc(member));
        if (lead && lane == 0) atomicAdd(&a.diag->exact_keys, (unsigned)cnt);
        break;
      }
      take_winner<S>(a, z, j, win);
    }
    if (lead) emit_slots<S>(a, z, t);
    if (lead && lane == 0 && token_exact) atomicAdd(&a.diag->tokens_exact, 1u);
    if (__ballot(bad != 0u) && lead && lane == 0) atomicOr(&a.diag->flags, MOE_DIAG_UNRESOLVED);
  }
}

template <int S, bool BF16>
static void launch_topk_s(const moe_dims &dm, int64_t T, const void *u, const void *w, const float *bias,
                          int32_t *idx, float *wout, const WsLayout &L, char *ws, hipStream_t st) {
  // group size, or 0 when routing is not group-limited
  const bool grouped = dm.n_group > 1 && dm.topk_group < dm.n_group;
  TopkArgs a{(const double *)(ws + L.logits), (const double *)(ws + L.unorm2), (const double *)(ws + L.wnorm),
             bias, u, w, T, dm.n_routed, dm.d_model, dm.top_k, router_bound_coeff(dm),
             grouped ? dm.n_routed / dm.n_group : 0, dm.topk_group, idx, wout, (DiagWords *)(ws + L.diag),
             (int32_t *)(ws + L.topk_list)};
  if (T <= MOE_TOPK_COOP_ALL) {
    topk_coop_kernel<S, BF16, false, 4><<<dim3((unsigned)T), 256, 0, st>>>(a);
    return;
  }
  const int64_t wgs = (T + TOPK_TOKENS_PER_WG - 1) / TOPK_TOKENS_PER_WG;
  topk_fast_kernel<S, BF16><<<dim3((unsigned)wgs), 256, 0, st>>>(a);
  topk_coop_kernel<S, BF16, true, 4><<<dim3((unsigned)TOPK_LIST_WGS), 256, 0, st>>>(a);
}

template <int S>
static void launch_topk_dt(const moe_dims &dm, int64_t T, const void *u, const void *w, const float *bias,
                           int32_t *idx, float *wout, const WsLayout &L, char *ws, hipStream_t st) {
  if (dm.dtype == MOE_BF16) launch_topk_s<S, true>(dm, T, u, w, bias, idx, wout, L, ws, st);
  else launch_topk_s<S, false>(dm, T, u, w, bias, idx, wout, L, ws, st);
}

hipError_t launch_topk(const moe_dims &dm, int64_t T, const void *u, const void *w_router, const float *bias,
                       int32_t *topk_idx, float *topk_w, const WsLayout &L, char *ws, hipStream_t st) {
  const int E = dm.n_routed;
  if (E <= 64) launch_topk_dt<1>(dm, T, u, w_router, bias, topk_idx, topk_w, L, ws, st);
  else if (E <= 128) launch_topk_dt<2>(dm, T, u, w_router, bias, topk_idx, topk_w, L, ws, st);
  else if (E <= 256) launch_topk_dt<4>(dm, T, u, w_router, bias, topk_idx, topk_w, L, ws, st);
  else if (E <= 512) launch_topk_dt<8>(dm, T, u, w_router, bias, topk_idx, topk_w, L, ws, st);
  else launch_topk_dt<16>(dm, T, u, w_router, bias, topk_idx, topk_w, L, ws, st);
  return hipGetLastError();
}

// --------------------------------------------------------------- diagnostics
__global__ void diag_clear_kernel(DiagWords *d) {
  if (threadIdx.x == 0) {
    d->flags = 0;
    d->tokens_exact = 0;
    d->exact_keys = 0;
    d->refinements = 0;
    d->deferred = 0;
  }
}

hipError_t launch_diag_clear(void *ws, hipStream_t st) {
  diag_clear_kernel<<<1, 64, 0, st>>>((DiagWords *)ws);
  return hipGetLastError();
}
