// Softmax over all routed experts + per-token top-k with exact ranking.
//
// Source: "What is an 'expert', really?" (glossary: the router keeps the top-k;
// softmax turns raw scores into blend weights that add to 1).  The selection
// key is the exact real logit of the stored inputs; ties go to the lower
// expert index; slot j holds the (j+1)-th largest key.  The kept weights are
// the full-softmax probabilities (not renormalised over the k kept experts).
//
// One wavefront per token.  Each of the k rounds picks the largest remaining
// key.  With computed logits L_e and bounds B_e (router.hip), let m be the
// largest lower bound L_e - B_e among the remaining experts; only experts with
// L_e + B_e >= m can hold the maximum.  When that set has one member it is the
// winner.  Otherwise its members' logits are recomputed in fp64 (exact
// products, fp64 sums; bound ~(d/64 + 8) 2^-52 ||u|| ||c||) and written back in
// place with their tighter bounds, and the round is re-decided.  Members are
// visited lowest index first by a wave-wide minimum.  Members whose
// fp64 intervals still overlap are compared exactly: each key becomes a 256-bit
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
#include "common.h"

double router_bound_coeff(const moe_dims &dm);

#define TOPK_TOKENS_PER_WG 4
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

// Wave-cooperative fp64 logit of expert e (uniform result): exact products,
// fp64 sums.  16-byte loads: lane l takes the 8 (bf16) or 4 (fp32) elements
// of chunk l, l + 64, ... (d is a multiple of 64), DOT_BATCH chunks of each
// row in flight at once, into two accumulators (each lane's chain of
// additions only gets shorter than the d / 64 the fp64 bound allows for).
#define DOT_BATCH 4
template <bool BF16>
__device__ double dot_f64(const void *urow, const void *w, const float *bias, int e, int d) {
  const int lane = threadIdx.x & 63;
  double acc[2] = {0.0, 0.0};
  const int nc = BF16 ? d / 8 : d / 4;  // 16-byte chunks per row
  const uint4 *up = (const uint4 *)urow;
  const uint4 *wp = BF16 ? (const uint4 *)((const uint16_t *)w + (int64_t)e * d)
                         : (const uint4 *)((const float *)w + (int64_t)e * d);
  for (int c0 = lane; c0 < nc; c0 += 64 * DOT_BATCH) {
    uint4 a[DOT_BATCH], b[DOT_BATCH];
#pragma unroll
    for (int q = 0; q < DOT_BATCH; ++q) {
      const int c = c0 + 64 * q;
      a[q] = c < nc ? up[c] : make_uint4(0, 0, 0, 0);  // zero chunks add exact zeros
      b[q] = c < nc ? wp[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < DOT_BATCH; ++q) {
      const uint32_t av[4] = {a[q].x, a[q].y, a[q].z, a[q].w}, bv[4] = {b[q].x, b[q].y, b[q].z, b[q].w};
      double &r = acc[q & 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (BF16) {
          r = fma((double)__uint_as_float(av[i] << 16), (double)__uint_as_float(bv[i] << 16), r);
          r = fma((double)__uint_as_float(av[i] & 0xffff0000u), (double)__uint_as_float(bv[i] & 0xffff0000u), r);
        } else {
          r = fma((double)__uint_as_float(av[i]), (double)__uint_as_float(bv[i]), r);
        }
      }
    }
  }
  double v = wave_sum_f64(acc[0] + acc[1]);
  if (bias) v += (double)bias[e];
  return v;
}

// Lowest expert index among the set bits of `bits` (bit s of lane l = expert
// l + 64 s) over the wave, or a large value when no bit is set: one ballot
// per register slot.
template <int S>
__device__ __forceinline__ int lowest_expert(unsigned bits) {
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const unsigned long long b = __ballot((bits >> s) & 1u);
    if (b) return (__ffsll((long long)b) - 1) + 64 * s;
  }
  return 0x7fffffff;
}

// Wave-wide fp64 max and sum with the same value in every lane: four DPP
// steps (lane i meets lanes i ^ 1, i ^ 2, then its mirror in 8 and in 16)
// leave every row of 16 lanes holding its row's result, and the four rows
// are combined from lanes 0, 16, 32, 48.  Each step pairs a lane with a
// partner that holds the same partial set, so every lane's sums see the same
// operands (in swapped order) and agree bit for bit.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)b, CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane((int)b, l), hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (long long)(unsigned)lo);
}
__device__ __forceinline__ double row_max_f64(double v) {
  v = fmax(v, dpp_f64<0xB1>(v));   // quad_perm [1, 0, 3, 2]
  v = fmax(v, dpp_f64<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  v = fmax(v, dpp_f64<0x141>(v));  // row_half_mirror
  return fmax(v, dpp_f64<0x140>(v));  // row_mirror
}
__device__ __forceinline__ double dpp_wave_max_f64(double v) {
  v = row_max_f64(v);
  return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)), fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
}
__device__ __forceinline__ double dpp_wave_sum_f64(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  v += dpp_f64<0x141>(v);
  v += dpp_f64<0x140>(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

template <int S, bool BF16>
__global__ __launch_bounds__(256) void topk_kernel(const double *__restrict__ logits, const double *__restrict__ un2,
                                                   const double *__restrict__ wn, const float *__restrict__ bias,
                                                   const void *__restrict__ u, const void *__restrict__ w,
                                                   int64_t T, int E, int d, int k, double c1, int G,
                                                   int topk_group, int32_t *__restrict__ idx_out,
                                                   float *__restrict__ w_out, DiagWords *diag) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * TOPK_TOKENS_PER_WG + (threadIdx.x >> 6);
  if (t >= T) return;
  double L[S], B[S];
  unsigned avail = 0;
  const double unorm = un2[t];
  const double su = sqrt(unorm);  // ||u_t||; wn[e] = ||c_e|| (the (1 + 2^-30) factor covers their rounding)
  const double NEG = -__builtin_huge_val();
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const int e = lane + 64 * s;
    if (e < E) {
      L[s] = logits[t * E + e];
      B[s] = c1 * su * wn[e] * (1.0 + 0x1p-30) + 0x1p-50 * fabs(L[s]) + d * 0x1p-120;
      avail |= 1u << s;
    } else {
      L[s] = NEG;
      B[s] = 0.0;
    }
  }
  // softmax statistics over all experts (fp64)
  double mx = NEG;
#pragma unroll
  for (int s = 0; s < S; ++s) mx = fmax(mx, L[s]);
  mx = dpp_wave_max_f64(mx);
  double sum = 0.0;
#pragma unroll
  for (int s = 0; s < S; ++s)
    if (avail & (1u << s)) sum += (double)expf((float)(L[s] - mx));
  sum = dpp_wave_sum_f64(sum);

  const void *urow = BF16 ? (const void *)((const uint16_t *)u + t * d) : (const void *)((const float *)u + t * d);
  bool token_exact = false;
  unsigned bad = 0;
  int eu = -100000;  // max exponent of |u_t,i|, computed on first need
  const double c64 = (d / 64 + 8) * 0x1p-52;  // fp64 refinement bound coefficient
  unsigned refined = 0;                         // slots whose L/B hold fp64 values
  unsigned long long kept = 0;                  // groups met so far (G > 0)
  int nkept = 0;
  for (int j = 0; j < k; ++j) {
    int win = -1;
    for (;;) {
      double mlo = NEG;
#pragma unroll
      for (int s = 0; s < S; ++s)
        if (avail & (1u << s)) mlo = fmax(mlo, L[s] - B[s]);
      mlo = dpp_wave_max_f64(mlo);
      unsigned member = 0;
#pragma unroll
      for (int s = 0; s < S; ++s)
        if ((avail & (1u << s)) && L[s] + B[s] >= mlo) member |= 1u << s;
      const int mine = __popc(member);
      const unsigned long long holders = __ballot(mine > 0);
      if (__popcll(holders) == 1 && __ballot(mine > 1) == 0) {
        // a single member: the one lane holding one, in its lowest set slot
        const int my = member ? lane + 64 * (__ffs(member) - 1) : 0;
        win = __builtin_amdgcn_readlane(my, __ffsll((long long)holders) - 1);
        break;
      }
      token_exact = true;
      unsigned need = member & ~refined;
      if (__ballot(need != 0u)) {
        // level 2: fp64 logits of the unrefined members, written back in place
        // (expert e lives in lane e % 64, register slot e / 64)
        for (int e = lowest_expert<S>(need); e != 0x7fffffff; e = lowest_expert<S>(need)) {
          const double l64 = dot_f64<BF16>(urow, w, bias, e, d);
          const double b64 = c64 * su * wn[e] * (1.0 + 0x1p-30) + 0x1p-51 * fabs(l64) + d * 0x1p-120;
#pragma unroll
          for (int s = 0; s < S; ++s)
            if (lane + 64 * s == e) {
              L[s] = l64;
              B[s] = b64;
              refined |= 1u << s;
              need &= ~(1u << s);
            }
        }
        if (lane == 0) atomicAdd(&diag->refinements, 1u);
        continue;  // re-decide the round with the tighter intervals
      }
      // level 3: exact tournament over the (all refined) members, ascending index
      if (eu == -100000) {
        int m = -100000;
        for (int i = lane; i < d; i += 64) m = max(m, exponent_of(load_elem<BF16>(urow, i)));
        eu = wave_max_i32(m);
      }
      int ew = -100000, eb = -100000;
      for (unsigned rest = member; ; ) {
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
      for (unsigned rest = member; ; ) {  // ascending expert order
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
      win = __builtin_amdgcn_readfirstlane(exact_win);
      const int cnt = wave_sum_i32(mine);
      if (lane == 0) atomicAdd(&diag->exact_keys, (unsigned)cnt);
      break;
    }
    if (G > 0) {  // group-limited: the winner's group is kept (it is one of the first topk_group met)
      const int g = win / G;
      if (!((kept >> g) & 1ull)) {
        kept |= 1ull << g;
        if (++nkept == topk_group) {
#pragma unroll
          for (int s = 0; s < S; ++s) {
            const int e = lane + 64 * s;
            if (e < E && !((kept >> (e / G)) & 1ull)) avail &= ~(1u << s);
          }
        }
      }
    }
    // the winner's lane takes it out and emits its slot
#pragma unroll
    for (int s = 0; s < S; ++s)
      if (lane + 64 * s == win) {
        avail &= ~(1u << s);
        idx_out[t * k + j] = win;
        w_out[t * k + j] = (float)((double)expf((float)(L[s] - mx)) / sum);
      }
  }
  if (lane == 0) {
    if (token_exact) atomicAdd(&diag->tokens_exact, 1u);
  }
  if (__ballot(bad != 0u) && lane == 0) atomicOr(&diag->flags, MOE_DIAG_UNRESOLVED);
}

template <int S>
static void launch_topk_s(const moe_dims &dm, int64_t T, const void *u, const void *w, const float *bias,
                          int32_t *idx, float *wout, const WsLayout &L, char *ws, hipStream_t st) {
  const double c1 = router_bound_coeff(dm);
  dim3 grid((unsigned)((T + TOPK_TOKENS_PER_WG - 1) / TOPK_TOKENS_PER_WG));
  const double *lg = (const double *)(ws + L.logits);
  const double *un2 = (const double *)(ws + L.unorm2);
  const double *wn = (const double *)(ws + L.wnorm);
  DiagWords *diag = (DiagWords *)(ws + L.diag);
  // group size, or 0 when routing is not group-limited
  const bool grouped = dm.n_group > 1 && dm.topk_group < dm.n_group;
  const int G = grouped ? dm.n_routed / dm.n_group : 0;
  if (dm.dtype == MOE_BF16)
    topk_kernel<S, true><<<grid, 256, 0, st>>>(lg, un2, wn, bias, u, w, T, dm.n_routed, dm.d_model, dm.top_k, c1,
                                               G, dm.topk_group, idx, wout, diag);
  else
    topk_kernel<S, false><<<grid, 256, 0, st>>>(lg, un2, wn, bias, u, w, T, dm.n_routed, dm.d_model, dm.top_k, c1,
                                                G, dm.topk_group, idx, wout, diag);
}

hipError_t launch_topk(const moe_dims &dm, int64_t T, const void *u, const void *w_router, const float *bias,
                       int32_t *topk_idx, float *topk_w, const WsLayout &L, char *ws, hipStream_t st) {
  const int E = dm.n_routed;
  if (E <= 64) launch_topk_s<1>(dm, T, u, w_router, bias, topk_idx, topk_w, L, ws, st);
  else if (E <= 128) launch_topk_s<2>(dm, T, u, w_router, bias, topk_idx, topk_w, L, ws, st);
  else if (E <= 256) launch_topk_s<4>(dm, T, u, w_router, bias, topk_idx, topk_w, L, ws, st);
  else if (E <= 512) launch_topk_s<8>(dm, T, u, w_router, bias, topk_idx, topk_w, L, ws, st);
  else launch_topk_s<16>(dm, T, u, w_router, bias, topk_idx, topk_w, L, ws, st);
  return hipGetLastError();
}

// --------------------------------------------------------------- diagnostics
__global__ void diag_clear_kernel(DiagWords *d) {
  if (threadIdx.x == 0) {
    d->flags = 0;
    d->tokens_exact = 0;
    d->exact_keys = 0;
    d->refinements = 0;
  }
}

hipError_t launch_diag_clear(void *ws, hipStream_t st) {
  diag_clear_kernel<<<1, 64, 0, st>>>((DiagWords *)ws);
  return hipGetLastError();
}
