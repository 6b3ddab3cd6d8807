// C-ABI entry points: host-side validation, workspace carve-up, stage launches.
//
// Every argument is validated on the host before the first HIP call, so a
// failing call enqueues nothing.  Nothing here copies device data to the host
// (except moe_read_diagnostics, which exists for tests).
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "common.h"

static thread_local char g_err[512] = "";

static moe_status fail(moe_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

static moe_status hip_fail(hipError_t e, const char *where) {
  return fail(MOE_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

#define MOE_TRY_HIP(expr, where)            \
  do {                                      \
    hipError_t e_ = (expr);                 \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

static bool al16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

static moe_status check_dims(const moe_dims *dm, int64_t T) {
  if (!dm) return fail(MOE_ERR_INVALID_VALUE, "dims is NULL");
  if (T < 0) return fail(MOE_ERR_INVALID_VALUE, "T < 0");
  const bool dense = dm->n_routed == 0;
  if (dense) {
    if (dm->top_k != 0) return fail(MOE_ERR_INVALID_VALUE, "a dense layer (n_routed == 0) needs top_k == 0");
    if (dm->d_ff_shared < 1) return fail(MOE_ERR_INVALID_VALUE, "a dense layer (n_routed == 0) needs d_ff_shared > 0");
  } else {
    if (dm->top_k < 1) return fail(MOE_ERR_INVALID_VALUE, "top_k < 1");
    if (dm->n_routed < 1) return fail(MOE_ERR_INVALID_VALUE, "n_routed < 0");
    if (dm->top_k > dm->n_routed) return fail(MOE_ERR_INVALID_VALUE, "top_k > n_routed");
    if (dm->d_ff < 1) return fail(MOE_ERR_INVALID_VALUE, "non-positive width");
  }
  if (dm->d_model < 1 || dm->d_ff < 0 || dm->d_ff_shared < 0) return fail(MOE_ERR_INVALID_VALUE, "non-positive width");
  if (dm->capacity < 0) return fail(MOE_ERR_INVALID_VALUE, "capacity < 0");
  if (dm->n_group < 0) return fail(MOE_ERR_INVALID_VALUE, "n_group < 0");
  if (dm->n_group > 1 && !dense) {
    if (dm->n_group > 64) return fail(MOE_ERR_UNSUPPORTED, "n_group > 64");
    if (dm->n_routed % dm->n_group) return fail(MOE_ERR_INVALID_VALUE, "n_routed is not a multiple of n_group");
    if (dm->topk_group < 1 || dm->topk_group > dm->n_group)
      return fail(MOE_ERR_INVALID_VALUE, "topk_group must be in [1, n_group]");
    if ((int64_t)dm->topk_group * (dm->n_routed / dm->n_group) < dm->top_k)
      return fail(MOE_ERR_INVALID_VALUE, "topk_group groups hold fewer than top_k experts");
  }
  if (dm->dtype != MOE_F32 && dm->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "unknown dtype %d", dm->dtype);
  if (dm->out_dtype != MOE_F32 && dm->out_dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "unknown out_dtype %d", dm->out_dtype);
  if (dm->top_k > MOE_MAX_TOPK) return fail(MOE_ERR_UNSUPPORTED, "top_k > 16");
  if (dm->n_routed > 1024) return fail(MOE_ERR_UNSUPPORTED, "n_routed > 1024");
  if (dm->d_model < 64 || dm->d_model > 32768 || dm->d_model % 64)
    return fail(MOE_ERR_UNSUPPORTED, "d_model must be a multiple of 64 in [64, 32768]");
  if (dm->d_ff % 64 || dm->d_ff > 65536) return fail(MOE_ERR_UNSUPPORTED, "d_ff must be a multiple of 64, <= 65536");
  if (dm->d_ff_shared % 64 || dm->d_ff_shared > 65536)
    return fail(MOE_ERR_UNSUPPORTED, "d_ff_shared must be a multiple of 64, <= 65536");
  if (T * (int64_t)dm->top_k >= (int64_t)1 << 31) return fail(MOE_ERR_UNSUPPORTED, "T * top_k >= 2^31");
  // one work-group of 512 work-items per token in the combine, one wave per
  // token in top-k and RMSNorm: with T <= 2^22 every such dispatch stays under
  // the 2^32 work-items of the dispatch packet's grid size
  if (T > MOE_MAX_TOKENS)
    return fail(MOE_ERR_UNSUPPORTED, "T = %lld exceeds %d tokens per call; split the token batch", (long long)T,
                MOE_MAX_TOKENS);
  return MOE_OK;
}

static moe_status need_routed(const moe_dims &dm) {
  if (dm.n_routed < 1) return fail(MOE_ERR_INVALID_VALUE, "this call needs routed experts (n_routed >= 1)");
  return MOE_OK;
}

static moe_status check_ptr(const void *p, const char *name) {
  if (!p) return fail(MOE_ERR_INVALID_VALUE, "%s is NULL", name);
  if (!al16(p)) return fail(MOE_ERR_INVALID_VALUE, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

#define MOE_CHECK(expr)              \
  do {                               \
    moe_status s_ = (expr);          \
    if (s_ != MOE_OK) return s_;     \
  } while (0)

static moe_status check_ws(const moe_dims &dm, int64_t T, const void *ws, size_t ws_bytes, WsLayout *L) {
  *L = moe_ws_layout(dm, T);
  MOE_CHECK(check_ptr(ws, "ws"));
  if (ws_bytes < L->total)
    return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", ws_bytes, L->total);
  return MOE_OK;
}

static moe_status check_weights(const moe_dims &dm, const moe_weights *w, bool need_router, bool need_experts) {
  if (!w) return fail(MOE_ERR_INVALID_VALUE, "weights is NULL");
  const bool dense = dm.n_routed == 0;
  if (need_router && !dense) MOE_CHECK(check_ptr(w->w_router, "w_router"));
  if (w->router_bias && ((uintptr_t)w->router_bias & 3u))
    return fail(MOE_ERR_INVALID_VALUE, "router_bias is not 4-byte aligned");
  if (need_experts) {
    if (!dense) {
      MOE_CHECK(check_ptr(w->w1, "w1"));
      MOE_CHECK(check_ptr(w->w3, "w3"));
      MOE_CHECK(check_ptr(w->w2, "w2"));
    }
    if (dm.d_ff_shared > 0) {
      MOE_CHECK(check_ptr(w->w1s, "w1s"));
      MOE_CHECK(check_ptr(w->w3s, "w3s"));
      MOE_CHECK(check_ptr(w->w2s, "w2s"));
    } else if (w->w1s || w->w3s || w->w2s) {
      return fail(MOE_ERR_INVALID_VALUE, "shared weights given but d_ff_shared == 0");
    }
  }
  return MOE_OK;
}

static moe_status check_opts(const moe_options *o) {
  if (!o) return MOE_OK;
  if (o->path < 0 || o->path > 2) return fail(MOE_ERR_INVALID_VALUE, "options.path must be 0, 1 or 2");
  if (o->n_events < 0 || (o->n_events > 0 && !o->events)) return fail(MOE_ERR_INVALID_VALUE, "bad options.events");
  return MOE_OK;
}

// Which expert-FFN kernels run: 1 prefill, 2 decode.  A dense layer's decode
// kernels stream its single weight set once per pass of up to 64 rows and
// take the tiled GEMMs beyond 256 tokens (measured crossover at the
// DeepSeek-V3 dense shape); a routed layer's experts see about T*k/N_r rows
// each.
static int pick_path(const moe_dims &dm, int64_t T, const moe_options *o) {
  const int want = o ? o->path : 0;
  if (want != 0) return want;
  if (dm.n_routed == 0) return T <= 256 ? 2 : 1;
  return (T * dm.top_k <= 2 * (int64_t)dm.n_routed && T <= 256) ? 2 : 1;
}

// Records events[base + i] at stage boundary i (when the caller gave it).
struct EventHook {
  const moe_options *o;
  hipStream_t st;
  int base = 0;
  void rec(int i) const {
    i += base;
    if (o && o->events && i < o->n_events && o->events[i]) (void)hipEventRecord((hipEvent_t)o->events[i], st);
  }
  hipEvent_t get(int i) const {
    i += base;
    return (o && o->events && i < o->n_events) ? (hipEvent_t)o->events[i] : nullptr;
  }
};

// The tile prefixes are read by every FFN kernel except the dense layers'
// decode kernels.
static bool needs_tile_offsets(const moe_dims &dm, int64_t T, const moe_options *o) {
  return !(dm.n_routed == 0 && dm.dtype == MOE_BF16 && pick_path(dm, T, o) == 2);
}

// The bf16 prefill GEMMs address their operands through buffer resources
// with 32-bit byte offsets: every matrix they read must stay under 4 GiB.
// The expert-FFN launches of the chosen path must each stay under 2^32
// work-items (the dispatch packet's grid size).
static moe_status check_path_limits(const moe_dims &dm, int64_t T, const moe_options *o) {
  const int path = pick_path(dm, T, o);
  if (dm.dtype == MOE_BF16 && path == 1) {
    const uint64_t lim = (uint64_t)1 << 32;
    const uint64_t R = (uint64_t)T * dm.top_k;
    if ((uint64_t)T * dm.d_model * 2 >= lim || R * dm.d_ff * 2 >= lim || (uint64_t)T * dm.d_ff_shared * 2 >= lim ||
        (uint64_t)dm.d_ff * dm.d_model * 2 >= lim || (uint64_t)dm.d_ff_shared * dm.d_model * 2 >= lim)
      return fail(MOE_ERR_UNSUPPORTED,
                  "prefill path: u [T, d], the hidden activations [T*k, f] / [T, f_s] and each weight matrix must "
                  "be under 4 GiB (T = %lld); split the token batch",
                  (long long)T);
  }
  const int64_t wgs = dm.dtype == MOE_F32 ? ffn_f32_max_workgroups(dm, T)
                      : path == 2         ? ffn_decode_max_workgroups(dm, T)
                                          : ffn_prefill_max_workgroups(dm, T);
  if (wgs * 256 >= ((int64_t)1 << 32))
    return fail(MOE_ERR_UNSUPPORTED,
                "expert FFN: a launch of %lld work-groups of 256 exceeds the 2^32 work-items of one dispatch "
                "(T = %lld); split the token batch",
                (long long)wgs, (long long)T);
  return MOE_OK;
}

static moe_status run_ffn(const moe_dims &dm, int64_t T, const void *u, const moe_weights &w, const int32_t *counts,
                          const int32_t *offsets, const int32_t *row_token, float *y_rows, float *y_sh,
                          const moe_options *o, const WsLayout &L, char *ws, hipStream_t st, hipEvent_t ev_mid) {
  if (dm.dtype == MOE_F32) {
    MOE_TRY_HIP(launch_ffn_f32(dm, T, u, w, offsets, row_token, y_rows, y_sh, L, ws, st, ev_mid), "expert ffn (f32)");
    return MOE_OK;
  }
  const int path = pick_path(dm, T, o);
  if (path == 2) {
    MOE_TRY_HIP(launch_ffn_decode(dm, T, u, w, counts, offsets, row_token, y_rows, y_sh, L, ws, st, ev_mid),
                "expert ffn (decode)");
  } else {
    MOE_TRY_HIP(launch_ffn_prefill_bf16(dm, T, u, w, offsets, row_token, y_rows, y_sh, L, ws, st, ev_mid),
                "expert ffn (prefill)");
  }
  return MOE_OK;
}

static moe_status check_eps(double eps) {
  if (!(eps >= 0.0) || eps == __builtin_inf()) return fail(MOE_ERR_INVALID_VALUE, "eps must be finite and >= 0");
  return MOE_OK;
}

// the byte ranges [a, a + na) and [b, b + nb) must not overlap
static moe_status check_no_overlap(const void *a, size_t na, const void *b, size_t nb, const char *name) {
  const uintptr_t pa = (uintptr_t)a, pb = (uintptr_t)b;
  if (pa < pb + nb && pb < pa + na) return fail(MOE_ERR_INVALID_VALUE, "%s overlaps x", name);
  return MOE_OK;
}

static size_t td_bytes(const moe_dims &dm, int64_t T, int dtype) {
  return (size_t)T * dm.d_model * (dtype == MOE_BF16 ? 2 : 4);
}

// Router, permutation, expert FFNs and combine on the (validated) input u;
// resid (NULL or the block input x) is added in the combine.  Stage events
// 1..6 as in moe_layer_forward (relative to ev.base); a dense layer has no
// routing stages and records 1..3 at the same point.
static moe_status run_layer(const moe_dims &dm, int64_t T, const void *u, const moe_weights &wts, const void *resid,
                            void *out, const moe_options *opts, const WsLayout &L, char *w, hipStream_t st,
                            const EventHook &ev) {
  int32_t *idx = (int32_t *)(w + L.topk_idx);
  float *gw = (float *)(w + L.topk_w);
  int32_t *counts = (int32_t *)(w + L.counts);
  int32_t *offsets = (int32_t *)(w + L.offsets);
  int32_t *row_token = (int32_t *)(w + L.row_token);
  int32_t *token_row = (int32_t *)(w + L.token_row);
  float *y_rows = (float *)(w + L.y_rows);
  float *y_sh = dm.d_ff_shared > 0 ? (float *)(w + L.y_sh) : nullptr;
  if (dm.n_routed == 0) MOE_TRY_HIP(launch_diag_clear(w, st), "diag clear");
  if (dm.n_routed > 0) {  // the router's first kernel clears the diagnostics
    MOE_TRY_HIP(launch_router_logits(dm, T, u, wts.w_router, wts.router_bias, L, w, true, st), "router logits");
    ev.rec(1);
    MOE_TRY_HIP(launch_topk(dm, T, u, wts.w_router, wts.router_bias, idx, gw, L, w, st), "top-k");
    ev.rec(2);
    if (T <= MOE_PERM_BLOCK) {  // one launch for the permutation and the tile prefixes
      MOE_TRY_HIP(launch_permute_small(dm, T, idx, counts, offsets, row_token, token_row,
                                       (int32_t *)(w + L.tile_off), L, w, st),
                  "permute");
    } else {
      MOE_TRY_HIP(launch_permute(dm, T, idx, counts, offsets, row_token, token_row, L, w, st), "permute");
      MOE_TRY_HIP(launch_tile_offsets(dm, T, counts, L, w, st), "tile offsets");
    }
  } else {
    ev.rec(1);
    ev.rec(2);
    if (needs_tile_offsets(dm, T, opts)) MOE_TRY_HIP(launch_tile_offsets(dm, T, counts, L, w, st), "tile offsets");
  }
  ev.rec(3);
  MOE_CHECK(run_ffn(dm, T, u, wts, counts, offsets, row_token, y_rows, y_sh, opts, L, w, st, ev.get(4)));
  ev.rec(5);
  MOE_TRY_HIP(launch_combine(dm, T, y_rows, y_sh, gw, token_row, resid, out, st), "combine");
  ev.rec(6);
  return MOE_OK;
}

// ------------------------------------------------ library-owned scratch memory
// moe_layer_forward_static's workspace: one array per device, allocated with
// the code object when the library is first used on that device and held
// until the process ends.  In host code `scratch` names a host-side stand-in
// of the array, not its device address; the device address is looked up once
// per device (with that device current) and only that address is handed to
// kernels.
static __device__ __align__(256) char scratch[MOE_STATIC_WS_BYTES];

#define MOE_MAX_DEVICES 64
static std::mutex g_scratch_mu;
static void *g_scratch_ptr[MOE_MAX_DEVICES];

// Device address of the current device's scratch array (looked up on first use).
static moe_status scratch_for_current_device(char **out) {
  int dev = -1;
  MOE_TRY_HIP(hipGetDevice(&dev), "static scratch: hipGetDevice");
  if (dev < 0 || dev >= MOE_MAX_DEVICES)
    return fail(MOE_ERR_UNSUPPORTED, "static scratch: device %d is beyond the %d devices supported", dev,
                MOE_MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    MOE_TRY_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "static scratch: hipGetSymbolAddress");
    if (!p) return fail(MOE_ERR_HIP, "static scratch: hipGetSymbolAddress returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = (char *)g_scratch_ptr[dev];
  return MOE_OK;
}

extern "C" {

const char *moe_last_error(void) { return g_err; }

moe_status moe_workspace_size(const moe_dims *dims, int64_t T, size_t *bytes) {
  MOE_CHECK(check_dims(dims, T));
  if (!bytes) return fail(MOE_ERR_INVALID_VALUE, "bytes is NULL");
  *bytes = moe_ws_layout(*dims, T).total;
  return MOE_OK;
}

moe_status moe_router_topk(const moe_dims *dims, int64_t T, const void *u, const void *w_router,
                           const float *router_bias, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                           void *stream) {
  MOE_CHECK(check_dims(dims, T));
  MOE_CHECK(need_routed(*dims));
  if (T == 0) return MOE_OK;
  MOE_CHECK(check_ptr(u, "u"));
  MOE_CHECK(check_ptr(w_router, "w_router"));
  if (router_bias && ((uintptr_t)router_bias & 3u)) return fail(MOE_ERR_INVALID_VALUE, "router_bias misaligned");
  MOE_CHECK(check_ptr(topk_idx, "topk_idx"));
  MOE_CHECK(check_ptr(topk_w, "topk_w"));
  WsLayout L;
  MOE_CHECK(check_ws(*dims, T, ws, ws_bytes, &L));
  hipStream_t st = (hipStream_t)stream;
  char *w = (char *)ws;
  MOE_TRY_HIP(launch_router_logits(*dims, T, u, w_router, router_bias, L, w, true, st), "router logits");
  MOE_TRY_HIP(launch_topk(*dims, T, u, w_router, router_bias, topk_idx, topk_w, L, w, st), "top-k");
  return MOE_OK;
}

moe_status moe_permute(const moe_dims *dims, int64_t T, const int32_t *topk_idx, int32_t *counts, int32_t *offsets,
                       int32_t *row_token, int32_t *token_row, void *ws, size_t ws_bytes, void *stream) {
  MOE_CHECK(check_dims(dims, T));
  MOE_CHECK(need_routed(*dims));
  if (T == 0) return MOE_OK;
  MOE_CHECK(check_ptr(topk_idx, "topk_idx"));
  MOE_CHECK(check_ptr(counts, "counts"));
  MOE_CHECK(check_ptr(offsets, "offsets"));
  MOE_CHECK(check_ptr(row_token, "row_token"));
  MOE_CHECK(check_ptr(token_row, "token_row"));
  WsLayout L;
  MOE_CHECK(check_ws(*dims, T, ws, ws_bytes, &L));
  hipStream_t st = (hipStream_t)stream;
  char *w = (char *)ws;
  MOE_TRY_HIP(launch_diag_clear(w, st), "diag clear");
  MOE_TRY_HIP(launch_permute(*dims, T, topk_idx, counts, offsets, row_token, token_row, L, w, st), "permute");
  return MOE_OK;
}

moe_status moe_expert_ffn(const moe_dims *dims, int64_t T, const void *u, const moe_weights *wts,
                          const int32_t *counts, const int32_t *offsets, const int32_t *row_token, float *y_rows,
                          float *y_shared, const moe_options *opts, void *ws, size_t ws_bytes, void *stream) {
  MOE_CHECK(check_dims(dims, T));
  MOE_CHECK(check_opts(opts));
  if (T == 0) return MOE_OK;
  MOE_CHECK(check_ptr(u, "u"));
  MOE_CHECK(check_weights(*dims, wts, false, true));
  if (dims->n_routed > 0) {
    MOE_CHECK(check_ptr(counts, "counts"));
    MOE_CHECK(check_ptr(offsets, "offsets"));
    MOE_CHECK(check_ptr(row_token, "row_token"));
    MOE_CHECK(check_ptr(y_rows, "y_rows"));
  } else {
    counts = offsets = nullptr;
    row_token = nullptr;
    y_rows = nullptr;
  }
  if (dims->d_ff_shared > 0) MOE_CHECK(check_ptr(y_shared, "y_shared"));
  else if (y_shared) return fail(MOE_ERR_INVALID_VALUE, "y_shared given but d_ff_shared == 0");
  WsLayout L;
  MOE_CHECK(check_ws(*dims, T, ws, ws_bytes, &L));
  MOE_CHECK(check_path_limits(*dims, T, opts));
  hipStream_t st = (hipStream_t)stream;
  EventHook ev{opts, st};
  if (needs_tile_offsets(*dims, T, opts))
    MOE_TRY_HIP(launch_tile_offsets(*dims, T, counts, L, (char *)ws, st), "tile offsets");
  ev.rec(0);
  MOE_CHECK(run_ffn(*dims, T, u, *wts, counts, offsets, row_token, y_rows, y_shared, opts, L, (char *)ws, st,
                    ev.get(1)));
  ev.rec(2);
  return MOE_OK;
}

moe_status moe_combine(const moe_dims *dims, int64_t T, const float *y_rows, const float *y_shared,
                       const float *topk_w, const int32_t *token_row, void *out, void *stream) {
  MOE_CHECK(check_dims(dims, T));
  if (T == 0) return MOE_OK;
  if (dims->top_k > 0) {
    MOE_CHECK(check_ptr(y_rows, "y_rows"));
    if (y_shared) MOE_CHECK(check_ptr(y_shared, "y_shared"));
    MOE_CHECK(check_ptr(topk_w, "topk_w"));
    MOE_CHECK(check_ptr(token_row, "token_row"));
  } else {
    MOE_CHECK(check_ptr(y_shared, "y_shared"));
    y_rows = topk_w = nullptr;
    token_row = nullptr;
  }
  MOE_CHECK(check_ptr(out, "out"));
  MOE_TRY_HIP(launch_combine(*dims, T, y_rows, y_shared, topk_w, token_row, nullptr, out, (hipStream_t)stream),
              "combine");
  return MOE_OK;
}

moe_status moe_layer_forward(const moe_dims *dims, int64_t T, const void *u, const moe_weights *wts, void *out,
                             const moe_options *opts, void *ws, size_t ws_bytes, void *stream) {
  MOE_CHECK(check_dims(dims, T));
  MOE_CHECK(check_opts(opts));
  if (T == 0) return MOE_OK;
  MOE_CHECK(check_ptr(u, "u"));
  MOE_CHECK(check_weights(*dims, wts, true, true));
  MOE_CHECK(check_ptr(out, "out"));
  WsLayout L;
  MOE_CHECK(check_ws(*dims, T, ws, ws_bytes, &L));
  MOE_CHECK(check_path_limits(*dims, T, opts));
  hipStream_t st = (hipStream_t)stream;
  EventHook ev{opts, st};
  ev.rec(0);
  return run_layer(*dims, T, u, *wts, nullptr, out, opts, L, (char *)ws, st, ev);
}

moe_status moe_layer_forward_static(const moe_dims *dims, int64_t T, const void *u, const moe_weights *wts,
                                    void *out, const moe_options *opts, void *stream) {
  MOE_CHECK(check_dims(dims, T));
  MOE_CHECK(check_opts(opts));
  if (T == 0) return MOE_OK;
  MOE_CHECK(check_ptr(u, "u"));
  MOE_CHECK(check_weights(*dims, wts, true, true));
  MOE_CHECK(check_ptr(out, "out"));
  const WsLayout L = moe_ws_layout(*dims, T);
  if (L.total > (size_t)MOE_STATIC_WS_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "static scratch: this call needs %zu bytes of workspace, the library's scratch holds %zu; "
                "use moe_layer_forward with a workspace or split the token batch",
                L.total, (size_t)MOE_STATIC_WS_BYTES);
  MOE_CHECK(check_path_limits(*dims, T, opts));
  char *w = nullptr;
  MOE_CHECK(scratch_for_current_device(&w));
  hipStream_t st = (hipStream_t)stream;
  EventHook ev{opts, st};
  ev.rec(0);
  return run_layer(*dims, T, u, *wts, nullptr, out, opts, L, w, st, ev);
}

moe_status moe_rmsnorm(const moe_dims *dims, int64_t T, const void *x, const float *norm_weight, double eps, void *u,
                       void *stream) {
  MOE_CHECK(check_dims(dims, T));
  if (T == 0) return MOE_OK;
  MOE_CHECK(check_ptr(x, "x"));
  MOE_CHECK(check_ptr(norm_weight, "norm_weight"));
  MOE_CHECK(check_ptr(u, "u"));
  MOE_CHECK(check_eps(eps));
  MOE_CHECK(check_no_overlap(x, td_bytes(*dims, T, dims->dtype), u, td_bytes(*dims, T, dims->dtype), "u"));
  MOE_TRY_HIP(launch_rmsnorm(*dims, T, x, norm_weight, eps, u, (hipStream_t)stream), "rmsnorm");
  return MOE_OK;
}

moe_status moe_block_forward(const moe_dims *dims, int64_t T, const void *x, const float *norm_weight, double eps,
                             const moe_weights *wts, void *out, const moe_options *opts, void *ws, size_t ws_bytes,
                             void *stream) {
  MOE_CHECK(check_dims(dims, T));
  MOE_CHECK(check_opts(opts));
  if (T == 0) return MOE_OK;
  MOE_CHECK(check_ptr(x, "x"));
  MOE_CHECK(check_ptr(norm_weight, "norm_weight"));
  MOE_CHECK(check_eps(eps));
  MOE_CHECK(check_weights(*dims, wts, true, true));
  MOE_CHECK(check_ptr(out, "out"));
  WsLayout L;
  MOE_CHECK(check_ws(*dims, T, ws, ws_bytes, &L));
  MOE_CHECK(check_path_limits(*dims, T, opts));
  MOE_CHECK(check_no_overlap(x, td_bytes(*dims, T, dims->dtype), out, td_bytes(*dims, T, dims->out_dtype), "out"));
  hipStream_t st = (hipStream_t)stream;
  char *w = (char *)ws;
  void *u = w + L.u_norm;
  EventHook ev{opts, st};
  ev.rec(0);
  MOE_TRY_HIP(launch_rmsnorm(*dims, T, x, norm_weight, eps, u, st), "rmsnorm");
  ev.rec(1);
  ev.base = 1;
  return run_layer(*dims, T, u, *wts, x, out, opts, L, w, st, ev);
}

moe_status moe_read_diagnostics(const void *ws, moe_diag *diag, void *stream) {
  if (!ws || !diag) return fail(MOE_ERR_INVALID_VALUE, "NULL argument");
  hipStream_t st = (hipStream_t)stream;
  MOE_TRY_HIP(hipMemcpyAsync(diag, ws, sizeof(moe_diag), hipMemcpyDeviceToHost, st), "read diagnostics");
  MOE_TRY_HIP(hipStreamSynchronize(st), "read diagnostics");
  return MOE_OK;
}

}  // extern "C"
