// C ABI of libqmoe: argument validation (host only, before any launch) and
// dispatch to the gfx950 kernels.
#include <math.h>

#include <mutex>

#include "qmoe.h"
#include "qmoe_internal.h"

#include <cstdlib>

using namespace qmoe;

namespace {

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

inline int block_of(int32_t fmt) { return fmt == QMOE_FMT_NVFP4 ? 16 : 32; }

inline qmoe_status check_launch(hipError_t e) { return e == hipSuccess ? QMOE_OK : QMOE_ELAUNCH; }

// Common checks of an FP4 weight descriptor.
qmoe_status check_weights(const qmoe_fp4_weights *w) {
  if (!w || !w->w || !w->scales) return QMOE_EINVAL;
  if (w->fmt != QMOE_FMT_NVFP4 && w->fmt != QMOE_FMT_MXFP4) return QMOE_EINVAL;
  if (w->E < 1 || w->K < 1 || w->N < 1) return QMOE_EINVAL;
  if (w->fmt == QMOE_FMT_NVFP4 && !w->gscale) return QMOE_EINVAL;
  if (!aligned16(w->w) || !aligned16(w->scales) || (w->gscale && !aligned16(w->gscale))) return QMOE_EALIGN;
  if (w->K % block_of(w->fmt) != 0) return QMOE_EUNSUPPORTED;
  // kernels address one expert's packed weights with 32-bit buffer offsets
  if ((int64_t)w->K * w->N / 2 >= ((int64_t)1 << 31)) return QMOE_EUNSUPPORTED;
  return QMOE_OK;
}

struct FcShape {
  int32_t rows;
  int32_t max_rows_per_expert;  // a token selects an expert at most once
};

qmoe_status check_fc(const qmoe_fp4_weights *w, int32_t T, int32_t k, const void *act, const void *offsets,
                     const void *out, qmoe_path path, FcShape *shape) {
  if (!act || !offsets || !out) return QMOE_EINVAL;
  if (T < 1 || k < 1) return QMOE_EINVAL;
  qmoe_status st = check_weights(w);
  if (st != QMOE_OK) return st;
  if (k > w->E) return QMOE_EINVAL;
  if (path != QMOE_PATH_AUTO && path != QMOE_PATH_GEMV && path != QMOE_PATH_GROUPED) return QMOE_EINVAL;
  if (!aligned16(act) || !aligned16(offsets) || !aligned16(out)) return QMOE_EALIGN;
  if (w->E > QMOE_MAX_EXPERTS || k > QMOE_MAX_TOPK) return QMOE_EUNSUPPORTED;
  if (w->N % 32 != 0) return QMOE_EUNSUPPORTED;
  const int64_t rows = (int64_t)T * k;
  if (rows > (1 << 24)) return QMOE_EUNSUPPORTED;
  shape->rows = (int32_t)rows;
  shape->max_rows_per_expert = T;
  return QMOE_OK;
}

// The GEMV grid's y dimension counts groups of eight (slot, column tile)
// items, at most 64 slots: within 65535 for up to 8191 column tiles.
constexpr int kGemvMaxColumnTiles = 8191;
inline bool gemv_grid_fits(const qmoe_fp4_weights *w) {
  return (w->N + kGemvTileN - 1) / kGemvTileN <= kGemvMaxColumnTiles;
}

// Resolves AUTO and checks the row window and tile shape of each path.
// AUTO follows the decode GEMV's 64-row window: the GEMV up to 64 expanded
// rows, the grouped MFMA GEMM (the dense contraction of prefill) above.  The
// grouped kernel also takes multi-row decode shapes when asked for
// explicitly (MXFP4 T=8 layer: 143 us grouped against 171 us GEMV).
qmoe_status resolve_path(qmoe_path path, int32_t rows, int32_t max_rows_per_expert, const qmoe_fp4_weights *w,
                         qmoe_path *out) {
  (void)max_rows_per_expert;
  qmoe_path p = path;
  if (p == QMOE_PATH_AUTO) p = rows <= QMOE_GEMV_MAX_ROWS ? QMOE_PATH_GEMV : QMOE_PATH_GROUPED;
  if (p == QMOE_PATH_GEMV && (rows > QMOE_GEMV_MAX_ROWS || !gemv_grid_fits(w))) return QMOE_EUNSUPPORTED;
  if (p == QMOE_PATH_GROUPED && (w->K % 64 != 0 || w->N % 128 != 0)) return QMOE_EUNSUPPORTED;
  // buffer resources address the activations of a call in 32 bits
  if (p == QMOE_PATH_GROUPED && (int64_t)rows * w->K * 2 >= ((int64_t)1 << 31)) return QMOE_EUNSUPPORTED;
  *out = p;
  return QMOE_OK;
}

qmoe_status run_fc(GemvArgs &a, const qmoe_fp4_weights *w, int max_rows, qmoe_path path, void *ws,
                   size_t *ws_bytes, hipStream_t stream) {
  const bool concat = a.concat != 0;
  const size_t need = path == QMOE_PATH_GROUPED ? grouped_workspace_bytes(a.rows, w->N, concat)
                                                : gemv_workspace_bytes(a.rows, max_rows, w->E, w->K, w->N, concat);
  if (!ws_bytes) return QMOE_EINVAL;
  if (!ws) {
    *ws_bytes = need;
    return QMOE_OK;
  }
  if (*ws_bytes < need) return QMOE_EWORKSPACE;
  if (!aligned16(ws)) return QMOE_EALIGN;
  a.w = w->w;
  a.scales = w->scales;
  a.gscale = w->gscale;
  a.E = w->E;
  a.K = w->K;
  a.N = w->N;
  const int fmt = w->fmt == QMOE_FMT_NVFP4 ? 0 : 1;
  if (path == QMOE_PATH_GROUPED) {
    if (!concat) return check_launch(launch_grouped(a, fmt, stream));
    // concatenated SwiGLU: g * u as float32 rows, then the pairing epilogue
    a.out_f32 = (float *)ws;
    qmoe_status st = check_launch(launch_grouped(a, fmt, stream));
    if (st != QMOE_OK) return st;
    a.partials = (float *)ws;
    a.nchunks = 1;
    return check_launch(launch_splitk_epilogue(a, stream));
  }
  gemv_plan(a, max_rows, ws);
  return check_launch(launch_fp4_gemv(a, fmt, max_rows, stream));
}

qmoe_status check_fp8_fc(const qmoe_fp8_weights *w, int32_t T, int32_t k, const void *act, const void *offsets,
                         const void *out, qmoe_path path, FcShape *shape, qmoe_path *resolved) {
  if (path != QMOE_PATH_AUTO && path != QMOE_PATH_GEMV && path != QMOE_PATH_GROUPED) return QMOE_EINVAL;
  if (!w || !w->w || !w->gscale || !act || !offsets || !out) return QMOE_EINVAL;
  if (T < 1 || k < 1 || w->E < 1 || w->K < 1 || w->N < 1 || k > w->E) return QMOE_EINVAL;
  if (!aligned16(w->w) || !aligned16(w->gscale) || !aligned16(act) || !aligned16(offsets) || !aligned16(out))
    return QMOE_EALIGN;
  if (w->E > QMOE_MAX_EXPERTS || k > QMOE_MAX_TOPK) return QMOE_EUNSUPPORTED;
  if (w->K % 16 != 0 || w->N % 32 != 0) return QMOE_EUNSUPPORTED;
  // one expert's bytes are addressed with 32-bit buffer offsets
  if ((int64_t)w->K * w->N >= ((int64_t)1 << 31)) return QMOE_EUNSUPPORTED;
  const int64_t rows = (int64_t)T * k;
  if (rows > (1 << 24)) return QMOE_EUNSUPPORTED;
  shape->rows = (int32_t)rows;
  shape->max_rows_per_expert = T;
  // AUTO: the grouped MFMA kernel beyond the decode window when K % 64 == 0
  qmoe_path p = path;
  if (p == QMOE_PATH_AUTO) p = (rows <= QMOE_GEMV_MAX_ROWS || w->K % 64 != 0) ? QMOE_PATH_GEMV : QMOE_PATH_GROUPED;
  if (p == QMOE_PATH_GROUPED && w->K % 64 != 0) return QMOE_EUNSUPPORTED;
  // the grouped kernel addresses the activations of a call in 32 bits
  if (p == QMOE_PATH_GROUPED && rows * w->K * 2 >= ((int64_t)1 << 31)) return QMOE_EUNSUPPORTED;
  *resolved = p;
  return QMOE_OK;
}

qmoe_status run_fp8(GemvArgs &a, const qmoe_fp8_weights *w, int max_rows, qmoe_path path, void *ws,
                    size_t *ws_bytes, hipStream_t stream) {
  const size_t need = fp8_workspace_bytes(a.rows, w->N, a.concat != 0);
  if (!ws_bytes) return QMOE_EINVAL;
  if (!ws) {
    *ws_bytes = need;
    return QMOE_OK;
  }
  if (*ws_bytes < need) return QMOE_EWORKSPACE;
  if (!aligned16(ws)) return QMOE_EALIGN;
  a.w = w->w;
  a.gscale = w->gscale;
  a.E = w->E;
  a.K = w->K;
  a.N = w->N;
  if (path == QMOE_PATH_GROUPED) return check_launch(launch_fp8_grouped(a, ws, stream));
  return check_launch(launch_fp8_gemv(a, max_rows, ws, stream));
}

qmoe_status layer_decode(const float *logits, const float *router_weights, const uint16_t *x, int32_t T, int32_t k,
                         const qmoe_fp4_weights *w1, const qmoe_fp4_weights *w2, const qmoe_swiglu *act,
                         int32_t route_in_fc1, int32_t *topk_idx, float *topk_w, int32_t *expert_offsets,
                         int32_t *perm_to_expanded, int32_t *expanded_to_perm, uint16_t *out, void *ws,
                         size_t *ws_bytes, hipStream_t stream);

}  // namespace

// Scratch of qmoe_fp4_moe_layer_decode_noalloc: both layers' split-K partial
// sums live here instead of in a caller's workspace.  A file-scope device
// array: every GPU the library runs on holds its own copy (zero-initialised
// when the code object loads) until the process ends.  In host code the name
// `scratch` is only a stand-in; device_scratch() resolves the current
// device's address once and every launch takes that address.
static __device__ __attribute__((aligned(256))) uint8_t scratch[QMOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`, resolved with hipGetSymbolAddress
// on the first call on that device (with the device current) and kept.
qmoe_status device_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QMOE_ELAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return QMOE_ELAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return QMOE_OK;
}

}  // namespace

extern "C" {

const char *qmoe_status_str(qmoe_status s) {
  switch (s) {
    case QMOE_OK: return "QMOE_OK";
    case QMOE_EINVAL: return "QMOE_EINVAL: invalid argument";
    case QMOE_EUNSUPPORTED: return "QMOE_EUNSUPPORTED: shape or path not supported";
    case QMOE_EALIGN: return "QMOE_EALIGN: device pointer not 16-byte aligned";
    case QMOE_EWORKSPACE: return "QMOE_EWORKSPACE: workspace too small";
    case QMOE_ELAUNCH: return "QMOE_ELAUNCH: kernel launch failed";
  }
  return "QMOE_UNKNOWN";
}

qmoe_status qmoe_route_topk(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *topk_idx, float *topk_w,
                            int32_t *expert_offsets, int32_t *perm_to_expanded, int32_t *expanded_to_perm,
                            hipStream_t stream) {
  if (!logits || !topk_idx || !topk_w || !expert_offsets || !perm_to_expanded || !expanded_to_perm)
    return QMOE_EINVAL;
  if (T < 1 || E < 1 || k < 1 || k > E) return QMOE_EINVAL;
  if (!aligned16(logits) || !aligned16(topk_idx) || !aligned16(topk_w) || !aligned16(expert_offsets) ||
      !aligned16(perm_to_expanded) || !aligned16(expanded_to_perm))
    return QMOE_EALIGN;
  if (E > QMOE_MAX_EXPERTS || k > QMOE_MAX_TOPK) return QMOE_EUNSUPPORTED;
  if ((int64_t)T * k > (1 << 24)) return QMOE_EUNSUPPORTED;
  return check_launch(
      launch_route(logits, nullptr, T, E, k, topk_idx, topk_w, expert_offsets, perm_to_expanded, expanded_to_perm,
                   stream));
}

qmoe_status qmoe_route_topk_router_weights(const float *logits, const float *router_weights, int32_t T, int32_t E,
                                           int32_t k, int32_t *topk_idx, float *topk_w, int32_t *expert_offsets,
                                           int32_t *perm_to_expanded, int32_t *expanded_to_perm, hipStream_t stream) {
  if (!logits || !router_weights || !topk_idx || !topk_w || !expert_offsets || !perm_to_expanded ||
      !expanded_to_perm)
    return QMOE_EINVAL;
  if (T < 1 || E < 1 || k < 1 || k > E) return QMOE_EINVAL;
  if (!aligned16(logits) || !aligned16(router_weights) || !aligned16(topk_idx) || !aligned16(topk_w) ||
      !aligned16(expert_offsets) || !aligned16(perm_to_expanded) || !aligned16(expanded_to_perm))
    return QMOE_EALIGN;
  if (E > QMOE_MAX_EXPERTS || k > QMOE_MAX_TOPK) return QMOE_EUNSUPPORTED;
  if ((int64_t)T * k > (1 << 24)) return QMOE_EUNSUPPORTED;
  return check_launch(launch_route(logits, router_weights, T, E, k, topk_idx, topk_w, expert_offsets,
                                   perm_to_expanded, expanded_to_perm, stream));
}

qmoe_status qmoe_fp4_resolve_path(int32_t T, int32_t k, const qmoe_fp4_weights *w, qmoe_path path,
                                  qmoe_path *resolved) {
  if (!resolved) return QMOE_EINVAL;
  if (T < 1 || k < 1) return QMOE_EINVAL;
  qmoe_status st = check_weights(w);
  if (st != QMOE_OK) return st;
  if (k > w->E) return QMOE_EINVAL;
  if (path != QMOE_PATH_AUTO && path != QMOE_PATH_GEMV && path != QMOE_PATH_GROUPED) return QMOE_EINVAL;
  if (w->E > QMOE_MAX_EXPERTS || k > QMOE_MAX_TOPK) return QMOE_EUNSUPPORTED;
  if (w->N % 32 != 0) return QMOE_EUNSUPPORTED;
  const int64_t rows = (int64_t)T * k;
  if (rows > (1 << 24)) return QMOE_EUNSUPPORTED;
  return resolve_path(path, (int32_t)rows, T, w, resolved);
}

qmoe_status qmoe_fp4_gemv_fc1_swiglu(const uint16_t *x, int32_t T, int32_t k, const qmoe_fp4_weights *w1,
                                     const int32_t *expert_offsets, const int32_t *perm_to_expanded,
                                     const qmoe_swiglu *act, uint16_t *h, void *ws, size_t *ws_bytes,
                                     qmoe_path path, hipStream_t stream) {
  FcShape sh;
  qmoe_status st = check_fc(w1, T, k, x, expert_offsets, h, path, &sh);
  if (st != QMOE_OK) return st;
  if (!perm_to_expanded) return QMOE_EINVAL;
  if (!aligned16(perm_to_expanded)) return QMOE_EALIGN;
  qmoe_path p;
  st = resolve_path(path, sh.rows, sh.max_rows_per_expert, w1, &p);
  if (st != QMOE_OK) return st;
  GemvArgs a = {};
  a.act = x;
  a.p2e = perm_to_expanded;
  a.offsets = expert_offsets;
  a.topk = k;
  a.rows = sh.rows;
  a.fc1 = 1;
  a.alpha = act ? act->alpha : 1.0f;
  a.beta = act ? act->beta : 0.0f;
  a.limit = act ? act->limit : INFINITY;
  const int32_t fusion = act ? act->fusion : QMOE_SWIGLU_INTERLEAVED;
  if (fusion != 0 && fusion != QMOE_SWIGLU_INTERLEAVED && fusion != QMOE_SWIGLU_CONCAT) return QMOE_EINVAL;
  a.concat = fusion == QMOE_SWIGLU_CONCAT;
  a.out_bf16 = h;
  return run_fc(a, w1, sh.max_rows_per_expert, p, ws, ws_bytes, stream);
}

qmoe_status qmoe_fp4_route_fc1_swiglu(const float *logits, const float *router_weights, const uint16_t *x,
                                      int32_t T, int32_t k, const qmoe_fp4_weights *w1, const qmoe_swiglu *act,
                                      int32_t *topk_idx, float *topk_w, int32_t *expert_offsets,
                                      int32_t *perm_to_expanded, int32_t *expanded_to_perm, uint16_t *h, void *ws,
                                      size_t *ws_bytes, hipStream_t stream) {
  if (!logits || !topk_idx || !topk_w || !expert_offsets || !perm_to_expanded || !expanded_to_perm)
    return QMOE_EINVAL;
  FcShape sh;
  qmoe_status st = check_fc(w1, T, k, x, expert_offsets, h, QMOE_PATH_GEMV, &sh);
  if (st != QMOE_OK) return st;
  if (!aligned16(logits) || (router_weights && !aligned16(router_weights)) || !aligned16(topk_idx) ||
      !aligned16(topk_w) || !aligned16(perm_to_expanded) || !aligned16(expanded_to_perm))
    return QMOE_EALIGN;
  // the maps of one call are ranked by one wave
  if (sh.rows > QMOE_GEMV_MAX_ROWS || !gemv_grid_fits(w1)) return QMOE_EUNSUPPORTED;
  GemvArgs a = {};
  a.act = x;
  a.topk = k;
  a.rows = sh.rows;
  a.fc1 = 1;
  a.alpha = act ? act->alpha : 1.0f;
  a.beta = act ? act->beta : 0.0f;
  a.limit = act ? act->limit : INFINITY;
  const int32_t fusion = act ? act->fusion : QMOE_SWIGLU_INTERLEAVED;
  if (fusion != 0 && fusion != QMOE_SWIGLU_INTERLEAVED && fusion != QMOE_SWIGLU_CONCAT) return QMOE_EINVAL;
  a.concat = fusion == QMOE_SWIGLU_CONCAT;
  a.out_bf16 = h;
  a.route_logits = logits;
  a.route_rw = router_weights;
  a.route_T = T;
  a.route_idx = topk_idx;
  a.route_w = topk_w;
  a.route_offsets = expert_offsets;
  a.route_p2e = perm_to_expanded;
  a.route_e2p = expanded_to_perm;
  return run_fc(a, w1, sh.max_rows_per_expert, QMOE_PATH_GEMV, ws, ws_bytes, stream);
}

qmoe_status qmoe_fp4_moe_layer_decode(const float *logits, const float *router_weights, const uint16_t *x,
                                      int32_t T, int32_t k, const qmoe_fp4_weights *w1, const qmoe_fp4_weights *w2,
                                      const qmoe_swiglu *act, int32_t route_in_fc1, int32_t *topk_idx, float *topk_w,
                                      int32_t *expert_offsets, int32_t *perm_to_expanded, int32_t *expanded_to_perm,
                                      uint16_t *out, void *ws, size_t *ws_bytes, hipStream_t stream) {
  return layer_decode(logits, router_weights, x, T, k, w1, w2, act, route_in_fc1, topk_idx, topk_w, expert_offsets,
                      perm_to_expanded, expanded_to_perm, out, ws, ws_bytes, stream);
}

qmoe_status qmoe_fp4_moe_layer_persistent(const float *logits, const float *router_weights, const uint16_t *x,
                                          int32_t T, int32_t k, const qmoe_fp4_weights *w1, const qmoe_fp4_weights *w2,
                                          const qmoe_swiglu *act, int32_t *topk_idx, float *topk_w,
                                          int32_t *expert_offsets, int32_t *perm_to_expanded,
                                          int32_t *expanded_to_perm, uint16_t *out, void *ws, size_t *ws_bytes,
                                          hipStream_t stream) {
  if (!logits || !topk_idx || !topk_w || !expert_offsets || !perm_to_expanded || !expanded_to_perm)
    return QMOE_EINVAL;
  FcShape sh;
  qmoe_status st = check_fc(w1, T, k, x, expert_offsets, out, QMOE_PATH_GEMV, &sh);
  if (st != QMOE_OK) return st;
  st = check_weights(w2);
  if (st != QMOE_OK) return st;
  if (w2->E != w1->E || w1->N != 2 * w2->K || w2->N != w1->K || w2->fmt != w1->fmt) return QMOE_EINVAL;
  if (!aligned16(logits) || (router_weights && !aligned16(router_weights)) || !aligned16(topk_idx) ||
      !aligned16(topk_w) || !aligned16(perm_to_expanded) || !aligned16(expanded_to_perm))
    return QMOE_EALIGN;
  const int32_t fusion = act ? act->fusion : QMOE_SWIGLU_INTERLEAVED;
  if (fusion != 0 && fusion != QMOE_SWIGLU_INTERLEAVED && fusion != QMOE_SWIGLU_CONCAT) return QMOE_EINVAL;
  const int32_t H = w1->K, I = w2->K;
  if (sh.rows > QMOE_GEMV_MAX_ROWS || H % 32 != 0) return QMOE_EUNSUPPORTED;
  if (I > 256 * kLayerMaxHChunks || H > 256 * kLayerMaxTiles2) return QMOE_EUNSUPPORTED;
  if (fusion == QMOE_SWIGLU_CONCAT && I % 256 != 0) return QMOE_EUNSUPPORTED;
  LayerArgs a = {};
  a.logits = logits;
  a.rw = router_weights;
  a.x = x;
  a.w1 = w1->w;
  a.s1 = w1->scales;
  a.g1 = w1->gscale;
  a.w2 = w2->w;
  a.s2 = w2->scales;
  a.g2 = w2->gscale;
  a.T = T;
  a.E = w1->E;
  a.k = k;
  a.H = H;
  a.I = I;
  a.concat = fusion == QMOE_SWIGLU_CONCAT;
  a.alpha = act ? act->alpha : 1.0f;
  a.beta = act ? act->beta : 0.0f;
  a.limit = act ? act->limit : INFINITY;
  a.idx = topk_idx;
  a.wts = topk_w;
  a.offsets = expert_offsets;
  a.p2e = perm_to_expanded;
  a.e2p = expanded_to_perm;
  a.out = out;
  a.rows = sh.rows;
  a.nch1 = (H + 255) / 256;
  a.nch2 = (I + 255) / 256;
  a.ntiles1 = (2 * I + 255) / 256;
  a.ntiles2 = (H + 255) / 256;
  a.max_polls = 1 << 18;
  // a smaller bound from the environment exercises the error path (tests)
  if (const char *env = getenv("QMOE_LAYER_MAX_POLLS")) {
    const long v = strtol(env, nullptr, 10);
    if (v >= 0 && v < a.max_polls) a.max_polls = (int32_t)v;
  }
  // workspace: counters, FC1 partial sums, FC2 partial sums (256-byte aligned parts)
  auto up = [](size_t v) { return (v + 255) & ~(size_t)255; };
  static_assert(((kLayerSyncBytes + 255) & ~(size_t)255) == QMOE_LAYER_SYNC_BYTES, "counter region");
  const size_t b_sync = QMOE_LAYER_SYNC_BYTES;
  const size_t b_p1 = up((size_t)a.nch1 * sh.rows * (2 * I) * sizeof(float));
  const size_t b_p2 = up((size_t)a.nch2 * sh.rows * H * sizeof(float));
  if (b_p1 >= ((size_t)1 << 31) || b_p2 >= ((size_t)1 << 31)) return QMOE_EUNSUPPORTED;
  if (!ws_bytes) return QMOE_EINVAL;
  if (!ws) {
    *ws_bytes = b_sync + b_p1 + b_p2;
    return QMOE_OK;
  }
  if (*ws_bytes < b_sync + b_p1 + b_p2) return QMOE_EWORKSPACE;
  if (!aligned16(ws)) return QMOE_EALIGN;
  char *base = (char *)ws;
  a.sync = (int32_t *)base;
  a.part1 = (float *)(base + b_sync);
  a.part2 = (float *)(base + b_sync + b_p1);
  return check_launch(launch_fp4_layer(a, w1->fmt == QMOE_FMT_NVFP4 ? 0 : 1, stream));
}

qmoe_status qmoe_fp4_moe_layer_decode_noalloc(const float *logits, const float *router_weights, const uint16_t *x,
                                              int32_t T, int32_t k, const qmoe_fp4_weights *w1,
                                              const qmoe_fp4_weights *w2, const qmoe_swiglu *act,
                                              int32_t route_in_fc1, int32_t *topk_idx, float *topk_w,
                                              int32_t *expert_offsets, int32_t *perm_to_expanded,
                                              int32_t *expanded_to_perm, uint16_t *out, hipStream_t stream) {
  // the argument checks and the scratch size, with nothing launched
  size_t need = 0;
  qmoe_status st = layer_decode(logits, router_weights, x, T, k, w1, w2, act, route_in_fc1, topk_idx, topk_w,
                                expert_offsets, perm_to_expanded, expanded_to_perm, out, nullptr, &need, stream);
  if (st != QMOE_OK) return st;
  if (need > (size_t)QMOE_NOALLOC_SCRATCH_BYTES) return QMOE_EWORKSPACE;
  void *ptr = nullptr;
  st = device_scratch(&ptr);
  if (st != QMOE_OK) return st;
  size_t have = (size_t)QMOE_NOALLOC_SCRATCH_BYTES;
  return layer_decode(logits, router_weights, x, T, k, w1, w2, act, route_in_fc1, topk_idx, topk_w, expert_offsets,
                      perm_to_expanded, expanded_to_perm, out, ptr, &have, stream);
}

}  // extern "C"

namespace {

qmoe_status layer_decode(const float *logits, const float *router_weights, const uint16_t *x, int32_t T, int32_t k,
                         const qmoe_fp4_weights *w1, const qmoe_fp4_weights *w2, const qmoe_swiglu *act,
                         int32_t route_in_fc1, int32_t *topk_idx, float *topk_w, int32_t *expert_offsets,
                         int32_t *perm_to_expanded, int32_t *expanded_to_perm, uint16_t *out, void *ws,
                         size_t *ws_bytes, hipStream_t stream) {
  if (!logits || !topk_idx || !topk_w || !expert_offsets || !perm_to_expanded || !expanded_to_perm)
    return QMOE_EINVAL;
  if (route_in_fc1 != 0 && route_in_fc1 != 1) return QMOE_EINVAL;
  FcShape sh;
  qmoe_status st = check_fc(w1, T, k, x, expert_offsets, out, QMOE_PATH_GEMV, &sh);
  if (st != QMOE_OK) return st;
  st = check_weights(w2);
  if (st != QMOE_OK) return st;
  if (w2->E != w1->E || w1->N != 2 * w2->K || w2->N != w1->K) return QMOE_EINVAL;
  if (!aligned16(logits) || (router_weights && !aligned16(router_weights)) || !aligned16(topk_idx) ||
      !aligned16(topk_w) || !aligned16(perm_to_expanded) || !aligned16(expanded_to_perm))
    return QMOE_EALIGN;
  if (sh.rows > QMOE_GEMV_MAX_ROWS || w2->N % 32 != 0 || w2->N % 8 != 0) return QMOE_EUNSUPPORTED;
  if (!gemv_grid_fits(w1) || !gemv_grid_fits(w2)) return QMOE_EUNSUPPORTED;
  const int32_t fusion = act ? act->fusion : QMOE_SWIGLU_INTERLEAVED;
  if (fusion != 0 && fusion != QMOE_SWIGLU_INTERLEAVED && fusion != QMOE_SWIGLU_CONCAT) return QMOE_EINVAL;
  // workspace: FC1's split-K partials (u, g applied), then FC2's
  const size_t p1 = (gemv_workspace_bytes(sh.rows, sh.max_rows_per_expert, w1->E, w1->K, w1->N, true) + 255) &
                    ~(size_t)255;
  const size_t p2 = gemv_workspace_bytes(sh.rows, sh.max_rows_per_expert, w2->E, w2->K, w2->N, true);
  // FC2's staging addresses FC1's partial planes with 32-bit buffer offsets
  if (p1 >= ((size_t)1 << 31)) return QMOE_EUNSUPPORTED;
  if (!ws_bytes) return QMOE_EINVAL;
  if (!ws) {
    *ws_bytes = p1 + p2;
    return QMOE_OK;
  }
  if (*ws_bytes < p1 + p2) return QMOE_EWORKSPACE;
  if (!aligned16(ws)) return QMOE_EALIGN;
  const int E = w1->E;
  if (!route_in_fc1) {
    st = check_launch(launch_route(logits, router_weights, T, E, k, topk_idx, topk_w, expert_offsets,
                                   perm_to_expanded, expanded_to_perm, stream));
    if (st != QMOE_OK) return st;
  }
  GemvArgs a1 = {};
  a1.act = x;
  a1.p2e = perm_to_expanded;
  a1.offsets = expert_offsets;
  a1.w = w1->w;
  a1.scales = w1->scales;
  a1.gscale = w1->gscale;
  a1.E = E;
  a1.K = w1->K;
  a1.N = w1->N;
  a1.topk = k;
  a1.rows = sh.rows;
  a1.fc1 = 1;
  a1.force_partials = 1;  // SwiGLU runs in FC2's staging
  a1.concat = fusion == QMOE_SWIGLU_CONCAT;
  if (route_in_fc1) {
    a1.route_logits = logits;
    a1.route_rw = router_weights;
    a1.route_T = T;
    a1.route_idx = topk_idx;
    a1.route_w = topk_w;
    a1.route_offsets = expert_offsets;
    a1.route_p2e = perm_to_expanded;
    a1.route_e2p = expanded_to_perm;
  }
  gemv_plan(a1, sh.max_rows_per_expert, ws);
  st = check_launch(launch_fp4_gemv(a1, w1->fmt == QMOE_FMT_NVFP4 ? 0 : 1, sh.max_rows_per_expert, stream));
  if (st != QMOE_OK) return st;
  GemvArgs a2 = {};
  a2.offsets = expert_offsets;
  a2.w = w2->w;
  a2.scales = w2->scales;
  a2.gscale = w2->gscale;
  a2.E = E;
  a2.K = w2->K;
  a2.N = w2->N;
  a2.topk = k;
  a2.rows = sh.rows;
  a2.fc1 = 0;
  a2.force_partials = 1;  // the finalize sums FC2's planes
  a2.h_partials = (const float *)ws;
  a2.h_nchunks = a1.nchunks;
  a2.h_concat = a1.concat;
  a2.h_alpha = act ? act->alpha : 1.0f;
  a2.h_beta = act ? act->beta : 0.0f;
  a2.h_limit = act ? act->limit : INFINITY;
  float *ws2 = (float *)((char *)ws + p1);
  gemv_plan(a2, sh.max_rows_per_expert, ws2);
  st = check_launch(launch_fp4_gemv(a2, w2->fmt == QMOE_FMT_NVFP4 ? 0 : 1, sh.max_rows_per_expert, stream));
  if (st != QMOE_OK) return st;
  const size_t plane = (size_t)sh.rows * w2->N;
  return check_launch(
      launch_finalize(ws2, a2.nchunks, plane, topk_w, expanded_to_perm, T, k, w2->N, out, stream));
}

}  // namespace

extern "C" {

qmoe_status qmoe_fp4_gemv_fc2(const uint16_t *h, int32_t T, int32_t k, const qmoe_fp4_weights *w2,
                              const int32_t *expert_offsets, float *y_rows, void *ws, size_t *ws_bytes,
                              qmoe_path path, hipStream_t stream) {
  FcShape sh;
  qmoe_status st = check_fc(w2, T, k, h, expert_offsets, y_rows, path, &sh);
  if (st != QMOE_OK) return st;
  qmoe_path p;
  st = resolve_path(path, sh.rows, sh.max_rows_per_expert, w2, &p);
  if (st != QMOE_OK) return st;
  GemvArgs a = {};
  a.act = h;
  a.offsets = expert_offsets;
  a.topk = k;
  a.rows = sh.rows;
  a.fc1 = 0;
  a.out_f32 = y_rows;
  return run_fc(a, w2, sh.max_rows_per_expert, p, ws, ws_bytes, stream);
}

qmoe_status qmoe_fp4_gemv_fc2_finalize(const uint16_t *h, int32_t T, int32_t k, const qmoe_fp4_weights *w2,
                                       const int32_t *expert_offsets, const float *topk_w,
                                       const int32_t *expanded_to_perm, uint16_t *out, void *ws, size_t *ws_bytes,
                                       qmoe_path path, hipStream_t stream) {
  FcShape sh;
  qmoe_status st = check_fc(w2, T, k, h, expert_offsets, out, path, &sh);
  if (st != QMOE_OK) return st;
  if (!topk_w || !expanded_to_perm) return QMOE_EINVAL;
  if (!aligned16(topk_w) || !aligned16(expanded_to_perm)) return QMOE_EALIGN;
  if (w2->N % 8 != 0) return QMOE_EUNSUPPORTED;
  qmoe_path p;
  st = resolve_path(path, sh.rows, sh.max_rows_per_expert, w2, &p);
  if (st != QMOE_OK) return st;
  GemvArgs a = {};
  a.act = h;
  a.offsets = expert_offsets;
  a.topk = k;
  a.rows = sh.rows;
  a.fc1 = 0;
  a.force_partials = 1;
  a.w = w2->w;
  a.scales = w2->scales;
  a.gscale = w2->gscale;
  a.E = w2->E;
  a.K = w2->K;
  a.N = w2->N;
  // workspace: the GEMV's split-K partials, or the grouped path's float32 rows
  const size_t plane = (size_t)sh.rows * w2->N;
  size_t need = p == QMOE_PATH_GROUPED
                    ? plane * sizeof(float)
                    : gemv_workspace_bytes(sh.rows, sh.max_rows_per_expert, w2->E, w2->K, w2->N, true);
  if (need < 256) need = 256;
  if (!ws_bytes) return QMOE_EINVAL;
  if (!ws) {
    *ws_bytes = need;
    return QMOE_OK;
  }
  if (*ws_bytes < need) return QMOE_EWORKSPACE;
  if (!aligned16(ws)) return QMOE_EALIGN;
  const int fmt = w2->fmt == QMOE_FMT_NVFP4 ? 0 : 1;
  int nsplit = 1;
  if (p == QMOE_PATH_GROUPED) {
    a.out_f32 = (float *)ws;
    st = check_launch(launch_grouped(a, fmt, stream));
  } else {
    gemv_plan(a, sh.max_rows_per_expert, ws);
    nsplit = a.nchunks;
    st = check_launch(launch_fp4_gemv(a, fmt, sh.max_rows_per_expert, stream));
  }
  if (st != QMOE_OK) return st;
  return check_launch(
      launch_finalize((const float *)ws, nsplit, plane, topk_w, expanded_to_perm, T, k, w2->N, out, stream));
}

qmoe_status qmoe_finalize(const float *y_rows, const float *topk_w, const int32_t *expanded_to_perm, int32_t T,
                          int32_t k, int32_t H, uint16_t *out, hipStream_t stream) {
  if (!y_rows || !topk_w || !expanded_to_perm || !out) return QMOE_EINVAL;
  if (T < 1 || k < 1 || H < 1) return QMOE_EINVAL;
  if (!aligned16(y_rows) || !aligned16(topk_w) || !aligned16(expanded_to_perm) || !aligned16(out))
    return QMOE_EALIGN;
  if (k > QMOE_MAX_TOPK || H % 8 != 0) return QMOE_EUNSUPPORTED;
  return check_launch(launch_finalize(y_rows, 1, 0, topk_w, expanded_to_perm, T, k, H, out, stream));
}

qmoe_status qmoe_dequant_fp4(const qmoe_fp4_weights *w, uint16_t *out, hipStream_t stream) {
  qmoe_status st = check_weights(w);
  if (st != QMOE_OK) return st;
  if (!out) return QMOE_EINVAL;
  if (!aligned16(out)) return QMOE_EALIGN;
  if (w->K % 64 != 0 || w->N % 256 != 0) return QMOE_EUNSUPPORTED;
  if (w->E > 65535 || w->K / 64 > 65535 || w->N / 256 > 65535) return QMOE_EUNSUPPORTED;
  return check_launch(
      launch_dequant(w->w, w->scales, w->gscale, w->E, w->K, w->N, w->fmt == QMOE_FMT_NVFP4 ? 0 : 1, out, stream));
}

qmoe_status qmoe_fp8_gemv_fc1_swiglu(const uint16_t *x, int32_t T, int32_t k, const qmoe_fp8_weights *w1,
                                     const int32_t *expert_offsets, const int32_t *perm_to_expanded,
                                     const qmoe_swiglu *act, uint16_t *h, void *ws, size_t *ws_bytes,
                                     qmoe_path path, hipStream_t stream) {
  FcShape sh;
  qmoe_path p;
  qmoe_status st = check_fp8_fc(w1, T, k, x, expert_offsets, h, path, &sh, &p);
  if (st != QMOE_OK) return st;
  if (!perm_to_expanded) return QMOE_EINVAL;
  if (!aligned16(perm_to_expanded)) return QMOE_EALIGN;
  GemvArgs a = {};
  a.act = x;
  a.p2e = perm_to_expanded;
  a.offsets = expert_offsets;
  a.topk = k;
  a.rows = sh.rows;
  a.fc1 = 1;
  a.alpha = act ? act->alpha : 1.0f;
  a.beta = act ? act->beta : 0.0f;
  a.limit = act ? act->limit : INFINITY;
  const int32_t fusion = act ? act->fusion : QMOE_SWIGLU_INTERLEAVED;
  if (fusion != 0 && fusion != QMOE_SWIGLU_INTERLEAVED && fusion != QMOE_SWIGLU_CONCAT) return QMOE_EINVAL;
  a.concat = fusion == QMOE_SWIGLU_CONCAT;
  a.out_bf16 = h;
  return run_fp8(a, w1, sh.max_rows_per_expert, p, ws, ws_bytes, stream);
}

qmoe_status qmoe_fp8_gemv_fc2(const uint16_t *h, int32_t T, int32_t k, const qmoe_fp8_weights *w2,
                              const int32_t *expert_offsets, float *y_rows, void *ws, size_t *ws_bytes,
                              qmoe_path path, hipStream_t stream) {
  FcShape sh;
  qmoe_path p;
  qmoe_status st = check_fp8_fc(w2, T, k, h, expert_offsets, y_rows, path, &sh, &p);
  if (st != QMOE_OK) return st;
  GemvArgs a = {};
  a.act = h;
  a.offsets = expert_offsets;
  a.topk = k;
  a.rows = sh.rows;
  a.fc1 = 0;
  a.out_f32 = y_rows;
  return run_fp8(a, w2, sh.max_rows_per_expert, p, ws, ws_bytes, stream);
}

qmoe_status qmoe_dequant_fp8(const qmoe_fp8_weights *w, uint16_t *out, hipStream_t stream) {
  if (!w || !w->w || !w->gscale || !out) return QMOE_EINVAL;
  if (w->E < 1 || w->K < 1 || w->N < 1) return QMOE_EINVAL;
  if (!aligned16(w->w) || !aligned16(w->gscale) || !aligned16(out)) return QMOE_EALIGN;
  if (((int64_t)w->K * w->N) % 16 != 0 || w->E > 65535) return QMOE_EUNSUPPORTED;
  return check_launch(launch_fp8_dequant(w->w, w->gscale, w->E, w->K, w->N, out, stream));
}

}  // extern "C"
