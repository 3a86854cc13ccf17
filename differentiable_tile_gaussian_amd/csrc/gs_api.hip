// The C ABI declared in include/gs.h: argument checks, workspace carving and the
// launches of the kernels in the other translation units.  No call allocates.
#include <algorithm>
#include <atomic>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "adam_math.h"
#include "gs_internal.h"
#include "profile.h"

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int32_t hip_fail(hipError_t e, const char* where) {
  return fail(GS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// The most (tile, Gaussian) pairs a call accepts: 2^32 - 2^25.  Kernels keep pair indices
// in 32 bits and add to an index below the count at most a split size (<= 2^24) or a
// block's items, which this margin keeps below 2^32.
constexpr uint64_t kMaxPairs = (uint64_t(1) << 32) - (uint64_t(1) << 25);

int32_t check_pairs(uint32_t total_pairs) {
  if (total_pairs > kMaxPairs)
    return fail(GS_ERR_CAPACITY, "pair count %u exceeds 2^32 - 2^25", total_pairs);
  return GS_OK;
}

inline hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

constexpr int32_t kDefaultSplitFirst = 2048;
constexpr int32_t kDefaultSplitChunk = 512;

bool split_ok(int32_t v) { return v == 0 || (v >= 4 && v <= (1 << 24) && (v & 3) == 0); }

// The call's settings with the defaults filled in (NULL: every default), or an error.
int32_t resolve_config(const gs_config* in, gs_config* out) {
  gs_config c = GS_CONFIG_DEFAULT;
  if (in) c = *in;
  if (c.grad_sums != GS_GRAD_SUMS_FLOAT && c.grad_sums != GS_GRAD_SUMS_FIXED)
    return fail(GS_ERR_INVALID_ARG, "cfg.grad_sums must be GS_GRAD_SUMS_FLOAT or GS_GRAD_SUMS_FIXED");
  if (c.active_sh_degree < -1 || c.active_sh_degree > 3)
    return fail(GS_ERR_INVALID_ARG, "cfg.active_sh_degree must be -1..3");
  if (c.mip_compensation != 0 && c.mip_compensation != 1)
    return fail(GS_ERR_INVALID_ARG, "cfg.mip_compensation must be 0 or 1");
  if (!split_ok(c.split_first) || !split_ok(c.split_chunk))
    return fail(GS_ERR_INVALID_ARG, "cfg.split_first and cfg.split_chunk must be 0 or multiples of 4 in [4, 2^24]");
  if (c.split_first == 0) c.split_first = kDefaultSplitFirst;
  if (c.split_chunk == 0) c.split_chunk = kDefaultSplitChunk;
  *out = c;
  return GS_OK;
}

// How the kernels shade a scene of a stored degree: the active higher bands,
// (d + 1)^2 - 1 with d the smaller of the stored and the active degree, and the
// compensation switch.
gsk::Shade shade_of(int deg, const gs_config& c) {
  const int a = c.active_sh_degree;
  const int d = (a < 0 || a > deg) ? deg : a;
  return gsk::Shade{(d + 1) * (d + 1) - 1, c.mip_compensation};
}

// The backward blend with the call's settings.
hipError_t launch_bwd_blend(const gs_proj& proj, int n, const uint32_t* vals, const uint32_t* ranges,
                            const gs_camera& cam, uint32_t pairs, const float* T_final, const uint32_t* n_contrib,
                            const float* dL_dimg, float* gscreen, void* ws, size_t ws_bytes, const gs_config& c,
                            hipStream_t s) {
  return gsk::launch_render_bwd(proj, n, vals, ranges, cam, pairs, T_final, n_contrib, dL_dimg, gscreen, ws,
                                ws_bytes, c.split_first, c.split_chunk, c.grad_sums == GS_GRAD_SUMS_FIXED, s);
}

// Render workspace bytes for the resolved settings.
size_t render_ws(int64_t n, uint32_t pairs, int W, int H, const gs_config& c) {
  return gsk::render_ws_bytes(W, H, pairs, c.split_first, c.split_chunk,
                              c.grad_sums == GS_GRAD_SUMS_FIXED ? (n > 0 ? n : 0) : 0);
}

int32_t check_camera(const gs_camera* cam) {
  if (!cam) return fail(GS_ERR_INVALID_ARG, "camera is null");
  if (cam->width <= 0 || cam->height <= 0) return fail(GS_ERR_INVALID_ARG, "image size must be positive");
  if (gsk::tiles_x(*cam) > 65535 || gsk::tiles_y(*cam) > 65535)
    return fail(GS_ERR_UNSUPPORTED, "more than 65535 tiles along one image axis");
  if (int64_t(gsk::tiles_x(*cam)) * gsk::tiles_y(*cam) > (int64_t(1) << 30))
    return fail(GS_ERR_UNSUPPORTED, "too many tiles");
  if (!(cam->fx > 0.0f) || !(cam->fy > 0.0f)) return fail(GS_ERR_INVALID_ARG, "focal lengths must be positive");
  if (!(cam->znear > 0.0f)) return fail(GS_ERR_INVALID_ARG, "znear must be positive");
  return GS_OK;
}

int32_t check_scene(const gs_scene* sc) {
  if (!sc) return fail(GS_ERR_INVALID_ARG, "scene is null");
  if (sc->n < 0 || sc->n >= (int64_t(1) << 31)) return fail(GS_ERR_INVALID_ARG, "n out of range");
  if (sc->sh_degree < 0 || sc->sh_degree > 3) return fail(GS_ERR_UNSUPPORTED, "SH degree must be 0..3");
  if (sc->n > 0 && !sc->params) return fail(GS_ERR_INVALID_ARG, "params is null");
  if (gsk::param_floats(sc->n, gsk::num_planes(sc->sh_degree)) >= (size_t(1) << 31))
    return fail(GS_ERR_UNSUPPORTED, "gs_param_floats(n, sh_degree) must stay below 2^31");
  return GS_OK;
}

int32_t check_proj(const gs_proj* p, int64_t n, bool need_order) {
  if (!p) return fail(GS_ERR_INVALID_ARG, "proj is null");
  if (need_order && (!p->offs || !p->n_visible || (n > 0 && (!p->order || !p->rect_order))))
    return fail(GS_ERR_INVALID_ARG, "proj.offs, proj.order, proj.rect_order or proj.n_visible is null");
  if (n > 0 && (!p->splat || !p->depth || !p->rect || !p->tiles))
    return fail(GS_ERR_INVALID_ARG, "a proj array is null");
  return GS_OK;
}

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// Preprocess workspace: pair count, per-block tile sums (one per 64 Gaussians: the
// projection kernel uses one per 256, the chain with projection one per 64),
// depth-order state.
struct PreWs {
  uint64_t* total64;
  uint32_t* block_tiles;
  void* depth_ws;
};

size_t block_sum_bytes(int64_t n) { return align256(size_t(gsk::div_up(n > 0 ? n : 1, 64)) * 4); }

size_t pre_ws_bytes(int64_t n) { return 256 + block_sum_bytes(n) + gsk::depth_order_ws_bytes(n); }

PreWs carve_pre(void* ws, int64_t n) {
  char* p = static_cast<char*>(ws);
  PreWs w;
  w.total64 = reinterpret_cast<uint64_t*>(p);
  w.block_tiles = reinterpret_cast<uint32_t*>(p + 256);
  w.depth_ws = p + 256 + block_sum_bytes(n);
  return w;
}

// The part of gs_preprocess after the projection kernels: the pair count to the host
// while the depth order is computed.
int32_t finish_preprocess(gs_proj* out, int n, float znear, const PreWs& w, uint32_t* total_pairs, hipStream_t s);

// Pinned host word the pair count is copied into, and the event that marks the copy,
// one per device and host thread, created on first use and kept for the process.
struct HostSlot {
  uint64_t* pinned = nullptr;
  hipEvent_t copied = nullptr;
};

HostSlot* host_slot() {
  thread_local HostSlot slots[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  HostSlot& h = slots[dev];
  if (!h.pinned) {
    void* p = nullptr;
    if (hipHostMalloc(&p, 4 * sizeof(uint64_t), hipHostMallocDefault) != hipSuccess) return nullptr;
    if (hipEventCreateWithFlags(&h.copied, hipEventDisableTiming) != hipSuccess) {
      (void)hipHostFree(p);
      return nullptr;
    }
    h.pinned = static_cast<uint64_t*>(p);
  }
  return &h;
}

}  // namespace

extern "C" {

const char* gs_last_error(void) { return g_err; }

int32_t gs_profile_enable(int32_t on, const char* only) {
  g_err[0] = 0;
  const hipError_t e = gsk::profile_enable(on != 0, only);
  if (e != hipSuccess) return hip_fail(e, "gs_profile_enable");
  return GS_OK;
}

int32_t gs_profile_query(int32_t max_names, char* names, int64_t* launches, double* total_ms) {
  g_err[0] = 0;
  if (max_names < 0) return fail(GS_ERR_INVALID_ARG, "max_names must be >= 0");
  if (max_names > 0 && (!names || !launches || !total_ms)) return fail(GS_ERR_INVALID_ARG, "null output buffer");
  int32_t written = 0;
  const hipError_t e = gsk::profile_query(max_names, names, launches, total_ms, &written);
  if (e != hipSuccess) return hip_fail(e, "gs_profile_query");
  return written;
}

size_t gs_workspace_bytes(int32_t which_call, int64_t n, uint32_t pairs, int32_t W, int32_t H, const gs_config* cfg) {
  gs_config c;
  if (resolve_config(cfg, &c) != GS_OK) return 0;
  switch (which_call) {
    case GS_WS_PREPROCESS: return pre_ws_bytes(n < 0 ? 0 : n);
    case GS_WS_BIN_SORT: return gsk::bin_sort_ws_bytes(pairs);
    case GS_WS_LOSS: return (W > 0 && H > 0) ? gsk::loss_ws_bytes(H, W) : 0;
    case GS_WS_RENDER: return (W > 0 && H > 0) ? render_ws(n, pairs, W, H, c) : 0;
    case GS_WS_DENSIFY: return gsk::densify_ws_bytes(n < 0 ? 0 : n);
    case GS_WS_LOSS_CHARBONNIER: return (W > 0 && H > 0) ? gsk::charbonnier_ws_bytes(H, W) : 0;
    case GS_WS_CAMERA_GRAD: return gsk::camera_grad_ws_bytes(n < 0 ? 0 : n);
    case GS_WS_RELOCATE: return gsk::relocate_ws_bytes(n < 0 ? 0 : n);
    default: return 0;
  }
}

int32_t gs_preprocess(const gs_scene* scene, const gs_camera* cam, gs_proj* out, uint32_t* total_pairs, void* ws,
                      size_t ws_bytes, const gs_config* cfg, void* stream) {
  g_err[0] = 0;
  int32_t st;
  gs_config c;
  if ((st = resolve_config(cfg, &c)) != GS_OK) return st;
  if ((st = check_scene(scene)) != GS_OK) return st;
  if ((st = check_camera(cam)) != GS_OK) return st;
  if ((st = check_proj(out, scene->n, true)) != GS_OK) return st;
  if (!total_pairs) return fail(GS_ERR_INVALID_ARG, "total_pairs is null");
  const size_t need = pre_ws_bytes(scene->n);
  if (!ws || ws_bytes < need) return fail(GS_ERR_CAPACITY, "preprocess workspace needs %zu bytes", need);
  hipStream_t s = as_stream(stream);
  const int n = int(scene->n);
  PreWs w = carve_pre(ws, n);
  hipError_t e = gsk::launch_preprocess_fwd(scene->params, n, scene->sh_degree, *cam, *out, w.block_tiles,
                                            w.total64, shade_of(scene->sh_degree, c), s);
  if (e != hipSuccess) return hip_fail(e, "preprocess_fwd");
  return finish_preprocess(out, n, cam->znear, w, total_pairs, s);
}

}  // extern "C"

namespace {

int32_t finish_preprocess(gs_proj* out, int n, float znear, const PreWs& w, uint32_t* total_pairs, hipStream_t s) {
  hipError_t e;
  // the pair count goes to the host while the depth order is computed
  HostSlot* hs = host_slot();
  if (!hs) return fail(GS_ERR_HIP, "cannot set up the pinned pair-count buffer");
  if (n > 0) {
    e = hipMemcpyAsync(hs->pinned, w.total64, sizeof(uint64_t), hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return hip_fail(e, "pair count copy");
  } else {
    *hs->pinned = 0;
  }
  e = hipEventRecord(hs->copied, s);
  if (e != hipSuccess) return hip_fail(e, "pair count event");
  e = gsk::launch_depth_order(*out, n, znear, w.depth_ws, s);
  if (e != hipSuccess) return hip_fail(e, "depth order");
  e = hipEventSynchronize(hs->copied);
  if (e != hipSuccess) return hip_fail(e, "preprocess sync");
  const uint64_t host_total = *hs->pinned;
  if (host_total > kMaxPairs)
    return fail(GS_ERR_CAPACITY, "pair count %llu exceeds 2^32 - 2^25", (unsigned long long)host_total);
  *total_pairs = uint32_t(host_total);
  return GS_OK;
}

}  // namespace

extern "C" {

int32_t gs_bin_sort(const gs_proj* proj, int64_t n, const gs_camera* cam, uint32_t total_pairs, uint32_t* keys,
                    uint32_t* vals, uint32_t capacity, uint32_t* ranges, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  int32_t st;
  if (n < 0 || n >= (int64_t(1) << 31)) return fail(GS_ERR_INVALID_ARG, "n out of range");
  if ((st = check_camera(cam)) != GS_OK) return st;
  if ((st = check_proj(proj, n, true)) != GS_OK) return st;
  if (!ranges) return fail(GS_ERR_INVALID_ARG, "ranges is null");
  if (total_pairs > 0 && (!keys || !vals)) return fail(GS_ERR_INVALID_ARG, "keys or vals is null");
  if (total_pairs > 0 && n == 0) return fail(GS_ERR_INVALID_ARG, "pairs without Gaussians");
  if ((st = check_pairs(total_pairs)) != GS_OK) return st;
  if (capacity < total_pairs)
    return fail(GS_ERR_CAPACITY, "key capacity %u < %u pairs", capacity, total_pairs);
  const size_t need = gsk::bin_sort_ws_bytes(total_pairs);
  if (total_pairs > 0 && (!ws || ws_bytes < need))
    return fail(GS_ERR_CAPACITY, "bin_sort workspace needs %zu bytes", need);
  hipError_t e = gsk::launch_bin_sort(*proj, int(n), *cam, total_pairs, keys, vals, ranges, ws, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "bin_sort");
  return GS_OK;
}

int32_t gs_render_fwd(const gs_proj* proj, int64_t n, const uint32_t* vals, const uint32_t* ranges,
                      uint32_t total_pairs, const gs_camera* cam, float* rgb, float* T_final,
                      uint32_t* n_contrib, void* ws, size_t ws_bytes, const gs_config* cfg, void* stream) {
  g_err[0] = 0;
  int32_t st;
  gs_config c;
  if ((st = resolve_config(cfg, &c)) != GS_OK) return st;
  if (n < 0 || n >= (int64_t(1) << 31)) return fail(GS_ERR_INVALID_ARG, "n out of range");
  if ((st = check_camera(cam)) != GS_OK) return st;
  if ((st = check_proj(proj, n, false)) != GS_OK) return st;
  if (!ranges || !rgb || !T_final || !n_contrib) return fail(GS_ERR_INVALID_ARG, "an output or ranges is null");
  if (total_pairs > 0 && !vals) return fail(GS_ERR_INVALID_ARG, "vals is null");
  if ((st = check_pairs(total_pairs)) != GS_OK) return st;
  const size_t need = gsk::render_ws_bytes(cam->width, cam->height, total_pairs, c.split_first, c.split_chunk, 0);
  if (!ws || ws_bytes < need) return fail(GS_ERR_CAPACITY, "render workspace needs %zu bytes", need);
  hipError_t e = gsk::launch_render_fwd(*proj, vals, ranges, *cam, total_pairs, rgb, T_final, n_contrib, ws,
                                        c.split_first, c.split_chunk, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "render_fwd");
  return GS_OK;
}

int32_t gs_loss_l1_dssim(const float* img, const float* target, int32_t H, int32_t W, float lambda_dssim,
                         float* loss_out, float* dL_dimg, void* ws, size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (!img || !target || !loss_out || !dL_dimg) return fail(GS_ERR_INVALID_ARG, "a loss argument is null");
  if (H <= 0 || W <= 0) return fail(GS_ERR_INVALID_ARG, "image size must be positive");
  if (int64_t(3) * H * W >= (int64_t(1) << 31)) return fail(GS_ERR_UNSUPPORTED, "image too large");
  if (!(lambda_dssim >= 0.0f && lambda_dssim <= 1.0f)) return fail(GS_ERR_INVALID_ARG, "lambda must be in [0, 1]");
  const size_t need = gsk::loss_ws_bytes(H, W);
  if (!ws || ws_bytes < need) return fail(GS_ERR_CAPACITY, "loss workspace needs %zu bytes", need);
  hipError_t e = gsk::launch_loss(img, target, H, W, lambda_dssim, loss_out, dL_dimg, ws, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "loss");
  return GS_OK;
}

int32_t gs_loss_l1_dssim_noalloc(const float* img, const float* target, int32_t H, int32_t W, float lambda_dssim,
                                 float* loss_out, float* dL_dimg, void* stream) {
  g_err[0] = 0;
  if (!img || !target || !loss_out || !dL_dimg) return fail(GS_ERR_INVALID_ARG, "a loss argument is null");
  if (H <= 0 || W <= 0) return fail(GS_ERR_INVALID_ARG, "image size must be positive");
  if (int64_t(3) * H * W >= (int64_t(1) << 31)) return fail(GS_ERR_UNSUPPORTED, "image too large");
  if (!(lambda_dssim >= 0.0f && lambda_dssim <= 1.0f)) return fail(GS_ERR_INVALID_ARG, "lambda must be in [0, 1]");
  const size_t need = gsk::loss_ws_bytes(H, W);
  if (need > gsk::loss_scratch_bytes())
    return fail(GS_ERR_CAPACITY, "a %d x %d image needs %zu bytes of loss scratch; the no-allocation loss has %zu",
                W, H, need, gsk::loss_scratch_bytes());
  void* scratch = nullptr;
  hipError_t e = gsk::loss_scratch(&scratch);
  if (e != hipSuccess) return hip_fail(e, "loss scratch address");
  e = gsk::launch_loss(img, target, H, W, lambda_dssim, loss_out, dL_dimg, scratch, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "loss");
  return GS_OK;
}

static int32_t render_bwd_common(const gs_scene* scene, const gs_proj* proj, const uint32_t* vals,
                                 const uint32_t* ranges, uint32_t total_pairs, const gs_camera* cam,
                                 const float* T_final, const uint32_t* n_contrib, const float* dL_dimg,
                                 float* gscreen, float* gparams, float weight, int accumulate, void* ws,
                                 size_t ws_bytes, const gs_config* cfg, void* stream) {
  int32_t st;
  gs_config c;
  if ((st = resolve_config(cfg, &c)) != GS_OK) return st;
  if ((st = check_scene(scene)) != GS_OK) return st;
  if ((st = check_camera(cam)) != GS_OK) return st;
  if ((st = check_proj(proj, scene->n, false)) != GS_OK) return st;
  if (!ranges || !T_final || !n_contrib || !dL_dimg) return fail(GS_ERR_INVALID_ARG, "a render input is null");
  if (scene->n > 0 && (!gscreen || !gparams)) return fail(GS_ERR_INVALID_ARG, "gscreen or gparams is null");
  if (total_pairs > 0 && !vals) return fail(GS_ERR_INVALID_ARG, "vals is null");
  if ((st = check_pairs(total_pairs)) != GS_OK) return st;
  const size_t need = render_ws(scene->n, total_pairs, cam->width, cam->height, c);
  if (!ws || ws_bytes < need) return fail(GS_ERR_CAPACITY, "render workspace needs %zu bytes", need);
  hipStream_t s = as_stream(stream);
  const int n = int(scene->n);
  hipError_t e = launch_bwd_blend(*proj, n, vals, ranges, *cam, total_pairs, T_final, n_contrib, dL_dimg, gscreen,
                                  ws, ws_bytes, c, s);
  if (e != hipSuccess) return hip_fail(e, "render_bwd");
  e = gsk::launch_preprocess_bwd(scene->params, n, scene->sh_degree, *cam, proj->tiles, gscreen, gparams,
                                 shade_of(scene->sh_degree, c), s, weight, accumulate);
  if (e != hipSuccess) return hip_fail(e, "preprocess_bwd");
  return GS_OK;
}

int32_t gs_render_bwd(const gs_scene* scene, const gs_proj* proj, const uint32_t* vals, const uint32_t* ranges,
                      uint32_t total_pairs, const gs_camera* cam, const float* T_final,
                      const uint32_t* n_contrib, const float* dL_dimg, float* gscreen, float* gparams, void* ws,
                      size_t ws_bytes, const gs_config* cfg, void* stream) {
  g_err[0] = 0;
  return render_bwd_common(scene, proj, vals, ranges, total_pairs, cam, T_final, n_contrib, dL_dimg, gscreen, gparams,
                           1.0f, 0, ws, ws_bytes, cfg, stream);
}

int32_t gs_render_bwd_weighted(const gs_scene* scene, const gs_proj* proj, const uint32_t* vals,
                               const uint32_t* ranges, uint32_t total_pairs, const gs_camera* cam,
                               const float* T_final, const uint32_t* n_contrib, const float* dL_dimg,
                               float* gscreen, float* gparams, float weight, int32_t accumulate, void* ws,
                               size_t ws_bytes, const gs_config* cfg, void* stream) {
  g_err[0] = 0;
  if (!std::isfinite(weight)) return fail(GS_ERR_INVALID_ARG, "weight must be finite");
  if (accumulate != 0 && accumulate != 1) return fail(GS_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  return render_bwd_common(scene, proj, vals, ranges, total_pairs, cam, T_final, n_contrib, dL_dimg, gscreen, gparams,
                           weight, accumulate, ws, ws_bytes, cfg, stream);
}

int32_t gs_camera_grad(const gs_scene* scene, const gs_proj* proj, const gs_camera* cam, const float* gscreen,
                       int32_t position_only, double* grad_out, void* ws, size_t ws_bytes, const gs_config* cfg,
                       void* stream) {
  g_err[0] = 0;
  int32_t st;
  gs_config c;
  if ((st = resolve_config(cfg, &c)) != GS_OK) return st;
  if ((st = check_scene(scene)) != GS_OK) return st;
  if ((st = check_camera(cam)) != GS_OK) return st;
  if ((st = check_proj(proj, scene->n, false)) != GS_OK) return st;
  if (!grad_out) return fail(GS_ERR_INVALID_ARG, "grad_out is null");
  if (position_only != 0 && position_only != 1) return fail(GS_ERR_INVALID_ARG, "position_only must be 0 or 1");
  if (scene->n > 0 && !gscreen) return fail(GS_ERR_INVALID_ARG, "gscreen is null");
  const size_t need = gsk::camera_grad_ws_bytes(scene->n);
  if (scene->n > 0 && (!ws || ws_bytes < need))
    return fail(GS_ERR_CAPACITY, "camera-gradient workspace needs %zu bytes", need);
  const hipError_t e = gsk::launch_camera_grad(scene->params, int(scene->n), scene->sh_degree, *cam, proj->tiles,
                                               gscreen, position_only, grad_out, ws, shade_of(scene->sh_degree, c),
                                               as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "camera_grad");
  return GS_OK;
}

static int32_t check_adam(int64_t n, int32_t sh_degree, const float* lr, double beta1, double beta2, double eps,
                          int32_t step) {
  if (n < 0 || n >= (int64_t(1) << 31)) return fail(GS_ERR_INVALID_ARG, "n out of range");
  if (sh_degree < 0 || sh_degree > 3) return fail(GS_ERR_UNSUPPORTED, "SH degree must be 0..3");
  if (!lr) return fail(GS_ERR_INVALID_ARG, "lr is null");
  if (gsk::param_floats(n, gsk::num_planes(sh_degree)) >= (size_t(1) << 31))
    return fail(GS_ERR_UNSUPPORTED, "gs_param_floats(n, sh_degree) must stay below 2^31");
  if (step < 1) return fail(GS_ERR_INVALID_ARG, "step must be >= 1");
  if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0) || !(eps >= 0.0))
    return fail(GS_ERR_INVALID_ARG, "bad Adam hyper-parameters");
  return GS_OK;
}

static gsk::AdamArgs adam_args(const float* lr, double beta1, double beta2, double eps, int32_t step) {
  gsk::AdamArgs a;
  for (int k = 0; k < 5; ++k) a.lr[k] = lr[k];
  a.b1 = float(beta1);
  a.b2 = float(beta2);
  a.omb1 = float(1.0 - beta1);
  a.omb2 = float(1.0 - beta2);
  a.eps = float(eps);
  a.inv_bc1 = float(1.0 / (1.0 - pow(beta1, double(step))));
  a.inv_bc2 = float(1.0 / (1.0 - pow(beta2, double(step))));
  return a;
}

int32_t gs_render_bwd_adam(float* params, int64_t n, int32_t sh_degree, const gs_proj* proj, const uint32_t* vals,
                           const uint32_t* ranges, uint32_t total_pairs, const gs_camera* cam,
                           const float* T_final, const uint32_t* n_contrib, const float* dL_dimg, float* gscreen,
                           float* m, float* v, const float* lr, double beta1, double beta2, double eps,
                           int32_t step, void* ws, size_t ws_bytes, const gs_config* cfg, void* stream) {
  g_err[0] = 0;
  int32_t st;
  gs_config c;
  if ((st = resolve_config(cfg, &c)) != GS_OK) return st;
  const gs_scene scene{n, sh_degree, params};
  if ((st = check_scene(&scene)) != GS_OK) return st;
  if ((st = check_adam(n, sh_degree, lr, beta1, beta2, eps, step)) != GS_OK) return st;
  if ((st = check_camera(cam)) != GS_OK) return st;
  if ((st = check_proj(proj, n, false)) != GS_OK) return st;
  if (!ranges || !T_final || !n_contrib || !dL_dimg) return fail(GS_ERR_INVALID_ARG, "a render input is null");
  if (n > 0 && (!gscreen || !m || !v)) return fail(GS_ERR_INVALID_ARG, "gscreen, m or v is null");
  if (total_pairs > 0 && !vals) return fail(GS_ERR_INVALID_ARG, "vals is null");
  if ((st = check_pairs(total_pairs)) != GS_OK) return st;
  const size_t need = render_ws(n, total_pairs, cam->width, cam->height, c);
  if (!ws || ws_bytes < need) return fail(GS_ERR_CAPACITY, "render workspace needs %zu bytes", need);
  hipStream_t s = as_stream(stream);
  hipError_t e = launch_bwd_blend(*proj, int(n), vals, ranges, *cam, total_pairs, T_final, n_contrib, dL_dimg,
                                  gscreen, ws, ws_bytes, c, s);
  if (e != hipSuccess) return hip_fail(e, "render_bwd");
  e = gsk::launch_chain_adam(params, int(n), sh_degree, *cam, proj->tiles, gscreen, m, v,
                             adam_args(lr, beta1, beta2, eps, step), shade_of(sh_degree, c), s);
  if (e != hipSuccess) return hip_fail(e, "chain_adam");
  return GS_OK;
}

int32_t gs_render_bwd_adam_project(float* params, int64_t n, int32_t sh_degree, const gs_proj* proj,
                                   const uint32_t* vals, const uint32_t* ranges, uint32_t total_pairs,
                                   const gs_camera* cam, const float* T_final, const uint32_t* n_contrib,
                                   const float* dL_dimg, float* gscreen, float* m, float* v, const float* lr,
                                   double beta1, double beta2, double eps, int32_t step, void* ws, size_t ws_bytes,
                                   const gs_camera* next_cam, gs_proj* next_out, uint32_t* next_total_pairs,
                                   void* pre_ws, size_t pre_ws_bytes_, float* densify_stats, const gs_config* cfg,
                                   void* stream) {
  g_err[0] = 0;
  int32_t st;
  gs_config c;
  if ((st = resolve_config(cfg, &c)) != GS_OK) return st;
  const gs_scene scene{n, sh_degree, params};
  if ((st = check_scene(&scene)) != GS_OK) return st;
  if ((st = check_adam(n, sh_degree, lr, beta1, beta2, eps, step)) != GS_OK) return st;
  if ((st = check_camera(cam)) != GS_OK) return st;
  if ((st = check_camera(next_cam)) != GS_OK) return st;
  if ((st = check_proj(proj, n, false)) != GS_OK) return st;
  if ((st = check_proj(next_out, n, true)) != GS_OK) return st;
  if (!next_total_pairs) return fail(GS_ERR_INVALID_ARG, "next_total_pairs is null");
  if (!ranges || !T_final || !n_contrib || !dL_dimg) return fail(GS_ERR_INVALID_ARG, "a render input is null");
  if (n > 0 && (!gscreen || !m || !v)) return fail(GS_ERR_INVALID_ARG, "gscreen, m or v is null");
  if (total_pairs > 0 && !vals) return fail(GS_ERR_INVALID_ARG, "vals is null");
  if ((st = check_pairs(total_pairs)) != GS_OK) return st;
  const size_t need = render_ws(n, total_pairs, cam->width, cam->height, c);
  if (!ws || ws_bytes < need) return fail(GS_ERR_CAPACITY, "render workspace needs %zu bytes", need);
  const size_t need_pre = pre_ws_bytes(n);
  if (!pre_ws || pre_ws_bytes_ < need_pre)
    return fail(GS_ERR_CAPACITY, "preprocess workspace needs %zu bytes", need_pre);
  hipStream_t s = as_stream(stream);
  hipError_t e = launch_bwd_blend(*proj, int(n), vals, ranges, *cam, total_pairs, T_final, n_contrib, dL_dimg,
                                  gscreen, ws, ws_bytes, c, s);
  if (e != hipSuccess) return hip_fail(e, "render_bwd");
  PreWs w = carve_pre(pre_ws, n);
  gsk::NextProj np;
  np.cam = *next_cam;
  np.tx = gsk::tiles_x(*next_cam);
  np.ty = gsk::tiles_y(*next_cam);
  np.splat = reinterpret_cast<float4*>(next_out->splat);
  np.depth = next_out->depth;
  np.rect = reinterpret_cast<uint2*>(next_out->rect);
  np.tiles = next_out->tiles;
  np.block_tiles = w.block_tiles;
  np.total = w.total64;
  e = gsk::launch_chain_adam_project(params, int(n), sh_degree, *cam, proj->tiles, gscreen, m, v,
                                     adam_args(lr, beta1, beta2, eps, step), np, densify_stats,
                                     shade_of(sh_degree, c), s);
  if (e != hipSuccess) return hip_fail(e, "chain_adam_project");
  return finish_preprocess(next_out, int(n), next_cam->znear, w, next_total_pairs, s);
}

int32_t gs_adam_step(float* params, const float* grads, float* m, float* v, int64_t n, int32_t sh_degree,
                     const float* lr, double beta1, double beta2, double eps, int32_t step, void* stream) {
  g_err[0] = 0;
  if (n < 0 || n >= (int64_t(1) << 31)) return fail(GS_ERR_INVALID_ARG, "n out of range");
  if (sh_degree < 0 || sh_degree > 3) return fail(GS_ERR_UNSUPPORTED, "SH degree must be 0..3");
  if (!lr) return fail(GS_ERR_INVALID_ARG, "lr is null");
  if (n > 0 && (!params || !grads || !m || !v)) return fail(GS_ERR_INVALID_ARG, "an Adam array is null");
  if (gsk::param_floats(n, gsk::num_planes(sh_degree)) >= (size_t(1) << 31))
    return fail(GS_ERR_UNSUPPORTED, "gs_param_floats(n, sh_degree) must stay below 2^31");
  if (step < 1) return fail(GS_ERR_INVALID_ARG, "step must be >= 1");
  if (!(beta1 >= 0.0 && beta1 < 1.0) || !(beta2 >= 0.0 && beta2 < 1.0) || !(eps >= 0.0))
    return fail(GS_ERR_INVALID_ARG, "bad Adam hyper-parameters");
  // bias corrections in fp64 on the host
  const double bc1 = 1.0 - pow(beta1, double(step));
  const double bc2 = 1.0 - pow(beta2, double(step));
  hipError_t e = gsk::launch_adam(params, grads, m, v, int(n), sh_degree, lr, float(beta1), float(beta2),
                                  float(1.0 - beta1), float(1.0 - beta2), float(eps), float(1.0 / bc1),
                                  float(1.0 / bc2), as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "adam");
  return GS_OK;
}

size_t gs_param_floats(int64_t n, int32_t sh_degree) {
  if (n < 0 || sh_degree < 0 || sh_degree > 3) return 0;
  return gsk::param_floats(n, gsk::num_planes(sh_degree));
}

static int32_t check_layout(const float* a, const float* b, int64_t n, int32_t sh_degree) {
  if (n < 0 || n >= (int64_t(1) << 31)) return fail(GS_ERR_INVALID_ARG, "n out of range");
  if (sh_degree < 0 || sh_degree > 3) return fail(GS_ERR_UNSUPPORTED, "SH degree must be 0..3");
  if (n > 0 && (!a || !b)) return fail(GS_ERR_INVALID_ARG, "a layout array is null");
  if (gsk::param_floats(n, gsk::num_planes(sh_degree)) >= (size_t(1) << 31))
    return fail(GS_ERR_UNSUPPORTED, "gs_param_floats(n, sh_degree) must stay below 2^31");
  return GS_OK;
}

int32_t gs_params_to_blocked(const float* planar, float* blocked, int64_t n, int32_t sh_degree, void* stream) {
  g_err[0] = 0;
  int32_t st;
  if ((st = check_layout(planar, blocked, n, sh_degree)) != GS_OK) return st;
  hipError_t e = gsk::launch_to_blocked(planar, blocked, int(n), gsk::num_planes(sh_degree), as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "to_blocked");
  return GS_OK;
}

int32_t gs_params_from_blocked(const float* blocked, float* planar, int64_t n, int32_t sh_degree, void* stream) {
  g_err[0] = 0;
  int32_t st;
  if ((st = check_layout(blocked, planar, n, sh_degree)) != GS_OK) return st;
  hipError_t e = gsk::launch_from_blocked(blocked, planar, int(n), gsk::num_planes(sh_degree), as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "from_blocked");
  return GS_OK;
}

int32_t gs_densify_accumulate(const gs_proj* proj, int64_t n, const float* gscreen, float* stats, void* stream) {
  g_err[0] = 0;
  if (n < 0 || n >= (int64_t(1) << 31)) return fail(GS_ERR_INVALID_ARG, "n out of range");
  if (n == 0) return GS_OK;
  if (!proj || !proj->tiles) return fail(GS_ERR_INVALID_ARG, "proj or proj.tiles is null");
  if (!gscreen || !stats) return fail(GS_ERR_INVALID_ARG, "gscreen or stats is null");
  const hipError_t e = gsk::launch_densify_accumulate(proj->tiles, int(n), gscreen, stats, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "densify_accumulate");
  return GS_OK;
}

int32_t gs_densify(const float* params, const float* m, const float* v, const float* stats, const float* rand,
                   int64_t n, int32_t sh_degree, double grad_threshold, double prune_opacity, double prune_scale,
                   double split_scale, int32_t reset_opacity, double opacity_cap, float* params_out, float* m_out,
                   float* v_out, float* stats_out, int64_t capacity, int64_t* n_out, int64_t* counts, void* ws,
                   size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (n < 0 || n >= (int64_t(1) << 31)) return fail(GS_ERR_INVALID_ARG, "n out of range");
  if (sh_degree < 0 || sh_degree > 3) return fail(GS_ERR_UNSUPPORTED, "SH degree must be 0..3");
  if (!n_out) return fail(GS_ERR_INVALID_ARG, "n_out is null");
  if (n > 0 && (!params || !m || !v || !stats || !rand)) return fail(GS_ERR_INVALID_ARG, "an input is null");
  if (!(grad_threshold >= 0.0) || !(prune_opacity >= 0.0 && prune_opacity < 1.0) || !(prune_scale > 0.0) ||
      !(split_scale > 0.0) || !std::isfinite(split_scale) ||
      (reset_opacity && !(opacity_cap > 0.0 && opacity_cap < 1.0)))
    return fail(GS_ERR_INVALID_ARG, "bad density-control thresholds");
  const bool write = params_out != nullptr;
  if (write) {
    if (!m_out || !v_out || !stats_out) return fail(GS_ERR_INVALID_ARG, "an output is null");
    if (capacity < 0 || gsk::param_floats(capacity, gsk::num_planes(sh_degree)) >= (size_t(1) << 31))
      return fail(GS_ERR_INVALID_ARG, "capacity out of range");
    const void* ins[5] = {params, m, v, stats, rand};
    const void* outs[4] = {params_out, m_out, v_out, stats_out};
    for (const void* o : outs)
      for (const void* x : ins)
        if (o == x) return fail(GS_ERR_INVALID_ARG, "an output is one of the inputs");
  }
  const size_t need = gsk::densify_ws_bytes(n);
  if (!ws || ws_bytes < need) return fail(GS_ERR_CAPACITY, "densify workspace needs %zu bytes", need);
  gsk::DensifyArgs a;
  a.grad_thr = float(grad_threshold);
  a.logit_prune = float(std::log(prune_opacity / (1.0 - prune_opacity)));
  a.lscale_prune = std::isinf(prune_scale) ? __builtin_inff() : float(std::log(prune_scale));
  a.lscale_split = float(std::log(split_scale));
  a.lscale_shrink = float(std::log(1.6));
  a.logit_cap = reset_opacity ? float(std::log(opacity_cap / (1.0 - opacity_cap))) : 0.0f;
  a.reset = reset_opacity ? 1 : 0;
  hipStream_t s = as_stream(stream);
  uint64_t tot[3] = {0, 0, 0};
  if (n > 0) {
    hipError_t e = gsk::launch_densify_count(params, int(n), sh_degree, stats, a, ws, s);
    if (e != hipSuccess) return hip_fail(e, "densify_count");
    HostSlot* hs = host_slot();
    if (!hs) return fail(GS_ERR_HIP, "cannot set up the pinned count buffer");
    e = hipMemcpyAsync(hs->pinned, gsk::carve_densify(ws, n).totals, 3 * sizeof(uint64_t), hipMemcpyDeviceToHost,
                       s);
    if (e != hipSuccess) return hip_fail(e, "densify count copy");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "densify sync");
    for (int k = 0; k < 3; ++k) tot[k] = hs->pinned[k];
  }
  const int64_t total = int64_t(tot[0] + tot[1] + 2 * tot[2]);
  *n_out = total;
  if (counts)
    for (int k = 0; k < 3; ++k) counts[k] = int64_t(tot[k]);
  if (!write) return GS_OK;
  if (total > capacity) return fail(GS_ERR_CAPACITY, "the new population (%lld) exceeds capacity (%lld)",
                                    (long long)total, (long long)capacity);
  if (n > 0) {
    const hipError_t e = gsk::launch_densify_write(params, m, v, int(n), sh_degree, rand, a, ws, uint32_t(tot[0]),
                                                   uint32_t(tot[1]), uint32_t(tot[2]), params_out, m_out, v_out,
                                                   stats_out, s);
    if (e != hipSuccess) return hip_fail(e, "densify_write");
  }
  return GS_OK;
}

int32_t gs_relocate(float* params, float* m, float* v, int64_t n, int32_t sh_degree, const float* rand,
                    double dead_opacity, double donor_opacity, int64_t max_moves, int64_t* moves_out, void* ws,
                    size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (n < 0 || n >= (int64_t(1) << 31)) return fail(GS_ERR_INVALID_ARG, "n out of range");
  if (sh_degree < 0 || sh_degree > 3) return fail(GS_ERR_UNSUPPORTED, "SH degree must be 0..3");
  if (!(dead_opacity > 0.0 && dead_opacity < 1.0) || !(donor_opacity > 0.0 && donor_opacity < 1.0) ||
      !(dead_opacity <= donor_opacity))
    return fail(GS_ERR_INVALID_ARG, "opacity thresholds must satisfy 0 < dead <= donor < 1");
  if (n > 0 && (!params || !m || !v || !rand)) return fail(GS_ERR_INVALID_ARG, "an array is null");
  if (n > 0 && gsk::param_floats(n, gsk::num_planes(sh_degree)) >= (size_t(1) << 31))
    return fail(GS_ERR_UNSUPPORTED, "gs_param_floats(n, sh_degree) must stay below 2^31");
  const size_t need = gsk::relocate_ws_bytes(n);
  if (!ws || ws_bytes < need) return fail(GS_ERR_CAPACITY, "relocation workspace needs %zu bytes", need);
  int64_t moves = 0;
  if (n > 0) {
    hipStream_t s = as_stream(stream);
    const float logit_dead = float(std::log(dead_opacity / (1.0 - dead_opacity)));
    const float logit_donor = float(std::log(donor_opacity / (1.0 - donor_opacity)));
    hipError_t e = gsk::launch_relocate_count(params, int(n), sh_degree, logit_dead, logit_donor, ws, s);
    if (e != hipSuccess) return hip_fail(e, "relocate_count");
    HostSlot* hs = host_slot();
    if (!hs) return fail(GS_ERR_HIP, "cannot set up the pinned count buffer");
    e = hipMemcpyAsync(hs->pinned, gsk::carve_relocate(ws, n).totals, 2 * sizeof(uint64_t), hipMemcpyDeviceToHost,
                       s);
    if (e != hipSuccess) return hip_fail(e, "relocate count copy");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "relocate sync");
    const int64_t dead = int64_t(hs->pinned[0]), donors = int64_t(hs->pinned[1]);
    moves = std::min(dead, donors);
    if (max_moves >= 0) moves = std::min(moves, max_moves);
    e = gsk::launch_relocate_move(params, m, v, int(n), sh_degree, rand, int(donors), int(moves),
                                  float(std::log(1.6)), ws, s);
    if (e != hipSuccess) return hip_fail(e, "relocate_move");
  }
  if (moves_out) *moves_out = moves;
  return GS_OK;
}

int32_t gs_loss_charbonnier(const float* img, const float* target, int32_t H, int32_t W, float delta,
                            const float* exposure, float* loss_out, float* dL_dimg, float* dL_dexposure, void* ws,
                            size_t ws_bytes, void* stream) {
  g_err[0] = 0;
  if (H <= 0 || W <= 0 || int64_t(H) * W > (int64_t(1) << 29)) return fail(GS_ERR_INVALID_ARG, "bad image size");
  if (!img || !target || !exposure || !loss_out || !dL_dimg) return fail(GS_ERR_INVALID_ARG, "an argument is null");
  if (!(delta > 0.0f) || !std::isfinite(delta)) return fail(GS_ERR_INVALID_ARG, "delta must be positive");
  const size_t need = gsk::charbonnier_ws_bytes(H, W);
  if (!ws || ws_bytes < need) return fail(GS_ERR_CAPACITY, "Charbonnier workspace needs %zu bytes", need);
  const hipError_t e = gsk::launch_charbonnier(img, target, H, W, delta, exposure, loss_out, dL_dimg, dL_dexposure,
                                               ws, as_stream(stream));
  if (e != hipSuccess) return hip_fail(e, "loss_charbonnier");
  return GS_OK;
}

}  // extern "C"
