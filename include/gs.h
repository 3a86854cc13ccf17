/*
 * gs.h -- C ABI of the MI355X (gfx950) tile-based differentiable Gaussian rasteriser.
 *
 * One training step for one camera is six calls, in this order:
 *
 *   gs_preprocess     project every Gaussian, count the 16x16 tiles it touches, order
 *                     the visible ones by depth and prefix-sum their counts in that
 *                     order; returns the number of (tile, Gaussian) pairs
 *   gs_bin_sort       order the (tile, Gaussian) pairs by tile, then depth, then id
 *                     (emission in the depth order of gs_preprocess, stable tile sort),
 *                     find each tile's [start, end) range
 *   gs_render_fwd     front-to-back alpha blending per pixel
 *   gs_loss_l1_dssim  0.8 L1 + 0.2 (1 - SSIM) and its image gradient
 *   gs_render_bwd     back-to-front blend with transmittance recovery, then the
 *                     per-Gaussian chain to parameter gradients
 *   gs_adam_step      Adam over every parameter plane
 *
 * Pages defining the operations (titles as they appear on the pages):
 *   [DR]   "Differentiable rasterisation" (splat-report knowledge base)
 *   [TBDR] "Tile-based differentiable rasterization in 3DGS" (learn-ml-visualized)
 *   [GST]  Gaussian splatting training study deck (bailiping.com)
 *   [GSG]  "How a computer rebuilds a real place out of soft colored dots called
 *          Gaussian Splats" (taosengine guide)
 *
 * Conventions for every entry point
 *   - Array arguments are DEVICE pointers owned by the caller, unless marked "host".
 *     The library never allocates, frees or retains caller memory.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on that stream and returns, except gs_preprocess, which waits
 *     for the pair count.
 *   - Arrays are fp32 unless stated otherwise.  Per-Gaussian parameter arrays
 *     (params, gradients, Adam moments) use the blocked layout below; other
 *     per-Gaussian arrays are planar, [plane][n]; images are [channel][H][W].
 *   - Return value: GS_OK or a negative gs_status; gs_last_error() then holds a
 *     message (per thread).  No C++ exception crosses the ABI.  On an argument
 *     error nothing is enqueued and no output is written.
 *
 * Scene parameters: P = 11 + 3 (deg + 1)^2 planes (14 at SH degree 0, 59 at degree 3):
 *   0-2 mean x, y, z | 3-5 log-scales | 6-9 quaternion w, x, y, z (need not be unit)
 *   10 opacity logit | 11-13 colour DC r, g, b (colour units, no basis factor)
 *   14 + 3 (k - 1) + ch, k = 1 .. (deg + 1)^2 - 1: spherical-harmonic band coefficients.
 *
 * Blocked parameter layout: the Gaussians are taken in groups of 64; a group stores its
 * P planes one after another, 64 floats each, so parameter p of Gaussian i is at
 *   ((i / 64) * P + p) * 64 + i % 64
 * and an array holds gs_param_floats(n, deg) = ceil(n / 64) * 64 * P floats.  The slots of
 * Gaussians i >= n in the last group are padding: never read as parameters, and left
 * untouched by every call except gs_params_to_blocked (which zeroes them).  Each group's
 * parameters are one contiguous stretch, which is what the per-Gaussian passes stream.
 */
#ifndef GS_H_
#define GS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gs_status {
  GS_OK = 0,
  GS_ERR_INVALID_ARG = -1,  /* null pointer, negative size, bad camera, step < 1 ... */
  GS_ERR_CAPACITY = -2,     /* key buffer or workspace too small, or more than 2^32 - 2^25 pairs
                               (every call that takes or returns a pair count checks it) */
  GS_ERR_UNSUPPORTED = -3,  /* SH degree outside 0..3, image larger than 65535 tiles per side */
  GS_ERR_HIP = -4           /* a HIP launch or runtime call failed */
} gs_status;

/* Pinhole camera, OpenCV axes (x right, y down, z forward): p_cam = R p_world + t.
 * Pixel (i, j) covers [i, i+1) x [j, j+1) and is sampled at its centre (i + 0.5, j + 0.5);
 * the image point of p_cam is (fx x/z + cx, fy y/z + cy).  [GSG] "Flattening a 3D blob";
 * [GST] Jacobian slide.  Gaussians with z <= znear are culled. */
typedef struct gs_camera {
  float R[9];           /* row-major world -> camera rotation */
  float t[3];
  float campos[3];      /* camera centre in world coordinates (= -R^T t), used for the SH view direction */
  float fx, fy, cx, cy; /* pixels */
  int32_t width, height;
  float znear;
  float bg[3];          /* background colour behind the last Gaussian */
} gs_camera;

typedef struct gs_scene {
  int64_t n;            /* number of Gaussians, 0 <= n < 2^31 */
  int32_t sh_degree;    /* 0..3 */
  const float* params;  /* device, blocked layout, gs_param_floats(n, sh_degree) floats */
} gs_scene;

/* Projected per-Gaussian state written by gs_preprocess and read by the later calls.
 * Device arrays allocated by the caller. */
typedef struct gs_proj {
  float* splat;         /* [n][12] packed record: u, v, A, B, C, opacity, r, g, b, hx, hy, tm
                           (screen centre, conic, opacity, clamped colour, the half-widths
                           of a box around (u, v) outside which no pixel centre gets
                           alpha >= 1/255: negative if none can, infinite if unbounded, and
                           tm, ln(255 opacity) widened by 1 % + 0.01: the bound on the
                           exponent within which a pixel can reach 1/255, negative or
                           infinite with the box); zero when culled */
  float* depth;         /* [n] camera-space z (the sort key's low 32 bits) */
  uint32_t* rect;       /* [n][2] tile rectangle, inclusive: x0 | y0 << 16, x1 | y1 << 16 */
  uint32_t* tiles;      /* [n] tiles touched, 0 when culled */
  uint32_t* order;      /* [n] ids of the visible Gaussians (tiles > 0) ordered by depth, then id;
                           the first *n_visible entries are written */
  uint32_t* n_visible;  /* [1] number of visible Gaussians */
  uint32_t* offs;       /* [n + 1] exclusive prefix sum of tiles[order[r]] over the visible r:
                           offs[r] is the first pair of the r-th Gaussian in depth order and
                           offs[*n_visible] = pair count (the first *n_visible + 1 entries are
                           written) */
  uint32_t* rect_order; /* [n][2] rect of the r-th visible Gaussian in depth order (the first
                           *n_visible entries are written), read by gs_bin_sort */
} gs_proj;

/* Per-call settings of the method's variants and of the blend's work split.  Every call that
 * depends on one takes a `const gs_config*`; NULL means GS_CONFIG_DEFAULT.  The library keeps no
 * settings between calls.
 *   grad_sums        how the backward blend sums the per-pixel gradient contributions:
 *     GS_GRAD_SUMS_FLOAT  fp32 atomics; the order of the additions varies from run to run.
 *     GS_GRAD_SUMS_FIXED  [GSG] "Making the parallel sums exact: fixed-point, and the conic
 *       trick": every wave-summed moment (position moments, the three second moments divided
 *       by a footprint size factor 1 + trace of the screen covariance, opacity, colour), times
 *       16384 and times the loss's element count 3 W H (so that the unit is that of the summed
 *       loss), clamped to +-1e9 and rounded to the nearest integer, is added with integer
 *       atomics (i32 within a tile block, i64 across blocks, so a Gaussian's total cannot wrap);
 *       a decode pass turns the sums into the same partials as the float mode.  Results are
 *       identical bit for bit from run to run; each addition is exact to 0.5 / (16384 * 3 W H).
 *       The render workspace then also holds 72 bytes per Gaussian.
 *   active_sh_degree the SH degree ramp ([GSG] "Spherical harmonics": only the first activeK =
 *     (activeDeg + 1)^2 - 1 band weights are summed, the active degree stepping up about every
 *     thousand steps; the inactive ones contribute nothing and receive no gradient until their
 *     band switches on): the projection and the chain sum the colour over the bands up to
 *     min(active_sh_degree, the scene's degree), and the other bands' gradients are zero (with
 *     the fused Adam their parameters stay unchanged while their moments are zero).  -1: every
 *     stored band.  Read by gs_preprocess, the backward calls and gs_camera_grad.
 *   mip_compensation Mip-Splatting opacity compensation ([GSG] "Flattening a 3D blob into a 2D
 *     oval": a correction so that the dilation does not make very small Gaussians brighter
 *     overall; the trainer's code multiplies the opacity by it in the extent and in alpha).
 *     With 1 the record's opacity is sigmoid(logit) comp, comp = sqrt(max(det V, 0) / det(V +
 *     0.3 I)), V the undilated screen covariance (the factor that gives the dilated footprint
 *     exactly the integral of the undilated one), so it also enters the extent, alpha and the
 *     skip boxes; the chain adds comp's gradient to the covariance's and scales the logit's by
 *     comp.  The blend is unchanged (it differentiates the record's opacity).  0: off.  Read by
 *     gs_preprocess, the backward calls and gs_camera_grad.
 *   split_first, split_chunk  the blend's work split: every tile's first split_first pairs are
 *     walked by one block; a tile with pixels still unfinished then has its remaining pairs
 *     walked in parallel chunks of split_chunk pairs.  0: the defaults 2048 and 512; otherwise
 *     multiples of 4 in [4, 2^24].  The results do not depend on them beyond rounding.  Read
 *     by gs_render_fwd, which records them in its workspace: the matching backward walks with
 *     the forward's values whatever its own cfg says (its cfg's values only size its launch).
 * Calls return GS_ERR_INVALID_ARG for a value outside these ranges. */
typedef struct gs_config {
  int32_t grad_sums;
  int32_t active_sh_degree;
  int32_t mip_compensation;
  int32_t split_first;
  int32_t split_chunk;
} gs_config;
enum { GS_GRAD_SUMS_FLOAT = 0, GS_GRAD_SUMS_FIXED = 1 };
#define GS_CONFIG_DEFAULT {GS_GRAD_SUMS_FLOAT, -1, 0, 0, 0}

/* Projection of every Gaussian and the tile count prefix sum.
 * [GST] parameter slide (exp log-scales, sigmoid logit, normalised quaternion);
 * [DR] "Forward" (Sigma' = J W Sigma W^T J^T) and "From a pixel error back to a quaternion"
 * (Sigma = R S S^T R^T); [GST] Jacobian slide (J and the 0.3 px^2 dilation); [GSG]
 * "Flattening a 3D blob into a 2D oval" (conic), "Why tiling, and the five stages" (extent
 * rad = sqrt(2 min(4.5, ln max(255 o, 1.0001))) sqrt(lambda_max), tile rectangle, count and
 * scan), "Spherical harmonics" (colour = DC + sum_k sh_k Y_k(normalize(mean - campos)),
 * clamped at 0).
 * The key path (camera-space depth, screen centre, extent, rectangle) is computed in IEEE
 * fp32 without contraction, with exp/log/sigmoid evaluated in fp64 and rounded once, so the
 * pair list is a deterministic function of the inputs.  The visible Gaussians are also put
 * in depth order (stable radix sort of the depth bits, so ties keep id order) for the
 * binning: out->order, out->n_visible, out->offs and out->rect_order.
 * out: caller-allocated gs_proj for scene->n Gaussians.  total_pairs: HOST pointer,
 * receives the pair count (= offs[n]).  ws: device workspace of
 * gs_workspace_bytes(GS_WS_PREPROCESS, n, 0, 0, 0, NULL) bytes.  Waits for the pair count only:
 * it is copied to the host before the depth ordering is enqueued, which may still be
 * running on `stream` when the call returns.  The library keeps one pinned 8-byte host
 * word and one event per device and host thread for this copy.  GS_ERR_CAPACITY if the
 * pair count exceeds 2^32 - 2^25 (the kernels keep pair indices in 32 bits). */
/* cfg: active_sh_degree, mip_compensation. */
int32_t gs_preprocess(const gs_scene* scene, const gs_camera* cam, gs_proj* out, uint32_t* total_pairs,
                      void* ws, size_t ws_bytes, const gs_config* cfg, void* stream);

/* Duplicate-with-keys, depth sort and tile ranges.  [GSG] "Why tiling, and the five stages"
 * (scatter, per-tile depth sort, ranges with the tie broken by id).  Every (tile, Gaussian)
 * pair of a visible Gaussian i (tile count > 0; tiles in row-major order over its rectangle)
 * is produced once, and the pairs are ordered by tile id (ty * tiles_x + tx), then by the
 * Gaussian's depth (as the bits of the positive float, i.e. numerically), then by i -- the
 * order of the 64-bit key tile << 32 | bits(depth[i]) with ties by id.  Computed from the
 * depth order gs_preprocess made: the pairs are emitted Gaussian by Gaussian in that order,
 * then stably radix-sorted by tile.
 * keys[capacity]: tile id of each sorted pair; vals[capacity]: its Gaussian id; the first
 * total_pairs entries are written.  ranges: [2][tiles_x * tiles_y] u32, ranges[0][t] = first,
 * ranges[1][t] = one past the last pair of tile t ((0, 0) for an empty tile).  proj: as
 * gs_preprocess left it (order, n_visible, offs and rect_order are read); total_pairs must be the
 * value gs_preprocess returned for the same proj.  ws: gs_workspace_bytes(GS_WS_BIN_SORT, n,
 * total_pairs, W, H, NULL).  GS_ERR_CAPACITY (nothing written) if capacity < total_pairs or the
 * workspace is short. */
int32_t gs_bin_sort(const gs_proj* proj, int64_t n, const gs_camera* cam, uint32_t total_pairs, uint32_t* keys,
                    uint32_t* vals, uint32_t capacity, uint32_t* ranges, void* ws, size_t ws_bytes, void* stream);

/* Front-to-back compositing, [GSG] "The painting itself: front-to-back alpha compositing";
 * [GST] opacity slide (cap 0.99, skip below 1/255, early termination); [TBDR] worked
 * examples.  For each pixel centre p and each pair of its tile in order:
 *   e = 0.5 (A dx^2 + C dy^2) + B dx dy with d = p - (u, v); alpha = min(0.99, o exp(-e));
 *   skip if alpha < 1/255; C += T alpha c; T *= 1 - alpha; stop once T < 1e-4.
 * rgb[3][H][W] = C + T bg; T_final[H][W] = T; n_contrib[H][W] = 1 + (index within the tile's
 * range) of the last blended pair, 0 if none ([DR] "The trick": only the final state is kept).
 * total_pairs: the pair count of the sort.  ws: gs_workspace_bytes(GS_WS_RENDER, n, total_pairs,
 * W, H, cfg) bytes; it keeps the state that the matching gs_render_bwd reads (the split sizes used,
 * the tile order and, for tiles whose list is walked in parallel chunks, the per-chunk boundary
 * states), so pass the same ws, unmodified, to that backward.  cfg: split_first, split_chunk. */
int32_t gs_render_fwd(const gs_proj* proj, int64_t n, const uint32_t* vals, const uint32_t* ranges,
                      uint32_t total_pairs, const gs_camera* cam, float* rgb, float* T_final,
                      uint32_t* n_contrib, void* ws, size_t ws_bytes, const gs_config* cfg, void* stream);

/* Loss (1 - lambda) L1 + lambda (1 - SSIM) and dL/dimg.  [GST] loss slides: L1 mean over
 * 3HW with zero subgradient at zero residual; SSIM with an 11 x 11 Gaussian window of
 * standard deviation 1.5, C1 = 0.01^2, C2 = 0.03^2, zero padding, averaged over pixels and
 * channels; no one-half on D-SSIM; lambda = 0.2 in the method.
 * img, target: [3][H][W].  loss_out: device float[3] = total, L1, mean SSIM.
 * dL_dimg: [3][H][W], overwritten.  ws: gs_workspace_bytes(GS_WS_LOSS, 0, 0, W, H, NULL). */
int32_t gs_loss_l1_dssim(const float* img, const float* target, int32_t H, int32_t W, float lambda_dssim,
                         float* loss_out, float* dL_dimg, void* ws, size_t ws_bytes, void* stream);

/* gs_loss_l1_dssim for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same loss and image
 * gradient, bit for bit, with the per-block partial sums in a static device array of the
 * library (256 KiB per GPU, held until the process ends) instead of a workspace argument.
 * Calls no allocator.  GS_ERR_CAPACITY for an image whose partial sums do not fit, i.e.
 * gs_workspace_bytes(GS_WS_LOSS, 0, 0, W, H, NULL) > 256 KiB (about 6000 x 6000 pixels is
 * the largest square that fits); other errors as gs_loss_l1_dssim.  Calls that overlap on
 * one GPU (other streams, other host threads) share that array and race: serialise them. */
int32_t gs_loss_l1_dssim_noalloc(const float* img, const float* target, int32_t H, int32_t W, float lambda_dssim,
                                 float* loss_out, float* dL_dimg, void* stream);

/* The trainer's other loss: Charbonnier with per-image exposure ([GSG] the loss code after
 * "The painting itself"; "Forgiving the camera and the light").  Per element
 *   err = gain img + bias - target,  root = sqrt(err^2 + delta^2),
 * gain = exp(exposure[0]), bias = exposure[1]; the loss is the mean of root - delta over the
 * 3HW elements, dL/dimg = gain err / root / 3HW, and dL_dexposure (nullable) receives the
 * means of (err / root) img gain (the log gain's gradient) and err / root (the bias's).
 * img, target, dL_dimg: [3][H][W]; exposure, dL_dexposure: device float[2]; loss_out: device
 * float[1]; delta > 0 (0.03 on the page).  The sums are formed in a fixed order (the result
 * is reproducible).  ws: gs_workspace_bytes(GS_WS_LOSS_CHARBONNIER, 0, 0, W, H, NULL). */
int32_t gs_loss_charbonnier(const float* img, const float* target, int32_t H, int32_t W, float delta,
                            const float* exposure, float* loss_out, float* dL_dimg, float* dL_dexposure, void* ws,
                            size_t ws_bytes, void* stream);

/* Backward pass.  Part 1, the blend: [DR] "The trick: recompute the blend state instead of
 * storing it"; [GSG] "The clever bit: a single backward sweep through the blend" and "From a
 * pixel's blame to the oval's shape and place"; [GST] compositing-derivative slide.  Each
 * pixel walks its tile's pairs from n_contrib - 1 down to 0, recovers T_i = T_{i+1} / (1 -
 * alpha_i), keeps S = colour behind (starting at bg T_final), and accumulates per Gaussian:
 *   dc += g alpha T;  dalpha = sum_ch g (c T - S / (1 - alpha));  when alpha is not capped:
 *   do += dalpha G, and through e: du, dv, dA, dB, dC.
 * gscreen: [n][9], per Gaussian du, dv, dA, dB, dC, d opacity, dr, dg, db (Gaussian-major,
 * so that the partials of one pair share a cache line) -- zeroed and filled here.
 * Part 2, the chain per Gaussian: [GSG] "The covariance chain" (conic -> V -> Sigma -> M ->
 * scale and quaternion, projection off |q|), "Where the position gradient comes from"
 * (mean path and the J(z) covariance path), "Spherical harmonics" (band gradients and the
 * view-direction term), sigmoid.  gparams: blocked layout, every Gaussian's P parameters
 * overwritten (zero for culled Gaussians); padding untouched.
 * proj, vals, ranges, total_pairs, T_final, n_contrib and ws must be those of the matching
 * forward (ws as that forward left it; its header holds the split sizes the forward used, and
 * a ws no forward of this image and pair count has written makes every screen partial and
 * parameter gradient NaN).  cfg: grad_sums, active_sh_degree, mip_compensation (the values the
 * projection used); its split sizes only size the launch; ws must hold gs_workspace_bytes(
 * GS_WS_RENDER, n, total_pairs, W, H, cfg) bytes. */
int32_t gs_render_bwd(const gs_scene* scene, const gs_proj* proj, const uint32_t* vals, const uint32_t* ranges,
                      uint32_t total_pairs, const gs_camera* cam, const float* T_final,
                      const uint32_t* n_contrib, const float* dL_dimg, float* gscreen, float* gparams, void* ws,
                      size_t ws_bytes, const gs_config* cfg, void* stream);

/* gs_render_bwd for a step over several views (the trainer's loop renders one view per step;
 * a batch of views is the same loop with their gradients summed before one Adam update).
 * Every Gaussian's P parameter gradients g of this view are written as
 *   gparams = weight g            (accumulate = 0), or
 *   gparams = gparams + weight g  (accumulate = 1, each entry read and rounded once more),
 * e.g. weight 1/B for the mean over B views, the first with accumulate = 0.  weight 1 with
 * accumulate 0 is gs_render_bwd exactly.  Other arguments, and errors, as gs_render_bwd;
 * GS_ERR_INVALID_ARG for a non-finite weight or accumulate other than 0 or 1. */
int32_t gs_render_bwd_weighted(const gs_scene* scene, const gs_proj* proj, const uint32_t* vals,
                               const uint32_t* ranges, uint32_t total_pairs, const gs_camera* cam,
                               const float* T_final, const uint32_t* n_contrib, const float* dL_dimg,
                               float* gscreen, float* gparams, float weight, int32_t accumulate, void* ws,
                               size_t ws_bytes, const gs_config* cfg, void* stream);

/* Camera-pose gradient ([GSG] "Forgiving the camera and the light": the pose receives the
 * loss's gradient like any other parameter).  With the rotation perturbed on the left,
 * W <- (I + [w]x) W, and the translation t (the camera centre is -W^T t), every visible
 * Gaussian (proj->tiles[i] > 0) contributes through T = J W of its covariance, through its
 * camera-space centre p = W m + t and through its colour's view direction:
 *   G = J^T dT + dp m^T + t gsh^T  (= dL/dW; gsh the view-direction part of dL/dm),
 *   dL/dw = (M21 - M12, M02 - M20, M10 - M01) with M = G W^T,   dL/dt = dp + W gsh.
 * position_only = 1 gives the trainer's own accumulation instead (the same section's
 * code): only the position path, i.e. the torque sum (p - t) x dp and dL/dt = sum dp, with
 * dp the camera-space position gradient (its projected-mean and J(z) parts); 0 gives the
 * exact derivative above.  GS_ERR_INVALID_ARG for another value.
 * grad_out: device double[6] = (dL/dw, dL/dt), overwritten.  scene, proj, cam and gscreen as
 * gs_render_bwd read and left them: the parameters before any update of this step (the fused
 * update calls overwrite them, so pose optimisation takes gs_render_bwd and gs_adam).  The
 * per-Gaussian terms are formed in double and summed in a fixed order (the result is
 * reproducible).  ws: gs_workspace_bytes(GS_WS_CAMERA_GRAD, n, 0, 0, 0, NULL).  cfg:
 * active_sh_degree, mip_compensation (as the projection used them).  Enqueues only. */
int32_t gs_camera_grad(const gs_scene* scene, const gs_proj* proj, const gs_camera* cam, const float* gscreen,
                       int32_t position_only, double* grad_out, void* ws, size_t ws_bytes, const gs_config* cfg,
                       void* stream);

/* Adam, [GSG] Adam section; per-group rates [DR] "From a pixel error back to a quaternion".
 *   m = b1 m + (1 - b1) g;  v = b2 v + (1 - b2) g^2;
 *   theta -= lr_group (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)
 * params, m, v: blocked layout, updated in place (padding untouched); grads: blocked layout.
 * Arrays 16-byte aligned take the vectorised kernel.  lr: HOST float[5] for the groups
 * means, log-scales, quaternion, opacity, colour (DC and bands).  beta1, beta2, eps are host
 * fp64 scalars: 1 - beta and the bias corrections are formed in fp64 and rounded once to
 * fp32 for the kernel.  step t >= 1. */
int32_t gs_adam_step(float* params, const float* grads, float* m, float* v, int64_t n, int32_t sh_degree,
                     const float* lr, double beta1, double beta2, double eps, int32_t step, void* stream);

/* gs_render_bwd followed by gs_adam_step, fused: the chain applies Adam to each parameter as
 * soon as its gradient is known, so the parameter gradient is never written to memory (it
 * saves two passes over the parameter arrays).  Same arguments and results as the two calls, with
 * params updated in place; gscreen holds the screen-space partials on return, as after
 * gs_render_bwd. */
int32_t gs_render_bwd_adam(float* params, int64_t n, int32_t sh_degree, const gs_proj* proj, const uint32_t* vals,
                           const uint32_t* ranges, uint32_t total_pairs, const gs_camera* cam,
                           const float* T_final, const uint32_t* n_contrib, const float* dL_dimg, float* gscreen,
                           float* m, float* v, const float* lr, double beta1, double beta2, double eps,
                           int32_t step, void* ws, size_t ws_bytes, const gs_config* cfg, void* stream);

/* gs_render_bwd_adam followed by gs_preprocess of the updated scene for the camera of the
 * next step ([GSG] "Putting every stage together": per step, pick a view, project, tile,
 * composite, loss, backward, Adam; here the next step's view is picked before this step's
 * update, which changes no result).  The chain projects each
 * Gaussian for next_cam from the parameters it has just computed, in the same kernel,
 * so they are not read back from memory; the projection, depth order, pair offsets
 * and pair count are those gs_preprocess(scene, next_cam, next_out, next_total_pairs,
 * pre_ws) would produce from the updated params, bit for bit.  next_out may be proj
 * itself (each Gaussian's tile count is read before its new record is written).
 * pre_ws: gs_workspace_bytes(GS_WS_PREPROCESS, n, 0, 0, 0, NULL) bytes.  densify_stats (device
 * float [n][2], nullable): when given, this step's observations are added to it as
 * gs_densify_accumulate would (from this step's tile counts, before they are replaced).
 * Waits for the next pair count as gs_preprocess does; errors as gs_render_bwd_adam and
 * gs_preprocess.  cfg as for gs_render_bwd; the projection for next_cam uses its
 * active_sh_degree and mip_compensation too. */
int32_t gs_render_bwd_adam_project(float* params, int64_t n, int32_t sh_degree, const gs_proj* proj,
                                   const uint32_t* vals, const uint32_t* ranges, uint32_t total_pairs,
                                   const gs_camera* cam, const float* T_final, const uint32_t* n_contrib,
                                   const float* dL_dimg, float* gscreen, float* m, float* v, const float* lr,
                                   double beta1, double beta2, double eps, int32_t step, void* ws, size_t ws_bytes,
                                   const gs_camera* next_cam, gs_proj* next_out, uint32_t* next_total_pairs,
                                   void* pre_ws, size_t pre_ws_bytes, float* densify_stats, const gs_config* cfg,
                                   void* stream);

/* Layout of the per-Gaussian parameter arrays (see the blocked layout above).
 * gs_param_floats: floats in a blocked array for n Gaussians (0 for bad arguments).
 * gs_params_to_blocked: planar [P][n] -> blocked, padding zeroed; gs_params_from_blocked:
 * blocked -> planar [P][n].  Device arrays owned by the caller, not overlapping; the
 * conversion is enqueued on `stream`. */
size_t gs_param_floats(int64_t n, int32_t sh_degree);
int32_t gs_params_to_blocked(const float* planar, float* blocked, int64_t n, int32_t sh_degree, void* stream);
int32_t gs_params_from_blocked(const float* blocked, float* planar, int64_t n, int32_t sh_degree, void* stream);

/* Workspace sizes, in bytes, for the calls that take one. */
/* Density control, statistics ([GST] density-control slide: screen-space centre gradient
 * magnitudes accumulated per visible observation).  After a step's backward (gs_render_bwd or
 * the fused calls), for every Gaussian with proj->tiles[i] > 0:
 *   stats[i][0] += |(du, dv)| (from gscreen[i][0..1]);  stats[i][1] += 1.
 * stats: device float [n][2], updated in place (zero it when a population starts).
 * gscreen, proj: as the backward left them.  Enqueues only. */
int32_t gs_densify_accumulate(const gs_proj* proj, int64_t n, const float* gscreen, float* stats, void* stream);

/* Density control, one densification ([GST] density-control slide; [GSG] "Densification").
 * For Gaussian i, with average a = stats[i][0] / stats[i][1] (0 when never observed) and s
 * its largest scale:
 *   pruned   if opacity < prune_opacity or s > prune_scale;
 *   else, if a >= grad_threshold: split if s > split_scale, else cloned;
 *   else kept.
 * The comparisons are taken on the stored logit and log-scales against the thresholds'
 * logit / log formed in double and rounded once to float (a prune_scale of +infinity
 * prunes by opacity only).  New population: the kept and cloned Gaussians in their order,
 * then the clones (exact copies), then the first and then the second children of the split
 * ones; the child of Gaussian i with c = 0, 1 has mean + Rq (s * eps), eps = rand[i][c][0..2]
 * (caller-drawn standard normals; Rq from the normalised quaternion, the identity for a zero
 * one; s the scales exp(log-scales)) and log-scales lowered by ln 1.6 ([GSG]: halves shrink by
 * 1.6), everything else copied.  Clones and children start with zero m and v; kept Gaussians
 * keep theirs.  With reset_opacity, every output's logit becomes min(logit, logit(opacity_cap))
 * and its opacity moments zero.  stats_out is zeroed for the outputs.
 * params, m, v: blocked layout for n; stats [n][2]; rand [n][2][3] (device).  Outputs: blocked
 * for capacity Gaussians (padding untouched), stats_out [capacity][2], none overlapping an
 * input.  *n_out (host) receives the new count and counts (host int64[3], nullable) the numbers
 * kept, cloned and split; with params_out == NULL only these are computed.  GS_ERR_CAPACITY
 * (nothing written) if the new count exceeds capacity.  ws: gs_workspace_bytes(GS_WS_DENSIFY,
 * n, 0, 0, 0, NULL).  Waits for the counts (one copy to a pinned host word). */
int32_t gs_densify(const float* params, const float* m, const float* v, const float* stats, const float* rand,
                   int64_t n, int32_t sh_degree, double grad_threshold, double prune_opacity, double prune_scale,
                   double split_scale, int32_t reset_opacity, double opacity_cap, float* params_out, float* m_out,
                   float* v_out, float* stats_out, int64_t capacity, int64_t* n_out, int64_t* counts, void* ws,
                   size_t ws_bytes, void* stream);

/* Relocation of the dead ([GSG] "Densification", the MCMC-style pass: Gaussians that have
 * become transparent are reused as copies of well-opaque ones, preferring the biggest; each
 * pair then shrinks by a factor 1.6 and restarts its Adam moments).  Gaussian i is dead when its opacity is below
 * dead_opacity (about 0.02 on the page), a donor when it is not dead, its opacity is above
 * donor_opacity (about 0.4) and its largest log-scale is not NaN (the comparisons on the
 * stored logit against the thresholds' logit formed in double and rounded once to float).
 * The donors are ranked by their largest log-scale, largest first, equal sizes in index
 * order; the k-th dead Gaussian in index order is moved to the k-th ranked donor, for k
 * below min(dead, donors) and below max_moves when max_moves >= 0.  A moved Gaussian takes
 * all of its donor's parameters, with the mean at donor mean + Rq (s eps) (eps =
 * rand[i][0..2], caller-drawn standard normals of the moved Gaussian i; Rq and s as for a
 * split child of gs_densify) and the log-scales lowered by ln 1.6; the donor's log-scales
 * are lowered by ln 1.6 too; both get zero m and v.  All other Gaussians are unchanged, and
 * so is the count.  params, m, v: blocked layout for n, updated in place; rand [n][3]
 * (device).  *moves_out (host, nullable): the number of moves.  ws: gs_workspace_bytes(
 * GS_WS_RELOCATE, n, 0, 0, 0, NULL).  Waits for the two counts (one copy to a pinned host buffer);
 * the donors are ranked by a stable radix sort of their inverted size keys (the library's own
 * radix passes), so equal sizes keep the order of their indices. */
int32_t gs_relocate(float* params, float* m, float* v, int64_t n, int32_t sh_degree, const float* rand,
                    double dead_opacity, double donor_opacity, int64_t max_moves, int64_t* moves_out, void* ws,
                    size_t ws_bytes, void* stream);

enum { GS_WS_PREPROCESS = 0, GS_WS_BIN_SORT = 1, GS_WS_LOSS = 2, GS_WS_RENDER = 3, GS_WS_DENSIFY = 4,
       GS_WS_LOSS_CHARBONNIER = 5, GS_WS_CAMERA_GRAD = 6, GS_WS_RELOCATE = 7 };

/* Workspace size in bytes for the call `which_call` (GS_WS_*) with n Gaussians, `pairs` pairs
 * and a W x H image; cfg as the call will receive it (NULL: defaults).  The render workspace
 * (GS_WS_RENDER) depends on cfg's split sizes and gradient-sum mode; the others do not. */
size_t gs_workspace_bytes(int32_t which_call, int64_t n, uint32_t pairs, int32_t W, int32_t H, const gs_config* cfg);

/* Optional per-kernel timing (instrumentation, not part of the method).  gs_profile_enable(1, only)
 * makes every later library call bracket each kernel launch whose name equals `only` (every
 * launch if `only` is NULL or "") with two HIP events recorded on the call's stream;
 * gs_profile_enable(0, NULL) stops it.  Either call waits for and drops the records held.
 * gs_profile_query waits for the recorded events and writes, per kernel name in first-seen
 * order, the name (NUL-terminated, in 64-byte slots of `names`), the number of launches and the
 * summed elapsed milliseconds; it returns the number of names written (at most max_names) or a
 * negative gs_status.  Host buffers, owned by the caller.  Not thread-safe against concurrent
 * library calls on other threads. */
int32_t gs_profile_enable(int32_t on, const char* only);
int32_t gs_profile_query(int32_t max_names, char* names, int64_t* launches, double* total_ms);

/* Message of the last failed call on this thread ("" if none). */
const char* gs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GS_H_ */
