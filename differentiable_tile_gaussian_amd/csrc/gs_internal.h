// Internal declarations shared by the HIP translation units of libgs.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gs.h"

namespace gsk {

constexpr int kTile = 16;          // 16x16 pixel tiles
constexpr int kTilePixels = kTile * kTile;

inline int tiles_x(const gs_camera& c) { return (c.width + kTile - 1) / kTile; }
inline int tiles_y(const gs_camera& c) { return (c.height + kTile - 1) / kTile; }
inline int num_planes(int deg) { return 11 + 3 * (deg + 1) * (deg + 1); }

inline unsigned div_up(int64_t a, int64_t b) { return unsigned((a + b - 1) / b); }

// Blocked per-Gaussian parameter layout: groups of kGB Gaussians, each group holding
// its P planes of kGB floats one after another.  Parameter p of Gaussian i is at
// ((i / kGB) P + p) kGB + i % kGB.
constexpr int kGB = 64;
inline size_t param_floats(int64_t n, int P) { return size_t((n + kGB - 1) / kGB) * kGB * size_t(P); }
// Address of plane 0 of Gaussian i (plane p is kGB * p floats further on).
template <typename T>
__host__ __device__ inline T* gaussian_base(T* params, int i, int P) {
  return params + size_t(i / kGB) * size_t(P) * kGB + (i % kGB);
}

// How a Gaussian is shaded, for the projection and its gradient: kact, the active SH
// bands ((d + 1)^2 - 1 for an active degree d; the degree ramp), and mip, whether the
// Mip-Splatting compensation sqrt(det V / det(V + 0.3 I)) multiplies the opacity.
struct Shade {
  int kact;
  int mip;
};

// ---- preprocess.hip
// block_tiles: div_up(n, 256) per-block sums of the tile counts; *total_pairs their sum.
hipError_t launch_preprocess_fwd(const float* params, int n, int deg, const gs_camera& cam, const gs_proj& out,
                                 uint32_t* block_tiles, uint64_t* total_pairs, Shade shade, hipStream_t s);
// *total += the sum of block_tiles[0 .. nb) (the caller's kernel zeroed *total).
hipError_t launch_tile_count_total(const uint32_t* block_tiles, int nb, uint64_t* total, hipStream_t s);

// ---- chain.hip (gscreen is read only)
struct AdamArgs;
// Where the chain with projection writes the next camera's records: tx, ty its tile
// grid; block_tiles one sum per 64 Gaussians; *total zeroed, then their sum.
struct NextProj {
  gs_camera cam;
  int tx, ty;
  float4* splat;
  float* depth;
  uint2* rect;
  uint32_t* tiles;
  uint32_t* block_tiles;
  uint64_t* total;
};
// The chain without Adam: gparams = weight g, or += weight g with accumulate.
hipError_t launch_preprocess_bwd(const float* params, int n, int deg, const gs_camera& cam,
                                 const uint32_t* tiles, const float* gscreen, float* gparams, Shade shade,
                                 hipStream_t s, float weight = 1.0f, int accumulate = 0);
// Camera-pose gradient: out (device double[6]) = (rotation, translation); ws holds
// camera_grad_ws_bytes(n) bytes of per-block sums.
size_t camera_grad_ws_bytes(int64_t n);
hipError_t launch_camera_grad(const float* params, int n, int deg, const gs_camera& cam, const uint32_t* tiles,
                              const float* gscreen, int position_only, double* out, void* ws, Shade shade,
                              hipStream_t s);
hipError_t launch_chain_adam(float* params, int n, int deg, const gs_camera& cam, const uint32_t* tiles,
                             const float* gscreen, float* m, float* v, const AdamArgs& a, Shade shade, hipStream_t s);
// The same, then the projection of the updated Gaussians into np (may alias tiles: each
// Gaussian's count is read before its new record is written) and np's pair count; with
// dstats ([n][2], nullable) also the density statistics of this step's observations.
hipError_t launch_chain_adam_project(float* params, int n, int deg, const gs_camera& cam, const uint32_t* tiles,
                                     const float* gscreen, float* m, float* v, const AdamArgs& a,
                                     const NextProj& np, float* dstats, Shade shade, hipStream_t s);

// ---- scan.hip: exclusive prefix sum of n u32 values into out[0..n], out[n] = total.
// The total is also written as u64 to *total64 (device) so that overflow of 32 bits is seen.
// With n_dev, the count is min(n, *n_dev) (read on the device; ws sized for n).
size_t scan_ws_bytes(int64_t n);
hipError_t launch_scan_u32(const uint32_t* in, uint32_t* out, int64_t n, uint64_t* total64, void* ws,
                           hipStream_t s, const uint32_t* n_dev = nullptr);

// ---- sort.hip
// depth order of the visible Gaussians (proj.order, proj.n_visible) and the pair
// offsets in that order (proj.offs), for a projection whose visible Gaussians all have
// depth > znear > 0; then emission and the tile sort of the pairs
size_t depth_order_ws_bytes(int64_t n);
hipError_t launch_depth_order(const gs_proj& proj, int n, float znear, void* ws, hipStream_t s);
size_t bin_sort_ws_bytes(uint32_t pairs);
// Stable ascending sort of count (key, value) pairs by the 32-bit key, in place (the
// hand-written radix passes of the binning); ws: sort_pairs_ws_bytes(capacity) bytes,
// capacity >= count.
size_t sort_pairs_ws_bytes(int64_t capacity);
hipError_t launch_sort_pairs_u32(uint32_t* keys, uint32_t* vals, uint32_t count, int64_t capacity, void* ws,
                                 hipStream_t s);
hipError_t launch_bin_sort(const gs_proj& proj, int n, const gs_camera& cam, uint32_t pairs, uint32_t* keys,
                           uint32_t* vals, uint32_t* ranges, void* ws, hipStream_t s);

// ---- densify.hip
// Thresholds in the stored domains (logit, log-scale), rounded once from double.
struct DensifyArgs {
  float grad_thr, logit_prune, lscale_prune, lscale_split, lscale_shrink, logit_cap;
  int reset;
};
// Workspace: per-Gaussian flags (kept, cloned, split), their exclusive prefix sums
// (n + 1 entries each), the three totals (u64), the scans' block sums, the source of each
// kept place and the sources of the clones and of the split parents, in their order.
struct DensifyWs {
  uint32_t* flag[3];
  uint32_t* offs[3];
  uint64_t* totals;
  void* scan_ws[3];
  uint32_t* src_keep;
  uint32_t* src;
};
size_t densify_ws_bytes(int64_t n);
DensifyWs carve_densify(void* ws, int64_t n);
// Relocation of the dead to the largest donors: flags, prefix sums and their totals (dead,
// donors), the donors' rank keys, the dead list, the donors' keys and indices (ranked in
// place) and the ranking sort's space (bytes: the whole workspace).
struct RelocateWs {
  uint32_t *fdead, *fdonor, *odead, *odonor;
  uint64_t* totals;
  void* scan_ws[2];
  uint32_t *key, *dead_list, *key_in, *idx_in;
  void* sort_ws;
  size_t bytes;
};
size_t relocate_ws_bytes(int64_t n);
RelocateWs carve_relocate(void* ws, int64_t n);
// Classifies, scans (totals[0] dead, totals[1] donors) and compacts; then, once the host
// knows the counts, ranks the donors and makes the moves.
hipError_t launch_relocate_count(const float* params, int n, int deg, float logit_dead, float logit_donor, void* ws,
                                 hipStream_t s);
hipError_t launch_relocate_move(float* params, float* m, float* v, int n, int deg, const float* rand, int donors,
                                int moves, float shrink, void* ws, hipStream_t s);
hipError_t launch_densify_accumulate(const uint32_t* tiles, int n, const float* gscreen, float* stats,
                                     hipStream_t s);
hipError_t launch_densify_count(const float* params, int n, int deg, const float* stats, const DensifyArgs& a,
                                void* ws, hipStream_t s);
hipError_t launch_densify_write(const float* params, const float* m, const float* v, int n, int deg,
                                const float* rand, const DensifyArgs& a, void* ws, uint32_t kept, uint32_t cloned,
                                uint32_t splits, float* params_out, float* m_out, float* v_out, float* stats_out,
                                hipStream_t s);

// ---- render.hip
// Render workspace: a header the forward writes (its split sizes), the split state, and
// for fixed-point gradient sums 72 bytes per Gaussian (n_fixed Gaussians, else 0).
size_t render_ws_bytes(int W, int H, uint32_t pairs, int first, int chunk, int64_t n_fixed);
hipError_t launch_render_fwd(const gs_proj& proj, const uint32_t* vals, const uint32_t* ranges,
                             const gs_camera& cam, uint32_t pairs, float* rgb, float* T_final,
                             uint32_t* n_contrib, void* ws, int first, int chunk, hipStream_t s);
// fixed: gradient sums in fixed point (reproducible bit for bit); gscreen holds the float
// partials on return either way.  first, chunk size the launch (and the fixed-point
// accumulators' place); the walk takes the forward's split sizes from the header.
hipError_t launch_render_bwd(const gs_proj& proj, int n, const uint32_t* vals, const uint32_t* ranges,
                             const gs_camera& cam, uint32_t pairs, const float* T_final,
                             const uint32_t* n_contrib, const float* dL_dimg, float* gscreen, void* ws,
                             size_t ws_bytes, int first, int chunk, bool fixed, hipStream_t s);

// ---- loss.hip
size_t loss_ws_bytes(int H, int W);
// The no-allocation loss's scratch: a file-scope device array of loss_scratch_bytes()
// bytes; loss_scratch gives its address on the current device (looked up once per device).
size_t loss_scratch_bytes();
hipError_t loss_scratch(void** out);
hipError_t launch_loss(const float* img, const float* target, int H, int W, float lambda, float* loss_out,
                       float* grad, void* ws, hipStream_t s);
size_t charbonnier_ws_bytes(int H, int W);
hipError_t launch_charbonnier(const float* img, const float* target, int H, int W, float delta, const float* exposure,
                              float* loss_out, float* grad, float* dexp, void* ws, hipStream_t s);

// ---- layout.hip: planar [P][n] <-> blocked (padding written as zero)
hipError_t launch_to_blocked(const float* planar, float* blocked, int n, int P, hipStream_t s);
hipError_t launch_from_blocked(const float* blocked, float* planar, int n, int P, hipStream_t s);

// ---- adam.hip (blocked arrays; padding slots are not touched)
hipError_t launch_adam(float* params, const float* grads, float* m, float* v, int n, int deg, const float lr[5],
                       float b1, float b2, float omb1, float omb2, float eps, float inv_bc1, float inv_bc2,
                       hipStream_t s);

}  // namespace gsk
