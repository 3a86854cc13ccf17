// Binning and depth sort ([GSG] "Why tiling, and the five stages": scatter, sort,
// segment boundaries; ties broken by Gaussian id).  The pairs end up ordered by
// tile, then depth, then Gaussian id, built in three steps:
//
//   depth sort    the visible Gaussians (tile count > 0), in id order, are sorted by
//                 the bits of their (positive) depth with a stable LSD radix sort;
//                 the first pass also compacts them, so later passes only see the
//                 visible ones.  Result: visible Gaussian ids by (depth, id).
//   emit          their tile counts, in that order, are prefix-summed; one thread
//                 per pair finds its Gaussian by binary search in the sums and
//                 writes (tile id, Gaussian id): the pairs of each Gaussian are
//                 consecutive and the Gaussians are in (depth, id) order.
//   tile sort     a stable LSD radix sort of the pairs by tile id, so within a
//                 tile they keep the (depth, id) order.
//   tile_ranges   first / one-past-last pair of each tile.
//
// Radix passes use 8-bit digits, reduce-then-scan:
//   upsweep   per-block digit histogram (LDS atomics)
//   scan      exclusive prefix over the digit-major [256][blocks] table
//   downsweep each wave ranks its 1024 consecutive items against a wave-private digit
//             histogram (64-lane ballots: no match-any on CDNA, 8 ballots give each
//             lane its peer mask), one barrier turns the four histograms into run
//             starts, then a local reorder through LDS and a coalesced scatter.
// Sorting the Gaussians by depth once, instead of every pair by a 64-bit (tile, depth)
// key, replaces six passes over 12-byte pairs by four passes over the visible
// Gaussians (about 40 % of them at the orbit cameras) and two over 8-byte pairs.
#include <algorithm>

#include "gs_internal.h"
#include "profile.h"

namespace gsk {
namespace {

constexpr int kSortThreads = 256;
constexpr int kSortItems = 16;
constexpr int kSortTile = kSortThreads * kSortItems;   // 4096 items per block
constexpr int kRadix = 256;
constexpr int kDepthPasses = 4;                         // 31 significant bits of a positive float

// Where a radix pass reads its items from.
enum Source {
  kFromKeys = 0,      // keys[idx], vals[idx], idx < count (count on the device if count_dev)
  kFromDepth = 1      // depth bits of Gaussian idx, value idx; only Gaussians with tiles[idx] > 0
};

struct PassIn {
  const uint32_t* keys;
  const uint32_t* vals;
  const float* depth;
  const uint32_t* tiles;
  uint32_t count;
  const uint32_t* count_dev;
};

template <int SRC>
__device__ inline bool load_item(const PassIn& in, uint32_t count, uint32_t idx, uint32_t& key, uint32_t& val) {
  if (idx >= count) return false;
  if (SRC == kFromDepth) {
    // both loads issued before either is tested
    const uint32_t t = in.tiles[idx];
    key = __float_as_uint(in.depth[idx]);
    val = idx;
    if (t == 0u) return false;
  } else {
    key = in.keys[idx];
    val = in.vals[idx];
  }
  return true;
}

__device__ inline uint32_t pass_count(const PassIn& in) { return in.count_dev ? *in.count_dev : in.count; }

template <int SRC>
__global__ void __launch_bounds__(kSortThreads) radix_upsweep_kernel(PassIn in, int shift, int nb,
                                                                      uint32_t* __restrict__ hist) {
  __shared__ uint32_t s_hist[kRadix];
  s_hist[threadIdx.x] = 0u;
  __syncthreads();
  const uint32_t count = pass_count(in);
  const uint32_t base = blockIdx.x * kSortTile;
  if (base < count) {
#pragma unroll 4
    for (int k = 0; k < kSortItems; ++k) {
      uint32_t key = 0, val = 0;
      if (load_item<SRC>(in, count, base + k * kSortThreads + threadIdx.x, key, val))
        atomicAdd(&s_hist[(key >> shift) & 0xffu], 1u);
    }
  }
  __syncthreads();
  hist[threadIdx.x * nb + blockIdx.x] = s_hist[threadIdx.x];
}

// hist_scan has kRadix * nb + 1 entries, the last one the total: with kFromDepth
// that is the number of visible Gaussians, which block 0 stores to *count_out.
// With rect_out, the item's value (a Gaussian id) is also looked up in val_rect and
// its tile rectangle and tile count written beside it (in the output order).
template <int SRC>
__global__ void __launch_bounds__(kSortThreads) radix_downsweep_kernel(
    PassIn in, int shift, int nb, const uint32_t* __restrict__ hist, const uint32_t* __restrict__ hist_scan,
    uint32_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out, uint32_t* __restrict__ count_out,
    const uint2* __restrict__ val_rect, uint2* __restrict__ rect_out, uint32_t* __restrict__ counts_out) {
  __shared__ uint32_t s_keys[kSortTile];
  __shared__ uint32_t s_vals[kSortTile];
  __shared__ uint32_t s_whist[kSortThreads / 64][kRadix];   // per-wave digit counts, then starts
  __shared__ uint32_t s_local[kRadix];    // block-local start of each digit
  __shared__ uint32_t s_global[kRadix];   // global start of (digit, this block)
  __shared__ uint32_t s_wtot[kSortThreads / 64];

  const int tid = threadIdx.x, lane = __lane_id(), wave = tid >> 6;
  if (count_out && blockIdx.x == 0 && tid == 0) *count_out = hist_scan[kRadix * nb];
  const uint32_t count = pass_count(in);
  const uint32_t base = blockIdx.x * kSortTile;
  if (base >= count) return;   // uniform per block
  // digit counts of this block and their block-local exclusive prefix
  uint32_t block_total;
  {
    const uint32_t cnt = hist[tid * nb + blockIdx.x];
    s_global[tid] = hist_scan[tid * nb + blockIdx.x];
    uint32_t v = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t t = __shfl_up(v, d, 64);
      if (lane >= d) v += t;
    }
    if (lane == 63) s_wtot[wave] = v;
    __syncthreads();
    uint32_t pre = 0;
    block_total = 0;
    for (int w = 0; w < kSortThreads / 64; ++w) {
      if (w < wave) pre += s_wtot[w];
      block_total += s_wtot[w];
    }
    s_local[tid] = pre + v - cnt;
    for (int w = 0; w < kSortThreads / 64; ++w) s_whist[w][tid] = 0u;
  }
  __syncthreads();
  // Each wave ranks its own 1024 consecutive items, 64 per round, with a wave-private
  // digit histogram: an item's rank among equal digits of its wave is the histogram
  // before its round plus its rank in the round (8 ballots give each lane its peers;
  // CDNA has no match-any).  Waves, rounds and lanes follow the items' order, so the
  // placement is stable.
  constexpr int kWaveItems = kSortTile / (kSortThreads / 64);
  constexpr int kRounds = kWaveItems / 64;
  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  uint32_t key[kRounds], val[kRounds], rk[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    key[r] = 0u;
    val[r] = 0u;
    const bool valid = load_item<SRC>(in, count, base + wave * kWaveItems + r * 64 + lane, key[r], val[r]);
    const uint32_t d = (key[r] >> shift) & 0xffu;
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (d >> b) & 1u;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const uint32_t before = valid ? s_whist[wave][d] : 0u;
    const uint32_t rank = __popcll(peers & lt_mask);
    // the read above is issued before this write, and one wave's LDS operations are
    // performed in order
    if (valid && rank == 0) s_whist[wave][d] = before + uint32_t(__popcll(peers));
    rk[r] = valid ? before + rank : 0xffffffffu;
  }
  __syncthreads();
  // per digit, the start of each wave's run: block-local start plus the earlier waves
  {
    uint32_t acc = s_local[tid];
#pragma unroll
    for (int w = 0; w < kSortThreads / 64; ++w) {
      const uint32_t t = s_whist[w][tid];
      s_whist[w][tid] = acc;
      acc += t;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    if (rk[r] != 0xffffffffu) {
      const uint32_t pos = s_whist[wave][(key[r] >> shift) & 0xffu] + rk[r];
      s_keys[pos] = key[r];
      s_vals[pos] = val[r];
    }
  }
  __syncthreads();
  for (uint32_t k = tid; k < block_total; k += kSortThreads) {
    const uint32_t key = s_keys[k];
    const uint32_t d = (key >> shift) & 0xffu;
    const uint32_t dst = s_global[d] + (k - s_local[d]);
    keys_out[dst] = key;
    vals_out[dst] = s_vals[k];
    if (rect_out) {
      const uint2 r = val_rect[s_vals[k]];
      rect_out[dst] = r;
      counts_out[dst] = ((r.y & 0xffffu) - (r.x & 0xffffu) + 1u) * ((r.y >> 16) - (r.x >> 16) + 1u);
    }
  }
}

// For every block of 256 pairs, the visible Gaussian (in depth order) that owns its
// first pair: Gaussian r owns pairs [offs[r], offs[r + 1]) and marks the blocks
// whose first pair falls there.  One thread per Gaussian.
__global__ void __launch_bounds__(256) block_starts_kernel(const uint32_t* __restrict__ offs,
                                                            const uint32_t* __restrict__ n_vis, int n,
                                                            uint32_t pairs, uint32_t* __restrict__ block_first) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n || uint32_t(r) >= *n_vis) return;
  const uint32_t b0 = (offs[r] + 255u) >> 8, e = min(offs[r + 1], pairs);
  for (uint32_t b = b0; (b << 8) < e; ++b) block_first[b] = uint32_t(r);
}

// One thread per pair: the Gaussian (in depth order) that owns it, and its tile.
// offs[r] is the first pair of the r-th visible Gaussian in depth order and
// rect_order[r] its tile rectangle.  The block's 256 pairs belong to at most 256
// consecutive Gaussians starting with block_first[block]; their offsets go to LDS
// and each thread searches there.
__global__ void __launch_bounds__(256) emit_pairs_kernel(const uint32_t* __restrict__ offs,
                                                          const uint32_t* __restrict__ n_vis,
                                                          const uint32_t* __restrict__ block_first,
                                                          const uint32_t* __restrict__ order,
                                                          const uint2* __restrict__ rect_order, int n, uint32_t pairs,
                                                          int tx, uint32_t* __restrict__ keys,
                                                          uint32_t* __restrict__ vals) {
  __shared__ uint32_t s_offs[256];
  const uint32_t p0 = blockIdx.x * 256u;
  const int nv = int(*n_vis);
  const uint32_t bf = block_first[blockIdx.x];
  const int r0 = int(bf < uint32_t(nv) ? bf : uint32_t(max(nv - 1, 0)));
  // Gaussians past the visible ones (or past the block) get an offset above every pair
  const int k = min(256, nv - r0);
  s_offs[threadIdx.x] = int(threadIdx.x) < k ? offs[r0 + int(threadIdx.x)] : 0xffffffffu;
  __syncthreads();
  const uint32_t p = p0 + threadIdx.x;
  if (p >= pairs) return;
  int lo = 0, hi = max(k, 1) - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_offs[mid] <= p) lo = mid; else hi = mid - 1;
  }
  const uint32_t g = order[r0 + lo];
  if (g >= uint32_t(n)) {   // only if total_pairs disagrees with the projection
    keys[p] = 0xffffffffu;
    vals[p] = 0u;
    return;
  }
  const uint32_t j = p - s_offs[lo];
  const uint2 r = rect_order[r0 + lo];
  const uint32_t x0 = r.x & 0xffffu, y0 = r.x >> 16, x1 = r.y & 0xffffu;
  const uint32_t w = x1 - x0 + 1;
  keys[p] = (y0 + j / w) * uint32_t(tx) + (x0 + j % w);
  vals[p] = g;
}

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int64_t count, uint32_t value) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < count) p[i] = value;
}

// Zero fill with 16-byte stores; p 16-byte aligned.
__global__ void zero_u32x4_kernel(uint4* __restrict__ p, int64_t count4) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < count4) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

void zero_u32(uint32_t* p, int64_t count, hipStream_t s) {
  if (count <= 0) return;
  GSK_PROF("fill_u32", s);
  const int64_t c4 = reinterpret_cast<uintptr_t>(p) % 16 == 0 ? count / 4 : 0;
  if (c4 > 0) zero_u32x4_kernel<<<div_up(c4, 256), 256, 0, s>>>(reinterpret_cast<uint4*>(p), c4);
  if (count > 4 * c4) fill_u32_kernel<<<div_up(count - 4 * c4, 256), 256, 0, s>>>(p + 4 * c4, count - 4 * c4, 0u);
}

// Four consecutive pairs per thread (one 16-byte load when the keys are 16-byte
// aligned); a pair whose tile differs from its left neighbour starts that tile's
// range, one whose tile differs from its right neighbour ends it.
__global__ void __launch_bounds__(256) tile_ranges_kernel(const uint32_t* __restrict__ tile_of_pair, uint32_t pairs,
                                                           int num_tiles, uint32_t* __restrict__ ranges,
                                                           bool aligned) {
  const uint32_t i0 = 4u * (blockIdx.x * blockDim.x + threadIdx.x);
  if (i0 >= pairs) return;
  uint32_t t[4];
  if (aligned && i0 + 3 < pairs) {
    const uint4 q = reinterpret_cast<const uint4*>(tile_of_pair)[i0 / 4];
    t[0] = q.x; t[1] = q.y; t[2] = q.z; t[3] = q.w;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) t[k] = i0 + k < pairs ? tile_of_pair[i0 + k] : 0u;
  }
  const uint32_t left = i0 > 0 ? tile_of_pair[i0 - 1] : 0u;
  const uint32_t right = i0 + 4 < pairs ? tile_of_pair[i0 + 4] : 0u;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t i = i0 + k;
    if (i >= pairs) break;
    const uint32_t tk = t[k];
    if (tk >= uint32_t(num_tiles)) continue;   // only if total_pairs disagrees with the tile counts
    const uint32_t l = k == 0 ? left : t[k - 1];
    const uint32_t r = k == 3 ? right : t[k + 1];
    if (i == 0 || l != tk) ranges[tk] = i;
    if (i == pairs - 1 || r != tk) ranges[num_tiles + tk] = i + 1;
  }
}

inline int bits_for(uint32_t max_value) {
  int b = 0;
  while (b < 32 && (uint64_t(max_value) >> b) != 0) ++b;
  return b;
}

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

int blocks_for(int64_t items) { return int(div_up(items > 0 ? items : 1, kSortTile)); }

// Bump allocator over a workspace; with a null base it only measures.
struct Carver {
  char* base;
  size_t off = 0;
  uint32_t* take(size_t bytes) {
    char* r = base ? base + off : nullptr;
    off += align256(bytes);
    return reinterpret_cast<uint32_t*>(r);
  }
};

struct RadixWs {
  uint32_t *hist, *hist_scan;   // kRadix * nb (+ 1)
  uint64_t* total64;
  void* scan_ws;
};

RadixWs carve_radix(Carver& c, int nb, int64_t also_scan) {
  const int64_t hist_n = int64_t(kRadix) * nb;
  RadixWs w;
  w.hist = c.take(size_t(hist_n) * 4);
  w.hist_scan = c.take(size_t(hist_n + 1) * 4);
  w.total64 = reinterpret_cast<uint64_t*>(c.take(8));
  w.scan_ws = c.take(scan_ws_bytes(std::max<int64_t>(hist_n, also_scan)));
  return w;
}

struct DepthWs {
  uint32_t *dk[2], *dv;         // ping-pong with proj.order, n each
  uint32_t* counts;             // n: tile counts in depth order
  RadixWs r;
};

size_t carve_depth(void* ws, int64_t n, DepthWs* out) {
  Carver c{static_cast<char*>(ws)};
  DepthWs w;
  const size_t sn = size_t(n) * 4;
  w.dk[0] = c.take(sn);
  w.dk[1] = c.take(sn);
  w.dv = c.take(sn);
  w.counts = c.take(sn);
  w.r = carve_radix(c, blocks_for(n), n);
  if (out) *out = w;
  return c.off;
}

struct PairWs {
  uint32_t *keys_alt, *vals_alt;   // pairs each
  uint32_t* block_first;           // one per 256 pairs
  RadixWs r;
};

size_t carve_pairs(void* ws, uint32_t pairs, PairWs* out) {
  Carver c{static_cast<char*>(ws)};
  PairWs w;
  w.keys_alt = c.take(size_t(pairs) * 4);
  w.vals_alt = c.take(size_t(pairs) * 4);
  w.block_first = c.take(size_t(div_up(pairs > 0 ? pairs : 1, 256)) * 4);
  w.r = carve_radix(c, blocks_for(pairs), 0);
  if (out) *out = w;
  return c.off;
}

template <int SRC>
hipError_t radix_pass(const PassIn& in, int nb, int shift, const RadixWs& w, uint32_t* keys_out,
                      uint32_t* vals_out, uint32_t* count_out, const uint2* val_rect, uint2* rect_out,
                      uint32_t* counts_out, hipStream_t s) {
  {
    GSK_PROF("radix_upsweep", s);
    radix_upsweep_kernel<SRC><<<nb, kSortThreads, 0, s>>>(in, shift, nb, w.hist);
  }
  hipError_t e = launch_scan_u32(w.hist, w.hist_scan, int64_t(kRadix) * nb, w.total64, w.scan_ws, s);
  if (e != hipSuccess) return e;
  GSK_PROF("radix_downsweep", s);
  radix_downsweep_kernel<SRC><<<nb, kSortThreads, 0, s>>>(in, shift, nb, w.hist, w.hist_scan, keys_out, vals_out,
                                                          count_out, val_rect, rect_out, counts_out);
  return hipGetLastError();
}

}  // namespace

size_t depth_order_ws_bytes(int64_t n) { return carve_depth(nullptr, n, nullptr); }

hipError_t launch_depth_order(const gs_proj& proj, int n, void* ws, hipStream_t s) {
  if (n == 0) {
    GSK_PROF("fill_u32", s);
    fill_u32_kernel<<<1, 256, 0, s>>>(proj.offs, 1, 0u);
    fill_u32_kernel<<<1, 256, 0, s>>>(proj.n_visible, 1, 0u);
    return hipGetLastError();
  }
  DepthWs w;
  carve_depth(ws, n, &w);
  hipError_t e;
  const int nb = blocks_for(n);
  zero_u32(w.counts, n, s);
  // pass 0 compacts the visible Gaussians into (dk[0], dv); later passes alternate
  // with (dk[1], order), so the fourth lands in proj.order
  {
    PassIn in{nullptr, nullptr, proj.depth, proj.tiles, uint32_t(n), nullptr};
    if ((e = radix_pass<kFromDepth>(in, nb, 0, w.r, w.dk[0], w.dv, proj.n_visible, nullptr, nullptr, nullptr,
                                    s)) != hipSuccess)
      return e;
  }
  for (int pass = 1; pass < kDepthPasses; ++pass) {
    const bool odd = pass & 1;
    PassIn in{odd ? w.dk[0] : w.dk[1], odd ? w.dv : proj.order, nullptr, nullptr, 0u, proj.n_visible};
    const bool last = pass == kDepthPasses - 1;
    if ((e = radix_pass<kFromKeys>(in, nb, 8 * pass, w.r, odd ? w.dk[1] : w.dk[0], odd ? proj.order : w.dv,
                                   nullptr, last ? reinterpret_cast<const uint2*>(proj.rect) : nullptr,
                                   last ? reinterpret_cast<uint2*>(proj.rect_order) : nullptr,
                                   last ? w.counts : nullptr, s)) != hipSuccess)
      return e;
  }
  // offs: first pair of each visible Gaussian in depth order; offs[n] = the pair count
  return launch_scan_u32(w.counts, proj.offs, n, w.r.total64, w.r.scan_ws, s);
}

size_t sort_pairs_ws_bytes(int64_t n) {
  Carver c{nullptr};
  c.take(size_t(n > 0 ? n : 1) * 4);
  c.take(size_t(n > 0 ? n : 1) * 4);
  carve_radix(c, blocks_for(n), 0);
  return c.off;
}

hipError_t launch_sort_pairs_u32(uint32_t* keys, uint32_t* vals, uint32_t count, int64_t capacity, void* ws,
                                 hipStream_t s) {
  if (count <= 1) return hipSuccess;
  Carver c{static_cast<char*>(ws)};
  uint32_t* alt_k = c.take(size_t(capacity) * 4);
  uint32_t* alt_v = c.take(size_t(capacity) * 4);
  const RadixWs r = carve_radix(c, blocks_for(capacity), 0);
  const int nb = blocks_for(count);
  // four 8-bit passes: keys -> alt -> keys -> alt -> keys
  for (int pass = 0; pass < 4; ++pass) {
    const bool even = (pass & 1) == 0;
    PassIn in{even ? keys : alt_k, even ? vals : alt_v, nullptr, nullptr, count, nullptr};
    const hipError_t e = radix_pass<kFromKeys>(in, nb, 8 * pass, r, even ? alt_k : keys, even ? alt_v : vals, nullptr,
                                               nullptr, nullptr, nullptr, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

size_t bin_sort_ws_bytes(uint32_t pairs) { return carve_pairs(nullptr, pairs, nullptr); }

hipError_t launch_bin_sort(const gs_proj& proj, int n, const gs_camera& cam, uint32_t pairs, uint32_t* keys,
                           uint32_t* vals, uint32_t* ranges, void* ws, hipStream_t s) {
  const int tx = tiles_x(cam), ty = tiles_y(cam);
  const int num_tiles = tx * ty;
  {
    GSK_PROF("fill_u32", s);
    fill_u32_kernel<<<div_up(2 * int64_t(num_tiles), 256), 256, 0, s>>>(ranges, 2 * int64_t(num_tiles), 0u);
  }
  if (pairs == 0) return hipGetLastError();
  PairWs w;
  carve_pairs(ws, pairs, &w);
  hipError_t e;
  const int tile_passes = (bits_for(uint32_t(num_tiles - 1)) + 7) / 8;
  // emit into the buffer that makes the last tile pass land in keys / vals
  uint32_t* k_src = (tile_passes & 1) ? w.keys_alt : keys;
  uint32_t* v_src = (tile_passes & 1) ? w.vals_alt : vals;
  uint32_t* k_dst = (tile_passes & 1) ? keys : w.keys_alt;
  uint32_t* v_dst = (tile_passes & 1) ? vals : w.vals_alt;
  {
    GSK_PROF("block_starts", s);
    block_starts_kernel<<<div_up(n, 256), 256, 0, s>>>(proj.offs, proj.n_visible, n, pairs, w.block_first);
  }
  {
    GSK_PROF("emit_pairs", s);
    emit_pairs_kernel<<<div_up(pairs, 256), 256, 0, s>>>(proj.offs, proj.n_visible, w.block_first, proj.order,
                                                         reinterpret_cast<const uint2*>(proj.rect_order), n, pairs,
                                                         tx, k_src, v_src);
  }
  // stable sort of the pairs by tile
  const int nbp = blocks_for(pairs);
  for (int pass = 0; pass < tile_passes; ++pass) {
    PassIn in{k_src, v_src, nullptr, nullptr, pairs, nullptr};
    if ((e = radix_pass<kFromKeys>(in, nbp, 8 * pass, w.r, k_dst, v_dst, nullptr, nullptr, nullptr, nullptr, s)) !=
        hipSuccess)
      return e;
    uint32_t* tk = k_src; k_src = k_dst; k_dst = tk;
    uint32_t* tv = v_src; v_src = v_dst; v_dst = tv;
  }
  {
    GSK_PROF("tile_ranges", s);
    tile_ranges_kernel<<<div_up(div_up(pairs, 4), 256), 256, 0, s>>>(
        keys, pairs, num_tiles, ranges, reinterpret_cast<uintptr_t>(keys) % 16 == 0);
  }
  return hipGetLastError();
}

}  // namespace gsk
