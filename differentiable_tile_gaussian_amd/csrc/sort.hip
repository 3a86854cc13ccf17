// Binning and depth sort ([GSG] "Why tiling, and the five stages": scatter, sort,
// segment boundaries; ties broken by Gaussian id).  The pairs end up ordered by
// tile, then depth, then Gaussian id, built in three steps:
//
//   depth sort    the visible Gaussians (tile count > 0), in id order, are sorted by
//                 d = bits(depth) - bits(znear) with a stable LSD radix sort: positive
//                 floats order as their bit patterns, and every visible depth exceeds
//                 znear > 0, so d orders the depths and is below 2^31.  The first pass
//                 also compacts the visible Gaussians and takes the maximum of d.  Three
//                 9-bit passes cover d < 2^27 (depths up to 2^27 ulps above znear:
//                 about 13000 at znear 0.2); a fourth runs only when some d is larger,
//                 its launches returning at once otherwise.  The device picks every
//                 pass's buffers from that count, so that the last pass lands in the
//                 order array; it also gathers each Gaussian's tile rectangle and count.
//   emit          their tile counts, in that order, are prefix-summed; the pairs are
//                 written in blocks of consecutive pairs, (tile id, Gaussian id) for the
//                 tiles of each Gaussian's rectangle: the pairs of each Gaussian are
//                 consecutive and the Gaussians are in (depth, id) order.
//   tile sort     a stable LSD radix sort of the pairs by tile id (its bits split evenly
//                 over the passes), so within a tile they keep the (depth, id) order.
//   tile_ranges   first / one-past-last pair of each tile, by a 64-ary search per tile.
//
// Radix passes use digits of up to 9 bits, reduce-then-scan:
//   upsweep   per-block digit histogram (LDS atomics; for tile digits, which crowd, one
//             atomic per distinct digit of a wave) into a [digits][blocks] table (blocks in an
//             XCD-aware order, below; rows for the pass's 2^bits digits only)
//   scan      per digit, exclusive prefix along its row and the row total, a row taken in
//             segments of 2048 blocks, one scan block each (the carry summed directly)
//   downsweep the digit bases from the row totals; each wave ranks its 1024
//             consecutive items against a wave-private digit histogram (64-lane ballots:
//             no match-any on CDNA, one ballot per digit bit gives each lane its peer
//             mask), one barrier turns the four histograms into run starts, then a local
//             reorder through LDS and a coalesced scatter.
// Sorting the Gaussians by depth once, instead of every pair by a 64-bit (tile, depth)
// key, replaces six passes over 12-byte pairs by three passes over the visible
// Gaussians (about 40 % of them at the orbit cameras) and two over 8-byte pairs.
#include <algorithm>
#include <cstring>

#include "gs_internal.h"
#include "profile.h"

namespace gsk {
namespace {

constexpr int kSortThreads = 256;
constexpr int kWaves = kSortThreads / 64;
constexpr int kSortItems = 16;
constexpr int kSortTile = kSortThreads * kSortItems;   // 4096 items per block
constexpr int kDigitBits = 9;
constexpr int kRadix = 1 << kDigitBits;                 // 512 digits
constexpr int kDepthPasses = 3;                         // always made: d < 2^27
constexpr int kDepthPassesMax = 4;                      // 36 bits >= the 31 of d

// The histogram tables hold one count per (digit, block) in an XCD-aware order.  Blocks
// are handed to the chip's 8 XCDs in turn (block b on XCD b % 8), each XCD with its own
// L2; a digit's entries of the 16 blocks b, b + 8, ..., b + 120 that share an XCD fill one
// 64-byte line, so the blocks' scattered 4-byte writes and reads of a digit meet in that
// L2 instead of each taking a line of HBM traffic.  Blocks go in groups of 128: a group
// holds, per digit, 128 entries, block 128 g + 8 k + x at position 16 x + k.
constexpr int kHistGroup = 128;
// The scan takes a row kScanStepGroups groups (kScanPer entries per thread) per block.
constexpr int kScanPer = 8;
constexpr int kScanStepGroups = kScanPer * kSortThreads / kHistGroup;   // 16
__host__ __device__ inline size_t hist_at(uint32_t d, uint32_t b) {
  const uint32_t g = b / kHistGroup, w = b % kHistGroup;
  return (size_t(g) * kRadix + d) * kHistGroup + (w % 8u) * 16u + w / 8u;
}
inline size_t hist_entries(int nb) { return size_t((nb + kHistGroup - 1) / kHistGroup) * kRadix * kHistGroup; }

// Where a radix pass reads its items from.
enum Source {
  kFromKeys = 0,      // keys[idx], vals[idx], idx < count (count on the device if count_dev)
  kFromDepth = 1      // d of Gaussian idx, value idx; only Gaussians with tiles[idx] > 0
};

struct PassIn {
  const uint32_t* keys;
  const uint32_t* vals;
  const float* depth;
  const uint32_t* tiles;
  uint32_t key_base;   // kFromDepth: the bits of znear
  uint32_t count;
  const uint32_t* count_dev;
};

// The depth sort's passes: pass p of np (3, or 4 when *dmax >= 2^27) writes buffer set
// (np - 1 - p) even ? 1 : 0 and reads the other set (p >= 1), so the last pass writes
// set 1, whose values array is the order array.  pass < 0: an ordinary pass with fixed
// buffers.
struct DepthPlan {
  uint32_t* k[2];
  uint32_t* v[2];
  uint32_t* bmax;   // pass 0: each block's maximum of d (0 without visible Gaussians)
  uint32_t* dmax;   // their maximum, stored by the first pass's scan
  int pass;
};

constexpr DepthPlan kNoPlan{{nullptr, nullptr}, {nullptr, nullptr}, nullptr, nullptr, -1};

__device__ inline int depth_passes(const DepthPlan& dp) {
  return (*dp.dmax >> (kDepthPasses * kDigitBits)) != 0u ? kDepthPassesMax : kDepthPasses;
}
// Uniform per launch: whether this pass has anything to do.
__device__ inline bool pass_runs(const DepthPlan& dp) { return dp.pass < kDepthPasses || dp.pass < depth_passes(dp); }
__device__ inline int plan_dst(const DepthPlan& dp) { return ((depth_passes(dp) - 1 - dp.pass) & 1) == 0 ? 1 : 0; }
// A depth pass after the first reads the set the pass before it wrote.
__device__ inline void plan_source(PassIn& in, const DepthPlan& dp) {
  if (dp.pass > 0) {
    const int src = 1 - plan_dst(dp);
    in.keys = dp.k[src];
    in.vals = dp.v[src];
  }
}

// Item idx of a pass (idx < count, count >= 1).  Loads are unconditional so that a
// thread's loads of several items are in flight together; returns whether the item
// takes part (kFromDepth: the Gaussian is visible).
template <int SRC>
__device__ inline bool load_item(const PassIn& in, uint32_t idx, uint32_t& key, uint32_t& val) {
  if (SRC == kFromDepth) {
    const uint32_t t = in.tiles[idx];
    const uint32_t b = __float_as_uint(in.depth[idx]);
    key = b > in.key_base ? b - in.key_base : 0u;
    val = idx;
    return t != 0u;
  } else {
    key = in.keys[idx];
    val = in.vals[idx];
    return true;
  }
}

__device__ inline uint32_t pass_count(const PassIn& in) { return in.count_dev ? *in.count_dev : in.count; }

// Exclusive prefix across the block of two independent per-thread values; the block
// totals go to tx, ty.  s: 2 * kWaves entries.
__device__ inline uint2 block_scan2(uint32_t x, uint32_t y, uint32_t* s, uint32_t& tx, uint32_t& ty) {
  const int lane = __lane_id(), wave = threadIdx.x >> 6;
  uint32_t ix = x, iy = y;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t a = __shfl_up(ix, d, 64), b = __shfl_up(iy, d, 64);
    if (lane >= d) {
      ix += a;
      iy += b;
    }
  }
  if (lane == 63) {
    s[wave] = ix;
    s[kWaves + wave] = iy;
  }
  __syncthreads();
  uint32_t px = 0, py = 0;
  tx = 0;
  ty = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (w < wave) {
      px += s[w];
      py += s[kWaves + w];
    }
    tx += s[w];
    ty += s[kWaves + w];
  }
  __syncthreads();   // s may be written again after this
  return make_uint2(px + ix - x, py + iy - y);
}

template <int SRC>
__global__ void __launch_bounds__(kSortThreads) radix_upsweep_kernel(PassIn in, DepthPlan dp, int shift, uint32_t mask,
                                                                      int nb, uint32_t* __restrict__ hist) {
  __shared__ uint32_t s_hist[kRadix];
  if (!pass_runs(dp)) return;
  plan_source(in, dp);
  for (int d = threadIdx.x; d < kRadix; d += kSortThreads) s_hist[d] = 0u;
  __syncthreads();
  const uint32_t count = pass_count(in);
  const uint32_t base = blockIdx.x * kSortTile;
  uint32_t kmax = 0u;
  if (base < count) {
    uint32_t key[kSortItems];
    bool ok[kSortItems];
#pragma unroll
    for (int k = 0; k < kSortItems; ++k) {
      const uint32_t idx = base + k * kSortThreads + threadIdx.x;
      uint32_t val;
      ok[k] = load_item<SRC>(in, min(idx, count - 1), key[k], val) && idx < count;
    }
    if (dp.pass >= 0) {
      // depth digits are spread: one LDS atomic per item
#pragma unroll
      for (int k = 0; k < kSortItems; ++k) {
        if (ok[k]) {
          atomicAdd(&s_hist[(key[k] >> shift) & mask], 1u);
          kmax = max(kmax, key[k]);
        }
      }
    } else {
      // tile digits crowd (a block's pairs come from few screen regions): one LDS atomic
      // per distinct digit of a wave's 64 items (a ballot per digit bit gives each lane
      // its peers; the lowest lane adds their number)
      const uint64_t lt_mask = (uint64_t(1) << __lane_id()) - 1;
      const int nbits = __popc(mask);
#pragma unroll
      for (int k = 0; k < kSortItems; ++k) {
        const uint32_t d = (key[k] >> shift) & mask;
        uint64_t peers = __ballot(ok[k]);
        for (int b = 0; b < nbits; ++b) {
          const bool bit = (d >> b) & 1u;
          const uint64_t m = __ballot(bit);
          peers &= bit ? m : ~m;
        }
        if (ok[k] && (peers & lt_mask) == 0) atomicAdd(&s_hist[d], uint32_t(__popcll(peers)));
      }
    }
  }
  if (SRC == kFromDepth) {
    __shared__ uint32_t s_max[kWaves];
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) kmax = max(kmax, uint32_t(__shfl_xor(kmax, d, 64)));
    if (__lane_id() == 0) s_max[threadIdx.x >> 6] = kmax;
    __syncthreads();
    if (threadIdx.x == 0) dp.bmax[blockIdx.x] = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
  }
  __syncthreads();
  // only the pass's digits have rows (a tile pass of 6 bits uses 64 of them)
  for (int d = threadIdx.x; d <= int(mask); d += kSortThreads) hist[hist_at(d, blockIdx.x)] = s_hist[d];
}

// Blocks (digit d, segment s): hist_scan[d][b] = sum of hist[d][b'] over b' < b, rowtot[d]
// the row sum.  A row is cut into segments of kScanStepGroups groups (2048 blocks), one block
// each: the block sums the row's complete groups before its segment, then takes the segment
// in one step (eight entries per thread): loaded in table order (coalesced), put in block
// order through LDS, scanned, and written back in table order; the last segment's block
// stores the row sum.  In the depth sort's first pass, block (0, 0) also reduces the blocks'
// maxima of d.
__global__ void __launch_bounds__(kSortThreads) radix_scan_kernel(DepthPlan dp, int nb,
                                                                   const uint32_t* __restrict__ hist,
                                                                   uint32_t* __restrict__ hist_scan,
                                                                   uint32_t* __restrict__ rowtot) {
  constexpr int kPer = kScanPer;
  constexpr int kStepGroups = kScanStepGroups;
  constexpr int kChunk = kStepGroups * kHistGroup;          // blocks per step
  __shared__ uint32_t s_scan[2 * kWaves];
  __shared__ uint32_t s_v[kChunk];
  if (!pass_runs(dp)) return;
  const int tid = threadIdx.x;
  if (dp.pass == 0 && blockIdx.x == 0 && blockIdx.y == 0) {
    uint32_t m = 0u;
    for (int b = tid; b < nb; b += kSortThreads) m = max(m, dp.bmax[b]);
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) m = max(m, uint32_t(__shfl_xor(m, d, 64)));
    if (__lane_id() == 0) s_scan[tid >> 6] = m;
    __syncthreads();
    if (tid == 0) *dp.dmax = max(max(s_scan[0], s_scan[1]), max(s_scan[2], s_scan[3]));
    __syncthreads();
  }
  const uint32_t d = blockIdx.x;
  const int groups = (nb + kHistGroup - 1) / kHistGroup;
  const int g_begin = int(blockIdx.y) * kStepGroups, g_end = min(groups, g_begin + kStepGroups);
  // carry: the row's sum over the groups before the segment (whole groups: only the last
  // group of a row can hold padding past nb, and it is in the last segment)
  uint32_t carry = 0u;
  if (g_begin > 0) {
    uint32_t part = 0u;
    const size_t row = size_t(d) * kHistGroup;
#pragma unroll 8
    for (int idx = tid; idx < g_begin * kHistGroup; idx += kSortThreads)
      part += hist[size_t(idx / kHistGroup) * kRadix * kHistGroup + row + size_t(idx % kHistGroup)];
    uint32_t unused;
    block_scan2(part, 0u, s_scan, carry, unused);
  }
  for (int g0 = g_begin; g0 < g_end; g0 += kStepGroups) {
    // table position j (group g0 + j / 128, place j % 128) holds block 128 (g0 + j / 128)
    // + 8 (place % 16) + place / 16; b0 = that block less 128 g0
    size_t at[kPer];
    uint32_t b0[kPer];
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int j = tid + kSortThreads * k, g = g0 + j / kHistGroup, place = j % kHistGroup;
      b0[k] = uint32_t(j / kHistGroup) * kHistGroup + uint32_t(place % 16) * 8u + uint32_t(place / 16);
      at[k] = (size_t(g) * kRadix + d) * kHistGroup + size_t(place);
      // blocks past nb (the last group's padding, never written) count 0
      s_v[b0[k]] = uint32_t(g0) * kHistGroup + b0[k] < uint32_t(nb) ? hist[at[k]] : 0u;
    }
    __syncthreads();
    uint32_t v[kPer], sum = 0u;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      v[k] = s_v[kPer * tid + k];
      sum += v[k];
    }
    uint32_t total, unused;
    uint32_t run = carry + block_scan2(sum, 0u, s_scan, total, unused).x;   // (its barriers order s_v)
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      s_v[kPer * tid + k] = run;
      run += v[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (uint32_t(g0) * kHistGroup + b0[k] < uint32_t(nb)) hist_scan[at[k]] = s_v[b0[k]];
    carry += total;
    __syncthreads();   // s_v is loaded again
  }
  if (tid == 0 && blockIdx.y == gridDim.y - 1) rowtot[d] = carry;
}

// With count_out, block 0 stores the number of items (for kFromDepth, of visible
// Gaussians).  The depth plan's last pass writes no keys; it looks every value (a
// Gaussian id) up in val_rect and writes the Gaussian's tile rectangle and tile count
// beside it.
template <int SRC>
__global__ void __launch_bounds__(kSortThreads) radix_downsweep_kernel(
    PassIn in, DepthPlan dp, int shift, uint32_t mask, int nb, const uint32_t* __restrict__ hist_scan,
    const uint32_t* __restrict__ rowtot, uint32_t* keys_out, uint32_t* vals_out, uint32_t* __restrict__ count_out,
    const uint2* __restrict__ val_rect, uint2* __restrict__ rect_out, uint32_t* __restrict__ counts_out) {
  __shared__ uint32_t s_keys[kSortTile];
  __shared__ uint32_t s_vals[kSortTile];
  __shared__ uint16_t s_whist[kWaves][kRadix];   // per-wave digit counts, then starts (<= 4096)
  __shared__ uint16_t s_local[kRadix];           // block-local start of each digit
  __shared__ uint32_t s_global[kRadix];          // global start of (digit, this block)
  __shared__ uint32_t s_scan[2 * kWaves];

  if (!pass_runs(dp)) return;
  plan_source(in, dp);
  bool last = false;
  if (dp.pass >= 0) {
    const int dst = plan_dst(dp);
    keys_out = dp.k[dst];
    vals_out = dp.v[dst];
    last = dp.pass == depth_passes(dp) - 1;
  }
  const int tid = threadIdx.x, lane = __lane_id(), wave = tid >> 6;
  const int d0 = 2 * tid;   // this thread's two digits
  // the digit bases: exclusive prefix of the row totals, plus the earlier blocks' counts
  // of the digit (block 0 also stores the number of items)
  {
    // digits above mask have no rows (and no items)
    const bool u0 = uint32_t(d0) <= mask, u1 = uint32_t(d0 + 1) <= mask;
    const uint32_t g0 = u0 ? hist_scan[hist_at(d0, blockIdx.x)] : 0u, g1 = u1 ? hist_scan[hist_at(d0 + 1, blockIdx.x)] : 0u;
    const uint32_t r0 = u0 ? rowtot[d0] : 0u, r1 = u1 ? rowtot[d0 + 1] : 0u;
    uint32_t all_total, unused;
    const uint32_t pre = block_scan2(r0 + r1, 0u, s_scan, all_total, unused).x;
    if (count_out && blockIdx.x == 0 && tid == 0) *count_out = all_total;
    s_global[d0] = pre + g0;
    s_global[d0 + 1] = pre + r0 + g1;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      s_whist[w][d0] = 0;
      s_whist[w][d0 + 1] = 0;
    }
  }
  const uint32_t count = pass_count(in);
  const uint32_t base = blockIdx.x * kSortTile;
  if (base >= count) return;   // uniform per block
  __syncthreads();
  // Each wave ranks its own 1024 consecutive items, 64 per round, with a wave-private
  // digit histogram: an item's rank among equal digits of its wave is the histogram
  // before its round plus its rank in the round (a ballot per digit bit gives each lane its peers;
  // CDNA has no match-any).  Waves, rounds and lanes follow the items' order, so the
  // placement is stable.
  constexpr int kWaveItems = kSortTile / kWaves;
  constexpr int kRounds = kWaveItems / 64;
  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  const int nbits = __popc(mask);
  uint32_t key[kRounds], val[kRounds], rk[kRounds];
  bool ok[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {   // every round's loads before any ranking
    const uint32_t idx = base + wave * kWaveItems + r * 64 + lane;
    ok[r] = load_item<SRC>(in, min(idx, count - 1), key[r], val[r]) && idx < count;
  }
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const bool valid = ok[r];
    const uint32_t d = (key[r] >> shift) & mask;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (d >> b) & 1u;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const uint32_t before = valid ? uint32_t(s_whist[wave][d]) : 0u;
    const uint32_t rank = __popcll(peers & lt_mask);
    // the read above is issued before this write, and one wave's LDS operations are
    // performed in order
    if (valid && rank == 0) s_whist[wave][d] = uint16_t(before + uint32_t(__popcll(peers)));
    rk[r] = valid ? before + rank : 0xffffffffu;
  }
  __syncthreads();
  // the block's count of each digit (summed over the waves) and their block-local prefix
  uint32_t block_total;
  {
    uint32_t c0 = 0u, c1 = 0u;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      c0 += s_whist[w][d0];
      c1 += s_whist[w][d0 + 1];
    }
    uint32_t unused;
    const uint32_t pre = block_scan2(c0 + c1, 0u, s_scan, block_total, unused).x;
    s_local[d0] = uint16_t(pre);
    s_local[d0 + 1] = uint16_t(pre + c0);
  }
  // per digit, the start of each wave's run: block-local start plus the earlier waves
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int d = d0 + j;
    uint32_t acc = s_local[d];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t t = s_whist[w][d];
      s_whist[w][d] = uint16_t(acc);
      acc += t;
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    if (rk[r] != 0xffffffffu) {
      const uint32_t pos = s_whist[wave][(key[r] >> shift) & mask] + rk[r];
      s_keys[pos] = key[r];
      s_vals[pos] = val[r];
    }
  }
  __syncthreads();
  // out in sorted order, sixteen places per thread (the last depth pass's rectangle
  // gathers issued together)
  uint32_t okey[kSortItems], oval[kSortItems], dst[kSortItems];
#pragma unroll
  for (int j = 0; j < kSortItems; ++j) {
    const uint32_t k = tid + j * kSortThreads;
    okey[j] = s_keys[k];
    oval[j] = s_vals[k];
    const uint32_t d = (okey[j] >> shift) & mask;
    dst[j] = s_global[d] + (k - s_local[d]);
  }
  if (last) {
    uint2 rc[kSortItems];
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) rc[j] = val_rect[tid + j * kSortThreads < block_total ? oval[j] : 0u];
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
      if (tid + j * kSortThreads < block_total) {
        vals_out[dst[j]] = oval[j];
        rect_out[dst[j]] = rc[j];
        counts_out[dst[j]] = ((rc[j].y & 0xffffu) - (rc[j].x & 0xffffu) + 1u) * ((rc[j].y >> 16) - (rc[j].x >> 16) + 1u);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kSortItems; ++j) {
      if (tid + j * kSortThreads < block_total) {
        keys_out[dst[j]] = okey[j];
        vals_out[dst[j]] = oval[j];
      }
    }
  }
}

// Pairs of the visible Gaussians in depth order: Gaussian r (its id order[r], its tile
// rectangle rect_order[r]) owns pairs [offs[r], offs[r + 1]) and writes (tile id, id) for
// the tiles of its rectangle in row-major order.  A block writes kEmitPairs consecutive
// pairs: block_first[block] is the Gaussian owning its first pair; the offsets of the
// Gaussians owning its pairs go to LDS (256 at a time, until they pass the block's end);
// each thread finds the owner of its first pair by binary search and walks kEmitPerThread
// consecutive pairs (stepping the rectangle's column and row), staging them in LDS; the
// block then writes them out coalesced.  Pairs past offs[n_vis] (only if total_pairs
// disagrees with the projection) get the tile 0xffffffff.
constexpr int kEmitPerThread = 8;
constexpr int kEmitPairs = 256 * kEmitPerThread;

// block_first[b]: the visible Gaussian that owns pair b * kEmitPairs (the last one for a
// block past offs[n_vis]).  One thread per visible Gaussian.
__global__ void __launch_bounds__(256) block_starts_kernel(const uint32_t* __restrict__ offs,
                                                            const uint32_t* __restrict__ n_vis, int n,
                                                            uint32_t pairs, uint32_t* __restrict__ block_first) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  const int nv = int(*n_vis);
  if (r >= n || r >= nv) return;
  // the last one also owns the blocks past its pairs; no block at or past `pairs` exists
  // (a pair count below the projection's must not write past the array)
  const uint32_t e = r == nv - 1 ? pairs : min(offs[r + 1], pairs);
  for (uint32_t b = (offs[r] + kEmitPairs - 1) / kEmitPairs; b * uint32_t(kEmitPairs) < e; ++b) block_first[b] = uint32_t(r);
}

__global__ void __launch_bounds__(256) emit_pairs_kernel(const uint32_t* __restrict__ offs,
                                                          const uint32_t* __restrict__ n_vis,
                                                          const uint32_t* __restrict__ block_first,
                                                          const uint32_t* __restrict__ order,
                                                          const uint2* __restrict__ rect_order, uint32_t pairs,
                                                          int tx, uint32_t* __restrict__ keys,
                                                          uint32_t* __restrict__ vals) {
  // staged pair q at q + q / 32: a thread's eight consecutive pairs (stride 8 across the
  // wave) then fall at most two to an LDS bank, and the read-out's consecutive ones none
  __shared__ uint32_t s_offs[kEmitPairs + 256];
  __shared__ uint32_t s_key[kEmitPairs + kEmitPairs / 32], s_val[kEmitPairs + kEmitPairs / 32];
  __shared__ uint32_t s_k;
  const int tid = threadIdx.x;
  const uint32_t nv = *n_vis;
  const uint32_t p0 = blockIdx.x * uint32_t(kEmitPairs);
  const uint32_t pend = min(p0 + uint32_t(kEmitPairs), pairs);
  const uint32_t r0 = min(block_first[blockIdx.x], nv);
  // offsets of Gaussians r0, r0 + 1, ... (offs[nv] is the pair count: an end marker)
  uint32_t k = 0;
  for (;;) {
    const uint32_t r = r0 + k + uint32_t(tid);
    const uint32_t o = r <= nv ? offs[r] : 0xffffffffu;
    s_offs[k + tid] = o;
    // the chunk is the last one needed once some loaded offset reaches the block's end
    const int past = __syncthreads_count(o >= pend);
    k += 256;
    if (past > 0 || k >= uint32_t(kEmitPairs)) break;
  }
  if (tid == 0) s_k = k;
  __syncthreads();
  const uint32_t kk = s_k;
  const uint32_t q0 = p0 + uint32_t(tid) * kEmitPerThread;
  if (q0 < pend) {
    // owner of q0: the last i with s_offs[i] <= q0
    uint32_t lo = 0, hi = kk - 1;
    while (lo < hi) {
      const uint32_t mid = (lo + hi + 1) >> 1;
      if (s_offs[mid] <= q0) lo = mid; else hi = mid - 1;
    }
    uint32_t i = lo;
    uint32_t next = i + 1 < kk ? s_offs[i + 1] : 0xffffffffu;
    uint32_t g = 0u, x = 0u, x0 = 0u, x1 = 0u, row = 0u;
    bool valid = false;
    auto owner = [&](uint32_t q) {
      const uint32_t r = r0 + i;
      valid = r < nv;
      if (!valid) return;
      g = order[r];
      const uint2 rc = rect_order[r];
      x0 = rc.x & 0xffffu;
      x1 = rc.y & 0xffffu;
      const uint32_t w = x1 - x0 + 1u, j = q - s_offs[i];
      x = x0 + j % w;
      row = ((rc.x >> 16) + j / w) * uint32_t(tx);
    };
    owner(q0);
#pragma unroll
    for (int m = 0; m < kEmitPerThread; ++m) {
      const uint32_t q = q0 + uint32_t(m);
      if (q >= pend) break;
      if (m > 0) {
        if (q >= next) {   // a new Gaussian starts here (each owns at least one pair)
          ++i;
          next = i + 1 < kk ? s_offs[i + 1] : 0xffffffffu;
          owner(q);
        } else if (++x > x1) {
          x = x0;
          row += uint32_t(tx);
        }
      }
      const uint32_t at = uint32_t(tid * kEmitPerThread + m);
      s_key[at + at / 32u] = valid ? row + x : 0xffffffffu;
      s_val[at + at / 32u] = valid ? g : 0u;
    }
  }
  __syncthreads();
#pragma unroll
  for (int m = 0; m < kEmitPerThread; ++m) {
    const uint32_t at = uint32_t(tid + 256 * m);
    if (p0 + at < pend) {
      keys[p0 + at] = s_key[at + at / 32u];
      vals[p0 + at] = s_val[at + at / 32u];
    }
  }
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

// One wave per tile t, four tiles per block: the first index in the sorted tiles whose
// tile is >= t and the first whose tile is >= t + 1 (pairs if none), both by a 64-ary
// search, one sample per lane per level; the range is (0, 0) when empty.
__global__ void __launch_bounds__(256) tile_ranges_kernel(const uint32_t* __restrict__ tile_of_pair, uint32_t pairs,
                                                           int num_tiles, uint32_t* __restrict__ ranges) {
  const uint32_t t = blockIdx.x * 4u + (threadIdx.x >> 6);
  if (t >= uint32_t(num_tiles)) return;
  const uint32_t lane = __lane_id();
  uint32_t lo[2] = {0u, 0u}, hi[2] = {pairs, pairs};   // each answer lies in [lo, hi]
  while (hi[0] - lo[0] > 64u || hi[1] - lo[1] > 64u) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      if (hi[b] - lo[b] <= 64u) continue;   // uniform per wave
      const uint32_t step = (hi[b] - lo[b] + 63u) / 64u;
      const uint32_t at = lo[b] + lane * step;
      const uint32_t c = __popcll(__ballot(at < hi[b] && tile_of_pair[at] < t + uint32_t(b)));
      if (c > 0) {
        const uint32_t nlo = lo[b] + (c - 1u) * step + 1u;
        hi[b] = min(hi[b], lo[b] + c * step);
        lo[b] = nlo;
      } else {
        hi[b] = lo[b];
      }
    }
  }
  uint32_t e[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const uint32_t at = lo[b] + lane;
    e[b] = lo[b] + uint32_t(__popcll(__ballot(at < hi[b] && tile_of_pair[at] < t + uint32_t(b))));
  }
  if (lane == 0) {
    ranges[t] = e[0] < e[1] ? e[0] : 0u;
    ranges[num_tiles + t] = e[0] < e[1] ? e[1] : 0u;
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
  uint32_t *hist, *hist_scan;   // hist_entries(nb) each
  uint32_t* rowtot;             // kRadix
};

RadixWs carve_radix(Carver& c, int nb) {
  const size_t hist_n = hist_entries(nb);
  RadixWs w;
  w.hist = c.take(hist_n * 4);
  w.hist_scan = c.take(hist_n * 4);
  w.rowtot = c.take(size_t(kRadix) * 4);
  return w;
}

struct DepthWs {
  uint32_t *dk[2], *dv;         // with proj.order: the depth passes' two buffer sets
  uint32_t* counts;             // n: tile counts in depth order (the first n_visible); counts[n]: the plan's dmax
  uint32_t* bmax;               // one per radix block
  uint64_t* total64;            // the offsets scan's total
  void* scan_ws;
  RadixWs r;
};

size_t carve_depth(void* ws, int64_t n, DepthWs* out) {
  Carver c{static_cast<char*>(ws)};
  DepthWs w;
  const size_t sn = size_t(n) * 4;
  w.dk[0] = c.take(sn);
  w.dk[1] = c.take(sn);
  w.dv = c.take(sn);
  w.counts = c.take(sn + 4);
  w.bmax = c.take(size_t(blocks_for(n)) * 4);
  w.total64 = reinterpret_cast<uint64_t*>(c.take(8));
  w.scan_ws = c.take(scan_ws_bytes(n));
  w.r = carve_radix(c, blocks_for(n));
  if (out) *out = w;
  return c.off;
}

struct PairWs {
  uint32_t *keys_alt, *vals_alt;   // pairs each
  uint32_t* block_first;           // one per emit block
  RadixWs r;
};

size_t carve_pairs(void* ws, uint32_t pairs, PairWs* out) {
  Carver c{static_cast<char*>(ws)};
  PairWs w;
  w.keys_alt = c.take(size_t(pairs) * 4);
  w.vals_alt = c.take(size_t(pairs) * 4);
  w.block_first = c.take(size_t(div_up(pairs > 0 ? pairs : 1, kEmitPairs)) * 4);
  w.r = carve_radix(c, blocks_for(pairs));
  if (out) *out = w;
  return c.off;
}

// One radix pass over the bits-wide digit at `shift`.
template <int SRC>
hipError_t radix_pass(const PassIn& in, const DepthPlan& dp, int nb, int shift, int bits, const RadixWs& w,
                      uint32_t* keys_out, uint32_t* vals_out, uint32_t* count_out, const uint2* val_rect,
                      uint2* rect_out, uint32_t* counts_out, hipStream_t s) {
  const uint32_t mask = (1u << bits) - 1u;
  {
    GSK_PROF("radix_upsweep", s);
    radix_upsweep_kernel<SRC><<<nb, kSortThreads, 0, s>>>(in, dp, shift, mask, nb, w.hist);
  }
  {
    GSK_PROF("radix_scan", s);
    const int segs = std::max(1, int(div_up(div_up(nb, kHistGroup), kScanStepGroups)));
    radix_scan_kernel<<<dim3(int(mask) + 1, segs), kSortThreads, 0, s>>>(dp, nb, w.hist, w.hist_scan, w.rowtot);
  }
  GSK_PROF("radix_downsweep", s);
  radix_downsweep_kernel<SRC><<<nb, kSortThreads, 0, s>>>(in, dp, shift, mask, nb, w.hist_scan, w.rowtot, keys_out,
                                                          vals_out, count_out, val_rect, rect_out, counts_out);
  return hipGetLastError();
}

}  // namespace

size_t depth_order_ws_bytes(int64_t n) { return carve_depth(nullptr, n, nullptr); }

hipError_t launch_depth_order(const gs_proj& proj, int n, float znear, void* ws, hipStream_t s) {
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
  uint32_t key_base;
  std::memcpy(&key_base, &znear, sizeof key_base);
  DepthPlan dp{{w.dk[0], w.dk[1]}, {w.dv, proj.order}, w.bmax, w.counts + n, 0};
  const uint2* rect = reinterpret_cast<const uint2*>(proj.rect);
  uint2* rect_order = reinterpret_cast<uint2*>(proj.rect_order);
  // pass 0 compacts the visible Gaussians; the last pass (2 or 3, chosen on the device)
  // lands in proj.order and writes their rectangles and counts in that order
  {
    PassIn in{nullptr, nullptr, proj.depth, proj.tiles, key_base, uint32_t(n), nullptr};
    if ((e = radix_pass<kFromDepth>(in, dp, nb, 0, kDigitBits, w.r, nullptr, nullptr, proj.n_visible, rect,
                                    rect_order, w.counts, s)) != hipSuccess)
      return e;
  }
  for (int pass = 1; pass < kDepthPassesMax; ++pass) {
    dp.pass = pass;
    PassIn in{nullptr, nullptr, nullptr, nullptr, 0u, 0u, proj.n_visible};
    if ((e = radix_pass<kFromKeys>(in, dp, nb, kDigitBits * pass, kDigitBits, w.r, nullptr, nullptr, nullptr,
                                   rect, rect_order, w.counts, s)) != hipSuccess)
      return e;
  }
  // offs: first pair of each visible Gaussian in depth order, offs[n_visible] = the pair
  // count (the scan covers the n_visible counts the last pass wrote)
  return launch_scan_u32(w.counts, proj.offs, n, w.total64, w.scan_ws, s, proj.n_visible);
}

size_t sort_pairs_ws_bytes(int64_t n) {
  Carver c{nullptr};
  c.take(size_t(n > 0 ? n : 1) * 4);
  c.take(size_t(n > 0 ? n : 1) * 4);
  carve_radix(c, blocks_for(n));
  return c.off;
}

hipError_t launch_sort_pairs_u32(uint32_t* keys, uint32_t* vals, uint32_t count, int64_t capacity, void* ws,
                                 hipStream_t s) {
  if (count <= 1) return hipSuccess;
  Carver c{static_cast<char*>(ws)};
  uint32_t* alt_k = c.take(size_t(capacity) * 4);
  uint32_t* alt_v = c.take(size_t(capacity) * 4);
  const RadixWs r = carve_radix(c, blocks_for(capacity));
  const int nb = blocks_for(count);
  // four 9-bit passes: keys -> alt -> keys -> alt -> keys
  for (int pass = 0; pass < 4; ++pass) {
    const bool even = (pass & 1) == 0;
    PassIn in{even ? keys : alt_k, even ? vals : alt_v, nullptr, nullptr, 0u, count, nullptr};
    const hipError_t e = radix_pass<kFromKeys>(in, kNoPlan, nb, kDigitBits * pass, std::min(kDigitBits, 32 - kDigitBits * pass),
                                               r, even ? alt_k : keys, even ? alt_v : vals, nullptr, nullptr,
                                               nullptr, nullptr, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

size_t bin_sort_ws_bytes(uint32_t pairs) { return carve_pairs(nullptr, pairs, nullptr); }

hipError_t launch_bin_sort(const gs_proj& proj, int n, const gs_camera& cam, uint32_t pairs, uint32_t* keys,
                           uint32_t* vals, uint32_t* ranges, void* ws, hipStream_t s) {
  const int tx = tiles_x(cam), ty = tiles_y(cam);
  const int num_tiles = tx * ty;
  if (pairs == 0) {   // every tile empty (with pairs, the range search writes every entry)
    GSK_PROF("fill_u32", s);
    fill_u32_kernel<<<div_up(2 * int64_t(num_tiles), 256), 256, 0, s>>>(ranges, 2 * int64_t(num_tiles), 0u);
    return hipGetLastError();
  }
  PairWs w;
  carve_pairs(ws, pairs, &w);
  hipError_t e;
  // the tile id's bits split evenly over the passes (few distinct values in a digit
  // would crowd the histogram counters)
  const int tile_bits = bits_for(uint32_t(num_tiles - 1));
  const int tile_passes = (tile_bits + kDigitBits - 1) / kDigitBits;
  const int low_bits = tile_passes > 0 ? (tile_bits + tile_passes - 1) / tile_passes : 0;
  // emit into the buffer that makes the last tile pass land in keys / vals
  uint32_t* k_src = (tile_passes & 1) ? w.keys_alt : keys;
  uint32_t* v_src = (tile_passes & 1) ? w.vals_alt : vals;
  uint32_t* k_dst = (tile_passes & 1) ? keys : w.keys_alt;
  uint32_t* v_dst = (tile_passes & 1) ? vals : w.vals_alt;
  const int nbp = blocks_for(pairs);
  const int nbe = int(div_up(pairs, kEmitPairs));
  {
    GSK_PROF("block_starts", s);
    block_starts_kernel<<<div_up(n, 256), 256, 0, s>>>(proj.offs, proj.n_visible, n, pairs, w.block_first);
  }
  {
    GSK_PROF("emit_pairs", s);
    emit_pairs_kernel<<<nbe, 256, 0, s>>>(proj.offs, proj.n_visible, w.block_first, proj.order,
                                          reinterpret_cast<const uint2*>(proj.rect_order), pairs, tx, k_src, v_src);
  }
  // stable sort of the pairs by tile
  for (int pass = 0; pass < tile_passes; ++pass) {
    PassIn in{k_src, v_src, nullptr, nullptr, 0u, pairs, nullptr};
    const int shift = low_bits * pass, bits = std::min(low_bits, tile_bits - shift);
    if ((e = radix_pass<kFromKeys>(in, kNoPlan, nbp, shift, bits, w.r, k_dst, v_dst, nullptr, nullptr, nullptr,
                                   nullptr, s)) != hipSuccess)
      return e;
    uint32_t* tk = k_src; k_src = k_dst; k_dst = tk;
    uint32_t* tv = v_src; v_src = v_dst; v_dst = tv;
  }
  {
    GSK_PROF("tile_ranges", s);
    tile_ranges_kernel<<<div_up(num_tiles, 4), 256, 0, s>>>(keys, pairs, num_tiles, ranges);
  }
  return hipGetLastError();
}

}  // namespace gsk
