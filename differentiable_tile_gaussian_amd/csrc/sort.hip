// Duplicate-with-keys, depth sort and tile ranges ([GSG] "Why tiling, and the
// five stages": scatter, sort, segment boundaries; ties broken by Gaussian id).
//
// emit_keys      one thread per pair: binary search of the pair index in the
//                tile-count prefix sum finds the owning Gaussian, the offset within
//                its rectangle gives the tile (row-major).  Coalesced 12-byte writes.
// radix passes   stable LSD radix sort of (u64 key, u32 value) on the key's
//                significant bits, 8 bits per pass, reduce-then-scan:
//                  upsweep   per-block digit histogram (LDS atomics)
//                  scan      exclusive prefix over the digit-major [256][blocks] table
//                  downsweep stable in-block ranking with 64-lane ballots (no
//                            match-any on CDNA: 8 ballots give each lane its peer mask),
//                            local reorder through LDS, coalesced scatter.
// tile_ranges    first / one-past-last pair of each tile.
#include "gs_internal.h"
#include "profile.h"

namespace gsk {
namespace {

constexpr int kSortThreads = 256;
constexpr int kSortItems = 16;
constexpr int kSortTile = kSortThreads * kSortItems;   // 4096 pairs per block
constexpr int kRadix = 256;

__global__ void __launch_bounds__(256) emit_keys_kernel(const uint32_t* __restrict__ offs, int n,
                                                         const float* __restrict__ depth,
                                                         const uint2* __restrict__ rect, uint32_t pairs, int tx,
                                                         uint64_t* __restrict__ keys, uint32_t* __restrict__ vals) {
  const uint32_t p = blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= pairs) return;
  // largest g with offs[g] <= p (offs is non-decreasing, offs[n] = pairs > p)
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= p) lo = mid; else hi = mid - 1;
  }
  const int g = lo;
  const uint32_t j = p - offs[g];
  const uint2 r = rect[g];
  const uint32_t x0 = r.x & 0xffffu, y0 = r.x >> 16, x1 = r.y & 0xffffu;
  const uint32_t w = x1 - x0 + 1;
  const uint32_t tile = (y0 + j / w) * uint32_t(tx) + (x0 + j % w);
  keys[p] = (uint64_t(tile) << 32) | uint64_t(__float_as_uint(depth[g]));
  vals[p] = uint32_t(g);
}

__global__ void __launch_bounds__(kSortThreads) radix_upsweep_kernel(const uint64_t* __restrict__ keys,
                                                                      uint32_t pairs, int shift, int nb,
                                                                      uint32_t* __restrict__ hist) {
  __shared__ uint32_t s_hist[kRadix];
  s_hist[threadIdx.x] = 0u;
  __syncthreads();
  const uint32_t base = blockIdx.x * kSortTile;
#pragma unroll 4
  for (int k = 0; k < kSortItems; ++k) {
    const uint32_t idx = base + k * kSortThreads + threadIdx.x;
    if (idx < pairs) atomicAdd(&s_hist[uint32_t(keys[idx] >> shift) & 0xffu], 1u);
  }
  __syncthreads();
  hist[threadIdx.x * nb + blockIdx.x] = s_hist[threadIdx.x];
}

__global__ void __launch_bounds__(kSortThreads) radix_downsweep_kernel(
    const uint64_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in, uint32_t pairs, int shift, int nb,
    const uint32_t* __restrict__ hist, const uint32_t* __restrict__ hist_scan, uint64_t* __restrict__ keys_out,
    uint32_t* __restrict__ vals_out) {
  __shared__ uint64_t s_keys[kSortTile];
  __shared__ uint32_t s_vals[kSortTile];
  __shared__ uint32_t s_wave_cnt[kSortThreads / 64][kRadix];
  __shared__ uint32_t s_run[kRadix];      // pairs of each digit already placed in this block
  __shared__ uint32_t s_local[kRadix];    // block-local start of each digit
  __shared__ uint32_t s_global[kRadix];   // global start of (digit, this block)
  __shared__ uint32_t s_wtot[kSortThreads / 64];

  const int tid = threadIdx.x, lane = __lane_id(), wave = tid >> 6;
  const uint32_t base = blockIdx.x * kSortTile;
  // digit counts of this block and their block-local exclusive prefix
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
    for (int w = 0; w < wave; ++w) pre += s_wtot[w];
    s_local[tid] = pre + v - cnt;
    s_run[tid] = 0u;
    for (int w = 0; w < kSortThreads / 64; ++w) s_wave_cnt[w][tid] = 0u;
  }
  __syncthreads();
  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  for (int r = 0; r < kSortItems; ++r) {
    const uint32_t idx = base + r * kSortThreads + tid;
    const bool valid = idx < pairs;
    uint64_t key = 0;
    uint32_t val = 0, d = 0;
    if (valid) {
      key = keys_in[idx];
      val = vals_in[idx];
      d = uint32_t(key >> shift) & 0xffu;
    }
    // lanes of this wave holding the same digit
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (d >> b) & 1u;
      const uint64_t m = __ballot(bit);
      peers &= bit ? m : ~m;
    }
    const uint32_t rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) s_wave_cnt[wave][d] = uint32_t(__popcll(peers));
    __syncthreads();
    if (valid) {
      uint32_t pos = s_local[d] + s_run[d] + rank;
      for (int w = 0; w < wave; ++w) pos += s_wave_cnt[w][d];
      s_keys[pos] = key;
      s_vals[pos] = val;
    }
    __syncthreads();
    {
      uint32_t add = 0;
      for (int w = 0; w < kSortThreads / 64; ++w) {
        add += s_wave_cnt[w][tid];
        s_wave_cnt[w][tid] = 0u;
      }
      s_run[tid] += add;
    }
    __syncthreads();
  }
  const uint32_t count = pairs - base < uint32_t(kSortTile) ? pairs - base : uint32_t(kSortTile);
  for (uint32_t k = tid; k < count; k += kSortThreads) {
    const uint64_t key = s_keys[k];
    const uint32_t d = uint32_t(key >> shift) & 0xffu;
    const uint32_t dst = s_global[d] + (k - s_local[d]);
    keys_out[dst] = key;
    vals_out[dst] = s_vals[k];
  }
}

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int64_t count, uint32_t value) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < count) p[i] = value;
}

__global__ void __launch_bounds__(256) tile_ranges_kernel(const uint64_t* __restrict__ keys, uint32_t pairs,
                                                           int num_tiles, uint32_t* __restrict__ ranges) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= pairs) return;
  const uint32_t t = uint32_t(keys[i] >> 32);
  if (i == 0 || uint32_t(keys[i - 1] >> 32) != t) ranges[t] = i;
  if (i == pairs - 1 || uint32_t(keys[i + 1] >> 32) != t) ranges[num_tiles + t] = i + 1;
}

inline int bits_for(uint32_t max_value) {
  int b = 0;
  while (b < 32 && (uint64_t(max_value) >> b) != 0) ++b;
  return b;
}

struct SortWs {
  uint64_t* keys_alt;
  uint32_t* vals_alt;
  uint32_t* hist;
  uint32_t* hist_scan;
  uint64_t* total64;
  void* scan_ws;
};

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

SortWs carve(void* ws, uint32_t pairs) {
  const int nb = int(div_up(pairs > 0 ? pairs : 1, kSortTile));
  const int64_t hist_n = int64_t(kRadix) * nb;
  char* p = static_cast<char*>(ws);
  SortWs w;
  w.keys_alt = reinterpret_cast<uint64_t*>(p); p += align256(size_t(pairs) * 8);
  w.vals_alt = reinterpret_cast<uint32_t*>(p); p += align256(size_t(pairs) * 4);
  w.hist = reinterpret_cast<uint32_t*>(p); p += align256(size_t(hist_n) * 4);
  w.hist_scan = reinterpret_cast<uint32_t*>(p); p += align256(size_t(hist_n + 1) * 4);
  w.total64 = reinterpret_cast<uint64_t*>(p); p += 256;
  w.scan_ws = p;
  return w;
}

}  // namespace

size_t bin_sort_ws_bytes(uint32_t pairs, int num_tiles) {
  (void)num_tiles;
  const int nb = int(div_up(pairs > 0 ? pairs : 1, kSortTile));
  const int64_t hist_n = int64_t(kRadix) * nb;
  return align256(size_t(pairs) * 8) + align256(size_t(pairs) * 4) + align256(size_t(hist_n) * 4) +
         align256(size_t(hist_n + 1) * 4) + 256 + align256(scan_ws_bytes(hist_n));
}

hipError_t launch_bin_sort(const gs_proj& proj, int n, const gs_camera& cam, uint32_t pairs, uint64_t* keys,
                           uint32_t* vals, uint32_t* ranges, void* ws, hipStream_t s) {
  const int tx = tiles_x(cam), ty = tiles_y(cam);
  const int num_tiles = tx * ty;
  {
    GSK_PROF("fill_u32", s);
    fill_u32_kernel<<<div_up(2 * int64_t(num_tiles), 256), 256, 0, s>>>(ranges, 2 * int64_t(num_tiles), 0u);
  }
  if (pairs == 0) return hipGetLastError();
  SortWs w = carve(ws, pairs);
  // significant key bits: 32 depth bits + enough for the largest tile id
  const int key_bits = 32 + bits_for(uint32_t(num_tiles - 1));
  const int passes = (key_bits + 7) / 8;
  // emit into the buffer that makes the last pass land in keys/vals
  uint64_t* k_src = (passes & 1) ? w.keys_alt : keys;
  uint32_t* v_src = (passes & 1) ? w.vals_alt : vals;
  uint64_t* k_dst = (passes & 1) ? keys : w.keys_alt;
  uint32_t* v_dst = (passes & 1) ? vals : w.vals_alt;
  {
    GSK_PROF("emit_keys", s);
    emit_keys_kernel<<<div_up(pairs, 256), 256, 0, s>>>(proj.offs, n, proj.depth,
                                                        reinterpret_cast<const uint2*>(proj.rect), pairs, tx, k_src,
                                                        v_src);
  }
  const int nb = int(div_up(pairs, kSortTile));
  const int64_t hist_n = int64_t(kRadix) * nb;
  for (int pass = 0; pass < passes; ++pass) {
    const int shift = 8 * pass;
    {
      GSK_PROF("radix_upsweep", s);
      radix_upsweep_kernel<<<nb, kSortThreads, 0, s>>>(k_src, pairs, shift, nb, w.hist);
    }
    hipError_t e = launch_scan_u32(w.hist, w.hist_scan, hist_n, w.total64, w.scan_ws, s);
    if (e != hipSuccess) return e;
    {
      GSK_PROF("radix_downsweep", s);
      radix_downsweep_kernel<<<nb, kSortThreads, 0, s>>>(k_src, v_src, pairs, shift, nb, w.hist, w.hist_scan, k_dst,
                                                         v_dst);
    }
    uint64_t* tk = k_src; k_src = k_dst; k_dst = tk;
    uint32_t* tv = v_src; v_src = v_dst; v_dst = tv;
  }
  {
    GSK_PROF("tile_ranges", s);
    tile_ranges_kernel<<<div_up(pairs, 256), 256, 0, s>>>(keys, pairs, num_tiles, ranges);
  }
  return hipGetLastError();
}

}  // namespace gsk
