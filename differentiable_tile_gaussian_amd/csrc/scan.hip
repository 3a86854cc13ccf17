// Exclusive prefix sum of u32 values (reduce, then apply).  Used for the per-Gaussian
// tile counts ([GSG] "Why tiling, and the five stages": the scan that reserves each
// Gaussian's slot range) and for the radix sort's digit histograms.  No inter-block
// waiting: two plain launches.  The first writes one sum per tile of 2048 values; in
// the second each block adds up the sums of the tiles before its own (a few hundred
// at most here, one or a few per thread) and scans its tile.
#include "gs_internal.h"
#include "profile.h"

namespace gsk {
namespace {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 8;
constexpr int kScanTile = kScanThreads * kScanItems;   // 2048 values per block

__device__ inline uint32_t wave_inclusive_scan(uint32_t v) {
  const int lane = __lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t t = __shfl_up(v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

// Exclusive scan across the 256 threads of a block; returns the prefix of this
// thread and writes the block total to *total.
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t* s_wave, uint32_t* total) {
  const int lane = __lane_id(), wave = threadIdx.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v);
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  uint32_t base = 0, tot = 0;
  for (int w = 0; w < kScanThreads / 64; ++w) {
    if (w < wave) base += s_wave[w];
    tot += s_wave[w];
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// The count scanned: n, or min(n, *n_dev) when the count is on the device.
__device__ inline int64_t scan_count(int64_t n, const uint32_t* n_dev) {
  return n_dev ? min(n, int64_t(*n_dev)) : n;
}

__global__ void __launch_bounds__(kScanThreads) scan_reduce_kernel(const uint32_t* __restrict__ in, int64_t n,
                                                                   const uint32_t* __restrict__ n_dev,
                                                                   uint64_t* __restrict__ block_sums) {
  __shared__ uint32_t s_wave[kScanThreads / 64];
  n = scan_count(n, n_dev);
  const int64_t base = int64_t(blockIdx.x) * kScanTile;
  if (base >= n) return;   // uniform per block
  uint32_t sum = 0;
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    const int64_t idx = base + int64_t(k) * kScanThreads + threadIdx.x;
    if (idx < n) sum += in[idx];
  }
  uint32_t total;
  block_exclusive_scan(sum, s_wave, &total);
  if (threadIdx.x == 0) block_sums[blockIdx.x] = total;
}

__global__ void __launch_bounds__(kScanThreads) scan_apply_kernel(const uint32_t* __restrict__ in, int64_t n,
                                                                  const uint32_t* __restrict__ n_dev,
                                                                  const uint64_t* __restrict__ block_sums,
                                                                  uint32_t* __restrict__ out,
                                                                  uint64_t* __restrict__ total64, bool vec) {
  __shared__ uint32_t s_wave[kScanThreads / 64];
  __shared__ uint64_t s_part[kScanThreads / 64];
  n = scan_count(n, n_dev);
  const int nb = int((n + kScanTile - 1) / kScanTile);   // the blocks with values
  if (nb == 0) {   // nothing to scan: out[0] = 0
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *total64 = 0u;
      out[0] = 0u;
    }
    return;
  }
  if (int(blockIdx.x) >= nb) return;   // uniform per block
  // the sums of the tiles before this one (the last block also adds its own: the total)
  const bool last = int(blockIdx.x) == nb - 1;
  const int upto = last ? nb : int(blockIdx.x);
  uint64_t pre = 0;
  for (int t = threadIdx.x; t < upto; t += kScanThreads) pre += block_sums[t];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) pre += __shfl_xor(pre, d, 64);
  if (__lane_id() == 0) s_part[threadIdx.x >> 6] = pre;
  __syncthreads();
  pre = 0;
#pragma unroll
  for (int w = 0; w < kScanThreads / 64; ++w) pre += s_part[w];
  if (last) {
    if (threadIdx.x == 0) {
      *total64 = pre;
      out[n] = uint32_t(pre);
    }
    pre -= block_sums[nb - 1];
  }
  // thread t owns kScanItems consecutive values of the block's tile
  const int64_t base = int64_t(blockIdx.x) * kScanTile + int64_t(threadIdx.x) * kScanItems;
  // (16-byte loads and stores where the arrays allow them and the values are all there)
  const bool full = vec && base + kScanItems <= n;
  uint32_t v[kScanItems];
  uint32_t sum = 0;
  if (full) {
    const uint4 q0 = reinterpret_cast<const uint4*>(in + base)[0], q1 = reinterpret_cast<const uint4*>(in + base)[1];
    v[0] = q0.x; v[1] = q0.y; v[2] = q0.z; v[3] = q0.w; v[4] = q1.x; v[5] = q1.y; v[6] = q1.z; v[7] = q1.w;
  } else {
#pragma unroll
    for (int k = 0; k < kScanItems; ++k) v[k] = (base + k < n) ? in[base + k] : 0u;
  }
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) sum += v[k];
  uint32_t total;
  uint32_t run = block_exclusive_scan(sum, s_wave, &total) + uint32_t(pre);
  uint32_t o[kScanItems];
#pragma unroll
  for (int k = 0; k < kScanItems; ++k) {
    o[k] = run;
    run += v[k];
  }
  if (full) {
    reinterpret_cast<uint4*>(out + base)[0] = make_uint4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<uint4*>(out + base)[1] = make_uint4(o[4], o[5], o[6], o[7]);
  } else {
#pragma unroll
    for (int k = 0; k < kScanItems; ++k)
      if (base + k < n) out[base + k] = o[k];
  }
}

__global__ void scan_empty_kernel(uint32_t* out, uint64_t* total64) {
  out[0] = 0u;
  *total64 = 0u;
}

}  // namespace

size_t scan_ws_bytes(int64_t n) { return size_t(div_up(n > 0 ? n : 1, kScanTile)) * sizeof(uint64_t); }

hipError_t launch_scan_u32(const uint32_t* in, uint32_t* out, int64_t n, uint64_t* total64, void* ws,
                           hipStream_t s, const uint32_t* n_dev) {
  if (n == 0) {
    {
      GSK_PROF("scan_empty", s);
      scan_empty_kernel<<<1, 1, 0, s>>>(out, total64);
    }
    return hipGetLastError();
  }
  const int nb = int(div_up(n, kScanTile));
  uint64_t* sums = static_cast<uint64_t*>(ws);
  {
    GSK_PROF("scan_reduce", s);
    scan_reduce_kernel<<<nb, kScanThreads, 0, s>>>(in, n, n_dev, sums);
  }
  {
    GSK_PROF("scan_apply", s);
    const bool vec = reinterpret_cast<uintptr_t>(in) % 16 == 0 && reinterpret_cast<uintptr_t>(out) % 16 == 0;
    scan_apply_kernel<<<nb, kScanThreads, 0, s>>>(in, n, n_dev, sums, out, total64, vec);
  }
  return hipGetLastError();
}

}  // namespace gsk
