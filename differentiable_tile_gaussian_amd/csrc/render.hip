// Tile blend kernels: front-to-back forward and back-to-front backward.
//
// Short path.  One 256-thread block per 16x16 tile, one thread per pixel; blocks
// take the tiles longest list first (a one-block bucket sort by log2 of the list
// length).  A tile's sorted pair list is walked in batches of 256: the block
// gathers a batch's records into LDS (double-buffered: the next batch's gather is
// issued before the current one is blended) and every pixel reads them as
// wave-wide broadcasts.  The per-entry arithmetic is branch-free: a pair that is
// skipped (alpha below 1/255) or comes after the pixel stopped is blended with
// alpha = 0, which leaves T and the colour unchanged bit for bit, so the result is
// that of the sequential walk with `continue` and `break`.
//
// Split path.  One block can only use one CU, and a few tiles carry lists of tens
// of thousands of pairs, so the first `first` pairs of every tile are walked as
// above and a tile whose pixels are not all finished then is split: its remaining
// pairs form chunks of `chunk` pairs that separate blocks walk at the same time.  The
// chunks of every tile longer than `first` (a candidate) are blocks of the same launch
// as the first segments, after them, so that they fill the CUs that the last long first
// segments leave idle, taken chunk index first (every candidate's chunk 0, then chunk 1,
// ...); a tile's first segment publishes, when it ends, whether the tile is split and
// each pixel's transmittance T_first.
//   chunk c   walks from T = 1 (the local transmittance and colour of the chunk), stops
//             a pixel once B T_local < 1e-4, B an upper bound of the transmittance in
//             front of the chunk (1 before T_first is out; then the tile's running chain,
//             below), also in fp32, where every factor is at most 1, so the overall T
//             has dropped below 1e-4 by then too and the combine finds the stop in this
//             chunk or an earlier one; drops pixels that an earlier chunk has already
//             saturated (a per-pixel "first saturating chunk" marker, polled); stops
//             altogether once the tile turns out not split.  Then it publishes its own
//             T and moves the tile's chain past itself: the chain holds, per pixel, the
//             product of T_first and the chunks' own T up to some chunk (an upper bound
//             of the front the combine will compute); once it is below 1e-4 for every
//             pixel, the tile's later chunks are not walked;
//   combine   per pixel, chains the chunks: T_front(c+1) = T_front(c) T_c and
//             colour += T_front(c) C_c, from T_front(0) = T_first, until the product
//             falls below 1e-4 (four threads per pixel, a quarter of the chunks each);
//   re-walk   the chunk where that happens is walked again from T_front with the
//             test T_front * T_local < 1e-4 to find the exact last pair;
//   finalize  writes the pixel and, back to front, the state at each chunk end
//             that the backward needs (T there and S, the colour behind it,
//             accumulated from the background and each chunk's own colour sum).
// The split path keeps per pixel one boundary state per chunk of a split tile.
// It changes only where products are rounded (T_front T_local instead of one
// running product).  No block ever waits for another: what a chunk reads from the
// others (device-scope loads) only tightens its bound when it is out.

// Backward.  Each pixel walks from its last contributing pair back to the first,
// recovering T by division and carrying S ([DR] "The trick"); every entry's nine
// partials are summed over the wave (transposed butterfly), then over the block's
// waves in LDS, then added to the Gaussian's gradient with one set of global
// atomics per (tile or chunk, Gaussian).  The geometric partials are summed as the
// moments of dL/de (dx, dy, dx^2, dx dy, dy^2 weighted); the conic turns them into
// du, dv, dA, dB, dC once per entry when the block flushes its sums.  Split tiles run
// one block per chunk, each starting from the boundary state the forward left.
//
// Both walks skip, per 8x8 quadrant, the pairs whose box (stored by the projection:
// no pixel centre outside it reaches alpha >= 1/255) misses the quadrant; each wave
// walks a list of the batch entries its quadrant needs.
//
// The conic is prescaled and the opacity taken to the exponent when a pair is staged:
// q = a' dx^2 + b' dx dy + c' dy^2 + log2 o with (a', b', c') = -log2(e) (A/2, B, C/2),
// so o exp(-e) is one exp2.
//
// Pages: [GSG] "The painting itself: front-to-back alpha compositing", "The clever
// bit: a single backward sweep through the blend", "From a pixel's blame to the
// oval's shape and place"; [DR] "The trick: recompute the blend state instead of
// storing it"; [GST] opacity slide (cap 0.99, skip below 1/255) and compositing-
// derivative slide.  ([GSG] is "How a computer rebuilds a real place out of soft
// colored dots called Gaussian Splats", [DR] "Differentiable rasterisation",
// [GST] the Gaussian splatting training study deck.)
#include <algorithm>

#include "gs_internal.h"
#include "profile.h"

namespace gsk {
namespace {

// Pixel of thread tid within its 16x16 tile: each wave of 64 threads covers one 8x8
// quadrant (a squarer footprint than four rows, so the pixels of a wave stop after
// more similar numbers of pairs and fewer lanes idle while the wave walks on).
__device__ inline int pixel_x(int tid) { return ((tid >> 6) & 1) * 8 + (tid & 7); }
__device__ inline int pixel_y(int tid) { return (tid >> 7) * 8 + ((tid >> 3) & 7); }
// Pixel coordinates of a tile's corner.
__device__ inline float tile_ox(int tile, int tx) { return float((tile % tx) * kTile); }
__device__ inline float tile_oy(int tile, int tx) { return float((tile / tx) * kTile); }

constexpr int kBatch = 256;
constexpr int kBlock = 256;   // threads of a tile block: one per pixel
constexpr float kAlphaMin = 1.0f / 255.0f;
constexpr float kAlphaCap = 0.99f;
constexpr float kTStop = 1e-4f;
constexpr float kLog2e = 1.44269504088896341f;
constexpr uint32_t kFlag = 0x80000000u;
constexpr uint32_t kIdx = 0x7fffffffu;
// A split candidate's first segment (SplitWs::state): still walking, unfinished pixels
// after it (the tile is split), or all pixels finished within it; kDoneBase + c: split,
// and the chunks' running transmittance chain has found every pixel finished by the end
// of chunk c (the later chunks are not walked).
constexpr uint32_t kPending = 0u, kSplit = 1u, kNotSplit = 2u, kDoneBase = 3u;
__host__ __device__ inline bool is_split(uint32_t st) { return st == kSplit || st >= kDoneBase; }
// The chain's products are bounds of the combine's own (other roundings): a chunk stops a
// pixel against its bound times kChainSlack, and the chain calls a pixel finished only
// below kTChainDone, so that the combine finds every stop in a chunk that was walked.
constexpr float kChainSlack = 1.001f;
constexpr float kTChainDone = 0.999e-4f;
constexpr uint32_t kChainLook = 8;   // chunks between the chain and the one moving it, at most

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workspace of one render (forward and its backward).  Per-slot arrays hold 256
// entries per split tile, per-item arrays 256 entries per chunk.
struct SplitWs {
  uint32_t* order;        // [NT] tiles, longest list first
  uint32_t* counters;     // [0] split candidates (slots), [1] chunks (items), [2] tiles walked
                          // before the chunks, [3] 1 if the dispatch is chunk index first
  int32_t* slot_of_tile;  // [NT] slot or -1
  uint32_t* slot_tile;    // [S]
  uint32_t* slot_first;   // [S] first item of the slot
  uint32_t* slot_nch;     // [S] chunks of the slot
  uint2* items;           // [I] (slot, chunk)
  float4* st4;            // [S][256] T and colour after the first segment
  uint32_t* stl;          // [S][256] last pair | done flag
  uint32_t* sat;          // [S][256] first chunk that saturated the pixel
  uint32_t* state;        // [S] the tile's first segment: kPending, kSplit or kNotSplit; or kDoneBase + c
  float* tfirst;          // [S][256] T in front of chunk chain[slot] (first: after the first segment;
                          // 0: finished there; -1: not out yet); the chunks advance it in order
  uint32_t* chain;        // [S] the chunk whose front tfirst holds (none before the first segment ends)
  uint32_t* disp;         // [I] chunks in dispatch order (chunk index major)
  uint32_t* rbase;        // [I] first dispatch place of the chunks with index c
  float* tl;              // [I][256] each chunk's own transmittance once walked (-1 before)
  float4* part4;          // [I][256] chunk partials, later (T_end, S_end) boundaries
  uint32_t* partl;        // [I][256] last pair in the chunk | stop flag
  int32_t* stopc;         // [S][256] chunk holding the last pair (-1: first segment, nch: none)
  float4* fin4;           // [S][256] final (or front) T and colour
  uint32_t* finl;         // [S][256] final (or front) last pair
  float4* bnd1;           // [S][256] T and S at the end of the first segment
};

__host__ __device__ inline size_t a256(size_t b) { return (b + 255) & ~size_t(255); }

struct SplitDims {
  size_t NT, S, I;
};

__host__ __device__ inline SplitDims split_dims(int W, int H, uint32_t pairs, int first, int chunk) {
  SplitDims d;
  d.NT = size_t((W + kTile - 1) / kTile) * ((H + kTile - 1) / kTile);
  const size_t s = size_t(pairs) / size_t(first) + 1;
  d.S = s < d.NT ? s : d.NT;
  d.I = size_t(pairs) / size_t(chunk) + d.S + 1;
  return d;
}

__host__ __device__ inline SplitWs carve(void* ws, const SplitDims& d) {
  char* p = static_cast<char*>(ws);
  SplitWs w;
  auto take = [&](size_t bytes) { char* q = p; p += a256(bytes); return q; };
  w.order = reinterpret_cast<uint32_t*>(take(d.NT * 4));
  w.counters = reinterpret_cast<uint32_t*>(take(16));
  w.slot_of_tile = reinterpret_cast<int32_t*>(take(d.NT * 4));
  w.slot_tile = reinterpret_cast<uint32_t*>(take(d.S * 4));
  w.slot_first = reinterpret_cast<uint32_t*>(take(d.S * 4));
  w.slot_nch = reinterpret_cast<uint32_t*>(take(d.S * 4));
  w.items = reinterpret_cast<uint2*>(take(d.I * 8));
  w.st4 = reinterpret_cast<float4*>(take(d.S * 256 * 16));
  w.stl = reinterpret_cast<uint32_t*>(take(d.S * 256 * 4));
  w.sat = reinterpret_cast<uint32_t*>(take(d.S * 256 * 4));
  w.state = reinterpret_cast<uint32_t*>(take(d.S * 4));
  w.tfirst = reinterpret_cast<float*>(take(d.S * 256 * 4));
  w.chain = reinterpret_cast<uint32_t*>(take(d.S * 4));
  w.disp = reinterpret_cast<uint32_t*>(take(d.I * 4));
  w.rbase = reinterpret_cast<uint32_t*>(take(d.I * 4));
  w.tl = reinterpret_cast<float*>(take(d.I * 256 * 4));
  w.part4 = reinterpret_cast<float4*>(take(d.I * 256 * 16));
  w.partl = reinterpret_cast<uint32_t*>(take(d.I * 256 * 4));
  w.stopc = reinterpret_cast<int32_t*>(take(d.S * 256 * 4));
  w.fin4 = reinterpret_cast<float4*>(take(d.S * 256 * 16));
  w.finl = reinterpret_cast<uint32_t*>(take(d.S * 256 * 4));
  w.bnd1 = reinterpret_cast<float4*>(take(d.S * 256 * 16));
  return w;
}

__host__ __device__ inline size_t carve_bytes(const SplitDims& d) {
  return a256(d.NT * 4) + a256(16) + a256(d.NT * 4) + 3 * a256(d.S * 4) + a256(d.I * 8) + a256(d.S * 256 * 16) +
         2 * a256(d.S * 256 * 4) + 2 * a256(d.S * 4) + a256(d.S * 256 * 4) + 2 * a256(d.I * 4) + a256(d.I * 256 * 4) + a256(d.I * 256 * 16) + a256(d.I * 256 * 4) + a256(d.S * 256 * 4) +
         a256(d.S * 256 * 16) + a256(d.S * 256 * 4) + a256(d.S * 256 * 16);
}

// A render workspace: this header, then the split state (carve), then, for fixed-point
// gradient sums, the backward's 64-bit accumulators.  The forward writes the header; the
// backward takes the split sizes and the carve from it, so that it walks the chunks the
// forward made whatever split sizes its own caller passes.
struct RenderHeader {
  uint32_t magic, first, chunk, num_tiles, pairs, W, H, pad;
  uint64_t split_bytes;
};
constexpr uint32_t kHeaderMagic = 0x47535731u;
constexpr size_t kHeaderBytes = 256;

// What the backward expects of the header: written by a forward of this image and pair
// count, with split sizes in range and a split state that ends within `avail` bytes.
struct HeaderCheck {
  const RenderHeader* h;
  int num_tiles, W, H;
  uint32_t pairs;
  uint64_t avail;
};

__device__ inline bool header_ok(const HeaderCheck& c, RenderHeader& h) {
  h = *c.h;
  if (h.magic != kHeaderMagic || h.num_tiles != uint32_t(c.num_tiles) || h.pairs != c.pairs ||
      h.W != uint32_t(c.W) || h.H != uint32_t(c.H))
    return false;
  if (h.first < 4u || h.chunk < 4u || h.first > (1u << 24) || h.chunk > (1u << 24)) return false;
  const uint64_t need = carve_bytes(split_dims(c.W, c.H, c.pairs, int(h.first), int(h.chunk)));
  return h.split_bytes == need && need <= c.avail;
}

// ---------------------------------------------------------------- tile order
// Exclusive prefix sums of one value per thread of a 1024-thread block (wave sums by
// shuffles, then the sixteen waves' totals), and their total.  All threads must call it.
__device__ inline uint32_t block_excl_scan(uint32_t v, uint32_t* s_w, uint32_t& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_w[w] = x;
  __syncthreads();
  if (w == 0) {
    uint32_t t = lane < 16 ? s_w[lane] : 0u;
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
      const uint32_t y = __shfl_up(t, d, 64);
      if (lane >= d) t += y;
    }
    if (lane < 16) s_w[16 + lane] = t;
  }
  __syncthreads();
  const uint32_t wbase = w ? s_w[16 + w - 1] : 0u;
  total = s_w[31];
  __syncthreads();
  return wbase + x - v;
}

// Tiles sorted by bucket 32 - clz(length), longest bucket first (order within a
// bucket is arbitrary).  One block; num_tiles may exceed the block size.  The block also
// writes the workspace header and gives every tile whose list is longer than `first` (a
// split candidate: whether it is split is known only when its first segment ends) a slot
// and the items of its chunks, taking the tiles in that order; the other tiles get none.
// The chunks are dispatched chunk index first (every candidate's chunk 0, then chunk 1,
// ...), so that a tile's chunk has mostly finished before its next ones start and the
// running transmittance chain can tell them when their tile is finished; with more than
// kMaxChunksOrdered chunks in a tile, tile by tile instead.
constexpr uint32_t kMaxChunksOrdered = 2048;
// Tiles of at least 2^(kEarlyBucket - 1) pairs (and every split candidate) are dispatched
// before the split chunks.
constexpr int kEarlyBucket = 9;
__global__ void __launch_bounds__(1024) tile_order_kernel(const uint32_t* __restrict__ ranges, int num_tiles,
                                                           SplitWs ws, int first, int chunk,
                                                           RenderHeader* __restrict__ hdr, RenderHeader h) {
  __shared__ uint32_t s_cnt[33];
  __shared__ uint32_t s_pos[33];
  __shared__ uint32_t s_slots, s_items, s_maxnch;
  __shared__ uint32_t s_h[kMaxChunksOrdered + 1];      // slots with that many chunks
  __shared__ uint32_t s_oslot[kMaxChunksOrdered + 1];  // first slot of those
  __shared__ uint32_t s_oitem[kMaxChunksOrdered + 1];  // their first item
  __shared__ uint32_t s_fill[kMaxChunksOrdered + 1];
  __shared__ uint32_t s_w[32];
  const int tid = threadIdx.x;
  if (tid < 33) s_cnt[tid] = 0u;
  if (tid == 0) {
    *hdr = h;
    s_slots = s_items = s_maxnch = 0u;
  }
  for (uint32_t c = tid; c <= kMaxChunksOrdered; c += blockDim.x) s_h[c] = s_fill[c] = 0u;
  __syncthreads();
  for (int t = tid; t < num_tiles; t += blockDim.x) {
    const uint32_t len = ranges[num_tiles + t] - ranges[t];
    const int b = len ? 32 - __clz(len) : 0;
    atomicAdd(&s_cnt[b], 1u);
    ws.slot_of_tile[t] = -1;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t acc = 0;
    for (int b = 32; b >= 0; --b) {
      s_pos[b] = acc;
      acc += s_cnt[b];
    }
  }
  __syncthreads();
  // the candidates sit in the buckets from that of first + 1 up: the order's first `span`
  const int bf = 32 - __clz(uint32_t(first) + 1u);
  const int span = int(s_pos[bf] + s_cnt[bf]);
  // the tiles of bucket eb and longer (every candidate among them) are walked before the
  // chunks, the others after them
  const int eb = min(kEarlyBucket, bf);
  const uint32_t early = s_pos[eb] + s_cnt[eb];
  __syncthreads();
  for (int t = tid; t < num_tiles; t += blockDim.x) {
    const uint32_t len = ranges[num_tiles + t] - ranges[t];
    const int b = len ? 32 - __clz(len) : 0;
    ws.order[atomicAdd(&s_pos[b], 1u)] = uint32_t(t);
  }
  __syncthreads();
  // the candidates' chunk counts; the slots sorted by them, most first, so that the
  // candidates with more than c chunks are the first slots and dispatch round c is
  // places rbase[c] + slot (tile order again with longer lists than the LDS tables hold)
  for (int p = tid; p < span; p += blockDim.x) {
    const uint32_t tile = ws.order[p];
    const int len = int(ranges[num_tiles + tile] - ranges[tile]);
    if (len > first) {
      const uint32_t nch = uint32_t((len - first + chunk - 1) / chunk);
      atomicMax(&s_maxnch, nch);
      atomicAdd(&s_h[nch < kMaxChunksOrdered ? nch : kMaxChunksOrdered], 1u);
    }
  }
  __syncthreads();
  const uint32_t maxnch = s_maxnch;
  const bool ordered = maxnch <= kMaxChunksOrdered;
  uint32_t run_s = 0u, run_i = 0u;   // slots and items (ordered)
  if (ordered) {
    // j = maxnch - k runs over the chunk counts k from the most down: the first slot and
    // item of the slots with k chunks are the sums over the counts above k
    for (uint32_t j0 = 0; j0 < maxnch; j0 += 1024) {
      const uint32_t j = j0 + uint32_t(tid), k = maxnch - j;
      const uint32_t h = j < maxnch ? s_h[k] : 0u;
      uint32_t ts, ti;
      const uint32_t es = block_excl_scan(h, s_w, ts), ei = block_excl_scan(h * k, s_w, ti);
      if (j < maxnch) {
        s_oslot[k] = run_s + es;
        s_oitem[k] = run_i + ei;
      }
      run_s += ts;
      run_i += ti;
    }
    __syncthreads();
    // round c (the chunks with index c) holds the slots with more than c chunks, s_oslot[c]
    // of them for c >= 1 and all of them for c = 0; rbase: the rounds' first places
    uint32_t run = 0u;
    for (uint32_t c0 = 0; c0 < maxnch; c0 += 1024) {
      const uint32_t c = c0 + uint32_t(tid);
      const uint32_t size = c < maxnch ? (c == 0 ? run_s : s_oslot[c]) : 0u;
      uint32_t tot;
      const uint32_t e = block_excl_scan(size, s_w, tot);
      if (c < maxnch) ws.rbase[c] = run + e;
      run += tot;
    }
  }
  __syncthreads();
  for (int p = tid; p < span; p += blockDim.x) {
    const uint32_t tile = ws.order[p];
    const int len = int(ranges[num_tiles + tile] - ranges[tile]);
    if (len > first) {
      const uint32_t nch = uint32_t((len - first + chunk - 1) / chunk);
      uint32_t slot, fi;
      if (ordered) {
        const uint32_t r = atomicAdd(&s_fill[nch], 1u);
        slot = s_oslot[nch] + r;
        fi = s_oitem[nch] + r * nch;
      } else {
        slot = atomicAdd(&s_slots, 1u);
        fi = atomicAdd(&s_items, nch);
      }
      ws.slot_tile[slot] = tile;
      ws.slot_first[slot] = fi;
      ws.slot_nch[slot] = nch;
      ws.slot_of_tile[tile] = int32_t(slot);
    }
  }
  __syncthreads();
  if (tid == 0) {
    ws.counters[0] = ordered ? run_s : s_slots;
    ws.counters[1] = ordered ? run_i : s_items;
    ws.counters[2] = early;
    ws.counters[3] = ordered ? 1u : 0u;
  }
}

// One block per slot: the slot's items, and its state reset (first segment pending, no T
// out yet, no chunk has saturated a pixel).
__global__ void __launch_bounds__(256) split_reset_kernel(SplitWs ws) {
  const uint32_t slot = blockIdx.x;
  if (slot >= ws.counters[0]) return;
  const int tid = threadIdx.x;
  const size_t so = size_t(slot) * 256 + tid;
  ws.sat[so] = 0xffffffffu;
  ws.tfirst[so] = -1.0f;
  if (tid == 0) {
    ws.state[slot] = kPending;
    ws.chain[slot] = 0xffffffffu;
  }
  const uint32_t fi = ws.slot_first[slot], nch = ws.slot_nch[slot];
  const bool ordered = ws.counters[3] != 0u;
  for (uint32_t c = tid; c < nch; c += 256) {
    ws.items[fi + c] = make_uint2(slot, c);
    ws.disp[ordered ? ws.rbase[c] + slot : fi + c] = fi + c;
  }
  for (uint32_t c = 0; c < nch; ++c) ws.tl[size_t(fi + c) * 256 + tid] = -1.0f;
}

// ------------------------------------------------------------ forward walk
// Quadrant mask of a pair in the tile with corner (ox, oy): bit 2 * qy + qx is set
// unless the pair's box (u +- bx, v +- by), outside which no pixel centre gets
// alpha >= 1/255, misses the pixel centres of 8x8 quadrant (qx, qy).  The walks
// skip a pair in a quadrant whose bit is clear: every pixel there would have skipped
// it, so the results are unchanged.
__device__ inline uint32_t quad_mask(float u, float v, float bx, float by, float ox, float oy) {
  if (bx < 0.0f) return 0u;                                // reaches no pixel
  if (!(bx <= 3.0e38f) || !(by <= 3.0e38f)) return 0xfu;   // unbounded
  const float x0 = u - bx - ox, x1 = u + bx - ox, y0 = v - by - oy, y1 = v + by - oy;
  const bool xl = x0 <= 7.5f && x1 >= 0.5f, xr = x0 <= 15.5f && x1 >= 8.5f;
  const bool yt = y0 <= 7.5f && y1 >= 0.5f, yb = y0 <= 15.5f && y1 >= 8.5f;
  return uint32_t(xl && yt) | (uint32_t(xr && yt) << 1) | (uint32_t(xl && yb) << 2) | (uint32_t(xr && yb) << 3);
}

// Narrows a quadrant mask with the ellipse itself: clears the bit of each quadrant whose
// rectangle of pixel centres holds no point with e = A X^2 / 2 + B X Y + C Y^2 / 2 <= tm
// (X, Y relative to (u, v)), tm being ln(255 o) widened for the blend's fp32 evaluation of
// e, here widened again by 1 % + 0.01 for this evaluation.  The minimum of e over a
// rectangle without the centre lies on its boundary, on each edge at the edge's own
// minimiser (Y = -B X / C on a vertical edge, X = -B Y / A on a horizontal one) clamped
// to the edge; the rectangle covers the quadrant's pixel centres, so the test only errs
// towards keeping a bit.  tm is infinite for an unbounded box and the mask is left as is.
__device__ inline uint32_t ellipse_mask(uint32_t m, float u, float v, float A, float B, float C, float tm,
                                        float ox, float oy) {
  if (m == 0u || !(tm <= 3.0e38f)) return m;
  const float thr = fmaf(tm, 1.01f, 0.01f);
  const float ha = 0.5f * A, hc = 0.5f * C;
  const float sy = -B * __builtin_amdgcn_rcpf(C), sx = -B * __builtin_amdgcn_rcpf(A);
  // pixel-centre lines 0.5, 7.5, 8.5, 15.5 from the tile corner, relative to the centre
  const float xs[4] = {(ox + 0.5f) - u, (ox + 7.5f) - u, (ox + 8.5f) - u, (ox + 15.5f) - u};
  const float ys[4] = {(oy + 0.5f) - v, (oy + 7.5f) - v, (oy + 8.5f) - v, (oy + 15.5f) - v};
  float emin[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) emin[q] = __builtin_inff();
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int h = k >> 1;   // the half (quadrant column or row) the line bounds
    // vertical edge X = xs[k] of quadrants (h, 0) and (h, 1)
    const float X = xs[k], Y = ys[k];
    const float lx = X * ha, ly = Y * hc;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const float y = __builtin_amdgcn_fmed3f(sy * X, ys[2 * r], ys[2 * r + 1]);
      const float ev = X * fmaf(B, y, lx) + hc * y * y;
      emin[2 * r + h] = fminf(emin[2 * r + h], ev);
      // horizontal edge Y = ys[k] of quadrants (0, h) and (1, h)
      const float x = __builtin_amdgcn_fmed3f(sx * Y, xs[2 * r], xs[2 * r + 1]);
      const float eh = Y * fmaf(B, x, ly) + ha * x * x;
      emin[2 * h + r] = fminf(emin[2 * h + r], eh);
    }
  }
  uint32_t out = 0u;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int qx = q & 1, qy = q >> 1;
    const bool inside = xs[2 * qx] <= 0.0f && xs[2 * qx + 1] >= 0.0f && ys[2 * qy] <= 0.0f && ys[2 * qy + 1] >= 0.0f;
    out |= uint32_t(inside || emin[q] <= thr) << q;
  }
  return m & out;
}

// Index of a zero-opacity record after each batch (alpha 0: blending it changes nothing).
constexpr int kPad = kBatch;
constexpr int kListLen = kBatch + 4;

// Writes to list, in increasing order, base + scale * e for the entries e = 0 .. last
// of a batch whose bit for the calling wave's quadrant is set, padded with
// base + scale * kPad to a multiple of 4; returns the padded length.  Wave-local: the
// list is read back by the same wave.
template <typename T>
__device__ inline int build_list(const uint32_t* m, int last, T* list, uint32_t base, uint32_t scale) {
  const int lane = __lane_id();
  const uint32_t quad = threadIdx.x >> 6;
  const uint64_t below = (uint64_t(1) << lane) - 1;
  int cnt = 0;
  for (int grp = 0; grp * 64 <= last; ++grp) {
    const int e = grp * 64 + lane;
    const bool bit = e <= last && ((m[e] >> quad) & 1u);
    const uint64_t bal = __ballot(bit);
    if (bit) list[cnt + __popcll(bal & below)] = T(base + scale * uint32_t(e));
    cnt += __popcll(bal);
  }
  const int pad = (4 - (cnt & 3)) & 3;
  if (lane < pad) list[cnt + lane] = T(base + scale * uint32_t(kPad));
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  return cnt + pad;
}

// The blend's coefficients of a pair from its record: a = (u, v, a', b'),
// b = (c', log2 o, r, g) with (a', b', c') = -log2(e) (A/2, B, C/2), so that
// o exp(-e) = exp2(pair_q(...)).  A record that no pixel may blend has log2 o = -inf.
__device__ inline void stage_coeffs(const float4& r0, const float4& r1, float4& a, float4& b) {
  a = make_float4(r0.x, r0.y, -0.5f * kLog2e * r0.z, -kLog2e * r0.w);
  b = make_float4(-0.5f * kLog2e * r1.x, __builtin_amdgcn_logf(r1.y), r1.z, r1.w);
}
constexpr float kNoOpacity = -__builtin_inff();   // log2 of a zero opacity

// q = a' dx^2 + b' dx dy + c' dy^2 + log2 o.  Both walks evaluate it with this one
// sequence of roundings (explicit fma and products, nothing left to contraction), so
// the backward recomputes exactly the alpha = min(0.99, exp2(q)) the forward blended.
__device__ inline float pair_q(float ap, float bp, float cp, float lo2, float dx, float dy) {
  const float t = fmaf(ap, dx, __fmul_rn(bp, dy));
  return fmaf(t, dx, fmaf(__fmul_rn(cp, dy), dy, lo2));
}

// A forward batch entry: one 48-byte LDS record, so that a wave reads an entry with
// three loads off one address (the walk lists hold the records' byte offsets).
struct FwdRec {
  float4 a;   // u, v, a', b'
  float4 b;   // c', log2 o, r, g
  float4 c;   // b, 1 + index of the pair in the tile's list (bits), unused, unused
};

struct FwdLds {
  FwdRec rec[2][kBatch + 1];  // entry kPad: a record no pixel blends
  uint32_t m[2][kBatch];      // quadrant masks
  uint32_t list[4][kListLen]; // per wave: byte offsets (within rec) of the entries it walks
};

__device__ inline FwdRec empty_fwd_rec() {
  FwdRec r;
  r.a = make_float4(0.f, 0.f, 0.f, 0.f);
  r.b = make_float4(0.f, kNoOpacity, 0.f, 0.f);
  r.c = make_float4(0.f, 0.f, 0.f, 0.f);
  return r;
}

// Record and quadrant mask of Gaussian g as the pair with index idx in its tile's list.
__device__ inline void stage_fwd(const float4* __restrict__ splat, uint32_t g, int idx, float ox, float oy,
                                 FwdRec& r, uint32_t& m) {
  const float4 r0 = splat[3 * g], r1 = splat[3 * g + 1], r2 = splat[3 * g + 2];
  stage_coeffs(r0, r1, r.a, r.b);
  r.c = make_float4(r2.x, __uint_as_float(uint32_t(idx + 1)), 0.f, 0.f);
  m = ellipse_mask(quad_mask(r0.x, r0.y, r2.y, r2.z, ox, oy), r0.x, r0.y, r0.z, r0.w, r1.x, r2.w, ox, oy);
}

struct PixelFwd {
  float T, c0, c1, c2;
  uint32_t last;   // 1 + index (within the tile's list) of the last blended pair, 0 if none
  bool done;
};

// Blends, in order, the entries of a wave's list (byte offsets of records within recs),
// four at a time, until every pixel of the wave is done; a pixel stops once pre * T < 1e-4.
// The calling wave has a pixel that is not done.
__device__ __forceinline__ void walk_list(const uint32_t* list, int len, const char* recs, PixelFwd& s, float fx,
                                          float fy, float pre) {
  bool all_done = false;
  for (int k = 0; k < len && !all_done; k += 4) {
    const uint4 ix = *reinterpret_cast<const uint4*>(list + k);
    const uint32_t off[4] = {ix.x, ix.y, ix.z, ix.w};
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const FwdRec& r = *reinterpret_cast<const FwdRec*>(recs + off[q4]);
      const float4 a = r.a, b = r.b;
      const float2 c = make_float2(r.c.x, r.c.y);
      const float dx = fx - a.x, dy = fy - a.y;
      float alpha = fminf(kAlphaCap, fast_exp2(pair_q(a.z, a.w, b.x, b.y, dx, dy)));
      const bool ok = !s.done && alpha >= kAlphaMin;
      alpha = ok ? alpha : 0.0f;
      const float w = alpha * s.T;
      s.c0 += w * b.z;
      s.c1 += w * b.w;
      s.c2 += w * c.x;
      s.T = s.T * (1.0f - alpha);
      s.last = ok ? __float_as_uint(c.y) : s.last;
      s.done = s.done || (pre * s.T < kTStop);
    }
    all_done = __all(s.done);
  }
}

// Walks the pairs [lo, hi) of a tile list starting at `start`.  A pixel stops once
// pre * T < 1e-4 (pre = 1 for a walk whose T is the overall transmittance).  With
// POLL (a chunk of a split candidate), after every batch: a pixel also stops when
// sat[tid] < chunk_id, and a pixel that saturates records chunk_id in sat[tid]; a pixel
// whose bound is not yet known (pre = 1) takes the tile's T after its first segment once
// tfirst[tid] holds it (>= 0); and every pixel stops once the tile turns out not split.
// Must be called by all 256 threads of the block.
template <bool POLL>
__device__ void fwd_walk(FwdLds& L, const float4* __restrict__ splat, const uint32_t* __restrict__ vals,
                         uint32_t start, int lo, int hi, float ox, float oy, float fx, float fy, float pre,
                         PixelFwd& s, uint32_t* sat, uint32_t chunk_id, const float* tfirst = nullptr,
                         const uint32_t* state = nullptr, bool known = true) {
  const int tid = threadIdx.x;
  if (lo >= hi) return;
  {
    FwdRec r = empty_fwd_rec();
    uint32_t m = 0u;
    if (lo + tid < hi) stage_fwd(splat, vals[start + uint32_t(lo + tid)], lo + tid, ox, oy, r, m);
    L.rec[0][tid] = r; L.m[0][tid] = m;
    if (tid < 2) L.rec[tid][kPad] = empty_fwd_rec();
  }
  __syncthreads();
  uint32_t* list = L.list[tid >> 6];
  const char* recs = reinterpret_cast<const char*>(&L.rec[0][0]);
  bool reported = s.done;
  int buf = 0;
  for (int base = lo; base < hi; base += kBatch) {
    const int nxt = base + kBatch + tid;
    FwdRec nr = empty_fwd_rec();
    uint32_t nm = 0u;
    if (nxt < hi) stage_fwd(splat, vals[start + uint32_t(nxt)], nxt, ox, oy, nr, nm);
    // walk the batch entries whose quadrant bit is set, in order, four at a time
    if (!__all(s.done)) {
      const int len = build_list(L.m[buf], kBatch - 1, list, uint32_t(buf * (kBatch + 1) * sizeof(FwdRec)),
                                 uint32_t(sizeof(FwdRec)));
      walk_list(list, len, recs, s, fx, fy, pre);
    }
    if (base + kBatch < hi) {
      L.rec[buf ^ 1][tid] = nr; L.m[buf ^ 1][tid] = nm;
    }
    if (POLL) {
      if (s.done && !reported) {
        atomicMin(&sat[tid], chunk_id);
        reported = true;
      }
      if (!s.done) {
        const uint32_t first_sat = __hip_atomic_load(&sat[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (first_sat < chunk_id) {
          s.done = true;
          reported = true;
        }
      }
      if (!s.done) {   // the chain may have moved on: a tighter bound
        const float tf = __hip_atomic_load(&tfirst[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tf >= 0.0f) {
          known = true;
          pre = fminf(pre, tf * kChainSlack);
          if (pre * s.T < kTStop) {   // a claim of its own, as in the blend
            s.done = true;
          }
        }
      }
      if (!s.done) {
        const uint32_t st = __hip_atomic_load(state, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (st == kNotSplit || (st >= kDoneBase && chunk_id > st - kDoneBase)) {
          s.done = true;
          reported = true;   // not a saturation: nothing to record
        }
      }
    }
    if (__syncthreads_count(s.done) == kBatch) break;
    buf ^= 1;
  }
}

// One chunk of a split candidate, walked from T = 1 (the chunk's own transmittance and
// colour).  Its pixels stop once B T < 1e-4, B an upper bound of the transmittance in front
// of the chunk: 1 while the tile's first segment still runs, its T after the first
// segment once that is out (every later factor is at most 1, also in fp32, so the overall
// T has dropped below 1e-4 by then too, and the combine finds the stop in this chunk or
// an earlier one); pixels that an earlier chunk has already saturated are dropped (a
// per-pixel "first saturating chunk", polled), and the whole walk once the first segment
// has finished every pixel (the tile is not split; what the chunk writes is then unused).
__device__ void split_chunk(FwdLds& L, const float4* __restrict__ splat, const uint32_t* __restrict__ vals,
                            const uint32_t* __restrict__ ranges, const SplitWs& ws, int num_tiles, int tx, int first,
                            int chunk, uint32_t item) {
  __shared__ uint32_t s_chain;
  const uint2 sc = ws.items[item];
  const uint32_t slot = sc.x, c = sc.y;
  const int tid = threadIdx.x;
  const uint32_t* state = ws.state + slot;
  // not walked: the tile turned out not split, or its chain found every pixel finished before
  const auto cut = [&]() {
    const uint32_t st = __hip_atomic_load(state, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return st == kNotSplit || (st >= kDoneBase && c > st - kDoneBase);
  };
  if (__syncthreads_count(cut()) == kBlock) return;
  const int tile = int(ws.slot_tile[slot]);
  const int px = (tile % tx) * kTile + pixel_x(tid);
  const int py = (tile / tx) * kTile + pixel_y(tid);
  const uint32_t start = ranges[tile];
  const int n = int(ranges[num_tiles + tile] - start);
  const int lo = first + int(c) * chunk, hi = min(lo + chunk, n);
  const size_t so = size_t(slot) * 256 + tid;
  const float tf = __hip_atomic_load(&ws.tfirst[so], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool known = tf >= 0.0f;
  const float pre = known ? tf * kChainSlack : 1.0f;
  PixelFwd s{1.0f, 0.0f, 0.0f, 0.0f, 0u, pre < kTStop};
  fwd_walk<true>(L, splat, vals, start, lo, hi, tile_ox(tile, tx), tile_oy(tile, tx), float(px) + 0.5f,
                 float(py) + 0.5f, pre, s, ws.sat + size_t(slot) * 256, c, ws.tfirst + size_t(slot) * 256, state,
                 known);
  if (__syncthreads_count(cut()) == kBlock) return;   // nothing of it is read
  const size_t io = size_t(item) * 256 + tid;
  ws.part4[io] = make_float4(s.T, s.c0, s.c1, s.c2);
  ws.partl[io] = s.last;
  // the chain: from where it stands (k <= c), past this chunk if the chunks in between have
  // published their own transmittance: T in front of the next chunk, an upper bound of the
  // combine's (every value any chunk writes here is one, also when two chunks move the
  // chain at once: a product that misses factors <= 1 is larger); one of them wins the
  // move; every pixel below kTChainDone: the later chunks are not needed
  __hip_atomic_store(&ws.tl[io], s.T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (tid == 0) s_chain = __hip_atomic_load(ws.chain + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  const uint32_t k = s_chain;
  if (k > c || c - k > kChainLook) return;
  const uint32_t fi = ws.slot_first[slot];
  float f = __hip_atomic_load(&ws.tfirst[so], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  bool ok = f >= 0.0f;
  float t[kChainLook];
#pragma unroll
  for (uint32_t j = 0; j < kChainLook; ++j)
    t[j] = k + j < c ? __hip_atomic_load(&ws.tl[size_t(fi + k + j) * 256 + tid], __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT)
                     : 1.0f;
#pragma unroll
  for (uint32_t j = 0; j < kChainLook; ++j) {
    ok = ok && t[j] >= 0.0f;
    f = f * t[j];
  }
  f = f * s.T;
  if (__syncthreads_count(ok) < kBlock) return;   // not all out yet: the chain stays
  if (tid == 0) s_chain = atomicCAS(ws.chain + slot, k, c + 1u);
  __syncthreads();
  if (s_chain != k) return;                        // another chunk moved it
  __hip_atomic_store(&ws.tfirst[so], f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int alive = __syncthreads_count(f >= kTChainDone);
  if (tid == 0 && alive == 0)
    __hip_atomic_store(ws.state + slot, kDoneBase + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Phase 1, one launch over num_tiles + the items' capacity blocks, in dispatch order: the
// first segments of the tiles of at least 256 pairs (longest list first), the chunks of the
// split candidates, the first segments of the other tiles (the short walks fill the CUs at
// the end), then blocks with nothing to do.  A candidate whose pixels are not all finished
// after its first segment is split: its block writes no output, leaves its state for the
// combine and publishes its per-pixel T for the chunks.
__global__ void __launch_bounds__(256) render_fwd_kernel(const float4* __restrict__ splat,
                                                          const uint32_t* __restrict__ vals,
                                                          const uint32_t* __restrict__ ranges, SplitWs ws,
                                                          int num_tiles, int tx, int W, int H, float bg0, float bg1,
                                                          float bg2, int first, int chunk, float* __restrict__ rgb,
                                                          float* __restrict__ T_final,
                                                          uint32_t* __restrict__ n_contrib) {
  __shared__ FwdLds L;
  const uint32_t early = ws.counters[2], items = ws.counters[1], b = blockIdx.x;
  uint32_t pos = b;   // place in the tile order
  if (b >= early) {
    if (b < early + items) {
      split_chunk(L, splat, vals, ranges, ws, num_tiles, tx, first, chunk, ws.disp[b - early]);
      return;
    }
    pos = b - items;
    if (pos >= uint32_t(num_tiles)) return;
  }
  const int tile = int(ws.order[pos]);
  const int tid = threadIdx.x;
  const int px = (tile % tx) * kTile + pixel_x(tid);
  const int py = (tile / tx) * kTile + pixel_y(tid);
  const bool inside = px < W && py < H;
  const uint32_t start = ranges[tile];
  const int n = int(ranges[num_tiles + tile] - start);
  PixelFwd s{1.0f, 0.0f, 0.0f, 0.0f, 0u, !inside};
  fwd_walk<false>(L, splat, vals, start, 0, min(n, first), tile_ox(tile, tx), tile_oy(tile, tx), float(px) + 0.5f,
                  float(py) + 0.5f, 1.0f, s, nullptr, 0u);
  if (n > first) {
    const uint32_t slot = uint32_t(ws.slot_of_tile[tile]);
    if (__syncthreads_count(s.done) < kBatch) {
      const size_t o = size_t(slot) * 256 + tid;
      ws.st4[o] = make_float4(s.T, s.c0, s.c1, s.c2);
      ws.stl[o] = s.last | (s.done ? kFlag : 0u);
      __hip_atomic_store(&ws.tfirst[o], s.done ? 0.0f : s.T, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (tid == 0) {
        __hip_atomic_store(ws.state + slot, kSplit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ws.chain + slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      return;
    }
    if (tid == 0) __hip_atomic_store(ws.state + slot, kNotSplit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (inside) {
    const int p = py * W + px;
    const int HW = W * H;
    rgb[p] = s.c0 + s.T * bg0;
    rgb[HW + p] = s.c1 + s.T * bg1;
    rgb[2 * HW + p] = s.c2 + s.T * bg2;
    T_final[p] = s.T;
    n_contrib[p] = s.last;
  }
}

// Phase 2: per split tile and pixel, chain the chunks from the first segment's state,
// T_front(c + 1) = T_front(c) T_c and colour += T_front(c) C_c, until the product falls
// below 1e-4: the chunk where it does holds the stop.  Four threads per pixel, each a
// quarter of the chunks: each first multiplies its quarter's T_c, the fronts of the
// quarters follow from those in quarter order, then each chains its quarter from its
// front; the first quarter that finds the stop decides it.  Chunk partials are loaded
// sixteen at a time before they are used.
constexpr int kCombG = 16;
__global__ void __launch_bounds__(1024) split_combine_kernel(SplitWs ws) {
  __shared__ float s_P[4][256];
  __shared__ float4 s_st[4][256];   // T at the quarter's stop (or end), colour the quarter added
  __shared__ int32_t s_stop[4][256];
  __shared__ uint32_t s_last[4][256];
  const uint32_t slot = blockIdx.x;
  if (slot >= ws.counters[0] || !is_split(ws.state[slot])) return;
  const int tid = threadIdx.x, q = tid >> 8, p = tid & 255;
  const size_t so = size_t(slot) * 256 + p;
  const uint32_t fi = ws.slot_first[slot], nch = ws.slot_nch[slot];
  const uint32_t m = (nch + 3u) / 4u, c0 = min(nch, uint32_t(q) * m), c1 = min(nch, c0 + m);
  const uint32_t l1 = ws.stl[so];
  const float4 s1 = ws.st4[so];
  const bool done0 = (l1 & kFlag) != 0u;
  // the quarter's own product
  float P = 1.0f;
  if (!done0) {
    for (uint32_t g = c0; g < c1; g += kCombG) {
      float t[kCombG];
#pragma unroll
      for (int k = 0; k < kCombG; ++k) t[k] = g + k < c1 ? ws.part4[size_t(fi + g + k) * 256 + p].x : 1.0f;
#pragma unroll
      for (int k = 0; k < kCombG; ++k) P = P * t[k];
    }
  }
  s_P[q][p] = P;
  __syncthreads();
  float T = s1.x;
  for (int k = 0; k < q; ++k) T = T * s_P[k][p];
  // the quarter chained from its front
  int32_t stop = -1;
  float a0s = 0.0f, a1s = 0.0f, a2s = 0.0f;
  uint32_t last = 0u;
  if (!done0) {
    for (uint32_t g = c0; g < c1 && stop < 0; g += kCombG) {
      float4 pc[kCombG];
      uint32_t lc[kCombG];
#pragma unroll
      for (int k = 0; k < kCombG; ++k) {
        if (g + k < c1) {
          pc[k] = ws.part4[size_t(fi + g + k) * 256 + p];
          lc[k] = ws.partl[size_t(fi + g + k) * 256 + p] & kIdx;
        }
      }
#pragma unroll
      for (int k = 0; k < kCombG; ++k) {
        const uint32_t c = g + k;
        if (c < c1 && stop < 0) {
          const float Tn = T * pc[k].x;
          if (Tn < kTStop) {
            stop = int32_t(c);
          } else {
            const float a0 = T * pc[k].y, a1 = T * pc[k].z, a2 = T * pc[k].w;
            ws.part4[size_t(fi + c) * 256 + p] = make_float4(Tn, a0, a1, a2);   // T at the chunk end, colour it added
            a0s += a0; a1s += a1; a2s += a2;
            T = Tn;
            if (lc[k]) last = lc[k];
          }
        }
      }
    }
  }
  s_st[q][p] = make_float4(T, a0s, a1s, a2s);
  s_stop[q][p] = stop;
  s_last[q][p] = last;
  __syncthreads();
  if (q != 0) return;
  float c0f = s1.y, c1f = s1.z, c2f = s1.w;
  uint32_t lastf = l1 & kIdx;
  float Tf = s1.x;
  int32_t stopf = -1;
  if (!done0) {
    stopf = int32_t(nch);
    for (int k = 0; k < 4; ++k) {
      const float4 st = s_st[k][p];
      c0f += st.y; c1f += st.z; c2f += st.w;
      if (s_last[k][p]) lastf = s_last[k][p];
      Tf = st.x;
      if (s_stop[k][p] >= 0) {
        stopf = s_stop[k][p];
        break;
      }
    }
  }
  ws.stopc[so] = stopf;
  ws.fin4[so] = make_float4(Tf, c0f, c1f, c2f);
  ws.finl[so] = lastf;
}

// Phase 3: walk again the chunk that holds a pixel's stop, from T_front, to find the pair.
__global__ void __launch_bounds__(256) split_rewalk_kernel(const float4* __restrict__ splat,
                                                            const uint32_t* __restrict__ vals,
                                                            const uint32_t* __restrict__ ranges, SplitWs ws,
                                                            int num_tiles, int tx, int first, int chunk) {
  __shared__ FwdLds L;
  const uint32_t item = blockIdx.x;
  if (item >= ws.counters[1]) return;
  const uint2 sc = ws.items[item];
  const uint32_t slot = sc.x, c = sc.y;
  if (!is_split(ws.state[slot])) return;
  const int tid = threadIdx.x;
  const size_t so = size_t(slot) * 256 + tid;
  const bool need = ws.stopc[so] == int32_t(c);
  if (__syncthreads_count(need) == 0) return;
  const int tile = int(ws.slot_tile[slot]);
  const int px = (tile % tx) * kTile + pixel_x(tid);
  const int py = (tile / tx) * kTile + pixel_y(tid);
  const uint32_t start = ranges[tile];
  const int n = int(ranges[num_tiles + tile] - start);
  const int lo = first + int(c) * chunk, hi = min(lo + chunk, n);
  float4 front = make_float4(1.f, 0.f, 0.f, 0.f);
  uint32_t lastf = 0;
  if (need) {
    front = ws.fin4[so];
    lastf = ws.finl[so];
  }
  PixelFwd s{1.0f, 0.0f, 0.0f, 0.0f, 0u, !need};
  fwd_walk<false>(L, splat, vals, start, lo, hi, tile_ox(tile, tx), tile_oy(tile, tx), float(px) + 0.5f,
                  float(py) + 0.5f, front.x, s, nullptr, 0u);
  if (need) {
    const float a0 = front.x * s.c0, a1 = front.x * s.c1, a2 = front.x * s.c2;
    const float Tf = front.x * s.T;
    ws.fin4[so] = make_float4(Tf, front.y + a0, front.z + a1, front.w + a2);
    ws.finl[so] = s.last ? s.last : lastf;
    ws.part4[size_t(item) * 256 + tid] = make_float4(Tf, a0, a1, a2);
  }
}

// Phase 4: outputs of split tiles, and the chunk-end states for the backward
// (T there and S = colour behind, summed from the background forward).
__global__ void __launch_bounds__(256) split_finalize_kernel(SplitWs ws, int tx, int W, int H, float bg0,
                                                              float bg1, float bg2, float* __restrict__ rgb,
                                                              float* __restrict__ T_final,
                                                              uint32_t* __restrict__ n_contrib) {
  const uint32_t slot = blockIdx.x;
  if (slot >= ws.counters[0] || !is_split(ws.state[slot])) return;
  const int tid = threadIdx.x;
  const int tile = int(ws.slot_tile[slot]);
  const int px = (tile % tx) * kTile + pixel_x(tid);
  const int py = (tile / tx) * kTile + pixel_y(tid);
  const size_t so = size_t(slot) * 256 + tid;
  const int32_t stop = ws.stopc[so];
  const float4 f = ws.fin4[so];
  if (px < W && py < H) {
    const int p = py * W + px;
    const int HW = W * H;
    rgb[p] = f.y + f.x * bg0;
    rgb[HW + p] = f.z + f.x * bg1;
    rgb[2 * HW + p] = f.w + f.x * bg2;
    T_final[p] = f.x;
    n_contrib[p] = ws.finl[so];
  }
  if (stop < 0) return;
  const uint32_t fi = ws.slot_first[slot], nch = ws.slot_nch[slot];
  float S0 = bg0 * f.x, S1 = bg1 * f.x, S2 = bg2 * f.x;
  int c = stop;
  if (uint32_t(stop) < nch) {
    const float4 ps = ws.part4[size_t(fi + stop) * 256 + tid];
    S0 += ps.y; S1 += ps.z; S2 += ps.w;
  } else {
    c = int(nch);
  }
  // chunks c - 1 .. 0, back to front, in groups of sixteen loaded ahead
  constexpr int kG = 16;
  for (int top = c - 1; top >= 0; top -= kG) {
    float4 pc[kG];
#pragma unroll
    for (int k = 0; k < kG; ++k)
      if (top - k >= 0) pc[k] = ws.part4[size_t(fi + uint32_t(top - k)) * 256 + tid];
#pragma unroll
    for (int k = 0; k < kG; ++k) {
      if (top - k >= 0) {
        ws.part4[size_t(fi + uint32_t(top - k)) * 256 + tid] = make_float4(pc[k].x, S0, S1, S2);
        S0 += pc[k].y; S1 += pc[k].z; S2 += pc[k].w;
      }
    }
  }
  ws.bnd1[so] = make_float4(ws.st4[so].x, S0, S1, S2);
}

// ----------------------------------------------------------- backward walk
// Lane exchanges without LDS: gfx950's v_permlane32_swap / v_permlane16_swap swap
// half-waves / adjacent rows between two registers, DPP moves within a row.
template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
constexpr int kRowRor8 = 0x128;       // lane i <- lane i ^ 8 within a 16-lane row
constexpr int kRowHalfMirror = 0x141; // lane i <- lane 7 - i within each 8 lanes
constexpr int kQuadXor2 = 0x4e;       // quad_perm [2, 3, 0, 1]
constexpr int kQuadXor1 = 0xb1;       // quad_perm [1, 0, 3, 2]

// a from lanes 0-31 and b from lanes 32-63 summed pairwise: lanes 0-31 get
// a(l) + a(l+32), lanes 32-63 get b(l-32) + b(l).
__device__ inline float fold32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Same between adjacent 16-lane rows: even rows get a(l) + a(l+16), odd rows b(l-16) + b(l).
__device__ inline float fold16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum 9 per-lane values over the 64 lanes of a wave.  Values 0..7 use a transposed
// butterfly (each exchange halves the values a lane carries), value 8 a plain one.
// On return lane l holds the total of value (l >> 3) in v[0] and every lane holds
// the total of value 8 in v[8].  All lanes of the wave must be active.
__device__ inline void wave_sum9(float* v) {
  const int lane = __lane_id();
  // distance 32: lanes 0-31 keep values 0-3, lanes 32-63 values 4-7
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] = fold32(v[k], v[k + 4]);
  v[8] = fold32(v[8], v[8]);
  // distance 16: even rows keep the first of each pair, odd rows the second
#pragma unroll
  for (int k = 0; k < 2; ++k) v[k] = fold16(v[k], v[k + 2]);
  v[8] = fold16(v[8], v[8]);
  // distance 8 within a row
  {
    const bool hi = lane & 8;
    const float send = hi ? v[0] : v[1];
    const float keep = hi ? v[1] : v[0];
    v[0] = keep + dpp<kRowRor8>(send);
  }
  v[8] += dpp<kRowRor8>(v[8]);
  // the last three lane bits: plain sums over 8 lanes
  v[0] += dpp<kRowHalfMirror>(v[0]);
  v[8] += dpp<kRowHalfMirror>(v[8]);
  v[0] += dpp<kQuadXor2>(v[0]);
  v[8] += dpp<kQuadXor2>(v[8]);
  v[0] += dpp<kQuadXor1>(v[0]);
  v[8] += dpp<kQuadXor1>(v[8]);
}

// Fixed-point gradient sums ([GSG] "Making the parallel sums exact": integers add in any
// order, so the sums are reproducible bit for bit; a blame is multiplied by 16384 and
// rounded, the second moments of a large footprint divided by a size factor first).
constexpr float kFixedUnit = 16384.0f;

// Size factor of a pair's footprint: 1 + the trace of its screen covariance (the inverse
// of the conic; the trace bounds the largest eigenvalue within a factor 2).  Explicit
// roundings, so that the walk and the decode compute the identical value; 1 when the
// conic is not positive definite.
__device__ inline float fixed_size_factor(float A, float B, float C) {
  const float det = __fsub_rn(__fmul_rn(A, C), __fmul_rn(B, B));
  const float tr = __fdiv_rn(__fadd_rn(A, C), det);
  return (det > 0.0f && tr >= 0.0f && tr < 1e30f) ? __fadd_rn(1.0f, tr) : 1.0f;
}

// Clamped to +-1e9 (the pages' bound) and rounded to the nearest integer.
__device__ inline int to_fixed(float x) { return int(rintf(fminf(fmaxf(x, -1e9f), 1e9f))); }

// The backward stages batches of kBwdBatch pairs (half the forward's, so that more
// blocks fit in a CU's LDS: 0.61 -> 0.56 ms on the 6M-Gaussian 1080p step; 64 is no faster).
constexpr int kBwdBatch = 128;

struct BwdLds {
  float4 a[2][kBwdBatch];     // u, v, a', b'
  float4 b[2][kBwdBatch];     // c', log2 o, r, g
  float c[2][kBwdBatch];      // b
  uint32_t id[2][kBwdBatch];
  uint32_t m[2][kBwdBatch];   // quadrant masks
  float inv_f[2][kBwdBatch];  // fixed-point sums: 1 / the pair's size factor
  float acc[kBwdBatch][9];    // per-entry sums over the block's waves (entry-major, as gscreen)
  uint16_t list[4][kBwdBatch + 4];
  uint32_t top;
};

template <bool FIXED>
__device__ inline void stage_bwd(const float4* __restrict__ splat, uint32_t g, float ox, float oy, float4& a,
                                 float4& b, float& c, uint32_t& m, float& inv_f) {
  const float4 r0 = splat[3 * g], r1 = splat[3 * g + 1], r2 = splat[3 * g + 2];
  stage_coeffs(r0, r1, a, b);
  c = r2.x;
  if (FIXED) inv_f = __fdiv_rn(1.0f, fixed_size_factor(r0.z, r0.w, r1.x));
  m = ellipse_mask(quad_mask(r0.x, r0.y, r2.y, r2.z, ox, oy), r0.x, r0.y, r0.z, r0.w, r1.x, r2.w, ox, oy);
}

struct PixelBwd {
  float T, S0, S1, S2;    // transmittance behind the next pair to walk, colour behind it
  float g0, g1, g2;       // dL/dpixel
  int top;                // pairs [lo, top) are walked, top - 1 first
};

// Walks pairs top-1 .. lo (top per pixel, at most hi) of a tile list, adding
// each pair's partials to gscreen.  Must be called by all 256 threads.  With FIXED the
// sums are integers ([GSG] "Making the parallel sums exact"): every wave-reduced moment,
// times `unit` (16384 times the loss's element count, so that the unit is that of the
// summed loss) and, for the three second moments, the pair's 1 / size factor, is rounded
// to an i32 and added with integer atomics, in LDS (i32: one tile's 256 pixels stay far
// below 2^31 units) and then into acc64 (i64, [n][9]: a Gaussian seen by a whole image
// can pass 2^31 units), which the decode kernel turns into gscreen; the order of the
// additions does not matter.
template <bool FIXED>
__device__ void bwd_walk(BwdLds& L, const float4* __restrict__ splat, const uint32_t* __restrict__ vals,
                         uint32_t start, int lo, float ox, float oy, float fx, float fy, PixelBwd& s,
                         float* __restrict__ gscreen, unsigned long long* __restrict__ acc64, float unit) {
  const int tid = threadIdx.x;
  const int lane = __lane_id();
  if (tid == 0) L.top = 0u;
  if (tid < kBwdBatch) {
#pragma unroll
    for (int k = 0; k < 9; ++k) L.acc[tid][k] = 0.0f;
  }
  __syncthreads();
  if (s.top > lo) atomicMax(&L.top, uint32_t(s.top));
  int wave_top = s.top;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) wave_top = max(wave_top, __shfl_xor(wave_top, d, 64));
  __syncthreads();
  int hi = int(L.top);
  if (hi <= lo) return;
  if (tid < kBwdBatch) {
    const int blo = max(hi - kBwdBatch, lo);
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = make_float4(0.f, kNoOpacity, 0.f, 0.f);
    float c = 0.f, f = 1.f;
    uint32_t g = 0, m = 0u;
    if (blo + tid < hi) {
      g = vals[start + uint32_t(blo + tid)];
      stage_bwd<FIXED>(splat, g, ox, oy, a, b, c, m, f);
    }
    L.a[0][tid] = a; L.b[0][tid] = b; L.c[0][tid] = c; L.id[0][tid] = g; L.m[0][tid] = m;
    if (FIXED) L.inv_f[0][tid] = f;
  }
  __syncthreads();
  uint16_t* list = L.list[tid >> 6];
  int buf = 0;
  while (hi > lo) {
    const int blo = max(hi - kBwdBatch, lo);
    const int nhi = blo, nlo = max(nhi - kBwdBatch, lo);
    float4 na = make_float4(0.f, 0.f, 0.f, 0.f), nb = make_float4(0.f, kNoOpacity, 0.f, 0.f);
    float ncr = 0.f, nf = 1.f;
    uint32_t ng = 0, nm = 0u;
    if (tid < kBwdBatch && nlo + tid < nhi) {
      ng = vals[start + uint32_t(nlo + tid)];
      stage_bwd<FIXED>(splat, ng, ox, oy, na, nb, ncr, nm, nf);
    }
    // entries 0 .. etop of the batch whose quadrant bit is set, last to first
    const int etop = min(hi, wave_top) - 1 - blo;
    int len = etop >= 0 ? build_list(L.m[buf], etop, list, 0u, 1u) : 0;
    while (len > 0 && list[len - 1] == uint16_t(kPad)) --len;
    for (int k = len - 1; k >= 0; --k) {
      const int e = list[k];
      const int j = blo + e;
      const float4 a = L.a[buf][e];
      const float4 b = L.b[buf][e];
      const float cb = L.c[buf][e];
      const float dx = fx - a.x, dy = fy - a.y;
      const float araw = fast_exp2(pair_q(a.z, a.w, b.x, b.y, dx, dy));   // o exp(-e)
      const float alpha = fminf(kAlphaCap, araw);
      const bool ok = j < s.top && alpha >= kAlphaMin;
      if (__ballot(ok) == 0) continue;
      // a pixel that does not blend this pair sees alpha 0: 1 / (1 - 0) is exactly 1,
      // so its T and S come through unchanged and all its partials are 0
      const float a_ok = ok ? alpha : 0.0f;
      const float inv = __builtin_amdgcn_rcpf(1.0f - a_ok);
      const float Tn = s.T * inv;           // transmittance in front of this pair
      const float w = a_ok * Tn;
      const float galpha =
          s.g0 * (b.z * Tn - s.S0 * inv) + s.g1 * (b.w * Tn - s.S1 * inv) + s.g2 * (cb * Tn - s.S2 * inv);
      const bool unc = ok && araw <= kAlphaCap;
      const float ge = unc ? -galpha * araw : 0.0f;   // dL/de = -o dL/do
      // the moments of dL/de over the pixels; the conic (and 1 / o for the opacity) is
      // applied when they are flushed
      float v[9];
      v[0] = ge * dx;
      v[1] = ge * dy;
      v[2] = v[0] * dx;
      v[3] = v[0] * dy;
      v[4] = v[1] * dy;
      v[5] = -ge;
      v[6] = s.g0 * w;
      v[7] = s.g1 * w;
      v[8] = s.g2 * w;
      s.S0 += b.z * w;
      s.S1 += b.w * w;
      s.S2 += cb * w;
      s.T = Tn;
      wave_sum9(v);
      if (FIXED) {
        int* acc = reinterpret_cast<int*>(&L.acc[e][0]);
        const int k = lane >> 3;
        const float sc = (k >= 2 && k <= 4) ? unit * L.inv_f[buf][e] : unit;
        if ((lane & 7) == 0) atomicAdd(&acc[k], to_fixed(v[0] * sc));
        if (lane == 0) atomicAdd(&acc[8], to_fixed(v[8] * unit));
      } else {
        if ((lane & 7) == 0) atomicAdd(&L.acc[e][lane >> 3], v[0]);
        if (lane == 0) atomicAdd(&L.acc[e][8], v[8]);
      }
    }
    if (tid < kBwdBatch && nlo < nhi) {
      L.a[buf ^ 1][tid] = na; L.b[buf ^ 1][tid] = nb; L.c[buf ^ 1][tid] = ncr; L.id[buf ^ 1][tid] = ng;
      L.m[buf ^ 1][tid] = nm;
      if (FIXED) L.inv_f[buf ^ 1][tid] = nf;
    }
    __syncthreads();
    if (!FIXED && tid < hi - blo) {
      // e = (A dx^2 + C dy^2) / 2 + B dx dy: du = -(A M_x + B M_y), dv = -(B M_x + C M_y),
      // dA = M_xx / 2, dB = M_xy, dC = M_yy / 2 for the moments M of dL/de
      // (the unscaled conic back from the staged coefficients: a' = -log2(e) A / 2, ...)
      const float cA = L.a[buf][tid].z * (-2.0f / kLog2e), cB = L.a[buf][tid].w * (-1.0f / kLog2e),
                  cC = L.b[buf][tid].x * (-2.0f / kLog2e);
      const float mx = L.acc[tid][0], my = L.acc[tid][1];
      L.acc[tid][0] = -(cA * mx + cB * my);
      L.acc[tid][1] = -(cB * mx + cC * my);
      L.acc[tid][2] *= 0.5f;
      L.acc[tid][4] *= 0.5f;
      // the opacity's sum is o dL/do (nonzero only if some pixel blended, so o > 0)
      const float so = L.acc[tid][5];
      if (so != 0.0f) L.acc[tid][5] = so * fast_exp2(-L.b[buf][tid].y);
    }
    if (!FIXED) __syncthreads();
    {
      // one thread per (entry, partial) in gscreen's own order, so that the atomics of a
      // wave land on a few cache lines (about 7 entries of 36 bytes) instead of 64
      float* flat = &L.acc[0][0];
      const int cnt9 = (hi - blo) * 9;
      for (int idx = tid; idx < cnt9; idx += kBlock) {
        const int e = idx / 9;
        const size_t o = size_t(L.id[buf][e]) * 9 + (idx - 9 * e);
        if (FIXED) {
          const int x = __float_as_int(flat[idx]);
          if (x != 0) atomicAdd(&acc64[o], (unsigned long long)(long long)x);
        } else {
          const float x = flat[idx];
          if (x != 0.0f) atomicAdd(&gscreen[o], x);
        }
        flat[idx] = 0.0f;
      }
    }
    __syncthreads();
    hi = blo;
    buf ^= 1;
  }
}

struct BwdArgs {
  const float4* splat;
  const uint32_t* vals;
  const uint32_t* ranges;
  int num_tiles, tx, W, H;
  uint32_t pairs;
  float bg0, bg1, bg2;
  int first, chunk;
  const float* T_final;
  const uint32_t* n_contrib;
  const float* dL_dimg;
  int n;
  float* gscreen;
  unsigned long long* acc64;   // fixed-point sums: [n][9] i64 accumulators
  float unit;                  // fixed-point sums: 16384 times the loss's element count
};

// A tile's first segment (the whole list for tiles that were not split).
template <bool FIXED>
__device__ void bwd_tile(BwdLds& L, const BwdArgs& A, const SplitWs& ws, int tile) {
  const float4* __restrict__ splat = A.splat;
  const uint32_t* __restrict__ vals = A.vals;
  const uint32_t* __restrict__ ranges = A.ranges;
  const int tx = A.tx, W = A.W, H = A.H, first = A.first;
  const float bg0 = A.bg0, bg1 = A.bg1, bg2 = A.bg2;
  const float* __restrict__ T_final = A.T_final;
  const uint32_t* __restrict__ n_contrib = A.n_contrib;
  const float* __restrict__ dL_dimg = A.dL_dimg;
  float* __restrict__ gscreen = A.gscreen;
  const int tid = threadIdx.x;
  const int px = (tile % tx) * kTile + pixel_x(tid);
  const int py = (tile / tx) * kTile + pixel_y(tid);
  const bool inside = px < W && py < H;
  const uint32_t start = ranges[tile];
  PixelBwd s{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0};
  if (inside) {
    const int HW = W * H, p = py * W + px;
    s.g0 = dL_dimg[p];
    s.g1 = dL_dimg[HW + p];
    s.g2 = dL_dimg[2 * HW + p];
    const int32_t slot = ws.slot_of_tile[tile];
    if (slot >= 0 && is_split(ws.state[slot]) && ws.stopc[size_t(slot) * 256 + tid] >= 0) {
      // the pixel's pairs continue past the first segment: start from its end state
      const float4 b = ws.bnd1[size_t(slot) * 256 + tid];
      s.T = b.x; s.S0 = b.y; s.S1 = b.z; s.S2 = b.w;
      s.top = first;
    } else {
      s.T = T_final[p];
      s.S0 = bg0 * s.T; s.S1 = bg1 * s.T; s.S2 = bg2 * s.T;
      s.top = int(n_contrib[p]);
    }
  }
  bwd_walk<FIXED>(L, splat, vals, start, 0, tile_ox(tile, tx), tile_oy(tile, tx), float(px) + 0.5f, float(py) + 0.5f,
                  s, gscreen, A.acc64, A.unit);
}

// One chunk of a split tile.
template <bool FIXED>
__device__ void bwd_chunk(BwdLds& L, const BwdArgs& A, const SplitWs& ws, uint32_t item) {
  const float4* __restrict__ splat = A.splat;
  const uint32_t* __restrict__ vals = A.vals;
  const uint32_t* __restrict__ ranges = A.ranges;
  const int num_tiles = A.num_tiles, tx = A.tx, W = A.W, H = A.H, first = A.first, chunk = A.chunk;
  const float bg0 = A.bg0, bg1 = A.bg1, bg2 = A.bg2;
  const float* __restrict__ T_final = A.T_final;
  const uint32_t* __restrict__ n_contrib = A.n_contrib;
  const float* __restrict__ dL_dimg = A.dL_dimg;
  float* __restrict__ gscreen = A.gscreen;
  const uint2 sc = ws.items[item];
  const uint32_t slot = sc.x, c = sc.y;
  if (!is_split(ws.state[slot])) return;   // a candidate that its first segment finished
  const int tile = int(ws.slot_tile[slot]);
  const int tid = threadIdx.x;
  const int px = (tile % tx) * kTile + pixel_x(tid);
  const int py = (tile / tx) * kTile + pixel_y(tid);
  const bool inside = px < W && py < H;
  const uint32_t start = ranges[tile];
  const int len = int(ranges[num_tiles + tile] - start);
  const int lo = first + int(c) * chunk, hi = min(lo + chunk, len);
  const size_t so = size_t(slot) * 256 + tid;
  PixelBwd s{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, lo};
  const int32_t stop = ws.stopc[so];
  if (inside && stop >= int32_t(c)) {
    const int HW = W * H, p = py * W + px;
    s.g0 = dL_dimg[p];
    s.g1 = dL_dimg[HW + p];
    s.g2 = dL_dimg[2 * HW + p];
    if (stop == int32_t(c)) {
      s.T = T_final[p];
      s.S0 = bg0 * s.T; s.S1 = bg1 * s.T; s.S2 = bg2 * s.T;
      s.top = int(n_contrib[p]);
    } else {
      const float4 b = ws.part4[size_t(item) * 256 + tid];
      s.T = b.x; s.S0 = b.y; s.S1 = b.z; s.S2 = b.w;
      s.top = hi;
    }
  }
  bwd_walk<FIXED>(L, splat, vals, start, lo, tile_ox(tile, tx), tile_oy(tile, tx), float(px) + 0.5f, float(py) + 0.5f,
                  s, gscreen, A.acc64, A.unit);
}

// The backward of every tile's first segment and of every chunk of the split tiles,
// in one launch: blocks [0, num_tiles) take the tiles longest first, the blocks
// after them the chunks, which are independent of the first segments (each starts
// from the state the forward left at its end) and so fill the CUs that the last
// long first segments leave idle.  The split sizes and the split state's layout come
// from the forward's header; the chunk blocks step through the forward's chunks
// `chunk_blocks` apart, so every chunk is walked whatever the launch size.  A header
// that no matching forward wrote makes every block return (the zeroing kernel then
// wrote NaN partials).
template <bool FIXED>
__global__ void __launch_bounds__(256) render_bwd_kernel(BwdArgs A, HeaderCheck hc, char* split_base,
                                                         uint32_t chunk_blocks) {
  __shared__ BwdLds L;
  RenderHeader h;
  if (!header_ok(hc, h)) return;
  const SplitWs ws = carve(split_base, split_dims(A.W, A.H, A.pairs, int(h.first), int(h.chunk)));
  A.first = int(h.first);
  A.chunk = int(h.chunk);
  const uint32_t b = blockIdx.x;
  if (b < uint32_t(A.num_tiles)) {
    bwd_tile<FIXED>(L, A, ws, int(ws.order[b]));
  } else {
    const uint32_t items = ws.counters[1];
    for (uint32_t item = b - uint32_t(A.num_tiles); item < items; item += chunk_blocks) {
      __syncthreads();   // the previous chunk's walk is done with the shared state
      bwd_chunk<FIXED>(L, A, ws, item);
    }
  }
}

// Fixed-point sums back to the partials: acc64[i] holds the i64 sums of the moments
// M_x, M_y, M_xx, M_xy, M_yy (the second moments divided by the size factor), of o dL/do
// and of the colour partials, all times `unit`; with the record's own conic and opacity
// (the values the walks used): du = -(A M_x + B M_y), dv = -(B M_x + C M_y), dA = M_xx / 2,
// dB = M_xy, dC = M_yy / 2, d opacity = (o dL/do) / o.  NaN everywhere if the walk did
// not run (header check failed).
__global__ void __launch_bounds__(256) fixed_decode_kernel(int n, const float4* __restrict__ splat,
                                                            const unsigned long long* __restrict__ acc64,
                                                            float* __restrict__ gscreen, float unit,
                                                            HeaderCheck hc) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float* g = gscreen + size_t(i) * 9;
  RenderHeader h;
  if (!header_ok(hc, h)) {
#pragma unroll
    for (int k = 0; k < 9; ++k) g[k] = __builtin_nanf("");
    return;
  }
  float q[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) q[k] = float((long long)acc64[size_t(i) * 9 + k]);
  const float4 r0 = splat[3 * i], r1 = splat[3 * i + 1];
  const float A = r0.z, B = r0.w, C = r1.x, o = r1.y;
  const float f = fixed_size_factor(A, B, C);
  const float mx = q[0] / unit, my = q[1] / unit;
  const float mxx = q[2] * f / unit, mxy = q[3] * f / unit, myy = q[4] * f / unit;
  g[0] = -(A * mx + B * my);
  g[1] = -(B * mx + C * my);
  g[2] = 0.5f * mxx;
  g[3] = mxy;
  g[4] = 0.5f * myy;
  g[5] = q[5] != 0.0f ? (q[5] / unit) / o : 0.0f;
#pragma unroll
  for (int k = 6; k < 9; ++k) g[k] = q[k] / unit;
}

// gscreen cleared before the walk adds to it, or NaN if the walk will not run (header
// check failed).  16-byte non-temporal stores over count4 groups of four floats (a pure
// write stream), then the count % 4 floats left.
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Grid-stride: a few thousand blocks, each thread storing 16 bytes per step.
__global__ void __launch_bounds__(256) zero_f32x4_kernel(f32x4* __restrict__ p, int64_t count4,
                                                          float* __restrict__ tail, int64_t ntail, HeaderCheck hc) {
  const int64_t i0 = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  RenderHeader h;
  const float v = header_ok(hc, h) ? 0.0f : __builtin_nanf("");
  for (int64_t i = i0; i < count4; i += stride) __builtin_nontemporal_store(f32x4{v, v, v, v}, p + i);
  for (int64_t i = i0; i < ntail; i += stride) tail[i] = v;   // all of it when p is not 16-byte aligned
}

__global__ void zero_u64_kernel(unsigned long long* __restrict__ p, int64_t count) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < count) p[i] = 0ull;
}

}  // namespace

size_t render_ws_bytes(int W, int H, uint32_t pairs, int first, int chunk, int64_t n_fixed) {
  return kHeaderBytes + carve_bytes(split_dims(W, H, pairs, first, chunk)) + a256(size_t(n_fixed) * 9 * 8);
}

hipError_t launch_render_fwd(const gs_proj& proj, const uint32_t* vals, const uint32_t* ranges,
                             const gs_camera& cam, uint32_t pairs, float* rgb, float* T_final,
                             uint32_t* n_contrib, void* wsp, int first, int chunk, hipStream_t s) {
  const int tx = tiles_x(cam), ty = tiles_y(cam);
  const int num_tiles = tx * ty;
  const SplitDims d = split_dims(cam.width, cam.height, pairs, first, chunk);
  const SplitWs ws = carve(static_cast<char*>(wsp) + kHeaderBytes, d);
  const RenderHeader h{kHeaderMagic, uint32_t(first), uint32_t(chunk), uint32_t(num_tiles), pairs,
                       uint32_t(cam.width), uint32_t(cam.height), 0u, uint64_t(carve_bytes(d))};
  const float4* splat = reinterpret_cast<const float4*>(proj.splat);
  {
    GSK_PROF("tile_order", s);
    tile_order_kernel<<<1, 1024, 0, s>>>(ranges, num_tiles, ws, first, chunk, static_cast<RenderHeader*>(wsp), h);
  }
  const bool split = pairs > uint32_t(first);
  if (split) {
    GSK_PROF("split_reset", s);
    split_reset_kernel<<<unsigned(d.S), 256, 0, s>>>(ws);
  }
  {
    GSK_PROF("render_fwd", s);
    const unsigned blocks = unsigned(num_tiles) + (split ? unsigned(d.I) : 0u);
    render_fwd_kernel<<<blocks, 256, 0, s>>>(splat, vals, ranges, ws, num_tiles, tx, cam.width, cam.height, cam.bg[0],
                                             cam.bg[1], cam.bg[2], first, chunk, rgb, T_final, n_contrib);
  }
  if (split) {
    const unsigned items = unsigned(d.I), slots = unsigned(d.S);
    {
      GSK_PROF("split_combine", s);
      split_combine_kernel<<<slots, 1024, 0, s>>>(ws);
    }
    {
      GSK_PROF("split_rewalk", s);
      split_rewalk_kernel<<<items, 256, 0, s>>>(splat, vals, ranges, ws, num_tiles, tx, first, chunk);
    }
    {
      GSK_PROF("split_finalize", s);
      split_finalize_kernel<<<slots, 256, 0, s>>>(ws, tx, cam.width, cam.height, cam.bg[0], cam.bg[1], cam.bg[2], rgb,
                                                  T_final, n_contrib);
    }
  }
  return hipGetLastError();
}

hipError_t launch_render_bwd(const gs_proj& proj, int n, const uint32_t* vals, const uint32_t* ranges,
                             const gs_camera& cam, uint32_t pairs, const float* T_final, const uint32_t* n_contrib,
                             const float* dL_dimg, float* gscreen, void* wsp, size_t ws_bytes, int first, int chunk,
                             bool fixed, hipStream_t s) {
  const int tx = tiles_x(cam), ty = tiles_y(cam);
  const int num_tiles = tx * ty;
  // the launch is sized with the caller's split sizes; the walk uses the forward's (header)
  const SplitDims d = split_dims(cam.width, cam.height, pairs, first, chunk);
  char* base = static_cast<char*>(wsp);
  // fixed-point accumulators at the end of the workspace (the caller checked that it holds
  // them after a split state of the caller's split sizes), so that their place does not
  // depend on the split sizes; the header check keeps the forward's split state before them
  const size_t acc_off = fixed ? ((ws_bytes - size_t(n) * 9 * 8) & ~size_t(255)) : ws_bytes;
  unsigned long long* acc64 = fixed ? reinterpret_cast<unsigned long long*>(base + acc_off) : nullptr;
  const uint64_t avail = acc_off - kHeaderBytes;
  const HeaderCheck hc{reinterpret_cast<const RenderHeader*>(base), num_tiles, cam.width, cam.height, pairs, avail};
  const float4* splat = reinterpret_cast<const float4*>(proj.splat);
  if (n > 0) {
    if (fixed) {
      GSK_PROF("zero_u64", s);
      const int64_t count = 9 * int64_t(n);
      zero_u64_kernel<<<div_up(count, 256), 256, 0, s>>>(acc64, count);
    } else {
      GSK_PROF("zero_f32", s);
      const int64_t count = 9 * int64_t(n);
      const bool vec = reinterpret_cast<uintptr_t>(gscreen) % 16 == 0;
      const int64_t count4 = vec ? count / 4 : 0;
      const int64_t ntail = count - 4 * count4;
      const int64_t threads = count4 > ntail ? count4 : ntail;
      const unsigned blocks = div_up(threads, 256) < 2048u ? div_up(threads, 256) : 2048u;
      zero_f32x4_kernel<<<blocks, 256, 0, s>>>(reinterpret_cast<f32x4*>(gscreen), count4, gscreen + 4 * count4,
                                               ntail, hc);
    }
  }
  const float unit = kFixedUnit * 3.0f * float(cam.width) * float(cam.height);
  const BwdArgs A{splat, vals, ranges, num_tiles, tx, cam.width, cam.height, pairs, cam.bg[0], cam.bg[1], cam.bg[2],
                  0, 0, T_final, n_contrib, dL_dimg, n, gscreen, acc64, unit};
  const uint32_t chunk_blocks = pairs > 0 ? uint32_t(d.I) : 0u;
  const unsigned blocks = unsigned(num_tiles) + chunk_blocks;
  {
    GSK_PROF("render_bwd", s);
    if (fixed)
      render_bwd_kernel<true><<<blocks, 256, 0, s>>>(A, hc, base + kHeaderBytes, chunk_blocks);
    else
      render_bwd_kernel<false><<<blocks, 256, 0, s>>>(A, hc, base + kHeaderBytes, chunk_blocks);
  }
  if (fixed && n > 0) {
    GSK_PROF("fixed_decode", s);
    fixed_decode_kernel<<<div_up(n, 256), 256, 0, s>>>(n, splat, acc64, gscreen, unit, hc);
  }
  return hipGetLastError();
}

}  // namespace gsk
