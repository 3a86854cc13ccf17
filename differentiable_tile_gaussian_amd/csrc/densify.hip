// Density control: per-step gradient statistics and one densification (clone, split,
// prune, opacity reset) of the blocked population.
//
// [GST] density-control slide: the screen-space centre gradient magnitude of every visible
// observation is accumulated and averaged over the observations; small Gaussians with a
// large average are cloned (an exact copy), large ones split into two children sampled
// around the parent with smaller scales, very transparent or oversized ones pruned; an
// opacity reset clamps opacity to at most a cap.  [GSG] "Densification": split halves
// shrink by 1.6 and a reshaped Gaussian starts with zero Adam moments.
//
// The new population is: the kept Gaussians in their order, then the clones, then the
// first and then the second children of the split ones (each group in the order of its
// parents).  A Gaussian's destination is a prefix sum of per-Gaussian flags, so the
// result does not depend on scheduling.  Decisions compare the stored logit and
// log-scales against thresholds rounded once from double on the host.
//
// Compiled without floating-point contraction: the split children's means are the
// written sequence of fp32 roundings.
#include "gs_internal.h"
#include "profile.h"

namespace gsk {
namespace {

// The std::max / std::min of the C++ library (NaN handling included).
__device__ inline float max_of(float a, float b) { return a < b ? b : a; }
__device__ inline float min_of(float a, float b) { return b < a ? b : a; }

enum : uint32_t { kPrune = 0, kKeep = 1, kClone = 2, kSplit = 3 };

__device__ inline uint32_t action(const float* g0, float2 st, const DensifyArgs& a) {
  const float lsmax = max_of(max_of(g0[3 * kGB], g0[4 * kGB]), g0[5 * kGB]);
  if (g0[10 * kGB] < a.logit_prune || lsmax > a.lscale_prune) return kPrune;
  const float avg = st.y > 0.0f ? st.x / st.y : 0.0f;
  if (!(avg >= a.grad_thr)) return kKeep;
  return lsmax > a.lscale_split ? kSplit : kClone;
}

__global__ void __launch_bounds__(256) densify_accumulate_kernel(int n, const uint32_t* __restrict__ tiles,
                                                                  const float* __restrict__ gscreen,
                                                                  float2* __restrict__ stats) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n || tiles[i] == 0u) return;
  const float du = gscreen[size_t(i) * 9], dv = gscreen[size_t(i) * 9 + 1];
  float2 s = stats[i];
  s.x += sqrtf(du * du + dv * dv);
  s.y += 1.0f;
  stats[i] = s;
}

// Flags of each Gaussian for the three prefix sums: kept, cloned, split.
__global__ void __launch_bounds__(256) densify_classify_kernel(const float* __restrict__ params, int n, int P,
                                                                const float2* __restrict__ stats, DensifyArgs a,
                                                                uint32_t* __restrict__ fkeep,
                                                                uint32_t* __restrict__ fclone,
                                                                uint32_t* __restrict__ fsplit) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t act = action(gaussian_base(params, i, P), stats[i], a);
  fkeep[i] = act == kKeep || act == kClone;
  fclone[i] = act == kClone;
  fsplit[i] = act == kSplit;
}

// Mean of a split child: mean + Rq (s * eps), Rq from the normalised quaternion (the
// identity for a zero one), s = exp(log-scales) rounded once from double.
__device__ inline void child_mean(const float* g0, const float* eps, float* out) {
  float s[3];
#pragma unroll
  for (int k = 0; k < 3; ++k) s[k] = float(exp(double(g0[(3 + k) * kGB])));
  float R[3][3] = {{1.f, 0.f, 0.f}, {0.f, 1.f, 0.f}, {0.f, 0.f, 1.f}};
  const float q0 = g0[6 * kGB], q1 = g0[7 * kGB], q2 = g0[8 * kGB], q3 = g0[9 * kGB];
  const float n2 = ((q0 * q0 + q1 * q1) + q2 * q2) + q3 * q3;
  if (n2 > 0.0f) {
    const float ql = sqrtf(n2);
    const float w = q0 / ql, x = q1 / ql, y = q2 / ql, z = q3 / ql;
    R[0][0] = 1.0f - 2.0f * (y * y + z * z);
    R[0][1] = 2.0f * (x * y - w * z);
    R[0][2] = 2.0f * (x * z + w * y);
    R[1][0] = 2.0f * (x * y + w * z);
    R[1][1] = 1.0f - 2.0f * (x * x + z * z);
    R[1][2] = 2.0f * (y * z - w * x);
    R[2][0] = 2.0f * (x * z - w * y);
    R[2][1] = 2.0f * (y * z + w * x);
    R[2][2] = 1.0f - 2.0f * (x * x + y * y);
  }
  const float d[3] = {s[0] * eps[0], s[1] * eps[1], s[2] * eps[2]};
#pragma unroll
  for (int r = 0; r < 3; ++r) out[r] = g0[r * kGB] + ((R[r][0] * d[0] + R[r][1] * d[1]) + R[r][2] * d[2]);
}

// Writes Gaussian g0 (its theta, m, v rows) as output d: fresh ones get zero moments;
// a child gets its own mean and the log-scales lowered by the shrink.  The planes go in
// groups of kPutGroup, all of a group's loads before its stores (the input and output
// arrays do not overlap), so that a thread keeps that many loads in flight.
constexpr int kPutGroup = 8;
__device__ inline void put(const float* __restrict__ g0, const float* __restrict__ m0, const float* __restrict__ v0,
                           float* __restrict__ params_out, float* __restrict__ m_out, float* __restrict__ v_out,
                           float2* __restrict__ stats_out, int d, int P, bool fresh, const float* mean,
                           const DensifyArgs& a) {
  float* gp = gaussian_base(params_out, d, P);
  float* gm = gaussian_base(m_out, d, P);
  float* gv = gaussian_base(v_out, d, P);
  for (int k0 = 0; k0 < P; k0 += kPutGroup) {
    float th[kPutGroup], mo[kPutGroup], vo[kPutGroup];
#pragma unroll
    for (int j = 0; j < kPutGroup; ++j) {
      const int k = k0 + j;
      th[j] = mo[j] = vo[j] = 0.0f;
      if (k < P) {
        th[j] = g0[k * kGB];
        if (!fresh) {
          mo[j] = m0[k * kGB];
          vo[j] = v0[k * kGB];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kPutGroup; ++j) {
      const int k = k0 + j;
      if (k < P) {
        float t = th[j], mm = mo[j], vv = vo[j];
        if (mean && k < 3) t = mean[k];
        if (mean && k >= 3 && k < 6) t = t - a.lscale_shrink;
        if (a.reset && k == 10) {
          t = min_of(t, a.logit_cap);
          mm = vv = 0.0f;
        }
        gp[k * kGB] = t;
        gm[k * kGB] = mm;
        gv[k * kGB] = vv;
      }
    }
  }
  stats_out[d] = make_float2(0.0f, 0.0f);
}

// The source of every place in the new population, one thread per source Gaussian: kept
// ones at their place (the prefix sum of the kept flags) in src_keep; cloned and split ones
// at their place among the clones or the split parents in src.
__global__ void __launch_bounds__(256) densify_index_kernel(int n, const uint32_t* __restrict__ fkeep,
                                                            const uint32_t* __restrict__ fclone,
                                                            const uint32_t* __restrict__ fsplit,
                                                            const uint32_t* __restrict__ offs_keep,
                                                            const uint32_t* __restrict__ offs_clone,
                                                            const uint32_t* __restrict__ offs_split, uint32_t cloned,
                                                            uint32_t* __restrict__ src_keep,
                                                            uint32_t* __restrict__ src) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (fkeep[i]) src_keep[offs_keep[i]] = uint32_t(i);
  if (fclone[i]) src[offs_clone[i]] = uint32_t(i);
  if (fsplit[i]) src[cloned + offs_split[i]] = uint32_t(i);
}

// The new population, one thread per place j (kept, then clones, then first and second
// children), so that a wave writes whole rows of the blocked layout; each thread reads its
// source's rows (a wave's kept sources are nearly consecutive; the new ones' moments start
// at zero and are not read).
__global__ void __launch_bounds__(256) densify_write_kernel(const float* __restrict__ params,
                                                            const float* __restrict__ m, const float* __restrict__ v,
                                                            int P, const float* __restrict__ rand,
                                                            const uint32_t* __restrict__ src_keep,
                                                            const uint32_t* __restrict__ src, uint32_t kept,
                                                            uint32_t cloned, uint32_t splits, DensifyArgs a,
                                                            float* __restrict__ params_out, float* __restrict__ m_out,
                                                            float* __restrict__ v_out, float2* __restrict__ stats_out) {
  const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t t = j - int64_t(kept);
  if (t >= int64_t(cloned) + 2 * int64_t(splits)) return;
  if (t < 0) {
    const int i = int(src_keep[j]);
    put(gaussian_base(params, i, P), gaussian_base(m, i, P), gaussian_base(v, i, P), params_out, m_out, v_out,
        stats_out, int(j), P, false, nullptr, a);
    return;
  }
  if (t < int64_t(cloned)) {
    const int i = int(src[t]);
    put(gaussian_base(params, i, P), nullptr, nullptr, params_out, m_out, v_out, stats_out, int(j), P, true, nullptr,
        a);
    return;
  }
  const int64_t u = t - int64_t(cloned);
  const int c = u >= int64_t(splits) ? 1 : 0;
  const int i = int(src[int64_t(cloned) + u - int64_t(c) * splits]);
  const float* g0 = gaussian_base(params, i, P);
  float mean[3];
  child_mean(g0, rand + (size_t(2) * i + c) * 3, mean);
  put(g0, nullptr, nullptr, params_out, m_out, v_out, stats_out, int(j), P, true, mean, a);
}

// ---- relocation of the dead ([GSG] "Densification", the MCMC-style pass)
// Dead: logit below logit(dead opacity); donor: not dead, logit above logit(donor
// opacity) and a largest log-scale that is not NaN.  key: the largest log-scale (-0 made
// +0) as an unsigned integer in the order of the floats, bit-inverted, so that a stable
// ascending radix sort ranks the donors largest first with equal sizes in index order.
__global__ void __launch_bounds__(256) relocate_classify_kernel(const float* __restrict__ params, int n, int P,
                                                                 float logit_dead, float logit_donor,
                                                                 uint32_t* __restrict__ fdead,
                                                                 uint32_t* __restrict__ fdonor,
                                                                 uint32_t* __restrict__ key) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float* g0 = gaussian_base(params, i, P);
  const float logit = g0[10 * kGB];
  const float lsmax = max_of(max_of(g0[3 * kGB], g0[4 * kGB]), g0[5 * kGB]);
  const bool dead = logit < logit_dead;
  fdead[i] = dead;
  fdonor[i] = !dead && logit > logit_donor && lsmax == lsmax;
  const uint32_t u = __float_as_uint(lsmax + 0.0f);
  key[i] = ~((u & 0x80000000u) ? ~u : (u | 0x80000000u));
}

// The dead in index order, and the donors' keys and indices in index order.
__global__ void __launch_bounds__(256) relocate_compact_kernel(int n, const uint32_t* __restrict__ fdead,
                                                                const uint32_t* __restrict__ fdonor,
                                                                const uint32_t* __restrict__ odead,
                                                                const uint32_t* __restrict__ odonor,
                                                                const uint32_t* __restrict__ key,
                                                                uint32_t* __restrict__ dead_list,
                                                                uint32_t* __restrict__ key_in,
                                                                uint32_t* __restrict__ idx_in) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (fdead[i]) dead_list[odead[i]] = uint32_t(i);
  if (fdonor[i]) {
    key_in[odonor[i]] = key[i];
    idx_in[odonor[i]] = uint32_t(i);
  }
}

// Move k: the k-th dead Gaussian takes the k-th ranked donor, placed at mean + Rq (s eps)
// with its own normals, both log-scales lowered by the shrink, both moments zeroed.  The
// dead and the donors are disjoint and each is used once, so the moves are independent;
// a thread reads its donor before it writes the donor's log-scales.
__global__ void __launch_bounds__(256) relocate_move_kernel(float* __restrict__ params, float* __restrict__ m,
                                                             float* __restrict__ v, int P,
                                                             const float* __restrict__ rand,
                                                             const uint32_t* __restrict__ dead_list,
                                                             const uint32_t* __restrict__ donor_ranked, int moves,
                                                             float shrink) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  if (k >= moves) return;
  const int bi = int(dead_list[k]), bd = int(donor_ranked[k]);
  float* gd = gaussian_base(params, bd, P);
  float* gi = gaussian_base(params, bi, P);
  float* md = gaussian_base(m, bd, P);
  float* mi = gaussian_base(m, bi, P);
  float* vd = gaussian_base(v, bd, P);
  float* vi = gaussian_base(v, bi, P);
  float mean[3];
  child_mean(gd, rand + size_t(3) * bi, mean);
  for (int pl = 0; pl < P; ++pl) {
    float th = gd[pl * kGB];
    if (pl < 3) th = mean[pl];
    if (pl >= 3 && pl < 6) th = th - shrink;
    gi[pl * kGB] = th;
    mi[pl * kGB] = vi[pl * kGB] = 0.0f;
    md[pl * kGB] = vd[pl * kGB] = 0.0f;
  }
  for (int pl = 3; pl < 6; ++pl) gd[pl * kGB] = gd[pl * kGB] - shrink;
}

}  // namespace

// Relocation workspace: two flag arrays and their prefix sums and scan space, the two
// totals, the keys, the dead list, the donors' keys and indices, and the space of the
// sort that ranks them.
RelocateWs carve_relocate(void* ws, int64_t n) {
  char* base = static_cast<char*>(ws);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* q = base ? base + off : nullptr;
    off += (bytes + 255) & ~size_t(255);
    return q;
  };
  const size_t items = size_t(n > 0 ? n : 1) * 4;
  RelocateWs w;
  w.fdead = reinterpret_cast<uint32_t*>(take(items));
  w.fdonor = reinterpret_cast<uint32_t*>(take(items));
  w.odead = reinterpret_cast<uint32_t*>(take(size_t(n + 1) * 4));
  w.odonor = reinterpret_cast<uint32_t*>(take(size_t(n + 1) * 4));
  w.totals = reinterpret_cast<uint64_t*>(take(16));
  w.scan_ws[0] = take(scan_ws_bytes(n));
  w.scan_ws[1] = take(scan_ws_bytes(n));
  w.key = reinterpret_cast<uint32_t*>(take(items));
  w.dead_list = reinterpret_cast<uint32_t*>(take(items));
  w.key_in = reinterpret_cast<uint32_t*>(take(items));
  w.idx_in = reinterpret_cast<uint32_t*>(take(items));
  w.sort_ws = take(sort_pairs_ws_bytes(n));
  w.bytes = off;
  return w;
}

size_t relocate_ws_bytes(int64_t n) { return carve_relocate(nullptr, n).bytes; }

hipError_t launch_relocate_count(const float* params, int n, int deg, float logit_dead, float logit_donor, void* ws,
                                 hipStream_t s) {
  RelocateWs w = carve_relocate(ws, n);
  {
    GSK_PROF("relocate_classify", s);
    relocate_classify_kernel<<<div_up(n, 256), 256, 0, s>>>(params, n, num_planes(deg), logit_dead, logit_donor,
                                                            w.fdead, w.fdonor, w.key);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_scan_u32(w.fdead, w.odead, n, w.totals, w.scan_ws[0], s);
  if (e != hipSuccess) return e;
  e = launch_scan_u32(w.fdonor, w.odonor, n, w.totals + 1, w.scan_ws[1], s);
  if (e != hipSuccess) return e;
  relocate_compact_kernel<<<div_up(n, 256), 256, 0, s>>>(n, w.fdead, w.fdonor, w.odead, w.odonor, w.key,
                                                         w.dead_list, w.key_in, w.idx_in);
  return hipGetLastError();
}

hipError_t launch_relocate_move(float* params, float* m, float* v, int n, int deg, const float* rand, int donors,
                                int moves, float shrink, void* ws, hipStream_t s) {
  RelocateWs w = carve_relocate(ws, n);
  if (moves <= 0) return hipSuccess;
  const hipError_t e = launch_sort_pairs_u32(w.key_in, w.idx_in, uint32_t(donors), n, w.sort_ws, s);
  if (e != hipSuccess) return e;
  GSK_PROF("relocate_move", s);
  relocate_move_kernel<<<div_up(moves, 256), 256, 0, s>>>(params, m, v, num_planes(deg), rand, w.dead_list,
                                                          w.idx_in, moves, shrink);
  return hipGetLastError();
}

hipError_t launch_densify_accumulate(const uint32_t* tiles, int n, const float* gscreen, float* stats,
                                     hipStream_t s) {
  if (n == 0) return hipSuccess;
  GSK_PROF("densify_accumulate", s);
  densify_accumulate_kernel<<<div_up(n, 256), 256, 0, s>>>(n, tiles, gscreen, reinterpret_cast<float2*>(stats));
  return hipGetLastError();
}

size_t densify_ws_bytes(int64_t n) {
  const size_t flags = (size_t(n > 0 ? n : 1) * 4 + 255) & ~size_t(255);
  const size_t offs = (size_t(n + 1) * 4 + 255) & ~size_t(255);
  return 5 * flags + 3 * offs + 256 + 3 * ((scan_ws_bytes(n) + 255) & ~size_t(255));
}

hipError_t launch_densify_count(const float* params, int n, int deg, const float* stats, const DensifyArgs& a,
                                void* ws, hipStream_t s) {
  DensifyWs w = carve_densify(ws, n);
  const int P = num_planes(deg);
  {
    GSK_PROF("densify_classify", s);
    densify_classify_kernel<<<div_up(n, 256), 256, 0, s>>>(params, n, P, reinterpret_cast<const float2*>(stats), a,
                                                           w.flag[0], w.flag[1], w.flag[2]);
  }
  hipError_t e = hipGetLastError();
  for (int k = 0; k < 3 && e == hipSuccess; ++k)
    e = launch_scan_u32(w.flag[k], w.offs[k], n, w.totals + k, w.scan_ws[k], s);
  return e;
}

hipError_t launch_densify_write(const float* params, const float* m, const float* v, int n, int deg,
                                const float* rand, const DensifyArgs& a, void* ws, uint32_t kept, uint32_t cloned,
                                uint32_t splits, float* params_out, float* m_out, float* v_out, float* stats_out,
                                hipStream_t s) {
  DensifyWs w = carve_densify(ws, n);
  {
    GSK_PROF("densify_index", s);
    densify_index_kernel<<<div_up(n, 256), 256, 0, s>>>(n, w.flag[0], w.flag[1], w.flag[2], w.offs[0], w.offs[1],
                                                        w.offs[2], cloned, w.src_keep, w.src);
  }
  const int64_t total = int64_t(kept) + int64_t(cloned) + 2 * int64_t(splits);
  if (total > 0) {
    GSK_PROF("densify_write", s);
    densify_write_kernel<<<div_up(total, 256), 256, 0, s>>>(params, m, v, num_planes(deg), rand, w.src_keep, w.src,
                                                            kept, cloned, splits, a, params_out, m_out, v_out,
                                                            reinterpret_cast<float2*>(stats_out));
  }
  return hipGetLastError();
}

DensifyWs carve_densify(void* ws, int64_t n) {
  char* p = static_cast<char*>(ws);
  DensifyWs w;
  const size_t flags = (size_t(n > 0 ? n : 1) * 4 + 255) & ~size_t(255);
  const size_t offs = (size_t(n + 1) * 4 + 255) & ~size_t(255);
  const size_t sw = (scan_ws_bytes(n) + 255) & ~size_t(255);
  for (int k = 0; k < 3; ++k) {
    w.flag[k] = reinterpret_cast<uint32_t*>(p);
    p += flags;
  }
  for (int k = 0; k < 3; ++k) {
    w.offs[k] = reinterpret_cast<uint32_t*>(p);
    p += offs;
  }
  w.totals = reinterpret_cast<uint64_t*>(p);
  p += 256;
  for (int k = 0; k < 3; ++k) {
    w.scan_ws[k] = p;
    p += sw;
  }
  w.src_keep = reinterpret_cast<uint32_t*>(p);
  w.src = reinterpret_cast<uint32_t*>(p + flags);
  return w;
}

}  // namespace gsk
