// Bucket-cache builder: normalise + pool + capped Ward per 512-key block, and
// the tree levels above the buckets.
//
// [catalog "Key points"]: keys are L2-normalised, pooled 4 at a time, and
// merged by Ward's method inside each 512-key block into buckets of about 8
// and at most 16 keys, each stored as a normalised centroid.
// [visual "How the hierarchy is built"]: the pooled key is the SUM of the 4
// unit keys; a full block is merged bottom-up into a fixed number of buckets;
// each bucket stores its centroid and the positions it holds; the tree
// variant repeats the process on the buckets.
//
// One workgroup (256 threads, 4 wave64) owns one block (or one tree group of
// up to 128 nodes).  All clustering state lives in LDS in fp64: the cluster
// means (128 x 64), the packed upper triangle of pairwise Ward costs
// (8,128 entries), and per-row nearest feasible partners.  Ward's cost is
// reducible, so after merging a and b only row a and rows whose nearest
// partner was a or b need a rescan; every other row only compares against
// the new cluster.  About 131 KiB of LDS per workgroup (gfx950 has 160 KiB).
#include "lsa_internal.h"

namespace lsa {
namespace {

constexpr int kThreads = 256;
constexpr int kN = 128;                 // items per group
constexpr int kStride = 65;             // padded row stride (doubles) of the means
constexpr int kPairs = kN * (kN - 1) / 2;

struct WardLds {
  double mean[kN * kStride];
  double cost[kPairs];
  double rowmin[kN];
  int rownn[kN];
  int size[kN];        // 0 = inactive
  int label[kN];       // item -> cluster slot (slot = smallest member = cluster id)
  int dirty[kN];
  int n_dirty;
  int rank[kN];        // slot -> bucket rank among active slots
  uint32_t pack[kN];   // rank -> packed member indices
};

__device__ __forceinline__ int tri(int a, int b) {  // a < b
  return a * (2 * kN - a - 1) / 2 + (b - a - 1);
}

__device__ __forceinline__ double pair_cost(const WardLds& L, int a, int b) {
  return a < b ? L.cost[tri(a, b)] : L.cost[tri(b, a)];
}

// Cross-lane helpers on DPP (no LDS round trips).  64-bit values move as two
// 32-bit halves; quad_perm [1,0,3,2] / [2,3,0,1], row_half_mirror and
// row_mirror combine lanes within rows of 16, readlane combines the 4 rows.
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t umin64(uint64_t a, uint64_t b) { return a < b ? a : b; }

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
  v = umin64(v, dpp_u64<0xB1>(v));
  v = umin64(v, dpp_u64<0x4E>(v));
  v = umin64(v, dpp_u64<0x141>(v));
  v = umin64(v, dpp_u64<0x140>(v));
  return umin64(umin64(readlane_u64(v, 0), readlane_u64(v, 16)),
                umin64(readlane_u64(v, 32), readlane_u64(v, 48)));
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  auto mn = [](uint32_t a, uint32_t b) { return a < b ? a : b; };
  v = mn(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
  v = mn(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
  v = mn(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
  v = mn(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
  return mn(mn((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
            mn((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
}

// sum over the 4 lanes of a quad (every lane of the quad gets the sum)
__device__ __forceinline__ double quad_sum_f64(double x) {
  uint64_t u = (uint64_t)__double_as_longlong(x);
  x += __longlong_as_double((long long)dpp_u64<0xB1>(u));
  u = (uint64_t)__double_as_longlong(x);
  x += __longlong_as_double((long long)dpp_u64<0x4E>(u));
  return x;
}

// Lexicographic (value, i) minimum across the 64 lanes of a wave (all lanes
// active).  Values are non-negative costs or +inf, whose bit patterns order
// like the values; the smallest value wins, then the smallest index among the
// lanes holding it.
__device__ __forceinline__ void wave_argmin(double& v, int& i) {
  const uint64_t bits = (uint64_t)__double_as_longlong(v);
  const uint64_t m = wave_min_u64(bits);
  const uint32_t k = wave_min_u32(bits == m ? (uint32_t)i : 0xFFFFFFFFu);
  v = __longlong_as_double((long long)m);
  i = (int)k;
}

// lexicographic (value, lo, hi) minimum across a wave (lo, hi < 128, or
// 0x7fffffff for none)
__device__ __forceinline__ void wave_argmin3(double& v, int& lo, int& hi) {
  const uint64_t bits = (uint64_t)__double_as_longlong(v);
  const uint64_t m = wave_min_u64(bits);
  const uint32_t key = ((uint32_t)(lo < kN ? lo : 0xFFFF) << 16) | (uint32_t)(hi < kN ? hi : 0xFFFF);
  const uint32_t k = wave_min_u32(bits == m ? key : 0xFFFFFFFFu);
  v = __longlong_as_double((long long)m);
  lo = (k >> 16) >= (uint32_t)kN ? 0x7fffffff : (int)(k >> 16);
  hi = (k & 0xFFFFu) >= (uint32_t)kN ? 0x7fffffff : (int)(k & 0xFFFFu);
}

// Rescan row r: nearest feasible active partner (smallest index on ties).  One wave.
__device__ void rescan_row(WardLds& L, int r, int cap, int lane) {
  double best = __builtin_inf();
  int bi = 0x7fffffff;
  const int sr = L.size[r];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    int j = lane + 64 * h;
    int sj = L.size[j];
    if (j != r && sj > 0 && sr + sj <= cap) {
      double c = pair_cost(L, r, j);
      if (c < best || (c == best && j < bi)) { best = c; bi = j; }
    }
  }
  wave_argmin(best, bi);
  if (lane == 0) { L.rowmin[r] = best; L.rownn[r] = bi; }
}

// Pairwise Ward costs of n singletons: 1*1/(1+1) * ||x_a - x_b||^2, into L.cost.
__device__ void init_costs(WardLds& L, int n) {
  const int tid = threadIdx.x;
  {
    const int q = tid & 3;          // 16-dim quarter
    const int rp = tid >> 2;        // rows ra = rp, rb = 127 - rp
    const int ra = rp, rb = kN - 1 - rp;
    double A[16], B[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      A[d] = L.mean[ra * kStride + 16 * q + d];
      B[d] = L.mean[rb * kStride + 16 * q + d];
    }
    for (int j = 1; j < n; ++j) {
      const bool da_on = j > ra && ra < n;
      const bool db_on = j > rb && rb < n;
      double sa = 0.0, sb = 0.0;
      if (da_on || db_on) {
#pragma unroll
        for (int d = 0; d < 16; ++d) {
          const double pj = L.mean[j * kStride + 16 * q + d];
          const double ea = A[d] - pj, eb = B[d] - pj;
          sa = __builtin_fma(ea, ea, sa);
          sb = __builtin_fma(eb, eb, sb);
        }
      }
      sa = quad_sum_f64(sa);
      sb = quad_sum_f64(sb);
      if (q == 0) {
        if (da_on) L.cost[tri(ra, j)] = 0.5 * sa;
        if (db_on) L.cost[tri(rb, j)] = 0.5 * sb;
      }
    }
  }
}

// Greedy capped Ward on the n active items whose means are in L.mean.
// Leaves L.size / L.label describing the final clusters.
__device__ void ward_core(WardLds& L, int n, int cap, int target) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  init_costs(L, n);
  __syncthreads();
  for (int r = wave; r < n; r += 4) rescan_row(L, r, cap, lane);
  if (tid == 0) L.n_dirty = 0;
  __syncthreads();

  for (int active = n; active > target; --active) {
    // (1) global best pair; every wave computes the same answer
    double v = __builtin_inf();
    int lo = 0x7fffffff, hi = 0x7fffffff;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int r = lane + 64 * h;
      if (L.size[r] > 0 && L.rowmin[r] < __builtin_inf()) {
        int nn = L.rownn[r];
        int l2 = r < nn ? r : nn, h2 = r < nn ? nn : r;
        double rv = L.rowmin[r];
        if (rv < v || (rv == v && (l2 < lo || (l2 == lo && h2 < hi)))) { v = rv; lo = l2; hi = h2; }
      }
    }
    wave_argmin3(v, lo, hi);
    if (lo >= kN || hi >= kN) break;  // no feasible pair (cannot happen for the caps used)
    const int a = lo, b = hi;       // a < b; merged cluster keeps slot a (its id)
    const int na = L.size[a], nb = L.size[b];
    __syncthreads();                // everyone has read rowmin/size before updates
    // (2) merge: mean, labels, sizes
    if (tid < 64) {
      const double m = ((double)na * L.mean[a * kStride + tid] +
                        (double)nb * L.mean[b * kStride + tid]) / (double)(na + nb);
      L.mean[a * kStride + tid] = m;
    } else if (tid < 64 + kN) {
      int j = tid - 64;
      if (L.label[j] == b) L.label[j] = a;
    } else if (tid == 64 + kN) {
      L.size[a] = na + nb;
      L.size[b] = 0;
    }
    __syncthreads();
    // (3) costs between a and every other active cluster (quad per cluster)
    {
      const int q = tid & 3;
      const int nab = na + nb;
      for (int o = tid >> 2; o < kN; o += kThreads / 4) {
        const int so = (o == b) ? 0 : L.size[o];
        double s = 0.0;
        if (so > 0 && o != a) {
#pragma unroll
          for (int d = 0; d < 16; ++d) {
            const double e = L.mean[o * kStride + 16 * q + d] - L.mean[a * kStride + 16 * q + d];
            s = __builtin_fma(e, e, s);
          }
        }
        s = quad_sum_f64(s);
        if (q == 0 && so > 0 && o != a) {
          const double c = (double)nab * (double)so / (double)(nab + so) * s;
          if (o < a) L.cost[tri(o, a)] = c; else L.cost[tri(a, o)] = c;
        }
      }
    }
    __syncthreads();
    // (4) nearest partners: rows touching a or b are rescanned, others compare with a
    if (tid < kN) {
      const int o = tid;
      const int so = L.size[o];
      if (so > 0) {
        const int nn = L.rownn[o];
        if (o == a || nn == a || nn == b) {
          int slot = atomicAdd(&L.n_dirty, 1);
          L.dirty[slot] = o;
        } else if (so + na + nb <= cap) {
          const double c = pair_cost(L, o, a);
          if (c < L.rowmin[o] || (c == L.rowmin[o] && a < nn)) { L.rowmin[o] = c; L.rownn[o] = a; }
        }
      }
    }
    __syncthreads();
    for (int i = wave; i < L.n_dirty; i += 4) rescan_row(L, L.dirty[i], cap, lane);
    __syncthreads();
    if (tid == 0) L.n_dirty = 0;
  }
  __syncthreads();
}

// Pairing of n singletons (capped Ward with a cap of two: the tree levels).
// The greedy order takes, one at a time, the unpaired pair with the smallest
// (cost, smaller id, larger id).  Two items that are each other's best
// partner under that order are always paired by it (no cheaper pair touches
// either of them), so every round pairs all such mutual partners at once and
// the items whose best partner was taken rescan: the pairs are those of the
// one-at-a-time order, in far fewer rounds.  Leaves L.size / L.label as
// ward_core does (a pair keeps the smaller id's slot).
__device__ void pair_core(WardLds& L, int n) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  init_costs(L, n);
  __syncthreads();
  for (int r = wave; r < n; r += 4) rescan_row(L, r, 2, lane);
  if (tid == 0) L.n_dirty = 0;
  __syncthreads();
  for (;;) {
    int mate = -1;
    if (tid < kN && L.size[tid] == 1 && L.rowmin[tid] < __builtin_inf()) {
      const int nn = L.rownn[tid];
      if (L.size[nn] == 1 && L.rownn[nn] == tid) mate = nn;
    }
    if (!__syncthreads_or(mate >= 0)) break;   // also: every decision read the old state
    if (mate > tid) { L.size[tid] = 2; L.size[mate] = 0; L.label[mate] = tid; }
    __syncthreads();
    if (tid < kN && L.size[tid] == 1 && L.rowmin[tid] < __builtin_inf() &&
        L.size[L.rownn[tid]] != 1) {
      const int slot = atomicAdd(&L.n_dirty, 1);
      L.dirty[slot] = tid;
    }
    __syncthreads();
    for (int i = wave; i < L.n_dirty; i += 4) rescan_row(L, L.dirty[i], 2, lane);
    __syncthreads();
    if (tid == 0) L.n_dirty = 0;
    __syncthreads();
  }
}

// Normalise the 512 keys of a block (fp64) and sum them by 4 into L.mean.
// A quad of lanes owns one pooled item (16 dims per lane); two rounds cover 128.
__device__ void load_pooled(WardLds& L, const float* __restrict__ src) {
  const int tid = threadIdx.x;
  const int q = tid & 3;
#pragma unroll 1
  for (int j = tid >> 2; j < kN; j += kThreads / 4) {
    double acc[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[d] = 0.0;
#pragma unroll 1
    for (int i = 0; i < kPool; ++i) {
      const float4* row = reinterpret_cast<const float4*>(src + (int64_t)(kPool * j + i) * kLatent + 16 * q);
      float x[16];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float4 f = row[v];
        x[4 * v] = f.x; x[4 * v + 1] = f.y; x[4 * v + 2] = f.z; x[4 * v + 3] = f.w;
      }
      double ss = 0.0;
#pragma unroll
      for (int d = 0; d < 16; ++d) ss = __builtin_fma((double)x[d], (double)x[d], ss);
      ss = quad_sum_f64(ss);
      const double nrm = __builtin_sqrt(ss);
      const bool zero = nrm < 1e-30;
#pragma unroll
      for (int d = 0; d < 16; ++d) acc[d] += zero ? 0.0 : (double)x[d] / nrm;
    }
#pragma unroll
    for (int d = 0; d < 16; ++d) L.mean[j * kStride + 16 * q + d] = acc[d];
  }
}

// Rank of every active slot among active slots (bucket / parent order).
__device__ void rank_slots(WardLds& L) {
  const int tid = threadIdx.x;
  if (tid < kN) {
    int r = 0;
    for (int s2 = 0; s2 < tid; ++s2) r += L.size[s2] > 0;
    L.rank[tid] = r;
  }
  __syncthreads();
}

// Store a unit vector (16 dims of it per thread) in the index dtype.
template <int DT>
__device__ __forceinline__ void store16(void* base, int64_t row, int q, const double* v) {
  if (DT == LSA_BF16) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(base) + row * kLatent + 16 * q;
    uint32_t w[8];
#pragma unroll
    for (int d = 0; d < 8; ++d)
      w[d] = (uint32_t)f64_to_bf16_rne(v[2 * d]) | ((uint32_t)f64_to_bf16_rne(v[2 * d + 1]) << 16);
    uint4* o = reinterpret_cast<uint4*>(dst);
    o[0] = make_uint4(w[0], w[1], w[2], w[3]);
    o[1] = make_uint4(w[4], w[5], w[6], w[7]);
  } else {
    float* dst = reinterpret_cast<float*>(base) + row * kLatent + 16 * q;
    float4* o = reinterpret_cast<float4*>(dst);
#pragma unroll
    for (int d = 0; d < 4; ++d)
      o[d] = make_float4((float)v[4 * d], (float)v[4 * d + 1], (float)v[4 * d + 2], (float)v[4 * d + 3]);
  }
}

template <int DT>
__device__ __forceinline__ double load_idx(const void* base, int64_t row, int d) {
  if (DT == LSA_BF16)
    return (double)bf16_to_f32(reinterpret_cast<const uint16_t*>(base)[row * kLatent + d]);
  return (double)reinterpret_cast<const float*>(base)[row * kLatent + d];
}

// v <- v / ||v|| over the 64 dims held by a quad of lanes (16 each).
__device__ __forceinline__ void quad_unit(double* v) {
  double ss = 0.0;
#pragma unroll
  for (int d = 0; d < 16; ++d) ss = __builtin_fma(v[d], v[d], ss);
  ss = quad_sum_f64(ss);  // quad-uniform control flow only reads lanes of the same quad
  const double n = __builtin_sqrt(ss);
  const bool zero = n < 1e-30;
#pragma unroll
  for (int d = 0; d < 16; ++d) v[d] = zero ? 0.0 : v[d] / n;
}

// One workgroup per full block: pooled keys -> 64 buckets.
template <int DT>
__device__ void ward_block_body(WardLds& L, const float* __restrict__ src, int64_t blk, void* cent,
                                uint32_t* __restrict__ members) {
  const int tid = threadIdx.x;
  load_pooled(L, src);
  if (tid < kN) { L.size[tid] = 1; L.label[tid] = tid; }
  __syncthreads();
  ward_core(L, kN, kCapItems, kBuckets);
  rank_slots(L);
  // member tables: pooled indices of each bucket, ascending, 0xFF padded
  if (tid < kN && L.size[tid] > 0 && L.rank[tid] < kBuckets) {
    uint32_t p = 0xFFFFFFFFu;
    int c = 0;
    for (int j = tid; j < kN && c < kCapItems; ++j) {
      if (L.label[j] == tid) {
        p = (p & ~(0xFFu << (8 * c))) | ((uint32_t)j << (8 * c));
        ++c;
      }
    }
    L.pack[L.rank[tid]] = p;
    members[blk * kBuckets + L.rank[tid]] = p;
  }
  __syncthreads();
  // centroids: unit vector of the sum of the members' pooled keys
  load_pooled(L, src);
  __syncthreads();
  {
    const int r = tid >> 2, q = tid & 3;
    const uint32_t p = L.pack[r];
    double v[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) v[d] = 0.0;
    for (int c = 0; c < kCapItems; ++c) {
      const uint32_t j = (p >> (8 * c)) & 0xFFu;
      if (j == 0xFFu) break;
#pragma unroll
      for (int d = 0; d < 16; ++d) v[d] += L.mean[j * kStride + 16 * q + d];
    }
    quad_unit(v);
    store16<DT>(cent, blk * kBuckets + r, q, v);
  }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void k_ward_blocks(const float* __restrict__ keys,
                                                          int64_t first_block, void* cent,
                                                          uint32_t* __restrict__ members) {
  __shared__ WardLds L;
  ward_block_body<DT>(L, keys + (int64_t)blockIdx.x * kBlock * kLatent, first_block + blockIdx.x,
                      cent, members);
}

// Blocks of different caches (decode: every sequence whose new key completed a block).
template <int DT>
__global__ __launch_bounds__(kThreads) void k_ward_jobs(WardJobs jobs) {
  __shared__ WardLds L;
  const int j = blockIdx.x;
  ward_block_body<DT>(L, jobs.keys[j], jobs.block[j], jobs.cent[j], jobs.members[j]);
}

// One workgroup per group of (up to) 128 nodes of the level below: greedy
// pairing by the singleton Ward cost; parents ordered by their smaller child.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_tree_groups(
    const void* __restrict__ child_cent, const int32_t* __restrict__ child_minb,
    int64_t n_child, int64_t g0, void* cent, int32_t* __restrict__ child,
    int32_t* __restrict__ minb, int child_is_bucket) {
  __shared__ WardLds L;
  const int tid = threadIdx.x;
  const int64_t G = g0 + blockIdx.x;
  const int64_t base = G * kTreeGroup;
  const int n = (int)((n_child - base) < kTreeGroup ? (n_child - base) : kTreeGroup);
  {
    const int j = tid >> 1, h = tid & 1;
    if (j < n) {
#pragma unroll 8
      for (int d = 0; d < 32; ++d) L.mean[j * kStride + 32 * h + d] = load_idx<DT>(child_cent, base + j, 32 * h + d);
    }
  }
  if (tid < kN) { L.size[tid] = tid < n ? 1 : 0; L.label[tid] = tid; }
  __syncthreads();
  pair_core(L, n);
  rank_slots(L);
  if (tid < n && L.size[tid] > 0 && L.rank[tid] < kTreeGroup / 2) {
    int other = -1;
    for (int j = tid + 1; j < n; ++j)
      if (L.label[j] == tid) { other = j; break; }
    const int64_t par = G * (kTreeGroup / 2) + L.rank[tid];
    const int64_t ca = base + tid, cb = other >= 0 ? base + other : -1;
    child[2 * par] = (int32_t)ca;
    child[2 * par + 1] = (int32_t)cb;
    int32_t ma = child_is_bucket ? (int32_t)(ca / kBuckets) : child_minb[ca];
    if (cb >= 0) {
      int32_t mb = child_is_bucket ? (int32_t)(cb / kBuckets) : child_minb[cb];
      ma = mb < ma ? mb : ma;
    }
    minb[par] = ma;
    L.pack[L.rank[tid]] = (uint32_t)tid | ((uint32_t)(other >= 0 ? other : 0xFF) << 8);
  }
  __syncthreads();
  const int n_par = (n + 1) / 2;
  {
    const int r = tid >> 2, q = tid & 3;
    if (r < n_par) {
      const uint32_t p = L.pack[r];
      const int64_t ca = base + (p & 0xFF);
      const uint32_t ob = (p >> 8) & 0xFF;
      const int64_t par = G * (kTreeGroup / 2) + r;
      double v[16];
      if (ob == 0xFF) {
        // one-child parent: the child's stored centroid, bit for bit
#pragma unroll
        for (int d = 0; d < 16; ++d) v[d] = load_idx<DT>(child_cent, ca, 16 * q + d);
      } else {
        const int64_t cb = base + ob;
#pragma unroll
        for (int d = 0; d < 16; ++d)
          v[d] = load_idx<DT>(child_cent, ca, 16 * q + d) + load_idx<DT>(child_cent, cb, 16 * q + d);
        quad_unit(v);
      }
      store16<DT>(cent, par, q, v);
    }
  }
}

__global__ void k_copy_rows(float* __restrict__ dst, const float* __restrict__ src, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = n * (kLatent / 4);
  if (i < total) reinterpret_cast<float4*>(dst)[i] = reinterpret_cast<const float4*>(src)[i];
}

}  // namespace

hipError_t launch_ward_blocks(const float* keys, int64_t first_block, int64_t n_blocks,
                              void* cent, uint32_t* members, int dtype, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  // grid.x is limited to 2^31 - 1 workgroups; far beyond any supported size
  if (dtype == LSA_BF16)
    hipLaunchKernelGGL(k_ward_blocks<LSA_BF16>, dim3((unsigned)n_blocks), dim3(kThreads), 0, s,
                       keys, first_block, cent, members);
  else
    hipLaunchKernelGGL(k_ward_blocks<LSA_F32>, dim3((unsigned)n_blocks), dim3(kThreads), 0, s,
                       keys, first_block, cent, members);
  return hipGetLastError();
}

hipError_t launch_tree_groups(const void* child_cent, const int32_t* child_minb,
                              int64_t n_child, int64_t g0, int64_t g1, void* cent,
                              int32_t* child, int32_t* minb, int dtype, int child_is_bucket,
                              hipStream_t s) {
  if (g1 <= g0) return hipSuccess;
  if (dtype == LSA_BF16)
    hipLaunchKernelGGL(k_tree_groups<LSA_BF16>, dim3((unsigned)(g1 - g0)), dim3(kThreads), 0, s,
                       child_cent, child_minb, n_child, g0, cent, child, minb, child_is_bucket);
  else
    hipLaunchKernelGGL(k_tree_groups<LSA_F32>, dim3((unsigned)(g1 - g0)), dim3(kThreads), 0, s,
                       child_cent, child_minb, n_child, g0, cent, child, minb, child_is_bucket);
  return hipGetLastError();
}

hipError_t launch_ward_jobs(const WardJobs& jobs, int n, int dtype, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (dtype == LSA_BF16)
    hipLaunchKernelGGL(k_ward_jobs<LSA_BF16>, dim3((unsigned)n), dim3(kThreads), 0, s, jobs);
  else
    hipLaunchKernelGGL(k_ward_jobs<LSA_F32>, dim3((unsigned)n), dim3(kThreads), 0, s, jobs);
  return hipGetLastError();
}

// ------------------------------------------------------------------ scan baselines
// Run summaries of the scan baselines ([72x "Why choosing costs so much"]: a
// token scan scores every key, a block scan every run of adjacent keys): for
// each aligned run of b keys of a full block, the unit vector of the sum of
// its unit keys (fp64, as the bucket centroids), rounded to the index dtype;
// for b = 1 the unit key itself.  One workgroup per block; a quad of lanes
// (16 dims each) owns one run at a time.
template <int DT>
__global__ __launch_bounds__(256) void k_scan_blocks(const float* __restrict__ keys,
                                                     int64_t first_block, void* cent, int b) {
  const int64_t blk = blockIdx.x;
  const float* src = keys + blk * kBlock * kLatent;
  const int tid = threadIdx.x, q = tid & 3;
  const int runs = kBlock / b;
#pragma unroll 1
  for (int r = tid >> 2; r < runs; r += 64) {
    double acc[16];
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[d] = 0.0;
#pragma unroll 1
    for (int i = 0; i < b; ++i) {
      const float4* row = reinterpret_cast<const float4*>(src + (int64_t)(r * b + i) * kLatent + 16 * q);
      float x[16];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float4 f = row[v];
        x[4 * v] = f.x; x[4 * v + 1] = f.y; x[4 * v + 2] = f.z; x[4 * v + 3] = f.w;
      }
      double ss = 0.0;
#pragma unroll
      for (int d = 0; d < 16; ++d) ss = __builtin_fma((double)x[d], (double)x[d], ss);
      ss = quad_sum_f64(ss);
      const double nrm = __builtin_sqrt(ss);
      const bool zero = nrm < 1e-30;
#pragma unroll
      for (int d = 0; d < 16; ++d) acc[d] += zero ? 0.0 : (double)x[d] / nrm;
    }
    double ss = 0.0;
#pragma unroll
    for (int d = 0; d < 16; ++d) ss = __builtin_fma(acc[d], acc[d], ss);
    ss = quad_sum_f64(ss);
    const double nrm = __builtin_sqrt(ss);
    const bool zero = nrm < 1e-30;
    const int64_t row = (first_block + blk) * runs + r;
    if constexpr (DT == LSA_BF16) {
      uint16_t* dst = reinterpret_cast<uint16_t*>(cent) + row * kLatent + 16 * q;
      uint32_t w[8];
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const uint16_t lo = f64_to_bf16_rne(zero ? 0.0 : acc[2 * d] / nrm);
        const uint16_t hi = f64_to_bf16_rne(zero ? 0.0 : acc[2 * d + 1] / nrm);
        w[d] = (uint32_t)lo | ((uint32_t)hi << 16);
      }
      uint4* o = reinterpret_cast<uint4*>(dst);
      o[0] = make_uint4(w[0], w[1], w[2], w[3]);
      o[1] = make_uint4(w[4], w[5], w[6], w[7]);
    } else {
      float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(cent) + row * kLatent + 16 * q);
#pragma unroll
      for (int v = 0; v < 4; ++v)
        o[v] = make_float4((float)(zero ? 0.0 : acc[4 * v] / nrm), (float)(zero ? 0.0 : acc[4 * v + 1] / nrm),
                           (float)(zero ? 0.0 : acc[4 * v + 2] / nrm), (float)(zero ? 0.0 : acc[4 * v + 3] / nrm));
    }
  }
}

hipError_t launch_scan_blocks(const float* keys, int64_t first_block, int64_t n_blocks, void* cent,
                              int run_keys, int dtype, hipStream_t s) {
  if (n_blocks <= 0) return hipSuccess;
  for (int64_t b0 = 0; b0 < n_blocks; b0 += 65535) {
    const int64_t nb = n_blocks - b0 < 65535 ? n_blocks - b0 : 65535;
    const float* src = keys + b0 * kBlock * kLatent;
    if (dtype == LSA_BF16)
      hipLaunchKernelGGL(k_scan_blocks<LSA_BF16>, dim3((unsigned)nb), dim3(256), 0, s, src,
                         first_block + b0, cent, run_keys);
    else
      hipLaunchKernelGGL(k_scan_blocks<LSA_F32>, dim3((unsigned)nb), dim3(256), 0, s, src,
                         first_block + b0, cent, run_keys);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_copy_rows(float* dst, const float* src, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t total = n * (kLatent / 4);
  hipLaunchKernelGGL(k_copy_rows, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, dst, src, n);
  return hipGetLastError();
}

}  // namespace lsa
