// Indexer: query normalisation, bucket scoring with the causal block mask,
// exact top-B bucket selection, tree beam search, best-first expansion with
// sinks and window.
//
// [visual "What one query actually does"]: the query is normalised and scored
// against bucket centroids (flat: every centroid of earlier complete blocks;
// tree: beam search level by level), the chosen buckets are opened best
// first until k far keys are collected, the first few tokens and a one-block
// recent window are always added, and one list is shared by all heads.
// [72x "The same steps in general"]: keys of an opened bucket that are
// already sinks or window keys are skipped and the next key takes their
// place; the list is returned sorted.
//
// Flat prefill selection is exact without materialising the
// (queries x buckets) score matrix:
//   1. k_thresh: bf16 MFMA scores on a 1/16 sample of bucket tiles, a per-query
//      histogram, and a threshold tau whose expected pass count is 5/4 of the
//      number of buckets kept (B) (2 B for the scans' runs);
//   2. k_score_lowpass / k_score_highpass (k_dec_filter in decode): every
//      eligible score on MFMA; scores >= tau are appended (score, bucket) to
//      a per-query candidate list;
//   3. k_select_expand: the buckets are taken in (score desc, bucket asc)
//      order until k far keys are reached (weighted select), expanded, the
//      far keys sorted, and sinks | far | window written.  A query whose
//      list overflowed `cap`, or whose candidates hold fewer than k far keys
//      while more buckets are eligible, is first redone exactly (radix select
//      on recomputed scores, ties to the lower bucket).
// Every bucket scoring >= tau is a candidate, so when the candidates hold k
// far keys every bucket ranked up to the crossing one is among them and the
// walk equals the walk over all eligible buckets.
#include "lsa_internal.h"

namespace lsa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kTile = 32;             // buckets per MFMA tile
constexpr int kSegTiles = 256;        // tiles per score_filter workgroup (8,192 buckets)
constexpr int kQueriesPerWg = 128;    // 4 waves x 32 queries
constexpr int kBins = 256;            // threshold histogram bins over [-1, 1]

__device__ __forceinline__ uint32_t f32_orderable(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int64_t qpos(const IndexCtx& c, int64_t i) {
  return c.per_seq ? c.pos[i] : c.q_start + i;
}
__device__ __forceinline__ const void* qcent(const IndexCtx& c, int64_t i) {
  return c.per_seq ? c.cent[i] : c.cent[0];
}
__device__ __forceinline__ const uint32_t* qmem(const IndexCtx& c, int64_t i) {
  return c.per_seq ? c.members[i] : c.members[0];
}
// Buckets a query at position p scores.  LSA: the buckets of complete
// blocks before the query's own block.  Scans (ctx.run_keys = b): every run
// of b consecutive keys that ends before the window starts.
__host__ __device__ __forceinline__ int64_t n_eligible(const IndexCtx& c, int64_t p) {
  if (c.run_keys == 0) return (int64_t)kBuckets * (p / kBlock);
  const int64_t w_start = p - c.window + 1 > 0 ? p - c.window + 1 : 0;
  return w_start / c.run_keys;
}

// Query held by column `col` of wave `wave` in query tile `qt` of an MFMA
// kernel.  Prefill: 32 queries per wave sharing one cache.  Decode: one query
// per wave (column 0), because every sequence has its own centroids.
__device__ __forceinline__ int64_t mfma_query(const IndexCtx& c, int64_t qt, int wave, int col) {
  if (c.per_seq) return col == 0 ? qt * 4 + wave : -1;
  return qt * kQueriesPerWg + 32 * wave + col;
}

// ------------------------------------------------------------------ qnorm
// 16 lanes per query, 4 dims each; fp64 norm, rounded to the index dtype.
template <int DT>
__global__ __launch_bounds__(256) void k_qnorm(const float* __restrict__ y, int64_t n,
                                               void* __restrict__ yhat, uint32_t* hist) {
  const int64_t i = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l = threadIdx.x & 15;
  if (hist && i < n) {       // clear this query's histogram (decode threshold)
#pragma unroll
    for (int b = 0; b < 16; ++b) hist[i * 256 + 16 * l + b] = 0u;
  }
  float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
  if (i < n) x = reinterpret_cast<const float4*>(y + i * kLatent)[l];
  double ss = (double)x.x * x.x;
  ss = __builtin_fma((double)x.y, (double)x.y, ss);
  ss = __builtin_fma((double)x.z, (double)x.z, ss);
  ss = __builtin_fma((double)x.w, (double)x.w, ss);
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) ss += __shfl_xor(ss, off, 64);
  if (i >= n) return;
  const double nr = __builtin_sqrt(ss);
  const bool zero = nr < 1e-30;
  const double v0 = zero ? 0.0 : x.x / nr, v1 = zero ? 0.0 : x.y / nr;
  const double v2 = zero ? 0.0 : x.z / nr, v3 = zero ? 0.0 : x.w / nr;
  if (DT == LSA_BF16) {
    uint2 w;
    w.x = (uint32_t)f64_to_bf16_rne(v0) | ((uint32_t)f64_to_bf16_rne(v1) << 16);
    w.y = (uint32_t)f64_to_bf16_rne(v2) | ((uint32_t)f64_to_bf16_rne(v3) << 16);
    reinterpret_cast<uint2*>(yhat)[i * 16 + l] = w;
  } else {
    reinterpret_cast<float4*>(yhat)[i * 16 + l] = make_float4((float)v0, (float)v1, (float)v2, (float)v3);
  }
}

// Decode preparation, 16 lanes per sequence: append the new latent key to the
// cache's staging row, normalise the query, clear the sampled histogram and
// the candidate count and status of the step.
template <int DT>
__global__ __launch_bounds__(256) void k_dec_prep(const float* __restrict__ y,
                                                  const float* __restrict__ k_new, AppendJobs jobs,
                                                  int64_t n, void* __restrict__ yhat, IndexWs ws) {
  const int64_t i = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int l = threadIdx.x & 15;
  if (i >= n) return;
  reinterpret_cast<float4*>(jobs.dst[i])[l] = reinterpret_cast<const float4*>(k_new + i * kLatent)[l];
#pragma unroll
  for (int b = 0; b < 16; ++b) ws.hist[i * 256 + 16 * l + b] = 0u;
  if (l == 0) { ws.cand_cnt[i] = 0; ws.status[i] = 0; }
  const float4 x = reinterpret_cast<const float4*>(y + i * kLatent)[l];
  double ss = (double)x.x * x.x;
  ss = __builtin_fma((double)x.y, (double)x.y, ss);
  ss = __builtin_fma((double)x.z, (double)x.z, ss);
  ss = __builtin_fma((double)x.w, (double)x.w, ss);
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) ss += __shfl_xor(ss, off, 16);
  const double nr = __builtin_sqrt(ss);
  const bool zero = nr < 1e-30;
  const double v0 = zero ? 0.0 : x.x / nr, v1 = zero ? 0.0 : x.y / nr;
  const double v2 = zero ? 0.0 : x.z / nr, v3 = zero ? 0.0 : x.w / nr;
  if (DT == LSA_BF16) {
    uint2 w;
    w.x = (uint32_t)f64_to_bf16_rne(v0) | ((uint32_t)f64_to_bf16_rne(v1) << 16);
    w.y = (uint32_t)f64_to_bf16_rne(v2) | ((uint32_t)f64_to_bf16_rne(v3) << 16);
    reinterpret_cast<uint2*>(yhat)[i * 16 + l] = w;
  } else {
    reinterpret_cast<float4*>(yhat)[i * 16 + l] = make_float4((float)v0, (float)v1, (float)v2, (float)v3);
  }
}

// ------------------------------------------------------------------ MFMA tile
// One wave scores 32 bucket rows (A) against 32 queries (B) with a 64-deep
// reduction.  Lane l holds row / column l % 32 and the 32 dims of half l / 32;
// A and B use the same dim order inside each MFMA, so the result is the full
// dot product.  Output: lane l, register r -> bucket row 8*(r/4) + 4*(l/32)
// + r%4 of the tile, query column l % 32.
struct QFrag {
  bf16x8 b[4];    // bf16: 4 MFMAs x 8 values
  float f[32];    // fp32: 32 MFMAs x 1 value
};

template <int DT>
__device__ __forceinline__ void load_qfrag(QFrag& q, const void* yhat, int64_t qi, bool valid,
                                           int half) {
  if (DT == LSA_BF16) {
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(yhat) +
                                                      qi * kLatent + 32 * half);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 u = valid ? src[j] : make_uint4(0, 0, 0, 0);
      q.b[j] = __builtin_bit_cast(bf16x8, u);
    }
  } else {
    const float* src = reinterpret_cast<const float*>(yhat) + qi * kLatent + 32 * half;
#pragma unroll
    for (int j = 0; j < 32; ++j) q.f[j] = valid ? src[j] : 0.f;
  }
}

template <int DT>
__device__ __forceinline__ f32x16 score_tile(const void* cent, int64_t row, int half,
                                             const QFrag& q) {
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  if (DT == LSA_BF16) {
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(cent) +
                                                      row * kLatent + 32 * half);
    uint4 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = src[j];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[j]), q.b[j], acc,
                                                    0, 0, 0);
  } else {
    const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(cent) +
                                                        row * kLatent + 32 * half);
    float a[32];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float4 v = src[j];
      a[4 * j] = v.x; a[4 * j + 1] = v.y; a[4 * j + 2] = v.z; a[4 * j + 3] = v.w;
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], q.f[j], acc, 0, 0, 0);
  }
  return acc;
}

__device__ __forceinline__ int tile_row(int r, int lane) {
  return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}

// Threshold sample: one bucket out of every 16, at offset 7 j mod 16 inside
// group j, so the sample covers every bucket rank of a block (ranks follow
// the smallest member, and early and late ranks differ in size and spread).
__device__ __forceinline__ int64_t sample_bucket(int64_t j) { return 16 * j + ((7 * j) & 15); }

// tau aims at a multiple of B buckets of the full set above it (B = top_b,
// enough buckets for k far keys when every bucket holds the fewest keys),
// divided by 16 samples.  LSA buckets hold two pooled items on average, so
// 5/4 B of them usually hold well over k far keys; a scan's runs all hold
// the same number of keys (B of them hold just k), so scans aim at 2 B.  When
// the candidates hold fewer than k far keys, the selection falls back to
// the exact top-B.
__host__ __device__ __forceinline__ int64_t tau_candidates(const IndexCtx& ctx) {
  const int64_t b = ctx.top_b > 0 ? ctx.top_b : 1;
  return ctx.run_keys ? 2 * b : (5 * b + 3) / 4;
}
__host__ __device__ __forceinline__ int64_t tau_samples(const IndexCtx& ctx) {
  return (tau_candidates(ctx) + kSampleStride - 1) / kSampleStride;
}

// ------------------------------------------------------------------ thresh
// Histogram of sampled scores per query -> tau.  Workgroup = 128 queries.
template <int DT>
__global__ __launch_bounds__(256) void k_thresh(IndexCtx ctx, IndexWs ws) {
  __shared__ uint32_t hist[kQueriesPerWg][kBins];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kQueriesPerWg * kBins; i += 256) (&hist[0][0])[i] = 0;
  const int col = lane & 31, half = lane >> 5;
  const int64_t qi = mfma_query(ctx, blockIdx.x, wave, col);
  const bool valid = qi >= 0 && qi < ctx.n;
  const int64_t ne = valid ? n_eligible(ctx, qpos(ctx, qi)) : 0;
  QFrag qf;
  load_qfrag<DT>(qf, ws.yhat, valid ? qi : 0, valid, half);
  // loop bound: the wave's largest eligible count
  int64_t wmax = ne;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    int64_t o = __shfl_xor(wmax, off, 64);
    wmax = o > wmax ? o : wmax;
  }
  const int64_t wq = mfma_query(ctx, blockIdx.x, wave, 0);
  const void* cent = qcent(ctx, wq < ctx.n ? wq : 0);
  __syncthreads();
  const int64_t n_samp = wmax / kSampleStride;          // sampled buckets of the widest query
  for (int64_t t = 0; t * kTile < n_samp; ++t) {
    const int64_t jl = t * kTile + col;                  // this lane's A row: sample jl
    f32x16 acc = score_tile<DT>(cent, jl < n_samp ? sample_bucket(jl) : 0, half, qf);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t j = t * kTile + tile_row(r, lane);
      const int64_t g = sample_bucket(j);
      if (j < n_samp && g < ne) {
        int bin = (int)__builtin_floorf((acc[r] + 1.0f) * (kBins / 2));
        bin = bin < 0 ? 0 : (bin >= kBins ? kBins - 1 : bin);
        atomicAdd(&hist[32 * wave + col][bin], 1u);
      }
    }
  }
  __syncthreads();
  if (tid < kQueriesPerWg) {
    const int64_t qj = mfma_query(ctx, blockIdx.x, tid >> 5, tid & 31);
    if (qj >= 0 && qj < ctx.n) {
      const int64_t nej = n_eligible(ctx, qpos(ctx, qj));
      float tau = -3.0e38f;
      if (nej > ctx.cap) {
        const int64_t want = tau_samples(ctx);
        int64_t cum = 0;
        for (int b = kBins - 1; b >= 0; --b) {
          cum += hist[tid][b];
          if (cum >= want) { tau = (float)b / (kBins / 2) - 1.0f; break; }
        }
      }
      ws.tau[qj] = tau;
      ws.cand_cnt[qj] = 0;
      ws.status[qj] = 0;
    }
  }
}

// Decode: the sampled histogram of one query is spread over many workgroups
// (grid.x = sample segments, grid.y = query tiles of 4, one query per wave)
// and accumulated in global memory; k_thresh_tau turns it into tau.
constexpr int kHistSegTiles = 8;   // sampled tiles per workgroup

template <int DT>
__global__ __launch_bounds__(256) void k_thresh_hist(IndexCtx ctx, IndexWs ws) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int64_t qi = mfma_query(ctx, blockIdx.y, wave, col);
  const bool valid = qi >= 0 && qi < ctx.n;
  const int64_t ne = valid ? n_eligible(ctx, qpos(ctx, qi)) : 0;
  int64_t wmax = ne;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    int64_t o = __shfl_xor(wmax, off, 64);
    wmax = o > wmax ? o : wmax;
  }
  const int64_t n_tiles = (wmax / kSampleStride + kTile - 1) / kTile;   // tiles of samples
  const int64_t s0 = (int64_t)blockIdx.x * kHistSegTiles;
  // wave-uniform exit: every lane must stay for the MFMAs (they read all 64 lanes)
  if (__ballot(s0 < n_tiles && ne > ctx.cap) == 0) return;
  QFrag qf;
  load_qfrag<DT>(qf, ws.yhat, valid ? qi : 0, valid, half);
  const int64_t wq = mfma_query(ctx, blockIdx.y, wave, 0);
  const void* cent = qcent(ctx, wq < ctx.n ? wq : 0);
  uint32_t* h = ws.hist + (valid ? qi : 0) * 256;
  const int64_t n_samp = wmax / kSampleStride;
  for (int64_t t = s0; t < n_tiles && t < s0 + kHistSegTiles; ++t) {
    const int64_t jl = t * kTile + col;
    f32x16 acc = score_tile<DT>(cent, jl < n_samp ? sample_bucket(jl) : 0, half, qf);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t j = t * kTile + tile_row(r, lane);
      const int64_t g = sample_bucket(j);
      if (j < n_samp && g < ne && ne > ctx.cap) {
        int bin = (int)__builtin_floorf((acc[r] + 1.0f) * (kBins / 2));
        bin = bin < 0 ? 0 : (bin >= kBins ? kBins - 1 : bin);
        atomicAdd(&h[bin], 1u);
      }
    }
  }
}

// `preset_all`: the 128-query path's convention (ne <= cap keeps every bucket
// at slot g, so the count starts at ne).
__global__ __launch_bounds__(64) void k_thresh_tau(IndexCtx ctx, IndexWs ws, int preset_all) {
  const int64_t qj = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (qj >= ctx.n) return;
  const int64_t nej = n_eligible(ctx, qpos(ctx, qj));
  float tau = -3.0e38f;
  if (nej > ctx.cap) {
    const int64_t want = tau_samples(ctx);
    const uint32_t* h = ws.hist + qj * 256;
    int64_t cum = 0;
    for (int b = kBins - 1; b >= 0; --b) {
      cum += h[b];
      if (cum >= want) { tau = (float)b / (kBins / 2) - 1.0f; break; }
    }
  }
  ws.tau[qj] = tau;
  ws.cand_cnt[qj] = (preset_all && nej <= ctx.cap) ? (int32_t)nej : 0;
  ws.status[qj] = 0;
}

// ------------------------------------------------------------------ score + filter
// grid.x = bucket segments of 8,192, grid.y = query tiles of 128.
template <int DT>
__global__ __launch_bounds__(256) void k_score_filter(IndexCtx ctx, IndexWs ws, int seg_tiles) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int64_t qi = mfma_query(ctx, blockIdx.y, wave, col);
  const bool valid = qi >= 0 && qi < ctx.n;
  const int64_t ne = valid ? n_eligible(ctx, qpos(ctx, qi)) : 0;
  int64_t wmax = ne;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    int64_t o = __shfl_xor(wmax, off, 64);
    wmax = o > wmax ? o : wmax;
  }
  const int64_t t0 = (int64_t)blockIdx.x * seg_tiles;
  int64_t t1 = (wmax + kTile - 1) / kTile;   // a scan's last tile may be partial
  if (t1 > t0 + seg_tiles) t1 = t0 + seg_tiles;
  if (t0 >= t1) return;
  QFrag qf;
  load_qfrag<DT>(qf, ws.yhat, valid ? qi : 0, valid, half);
  const float tau = valid ? ws.tau[qi] : 3.0e38f;
  const int64_t wq = mfma_query(ctx, blockIdx.y, wave, 0);
  const void* cent = qcent(ctx, wq < ctx.n ? wq : 0);
  uint2* cand = ws.cand + (valid ? qi : 0) * (int64_t)ctx.cap;
  for (int64_t t = t0; t < t1; ++t) {
    f32x16 acc = score_tile<DT>(cent, t * kTile + col, half, qf);
    float m = acc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) m = fmaxf(m, acc[r]);
    if (__ballot(m >= tau) == 0) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t g = t * kTile + tile_row(r, lane);
      if (acc[r] >= tau && g < ne) {
        const int slot = atomicAdd(&ws.cand_cnt[qi], 1);
        if (slot < ctx.cap) cand[slot] = make_uint2(__float_as_uint(acc[r]), (uint32_t)g);
      }
    }
  }
}

// ------------------------------------------------------------------ bf16 prefill scoring, 128 queries per wave
// Prefill queries share one cache, so every wave can hold the fragments of
// all 128 queries of its workgroup (4 groups of 32 columns) and score its own
// 32-bucket tiles against them: 16 MFMAs per tile, and each centroid row is
// read once per workgroup instead of once per wave.  The 4 waves interleave
// tiles; each keeps the next two tiles in flight.  grid.x walks query tiles,
// so the workgroups that read one bucket segment are dispatched together and
// share it in L2.
//
// Candidate convention of this path: a query with no more eligible buckets
// than candidate slots (ne <= cap) keeps all of them, each stored directly at
// slot g with the count preset to ne; other queries append (score, bucket)
// for scores >= tau, staged in LDS and flushed with one atomic per query.
constexpr int kCapL = 40;           // LDS candidate slots per query and workgroup
constexpr int kSelectWideQueries = 64;   // up to this many queries: 1,024-thread selection

// NG query groups of 32 per wave (4 for 128 queries)
template <int NG>
struct QGroups {
  bf16x8 b[NG][4];                  // [query group][k step]
};
using Q128 = QGroups<4>;

template <int NG>
__device__ __forceinline__ void load_q128(QGroups<NG>& q, const void* yhat, int64_t q0, int64_t n,
                                          int col, int half) {
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const int64_t qi = q0 + 32 * j + col;
    const bool valid = qi < n;
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(yhat) +
                                                      (valid ? qi : 0) * kLatent + 32 * half);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 u = valid ? src[kk] : make_uint4(0, 0, 0, 0);
      q.b[j][kk] = __builtin_bit_cast(bf16x8, u);
    }
  }
}

__device__ __forceinline__ void load_atile(uint4 (&a)[4], const void* cent, int64_t row, int half) {
  const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(cent) +
                                                    row * kLatent + 32 * half);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) a[kk] = src[kk];
}

__device__ __forceinline__ void mfma_q128(f32x16 (&acc)[4], const uint4 (&a)[4], const Q128& q) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[kk]), q.b[j][kk],
                                                       acc[j], 0, 0, 0);
  }
}

// One tile for the low-pass path: the MFMAs run query group by query group,
// and the 16-row max and ballot of group j are computed while the MFMAs of
// group j + 1 execute (the scheduling barriers ask for 1 MFMA, then 3 VALU).
__device__ __forceinline__ float max16(const f32x16& v);

template <int NG>
__device__ __forceinline__ void mfma_q128_masks(f32x16 (&acc)[NG], uint64_t (&mks)[NG],
                                                const uint4 (&a)[4], const QGroups<NG>& q,
                                                const float (&tau)[NG]) {
#pragma unroll
  for (int j = 0; j < NG; ++j) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[kk]), q.b[j][kk],
                                                       acc[j], 0, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < NG; ++j) mks[j] = __ballot(max16(acc[j]) >= tau[j]);
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
#pragma unroll
  for (int i = 0; i < 4 * (NG - 1); ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
  }
}

__device__ __forceinline__ float max16(const f32x16& v) {
  float m0 = __builtin_fmaxf(__builtin_fmaxf(v[0], v[1]), v[2]);
  float m1 = __builtin_fmaxf(__builtin_fmaxf(v[3], v[4]), v[5]);
  float m2 = __builtin_fmaxf(__builtin_fmaxf(v[6], v[7]), v[8]);
  float m3 = __builtin_fmaxf(__builtin_fmaxf(v[9], v[10]), v[11]);
  float m4 = __builtin_fmaxf(__builtin_fmaxf(v[12], v[13]), v[14]);
  m0 = __builtin_fmaxf(__builtin_fmaxf(m0, m1), m2);
  m3 = __builtin_fmaxf(__builtin_fmaxf(m3, m4), v[15]);
  return __builtin_fmaxf(m0, m3);
}

// Per-lane view of the NG queries (one per group) whose column this lane holds.
template <int NG>
struct QColsN {
  int32_t qi[NG];
  int32_t ne[NG];
  float tau[NG];
  bool all[NG];
};
using QCols = QColsN<4>;

template <int NG>
__device__ __forceinline__ int32_t load_qcols(QColsN<NG>& c, const IndexCtx& ctx, const float* tau,
                                              int64_t q0, int col) {
  int32_t nmax = 0;
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const int64_t qi = q0 + 32 * j + col;
    const bool valid = qi < ctx.n;
    c.qi[j] = valid ? (int32_t)qi : 0;
    c.ne[j] = valid ? (int32_t)n_eligible(ctx, ctx.q_start + qi) : 0;
    c.tau[j] = (valid && tau) ? tau[qi] : 3.0e38f;
    c.all[j] = valid && c.ne[j] <= ctx.cap;
    nmax = c.ne[j] > nmax ? c.ne[j] : nmax;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const int32_t o = __shfl_xor(nmax, off, 64);
    nmax = o > nmax ? o : nmax;
  }
  return __builtin_amdgcn_readfirstlane(nmax);   // the same in every wave of the workgroup
}

// Low-pass epilogue (few candidates per query and tile).  In the tile loop
// each lane only takes the max of its 16 scores per query group (8 v_max3)
// and compares it with the query's tau; a lane whose max passes copies its 16
// scores into its wave's LDS ring (slots from a ballot, no atomics).  Full
// passes of 64 ring entries, one per lane, then find the passing rows and
// append them to the query's LDS list (global memory once the list is full).
constexpr int kRing = 128;          // ring entries per wave (power of two)

template <int NQ>
struct LowPassLds {
  int cnt[NQ];                                        // candidates per query
  float tau[NQ];
  int32_t ne[NQ];                                     // eligible buckets per query
  uint2 buf[NQ * kCapL];                              // (score bits, bucket)
  float ent[4][kRing][16];                            // ring of flagged lanes per wave
  uint32_t meta[4][kRing];                            // tile << 8 | half << 7 | query
};

// One pass over up to 64 ring entries starting at `head` (wave-uniform).
template <class LL>
__device__ __forceinline__ void ring_pass(LL& L, const IndexCtx& ctx, const IndexWs& ws,
                                          int64_t q0, int wave, int lane, uint32_t head,
                                          uint32_t count) {
  __builtin_amdgcn_wave_barrier();
  if ((uint32_t)lane < count) {
    const uint32_t e = (head + (uint32_t)lane) & (kRing - 1);
    const uint32_t meta = L.meta[wave][e];
    const int ql = meta & 127;
    const int32_t gb = (int32_t)(meta >> 8) * kTile + 4 * (int)((meta >> 7) & 1);
    const float tau = L.tau[ql];
    const int32_t ne = L.ne[ql];
    const float4* src = reinterpret_cast<const float4*>(L.ent[wave][e]);
    uint32_t bits = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 x = src[i];
      bits |= (uint32_t)(x.x >= tau) << (4 * i);
      bits |= (uint32_t)(x.y >= tau) << (4 * i + 1);
      bits |= (uint32_t)(x.z >= tau) << (4 * i + 2);
      bits |= (uint32_t)(x.w >= tau) << (4 * i + 3);
    }
    // rows 4i..4i+3 hold buckets gb + 8i .. gb + 8i + 3; only the last
    // eligible tile of a query cuts a run
    if (gb + 27 >= ne) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int v = ne - (gb + 8 * i);
        v = v < 0 ? 0 : (v > 4 ? 4 : v);
        bits &= ~((0xFu & ~((1u << v) - 1u)) << (4 * i));
      }
    }
    if (bits) {
      int slot = atomicAdd(&L.cnt[ql], __popc(bits));
      const int64_t qi = q0 + ql;
      const float* row = L.ent[wave][e];
      do {
        const int r = __builtin_ctz(bits);
        bits &= bits - 1;
        const uint2 c = make_uint2(__float_as_uint(row[r]), (uint32_t)(gb + 8 * (r >> 2) + (r & 3)));
        if (slot < kCapL) {
          L.buf[ql * kCapL + slot] = c;
        } else {
          const int gs = atomicAdd(&ws.cand_cnt[qi], 1);
          if (gs < ctx.cap) ws.cand[qi * ctx.cap + gs] = c;
        }
        ++slot;
      } while (bits);
    }
  }
  __builtin_amdgcn_wave_barrier();
}

// Copy the lanes flagged in the per-group ballots into the ring; a group that
// would not fit first drains one full pass (more than 64 entries are queued
// whenever that happens).
template <class LL, int NG>
__device__ __forceinline__ void ring_push(LL& L, const IndexCtx& ctx, const IndexWs& ws,
                                          const f32x16 (&acc)[NG], const uint64_t (&mks)[NG],
                                          int32_t t, int64_t q0, int wave, int lane, int col,
                                          int half, uint32_t& head, uint32_t& tail) {
#pragma unroll
  for (int j = 0; j < NG; ++j) {
    const uint64_t mk = mks[j];
    if (mk == 0) continue;
    const uint32_t n = (uint32_t)__popcll(mk);
    if (tail - head + n > (uint32_t)kRing) {
      ring_pass(L, ctx, ws, q0, wave, lane, head, 64u);
      head += 64u;
    }
    if ((mk >> lane) & 1ull) {
      const uint32_t e = (tail + __builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32),
                                  __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u))) & (kRing - 1);
      float4* dst = reinterpret_cast<float4*>(L.ent[wave][e]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        dst[i] = make_float4(acc[j][4 * i], acc[j][4 * i + 1], acc[j][4 * i + 2], acc[j][4 * i + 3]);
      L.meta[wave][e] = ((uint32_t)t << 8) | ((uint32_t)half << 7) | (uint32_t)(32 * j + col);
    }
    tail += n;
  }
}

// after a tile's epilogue (its accumulators are dead): full passes only,
// or everything at the end
template <class LL>
__device__ __forceinline__ void ring_drain(LL& L, const IndexCtx& ctx, const IndexWs& ws,
                                           int64_t q0, int wave, int lane, uint32_t& head,
                                           uint32_t tail, bool all) {
  while (tail - head >= 64u || (all && tail != head)) {
    const uint32_t c = tail - head < 64u ? tail - head : 64u;
    ring_pass(L, ctx, ws, q0, wave, lane, head, c);
    head += c;
  }
}

// High-pass epilogue (many candidates, or every eligible bucket kept): per
// query and tile one atomic reserves the slots of both lanes that hold the
// query's 32 rows; queries with ne <= cap store bucket g at slot g.  It runs in
// two halves around the next tile's loads: the passing rows and the four slot
// reservations first, the stores after.  The wait for a returning atomic
// covers every memory operation issued before it, so reservations issued
// after the next tile's loads would wait for those loads too.
struct HpRes {
  uint32_t bits01, bits23;          // passing rows of query groups 0..3, 16 bits each
  int base[4];                      // reserved slot (lanes of the first half)
};

__device__ __forceinline__ HpRes highpass_reserve(const f32x16 (&acc)[4], int32_t t,
                                                  const QCols& qc, int lane, int half,
                                                  const IndexWs& ws) {
  HpRes h;
  h.bits01 = h.bits23 = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t bits = 0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int32_t g = t * kTile + tile_row(r, lane);
      const bool p = (qc.all[j] || acc[j][r] >= qc.tau[j]) && g < qc.ne[j];
      bits |= (uint32_t)p << r;
    }
    if (j < 2) h.bits01 |= bits << (16 * j);
    else h.bits23 |= bits << (16 * (j - 2));
    const int nl = __popc(bits);
    const int np = __shfl_xor(nl, 32, 64);
    h.base[j] = 0;
    if (!qc.all[j] && half == 0 && nl + np > 0)
      h.base[j] = atomicAdd(&ws.cand_cnt[qc.qi[j]], nl + np);
  }
  return h;
}

__device__ __forceinline__ void highpass_store(const f32x16 (&acc)[4], int32_t t, const QCols& qc,
                                               const HpRes& h, int lane, int col, int half,
                                               const IndexWs& ws, int cap) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t bits = ((j < 2 ? h.bits01 : h.bits23) >> (16 * (j & 1))) & 0xFFFFu;
    if (__ballot(bits != 0) == 0) continue;
    uint2* dst = ws.cand + (int64_t)qc.qi[j] * cap;
    const int np = __shfl_xor(__popc(bits), 32, 64);
    // one predicated store per row: bucket g goes to slot g (every bucket
    // kept) or to the next appended slot while the list has room
    int slot = __shfl(h.base[j], col, 64) + (half ? np : 0);
    const bool all = qc.all[j];
    const int lim = all ? 0x7fffffff : cap;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool pr = ((bits >> r) & 1u) != 0;
      const uint32_t g = (uint32_t)(t * kTile + tile_row(r, lane));
      const uint32_t d = all ? g : (uint32_t)slot;
      if (pr & (slot < lim)) dst[d] = make_uint2(__float_as_uint(acc[j][r]), g);
      slot += pr ? 1 : 0;
    }
  }
}

// High-pass scoring: query tiles whose queries keep a large share of their
// eligible buckets (or all of them).  128 queries per workgroup, each wave
// scores its own tiles against all of them; grid.x = query tiles [0, x),
// grid.y = bucket segments.
__global__ __launch_bounds__(256, 2) void k_score_highpass(IndexCtx ctx, IndexWs ws,
                                                           int seg_tiles) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int64_t q0 = (int64_t)blockIdx.x * kQueriesPerWg;
  QCols qc;
  const int32_t nmax = load_qcols(qc, ctx, ws.tau, q0, col);
  const int32_t t0 = (int32_t)blockIdx.y * seg_tiles;
  int32_t t1 = (nmax + kTile - 1) / kTile;
  if (t1 > t0 + seg_tiles) t1 = t0 + seg_tiles;
  if (t0 >= t1) return;                                  // uniform over the workgroup
  Q128 q;
  load_q128(q, ws.yhat, q0, ctx.n, col, half);
  const void* cent = ctx.cent[0];
  const int32_t tl = t1 - 1;
  // two register buffers: each is reloaded (clamped to the last tile, so the
  // number of loads in flight is the same on every path) as soon as its
  // MFMAs have been issued, before the epilogue of the tile it held
  uint4 ra[4], rb[4];
  int32_t t = t0 + wave;
  load_atile(ra, cent, (int64_t)(t < tl ? t : tl) * kTile + col, half);
  __builtin_amdgcn_sched_barrier(0);   // keep ra's loads older than rb's
  load_atile(rb, cent, (int64_t)(t + 4 < tl ? t + 4 : tl) * kTile + col, half);
  for (; t < t1; t += 8) {
    f32x16 acc[4];
    mfma_q128(acc, ra, q);
    HpRes h = highpass_reserve(acc, t, qc, lane, half, ws);
    load_atile(ra, cent, (int64_t)(t + 8 < tl ? t + 8 : tl) * kTile + col, half);
    highpass_store(acc, t, qc, h, lane, col, half, ws, ctx.cap);
    mfma_q128(acc, rb, q);
    const bool more = t + 4 < t1;
    if (more) h = highpass_reserve(acc, t + 4, qc, lane, half, ws);
    load_atile(rb, cent, (int64_t)(t + 12 < tl ? t + 12 : tl) * kTile + col, half);
    if (more) highpass_store(acc, t + 4, qc, h, lane, col, half, ws, ctx.cap);
  }
}

// Low-pass scoring: query tiles whose queries keep a small share of their
// eligible buckets.  Same tile loop as the high-pass kernel; the epilogue
// buffers flagged lanes (lowpass_buffer) and expands the buffer after a
// tile when it is half full, so the expansion never runs while a tile's
// accumulators are live.  grid.x = query tiles from qt0 on, grid.y =
// bucket segments.
template <int NG>
__global__ __launch_bounds__(256, 2) void k_score_lowpass(IndexCtx ctx, IndexWs ws, int seg_tiles,
                                                          int64_t qbase) {
  constexpr int NQ = 32 * NG;                            // queries per workgroup
  __shared__ __attribute__((aligned(16))) LowPassLds<NQ> L;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int64_t q0 = qbase + (int64_t)blockIdx.x * NQ;
  QColsN<NG> qc;
  const int32_t nmax = load_qcols(qc, ctx, ws.tau, q0, col);
  const int32_t t0 = (int32_t)blockIdx.y * seg_tiles;
  int32_t t1 = (nmax + kTile - 1) / kTile;
  if (t1 > t0 + seg_tiles) t1 = t0 + seg_tiles;
  if (t0 >= t1) return;                                  // uniform over the workgroup
  if (tid < NQ) {
    const bool valid = q0 + tid < ctx.n;
    L.cnt[tid] = 0;
    L.tau[tid] = valid ? ws.tau[q0 + tid] : 3.0e38f;
    L.ne[tid] = valid ? (int32_t)n_eligible(ctx, ctx.q_start + q0 + tid) : 0;
  }
  QGroups<NG> q;
  load_q128(q, ws.yhat, q0, ctx.n, col, half);
  const void* cent = ctx.cent[0];
  const int32_t tl = t1 - 1;
  __syncthreads();
  uint32_t head = 0, tail = 0;                           // ring indices, wave-uniform
  uint4 ra[4], rb[4];
  int32_t t = t0 + wave;
  load_atile(ra, cent, (int64_t)(t < tl ? t : tl) * kTile + col, half);
  __builtin_amdgcn_sched_barrier(0);   // keep ra's loads older than rb's
  load_atile(rb, cent, (int64_t)(t + 4 < tl ? t + 4 : tl) * kTile + col, half);
  for (; t < t1; t += 8) {
    f32x16 acc[NG];
    uint64_t mks[NG];
    mfma_q128_masks(acc, mks, ra, q, qc.tau);
    load_atile(ra, cent, (int64_t)(t + 8 < tl ? t + 8 : tl) * kTile + col, half);
    ring_push(L, ctx, ws, acc, mks, t, q0, wave, lane, col, half, head, tail);
    ring_drain(L, ctx, ws, q0, wave, lane, head, tail, false);
    mfma_q128_masks(acc, mks, rb, q, qc.tau);
    load_atile(rb, cent, (int64_t)(t + 12 < tl ? t + 12 : tl) * kTile + col, half);
    if (t + 4 < t1) {
      ring_push(L, ctx, ws, acc, mks, t + 4, q0, wave, lane, col, half, head, tail);
      ring_drain(L, ctx, ws, q0, wave, lane, head, tail, false);
    }
  }
  ring_drain(L, ctx, ws, q0, wave, lane, head, tail, true);
  __syncthreads();
  // flush: two threads per query
  const int ql = tid >> 1, sub = tid & 1;
  if (ql < NQ) {
    const int64_t qi = q0 + ql;
    int n = L.cnt[ql];
    n = n < kCapL ? n : kCapL;
    int base = 0;
    if (sub == 0 && n > 0 && qi < ctx.n) base = atomicAdd(&ws.cand_cnt[qi], n);
    base = __shfl(base, lane & ~1, 64);
    if (qi < ctx.n) {
      uint2* dst = ws.cand + qi * (int64_t)ctx.cap;
      for (int i = sub; i < n; i += 2)
        if (base + i < ctx.cap) dst[base + i] = L.buf[ql * kCapL + i];
    }
  }
}

// Threshold for the same path: every wave scores its own sampled tiles
// against the workgroup's 128 queries into one LDS histogram per query.  With
// few query tiles the samples are split over grid.y workgroups whose
// histograms are added in global memory and finished by k_thresh_tau.
__global__ __launch_bounds__(512, 1) void k_thresh_q128(IndexCtx ctx, IndexWs ws, int seg_tiles,
                                                        int split) {
  // one row per query, padded by a word: lanes of different queries whose
  // scores fall in the same bin then add into different LDS banks
  constexpr int kRow = kBins + 1;
  __shared__ uint32_t hist[kQueriesPerWg][kRow];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int64_t q0 = (int64_t)blockIdx.x * kQueriesPerWg;
  for (int i = tid; i < kQueriesPerWg * kRow; i += 512) (&hist[0][0])[i] = 0;
  QCols qc;
  const int32_t nmax = load_qcols(qc, ctx, nullptr, q0, col);
  const int32_t n_samp = nmax / kSampleStride;            // samples of the widest query
  const int32_t s0 = (int32_t)blockIdx.y * seg_tiles;
  int32_t s1 = (n_samp + kTile - 1) / kTile;
  if (s1 > s0 + seg_tiles) s1 = s0 + seg_tiles;
  Q128 q;
  load_q128(q, ws.yhat, q0, ctx.n, col, half);
  const void* cent = ctx.cent[0];
  __syncthreads();
  if (s0 < s1) {
    const int32_t jlast = n_samp - 1;
    auto row_of = [&](int32_t t) {
      const int32_t j = t * kTile + col;
      return sample_bucket(j < jlast ? j : jlast);
    };
    // bin of a score: (s + 1) * 128 truncated, clamped to [0, 255] (the
    // clamp taken on the float first: the same bin for every finite s)
    auto bin_of = [](float sc) {
      return (int)__builtin_amdgcn_fmed3f((sc + 1.0f) * (kBins / 2), 0.f, (float)(kBins - 1));
    };
    auto epilogue = [&](const f32x16 (&acc)[4], int32_t t) {
      // sample jj's bucket 16 jj + (7 jj & 15) grows with jj, so a tile whose
      // last sample is eligible for a query is eligible in every row
      const int32_t jl = t * kTile + kTile - 1;
      const bool in_samp = jl < n_samp;
      const int32_t gl = 16 * jl + ((7 * jl) & 15);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (qc.all[j]) continue;
        uint32_t* hrow = hist[32 * j + col];
        if (in_samp && gl < qc.ne[j]) {
#pragma unroll
          for (int r = 0; r < 16; ++r) atomicAdd(&hrow[bin_of(acc[j][r])], 1u);
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int32_t jj = t * kTile + tile_row(r, lane);
            if (jj < n_samp && 16 * jj + ((7 * jj) & 15) < qc.ne[j])
              atomicAdd(&hrow[bin_of(acc[j][r])], 1u);
          }
        }
      }
    };
    constexpr int W = 8;
    uint4 ra[4], rb[4];
    int32_t t = s0 + wave;
    const int32_t tl = s1 - 1;
    load_atile(ra, cent, row_of(t < tl ? t : tl), half);
    __builtin_amdgcn_sched_barrier(0);
    load_atile(rb, cent, row_of(t + W < tl ? t + W : tl), half);
    for (; t < s1; t += 2 * W) {
      f32x16 acc[4];
      mfma_q128(acc, ra, q);
      load_atile(ra, cent, row_of(t + 2 * W < tl ? t + 2 * W : tl), half);
      epilogue(acc, t);
      mfma_q128(acc, rb, q);
      load_atile(rb, cent, row_of(t + 3 * W < tl ? t + 3 * W : tl), half);
      if (t + W < s1) epilogue(acc, t + W);
    }
  }
  __syncthreads();
  if (split) {
    for (int i = tid; i < kQueriesPerWg * kBins; i += 512) {
      const uint32_t v = hist[i / kBins][i % kBins];
      const int64_t qj = q0 + i / kBins;
      if (v && qj < ctx.n) atomicAdd(&ws.hist[qj * kBins + (i % kBins)], v);
    }
    return;
  }
  if (tid < kQueriesPerWg) {
    const int64_t qj = q0 + tid;
    if (qj < ctx.n) {
      const int64_t nej = n_eligible(ctx, ctx.q_start + qj);
      float tau = -3.0e38f;
      if (nej > ctx.cap) {
        const int64_t want = tau_samples(ctx);
        int64_t cum = 0;
        for (int b = kBins - 1; b >= 0; --b) {
          cum += hist[tid][b];
          if (cum >= want) { tau = (float)b / (kBins / 2) - 1.0f; break; }
        }
      }
      ws.tau[qj] = tau;
      ws.cand_cnt[qj] = nej <= ctx.cap ? (int32_t)nej : 0;
      ws.status[qj] = 0;
    }
  }
}

__global__ __launch_bounds__(256) void k_fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

// ------------------------------------------------------------------ max over query heads
// [catalog "Key points"], N-LSA: bucket selection uses the max score across
// heads.  A query position brings H query heads (ctx.heads = 2, 4 or 8); a
// bucket's score is the largest of its H dot products.  Prefill, bf16: a
// workgroup takes NQ = 128 / H query positions, whose 128 head vectors form
// the A operand of 32x32x16 MFMAs (4 groups of 32 rows, held by every wave),
// and a tile of 32 buckets the B operand, so a lane holds one bucket's scores
// against 16 head rows of a group; rows 8 (r / 4) + 4 half + (r % 4) are H
// consecutive heads of one position, so the max over heads is a max over
// min(H, 4) registers (and, for H = 8, over the lane pair 32 apart).
template <int H>
__device__ __forceinline__ void load_heads(bf16x8 (&a)[4][4], const void* yhat, int64_t q0,
                                           int64_t n, int col, int half) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 32 * j + col;                       // workgroup-local head row
    const int64_t qi = q0 + row / H;
    const bool valid = qi < n;
    const uint4* src = reinterpret_cast<const uint4*>(
        reinterpret_cast<const uint16_t*>(yhat) + ((valid ? qi : 0) * H + row % H) * kLatent +
        32 * half);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      a[j][kk] = __builtin_bit_cast(bf16x8, valid ? src[kk] : make_uint4(0, 0, 0, 0));
  }
}

// Scores of one group j: m[i] = the max over heads of the i-th position this
// lane holds (E = 16 / min(H, 4) of them), position (workgroup-local)
// mh_pos<H>(j, i, half).
template <int H>
__device__ __forceinline__ void mh_max(const f32x16& acc, float (&m)[16 / (H < 4 ? H : 4)]) {
  constexpr int R = H < 4 ? H : 4;
#pragma unroll
  for (int i = 0; i < 16 / R; ++i) {
    float x = acc[R * i];
#pragma unroll
    for (int u = 1; u < R; ++u) x = fmaxf(x, acc[R * i + u]);
    if constexpr (H == 8) x = fmaxf(x, __shfl_xor(x, 32, 64));
    m[i] = x;
  }
}

template <int H>
__device__ __forceinline__ int mh_pos(int j, int i, int half) {
  // the first head row of value i: 8 (i R / 4) + 4 half + (i R) % 4
  constexpr int R = H < 4 ? H : 4;
  const int row = 8 * ((R * i) >> 2) + (H == 8 ? 0 : 4 * half) + ((R * i) & 3);
  return (32 * j + row) / H;
}

template <int H>
__global__ __launch_bounds__(256) void k_mh_thresh(IndexCtx ctx, IndexWs ws) {
  constexpr int NQ = 128 / H;
  constexpr int E = 16 / (H < 4 ? H : 4);
  __shared__ uint32_t hist[NQ][kBins];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int64_t q0 = (int64_t)blockIdx.x * NQ;
  for (int i = tid; i < NQ * kBins; i += 256) (&hist[0][0])[i] = 0;
  const int64_t qlast = q0 + NQ - 1 < ctx.n - 1 ? q0 + NQ - 1 : ctx.n - 1;
  const int64_t nmax = n_eligible(ctx, qpos(ctx, qlast));        // grows with the position
  const int64_t n_samp = nmax / kSampleStride;
  bf16x8 a[4][4];
  load_heads<H>(a, ws.yhat, q0, ctx.n, col, half);
  const void* cent = ctx.cent[0];
  __syncthreads();
  for (int64_t t = wave; t * kTile < n_samp; t += 4) {
    const int64_t jl = t * kTile + col;
    uint4 b[4];
    load_atile(b, cent, sample_bucket(jl < n_samp ? jl : n_samp - 1), half);
    const int64_t g = sample_bucket(jl);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j][kk], __builtin_bit_cast(bf16x8, b[kk]),
                                                      acc, 0, 0, 0);
      float m[E];
      mh_max<H>(acc, m);
#pragma unroll
      for (int i = 0; i < E; ++i) {
        if (H == 8 && (i >> 1) != half) continue;          // each half counts two positions
        const int ql = mh_pos<H>(j, i, half);
        const int64_t qi = q0 + ql;
        if (jl < n_samp && qi < ctx.n && g < n_eligible(ctx, qpos(ctx, qi))) {
          int bin = (int)((m[i] + 1.0f) * (kBins / 2));
          bin = bin < 0 ? 0 : (bin >= kBins ? kBins - 1 : bin);
          atomicAdd(&hist[ql][bin], 1u);
        }
      }
    }
  }
  __syncthreads();
  if (tid < NQ) {
    const int64_t qj = q0 + tid;
    if (qj < ctx.n) {
      const int64_t nej = n_eligible(ctx, qpos(ctx, qj));
      float tau = -3.0e38f;
      if (nej > ctx.cap) {
        const int64_t want = tau_samples(ctx);
        int64_t cum = 0;
        for (int b = kBins - 1; b >= 0; --b) {
          cum += hist[tid][b];
          if (cum >= want) { tau = (float)b / (kBins / 2) - 1.0f; break; }
        }
      }
      ws.tau[qj] = tau;
      ws.cand_cnt[qj] = nej <= ctx.cap ? (int32_t)nej : 0;
      ws.status[qj] = 0;
    }
  }
}

// Every eligible bucket's max-over-heads score against tau; a position that
// keeps all its buckets (ne <= cap) stores bucket g at slot g, the others
// append with one atomic per position and half-wave.  grid.x = position
// tiles of NQ, grid.y = bucket segments of seg_tiles tiles; the 4 waves take
// every 4th tile.
template <int H>
__global__ __launch_bounds__(256) void k_mh_filter(IndexCtx ctx, IndexWs ws, int seg_tiles) {
  constexpr int NQ = 128 / H;
  constexpr int E = 16 / (H < 4 ? H : 4);
  __shared__ float s_tau[NQ];
  __shared__ int32_t s_ne[NQ];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  const int64_t q0 = (int64_t)blockIdx.x * NQ;
  const int64_t qlast = q0 + NQ - 1 < ctx.n - 1 ? q0 + NQ - 1 : ctx.n - 1;
  const int64_t nmax = n_eligible(ctx, qpos(ctx, qlast));
  const int64_t t0 = (int64_t)blockIdx.y * seg_tiles;
  int64_t t1 = (nmax + kTile - 1) / kTile;
  if (t1 > t0 + seg_tiles) t1 = t0 + seg_tiles;
  if (t0 >= t1) return;                                       // uniform over the workgroup
  if (tid < NQ) {
    const int64_t qi = q0 + tid;
    const bool valid = qi < ctx.n;
    s_tau[tid] = valid ? ws.tau[qi] : 3.0e38f;
    s_ne[tid] = valid ? (int32_t)n_eligible(ctx, qpos(ctx, qi)) : 0;
  }
  bf16x8 a[4][4];
  load_heads<H>(a, ws.yhat, q0, ctx.n, col, half);
  const void* cent = ctx.cent[0];
  __syncthreads();
  for (int64_t t = t0 + wave; t < t1; t += 4) {
    uint4 b[4];
    load_atile(b, cent, t * kTile + col, half);
    const int64_t g = t * kTile + col;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j][kk], __builtin_bit_cast(bf16x8, b[kk]),
                                                      acc, 0, 0, 0);
      float m[E];
      mh_max<H>(acc, m);
      // iteration i: the lanes of each half hold one position (for H = 8 the
      // two halves hold the same four; half h appends positions 2h, 2h + 1)
#pragma unroll
      for (int i = 0; i < E; ++i) {
        const bool mine = H != 8 || (i >> 1) == half;
        const int ql = mh_pos<H>(j, i, half);
        const int64_t qi = q0 + ql;
        const bool all = s_ne[ql] <= ctx.cap;
        const bool pass = mine && qi < ctx.n && g < s_ne[ql] && (all || m[i] >= s_tau[ql]);
        const uint64_t bal = __ballot(pass && !all);
        const uint64_t mh = half ? (bal >> 32) : (bal & 0xFFFFFFFFull);
        int base = 0;
        if (mh && col == 0) base = atomicAdd(&ws.cand_cnt[qi], __popcll(mh));
        base = __shfl(base, 32 * half, 64);
        if (pass) {
          uint2* dst = ws.cand + qi * (int64_t)ctx.cap;
          const uint2 e = make_uint2(__float_as_uint(m[i]), (uint32_t)g);
          if (all) {
            dst[g] = e;
          } else {
            const int slot = base + __popcll(mh & ((1ull << col) - 1ull));
            if (slot < ctx.cap) dst[slot] = e;
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ decode scoring (bf16)
// Decode scores one query per sequence against that sequence's own
// centroids: a matrix-vector product, bound by reading 128 B per bucket.
// Eight lanes share a centroid row (16 B = 8 dims each), so one wave-wide
// load reads 8 consecutive rows (1 KiB, fully coalesced) and the partial dot
// products are summed across the 8 lanes; each lane keeps 8 loads in flight.
constexpr int kDecMinRowsPerWg = 1024;  // fewest buckets per filter workgroup
constexpr int kDecSampPerWg = 512;      // sampled buckets per threshold workgroup

__device__ __forceinline__ void load_q8(float (&yq)[8], const void* yhat, int64_t qi, int sub) {
  const uint4 u = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(yhat) +
                                                 qi * kLatent)[sub];
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    yq[2 * e] = bf16_to_f32((uint16_t)(w[e] & 0xffffu));
    yq[2 * e + 1] = bf16_to_f32((uint16_t)(w[e] >> 16));
  }
}

__device__ __forceinline__ float dot8(const uint4& u, const float (&yq)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s = __builtin_fmaf(__uint_as_float(w[e] << 16), yq[2 * e], s);
    s = __builtin_fmaf(__uint_as_float(w[e] & 0xffff0000u), yq[2 * e + 1], s);
  }
  return s;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// sum over the 8 lanes of a row with DPP (quad xor 1, quad xor 2, half-row
// mirror): every lane of the 8 ends with the same sum
__device__ __forceinline__ float sum8(float s) {
  s += dpp_f<0xB1>(s);
  s += dpp_f<0x4E>(s);
  s += dpp_f<0x141>(s);
  return s;
}

// 64 rows per batch per wave: row rb + 8 k + (lane / 8), dims 8 (lane % 8) ..
__device__ __forceinline__ void load_rows8(uint4 (&u)[8], const uint4* cent, int64_t rb,
                                           int64_t rlast, int grp, int sub) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    int64_t row = rb + 8 * k + grp;
    row = row < rlast ? row : rlast;
    u[k] = cent[row * 8 + sub];
  }
}

constexpr int kDecStage = 64;           // LDS candidate slots per wave
constexpr int kDecStageAll = 512;       // ... when they hold every row of the wave

// tau of query qi from its sampled histogram, computed by one wave: lane l
// sums the 4 bins 4 (63 - l) .. 4 (63 - l) + 3, so an inclusive prefix over
// lanes counts samples from the top bin down; tau is the lower edge of the
// bin where the count reaches tau_samples (the same in every lane)
__device__ __forceinline__ float dec_tau_wave(const IndexCtx& ctx, const IndexWs& ws, int64_t qi,
                                             int lane) {
  const int64_t ne = n_eligible(ctx, ctx.pos[qi]);
  if (ne <= ctx.cap) return -3.0e38f;
  const uint32_t* h = ws.hist + qi * kBins;
  const int b0 = 4 * (63 - lane);
  const uint32_t c0 = h[b0], c1 = h[b0 + 1], c2 = h[b0 + 2], c3 = h[b0 + 3];
  const uint32_t mine = c0 + c1 + c2 + c3;
  uint32_t incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  const uint32_t want = (uint32_t)tau_samples(ctx);
  const uint64_t hit = __ballot(incl >= want);
  if (!hit) return -3.0e38f;
  const int l = __builtin_ctzll(hit);
  float tau = 0.f;
  if (lane == l) {
    uint32_t cum = incl - mine;
    int b = b0 + 3;
    const uint32_t cs[4] = {c0, c1, c2, c3};
    for (int e = 3; e >= 0; --e) {
      cum += cs[e];
      b = b0 + e;
      if (cum >= want) break;
    }
    tau = (float)b / (kBins / 2) - 1.0f;
  }
  return __shfl(tau, l, 64);
}

// grid.x = chunks of `rows_per_wg` buckets (a multiple of 256), grid.y =
// query (sequence).  Scores >= tau are staged per wave in LDS; at the end the
// workgroup reserves its slots with one atomic (a sequence's counter is hit
// once per workgroup, not once per wave, so the same-address atomics that
// end every workgroup stay few).  The candidate count starts at zero
// (k_dec_prep).  Each wave keeps two batches of 8 row loads in flight.
// S: LDS candidate slots per wave.  With S = kDecStageAll the launcher
// guarantees that a wave's rows (rows_per_wg / 4) fit, so the loop holds no
// global memory operation besides its loads: with a store or an atomic that
// may be in flight beside them, the compiler waits for every load before
// using any (the batches then stop overlapping).
template <int S>
__global__ __launch_bounds__(256) void k_dec_filter(IndexCtx ctx, IndexWs ws, int rows_per_wg) {
  __shared__ uint2 s_buf[4][S];
  __shared__ int s_cnt[4];
  __shared__ int s_base;
  const int64_t qi = blockIdx.y;
  const int64_t ne = n_eligible(ctx, ctx.pos[qi]);
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_wg;
  if (r0 >= ne) return;                                  // uniform over the workgroup
  const int64_t r1 = r0 + rows_per_wg < ne ? r0 + rows_per_wg : ne;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane & 7, grp = lane >> 3;
  const uint4* cent = reinterpret_cast<const uint4*>(ctx.cent[qi]);
  const int64_t rlast = r1 - 1;
  int64_t rb = r0 + 64 * wave;
  uint4 ua[8], ub[8];
  load_rows8(ua, cent, rb, rlast, grp, sub);            // in flight while tau is derived
  float yq[8];
  load_q8(yq, ws.yhat, qi, sub);
  // every wave derives tau from the sampled histogram (the same value)
  const float tau = dec_tau_wave(ctx, ws, qi, lane);
  uint2* cand = ws.cand + qi * (int64_t)ctx.cap;
  uint2* stage = s_buf[wave];
  int cnt = 0;                                           // wave-uniform
  // a full stage goes out on its own (rare: the stage holds 64 candidates)
  auto flush_wave = [&]() {
    __builtin_amdgcn_wave_barrier();
    int base = 0;
    if (lane == 0) base = atomicAdd(&ws.cand_cnt[qi], cnt);
    base = __shfl(base, 0, 64);
    if (lane < cnt && base + lane < ctx.cap) cand[base + lane] = stage[lane];
    __builtin_amdgcn_wave_barrier();
    cnt = 0;
  };
  auto process = [&](const uint4 (&u)[8], int64_t rbb) {
    float sc[8];
    uint64_t m[8];
    int npass = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      sc[k] = sum8(dot8(u[k], yq));
      const bool pass = (sub == 0) & (rbb + 8 * k + grp < r1) & (sc[k] >= tau);
      m[k] = __ballot(pass);
      npass += __popcll(m[k]);
    }
    npass = __builtin_amdgcn_readfirstlane(npass);
    if (npass == 0) return;
    int base = cnt;
    uint2* dst = stage;
    if constexpr (S == kDecStage) {
      if (cnt + npass > S) flush_wave();
      base = cnt;
      if (npass > S) {                                     // only when every row passes
        int g = 0;
        if (lane == 0) g = atomicAdd(&ws.cand_cnt[qi], npass);
        base = __shfl(g, 0, 64);
        dst = cand;
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      if ((m[k] >> lane) & 1ull) {
        const int slot = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m[k] >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m[k], 0u));
        if (dst != cand || slot < ctx.cap)
          dst[slot] = make_uint2(__float_as_uint(sc[k]), (uint32_t)(rbb + 8 * k + grp));
      }
      base += __popcll(m[k]);
    }
    if (dst == stage) cnt += npass;
  };
  // batches of 64 rows per wave, 256 rows per workgroup step; the next
  // batch is requested before the current one is used (loads past r1 are
  // clamped to the last row and masked in process)
  for (;; rb += 512) {
    load_rows8(ub, cent, rb + 256, rlast, grp, sub);
    __builtin_amdgcn_sched_barrier(0);
    if (rb < r1) process(ua, rb);
    if (rb + 256 >= r1) break;
    load_rows8(ua, cent, rb + 512, rlast, grp, sub);
    __builtin_amdgcn_sched_barrier(0);
    process(ub, rb + 256);
    if (rb + 512 >= r1) break;
  }
  // one reservation per workgroup for what the waves still hold
  if (threadIdx.x < 4) s_cnt[threadIdx.x] = 0;
  __syncthreads();
  if (lane == 0) s_cnt[wave] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int tot = s_cnt[0] + s_cnt[1] + s_cnt[2] + s_cnt[3];
    s_base = tot > 0 ? atomicAdd(&ws.cand_cnt[qi], tot) : 0;
  }
  __syncthreads();
  int off = s_base;
  for (int w = 0; w < wave; ++w) off += s_cnt[w];
  for (int i = lane; i < cnt; i += 64)
    if (off + i < ctx.cap) cand[off + i] = stage[i];
}

// Sampled histogram for the decode threshold: grid.x = chunks of
// kDecSampPerWg samples, grid.y = query; one LDS histogram per workgroup,
// added into the query's global histogram (cleared by k_qnorm).
__global__ __launch_bounds__(256) void k_dec_hist(IndexCtx ctx, IndexWs ws) {
  __shared__ uint32_t h[kBins];
  const int64_t qi = blockIdx.y;
  const int64_t ne = n_eligible(ctx, ctx.pos[qi]);
  const int64_t n_samp = ne / kSampleStride;
  const int64_t j0 = (int64_t)blockIdx.x * kDecSampPerWg;
  if (ne <= ctx.cap || j0 >= n_samp) return;
  const int64_t j1 = j0 + kDecSampPerWg < n_samp ? j0 + kDecSampPerWg : n_samp;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int sub = lane & 7, grp = lane >> 3;
  h[tid] = 0u;
  float yq[8];
  load_q8(yq, ws.yhat, qi, sub);
  const uint4* cent = reinterpret_cast<const uint4*>(ctx.cent[qi]);
  __syncthreads();
  for (int64_t jb = j0 + 64 * wave; jb < j1; jb += 256) {
    uint4 u[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      int64_t j = jb + 8 * k + grp;
      j = j < j1 ? j : j1 - 1;
      u[k] = cent[sample_bucket(j) * 8 + sub];
    }
    __builtin_amdgcn_sched_barrier(0);   // all 8 loads before any use
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float s = sum8(dot8(u[k], yq));
      const int64_t j = jb + 8 * k + grp;
      if ((sub == 0) & (j < j1)) {
        int bin = (int)((s + 1.0f) * (kBins / 2));
        bin = bin < 0 ? 0 : (bin >= kBins ? kBins - 1 : bin);
        atomicAdd(&h[bin], 1u);
      }
    }
  }
  __syncthreads();
  if (h[tid]) atomicAdd(&ws.hist[qi * kBins + tid], h[tid]);
}

// ------------------------------------------------------------------ exact select
// Scalar (VALU) score of bucket g, same inputs as the MFMA path.
template <int DT>
__device__ __forceinline__ float vscore(const void* cent, int64_t g, const float* yq) {
  float s = 0.f;
  if (DT == LSA_BF16) {
    const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(cent) + g * kLatent);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint4 u = src[j];
      uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s = __builtin_fmaf(bf16_to_f32((uint16_t)(w[e] & 0xffff)), yq[8 * j + 2 * e], s);
        s = __builtin_fmaf(bf16_to_f32((uint16_t)(w[e] >> 16)), yq[8 * j + 2 * e + 1], s);
      }
    }
  } else {
    const float4* src = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(cent) + g * kLatent);
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float4 v = src[j];
      s = __builtin_fmaf(v.x, yq[4 * j], s);
      s = __builtin_fmaf(v.y, yq[4 * j + 1], s);
      s = __builtin_fmaf(v.z, yq[4 * j + 2], s);
      s = __builtin_fmaf(v.w, yq[4 * j + 3], s);
    }
  }
  return s;
}

// Scores of two rows (same summation order as vscore); both rows' loads are
// issued before either product, then `between` runs (more independent
// loads), then the products.
template <int DT, class F>
__device__ __forceinline__ void vscore2(const void* cent, int64_t ga, int64_t gb, const float* yq,
                                        float& sa, float& sb, F between) {
  if (DT == LSA_BF16) {
    const uint4* pa = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(cent) + ga * kLatent);
    const uint4* pb = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(cent) + gb * kLatent);
    uint4 ua[8], ub[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) ua[j] = pa[j];
#pragma unroll
    for (int j = 0; j < 8; ++j) ub[j] = pb[j];
    __builtin_amdgcn_sched_barrier(0);
    between();
    __builtin_amdgcn_sched_barrier(0);
    float x = 0.f, y = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t wa[4] = {ua[j].x, ua[j].y, ua[j].z, ua[j].w};
      const uint32_t wb[4] = {ub[j].x, ub[j].y, ub[j].z, ub[j].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x = __builtin_fmaf(bf16_to_f32((uint16_t)(wa[e] & 0xffff)), yq[8 * j + 2 * e], x);
        x = __builtin_fmaf(bf16_to_f32((uint16_t)(wa[e] >> 16)), yq[8 * j + 2 * e + 1], x);
        y = __builtin_fmaf(bf16_to_f32((uint16_t)(wb[e] & 0xffff)), yq[8 * j + 2 * e], y);
        y = __builtin_fmaf(bf16_to_f32((uint16_t)(wb[e] >> 16)), yq[8 * j + 2 * e + 1], y);
      }
    }
    sa = x;
    sb = y;
  } else {
    between();
    sa = vscore<DT>(cent, ga, yq);
    sb = vscore<DT>(cent, gb, yq);
  }
}

template <int DT>
__device__ __forceinline__ void load_yq(float* yq, const void* yhat, int64_t qi) {
  if (DT == LSA_BF16) {
    const uint16_t* src = reinterpret_cast<const uint16_t*>(yhat) + qi * kLatent;
#pragma unroll
    for (int d = 0; d < kLatent; ++d) yq[d] = bf16_to_f32(src[d]);
  } else {
    const float* src = reinterpret_cast<const float*>(yhat) + qi * kLatent;
#pragma unroll
    for (int d = 0; d < kLatent; ++d) yq[d] = src[d];
  }
}

// Max over the H query heads of query qi (bf16 yhat rows qi * H .. qi * H +
// H - 1) of their dot products with bucket row g: the exact fallback's score
// when queries bring several heads.
__device__ __forceinline__ float vscore_heads(const void* cent, int64_t g, const void* yhat,
                                              int64_t qi, int H) {
  const uint4* c = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(cent) + g * kLatent);
  uint4 cv[8];
#pragma unroll
  for (int v = 0; v < 8; ++v) cv[v] = c[v];
  float best = -__builtin_inff();
  for (int h = 0; h < H; ++h) {
    const uint4* y = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(yhat) +
                                                    (qi * H + h) * kLatent);
    float acc = 0.f;
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      const uint4 yv = y[v];
      const uint32_t cw[4] = {cv[v].x, cv[v].y, cv[v].z, cv[v].w};
      const uint32_t yw[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = __builtin_fmaf(bf16_to_f32((uint16_t)cw[e]), bf16_to_f32((uint16_t)yw[e]), acc);
        acc = __builtin_fmaf(bf16_to_f32((uint16_t)(cw[e] >> 16)), bf16_to_f32((uint16_t)(yw[e] >> 16)), acc);
      }
    }
    best = fmaxf(best, acc);
  }
  return best;
}

// 256-thread exclusive prefix sum; returns the exclusive value, *total = sum.
// Exclusive prefix sum of one int per thread over a workgroup of NT threads
// (wsum: NT / 64 ints of LDS); *total receives the sum of all.
template <int NT>
__device__ __forceinline__ int block_scan_nt(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    if (w < wave) base += wsum[w];
    tot += wsum[w];
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

__device__ __forceinline__ int block_scan_excl(int v, int* wsum, int* total) {
  return block_scan_nt<256>(v, wsum, total);
}

// Exact top-B of one query, for a workgroup whose candidate list is unusable
// (more than `cap` candidates, or fewer than k far keys in them while more
// buckets are eligible) or when exact selection is forced: the B-th largest
// score by 4 radix passes of 8 bits over the
// order-preserving integer image of the fp32 score, then every bucket above
// it and, among buckets equal to it, the lowest.  Writes raw score bits to
// skey[] and buckets to sbkt[] (LDS) and returns the count (min(B, ne)).
// `heads`: query heads per position (1 unless max-over-heads scoring; a
// compile-time 1 keeps the multi-head scorer out of the bucket kernels).
template <int DT, int NT = 256>
__device__ int exact_select_lds(const IndexCtx& ctx, const IndexWs& ws, int64_t qi, int64_t ne,
                                int64_t beff, uint32_t* skey, uint32_t* sbkt, uint32_t* hist,
                                uint32_t* s_prefix, uint32_t* s_want, int* wsum, int* s_out,
                                int heads) {
  const int tid = threadIdx.x;
  const void* cent = qcent(ctx, qi);
  float yq[kLatent];
  load_yq<DT>(yq, ws.yhat, qi);
  uint32_t prefix = 0, mask = 0;
  uint32_t want = (uint32_t)beff;
  if (tid == 0) *s_out = 0;
  if (beff > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int b = tid; b < 256; b += NT) hist[b] = 0;
      __syncthreads();
      for (int64_t g = tid; g < ne; g += NT) {
        const uint32_t key = f32_orderable(heads > 1 ? vscore_heads(cent, g, ws.yhat, qi, heads)
                                                     : vscore<DT>(cent, g, yq));
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid == 0) {
        uint32_t cum = 0;
        for (int b = 255; b >= 0; --b) {
          if (cum + hist[b] >= want) {
            *s_prefix = prefix | ((uint32_t)b << shift);
            *s_want = want - cum;
            break;
          }
          cum += hist[b];
        }
      }
      __syncthreads();
      prefix = *s_prefix;
      want = *s_want;
      mask |= 255u << shift;
      __syncthreads();
    }
    int eq_base = 0;
    for (int64_t g0 = 0; g0 < ne; g0 += NT) {
      const int64_t g = g0 + tid;
      float s = 0.f;
      uint32_t key = 0;
      if (g < ne) {
        s = heads > 1 ? vscore_heads(cent, g, ws.yhat, qi, heads) : vscore<DT>(cent, g, yq);
        key = f32_orderable(s);
      }
      const int gt = (g < ne) && key > prefix;
      const int eq = (g < ne) && key == prefix;
      int eq_tot;
      const int eq_rank = eq_base + block_scan_nt<NT>(eq, wsum, &eq_tot);
      if (gt || (eq && eq_rank < (int)want)) {
        const int slot = atomicAdd(s_out, 1);
        if (slot < ctx.cap) { skey[slot] = __float_as_uint(s); sbkt[slot] = (uint32_t)g; }
      }
      eq_base += eq_tot;
    }
  }
  __syncthreads();
  if (tid == 0) ws.status[qi] = 1;
  return (int)beff;
}

// ------------------------------------------------------------------ tree search
// One wave per query.  Beam descent from the root, keeping the best `beam`
// eligible children (score desc, node asc) on every level down to lstar; then
// every eligible bucket under the final beam becomes a candidate.
// The `keep` largest of up to 128 unique nonzero 64-bit keys held two per lane
// (zero = empty): the keep-th largest upper half (score) by a bitwise search
// with wave ballots, then, only when that score is tied, the same search on
// the lower half among the tied keys.  Returns each lane's two "selected"
// flags; exactly `keep` keys are selected (keep <= number of nonzero keys).
__device__ __forceinline__ uint32_t kth_largest_u32(uint32_t a, uint32_t b, bool va, bool vb,
                                                    int keep) {
  uint32_t prefix = 0;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t cand = prefix | (1u << bit);
    const int cnt = __popcll(__ballot(va && a >= cand)) + __popcll(__ballot(vb && b >= cand));
    if (cnt >= keep) prefix = cand;
  }
  return prefix;
}

__device__ __forceinline__ void wave_select_top(uint64_t e0, uint64_t e1, int keep, bool& s0,
                                                bool& s1) {
  const uint32_t u0 = (uint32_t)(e0 >> 32), u1 = (uint32_t)(e1 >> 32);
  const uint32_t smin = kth_largest_u32(u0, u1, true, true, keep);
  const int gt = __popcll(__ballot(u0 > smin)) + __popcll(__ballot(u1 > smin));
  const bool q0 = u0 == smin, q1 = u1 == smin;
  const int eq = __popcll(__ballot(q0)) + __popcll(__ballot(q1));
  const int need = keep - gt;
  if (need == eq) {
    s0 = u0 >= smin;
    s1 = u1 >= smin;
  } else {
    // tied scores: the lower halves (complemented node ids) break the tie
    const uint32_t v0 = (uint32_t)e0, v1 = (uint32_t)e1;
    const uint32_t vmin = kth_largest_u32(v0, v1, q0, q1, need);
    s0 = u0 > smin || (q0 && v0 >= vmin);
    s1 = u1 > smin || (q1 && v1 >= vmin);
  }
}

template <int DT>
__global__ __launch_bounds__(64) void k_tree_search(IndexCtx ctx, TreeCtx tc, IndexWs ws) {
  extern __shared__ int32_t tsm[];
  int32_t* bufA = tsm;
  int32_t* bufB = tsm + ctx.cap;
  __shared__ int32_t beam[kMaxBeam];
  __shared__ int s_nbeam;
  const int lane = threadIdx.x;
  const int64_t qi = blockIdx.x;
  if (qi >= ctx.n) return;
  const int64_t p = qpos(ctx, qi);
  const int64_t qb = p / kBlock;
  const int64_t ne = n_eligible(ctx, p);
  if (lane == 0) { ws.status[qi] = 0; }
  if (ne == 0) {
    if (lane == 0) ws.cand_cnt[qi] = 0;
    return;
  }
  float yq[kLatent];
  load_yq<DT>(yq, ws.yhat, qi);
  if (lane == 0) { beam[0] = 0; s_nbeam = 1; }
  __builtin_amdgcn_wave_barrier();
  __syncthreads();
  int nbeam = 1;
  for (int lvl = tc.height - 1; lvl >= tc.lstar; --lvl) {
    // both children of beam slot `lane`: one 8-byte load of the pair, then
    // both centroids and smallest blocks together (index 0 stands in for a
    // missing child and is masked afterwards)
    const int32_t* chl = tc.child[lvl + 1];
    const void* cl = tc.cent[lvl];
    const int32_t* mbl = tc.minb[lvl];
    int32_t c0 = -1, c1 = -1;
    if (lane < nbeam) {
      const int2 cc = reinterpret_cast<const int2*>(chl)[beam[lane]];
      c0 = cc.x;
      c1 = cc.y;
    }
    const int32_t g0 = c0 >= 0 ? c0 : 0, g1 = c1 >= 0 ? c1 : 0;
    int64_t mb0 = (int64_t)g0 / kBuckets, mb1 = (int64_t)g1 / kBuckets;
    float sc0, sc1;
    vscore2<DT>(cl, g0, g1, yq, sc0, sc1, [&]() {
      if (lvl > 0) {
        mb0 = mbl[g0];
        mb1 = mbl[g1];
      }
    });
    uint64_t e[2];
    e[0] = (c0 >= 0 && mb0 < qb)
               ? ((uint64_t)f32_orderable(sc0) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)c0) : 0ull;
    e[1] = (c1 >= 0 && mb1 < qb)
               ? ((uint64_t)f32_orderable(sc1) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)c1) : 0ull;
    // valid entries are nonzero (the order-preserving image of a finite score
    // is at least 0x00800000); the next beam is the set of the `keep` largest
    // keys (score desc, node asc), in no particular order
    const int nvalid = __popcll(__ballot(e[0] != 0)) + __popcll(__ballot(e[1] != 0));
    const int keep = nvalid < tc.beam ? nvalid : tc.beam;
    bool s0 = false, s1 = false;
    if (keep > 0) wave_select_top(e[0], e[1], keep, s0, s1);
    const uint64_t m0 = __ballot(s0), m1 = __ballot(s1);
    const int p0 = __popcll(m0 & ((1ull << lane) - 1ull));
    const int p1 = __popcll(m0) + __popcll(m1 & ((1ull << lane) - 1ull));
    __syncthreads();
    if (s0 && p0 < keep) beam[p0] = (int32_t)(0xFFFFFFFFu - (uint32_t)(e[0] & 0xFFFFFFFFu));
    if (s1 && p1 < keep) beam[p1] = (int32_t)(0xFFFFFFFFu - (uint32_t)(e[1] & 0xFFFFFFFFu));
    nbeam = keep;
    __syncthreads();
  }
  // expand the final beam down to the buckets
  int n = nbeam;
  for (int j = lane; j < n; j += 64) bufA[j] = beam[j];
  __syncthreads();
  int32_t* cur = bufA;
  int32_t* nxt = bufB;
  for (int lvl = tc.lstar; lvl >= 1; --lvl) {
    int base = 0;
    for (int j0 = 0; j0 < n; j0 += 32) {
      const int j = j0 + (lane >> 1);
      int32_t c = -1;
      if (j < n) c = tc.child[lvl][2 * cur[j] + (lane & 1)];
      const uint64_t bal = __ballot(c >= 0);
      const int pos = base + __popcll(bal & ((1ull << lane) - 1ull));
      if (c >= 0 && pos < ctx.cap) nxt[pos] = c;
      base += __popcll(bal);
    }
    n = base < ctx.cap ? base : ctx.cap;
    __syncthreads();
    int32_t* t = cur; cur = nxt; nxt = t;
  }
  // score eligible buckets and write the candidate list
  uint2* cand = ws.cand + qi * (int64_t)ctx.cap;
  int out = 0;
  // four buckets per lane per round, so their centroid loads overlap
  for (int j0 = 0; j0 < n; j0 += 256) {
    int32_t g[4];
    bool ok[4];
    float s[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = j0 + 64 * u + lane;
      g[u] = j < n ? cur[j] : -1;
      ok[u] = g[u] >= 0 && (int64_t)g[u] < ne;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) s[u] = vscore<DT>(tc.cent[0], ok[u] ? g[u] : 0, yq);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint64_t bal = __ballot(ok[u]);
      const int pos = out + __popcll(bal & ((1ull << lane) - 1ull));
      if (ok[u]) cand[pos] = make_uint2(__float_as_uint(s[u]), (uint32_t)g[u]);
      out += __popcll(bal);
    }
  }
  if (lane == 0) ws.cand_cnt[qi] = out;
}

// ------------------------------------------------------------------ wide / fixed-level tree search
// Beams wider than a wave (up to kMaxBeamWide nodes) and the fixed-level
// search ([visual "A worked example"], table of search styles: score coarse
// groups, then refine inside the winners): the first stage scores every
// eligible node of the start level S (the root's children when S is the top)
// and keeps the best `beam`; each level below keeps the best `beam` of the
// kept nodes' eligible children, down to l*; the eligible buckets under the
// final beam become the candidates, as in k_tree_search.  One workgroup of
// 256 threads per query.  "Best" is (score desc, node asc): a radix select of
// the beam-th largest orderable score (4 passes of 8 bits), then the nodes
// above it and, among the nodes equal to it, the lowest.
constexpr int kWideNT = 256;

// The beam-th largest orderable score among items 0 .. n-1 (key(i) = 0: not
// an item), and how many items equal to it are to be taken.  Every thread
// returns the same values.
template <class Key>
__device__ __forceinline__ void wide_threshold(int64_t n, int want, Key key, uint32_t* hist,
                                               uint32_t* s_prefix, uint32_t* s_want,
                                               uint32_t& prefix, uint32_t& need) {
  const int tid = threadIdx.x;
  uint32_t pre = 0, mask = 0, w = (uint32_t)want;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int b = tid; b < 256; b += kWideNT) hist[b] = 0;
    __syncthreads();
    for (int64_t i = tid; i < n; i += kWideNT) {
      const uint32_t k = key(i);
      if (k && (k & mask) == pre) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      uint32_t cum = 0;
      // fewer items than wanted (known after the first pass): take them all,
      // i.e. every key above 0 and none equal to it
      *s_prefix = 0;
      *s_want = 0;
      for (int b = 255; b >= 0; --b) {
        if (cum + hist[b] >= w) {
          *s_prefix = pre | ((uint32_t)b << shift);
          *s_want = w - cum;
          break;
        }
        cum += hist[b];
      }
    }
    __syncthreads();
    pre = *s_prefix;
    w = *s_want;
    mask |= 255u << shift;
    __syncthreads();
    if (pre == 0) break;            // uniform: every thread read the same value
  }
  prefix = pre;
  need = w;
}

template <int DT>
__global__ __launch_bounds__(kWideNT) void k_tree_search_wide(IndexCtx ctx, TreeCtx tc, IndexWs ws) {
  extern __shared__ int32_t tsm[];
  int32_t* bufA = tsm;
  int32_t* bufB = tsm + ctx.cap;
  __shared__ uint32_t ckey[2 * kMaxBeamWide];     // children of the beam: orderable score
  __shared__ int32_t cnode[2 * kMaxBeamWide];     //   and node
  __shared__ int32_t beam[kMaxBeamWide];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix, s_want;
  __shared__ int wsum[kWideNT / 64];
  __shared__ int s_cnt;
  const int tid = threadIdx.x;
  const int64_t qi = blockIdx.x;
  if (qi >= ctx.n) return;
  const int64_t p = qpos(ctx, qi);
  const int64_t qb = p / kBlock;
  const int64_t ne = n_eligible(ctx, p);
  if (tid == 0) ws.status[qi] = 0;
  if (ne == 0) {
    if (tid == 0) ws.cand_cnt[qi] = 0;
    return;
  }
  float yq[kLatent];
  load_yq<DT>(yq, ws.yhat, qi);
  const int S = tc.start;
  int nbeam;
  // ---- first stage: every eligible node of level S (S < height), or the root
  if (S >= tc.height) {
    if (tid == 0) beam[0] = 0;
    nbeam = 1;
  } else {
    const int64_t nS = tc.nodes[S];
    const void* cS = tc.cent[S];
    const int32_t* mS = tc.minb[S];
    auto elig = [&](int64_t g) { return S == 0 ? g < ne : (int64_t)mS[g] < qb; };
    auto key = [&](int64_t g) -> uint32_t {
      return elig(g) ? f32_orderable(vscore<DT>(cS, g, yq)) : 0u;
    };
    uint32_t prefix, need;
    wide_threshold(nS, tc.beam, key, hist, &s_prefix, &s_want, prefix, need);
    // in node order: every node above the threshold, and the first `need` equal to it
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    int eq_base = 0;
    for (int64_t g0 = 0; g0 < nS; g0 += kWideNT) {
      const int64_t g = g0 + tid;
      const uint32_t k = g < nS ? key(g) : 0u;
      const int gt = k != 0 && k > prefix;
      const int eq = k != 0 && k == prefix;
      int eq_tot;
      const int eq_rank = eq_base + block_scan_nt<kWideNT>(eq, wsum, &eq_tot);
      if (gt || (eq && eq_rank < (int)need)) {
        const int slot = atomicAdd(&s_cnt, 1);
        if (slot < kMaxBeamWide) beam[slot] = (int32_t)g;
      }
      eq_base += eq_tot;
    }
    __syncthreads();
    nbeam = s_cnt < tc.beam ? s_cnt : tc.beam;
    __syncthreads();
  }
  // ---- descent: the best `beam` eligible children of the kept nodes, level by level
  for (int lvl = (S < tc.height ? S : tc.height) - 1; lvl >= tc.lstar; --lvl) {
    const int32_t* chl = tc.child[lvl + 1];
    const void* cl = tc.cent[lvl];
    const int32_t* mbl = tc.minb[lvl];
    const int n = 2 * nbeam;
    for (int i = tid; i < n; i += kWideNT) {
      const int32_t c = chl[2 * (int64_t)beam[i >> 1] + (i & 1)];
      bool ok = c >= 0;
      if (ok) ok = lvl == 0 ? (int64_t)c < ne : (int64_t)mbl[c] < qb;
      cnode[i] = c;
      ckey[i] = ok ? f32_orderable(vscore<DT>(cl, c, yq)) : 0u;
    }
    __syncthreads();
    uint32_t prefix, need;
    wide_threshold(n, tc.beam, [&](int64_t i) { return ckey[i]; }, hist, &s_prefix, &s_want,
                   prefix, need);
    // the items equal to the threshold: the `need` lowest nodes among them
    // (their number is small; ties need equal scores)
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    for (int i = tid; i < n; i += kWideNT) {
      const uint32_t k = ckey[i];
      bool take = k != 0 && k > prefix;
      if (k != 0 && k == prefix) {
        int lower = 0;
        for (int j = 0; j < n; ++j) lower += ckey[j] == prefix && cnode[j] < cnode[i];
        take = lower < (int)need;
      }
      if (take) {
        const int slot = atomicAdd(&s_cnt, 1);
        if (slot < kMaxBeamWide) beam[slot] = cnode[i];
      }
    }
    __syncthreads();
    nbeam = s_cnt < tc.beam ? s_cnt : tc.beam;
    __syncthreads();
  }
  // ---- the buckets under the final beam
  int n = nbeam;
  for (int j = tid; j < n; j += kWideNT) bufA[j] = beam[j];
  __syncthreads();
  int32_t* cur = bufA;
  int32_t* nxt = bufB;
  for (int lvl = tc.lstar; lvl >= 1; --lvl) {
    if (tid == 0) s_cnt = 0;
    __syncthreads();
    for (int i = tid; i < 2 * n; i += kWideNT) {
      const int32_t c = tc.child[lvl][2 * (int64_t)cur[i >> 1] + (i & 1)];
      if (c >= 0) {
        const int slot = atomicAdd(&s_cnt, 1);
        if (slot < ctx.cap) nxt[slot] = c;
      }
    }
    __syncthreads();
    n = s_cnt < ctx.cap ? s_cnt : ctx.cap;
    __syncthreads();
    int32_t* t = cur; cur = nxt; nxt = t;
  }
  uint2* cand = ws.cand + qi * (int64_t)ctx.cap;
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  for (int j = tid; j < n; j += kWideNT) {
    const int32_t g = cur[j];
    if (g >= 0 && (int64_t)g < ne) {
      const float sc = vscore<DT>(tc.cent[0], g, yq);
      const int slot = atomicAdd(&s_cnt, 1);
      cand[slot] = make_uint2(__float_as_uint(sc), (uint32_t)g);
    }
  }
  __syncthreads();
  if (tid == 0) ws.cand_cnt[qi] = s_cnt;
}

// ------------------------------------------------------------------ select + expand
// Lanes of the wave whose 8-bit digit equals this lane's (among `active`).
// lanes of `active` whose digit d (DB bits) equals this lane's
template <int DB>
__device__ __forceinline__ uint64_t match_digit(uint32_t d, uint64_t active) {
  uint64_t peers = active;
#pragma unroll
  for (int bit = 0; bit < DB; ++bit) {
    const uint64_t m = __ballot((d >> bit) & 1u);
    peers &= ((d >> bit) & 1u) ? m : ~m;
  }
  return peers;
}

// LSD radix sort (DB-bit digits) of n non-negative int32 keys in LDS that are
// distinct in their bits lo and up, ascending by those bits, by a workgroup of
// NT threads of which the first NW waves hold the keys (4, or 8 when NT >=
// 1024; at most NT / 64 x 256 / 2^DB).  Wave w owns the contiguous chunk
// [w*ch, (w+1)*ch); `tmp` is a second buffer of n ints, `cnt` NW x 2^DB
// counters (one row per wave).  After the first pass the scatter ranks lanes
// with equal digits by ballots, which keeps those passes stable.  Returns the
// buffer that holds the result.
template <int DB, int NT = 256>
__device__ int32_t* radix_sort_i32(int32_t* keys, int32_t* tmp, int n, int max_key, int lo,
                                   uint32_t* cnt) {
  constexpr int NB = 1 << DB;
  // at most four waves hold keys (eight in a workgroup of 1,024 threads, whose
  // query waits on it alone: measured best for the 500 - 1,100 items of a
  // decode step): fewer counters to clear and scan, which is what a sort of a
  // few hundred keys by a wide workgroup spends its time on
  constexpr int NW0 = NT >= 1024 ? 8 : ((NT / 64) < 4 ? (NT / 64) : 4);
  constexpr int NWc = (NT / 64) * 256 / NB;
  constexpr int NW = NW0 < NWc ? NW0 : NWc;
  static_assert(NW >= 1, "counters of one wave fit");
  constexpr int E = NB * NW / NT;                // counters per thread in the scan
  static_assert(E >= 1 && NB * NW == E * NT, "counter layout");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ch = (n + NW - 1) / NW;
  const int c0 = wave * ch;
  const int c1 = (c0 + ch) < n ? (c0 + ch) : n;
  int bits = lo;
  while (bits < 31 && (max_key >> bits) != 0) bits += DB;
  __shared__ int wsum_r[NT / 64];
  for (int shift = lo; shift < bits; shift += DB) {
    for (int i = tid; i < NW * NB; i += NT) cnt[i] = 0;
    __syncthreads();
    uint32_t* my = cnt + wave * NB;
    // histogram: one LDS atomic per key into its wave's counters.  Lanes with
    // the same digit (sorted runs share their high digits) serialise in the
    // LDS unit, which this kernel leaves mostly idle, instead of costing the
    // eight ballots and per-lane selects of match_digit in VALU, which bound it
    for (int e0 = c0; e0 < c1; e0 += 64) {
      const int e = e0 + lane;
      if (e < c1) atomicAdd(&my[((uint32_t)keys[e] >> shift) & (NB - 1)], 1u);
    }
    __syncthreads();
    {
      // digit-major, wave-minor exclusive offsets; thread t owns the E
      // consecutive (digit, wave) counters E t .. E t + E - 1
      uint32_t tot = 0;
#pragma unroll
      for (int q = 0; q < E; ++q) {
        const int x = E * tid + q;
        tot += cnt[(x % NW) * NB + x / NW];
      }
      int all;
      uint32_t run = (uint32_t)block_scan_nt<NT>((int)tot, wsum_r, &all);
#pragma unroll
      for (int q = 0; q < E; ++q) {
        const int x = E * tid + q;
        const uint32_t v = cnt[(x % NW) * NB + x / NW];
        cnt[(x % NW) * NB + x / NW] = run;
        run += v;
      }
    }
    __syncthreads();
    if (shift == lo) {
      // first pass: the input order carries nothing to keep, so equal digits
      // may land in any order (the keys are distinct in the sorted bits, so
      // later passes still order them fully): slots straight from the atomics
      for (int e0 = c0; e0 < c1; e0 += 64) {
        const int e = e0 + lane;
        if (e < c1) {
          const int32_t key = keys[e];
          tmp[atomicAdd(&my[((uint32_t)key >> shift) & (NB - 1)], 1u)] = key;
        }
      }
    } else {
      for (int e0 = c0; e0 < c1; e0 += 64) {
        const int e = e0 + lane;
        const bool ok = e < c1;
        const uint64_t active = __ballot(ok);
        const int32_t key = ok ? keys[e] : 0;
        const uint32_t d = ((uint32_t)key >> shift) & (NB - 1);
        const uint64_t peers = match_digit<DB>(d, active);
        if (ok) {
          const int rank = __popcll(peers & ((1ull << lane) - 1ull));
          const uint32_t base = my[d];
          tmp[base + rank] = key;
          if (rank == 0) my[d] = base + (uint32_t)__popcll(peers);
        }
      }
    }
    __syncthreads();
    int32_t* t = keys; keys = tmp; tmp = t;
  }
  return keys;
}

// Weighted radix select over items i < c that pass `filt`, ordered by a
// 32-bit key descending: finds the key K at which the running weight (from
// the largest key down) reaches `want`.  On return `want` is the weight
// still needed from the items whose key equals K.  Requires the total weight
// of the passing items to be >= want.
template <int NT, class KeyF, class FiltF>
__device__ uint32_t weighted_select(int c, KeyF key, FiltF filt, const uint8_t* w, uint32_t& want,
                                    uint32_t (*hist)[256], uint32_t* s_prefix, uint32_t* s_want) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[0][tid] = 0;
    __syncthreads();
    for (int i = tid; i < c; i += NT) {
      const uint32_t kv = key(i);
      if ((kv & mask) == prefix && w[i] && filt(i)) atomicAdd(&hist[0][(kv >> shift) & 255u], (uint32_t)w[i]);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns digits 4l .. 4l+3; weight of higher digits by a suffix scan
      const int l = tid;
      const uint32_t h0 = hist[0][4 * l], h1 = hist[0][4 * l + 1];
      const uint32_t h2 = hist[0][4 * l + 2], h3 = hist[0][4 * l + 3];
      const uint32_t lsum = h0 + h1 + h2 + h3;
      uint32_t x = lsum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_down(x, off, 64);
        if (l + off < 64) x += y;
      }
      const uint32_t above = x - lsum;   // weight of digits > 4l + 3
      const uint32_t c3 = above + h3, c2 = c3 + h2, c1 = c2 + h1, c0 = c1 + h0;
      int dig = -1;
      uint32_t before = 0;
      if (above < want && c3 >= want) { dig = 4 * l + 3; before = above; }
      else if (c3 < want && c2 >= want) { dig = 4 * l + 2; before = c3; }
      else if (c2 < want && c1 >= want) { dig = 4 * l + 1; before = c2; }
      else if (c1 < want && c0 >= want) { dig = 4 * l; before = c1; }
      if (dig >= 0) {
        *s_prefix = prefix | ((uint32_t)dig << shift);
        *s_want = want - before;
      }
    }
    __syncthreads();
    prefix = *s_prefix;
    want = *s_want;
    mask |= 255u << shift;
    __syncthreads();
  }
  return prefix;
}


// ---- selection helpers ----------------------------------------------------
// A query that waits alone on its workgroup (decode) pays for every barrier of
// the selection; these take the weighted select (every workgroup size) and,
// with 1,024 threads, the far-key sort in far fewer of them.

// Weighted selection in one histogram pass: candidates i < c of weight w[i] >
// 0, ordered by key descending, then bucket ascending; finds the candidate at
// which the running weight reaches `want` (its key, its bucket, and the weight
// still needed from it).  The keys are binned linearly over their range into
// kRangeBins bins (a monotone map, so every bin above the crossing one is taken
// whole); the crossing bin is then ranked exactly by one wave.  Returns false
// (uniformly) when that bin holds more than 64 candidates; the caller then
// takes the radix passes.  Workgroups of many queries (256 or 512 threads)
// use it too, with as many bins as their radix histograms hold.
constexpr int kRangeSel = 4 + 3 * 64;   // words of `sh`

template <int NT>
__device__ bool range_select(int c, const uint32_t* key, const uint32_t* bkt, const uint8_t* w,
                             uint32_t want, uint32_t* bins, uint32_t* sh, int* wsum,
                             uint32_t& key_out, uint32_t& bkt_out, uint32_t& rest_out) {
  constexpr int kRangeBins = NT >= 512 ? 2048 : 1024;   // <= the NT / 64 x 256 radix bins
  static_assert(NT >= 256 && kRangeBins % NT == 0 && kRangeBins <= NT / 64 * 256, "bins per thread");
  constexpr int E = kRangeBins / NT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // key range of the weighted candidates
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int i = tid; i < c; i += NT)
    if (w[i]) { lo = min(lo, key[i]); hi = max(hi, key[i]); }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo = min(lo, (uint32_t)__shfl_xor((int)lo, off, 64));
    hi = max(hi, (uint32_t)__shfl_xor((int)hi, off, 64));
  }
  uint32_t* s_lo = sh + 4;                     // [NT / 64] (reused below)
  uint32_t* s_hi = sh + 4 + 64;
  if (lane == 0) { s_lo[wave] = lo; s_hi[wave] = hi; }
  for (int b = tid; b < kRangeBins; b += NT) bins[b] = 0u;
  if (tid == 0) sh[2] = 0u;
  __syncthreads();
  lo = 0xFFFFFFFFu; hi = 0u;
#pragma unroll
  for (int q = 0; q < NT / 64; ++q) { lo = min(lo, s_lo[q]); hi = max(hi, s_hi[q]); }
  const float scale = (float)kRangeBins / ((float)(hi - lo) + 1.0f);
  auto bin_of = [&](uint32_t kv) {
    const int b = (int)((float)(kv - lo) * scale);
    return b < 0 ? 0 : (b >= kRangeBins ? kRangeBins - 1 : b);
  };
  __syncthreads();                             // s_lo / s_hi read before reuse
  for (int i = tid; i < c; i += NT)
    if (w[i]) atomicAdd(&bins[bin_of(key[i])], (uint32_t)w[i]);
  __syncthreads();
  // thread t owns bins kRangeBins - 1 - (E t + q), q < E (descending)
  uint32_t hb[E], mine = 0;
#pragma unroll
  for (int q = 0; q < E; ++q) { hb[q] = bins[kRangeBins - 1 - (E * tid + q)]; mine += hb[q]; }
  int all;
  uint32_t above = (uint32_t)block_scan_nt<NT>((int)mine, wsum, &all);
#pragma unroll
  for (int q = 0; q < E; ++q) {
    if (above < want && above + hb[q] >= want) { sh[0] = (uint32_t)(kRangeBins - 1 - (E * tid + q)); sh[1] = above; }
    above += hb[q];
  }
  __syncthreads();
  const int bstar = (int)sh[0];
  const uint32_t before = sh[1];
  // the crossing bin's candidates
  uint32_t* e_key = sh + 4;
  uint32_t* e_bkt = sh + 4 + 64;
  uint32_t* e_w = sh + 4 + 128;
  for (int i = tid; i < c; i += NT)
    if (w[i] && bin_of(key[i]) == bstar) {
      const uint32_t slot = atomicAdd(&sh[2], 1u);
      if (slot < 64) { e_key[slot] = key[i]; e_bkt[slot] = bkt[i]; e_w[slot] = w[i]; }
    }
  __syncthreads();
  const uint32_t n = sh[2];
  if (n > 64) return false;
  if (wave == 0) {
    // rank them by (key desc, bucket asc): lane l counts the weight of the
    // candidates ranked before its own (broadcast reads of the slots)
    const bool ok = (uint32_t)lane < n;
    const uint32_t mk = ok ? e_key[lane] : 0u, mb = ok ? e_bkt[lane] : 0u;
    uint32_t ahead = 0;
    for (uint32_t j = 0; j < n; ++j) {
      const uint32_t kj = e_key[j], bj = e_bkt[j];
      ahead += (kj > mk || (kj == mk && bj < mb)) ? e_w[j] : 0u;
    }
    const uint32_t wl = ok ? e_w[lane] : 0u;
    if (ok && before + ahead < want && before + ahead + wl >= want) {
      sh[0] = mk;
      sh[1] = mb;
      sh[3] = want - before - ahead;
    }
  }
  __syncthreads();
  key_out = sh[0];
  bkt_out = sh[1];
  rest_out = sh[3];
  __syncthreads();                             // sh read before any later reuse
  return true;
}

// One workgroup per query.  The walk over buckets ranked by (score desc,
// bucket asc) stops at the bucket where the running count of far keys
// reaches k.  That bucket is found without sorting: a radix select on the
// fp32 scores weighted by each bucket's far-key contribution gives the score
// S* at which the running sum crosses k; buckets above S* are taken whole,
// buckets tied at S* are walked in bucket order, the crossing one is cut.
// A candidate list is used when it holds every bucket scoring at least tau
// and k far keys (or every eligible bucket); else the exact top-B replaces
// it, so the crossing lies inside it.  The far keys are then radix-sorted.
// PER = candidate slots per thread (cap / NT): thread t owns candidates
// t, t + NT, ..., whose member words stay in registers from the contribution
// count to the emission.  NT = 256 for many queries; a few queries (decode)
// take NT = 1,024, which shortens every data-parallel phase of the one
// workgroup that a query waits on.
template <int DT, int PER, int NT = 256, bool SCAN = false>
__global__ __launch_bounds__(NT) void k_select_expand(IndexCtx ctx, IndexWs ws, int32_t* idx,
                                                       int32_t* count, int32_t* ranked,
                                                       int exact_mode) {
  extern __shared__ uint64_t sm[];
  const int cap = ctx.cap;
  const int kf = ctx.k > 1 ? ctx.k : 1;
  uint32_t* skey = reinterpret_cast<uint32_t*>(sm);           // [cap] orderable scores
  uint32_t* sbkt = skey + cap;                                // [cap] bucket ids
  uint8_t* contrib = reinterpret_cast<uint8_t*>(sbkt + cap);  // [cap]
  // the far items and the radix sort's second buffer: where skey/sbkt were
  // when both fit there (kf <= cap: every thread holds its candidates' bucket
  // ids in registers before the items are written), else far after contrib
  // and the second buffer over skey/sbkt (kf <= 2 cap since cap >= 3 B >
  // 3 k / 4).  The launcher sizes the dynamic LDS by the same rule.
  const bool far_low = kf <= cap;
  int32_t* far = far_low ? reinterpret_cast<int32_t*>(sm)
                         : reinterpret_cast<int32_t*>(contrib + cap);   // [kf]
  int32_t* far2 = far_low ? far + kf : reinterpret_cast<int32_t*>(sm);
  __shared__ uint32_t hist[NT / 64][256];
  __shared__ int wsum[NT / 64];
  __shared__ uint32_t s_prefix, s_want;
  __shared__ int s_total, s_trunc_m;
  __shared__ uint32_t s_rsel[kRangeSel];
  const int tid = threadIdx.x;
  const int64_t qi = blockIdx.x;
  // keys per scan run; 0 for buckets (a compile-time 0 keeps the scan
  // branches out of the bucket kernels, as SCAN = false also keeps out the
  // max-over-heads scorer of the exact fallback: SCAN selects the instance
  // for scans and for max-over-heads scoring)
  const int run_keys = SCAN ? ctx.run_keys : 0;
  if (qi >= ctx.n) return;
  const int64_t p = qpos(ctx, qi);
  const uint32_t* mem = qmem(ctx, qi);
  const int64_t s_end = p + 1 < ctx.n_sink ? p + 1 : ctx.n_sink;
  const int64_t w_start = p - ctx.window + 1 > 0 ? p - ctx.window + 1 : 0;
  // candidates (raw score bits, bucket) into LDS: from the scoring pass, or
  // from the exact selection when that list is unusable (exact_mode 1) or
  // always (exact_mode 2); tree candidates are taken as they are (mode 0)
  const uint2* cand = ws.cand + qi * (int64_t)cap;
  uint2 e[PER];
  if constexpr (NT >= 1024) {
    // a few queries (decode): every slot is requested together with the count,
    // which saves the count's latency on the path that a query waits on
#pragma unroll
    for (int jj = 0; jj < PER; ++jj) {
      const int i = tid + NT * jj;
      e[jj] = i < cap ? cand[i] : make_uint2(0, 0);
    }
  }
  int c = ws.cand_cnt[qi];
  bool used_exact = false;
  const int64_t ne = n_eligible(ctx, p);
  const int64_t beff = ne < ctx.top_b ? ne : ctx.top_b;
  // the scoring pass's candidates serve unless they overflowed the list (or
  // the ranking output asks for B buckets and they are fewer)
  bool need_exact = exact_mode == 2 || (exact_mode == 1 && (c > cap || (ranked && c < beff)));
  if (!need_exact) {
    c = c < cap ? c : cap;
    if constexpr (NT < 1024) {
#pragma unroll
      for (int jj = 0; jj < PER; ++jj) {
        const int i = tid + NT * jj;
        e[jj] = i < c ? cand[i] : make_uint2(0, 0);
      }
    }
#pragma unroll
    for (int jj = 0; jj < PER; ++jj) {
      const int i = tid + NT * jj;
      if (i < c) { skey[i] = e[jj].x; sbkt[i] = e[jj].y; }
    }
  }
  int total;
  // member words of this thread's candidates (all loads issued together;
  // from the candidate registers when they hold the list, before the barrier)
  uint32_t mw[PER];
#pragma unroll 1
  for (int pass = 0; pass < 2; ++pass) {
    if (need_exact) {
      used_exact = true;
      c = exact_select_lds<DT, NT>(ctx, ws, qi, ne, beff, skey, sbkt, &hist[0][0], &s_prefix,
                                   &s_want, wsum, &s_total, SCAN ? ctx.heads : 1);
    }
    const bool mw_early = NT >= 1024 && !used_exact;
    if (mw_early) {
#pragma unroll
      for (int jj = 0; jj < PER; ++jj) {
        const int i = tid + NT * jj;
        mw[jj] = (i < c && run_keys == 0) ? mem[e[jj].y] : 0xFFFFFFFFu;
      }
    }
    __syncthreads();
    if (!mw_early) {
#pragma unroll
      for (int jj = 0; jj < PER; ++jj) {
        const int i = tid + NT * jj;
        mw[jj] = (i < c && run_keys == 0) ? mem[sbkt[i]] : 0xFFFFFFFFu;
      }
    }
    // far-key contributions (members outside the near set)
    int my_w = 0;
#pragma unroll
    for (int jj = 0; jj < PER; ++jj) {
      const int i = tid + NT * jj;
      if (i >= c) continue;
      const uint32_t g = sbkt[i];
      const uint32_t m = mw[jj];
      const int64_t kb = (int64_t)(g / kBuckets) * kBlock;
      int ci = 0;
      if (run_keys) {
        // a scan's run: its keys that are not sinks (every eligible run ends
        // before the window)
        const int64_t r0 = (int64_t)g * run_keys;
        const int64_t lo = s_end > r0 ? s_end : r0;
        ci = r0 + run_keys > lo ? (int)(r0 + run_keys - lo) : 0;
      } else if (kb >= s_end && kb + kBlock <= w_start) {
        // block without sink or window keys: every member key is far
#pragma unroll
        for (int q = 0; q < kCapItems; ++q) ci += ((m >> (8 * q)) & 0xFFu) != 0xFFu ? kPool : 0;
      } else {
#pragma unroll
        for (int q = 0; q < kCapItems; ++q) {
          const uint32_t j = (m >> (8 * q)) & 0xFFu;
          if (j != 0xFFu) {
#pragma unroll
            for (int u = 0; u < kPool; ++u) {
              const int64_t key = kb + kPool * j + u;
              ci += !(key < s_end || key >= w_start);
            }
          }
        }
      }
      skey[i] = f32_orderable(__uint_as_float(skey[i]));
      contrib[i] = (uint8_t)ci;
      my_w += ci;
    }
    if (tid == 0) { s_trunc_m = 0; s_total = 0; }
    (void)block_scan_nt<NT>(my_w, wsum, &total);   // also orders the LDS writes above
    // candidates above tau holding fewer than k far keys while more buckets
    // are eligible: the exact top-B instead (uniform over the workgroup)
    need_exact = exact_mode == 1 && !used_exact && ctx.k > 0 && total < ctx.k && c < ne;
    if (!need_exact) break;
  }
  // optional output: the kept buckets best first (O(c^2) ranking; for tests)
  if (ranked) {
    const int nb = c < ctx.top_b ? c : ctx.top_b;
    for (int r = nb + tid; r < ctx.top_b; r += NT) ranked[qi * ctx.top_b + r] = -1;
    for (int i = tid; i < c; i += NT) {
      int ahead = 0;
      for (int j = 0; j < c; ++j)
        ahead += skey[j] > skey[i] || (skey[j] == skey[i] && sbkt[j] < sbkt[i]);
      if (ahead < nb) ranked[qi * ctx.top_b + ahead] = (int32_t)sbkt[i];
    }
  }
  // ---- weighted radix select: score S* where the running far-key count reaches k,
  // then the bucket g* among the buckets tied at S* (lowest bucket first)
  const int k = ctx.k;
  uint32_t prefix = 0, gstar_key = 0, want = (uint32_t)k;
  const bool cut = k > 0 && total >= k;
  if (cut) {
    bool fast = false;
    {
      uint32_t ko, bo, ro;
      fast = range_select<NT>(c, skey, sbkt, contrib, want, &hist[0][0], s_rsel, wsum, ko, bo, ro);
      if (fast) { prefix = ko; gstar_key = 0xFFFFFFFFu - bo; want = ro; }
    }
    if (!fast) {
    prefix = weighted_select<NT>(c, [&](int i) { return skey[i]; }, [&](int) { return true; },
                             contrib, want, hist, &s_prefix, &s_want);
    const uint32_t sstar = prefix;
    // buckets tied at S*: almost always one, which is then the cut bucket
    int n_eq = 0;
    for (int i = tid; i < c; i += NT)
      if (skey[i] == sstar && contrib[i]) { ++n_eq; s_prefix = 0xFFFFFFFFu - sbkt[i]; }
    int eq_tot;
    (void)block_scan_nt<NT>(n_eq, wsum, &eq_tot);
    if (eq_tot == 1) {
      gstar_key = s_prefix;
    } else {
      gstar_key = weighted_select<NT>(c, [&](int i) { return 0xFFFFFFFFu - sbkt[i]; },
                                  [&](int i) { return skey[i] == sstar; }, contrib, want, hist,
                                  &s_prefix, &s_want);
    }
    }
    if (tid == 0) s_trunc_m = (int)want;
  }
  __syncthreads();
  // ---- emit far keys: whole buckets above S* (every bucket without a cut),
  // the cut bucket's first members.  They are emitted as pooled items (4
  // consecutive keys at a multiple of 4) with the mask of their keys taken:
  // an item belongs to one bucket, so sorting the items by position sorts the
  // keys, with a quarter of the elements.
  const int trunc_m = s_trunc_m;
  const uint32_t gstar = 0xFFFFFFFFu - gstar_key;
  const int n_far = cut ? k : total;
  static_assert(kPool == 4, "items are packed as (position / 4) << 4 | 4-bit key mask");
  // the items of candidate i (bucket or run g) taking `take` far keys, in
  // member (= key) order
  auto for_items = [&](int i, uint32_t g, uint32_t m, int take, auto&& f) {
    if (run_keys) {
      // a scan's run of b keys (b = 1, 4 or 8, aligned to b): its first
      // `take` keys that are not sinks, as items of 4 keys
      const int64_t r0 = (int64_t)g * run_keys;
      if (run_keys == 1) {
        if (take > 0 && r0 >= s_end) f((int32_t)(((r0 >> 2) << 4) | (1 << (r0 & 3))));
        return;
      }
      for (int q = 0; q < run_keys / kPool && take > 0; ++q) {
        const int64_t k0 = r0 + kPool * q;
        uint32_t mask = 0;
#pragma unroll
        for (int u = 0; u < kPool; ++u)
          if (take > 0 && k0 + u >= s_end) { mask |= 1u << u; --take; }
        if (mask) f((int32_t)((k0 >> 2) << 4) | (int32_t)mask);
      }
      return;
    }
    const int64_t kb = (int64_t)(g / kBuckets) * kBlock;
    const bool clean = kb >= s_end && kb + kBlock <= w_start;   // no sink or window key
    if (clean && take == (int)contrib[i]) {
      // the whole bucket: every member item with all of its keys
#pragma unroll
      for (int q = 0; q < kCapItems; ++q) {
        const uint32_t j = (m >> (8 * q)) & 0xFFu;
        if (j != 0xFFu) f((int32_t)(((kb + kPool * j) >> 2) << 4) | 15);
      }
      return;
    }
#pragma unroll
    for (int q = 0; q < kCapItems; ++q) {
      const uint32_t j = (m >> (8 * q)) & 0xFFu;
      if (j == 0xFFu || take <= 0) break;
      const int64_t k0 = kb + kPool * j;
      uint32_t mask = 0;
#pragma unroll
      for (int u = 0; u < kPool; ++u) {
        const int64_t key = k0 + u;
        if (take > 0 && (clean || !(key < s_end || key >= w_start))) { mask |= 1u << u; --take; }
      }
      if (mask) f((int32_t)((k0 >> 2) << 4) | (int32_t)mask);
    }
  };
  int n_items;
  {
    auto take_of = [&](int i) -> int {
      if (!cut || skey[i] > prefix || (skey[i] == prefix && sbkt[i] < gstar)) return contrib[i];
      if (skey[i] == prefix && sbkt[i] == gstar) return trunc_m;
      return 0;
    };
    int tk[PER];
    uint32_t gb[PER];
    int mine = 0;
#pragma unroll
    for (int jj = 0; jj < PER; ++jj) {
      const int i = tid + NT * jj;
      tk[jj] = i < c ? take_of(i) : 0;
      gb[jj] = i < c ? sbkt[i] : 0u;
      if (tk[jj] > 0) for_items(i, gb[jj], mw[jj], tk[jj], [&](int32_t) { ++mine; });
    }
    // the scan's barriers also end every read of skey/sbkt, which far may overwrite
    int o = block_scan_nt<NT>(mine, wsum, &n_items);
#pragma unroll
    for (int jj = 0; jj < PER; ++jj)
      if (tk[jj] > 0)
        for_items(tid + NT * jj, gb[jj], mw[jj], tk[jj], [&](int32_t it) { far[o++] = it; });
  }
  __syncthreads();
  // sort by position (bits 4 and up); positions are below p.  A token scan
  // (runs of one key) emits one item per key, so two items may share a
  // position: their one-bit masks (bits 0..3) then order them, and the sort
  // takes every bit
  const int max_item = ((int)((p > 0 ? p : 0) >> 2) << 4) | 15;
  const int32_t* items = radix_sort_i32<8, NT>(far, far2, n_items, max_item, run_keys == 1 ? 0 : 4,
                                               &hist[0][0]);
  // sinks | far | window, -1 padded; the far keys come from the sorted items,
  // each thread expanding a contiguous run of them
  int32_t* out = idx + qi * (int64_t)ctx.list_len;
  int cnt;
  if (w_start <= s_end) {
    cnt = (int)(p + 1);
    for (int i = tid; i < ctx.list_len; i += NT) out[i] = i < cnt ? i : -1;
  } else {
    const int ns = (int)s_end, nw = (int)(p - w_start + 1);
    cnt = ns + n_far + nw;
    const int run = (n_items + NT - 1) / NT;
    const int i0 = tid * run < n_items ? tid * run : n_items;
    const int i1 = i0 + run < n_items ? i0 + run : n_items;
    int nk = 0;
    for (int i = i0; i < i1; ++i) nk += __popc((uint32_t)items[i] & 15u);
    int tot_k;
    int o = ns + block_scan_nt<NT>(nk, wsum, &tot_k);
    for (int i = i0; i < i1; ++i) {
      const int32_t it = items[i];
      const int32_t base = (it >> 4) << 2;
#pragma unroll
      for (int u = 0; u < kPool; ++u)
        if ((it >> u) & 1) out[o++] = base + u;
    }
    for (int i = tid; i < ctx.list_len; i += NT) {
      if (i < ns) out[i] = i;
      else if (i >= ns + n_far && i < cnt) out[i] = (int32_t)(w_start + (i - ns - n_far));
      else if (i >= cnt) out[i] = -1;
    }
  }
  if (tid == 0) count[qi] = cnt;
}

}  // namespace

// ------------------------------------------------------------------ launchers

hipError_t launch_qnorm(const float* y, int64_t n, void* yhat, int dtype, uint32_t* hist,
                        hipStream_t s) {
  if (n <= 0) return hipSuccess;
  dim3 grid((unsigned)((n + 15) / 16));
  if (dtype == LSA_BF16) hipLaunchKernelGGL(k_qnorm<LSA_BF16>, grid, dim3(256), 0, s, y, n, yhat, hist);
  else hipLaunchKernelGGL(k_qnorm<LSA_F32>, grid, dim3(256), 0, s, y, n, yhat, hist);
  return hipGetLastError();
}

hipError_t launch_dec_prep(const float* y, const float* k_new, const AppendJobs& jobs, int64_t n,
                           void* yhat, const IndexWs& ws, int dtype, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  dim3 grid((unsigned)((n + 15) / 16));
  if (dtype == LSA_BF16)
    hipLaunchKernelGGL(k_dec_prep<LSA_BF16>, grid, dim3(256), 0, s, y, k_new, jobs, n, yhat, ws);
  else
    hipLaunchKernelGGL(k_dec_prep<LSA_F32>, grid, dim3(256), 0, s, y, k_new, jobs, n, yhat, ws);
  return hipGetLastError();
}

static int64_t query_tiles(const IndexCtx& ctx) {
  return ctx.per_seq ? (ctx.n + 3) / 4 : (ctx.n + kQueriesPerWg - 1) / kQueriesPerWg;
}

hipError_t launch_thresh(const IndexCtx& ctx, const IndexWs& ws, int dtype, hipStream_t s) {
  if (ctx.n <= 0) return hipSuccess;
  if (ctx.heads > 1) {
    // prefill, bf16: 128 / H positions per workgroup
    const unsigned gx = (unsigned)((ctx.n * ctx.heads + 127) / 128);
    if (ctx.heads == 2) hipLaunchKernelGGL(k_mh_thresh<2>, dim3(gx), dim3(256), 0, s, ctx, ws);
    else if (ctx.heads == 4) hipLaunchKernelGGL(k_mh_thresh<4>, dim3(gx), dim3(256), 0, s, ctx, ws);
    else hipLaunchKernelGGL(k_mh_thresh<8>, dim3(gx), dim3(256), 0, s, ctx, ws);
    return hipGetLastError();
  }
  if (ctx.per_seq && dtype == LSA_BF16) {
    int64_t max_samp = 0;
    for (int64_t i = 0; i < ctx.n; ++i) {
      const int64_t ns = n_eligible(ctx, ctx.pos[i]) / kSampleStride;
      max_samp = ns > max_samp ? ns : max_samp;
    }
    const int64_t gx = (max_samp + kDecSampPerWg - 1) / kDecSampPerWg;
    // tau itself is derived by every k_dec_filter wave from the histogram
    if (gx > 0)
      hipLaunchKernelGGL(k_dec_hist, dim3((unsigned)gx, (unsigned)ctx.n), dim3(256), 0, s, ctx, ws);
    return hipGetLastError();
  }
  if (ctx.per_seq) {
    // decode: many workgroups per query, global histogram, then tau
    int64_t max_tiles = 0;
    for (int64_t i = 0; i < ctx.n; ++i) {
      const int64_t t = n_eligible(ctx, ctx.pos[i]) / kTile;
      max_tiles = t > max_tiles ? t : max_tiles;
    }
    // tiles of 32 sampled buckets (one bucket in 16), kHistSegTiles per workgroup
    const int64_t samp_tiles = (max_tiles * kTile / kSampleStride + kTile - 1) / kTile;
    const int64_t gx = (samp_tiles + kHistSegTiles - 1) / kHistSegTiles;
    if (gx > 0) {
      dim3 grid((unsigned)gx, (unsigned)query_tiles(ctx));
      if (dtype == LSA_BF16) hipLaunchKernelGGL(k_thresh_hist<LSA_BF16>, grid, dim3(256), 0, s, ctx, ws);
      else hipLaunchKernelGGL(k_thresh_hist<LSA_F32>, grid, dim3(256), 0, s, ctx, ws);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_thresh_tau, dim3((unsigned)((ctx.n + 63) / 64)), dim3(64), 0, s, ctx, ws, 0);
    return hipGetLastError();
  }
  if (dtype == LSA_BF16) {
    // 128 queries per wave; split the samples when there are few query tiles
    const int64_t qt = query_tiles(ctx);
    const int64_t last = ctx.q_start + ctx.n - 1;
    const int64_t samp_tiles = (n_eligible(ctx, last) / kSampleStride + kTile - 1) / kTile;
    int64_t split = qt < 128 ? (256 + qt - 1) / qt : 1;
    const int64_t max_split = (samp_tiles + 15) / 16;
    if (split > max_split) split = max_split;
    if (split < 1) split = 1;
    const int64_t seg = (samp_tiles + split - 1) / split;
    if (split > 1) {
      const int64_t nh = ctx.n * kBins;
      const int64_t gb = (nh + 255) / 256 < 4096 ? (nh + 255) / 256 : 4096;
      hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)gb), dim3(256), 0, s, ws.hist, nh, 0u);
    }
    hipLaunchKernelGGL(k_thresh_q128, dim3((unsigned)qt, (unsigned)split), dim3(512), 0, s, ctx, ws,
                       (int)(seg > 0 ? seg : 1), (int)(split > 1));
    if (split > 1)
      hipLaunchKernelGGL(k_thresh_tau, dim3((unsigned)((ctx.n + 63) / 64)), dim3(64), 0, s, ctx, ws, 1);
    return hipGetLastError();
  }
  dim3 grid((unsigned)query_tiles(ctx));
  if (dtype == LSA_BF16) hipLaunchKernelGGL(k_thresh<LSA_BF16>, grid, dim3(256), 0, s, ctx, ws);
  else hipLaunchKernelGGL(k_thresh<LSA_F32>, grid, dim3(256), 0, s, ctx, ws);
  return hipGetLastError();
}

hipError_t launch_score_filter(const IndexCtx& ctx, const IndexWs& ws, int dtype,
                               int64_t max_tiles, hipStream_t s) {
  if (ctx.n <= 0 || max_tiles <= 0) return hipSuccess;
  if (ctx.heads > 1) {
    constexpr int kSeg = 128;                       // tiles (4,096 buckets) per workgroup
    const dim3 grid((unsigned)((ctx.n * ctx.heads + 127) / 128), (unsigned)((max_tiles + kSeg - 1) / kSeg));
    if (ctx.heads == 2) hipLaunchKernelGGL(k_mh_filter<2>, grid, dim3(256), 0, s, ctx, ws, kSeg);
    else if (ctx.heads == 4) hipLaunchKernelGGL(k_mh_filter<4>, grid, dim3(256), 0, s, ctx, ws, kSeg);
    else hipLaunchKernelGGL(k_mh_filter<8>, grid, dim3(256), 0, s, ctx, ws, kSeg);
    return hipGetLastError();
  }
  if (!ctx.per_seq && dtype == LSA_BF16) {
    // segment length: about kCapL / 2 expected candidates per query for the
    // widest query (tau_candidates of ne_max pass), so the LDS lists rarely overflow;
    // when even 16 tiles expect more, workgroups take the high-pass epilogue
    // and longer segments only save query loads
    const int64_t last = ctx.q_start + ctx.n - 1;
    const int64_t ne_max = n_eligible(ctx, last);
    const int64_t seg_buckets = (int64_t)(kCapL / 2) * ne_max / tau_candidates(ctx);
    int64_t seg = seg_buckets / kTile;
    seg = seg < 16 ? 16 : (seg > 512 ? 512 : seg & ~(int64_t)7);
    if (seg_buckets < 16 * kTile) seg = 128;
    // query tiles [x_lp, qt) are low-pass (ne grows with the position, so the
    // first query of a tile has its smallest ne); earlier tiles are high-pass
    const int64_t qt = query_tiles(ctx);
    const int64_t nseg = (max_tiles + seg - 1) / seg;
    int64_t x_lp = qt;
    for (int64_t x = 0; x < qt; ++x) {
      const int64_t nmin = n_eligible(ctx, ctx.q_start + x * kQueriesPerWg);
      if (nmin > ctx.cap && seg * kTile * tau_candidates(ctx) <= (int64_t)(kCapL / 2) * nmin) {
        x_lp = x;
        break;
      }
    }
    if (x_lp > 0)
      hipLaunchKernelGGL(k_score_highpass, dim3((unsigned)x_lp, (unsigned)nseg), dim3(256), 0, s,
                         ctx, ws, (int)seg);
    if (x_lp < qt) {
      // 128 queries per workgroup (4 groups of 32 per wave); 3 groups (96
      // queries) measured slower at two or three waves per SIMD
      constexpr int kNG = 4;
      const int64_t qb = x_lp * kQueriesPerWg;
      const int64_t nt = (ctx.n - qb + 32 * kNG - 1) / (32 * kNG);
      hipLaunchKernelGGL(k_score_lowpass<kNG>, dim3((unsigned)nt, (unsigned)nseg), dim3(256), 0, s,
                         ctx, ws, (int)seg, qb);
    }
    return hipGetLastError();
  }
  if (ctx.per_seq && dtype == LSA_BF16) {
    // about 1,024 workgroups in all, at least kDecMinRowsPerWg buckets each
    const int64_t rows = max_tiles * kTile;
    int64_t steps = (rows * ctx.n + 1024 * 256 - 1) / (1024 * 256);
    if (steps < kDecMinRowsPerWg / 256) steps = kDecMinRowsPerWg / 256;
    const int64_t per = 256 * steps;
    const int64_t gx = (rows + per - 1) / per;
    if (per / 4 <= kDecStageAll)
      hipLaunchKernelGGL(k_dec_filter<kDecStageAll>, dim3((unsigned)gx, (unsigned)ctx.n), dim3(256),
                         0, s, ctx, ws, (int)per);
    else
      hipLaunchKernelGGL(k_dec_filter<kDecStage>, dim3((unsigned)gx, (unsigned)ctx.n), dim3(256), 0,
                         s, ctx, ws, (int)per);
    return hipGetLastError();
  }
  // decode has few queries: shorter segments give enough workgroups to stream HBM
  const int seg = ctx.per_seq ? 32 : kSegTiles;
  dim3 grid((unsigned)((max_tiles + seg - 1) / seg), (unsigned)query_tiles(ctx));
  if (dtype == LSA_BF16) hipLaunchKernelGGL(k_score_filter<LSA_BF16>, grid, dim3(256), 0, s, ctx, ws, seg);
  else hipLaunchKernelGGL(k_score_filter<LSA_F32>, grid, dim3(256), 0, s, ctx, ws, seg);
  return hipGetLastError();
}

static void allow_large_lds(const void* fn, size_t bytes = 128 * 1024);

hipError_t launch_tree_search(const IndexCtx& ctx, const TreeCtx& tc, const IndexWs& ws,
                              int dtype, hipStream_t s) {
  if (ctx.n <= 0) return hipSuccess;
  if (tc.beam > kMaxBeam || tc.start < tc.height) {
    // wider beams and the fixed-level first stage: one workgroup per query
    const size_t smem = (size_t)2 * ctx.cap * sizeof(int32_t);
    allow_large_lds(reinterpret_cast<const void*>(k_tree_search_wide<LSA_BF16>));
    allow_large_lds(reinterpret_cast<const void*>(k_tree_search_wide<LSA_F32>));
    dim3 grid((unsigned)ctx.n);
    if (dtype == LSA_BF16)
      hipLaunchKernelGGL(k_tree_search_wide<LSA_BF16>, grid, dim3(kWideNT), smem, s, ctx, tc, ws);
    else
      hipLaunchKernelGGL(k_tree_search_wide<LSA_F32>, grid, dim3(kWideNT), smem, s, ctx, tc, ws);
    return hipGetLastError();
  }
  static bool once = false;
  if (!once) {
    allow_large_lds(reinterpret_cast<const void*>(k_tree_search<LSA_BF16>));
    allow_large_lds(reinterpret_cast<const void*>(k_tree_search<LSA_F32>));
    once = true;
  }
  const size_t smem = (size_t)2 * ctx.cap * sizeof(int32_t);
  dim3 grid((unsigned)ctx.n);
  if (dtype == LSA_BF16) hipLaunchKernelGGL(k_tree_search<LSA_BF16>, grid, dim3(64), smem, s, ctx, tc, ws);
  else hipLaunchKernelGGL(k_tree_search<LSA_F32>, grid, dim3(64), smem, s, ctx, tc, ws);
  return hipGetLastError();
}

// Kernels whose dynamic LDS grows with k may need more than the default 64 KiB.
// The request is advisory: an error from it is consumed so that it cannot be
// mistaken for a launch failure by the next hipGetLastError.
static void allow_large_lds(const void* fn, size_t bytes) {
  (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  (void)hipGetLastError();
}

static int pow2_ceil_host(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

hipError_t launch_select_expand(const IndexCtx& ctx, const IndexWs& ws, int32_t* idx,
                                int32_t* count, int32_t* ranked, int dtype, int exact_mode,
                                hipStream_t s) {
  if (ctx.n <= 0) return hipSuccess;
  const int64_t kf = ctx.k > 1 ? ctx.k : 1;
  if (kf > 2 * (int64_t)ctx.cap) return hipErrorInvalidValue;   // the far-key sort reuses 8 cap bytes
  // far items over the candidates' keys and buckets when they fit there
  const size_t smem = (size_t)ctx.cap * 9 + (kf <= ctx.cap ? 0 : (size_t)kf * 4);
  auto launch = [&](auto kern, int nt) {
    allow_large_lds(reinterpret_cast<const void*>(kern), smem > 128 * 1024 ? smem : 128 * 1024);
    hipLaunchKernelGGL(kern, dim3((unsigned)ctx.n), dim3(nt), smem, s, ctx, ws, idx, count, ranked,
                       exact_mode);
  };
  // the bucket kernel, or its scan-run instance
  auto run = [&](auto kern, auto scan_kern, int nt) {
    if (ctx.run_keys || ctx.heads > 1) launch(scan_kern, nt);
    else launch(kern, nt);
  };
#define SELECT_KERNEL(DT_, PER_, NT_) \
  run(k_select_expand<DT_, PER_, NT_>, k_select_expand<DT_, PER_, NT_, true>, NT_)
  if (ctx.cap > 8192) {
    // the longest candidate lists (up to 16 slots per thread of 1,024)
    if ((ctx.cap + 1023) / 1024 > 16) return hipErrorInvalidValue;
    if (dtype == LSA_BF16) SELECT_KERNEL(LSA_BF16, 16, 1024);
    else SELECT_KERNEL(LSA_F32, 16, 1024);
    return hipGetLastError();
  }
  if (ctx.n <= kSelectWideQueries) {
    // candidate slots per thread of a 1,024-thread workgroup: 2, 4 or 8
    const int per = (ctx.cap + 1023) / 1024;
    if (per > 8) return hipErrorInvalidValue;
    if (dtype == LSA_BF16) {
      if (per <= 2) SELECT_KERNEL(LSA_BF16, 2, 1024);
      else if (per <= 4) SELECT_KERNEL(LSA_BF16, 4, 1024);
      else SELECT_KERNEL(LSA_BF16, 8, 1024);
    } else {
      if (per <= 2) SELECT_KERNEL(LSA_F32, 2, 1024);
      else if (per <= 4) SELECT_KERNEL(LSA_F32, 4, 1024);
      else SELECT_KERNEL(LSA_F32, 8, 1024);
    }
    return hipGetLastError();
  }
  // long candidate lists (cap >= 4,096): 512 threads per query (measured
  // faster at k = 4,096; slower at k = 2,048, where 256 threads keep more
  // workgroups per compute unit)
  if (ctx.cap >= 4096) {
    const int per512 = (ctx.cap + 511) / 512;
    if (per512 > 16) return hipErrorInvalidValue;
    if (dtype == LSA_BF16) {
      if (per512 <= 8) SELECT_KERNEL(LSA_BF16, 8, 512);
      else SELECT_KERNEL(LSA_BF16, 16, 512);
    } else {
      if (per512 <= 8) SELECT_KERNEL(LSA_F32, 8, 512);
      else SELECT_KERNEL(LSA_F32, 16, 512);
    }
    return hipGetLastError();
  }
  // candidate slots per thread: cap / 256 rounded up to 8, 16 or 32
  const int per = (ctx.cap + 255) / 256;
  if (per > 32) return hipErrorInvalidValue;
  if (dtype == LSA_BF16) {
    if (per <= 8) SELECT_KERNEL(LSA_BF16, 8, 256);
    else if (per <= 16) SELECT_KERNEL(LSA_BF16, 16, 256);
    else SELECT_KERNEL(LSA_BF16, 32, 256);
  } else {
    if (per <= 8) SELECT_KERNEL(LSA_F32, 8, 256);
    else if (per <= 16) SELECT_KERNEL(LSA_F32, 16, 256);
    else SELECT_KERNEL(LSA_F32, 32, 256);
  }
  return hipGetLastError();
#undef SELECT_KERNEL
}

}  // namespace lsa
