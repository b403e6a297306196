// Internal declarations of the LSA library (device helpers, launchers).
// gfx950 only: 64-wide wavefronts, 160 KiB LDS per CU, bf16 MFMA.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lsa.h"

namespace lsa {

constexpr int kLatent = 64;        // latent dimension
constexpr int kPool = 4;           // keys per pooled key
constexpr int kBlock = 512;        // keys per cluster block
constexpr int kItems = kBlock / kPool;  // pooled keys per block: 128
constexpr int kBuckets = 64;       // buckets per block
constexpr int kCapItems = 4;       // 16 keys = 4 pooled keys
constexpr int kTreeGroup = 128;    // tree: nodes paired inside groups of 128
constexpr int kMaxLevels = 32;
constexpr int kMaxK = 8192;
constexpr int kMaxWindow = 8192;
constexpr int kHeadDim = 128;
constexpr int kMaxSeq = 32;        // sequences per batched decode launch
constexpr int kMaxBeam = 64;        // beam of the one-wave tree search
constexpr int kMaxBeamWide = 512;   // beam of the one-workgroup tree search
constexpr int kMaxCap = 16384;     // candidate slots per query (>= 3 B, see cand_cap)
// dynamic LDS the selection may take (cap * 9 + k * 4 bytes): 160 KiB less its
// static arrays at 1,024 threads
constexpr int kSelectLdsMax = 160 * 1024 - 16640;
constexpr int kSampleStride = 16;  // threshold sample: every 16th tile of 32 buckets

// ---------------------------------------------------------------- numerics

// fp64 -> bfloat16 bits, round to nearest even (8 significant bits).
__host__ __device__ inline uint16_t f64_to_bf16_rne(double x) {
  union { double d; uint64_t u; } v;
  v.d = x;
  const uint64_t sign = v.u & 0x8000000000000000ull;
  const uint64_t mag = v.u & 0x7fffffffffffffffull;
  const int e = (int)(mag >> 52) - 1023;
  if (mag == 0) return (uint16_t)(sign >> 48);
  if (e >= -126) {
    // normal bf16 range: drop 45 of the 52 fraction bits with nearest-even
    const uint64_t lsb = (mag >> 45) & 1ull;
    uint64_t r = mag + 0x0FFFFFFFFFFFull + lsb;
    r &= ~((1ull << 45) - 1ull);
    const int er = (int)(r >> 52) - 1023;
    if (er > 127) return (uint16_t)((sign >> 48) | 0x7f80u);  // overflow -> inf
    const uint32_t frac = (uint32_t)((r >> 45) & 0x7f);
    return (uint16_t)((sign >> 48) | ((uint32_t)(er + 127) << 7) | frac);
  }
  // subnormal bf16: quantum 2^-133
  double q = __builtin_rint(__builtin_ldexp(__builtin_fabs(x), 133));
  uint32_t m = (uint32_t)q;  // <= 128 (128 rounds up to the smallest normal)
  return (uint16_t)((sign >> 48) | m);
}

__host__ __device__ inline float bf16_to_f32(uint16_t b) {
  union { uint32_t u; float f; } v;
  v.u = ((uint32_t)b) << 16;
  return v.f;
}

// fp32 -> bfloat16 bits, nearest even (finite inputs).
__host__ __device__ inline uint16_t f32_to_bf16_rne(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  const uint32_t lsb = (v.u >> 16) & 1u;
  return (uint16_t)((v.u + 0x7fffu + lsb) >> 16);
}

// ---------------------------------------------------------------- cache state

struct CacheLayout {
  int64_t max_blocks;
  int64_t off_staging, off_cent, off_members;
  int64_t lvl_cap[kMaxLevels];
  int64_t off_lvl_cent[kMaxLevels], off_lvl_child[kMaxLevels], off_lvl_minb[kMaxLevels];
  int n_levels;  // highest level with storage
  int64_t total;
};

struct CacheState {
  lsa_params prm;
  int64_t max_tokens;
  int64_t n_tokens;
  int64_t n_blocks;
  char* base;
  int64_t bytes;
  CacheLayout lay;
  int tree;                // 1 if a tree is maintained
  int height;              // current levels above the buckets
  int64_t level_n[kMaxLevels];
};

inline size_t idx_elem_bytes(int dtype) { return dtype == LSA_BF16 ? 2 : 4; }

// ---------------------------------------------------------------- indexer context

// Describes the queries of one indexer launch.  Prefill: one cache, query i
// at position q_start + i.  Decode: query i belongs to sequence i (own cache,
// position pos[i]).
struct IndexCtx {
  int64_t n;
  int64_t q_start;
  int32_t per_seq;
  int32_t k, n_sink, window;
  int32_t top_b;          // buckets kept before expansion
  int32_t cap;            // candidate slots per query
  int32_t list_len;
  int32_t run_keys;       // 0: LSA buckets; b = 1, 4, 8: a scan over runs of b keys
  int32_t heads;          // query heads per position (bucket score = max over them)
  const void* cent[kMaxSeq];
  const uint32_t* members[kMaxSeq];
  int64_t pos[kMaxSeq];
};

struct TreeCtx {
  int height;
  int lstar;
  int beam;
  int start;                          // first-stage level (height: start at the root)
  int64_t nodes[kMaxLevels];          // nodes per level
  const void* cent[kMaxLevels];       // level 0 = buckets
  const int32_t* child[kMaxLevels];   // level >= 1
  const int32_t* minb[kMaxLevels];    // level >= 1
};

struct IndexWs {
  void* yhat;          // [n, 64] index dtype
  float* tau;          // [n]
  int32_t* cand_cnt;   // [n]
  uint2* cand;         // [n, cap] (score bits, bucket)
  int32_t* status;     // [n] 1 if the exact path was used
  uint32_t* hist;      // [n, 256] sampled-score histogram (decode)
};

// Decode bookkeeping launched once per step for all sequences.
constexpr int kMaxDecode = 64;        // sequences per lsa_index_decode call
struct WardJobs {
  const float* keys[kMaxDecode];      // 512 staged keys of the completed block
  int64_t block[kMaxDecode];
  void* cent[kMaxDecode];
  uint32_t* members[kMaxDecode];
};
struct AppendJobs {
  float* dst[kMaxDecode];             // staging row of each sequence's new key
};

// ---------------------------------------------------------------- launchers
// All launchers enqueue on `s` and return hipSuccess or the launch error.

hipError_t launch_ward_blocks(const float* keys, int64_t first_block, int64_t n_blocks,
                              void* cent, uint32_t* members, int dtype, hipStream_t s);
hipError_t launch_tree_groups(const void* child_cent, const int32_t* child_minb,
                              int64_t n_child, int64_t g0, int64_t g1, void* cent,
                              int32_t* child, int32_t* minb, int dtype, int child_is_bucket,
                              hipStream_t s);
hipError_t launch_copy_rows(float* dst, const float* src, int64_t n, hipStream_t s);
hipError_t launch_scan_blocks(const float* keys, int64_t first_block, int64_t n_blocks, void* cent,
                              int run_keys, int dtype, hipStream_t s);
hipError_t launch_ward_jobs(const WardJobs& jobs, int n, int dtype, hipStream_t s);

hipError_t launch_qnorm(const float* y, int64_t n, void* yhat, int dtype, uint32_t* hist,
                        hipStream_t s);
hipError_t launch_dec_prep(const float* y, const float* k_new, const AppendJobs& jobs, int64_t n,
                           void* yhat, const IndexWs& ws, int dtype, hipStream_t s);
hipError_t launch_thresh(const IndexCtx& ctx, const IndexWs& ws, int dtype, hipStream_t s);
hipError_t launch_score_filter(const IndexCtx& ctx, const IndexWs& ws, int dtype,
                               int64_t max_tiles, hipStream_t s);
hipError_t launch_tree_search(const IndexCtx& ctx, const TreeCtx& tc, const IndexWs& ws,
                              int dtype, hipStream_t s);
hipError_t launch_select_expand(const IndexCtx& ctx, const IndexWs& ws, int32_t* idx,
                                int32_t* count, int32_t* ranked, int dtype, int exact_mode,
                                hipStream_t s);

// rows per bf16 attention launch (a call over more rows issues several)
int64_t attention_launch_rows();
hipError_t launch_dense_attention(const void* q, const void* k, const void* v, int64_t rows,
                                  int64_t q_start, int64_t Tk, int32_t Hq, int32_t Hkv,
                                  int64_t band, float scale, void* out, hipStream_t s);
bool attention_head_major(int32_t B, int64_t Tmax, int32_t Hkv, int32_t D, int dtype);
hipError_t launch_attention(const void* q, const void* k, const void* v, int32_t B, int64_t Tq,
                            int64_t Tmax, int32_t Hq, int32_t Hkv, const int32_t* idx,
                            const int32_t* count, int32_t L_max, float scale, int dtype,
                            int32_t splits, void* out, float* ws, hipStream_t s);
// the softmax state of each row's near set (sinks and window), written into
// po [nrows, Hq, 128], pm and pl [nrows, Hq] for rows row0 .. row0 + nrows - 1
hipError_t launch_near_attention(const void* q, const void* k, const void* v, int64_t row0,
                                 int64_t nrows, int64_t Tq, int64_t q_start, int64_t Tmax,
                                 int32_t Hq, int32_t Hkv, int64_t n_sink, int64_t window,
                                 float scale, float* po, float* pm, float* pl, hipStream_t s);
// bytes of near state that launch_attention_prefill needs for `rows` rows
int64_t near_state_bytes(int64_t rows, int32_t Hq);
// prefill attention in two parts: near set dense per tile of rows, then the
// far entries of each list gathered on top of that state
hipError_t launch_attention_prefill(const void* q, const void* k, const void* v, int32_t B,
                                    int64_t Tq, int64_t q_start, int64_t Tmax, int32_t Hq,
                                    int32_t Hkv, const int32_t* idx, const int32_t* count,
                                    int32_t L_max, int64_t n_sink, int64_t window, float scale,
                                    void* out, float* ws, hipStream_t s);

}  // namespace lsa
