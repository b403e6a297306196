// Host side of the C ABI declared in include/lsa.h: argument validation,
// cache layout inside caller memory, and kernel orchestration on the
// caller's stream.  Nothing here allocates device memory or synchronises.
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>

#include "lsa_internal.h"

using namespace lsa;

struct lsa_cache {
  CacheState st;
};

// Split partials of lsa_sparse_attention_static, for callers that cannot
// allocate device memory: a fixed array that every GPU the library runs on
// holds (its own copy, at its own address) until the process ends.  Host
// code never passes this name to a kernel; it uses the address that
// hipGetSymbolAddress returns on each device (static_scratch below).
static __device__ __align__(256) char scratch[LSA_STATIC_SCRATCH_BYTES];

namespace {

constexpr int64_t kAlign = 256;

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
hipError_t static_scratch(float** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = reinterpret_cast<float*>(addr[dev]);
  return hipSuccess;
}

int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int pow2_ceil(int64_t x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// structural parameters the kernels are written for
int check_structure(const lsa_params* p) {
  if (p->d_latent != kLatent || p->n_pool != kPool || p->block_keys != kBlock ||
      p->n_buckets != kBuckets || p->bucket_cap_keys != kCapItems * kPool)
    return LSA_ERR_UNSUPPORTED;
  if (p->index_dtype != LSA_F32 && p->index_dtype != LSA_BF16) return LSA_ERR_UNSUPPORTED;
  if (p->mode != LSA_FLAT && p->mode != LSA_TREE) return LSA_ERR_UNSUPPORTED;
  if (p->scan_keys != 0 && p->scan_keys != 1 && p->scan_keys != 4 && p->scan_keys != 8)
    return LSA_ERR_UNSUPPORTED;
  if (p->scan_keys && p->mode != LSA_FLAT) return LSA_ERR_UNSUPPORTED;
  if (p->score_heads < 0 || p->score_heads > 8 || (p->score_heads & (p->score_heads - 1)))
    return LSA_ERR_UNSUPPORTED;
  // several query heads: flat bf16 prefill over LSA buckets
  if (p->score_heads > 1 &&
      (p->mode != LSA_FLAT || p->scan_keys || p->index_dtype != LSA_BF16))
    return LSA_ERR_UNSUPPORTED;
  return LSA_OK;
}

int check_query(const lsa_params* p) {
  if (p->k < 0 || p->k > kMaxK) return LSA_ERR_UNSUPPORTED;
  if (p->n_sink < 0 || p->n_sink > kMaxWindow) return LSA_ERR_UNSUPPORTED;
  if (p->window < 1 || p->window > kMaxWindow) return LSA_ERR_UNSUPPORTED;
  if (p->beam < 1 || p->beam > kMaxBeamWide) return LSA_ERR_UNSUPPORTED;
  if (p->start_level < -1 || p->start_level >= kMaxLevels) return LSA_ERR_UNSUPPORTED;
  if (p->leaf_level < -1 || p->leaf_level >= kMaxLevels) return LSA_ERR_UNSUPPORTED;
  if (p->exact_select != 0 && p->exact_select != 1) return LSA_ERR_UNSUPPORTED;
  // a scan's runs are summarised block by block, so every run it scores must
  // lie in a complete block: the window has to cover the query's own block
  if (p->scan_keys && p->window < kBlock) return LSA_ERR_UNSUPPORTED;
  return LSA_OK;
}

// Buckets kept per query before expansion.  A bucket without a sink or
// window key gives at least kPool far keys; on top of ceil(k / kPool) such
// buckets come every bucket that can hold a sink or window key: all buckets
// of each eligible block the window reaches back into, and one per pooled
// item of the sinks.  (Default window 512 and 4 sinks: ceil(k / 4) + 65.)
int32_t top_b(const lsa_params* p) {
  if (p->scan_keys) {
    // a scan's eligible runs end before the window; only runs holding a
    // sink give fewer than scan_keys far keys
    return (p->k + p->scan_keys - 1) / p->scan_keys + (p->n_sink + p->scan_keys - 1) / p->scan_keys;
  }
  const int32_t win_blocks = (p->window - 1 + kBlock - 1) / kBlock;
  return (p->k + kPool - 1) / kPool + kBuckets * win_blocks + (p->n_sink + kPool - 1) / kPool;
}

// candidate slots per query: >= 3 B (tau aims at ~5/4 B): a power of two up to
// 8,192, beyond that a multiple of 1,024
int32_t cand_cap(const lsa_params* p) {
  const int64_t want = 3 * (int64_t)top_b(p);
  if (want > 8192) return (int32_t)((want + 1023) / 1024 * 1024);
  int c = pow2_ceil(want);
  return c < 256 ? 256 : c;
}

int leaf_level(const lsa_params* p) {
  if (p->leaf_level >= 0) return p->leaf_level;
  int l = 0;
  while ((int64_t)p->beam << l < top_b(p)) ++l;
  return l;
}

// rows of the centroid table per full block: 64 buckets, or a scan's runs
int64_t rows_per_block(const lsa_params* p) {
  return p->scan_keys ? kBlock / p->scan_keys : kBuckets;
}

CacheLayout make_layout(int64_t max_blocks, int dtype, int tree, int64_t per_block) {
  CacheLayout L;
  memset(&L, 0, sizeof(L));
  L.max_blocks = max_blocks;
  const int64_t esz = (int64_t)idx_elem_bytes(dtype);
  const int64_t nb = max_blocks * per_block;
  int64_t off = 0;
  L.off_staging = off;
  off = align_up(off + (int64_t)kBlock * kLatent * 4);
  L.off_cent = off;
  off = align_up(off + nb * kLatent * esz);
  L.off_members = off;
  if (per_block == kBuckets) off = align_up(off + nb * 4);   // scans keep no member table
  L.lvl_cap[0] = nb;
  L.n_levels = 0;
  if (tree && nb > 1) {
    int64_t n = nb;
    int l = 0;
    while (n > 1 && l + 1 < kMaxLevels) {
      n = (n + 1) / 2;
      ++l;
      L.lvl_cap[l] = n;
      L.off_lvl_cent[l] = off;
      off = align_up(off + n * kLatent * esz);
      L.off_lvl_child[l] = off;
      off = align_up(off + n * 8);
      L.off_lvl_minb[l] = off;
      off = align_up(off + n * 4);
    }
    L.n_levels = l;
  }
  L.total = off;
  return L;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int hip_status(hipError_t e) { return e == hipSuccess ? LSA_OK : LSA_ERR_HIP; }

void* lvl_cent(const CacheState& c, int l) {
  return l == 0 ? (void*)(c.base + c.lay.off_cent) : (void*)(c.base + c.lay.off_lvl_cent[l]);
}
int32_t* lvl_child(const CacheState& c, int l) {
  return reinterpret_cast<int32_t*>(c.base + c.lay.off_lvl_child[l]);
}
int32_t* lvl_minb(const CacheState& c, int l) {
  return reinterpret_cast<int32_t*>(c.base + c.lay.off_lvl_minb[l]);
}

// Rebuild the tree levels above buckets [64 * old_blocks, 64 * n_blocks).
int update_tree(CacheState& c, int64_t old_blocks, hipStream_t s) {
  int64_t n_child = c.n_blocks * kBuckets;
  int64_t changed = old_blocks * kBuckets;
  int l = 1;
  while (n_child > 1) {
    if (l > c.lay.n_levels) return LSA_ERR_CAPACITY;
    const int64_t g0 = changed / kTreeGroup;
    const int64_t g1 = (n_child + kTreeGroup - 1) / kTreeGroup;
    hipError_t e = launch_tree_groups(lvl_cent(c, l - 1), l == 1 ? nullptr : lvl_minb(c, l - 1),
                                      n_child, g0, g1, lvl_cent(c, l), lvl_child(c, l),
                                      lvl_minb(c, l), c.prm.index_dtype, l == 1, s);
    if (e != hipSuccess) return LSA_ERR_HIP;
    changed = g0 * (kTreeGroup / 2);
    n_child = (n_child + 1) / 2;
    c.level_n[l] = n_child;
    ++l;
  }
  c.height = l - 1;
  return LSA_OK;
}

// Append n keys (device fp32 rows) and cluster every block that fills up.
int append_keys(CacheState& c, const float* keys, int64_t n, hipStream_t s) {
  const int64_t old_blocks = c.n_blocks;
  const int64_t r = c.n_tokens % kBlock;
  int64_t used = 0;
  hipError_t e;
  if (r > 0) {
    const int64_t take = (kBlock - r) < n ? (kBlock - r) : n;
    float* stg = reinterpret_cast<float*>(c.base + c.lay.off_staging);
    e = launch_copy_rows(stg + r * kLatent, keys, take, s);
    if (e != hipSuccess) return LSA_ERR_HIP;
    used = take;
    if (r + take == kBlock) {
      e = c.prm.scan_keys
              ? launch_scan_blocks(stg, c.n_blocks, 1, c.base + c.lay.off_cent, c.prm.scan_keys,
                                   c.prm.index_dtype, s)
              : launch_ward_blocks(stg, c.n_blocks, 1, c.base + c.lay.off_cent,
                                   reinterpret_cast<uint32_t*>(c.base + c.lay.off_members),
                                   c.prm.index_dtype, s);
      if (e != hipSuccess) return LSA_ERR_HIP;
      c.n_blocks += 1;
    }
  }
  const int64_t full = (n - used) / kBlock;
  if (full > 0) {
    e = c.prm.scan_keys
            ? launch_scan_blocks(keys + used * kLatent, c.n_blocks, full, c.base + c.lay.off_cent,
                                 c.prm.scan_keys, c.prm.index_dtype, s)
            : launch_ward_blocks(keys + used * kLatent, c.n_blocks, full, c.base + c.lay.off_cent,
                                 reinterpret_cast<uint32_t*>(c.base + c.lay.off_members),
                                 c.prm.index_dtype, s);
    if (e != hipSuccess) return LSA_ERR_HIP;
    c.n_blocks += full;
    used += full * kBlock;
  }
  const int64_t rem = n - used;
  if (rem > 0) {
    float* stg = reinterpret_cast<float*>(c.base + c.lay.off_staging);
    e = launch_copy_rows(stg, keys + used * kLatent, rem, s);
    if (e != hipSuccess) return LSA_ERR_HIP;
  }
  c.n_tokens += n;
  if (c.tree && c.n_blocks > old_blocks) return update_tree(c, old_blocks, s);
  return LSA_OK;
}

struct WsLayout {
  int64_t off_yhat, off_tau, off_cnt, off_status, off_hist, off_cand, total;
};

int heads(const lsa_params* p) { return p->score_heads > 1 ? p->score_heads : 1; }

WsLayout index_ws_layout(const lsa_params* p, int64_t nq) {
  WsLayout w;
  int64_t off = 0;
  w.off_yhat = off;
  off = align_up(off + nq * heads(p) * kLatent * (int64_t)idx_elem_bytes(p->index_dtype));
  w.off_tau = off;
  off = align_up(off + nq * 4);
  w.off_cnt = off;
  off = align_up(off + nq * 4);
  w.off_status = off;
  off = align_up(off + nq * 4);
  w.off_hist = off;
  off = align_up(off + nq * 256 * 4);
  w.off_cand = off;
  off = align_up(off + nq * (int64_t)cand_cap(p) * 8);
  w.total = off;
  return w;
}

IndexWs make_ws(void* base, const WsLayout& w) {
  char* b = reinterpret_cast<char*>(base);
  IndexWs ws;
  ws.yhat = b + w.off_yhat;
  ws.tau = reinterpret_cast<float*>(b + w.off_tau);
  ws.cand_cnt = reinterpret_cast<int32_t*>(b + w.off_cnt);
  ws.status = reinterpret_cast<int32_t*>(b + w.off_status);
  ws.cand = reinterpret_cast<uint2*>(b + w.off_cand);
  ws.hist = reinterpret_cast<uint32_t*>(b + w.off_hist);
  return ws;
}

IndexCtx base_ctx(const lsa_params* p, int64_t n) {
  IndexCtx ctx;
  memset(&ctx, 0, sizeof(ctx));
  ctx.n = n;
  ctx.k = p->k;
  ctx.n_sink = p->n_sink;
  ctx.window = p->window;
  ctx.top_b = top_b(p);
  ctx.cap = cand_cap(p);
  ctx.list_len = p->n_sink + p->window + p->k;
  ctx.run_keys = p->scan_keys;
  ctx.heads = heads(p);
  return ctx;
}

TreeCtx make_tree_ctx(const CacheState& c, const lsa_params* p) {
  TreeCtx tc;
  memset(&tc, 0, sizeof(tc));
  tc.height = c.height;
  tc.lstar = leaf_level(p);
  tc.beam = p->beam;
  // the first stage's level: the root (height), or s clamped to [l*, height]
  tc.start = c.height;
  if (p->start_level >= 0 && p->start_level < c.height)
    tc.start = p->start_level > tc.lstar ? p->start_level : tc.lstar;
  tc.nodes[0] = c.n_blocks * kBuckets;
  for (int l = 1; l <= c.height; ++l) tc.nodes[l] = c.level_n[l];
  tc.cent[0] = lvl_cent(c, 0);
  for (int l = 1; l <= c.height; ++l) {
    tc.cent[l] = lvl_cent(c, l);
    tc.child[l] = lvl_child(c, l);
    tc.minb[l] = lvl_minb(c, l);
  }
  return tc;
}

// Select + expand for the queries described by ctx (yhat already written).
// `tree` != null: beam search candidates; else flat (sampled threshold + filter).
int run_selection(const IndexCtx& ctx, const IndexWs& ws, const lsa_params* p,
                  const TreeCtx* tree, int64_t max_elig, int32_t* idx, int32_t* count,
                  int32_t* ranked, hipStream_t s) {
  const int dt = p->index_dtype;
  hipError_t e;
  // exact selection mode of the expansion kernel: 0 = tree candidates as they
  // are, 1 = redo a query whose flat candidate list is unusable, 2 = always
  int exact_mode = 0;
  if (tree) {
    e = launch_tree_search(ctx, *tree, ws, dt, s);
    if (e != hipSuccess) return LSA_ERR_HIP;
  } else {
    e = launch_thresh(ctx, ws, dt, s);
    if (e != hipSuccess) return LSA_ERR_HIP;
    if (!p->exact_select) {
      e = launch_score_filter(ctx, ws, dt, (max_elig + 31) / 32, s);
      if (e != hipSuccess) return LSA_ERR_HIP;
    }
    exact_mode = p->exact_select ? 2 : 1;
  }
  e = launch_select_expand(ctx, ws, idx, count, ranked, dt, exact_mode, s);
  return hip_status(e);
}


// Argument checks shared by both attention entry points (no launch); *need
// receives the split-partials bytes.  1 = nothing to do.
int check_attention(const void* q, const void* k_cache, const void* v_cache, int32_t B,
                    int64_t Tq, int64_t Tmax, int32_t Hq, int32_t Hkv, int32_t D,
                    const int32_t* idx, const int32_t* count, int32_t L_max, int32_t dtype,
                    int32_t splits, const void* out, int64_t* need) {
  if (B < 0 || Tq < 0 || Tmax < 0 || L_max < 0 || splits < 1) return LSA_ERR_ARG;
  if (D != kHeadDim || Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0 || Hq / Hkv > 16)
    return LSA_ERR_UNSUPPORTED;
  if (dtype != LSA_F32 && dtype != LSA_BF16) return LSA_ERR_UNSUPPORTED;
  if ((int64_t)B * Tq == 0) return 1;
  if (!q || !k_cache || !v_cache || !idx || !count || !out) return LSA_ERR_ARG;
  if (Tmax < 1) return LSA_ERR_ARG;   // invalid list entries read token 0 (with zero weight)
  if ((int64_t)B * Tq > (int64_t)0x7fffffff || splits > 65535) return LSA_ERR_UNSUPPORTED;
  if (splits > 1 && (int64_t)B * Tq * Hq * 2 > (int64_t)0x7fffffff) return LSA_ERR_UNSUPPORTED;
  *need = lsa_attention_workspace_bytes(B, Tq, Hq, D, splits);
  return LSA_OK;
}

}  // namespace

// ====================================================================== API

extern "C" {

int32_t lsa_params_bytes(void) { return (int32_t)sizeof(lsa_params); }

void lsa_default_params(lsa_params* p) {
  if (!p) return;
  p->d_latent = kLatent;
  p->n_pool = kPool;
  p->block_keys = kBlock;
  p->n_buckets = kBuckets;
  p->bucket_cap_keys = kCapItems * kPool;
  p->k = 2048;
  p->n_sink = 4;
  p->window = 512;
  p->mode = LSA_FLAT;
  p->beam = 64;
  p->leaf_level = -1;
  p->index_dtype = LSA_BF16;
  p->exact_select = 0;
  p->scan_keys = 0;
  p->score_heads = 0;
  p->start_level = -1;
}

const char* lsa_status_string(int status) {
  switch (status) {
    case LSA_OK: return "ok";
    case LSA_ERR_ARG: return "invalid argument";
    case LSA_ERR_UNSUPPORTED: return "unsupported parameter or shape";
    case LSA_ERR_WORKSPACE: return "workspace too small";
    case LSA_ERR_CAPACITY: return "cache capacity exceeded";
    case LSA_ERR_HIP: return "HIP launch or runtime error";
    case LSA_ERR_STATE: return "cache state does not allow this call";
    default: return "unknown status";
  }
}

int lsa_check_params(const lsa_params* p) {
  if (!p) return LSA_ERR_ARG;
  int rc = check_structure(p);
  if (rc) return rc;
  rc = check_query(p);
  if (rc) return rc;
  // the selection holds every candidate of a query in one workgroup's LDS
  if (cand_cap(p) > kMaxCap) return LSA_ERR_UNSUPPORTED;
  if ((int64_t)cand_cap(p) * 9 + 4 * (int64_t)(p->k > 1 ? p->k : 1) > kSelectLdsMax)
    return LSA_ERR_UNSUPPORTED;
  if (p->mode == LSA_TREE && ((int64_t)p->beam << leaf_level(p)) > cand_cap(p))
    return LSA_ERR_UNSUPPORTED;
  return LSA_OK;
}

int32_t lsa_list_len(const lsa_params* p) {
  int rc = lsa_check_params(p);
  if (rc) return rc;
  return p->n_sink + p->window + p->k;
}

int32_t lsa_top_buckets(const lsa_params* p) {
  int rc = lsa_check_params(p);
  if (rc) return rc;
  return top_b(p);
}

int64_t lsa_cache_bytes(const lsa_params* p, int64_t max_tokens) {
  int rc = lsa_check_params(p);
  if (rc) return rc;
  if (max_tokens < 0 || max_tokens > (int64_t)0x7fffffff) return LSA_ERR_ARG;
  return make_layout(max_tokens / kBlock, p->index_dtype, p->mode == LSA_TREE,
                     rows_per_block(p)).total;
}

int lsa_cache_init(const lsa_params* p, int64_t max_tokens, void* cache_mem, int64_t bytes,
                   lsa_cache** out) {
  if (!p || !out || !cache_mem) return LSA_ERR_ARG;
  int rc = lsa_check_params(p);
  if (rc) return rc;
  if (max_tokens < 0 || max_tokens > (int64_t)0x7fffffff) return LSA_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(cache_mem) % kAlign) return LSA_ERR_ARG;
  CacheLayout lay = make_layout(max_tokens / kBlock, p->index_dtype, p->mode == LSA_TREE,
                                rows_per_block(p));
  if (bytes < lay.total) return LSA_ERR_CAPACITY;
  lsa_cache* c = new (std::nothrow) lsa_cache;
  if (!c) return LSA_ERR_ARG;
  memset(&c->st, 0, sizeof(c->st));
  c->st.prm = *p;
  c->st.max_tokens = max_tokens;
  c->st.base = reinterpret_cast<char*>(cache_mem);
  c->st.bytes = bytes;
  c->st.lay = lay;
  c->st.tree = p->mode == LSA_TREE;
  *out = c;
  return LSA_OK;
}

int lsa_cache_release(lsa_cache* c) {
  if (!c) return LSA_ERR_ARG;
  delete c;
  return LSA_OK;
}

int64_t lsa_cache_tokens(const lsa_cache* c) {
  if (!c) return LSA_ERR_ARG;
  return c->st.n_tokens;
}

int lsa_cache_get_view(const lsa_cache* c, lsa_cache_view* out) {
  if (!c || !out) return LSA_ERR_ARG;
  memset(out, 0, sizeof(*out));
  const CacheState& s = c->st;
  out->n_tokens = s.n_tokens;
  out->n_blocks = s.n_blocks;
  out->n_buckets = s.n_blocks * rows_per_block(&s.prm);
  out->centroids = s.base + s.lay.off_cent;
  out->members = s.prm.scan_keys ? nullptr : reinterpret_cast<uint32_t*>(s.base + s.lay.off_members);
  out->staging = reinterpret_cast<float*>(s.base + s.lay.off_staging);
  out->tree_height = s.tree ? s.height : 0;
  out->level_nodes[0] = s.n_blocks * rows_per_block(&s.prm);
  if (s.tree) {
    for (int l = 1; l <= s.height; ++l) {
      out->level_nodes[l] = s.level_n[l];
      out->level_centroids[l] = lvl_cent(s, l);
      out->level_child[l] = lvl_child(s, l);
      out->level_min_block[l] = lvl_minb(s, l);
    }
  }
  return LSA_OK;
}

int build_bucket_cache(lsa_cache* c, const float* latent_keys, int64_t n_new, void* stream) {
  if (!c || n_new < 0) return LSA_ERR_ARG;
  if (n_new == 0) return LSA_OK;
  if (!latent_keys) return LSA_ERR_ARG;
  if (c->st.n_tokens + n_new > c->st.max_tokens) return LSA_ERR_CAPACITY;
  return append_keys(c->st, latent_keys, n_new, as_stream(stream));
}

int64_t lsa_index_workspace_bytes(const lsa_params* p, int64_t max_queries) {
  int rc = lsa_check_params(p);
  if (rc) return rc;
  if (max_queries < 0) return LSA_ERR_ARG;
  return index_ws_layout(p, max_queries).total;
}

int64_t lsa_index_status_offset(const lsa_params* p, int64_t n_queries) {
  int rc = lsa_check_params(p);
  if (rc) return rc;
  if (n_queries < 0) return LSA_ERR_ARG;
  return index_ws_layout(p, n_queries).off_status;
}

int lsa_index_prefill(const lsa_cache* c, const float* latent_q, int64_t q_start, int64_t Tq,
                      const lsa_params* p, int32_t* idx, int32_t* count, int32_t* ranked,
                      void* workspace, int64_t ws_bytes, void* stream) {
  if (!c || !p || q_start < 0 || Tq < 0) return LSA_ERR_ARG;
  int rc = lsa_check_params(p);
  if (rc) return rc;
  const CacheState& st = c->st;
  if (p->index_dtype != st.prm.index_dtype || p->scan_keys != st.prm.scan_keys) return LSA_ERR_ARG;
  if (Tq == 0) return LSA_OK;
  if (!latent_q || !idx || !count || !workspace) return LSA_ERR_ARG;
  if (q_start + Tq > (int64_t)0x7fffffff) return LSA_ERR_ARG;
  const int64_t last = q_start + Tq - 1;
  if (last / kBlock > st.n_blocks) return LSA_ERR_STATE;
  const bool tree = p->mode == LSA_TREE;
  if (tree && !st.tree) return LSA_ERR_STATE;
  const WsLayout wl = index_ws_layout(p, Tq);
  if (ws_bytes < wl.total) return LSA_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  IndexWs ws = make_ws(workspace, wl);
  IndexCtx ctx = base_ctx(p, Tq);
  ctx.q_start = q_start;
  ctx.per_seq = 0;
  ctx.cent[0] = lvl_cent(st, 0);
  ctx.members[0] = reinterpret_cast<const uint32_t*>(st.base + st.lay.off_members);
  hipError_t e = launch_qnorm(latent_q, Tq * heads(p), ws.yhat, p->index_dtype, nullptr, s);
  if (e != hipSuccess) return LSA_ERR_HIP;
  int64_t max_elig = (last / kBlock) * kBuckets;
  if (p->scan_keys) max_elig = (last - p->window + 1 > 0 ? last - p->window + 1 : 0) / p->scan_keys;
  TreeCtx tc;
  const TreeCtx* tp = nullptr;
  if (tree && st.height > 0 && leaf_level(p) < st.height) {
    tc = make_tree_ctx(st, p);
    tp = &tc;
  }
  return run_selection(ctx, ws, p, tp, max_elig, idx, count, ranked, s);
}

int lsa_index_decode(lsa_cache* const* caches, int32_t B, const float* latent_q,
                     const float* latent_k_new, const lsa_params* p, int32_t* idx,
                     int32_t* count, void* workspace, int64_t ws_bytes, void* stream) {
  if (!caches || !p || B < 0 || B > kMaxDecode) return LSA_ERR_ARG;
  int rc = lsa_check_params(p);
  if (rc) return rc;
  if (p->scan_keys || p->score_heads > 1) return LSA_ERR_UNSUPPORTED;   // prefill variants
  if (B == 0) return LSA_OK;
  if (!latent_q || !latent_k_new || !idx || !count || !workspace) return LSA_ERR_ARG;
  const bool tree = p->mode == LSA_TREE;
  for (int b = 0; b < B; ++b) {
    if (!caches[b]) return LSA_ERR_ARG;
    const CacheState& st = caches[b]->st;
    if (st.prm.index_dtype != p->index_dtype) return LSA_ERR_ARG;
    if (st.n_tokens + 1 > st.max_tokens) return LSA_ERR_CAPACITY;
    if (tree && !st.tree) return LSA_ERR_STATE;
    for (int b2 = 0; b2 < b; ++b2)
      if (caches[b2] == caches[b]) return LSA_ERR_ARG;
  }
  const WsLayout wl = index_ws_layout(p, B);
  if (ws_bytes < wl.total) return LSA_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  // append the new key of every sequence and prepare the step (one launch),
  // then cluster every block that this key completed (one launch), then
  // update trees
  {
    AppendJobs aj;
    WardJobs wj;
    memset(&aj, 0, sizeof(aj));
    memset(&wj, 0, sizeof(wj));
    int nfire = 0;
    for (int b = 0; b < B; ++b) {
      CacheState& st = caches[b]->st;
      float* stg = reinterpret_cast<float*>(st.base + st.lay.off_staging);
      aj.dst[b] = stg + (st.n_tokens % kBlock) * kLatent;
      if ((st.n_tokens + 1) % kBlock == 0) {
        wj.keys[nfire] = stg;
        wj.block[nfire] = st.n_blocks;
        wj.cent[nfire] = st.base + st.lay.off_cent;
        wj.members[nfire] = reinterpret_cast<uint32_t*>(st.base + st.lay.off_members);
        ++nfire;
      }
    }
    // one launch: append the new keys, normalise the queries, clear the
    // per-step histograms and counts
    hipError_t e = launch_dec_prep(latent_q, latent_k_new, aj, B, make_ws(workspace, wl).yhat,
                                   make_ws(workspace, wl), p->index_dtype, s);
    if (e != hipSuccess) return LSA_ERR_HIP;
    e = launch_ward_jobs(wj, nfire, p->index_dtype, s);
    if (e != hipSuccess) return LSA_ERR_HIP;
    for (int b = 0; b < B; ++b) {
      CacheState& st = caches[b]->st;
      const int64_t old_blocks = st.n_blocks;
      st.n_tokens += 1;
      if (st.n_tokens % kBlock == 0) {
        st.n_blocks += 1;
        if (st.tree) {
          rc = update_tree(st, old_blocks, s);
          if (rc) return rc;
        }
      }
    }
  }
  IndexWs ws = make_ws(workspace, wl);
  const int L = p->n_sink + p->window + p->k;
  if (tree) {
    // tree search is per cache: one launch per sequence
    for (int b = 0; b < B; ++b) {
      const CacheState& st = caches[b]->st;
      IndexCtx ctx = base_ctx(p, 1);
      ctx.per_seq = 1;
      ctx.pos[0] = st.n_tokens - 1;
      ctx.cent[0] = lvl_cent(st, 0);
      ctx.members[0] = reinterpret_cast<const uint32_t*>(st.base + st.lay.off_members);
      IndexWs wsb = ws;
      wsb.yhat = reinterpret_cast<char*>(ws.yhat) + (int64_t)b * kLatent * idx_elem_bytes(p->index_dtype);
      wsb.tau += b; wsb.cand_cnt += b; wsb.status += b;
      wsb.hist += (int64_t)b * 256;
      wsb.cand += (int64_t)b * ctx.cap;
      const int64_t max_elig = (ctx.pos[0] / kBlock) * kBuckets;
      TreeCtx tc;
      const TreeCtx* tp = nullptr;
      if (st.height > 0 && leaf_level(p) < st.height) {
        tc = make_tree_ctx(st, p);
        tp = &tc;
      }
      rc = run_selection(ctx, wsb, p, tp, max_elig, idx + (int64_t)b * L, count + b, nullptr, s);
      if (rc) return rc;
    }
    return LSA_OK;
  }
  for (int b0 = 0; b0 < B; b0 += kMaxSeq) {
    const int nb = (B - b0) < kMaxSeq ? (B - b0) : kMaxSeq;
    IndexCtx ctx = base_ctx(p, nb);
    ctx.per_seq = 1;
    int64_t max_elig = 0;
    for (int i = 0; i < nb; ++i) {
      const CacheState& st = caches[b0 + i]->st;
      ctx.pos[i] = st.n_tokens - 1;
      ctx.cent[i] = lvl_cent(st, 0);
      ctx.members[i] = reinterpret_cast<const uint32_t*>(st.base + st.lay.off_members);
      const int64_t ne = (ctx.pos[i] / kBlock) * kBuckets;
      max_elig = ne > max_elig ? ne : max_elig;
    }
    IndexWs wsb = ws;
    wsb.yhat = reinterpret_cast<char*>(ws.yhat) + (int64_t)b0 * kLatent * idx_elem_bytes(p->index_dtype);
    wsb.tau += b0; wsb.cand_cnt += b0; wsb.status += b0;
    wsb.hist += (int64_t)b0 * 256;
    wsb.cand += (int64_t)b0 * ctx.cap;
    rc = run_selection(ctx, wsb, p, nullptr, max_elig, idx + (int64_t)b0 * L, count + b0, nullptr, s);
    if (rc) return rc;
  }
  return LSA_OK;
}

int64_t lsa_attention_workspace_bytes(int32_t B, int64_t Tq, int32_t Hq, int32_t D,
                                      int32_t splits) {
  if (B < 0 || Tq < 0 || Hq <= 0 || D != kHeadDim || splits < 1) return LSA_ERR_ARG;
  if (splits == 1) return 0;
  const int64_t rows = (int64_t)B * Tq;
  return rows * splits * Hq * ((int64_t)kHeadDim + 2) * 4;
}

int64_t lsa_attention_launch_rows(void) { return attention_launch_rows(); }

int32_t lsa_attention_head_major(int32_t B, int64_t Tmax, int32_t Hkv, int32_t D, int32_t dtype) {
  return attention_head_major(B, Tmax, Hkv, D, dtype) ? 1 : 0;
}

int32_t lsa_attention_default_splits(int64_t rows, int32_t L_max) {
  if (rows <= 0 || L_max <= 0) return 1;
  int32_t splits = 1;
  while (splits < 256 && rows * splits < 256 && L_max / (2 * splits) >= 32) splits *= 2;
  return splits;
}

int lsa_sparse_attention(const void* q, const void* k_cache, const void* v_cache, int32_t B,
                         int64_t Tq, int64_t Tmax, int32_t Hq, int32_t Hkv, int32_t D,
                         const int32_t* idx, const int32_t* count, int32_t L_max, float scale,
                         int32_t dtype, int32_t splits, void* out, void* workspace,
                         int64_t ws_bytes, void* stream) {
  int64_t need = 0;
  const int rc = check_attention(q, k_cache, v_cache, B, Tq, Tmax, Hq, Hkv, D, idx, count, L_max,
                                 dtype, splits, out, &need);
  if (rc) return rc < 0 ? rc : LSA_OK;
  if (need > 0 && (!workspace || ws_bytes < need)) return LSA_ERR_WORKSPACE;
  hipError_t e = launch_attention(q, k_cache, v_cache, B, Tq, Tmax, Hq, Hkv, idx, count, L_max,
                                  scale, dtype, splits, out, reinterpret_cast<float*>(workspace),
                                  as_stream(stream));
  return hip_status(e);
}

int64_t lsa_prefill_attention_workspace_bytes(int32_t B, int64_t Tq, int32_t Hq, int32_t D) {
  if (B < 0 || Tq < 0 || Hq <= 0 || D != kHeadDim) return LSA_ERR_ARG;
  return near_state_bytes((int64_t)B * Tq, Hq);
}

int lsa_sparse_attention_prefill(const void* q, const void* k_cache, const void* v_cache,
                                 int32_t B, int64_t Tq, int64_t q_start, int64_t Tmax,
                                 int32_t Hq, int32_t Hkv, int32_t D, const int32_t* idx,
                                 const int32_t* count, int32_t L_max, int32_t n_sink,
                                 int32_t window, float scale, int32_t dtype, void* out,
                                 void* workspace, int64_t ws_bytes, void* stream) {
  int64_t need = 0;
  const int rc = check_attention(q, k_cache, v_cache, B, Tq, Tmax, Hq, Hkv, D, idx, count, L_max,
                                 dtype, 1, out, &need);
  if (rc < 0) return rc;
  if (dtype != LSA_BF16) return LSA_ERR_UNSUPPORTED;
  const int32_t G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return LSA_ERR_UNSUPPORTED;
  if (q_start < 0 || n_sink < 0 || window < 1) return LSA_ERR_ARG;
  if (rc) return LSA_OK;                       // no rows
  if (q_start + Tq > Tmax) return LSA_ERR_ARG;
  if (Hkv > 65535 || Tmax > 0x7fffffff) return LSA_ERR_UNSUPPORTED;   // 32-bit positions
  need = near_state_bytes((int64_t)B * Tq, Hq);
  if (!workspace || ws_bytes < need) return LSA_ERR_WORKSPACE;
  hipError_t e = launch_attention_prefill(q, k_cache, v_cache, B, Tq, q_start, Tmax, Hq, Hkv, idx,
                                          count, L_max, n_sink, window, scale, out,
                                          reinterpret_cast<float*>(workspace), as_stream(stream));
  return hip_status(e);
}

int lsa_dense_attention(const void* q, const void* k_cache, const void* v_cache, int64_t Tq,
                        int64_t q_start, int64_t Tk, int32_t Hq, int32_t Hkv, int32_t D,
                        int64_t band, float scale, int32_t dtype, void* out, void* stream) {
  if (Tq < 0 || q_start < 0 || Tk < 0 || band < 1) return LSA_ERR_ARG;
  if (dtype != LSA_BF16 || D != kHeadDim || Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0)
    return LSA_ERR_UNSUPPORTED;
  const int32_t G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return LSA_ERR_UNSUPPORTED;
  if (Tq == 0) return LSA_OK;
  if (!q || !k_cache || !v_cache || !out) return LSA_ERR_ARG;
  if (q_start + Tq > Tk) return LSA_ERR_ARG;
  if (Hkv > 65535) return LSA_ERR_UNSUPPORTED;
  hipError_t e = launch_dense_attention(q, k_cache, v_cache, Tq, q_start, Tk, Hq, Hkv, band, scale,
                                        out, as_stream(stream));
  return hip_status(e);
}

int lsa_sparse_attention_static(const void* q, const void* k_cache, const void* v_cache,
                                int32_t B, int64_t Tq, int64_t Tmax, int32_t Hq, int32_t Hkv,
                                int32_t D, const int32_t* idx, const int32_t* count,
                                int32_t L_max, float scale, int32_t dtype, int32_t splits,
                                void* out, void* stream) {
  int64_t need = 0;
  const int rc = check_attention(q, k_cache, v_cache, B, Tq, Tmax, Hq, Hkv, D, idx, count, L_max,
                                 dtype, splits, out, &need);
  if (rc) return rc < 0 ? rc : LSA_OK;
  if (need > LSA_STATIC_SCRATCH_BYTES) return LSA_ERR_CAPACITY;
  float* ws = nullptr;
  if (need > 0) {
    hipError_t e = static_scratch(&ws);
    if (e != hipSuccess) return LSA_ERR_HIP;
  }
  hipError_t e = launch_attention(q, k_cache, v_cache, B, Tq, Tmax, Hq, Hkv, idx, count, L_max,
                                  scale, dtype, splits, out, ws, as_stream(stream));
  return hip_status(e);
}

}  // extern "C"
