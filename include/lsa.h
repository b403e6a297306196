/*
 * lsa.h -- C ABI of the Latent Sparse Attention (LSA) indexing + sparse
 * attention library for AMD Instinct MI355X (gfx950).
 *
 * Page citations use these short names (the pages are public web pages on
 * the paper "Latent Sparse Attention: Towards Subquadratic Ultra-Long Context
 * Attention"):
 *   [summary]  "Latent Sparse Attention: Towards Subquadratic Ultra-Long
 *              Context Attention" (paper summary page)
 *   [catalog]  "Latent Sparse Attention (LSA): A Card-Catalog Approach to
 *              Subquadratic Ultra-Long Context Attention" (forum post)
 *   [72x]      "Latent Sparse Attention: 72x in One Layer, 9x for the Whole
 *              Model at 10M Tokens" (blog post)
 *   [visual]   "Latent Sparse Attention at 10M tokens -- Hierarchical key
 *              clusters" (explainer)
 *
 * Conventions shared by every entry point
 *   - Ownership: the caller owns every device buffer (cache storage,
 *     workspaces, inputs, outputs).  The library never allocates device
 *     memory; it only allocates the small host-side lsa_cache handle.
 *   - Execution: every call that takes a `stream` enqueues its kernels on that
 *     HIP stream (a hipStream_t passed as void*, NULL = default stream) and
 *     returns without synchronising.  Outputs are valid once the stream has
 *     reached that point.
 *   - Errors: calls return LSA_OK (0) or a negative lsa_status.  All
 *     arguments are validated on the host before anything is enqueued; a
 *     rejected call changes nothing.  A launch failure returns LSA_ERR_HIP.
 *   - Layout: row-major, contiguous.  Key positions are int32 (< 2^31).
 *     Index lists are ascending and padded with -1.
 *   - Concurrency: calls on the same cache must not overlap; separate caches
 *     are independent.
 *   - Supported shapes: d_latent 64, n_pool 4, block 512, 64 buckets per
 *     block, bucket cap 16 keys, head_dim 128, Hq % Hkv == 0,
 *     Hq / Hkv <= 16, 0 <= k <= 8192, 0 <= n_sink <= 8192,
 *     1 <= window <= 8192, and the candidates of one query must fit one
 *     workgroup's LDS: with cap = 3 * lsa_top_buckets(p) rounded up (to a
 *     power of two up to 8,192, else to a multiple of 1,024), cap <= 16,384
 *     and 9 * cap + 4 * k <= 147,200 bytes (this holds for every k with the
 *     default window and sinks).  Anything else returns LSA_ERR_UNSUPPORTED.
 */
#ifndef LSA_H
#define LSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LSA_OK = 0,
  LSA_ERR_ARG = -1,         /* null pointer, negative size, inconsistent arguments */
  LSA_ERR_UNSUPPORTED = -2, /* parameter value outside the supported shapes */
  LSA_ERR_WORKSPACE = -3,   /* workspace smaller than the matching *_workspace_bytes */
  LSA_ERR_CAPACITY = -4,    /* cache storage too small / appending past max_tokens */
  LSA_ERR_HIP = -5,         /* a HIP launch or API call failed */
  LSA_ERR_STATE = -6        /* e.g. a tree query on a cache built without a tree */
} lsa_status;

enum { LSA_F32 = 0, LSA_BF16 = 1 };  /* element types */
enum { LSA_FLAT = 0, LSA_TREE = 1 }; /* search modes */

/*
 * Method parameters.  [catalog "Key points"]: 64-d latent keys, pooled by 4,
 * 512-key cluster blocks, buckets of about 8 and at most 16 keys.
 * [72x "The same steps in general"]: k far keys, 4 sinks, a 512-key window.
 */
typedef struct {
  int32_t d_latent;        /* latent dimension: 64 */
  int32_t n_pool;          /* unit keys summed per pooled key: 4 */
  int32_t block_keys;      /* keys per cluster block: 512 */
  int32_t n_buckets;       /* buckets per full block: 64 */
  int32_t bucket_cap_keys; /* max keys per bucket: 16 */
  int32_t k;               /* far keys per query, 0..8192 */
  int32_t n_sink;          /* leading keys always read (clipped to the query) */
  int32_t window;          /* recent keys always read, query included */
  int32_t mode;            /* LSA_FLAT or LSA_TREE (cache: build a tree too) */
  int32_t beam;            /* tree beam width, 1..512 (beyond 64 a workgroup per query) */
  int32_t leaf_level;      /* tree: level where the beam stops; -1 = smallest l
                              with beam * 2^l >= lsa_top_buckets(p) */
  int32_t index_dtype;     /* stored centroids and normalised queries: LSA_F32 | LSA_BF16 */
  int32_t exact_select;    /* 0: sampled threshold + exact fallback; 1: always exact */
  int32_t scan_keys;       /* 0: LSA buckets.  1, 4, 8: a scan baseline instead
                              ([72x "Why choosing costs so much"], "One real query,
                              start to finish"): a token scan (1) scores every key,
                              a block scan every aligned run of 4 or 8 keys; see
                              the scan section below */
  int32_t score_heads;     /* 0 or 1: one latent query per position.  2, 4, 8: that
                              many query heads per position, and a bucket scores
                              the max over the heads' dot products ([catalog "Key
                              points"], N-LSA: bucket selection uses the max score
                              across heads); latent_q is then [Tq, H, 64].  Flat
                              bf16 prefill only */
  int32_t start_level;     /* tree: -1 = the beam starts at the root.  s >= 0:
                              every eligible node of level s is scored first and
                              the best `beam` kept, then the beam descends (the
                              fixed-level search of [visual "A worked example"]'s
                              table: score coarse groups, refine inside the
                              winners; s = leaf level is the two-stage search).
                              Clamped to [leaf level, tree height] */
} lsa_params;

/* Fills *p with the defaults above (k = 2048, flat, bf16). */
void lsa_default_params(lsa_params* p);

/* sizeof(lsa_params) in this build: a binding checks it against its own
 * copy of the struct before passing one (a mismatch means a binding and a
 * library from different versions). */
int32_t lsa_params_bytes(void);

/* Human-readable name of a status code (static storage). */
const char* lsa_status_string(int status);

/* LSA_OK if *p is within the supported shapes. */
int lsa_check_params(const lsa_params* p);

/* Index list length n_sink + window + k (or a negative status). */
int32_t lsa_list_len(const lsa_params* p);

/* Buckets kept per query before expansion:
 *   B = ceil(k / n_pool) + n_buckets * ceil((window - 1) / block_keys)
 *       + ceil(n_sink / n_pool)
 * (ceil(k / 4) + 65 for the default window of 512 and 4 sinks).  The B best
 * buckets always hold k far keys, or every eligible bucket is kept: a bucket
 * holding no sink or window key gives at least n_pool far keys, and the
 * window reaches back into at most ceil((window - 1) / block_keys) eligible
 * blocks of n_buckets buckets, the sinks into ceil(n_sink / n_pool) buckets
 * ([72x "The same steps in general"]: keys of an opened bucket that are
 * already sinks or window keys are skipped and the next key takes their
 * place, so opening stops only once k far keys are taken). */
int32_t lsa_top_buckets(const lsa_params* p);

/* ---------------------------------------------------------------- cache --
 * The bucket cache [catalog "Summary", "Key points"], [visual "How the
 * hierarchy is built"]: per full 512-key block, 64 buckets, each a unit
 * centroid (index_dtype, 64 values) and a member table (4 bytes: the
 * block-local pooled indices of its members, ascending, 0xFF = unused); in
 * tree mode also the tree levels above the buckets.  Buckets are numbered
 * 64 * block + rank of their smallest pooled index.  Keys of the trailing
 * partial block are staged in the cache until the block is full. */
typedef struct lsa_cache lsa_cache;

/* Device bytes needed for a cache that can hold max_tokens keys. */
int64_t lsa_cache_bytes(const lsa_params* p, int64_t max_tokens);

/* Creates a host handle over caller-owned device memory `cache_mem` of
 * `bytes` bytes (>= lsa_cache_bytes).  The cache starts empty.  Structural
 * parameters (d_latent .. bucket_cap_keys, index_dtype, mode) are fixed here. */
int lsa_cache_init(const lsa_params* p, int64_t max_tokens, void* cache_mem, int64_t bytes,
                   lsa_cache** out);

/* Frees the host handle only; the device memory stays the caller's. */
int lsa_cache_release(lsa_cache* c);

/* Number of keys appended so far. */
int64_t lsa_cache_tokens(const lsa_cache* c);

/* Device addresses and sizes inside a cache, for reading it back. */
typedef struct {
  int64_t n_tokens;        /* keys appended */
  int64_t n_blocks;        /* full (clustered) blocks */
  int64_t n_buckets;       /* 64 * n_blocks */
  void* centroids;         /* [max_buckets, 64] index_dtype */
  uint32_t* members;       /* [max_buckets] packed pooled indices */
  float* staging;          /* [block_keys, 64] fp32 keys of the partial block */
  int32_t tree_height;     /* levels above the buckets (0 without a tree) */
  int64_t level_nodes[32]; /* nodes per level, level 0 = buckets */
  void* level_centroids[32];  /* level >= 1: [n, 64] index_dtype */
  int32_t* level_child[32];   /* level >= 1: [n, 2] child indices, -1 = none */
  int32_t* level_min_block[32]; /* level >= 1: [n] smallest block below */
} lsa_cache_view;

int lsa_cache_get_view(const lsa_cache* c, lsa_cache_view* out);

/* ------------------------------------------------------- cache builder --
 * build_bucket_cache appends n_new latent keys (device fp32 [n_new, 64]) to
 * the cache and clusters every block that becomes full: keys are
 * L2-normalised, every 4 consecutive unit keys are summed into a pooled key,
 * and the 128 pooled keys of the block are merged bottom-up by Ward's method
 * into 64 buckets of at most 4 pooled keys (16 keys) [catalog "Key points"],
 * [72x "The same steps in general"], [visual "How the hierarchy is built"].
 * Greedy global-minimum merging among feasible pairs, ties to the smallest
 * pair of cluster ids, normalisation and Ward costs in fp64.  Centroids are
 * the unit vector of the sum of the members' pooled keys, rounded to
 * index_dtype (nearest even).  In tree mode the tree levels above the new
 * buckets are rebuilt.  Blocks never change once clustered.
 * No workspace is needed.  Returns LSA_ERR_CAPACITY past max_tokens. */
int build_bucket_cache(lsa_cache* c, const float* latent_keys, int64_t n_new, void* stream);

/* ------------------------------------------------------------- indexer --
 * Workspace for lsa_index_prefill with up to max_queries queries, or for
 * lsa_index_decode with a batch of max_queries sequences. */
int64_t lsa_index_workspace_bytes(const lsa_params* p, int64_t max_queries);

/* Byte offset, inside the workspace of an lsa_index_prefill call over
 * n_queries queries (or an lsa_index_decode call over n_queries sequences),
 * of the int32 flag per query that the call leaves behind: 1 when that
 * query's B best buckets were selected by the exact fallback (its
 * candidate list from the sampled score threshold held more candidates than
 * fit, or fewer than k far keys while more buckets were eligible, so every
 * eligible bucket was rescored in one workgroup; with a `ranked` output
 * also when it held fewer than B buckets), 0 otherwise (always 1 with
 * exact_select).  The flags stay
 * valid, once the stream has passed the call, until the workspace is
 * reused.  Negative status on invalid parameters. */
int64_t lsa_index_status_offset(const lsa_params* p, int64_t n_queries);

/*
 * lsa_index_prefill: index lists for the Tq queries at positions
 * q_start .. q_start+Tq-1 of the sequence whose keys are in `c`.
 *   latent_q  device fp32 [Tq, 64]
 *   idx       device int32 [Tq, L] with L = lsa_list_len(p): ascending key
 *             positions, -1 padded
 *   count     device int32 [Tq]: valid entries of each row
 *   ranked    optional device int32 [Tq, lsa_top_buckets(p)]: the buckets
 *             kept before expansion, best first (-1 padded); may be NULL
 * Steps [visual "What one query actually does"], [72x "The same steps in
 * general"]: the query is normalised (fp64) and rounded to index_dtype; in
 * flat mode every eligible bucket (block < position / 512, i.e. complete
 * earlier blocks) is scored, in tree mode a beam search descends the tree
 * [catalog "Key points"]; buckets are ranked by (score desc, bucket asc),
 * opened best-first taking member keys (ascending) that are not sinks or
 * window keys until k far keys are collected; the list is the sorted union
 * of sinks, far keys and window.  One list per query, shared by all heads.
 * The cache may hold keys past the queries (the block mask ignores them),
 * but it must hold every block that is complete before the last query:
 * (q_start + Tq - 1) / 512 <= number of full blocks, else LSA_ERR_STATE.
 */
int lsa_index_prefill(const lsa_cache* c, const float* latent_q, int64_t q_start, int64_t Tq,
                      const lsa_params* p, int32_t* idx, int32_t* count, int32_t* ranked,
                      void* workspace, int64_t ws_bytes, void* stream);

/*
 * lsa_index_decode: one decode step for B independent sequences.
 *   caches        host array [B] of handles (distinct caches)
 *   latent_q      device fp32 [B, 64]: the new query of each sequence
 *   latent_k_new  device fp32 [B, 64]: the new key of each sequence
 * For sequence b with p = lsa_cache_tokens(caches[b]) the new key becomes
 * position p; if it completes a block ((p+1) % 512 == 0) that block is
 * clustered (and the tree updated) [visual "How the hierarchy is built"];
 * then the index list of the query at position p is written to idx[b] /
 * count[b] exactly as lsa_index_prefill would.  The caller appends the
 * matching K/V rows to its own KV cache.  B <= 64.
 */
int lsa_index_decode(lsa_cache* const* caches, int32_t B, const float* latent_q,
                     const float* latent_k_new, const lsa_params* p, int32_t* idx,
                     int32_t* count, void* workspace, int64_t ws_bytes, void* stream);

/* ----------------------------------------------------- sparse attention --
 * Workspace for lsa_sparse_attention (split partials; 0 when splits == 1). */
int64_t lsa_attention_workspace_bytes(int32_t B, int64_t Tq, int32_t Hq, int32_t D,
                                      int32_t splits);

/* Rows per launch of the bf16 attention: a call over more query rows issues
 * ceil(B * Tq / this) launches back to back on its stream, so that the rows
 * in flight stay neighbours (their lists share keys in the caches). */
int64_t lsa_attention_launch_rows(void);

/* 1 when lsa_sparse_attention in bf16 runs one workgroup per (query row,
 * KV head), grouping each KV head's workgroups on their own XCDs when Hkv
 * divides 8: always for Hkv != 4, and for Hkv = 4 when the K and V caches
 * hold at most 256 MiB each (B * Tmax * Hkv * D * 2 bytes).  0 when each
 * workgroup takes a whole row (Hkv = 4 with larger caches, where reading
 * each listed token's rows of all heads together pays more than the per-XCD
 * cache reuse), and for fp32 or D != 128.  Both layouts compute the same
 * results. */
int32_t lsa_attention_head_major(int32_t B, int64_t Tmax, int32_t Hkv, int32_t D, int32_t dtype);

/* A split count for lsa_sparse_attention: the largest power of two (<= 256)
 * that keeps at least 32 listed keys per split and rows * splits <= 256
 * (one row's split per compute unit), so that few query rows (decode) still
 * spread over the whole chip.  rows = B * Tq. */
int32_t lsa_attention_default_splits(int64_t rows, int32_t L_max);

/*
 * lsa_sparse_attention [visual "Intro", "What one query actually does"]:
 * ordinary softmax attention of every query head over the keys listed for
 * its query; head h reads KV head h * Hkv / Hq (GQA), all heads of a query
 * share its list.
 *   q        [B, Tq, Hq, D]      dtype
 *   k_cache  [B, Tmax, Hkv, D]   dtype
 *   v_cache  [B, Tmax, Hkv, D]   dtype
 *   idx      [B, Tq, L_max] int32 key positions (< Tmax), count [B, Tq]
 *   out      [B, Tq, Hq, D]      dtype
 * dtype LSA_BF16 (fp32 accumulation, fp32 softmax) or LSA_F32.
 * scale multiplies q.k (pass 1/sqrt(D)).  splits >= 1 splits each list into
 * that many parts whose partial softmax states are combined afterwards
 * (decode); needs lsa_attention_workspace_bytes of workspace.
 * A row with count 0 produces zeros.  List entries outside [0, Tmax) and
 * entries past a row's count are ignored; the bf16 kernels still load token
 * 0's rows for them (with zero weight), so Tmax must be at least 1 when
 * B * Tq > 0 (else LSA_ERR_ARG).
 */
int lsa_sparse_attention(const void* q, const void* k_cache, const void* v_cache, int32_t B,
                         int64_t Tq, int64_t Tmax, int32_t Hq, int32_t Hkv, int32_t D,
                         const int32_t* idx, const int32_t* count, int32_t L_max, float scale,
                         int32_t dtype, int32_t splits, void* out, void* workspace,
                         int64_t ws_bytes, void* stream);

/* ------------------------------------------------ prefill attention --
 * Attention for a prefill chunk whose lists hold the sinks and the recent
 * window, as every list lsa_index_prefill writes does ([72x "The same steps
 * in general"]; [visual "What one query actually does"]: sinks and window
 * are always read).  For the query row (b, t) at position p = q_start + t its
 * near set is N(p) = [0, min(p + 1, n_sink)) U [max(p - window + 1, 0), p];
 * the row attends over N(p) and over every entry of its list that lies
 * outside N(p) (entries outside [0, Tmax) and past the count are ignored, as
 * in lsa_sparse_attention).  For lists from lsa_index_prefill with the same
 * n_sink, window and q_start this is exactly lsa_sparse_attention over the
 * same lists (up to the order of rounding).
 * The near set is attended once per tile of neighbouring rows (dense
 * MFMA tiles over the tile's sinks and the union of its windows, whose K/V
 * rows are read once per tile instead of once per row) and the list's other
 * entries are gathered per row on top of that softmax state.
 *   q [B, Tq, Hq, 128], k_cache / v_cache [B, Tmax, Hkv, 128], idx
 *   [B, Tq, L_max], count [B, Tq], out [B, Tq, Hq, 128]; bf16 only,
 *   Hq / Hkv in {1, 2, 4, 8, 16}; q_start + Tq <= Tmax < 2^31; n_sink >= 0,
 *   window >= 1.
 * workspace: at least lsa_prefill_attention_workspace_bytes(B, Tq, Hq, D)
 * bytes of device memory (the near state of one launch's rows), caller-owned.
 * Returns LSA_ERR_UNSUPPORTED for fp32 or other shapes (use
 * lsa_sparse_attention), LSA_ERR_ARG for inconsistent sizes or null
 * pointers, LSA_ERR_WORKSPACE when the workspace is missing or short. */
int64_t lsa_prefill_attention_workspace_bytes(int32_t B, int64_t Tq, int32_t Hq, int32_t D);
int lsa_sparse_attention_prefill(const void* q, const void* k_cache, const void* v_cache,
                                 int32_t B, int64_t Tq, int64_t q_start, int64_t Tmax,
                                 int32_t Hq, int32_t Hkv, int32_t D, const int32_t* idx,
                                 const int32_t* count, int32_t L_max, int32_t n_sink,
                                 int32_t window, float scale, int32_t dtype, void* out,
                                 void* workspace, int64_t ws_bytes, void* stream);

/* ------------------------------------------------------- dense attention --
 * The full attention LSA is measured against ([summary], [abstract]: 72.4x
 * prefill over full attention at 10M tokens): for each query row at position
 * p = q_start + r, softmax attention of every query head over the keys
 * [max(0, p - band + 1), p] of its KV head (band >= p + 1, e.g. INT64_MAX:
 * every earlier key, dense causal attention; band = W: the recent window
 * alone).  bf16, head_dim 128, Hq / Hkv in {1, 2, 4, 8, 16}.
 *   q        [Tq, Hq, 128]   rows for positions q_start .. q_start + Tq - 1
 *   k_cache  [Tk, Hkv, 128], v_cache likewise; q_start + Tq <= Tk
 *   out      [Tq, Hq, 128]
 * scale multiplies q.k.  No workspace; asynchronous on `stream`.  Other
 * shapes or dtypes return LSA_ERR_UNSUPPORTED, q_start + Tq > Tk or band < 1
 * LSA_ERR_ARG. */
int lsa_dense_attention(const void* q, const void* k_cache, const void* v_cache, int64_t Tq,
                        int64_t q_start, int64_t Tk, int32_t Hq, int32_t Hkv, int32_t D,
                        int64_t band, float scale, int32_t dtype, void* out, void* stream);

/* ------------------------------------------- allocation-free attention --
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation as lsa_sparse_attention, with the split partials kept in a
 * fixed device array of LSA_STATIC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on (one copy per device, kept until the process ends).
 * The caller still owns q, the K/V caches, the lists and `out`; nothing is
 * allocated.  The array of the current device is used, so the stream must
 * belong to the current device.  Calls that overlap on one device (on
 * different streams) race on the array; calls on one stream do not.
 * Returns LSA_ERR_CAPACITY when the partials, i.e.
 * lsa_attention_workspace_bytes(B, Tq, Hq, D, splits), exceed the array
 * (splits == 1 needs none), and otherwise what lsa_sparse_attention
 * returns. */
#define LSA_STATIC_SCRATCH_BYTES (16 << 20)
int lsa_sparse_attention_static(const void* q, const void* k_cache, const void* v_cache,
                                int32_t B, int64_t Tq, int64_t Tmax, int32_t Hq, int32_t Hkv,
                                int32_t D, const int32_t* idx, const int32_t* count,
                                int32_t L_max, float scale, int32_t dtype, int32_t splits,
                                void* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LSA_H */
