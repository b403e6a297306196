// Dense (and banded) causal attention over contiguous key ranges, bf16, and
// the near-set part of the prefill attention (k_near_attn, below).
//
// The baseline the pages compare sparse attention with is full attention
// ([72x "Why choosing costs so much"]; [summary]: 72.4x prefill over full
// attention at 10M tokens): every query attends to every key up to its own
// position.  The same kernel with a band of W keys computes attention over
// the recent window [p - W + 1, p] alone.
//
// Layout: Q [rows, Hq, 128] for positions q_start .. q_start + rows - 1,
// K / V [Tk, Hkv, 128], out [rows, Hq, 128]; head h reads KV head h / G.
// A workgroup takes one KV head and 8 waves x (16 / G) consecutive positions;
// each wave owns 16 MFMA columns = (16 / G) positions x G heads.  Key tiles of
// 16 keys (4 KiB of K and 4 KiB of V for the KV head) are staged in LDS by the
// whole workgroup, double buffered, one barrier per tile; the products are
// taken transposed (S^T = K Q^T with 16x16x32 MFMAs, O^T = V^T P^T with
// 16x16x16 MFMAs and transposing LDS reads of V), so P never leaves
// registers.  Online softmax in base 2 per column.
#include "lsa_internal.h"

namespace lsa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;

__device__ __forceinline__ uint2 tr16(const uint16_t* p) {
  v4s_t r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t*)(p));
  return __builtin_bit_cast(uint2, r);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

constexpr int kDenseWaves = 8;
constexpr int kDenseNT = 64 * kDenseWaves;
constexpr int kKTile = 16 * 256;              // 16 keys x 256 B (one KV head)

struct DenseArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  int64_t rows, q_start, Tk;
  int64_t band;             // keys [p - band + 1, p]; >= p + 1 covers every key
  int32_t Hq, Hkv, G;
  float scale_log2;         // scale * log2(e)
};

template <int G>
__global__ __launch_bounds__(kDenseNT) void k_dense_attn(DenseArgs a) {
  constexpr int PW = 16 / G;                  // positions per wave
  constexpr int P = kDenseWaves * PW;         // positions per workgroup
  __shared__ __attribute__((aligned(16))) char lds[2][2][kKTile];   // [buffer][K, V]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kvh = blockIdx.y;
  const int64_t r0 = (int64_t)blockIdx.x * P;                // first row of the workgroup
  const int r16 = lane & 15, u = lane >> 4;
  // this lane's MFMA column: position pw, head g of the KV head's group
  const int pw = r16 / G, g = r16 % G;
  const int64_t row = r0 + (int64_t)wave * PW + pw;
  const bool row_ok = row < a.rows;
  const int64_t p = a.q_start + (row_ok ? row : a.rows - 1);
  const int64_t lo = p - a.band + 1 > 0 ? p - a.band + 1 : 0;
  // the wave's key range and the workgroup's
  const int64_t w_row0 = r0 + (int64_t)wave * PW;
  const int64_t w_plast = a.q_start + (w_row0 + PW - 1 < a.rows ? w_row0 + PW - 1 : a.rows - 1);
  const int64_t w_pfirst = a.q_start + (w_row0 < a.rows ? w_row0 : a.rows - 1);
  const int64_t w_lo = w_pfirst - a.band + 1 > 0 ? w_pfirst - a.band + 1 : 0;
  const int64_t g_last = a.q_start + (r0 + P - 1 < a.rows ? r0 + P - 1 : a.rows - 1);
  const int64_t g_first = a.q_start + r0;
  const int64_t g_lo = g_first - a.band + 1 > 0 ? g_first - a.band + 1 : 0;
  const int64_t t_first = g_lo >> 4, t_last = g_last >> 4;
  const bool wave_live = w_row0 < a.rows;

  // Q^T fragments: lane (column r16, u) holds dims 32 j + 8 u .. + 7
  bf16x8 qf[4];
  {
    const int64_t h = (int64_t)kvh * G + g;
    const u32x4_t* qrow = reinterpret_cast<const u32x4_t*>(
        a.q + ((row_ok ? row : 0) * a.Hq + h) * kHeadDim);
#pragma unroll
    for (int j = 0; j < 4; ++j) qf[j] = __builtin_bit_cast(bf16x8, row_ok ? qrow[4 * j + u] : u32x4_t{0, 0, 0, 0});
  }
  f32x4 o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -1e30f, lp = 0.f;
  const float sl = a.scale_log2;

  // tile loads: threads 0..255 take K, 256..511 V; thread t: key (t & 255) / 16,
  // 16-byte chunk t % 16 of the key's 256 B head row
  const int ld_v = tid >> 8, ld_key = (tid & 255) >> 4, ld_ch = tid & 15;
  const uint16_t* src = ld_v ? a.v : a.k;
  auto fetch = [&](int64_t t) -> u32x4_t {
    int64_t key = t * 16 + ld_key;
    key = key < a.Tk ? key : a.Tk - 1;
    return *reinterpret_cast<const u32x4_t*>(src + (key * a.Hkv + kvh) * kHeadDim + 8 * ld_ch);
  };
  auto put = [&](int buf, u32x4_t x) {
    const int rr = ld_key;
    const int sw = ld_v ? (ld_ch ^ (2 * (rr & 7))) : (ld_ch ^ rr);
    *reinterpret_cast<u32x4_t*>(&lds[buf][ld_v][256 * rr + 16 * sw]) = x;
  };
  // transposing V reads: source lane s of a 16-lane group points at key row
  // 4 u + (s >> 2), dims 16 j + 4 (s & 3) .. +3; lane (r16, u) receives dim
  // 16 j + r16 of keys 4 u .. 4 u + 3
  const int sk = 4 * u + (r16 >> 2), cv = (r16 & 3) >> 1, vsw = 2 * (sk & 7);

  put(0, fetch(t_first));
  __syncthreads();
  for (int64_t t = t_first; t <= t_last; ++t) {
    const int buf = (int)((t - t_first) & 1);
    u32x4_t nx{0, 0, 0, 0};
    if (t < t_last) nx = fetch(t + 1);
    const int64_t kb = t * 16;
    // the wave computes only tiles that meet its key range
    if (wave_live && kb + 15 >= w_lo && kb <= w_plast) {
      const char* kt = lds[buf][0];
      const char* vt = lds[buf][1];
      u32x4_t kf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        kf[j] = *reinterpret_cast<const u32x4_t*>(kt + 256 * r16 + 16 * ((4 * j + u) ^ r16));
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[j]), qf[j], sacc,
                                                       0, 0, 0);
      // keys 4 u + i of this tile against the column's range [lo, p]
      bool ok[4];
      float x = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t key = kb + 4 * u + i;
        ok[i] = row_ok && key >= lo && key <= p;
        if (ok[i]) x = fmaxf(x, sacc[i] * sl);
      }
      x = fmaxf(x, __shfl_xor(x, 16, 64));
      x = fmaxf(x, __shfl_xor(x, 32, 64));
      const float mn = fmaxf(m, x);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      lp *= alpha;
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[j][i] *= alpha;
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = ok[i] ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], sl, -m)) : 0.f;
        lp += pv[i];
      }
      uint2 w2;
      w2.x = pack2(pv[0], pv[1]);
      w2.y = pack2(pv[2], pv[3]);
      const v4s_t pb4 = __builtin_bit_cast(v4s_t, w2);
      const char* vrd = vt + 256 * sk + 8 * (r16 & 1);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const v4s_t va4 = __builtin_bit_cast(
            v4s_t, tr16(reinterpret_cast<const uint16_t*>(vrd + 16 * ((2 * j + cv) ^ vsw))));
        o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va4, pb4, o[j], 0, 0, 0);
      }
    }
    if (t < t_last) put(buf ^ 1, nx);
    __syncthreads();
  }
  float l = lp;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (row_ok) {
    const int64_t h = (int64_t)kvh * G + g;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* orow = a.out + (row * a.Hq + h) * kHeadDim + 4 * u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint2 w;
      w.x = pack2(o[j][0] * inv, o[j][1] * inv);
      w.y = pack2(o[j][2] * inv, o[j][3] * inv);
      *reinterpret_cast<uint2*>(orow + 16 * j) = w;
    }
  }
}


// ---------------------------------------------------------------------------
// The near part of a query's list, dense.  Every list the index writes holds
// the sinks and the recent window ([72x "The same steps in general"]; [visual
// "What one query actually does"]: the sinks and the window are always
// read): keys [0, min(p + 1, S)) and [max(p - W + 1, 0), p] for a query at
// position p.  Consecutive queries share almost all of them (the windows of
// 32 neighbours cover W + 31 keys), so instead of gathering them once per
// query they are attended here once per tile of neighbouring queries (one KV
// head, 8 waves, each with two groups of 16 MFMA columns), over the tile's
// sink keys and the union of its windows.  The result is the softmax state of
// that partial attention per (row, head): O relative to the reference max m
// (base 2, scaled), m, and the sum l; the gather kernel starts from it and
// adds the list's remaining (far) keys.
constexpr int kNearTile = 32;               // keys per near tile
constexpr int kNearRing = 4;                // K/V tiles in flight per near workgroup

struct NearArgs {
  const uint16_t* q;        // [B * Tq, Hq, 128]
  const uint16_t* k;        // [B, Tmax, Hkv, 128]
  const uint16_t* v;
  float* po;                // [nrows, Hq, 128]: O of rows row0 .. row0 + nrows - 1
  float* pm;                // [nrows, Hq]: m (base 2, scale applied)
  float* pl;                // [nrows, Hq]: l
  int64_t row0, nrows;      // the launch's rows (global row = b * Tq + t)
  int64_t Tq, q_start, Tmax, n_sink, window;
  int64_t tile0, tiles_per_seq, ntiles;   // the launch's tiles: tile0 .. tile0 + ntiles - 1
  int32_t Hq, Hkv;
  float scale_log2;
};

// One workgroup per tile of P = 8 waves x 2 x 16 / G neighbouring positions
// and one KV head: each wave owns two groups of 16 MFMA columns (positions x
// the KV head's G query heads), so every K and V fragment it reads from LDS
// feeds two products.
constexpr int kNearGroups = 2;                // 16-column groups per wave
constexpr float kNearLazy = 8.f;              // lazy max: rescale past 2^8

template <int G>
__global__ __launch_bounds__(kDenseNT) void k_near_attn(NearArgs a) {
  constexpr int PW = 16 / G;                  // positions per 16-column group
  constexpr int CG = kNearGroups;
  constexpr int P = kDenseWaves * CG * PW;    // positions per workgroup
  constexpr int KT = kNearTile;
  __shared__ __attribute__((aligned(16))) char lds[2][2][KT * 256];   // [buffer][K, V]
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kvh = blockIdx.y;
  // neighbouring tiles share almost all of their window keys: the XCD that a
  // workgroup runs on (blockIdx.x mod 8) takes a contiguous range of tiles,
  // so that they meet in its L2
  const int64_t per_xcd = (a.ntiles + 7) / 8;
  const int64_t local = (int64_t)(blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (local >= a.ntiles) return;                            // uniform over the workgroup
  const int64_t tile = a.tile0 + local;
  const int64_t b = tile / a.tiles_per_seq;
  const int64_t t0 = (tile % a.tiles_per_seq) * P;           // first position index of the tile
  const int64_t t_end = t0 + P < a.Tq ? t0 + P : a.Tq;       // one past the last
  const int r16 = lane & 15, u = lane >> 4;
  const int pw = r16 / G, g = r16 % G;
  // this lane's columns: group c has position index t[c], global row b * Tq + t[c]
  const int64_t wt0 = t0 + (int64_t)wave * CG * PW;          // the wave's first position
  int64_t grow[CG], p[CG], s_end[CG], w_start[CG];
  bool col_ok[CG];
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    const int64_t t = wt0 + c * PW + pw;
    grow[c] = b * a.Tq + t;
    col_ok[c] = t < a.Tq && grow[c] >= a.row0 && grow[c] < a.row0 + a.nrows;
    p[c] = a.q_start + (t < a.Tq ? t : a.Tq - 1);
    s_end[c] = p[c] + 1 < a.n_sink ? p[c] + 1 : a.n_sink;
    w_start[c] = p[c] - a.window + 1 > 0 ? p[c] - a.window + 1 : 0;
  }
  // the workgroup's keys: sinks [0, sk_end), then the windows up to p_last
  const int64_t p_first = a.q_start + t0, p_last = a.q_start + t_end - 1;
  const int64_t sk_end = p_last + 1 < a.n_sink ? p_last + 1 : a.n_sink;
  const int64_t wk_lo = p_first - a.window + 1 > 0 ? p_first - a.window + 1 : 0;
  const int64_t ts_end = (sk_end + KT - 1) / KT;                // sink tiles [0, ts_end)
  const int64_t tw0 = wk_lo / KT > ts_end ? wk_lo / KT : ts_end;
  const int64_t n_tiles = ts_end + (p_last / KT >= tw0 ? p_last / KT - tw0 + 1 : 0);
  auto tile_of = [&](int64_t i) -> int64_t { return i < ts_end ? i : tw0 + (i - ts_end); };
  // the wave's keys, to skip tiles that none of its columns reads
  const bool wave_live = wt0 < t_end;
  const int64_t wp_first = a.q_start + wt0;
  const int64_t wp_last = a.q_start + (wt0 + CG * PW - 1 < t_end - 1 ? wt0 + CG * PW - 1 : t_end - 1);
  const int64_t ws_end = wp_last + 1 < a.n_sink ? wp_last + 1 : a.n_sink;
  const int64_t ww_lo = wp_first - a.window + 1 > 0 ? wp_first - a.window + 1 : 0;

  bf16x8 qf[CG][4];
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    const int64_t h = (int64_t)kvh * G + g;
    const u32x4_t* qrow =
        reinterpret_cast<const u32x4_t*>(a.q + ((col_ok[c] ? grow[c] : 0) * a.Hq + h) * kHeadDim);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      qf[c][j] = __builtin_bit_cast(bf16x8, col_ok[c] ? qrow[4 * j + u] : u32x4_t{0, 0, 0, 0});
  }
  f32x4 o[CG][8];
  float m[CG], lp[CG];
#pragma unroll
  for (int c = 0; c < CG; ++c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) o[c][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[c] = -1e30f;
    lp[c] = 0.f;
  }
  const float sl = a.scale_log2;
  // positions as 32-bit values (the host keeps Tmax below 2^31)
  int32_t p32[CG], se32[CG], ws32[CG];
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    // an invalid column takes an empty near set
    p32[c] = col_ok[c] ? (int32_t)p[c] : -1;
    se32[c] = (int32_t)s_end[c];
    ws32[c] = (int32_t)w_start[c];
  }
  // a tile inside every column's window needs no mask: keys >= the largest
  // window start and <= the smallest position of the wave (all columns valid)
  bool all_ok = true;
#pragma unroll
  for (int c = 0; c < CG; ++c) all_ok &= col_ok[c];
  const bool wave_full = __builtin_amdgcn_readfirstlane(__ballot(!all_ok) == 0 ? 1 : 0) != 0;
  const int64_t full_lo = wp_last - a.window + 1, full_hi = wp_first;

  // tile loads: threads 0..255 take K, 256..511 V; thread t: 16-byte chunk
  // t % 16 of keys (t & 255) / 16 and that + 16
  const int ld_v = tid >> 8, ld_key = (tid & 255) >> 4, ld_ch = tid & 15;
  const uint16_t* src = (ld_v ? a.v : a.k) + b * a.Tmax * a.Hkv * kHeadDim;
  struct Chunk { u32x4_t x[2]; };
  auto fetch = [&](int64_t i) -> Chunk {
    Chunk c;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      int64_t key = tile_of(i) * KT + 16 * hh + ld_key;
      key = key < a.Tmax ? key : a.Tmax - 1;
      c.x[hh] = *reinterpret_cast<const u32x4_t*>(src + (key * a.Hkv + kvh) * kHeadDim + 8 * ld_ch);
    }
    return c;
  };
  // chunks XOR swizzled by row: K by (row & 15), V by 2 (row & 7)
  auto put = [&](int buf, const Chunk& c) {
    const int sw = ld_v ? (ld_ch ^ (2 * (ld_key & 7))) : (ld_ch ^ ld_key);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      *reinterpret_cast<u32x4_t*>(&lds[buf][ld_v][256 * (16 * hh + ld_key) + 16 * sw]) = c.x[hh];
  };
  const int sk = 4 * u + (r16 >> 2), cv = (r16 & 3) >> 1, vsw = 2 * (sk & 7);

  // kNearRing tiles are requested ahead of the one computed (each thread
  // holds its 32 bytes of each in registers); one barrier per tile, the LDS
  // tiles double buffered.  A tile is two halves of 16 keys: the scores of
  // half hh come from 16x16x32 products S^T = K Q^T (lane (column, u) gets
  // keys 16 hh + 4 u .. + 3), and O^T += V^T P^T is one 16x16x32 product per
  // 16 dims whose k index 8 u + e stands for key 4 u + e (e < 4) or
  // 16 + 4 u + e - 4 (e >= 4), so each lane's eight probabilities are its own
  // scores of the two halves and V^T takes one transposing read per half.
  Chunk ring[kNearRing];
  // Q first: with only ring loads pending in the loop, each tile's wait is
  // kNearRing - 1 later loads
  __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0)
#pragma unroll
  for (int j = 0; j < kNearRing; ++j) {
    ring[j] = fetch(j < n_tiles ? j : n_tiles - 1);
    __builtin_amdgcn_sched_barrier(0);         // keep the loads in ring order
  }
  for (int64_t i0 = 0; i0 < n_tiles; i0 += kNearRing) {
#pragma unroll
    for (int j = 0; j < kNearRing; ++j) {
      // whole ring cycles: tiles past the end are staged (a repeat of the
      // last one) but not computed, and every load is unconditional (past the
      // end it repeats the last tile), so that each wait on the ring is the
      // same count of later loads
      const int64_t i = i0 + j;
      const int buf = j & 1;                   // kNearRing is even: buffers alternate
      put(buf, ring[j]);
      __syncthreads();
      ring[j] = fetch(i + kNearRing < n_tiles ? i + kNearRing : n_tiles - 1);
      const int64_t kb = tile_of(i < n_tiles ? i : n_tiles - 1) * KT;
      if (i < n_tiles && wave_live && (kb < ws_end || (kb + KT - 1 >= ww_lo && kb <= wp_last))) {
        const char* kt = lds[buf][0];
        const char* vt = lds[buf][1];
        f32x4 sacc[CG][2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          u32x4_t kf[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            kf[jj] = *reinterpret_cast<const u32x4_t*>(kt + 256 * (16 * hh + r16) +
                                                       16 * ((4 * jj + u) ^ r16));
#pragma unroll
          for (int c = 0; c < CG; ++c) {
            sacc[c][hh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              sacc[c][hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  __builtin_bit_cast(bf16x8, kf[jj]), qf[c][jj], sacc[c][hh], 0, 0, 0);
          }
        }
        const bool full = wave_full && kb >= full_lo && kb + KT - 1 <= full_hi;
        const int32_t kq = (int32_t)kb + 4 * u;            // this lane's first key
        bf16x8 pb8[CG];
#pragma unroll
        for (int c = 0; c < CG; ++c) {
          // scaled scores of keys 16 hh + 4 u + e (base 2); keys outside the
          // column's near set get -inf
          float xs[8];
          if (full) {                            // uniform: no key of the tile is masked
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
              for (int e = 0; e < 4; ++e) xs[4 * hh + e] = sacc[c][hh][e] * sl;
          } else {
            // non-short-circuit operators: lane masks, no branches
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int32_t key = kq + 16 * hh + e;
                const bool ok = (key <= p32[c]) & ((key < se32[c]) | (key >= ws32[c]));
                xs[4 * hh + e] = ok ? sacc[c][hh][e] * sl : -__builtin_inff();
              }
          }
          bool up = false;
#pragma unroll
          for (int e = 0; e < 8; ++e) up |= xs[e] > m[c] + kNearLazy;
          // lazy reference max: O and l are rescaled only when a score
          // exceeds it by more than 2^kNearLazy (they always share it, so the
          // result does not depend on when that happens)
          if (__ballot(up)) {
            float x = fmaxf(fmaxf(fmaxf(xs[0], xs[1]), fmaxf(xs[2], xs[3])),
                            fmaxf(fmaxf(xs[4], xs[5]), fmaxf(xs[6], xs[7])));
            x = fmaxf(x, __shfl_xor(x, 16, 64));
            x = fmaxf(x, __shfl_xor(x, 32, 64));
            const float mn = fmaxf(m[c], x);
            const float alpha = __builtin_amdgcn_exp2f(m[c] - mn);
            m[c] = mn;
            lp[c] *= alpha;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
#pragma unroll
              for (int e = 0; e < 4; ++e) o[c][jj][e] *= alpha;
          }
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pv[e] = __builtin_amdgcn_exp2f(xs[e] - m[c]);
            lp[c] += pv[e];
          }
          u32x4_t w4;
          w4.x = pack2(pv[0], pv[1]);
          w4.y = pack2(pv[2], pv[3]);
          w4.z = pack2(pv[4], pv[5]);
          w4.w = pack2(pv[6], pv[7]);
          pb8[c] = __builtin_bit_cast(bf16x8, w4);
        }
        const char* vrd = vt + 256 * sk + 8 * (r16 & 1);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int off = 16 * ((2 * jj + cv) ^ vsw);
          const uint2 v0 = tr16(reinterpret_cast<const uint16_t*>(vrd + off));
          const uint2 v1 = tr16(reinterpret_cast<const uint16_t*>(vrd + 16 * 256 + off));
          const bf16x8 va8 = __builtin_bit_cast(bf16x8, u32x4_t{v0.x, v0.y, v1.x, v1.y});
#pragma unroll
          for (int c = 0; c < CG; ++c)
            o[c][jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va8, pb8[c], o[c][jj], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    float l = lp[c];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if (col_ok[c]) {
      const int64_t h = (int64_t)kvh * G + g;
      const int64_t slot = (grow[c] - a.row0) * a.Hq + h;
      float* orow = a.po + slot * kHeadDim + 4 * u;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<float4*>(orow + 16 * j) = make_float4(o[c][j][0], o[c][j][1], o[c][j][2],
                                                                o[c][j][3]);
      if (u == 0) { a.pm[slot] = m[c]; a.pl[slot] = l; }
    }
  }
}

}  // namespace

hipError_t launch_dense_attention(const void* q, const void* k, const void* v, int64_t rows,
                                  int64_t q_start, int64_t Tk, int32_t Hq, int32_t Hkv,
                                  int64_t band, float scale, void* out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  DenseArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.out = (uint16_t*)out;
  a.rows = rows; a.q_start = q_start; a.Tk = Tk; a.band = band;
  a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.scale_log2 = scale * 1.4426950408889634f;
  const int G = Hq / Hkv;
  const int P = kDenseWaves * (16 / G);
  dim3 grid((unsigned)((rows + P - 1) / P), (unsigned)Hkv);
  switch (G) {
    case 1: hipLaunchKernelGGL(k_dense_attn<1>, grid, dim3(kDenseNT), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_dense_attn<2>, grid, dim3(kDenseNT), 0, s, a); break;
    case 4: hipLaunchKernelGGL(k_dense_attn<4>, grid, dim3(kDenseNT), 0, s, a); break;
    case 8: hipLaunchKernelGGL(k_dense_attn<8>, grid, dim3(kDenseNT), 0, s, a); break;
    case 16: hipLaunchKernelGGL(k_dense_attn<16>, grid, dim3(kDenseNT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_near_attention(const void* q, const void* k, const void* v, int64_t row0,
                                 int64_t nrows, int64_t Tq, int64_t q_start, int64_t Tmax,
                                 int32_t Hq, int32_t Hkv, int64_t n_sink, int64_t window,
                                 float scale, float* po, float* pm, float* pl, hipStream_t s) {
  if (nrows <= 0) return hipSuccess;
  const int G = Hq / Hkv;
  if (G < 1 || G > 16 || 16 % G != 0 || Hq % Hkv != 0) return hipErrorInvalidValue;
  const int P = kDenseWaves * kNearGroups * (16 / G);
  NearArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.po = po; a.pm = pm; a.pl = pl;
  a.row0 = row0; a.nrows = nrows;
  a.Tq = Tq; a.q_start = q_start; a.Tmax = Tmax; a.n_sink = n_sink; a.window = window;
  a.tiles_per_seq = (Tq + P - 1) / P;
  // the tiles holding the launch's first and last rows (tiles never straddle
  // two sequences; a tile cut by the launch's bounds writes its rows only)
  auto tile_of_row = [&](int64_t r) { return (r / Tq) * a.tiles_per_seq + (r % Tq) / P; };
  a.tile0 = tile_of_row(row0);
  a.ntiles = tile_of_row(row0 + nrows - 1) - a.tile0 + 1;
  a.Hq = Hq; a.Hkv = Hkv;
  a.scale_log2 = scale * 1.4426950408889634f;
  // eight XCD ranges of ceil(ntiles / 8) tiles each
  dim3 grid((unsigned)(8 * ((a.ntiles + 7) / 8)), (unsigned)Hkv);
  switch (G) {
    case 1: hipLaunchKernelGGL(k_near_attn<1>, grid, dim3(kDenseNT), 0, s, a); break;
    case 2: hipLaunchKernelGGL(k_near_attn<2>, grid, dim3(kDenseNT), 0, s, a); break;
    case 4: hipLaunchKernelGGL(k_near_attn<4>, grid, dim3(kDenseNT), 0, s, a); break;
    case 8: hipLaunchKernelGGL(k_near_attn<8>, grid, dim3(kDenseNT), 0, s, a); break;
    case 16: hipLaunchKernelGGL(k_near_attn<16>, grid, dim3(kDenseNT), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lsa
