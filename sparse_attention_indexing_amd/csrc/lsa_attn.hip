// Gather softmax attention over per-query key lists.
//
// [visual "Intro", "What one query actually does"]: after selection,
// ordinary attention runs over the sinks, the selected keys and the window,
// and one index list per query is shared by all of its attention heads.
//
// bf16 path (k_attn_bf16): one wave per (query row, KV head, split).  The GQA
// group of G <= 16 query heads forms one side of 16x16 bf16 MFMAs, so every
// gathered K/V row (256 B per KV head) is read once for the whole group.
// Online softmax in fp32; P is rounded to bf16 for the PV product.  fp32
// path (k_attn_f32): one wave per (query row, head).
#include "lsa_internal.h"

namespace lsa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

// bf16 rows are launched this many at a time.  A launch ends only when all of
// its rows are done, so the rows in flight stay neighbours, whose lists share
// many keys in L2 and the Infinity Cache; one launch over all rows lets the
// rows in flight drift apart.  At 128K queries 1,024-row launches take 17%
// less time than one launch (512 / 2,048 / 4,096 rows: +4 / +1.5 / +9%); at
// 1M and 10M tokens the size hardly matters.
constexpr int64_t kRowsPerLaunch = 1024;

__device__ __forceinline__ void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* idx;
  const int32_t* count;
  uint16_t* out;
  float* ws;            // split partials: O [rows, splits, Hq, 128], then m, l [rows, splits, Hq]
  int64_t rows;         // B * Tq
  int64_t row0, nrows;  // rows of this launch: row0 .. row0 + nrows - 1
  int64_t Tq, Tmax;
  int32_t Hq, Hkv, G, L, splits;
  float scale;
  float scale_log2;     // scale * log2(e): softmax in base 2
  // far-key mode: the softmax state of the near set (sinks and window) of
  // each launch row, [nrows, Hq, 128] O, [nrows, Hq] m (base 2) and l, from
  // k_near_attn; the kernel adds the list's entries outside the near set
  const float* near_o;
  const float* near_m;
  const float* near_l;
  int64_t q_start, n_sink, window;
  int64_t nrows_launch;  // rows per launch (launch parity = row0 / nrows_launch)
};

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// Transposing LDS read (gfx950): within each 16-lane group, lane l receives
// element (l & 3) of the 8-byte words read by lanes (l >> 2) + 4j, j = 0..3.
// With lane s of the group pointing at row r0 + (s >> 2), column c0 + 4 (s & 3)
// of a row-major 16-bit matrix, lane l gets column c0 + l of rows r0 .. r0+3.
__device__ __forceinline__ uint2 ds_read_tr16(const uint16_t* p) {
  v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p));
  return __builtin_bit_cast(uint2, r);
}

// ---------------------------------------------------------------------------
// bf16 attention, register staged.  Every wave owns one (row, KV head) and
// streams that head's K and V rows (256 B each per token) on its own: no
// barrier inside the loop.  HKV is the number of KV heads (0: any, read from
// the arguments; 4, the shape of the 128K .. 10M workloads, as a constant).
// Two workgroup shapes (NW waves per workgroup):
//   NW = 4 (HKV = 4): one row per workgroup, wave w takes KV head w.  The
//     four waves read each listed token's whole 1 KiB K and V rows together,
//     the better pattern once K/V are much larger than the caches (1M, 10M
//     tokens).
//   NW = 1: one (row, head) per workgroup.  When the head count divides 8,
//     the XCD that a workgroup runs on (blockIdx.x mod 8) fixes its head:
//     XCDs h, h + Hkv, ... serve KV head h, each for its share of the
//     launch's rows.  Each XCD's L2 then holds one head's rows for many
//     neighbouring queries, which pays when K/V fit the Infinity Cache (the
//     128K workload: 128 MiB each, XCDs h and h + 4 per head, a quarter of
//     the bytes per token for four times as many queries as with NW = 4).
// Tiles of 16 tokens are loaded with 16-byte loads, each instruction reading
// four tokens' whole 256 B head rows (whole cache lines), into a ring of
// kRing4 register buffers, kRing4 - 1 tiles ahead of the one being computed,
// so each wave keeps 16 KiB in flight.  K and V then go to per-wave LDS
// tiles.  The products are taken transposed, S^T = K Q^T and O^T = V^T P^T,
// so that the scores come out with one head per lane column and four keys
// per lane, which is the layout of P^T as an MFMA operand: P stays in
// registers.  The K tile's 16-byte chunks are XOR swizzled by row
// (chunk ^ row) so that the reads of the K operands (16x16x32 MFMAs; for
// product j, lane (key n, u) takes bytes [16 (4j + u), +16) of key n, and Q
// uses the same dim order) hit distinct banks; the V tile's chunks are
// swizzled by chunk ^ 2 (row & 7) for the transposing reads of V^T.  Loading
// K straight into the MFMA layout instead (16 keys x 64 B per instruction,
// two requests per cache line) made the loop bound by L2 requests.  The
// loop runs whole ring cycles: tiles at or past the end, and invalid list
// entries, load token 0 with zero weight.
// The row's index list is staged in LDS, kList4<NW> entries at a time, each
// entry checked once there: invalid entries, and the tail of the last tile
// past the count, are stored as -1, and 16 more -1 entries after the stage
// serve the padding tiles.  In the loop an entry e < 0 loads token 0 and
// gets zero weight.
//
// Softmax in base 2 with a lazy reference max m per head row: the O and l
// accumulators are rescaled only when a score exceeds m by more than 2^kLazy
// (O and l always share the reference, so the result does not depend on
// when this happens); l is summed per lane and reduced once at the end.
constexpr int kRing4 = 3;                      // register buffers per wave
constexpr int kVTile4 = 16 * 256;              // K or V tile of one KV head in LDS (bytes)
constexpr int kWave4 = 2 * kVTile4;            // LDS of one wave: V tile, K tile
// index-list entries staged at a time, and per thread in one batch of loads;
// with NW = 1, 2,816 entries let eight workgroups share a CU's 160 KiB
template <int NW> constexpr int kList4 = NW == 4 ? 8192 : 2816;
template <int NW> constexpr int kBatch4 = NW == 4 ? 12 : 44;
template <int NW> constexpr int kLds4 = NW * kWave4 + (kList4<NW> + 16) * 4;
static_assert(8 * kLds4<1> <= 160 * 1024 && 2 * kLds4<4> <= 160 * 1024, "LDS per CU");
static_assert(kBatch4<1> * 64 == kList4<1>, "one batch stages a whole chunk");
// K and V caches of at most this many bytes each (B * Tmax * Hkv * D * 2)
// take the per-head workgroups.  Measured against one workgroup per row: 23%
// less attention time at 128 MiB (128K tokens), 6-7% more at 1 GiB and
// beyond (1M and 10M tokens, 16 x 1M decode); sizes in between were not
// measured.
constexpr int64_t kHeadMajorMaxKvBytes = 256ll << 20;
constexpr float kLazy = 8.f;

typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// two floats -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// NW = 1 with hkv KV heads: whether each XCD serves one head (hkv divides 8)
__host__ __device__ constexpr bool xcd_per_head(int hkv, int64_t nrows) {
  return nrows >= 8 && hkv <= 8 && 8 % hkv == 0;
}

// grid.x of a launch of nrows rows
template <int NW>
int64_t attn_grid(int hkv, int64_t nrows) {
  if (NW == 4) return nrows >= 8 ? (nrows + 7) / 8 * 8 : nrows;
  if (xcd_per_head(hkv, nrows)) return 8 * ((nrows + 8 / hkv - 1) / (8 / hkv));
  return hkv * nrows;
}

template <int NW, int HKV, bool NEAR = false>
__global__ __launch_bounds__(64 * NW, 2) void k_attn_bf16(AttnArgs a) {
  static_assert(NW == 1 || HKV == 4, "one workgroup per row is written for four KV heads");
  extern __shared__ __attribute__((aligned(16))) char lds4[];
  constexpr int NT = 64 * NW, kList = kList4<NW>, kB = kBatch4<NW>;
  const int hkv = HKV ? HKV : a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6);
  // with 8+ rows, workgroups of consecutive rows (which share many keys) go
  // to the same XCD; with fewer rows the splits of a row spread over the XCDs
  int64_t row;
  int kvh;
  if constexpr (NW == 4) {
    row = blockIdx.x;
    kvh = wave;
    if (a.nrows >= 8) {
      const int64_t per_xcd = (a.nrows + 7) / 8;
      row = (int64_t)(blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    }
  } else if (xcd_per_head(hkv, a.nrows)) {
    const int x = blockIdx.x & 7, parts = 8 / hkv;
    kvh = x % hkv;
    row = (int64_t)(x / hkv) * ((a.nrows + parts - 1) / parts) + (blockIdx.x >> 3);
  } else {
    row = blockIdx.x / hkv;
    kvh = blockIdx.x % hkv;
  }
  // every wave of the workgroup has the same row, so the return is uniform
  if (row >= a.nrows) return;
  // list stages are written by one wave (NW = 1) or by the whole workgroup
  auto stage_sync = [] {
    if constexpr (NW == 1) wave_fence(); else __syncthreads();
  };
  row += a.row0;
  const int split = blockIdx.y;
  const int64_t b = row / a.Tq;
  // split ranges come from the list capacity, so the list can be staged while
  // the row's count is still in flight; the count only trims the range
  const int per = (a.L + a.splits - 1) / a.splits;
  const int k0 = split * per;
  const int kend = (k0 + per) < a.L ? (k0 + per) : a.L;
  const int navail = kend > k0 ? kend - k0 : 0;
  int cnt = a.count[row];
  cnt = cnt < 0 ? 0 : (cnt > a.L ? a.L : cnt);
  const int k1 = kend < cnt ? kend : cnt;
  const int n = k1 > k0 ? k1 - k0 : 0;
  const int32_t* lst = a.idx + row * (int64_t)a.L + k0;
  // one token's K (or V) row holds all hkv heads: 256 B each
  const uint64_t tok = (uint64_t)hkv * 256;
  const char* kb = reinterpret_cast<const char*>(a.k + b * a.Tmax * hkv * kHeadDim) + kvh * 256;
  const char* vb = reinterpret_cast<const char*>(a.v + b * a.Tmax * hkv * kHeadDim) + kvh * 256;
  char* vt = lds4 + wave * kWave4;
  char* kt = vt + kVTile4;
  int32_t* slist = reinterpret_cast<int32_t*>(lds4 + NW * kWave4);
  const int r16 = lane & 15, u = lane >> 4;
  // token indices below tlim are valid (unsigned compare rejects e < 0)
  const uint32_t tlim = a.Tmax < 0x7fffffff ? (uint32_t)a.Tmax : 0x7fffffffu;

  // the first batch of list entries is requested before anything else: the
  // tiles' addresses wait on it
  const int m0 = navail < kList ? navail : kList;      // entries of the first chunk
  int32_t t0[kB];
  if constexpr (!NEAR) {
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int i = tid + NT * u;
      t0[u] = i < m0 ? lst[i] : 0;
    }
  }
  // a negative scale is applied as |scale| to -q (flipping bf16 sign bits is
  // exact), so the threshold test below can compare raw scores
  const float sl = fabsf(a.scale_log2), inv_sl = 1.f / sl;
  bf16x8 qf[4];
  {
    const bool ok = r16 < a.G;
    const uint32_t flip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
    const u32x4_t* qrow = reinterpret_cast<const u32x4_t*>(
        a.q + (row * a.Hq + (int64_t)kvh * a.G + (ok ? r16 : 0)) * kHeadDim);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4_t w = ok ? qrow[4 * j + u] : u32x4_t{0, 0, 0, 0};
      qf[j] = __builtin_bit_cast(bf16x8, w ^ flip);
    }
  }
  f32x4 o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // lane (head r16, u): m, the head's reference max (uniform over the head's
  // four lanes), with a finite floor so that exp2(-inf - m) = 0; mth, the raw
  // score above which a key moves the reference (m + 2^kLazy); lp, this
  // lane's partial sum over its keys 4u .. 4u + 3 of every tile
  float m = -1e30f, lp = 0.f, mth = -__builtin_inff();
  // far-key mode: the query's position p and its near set [0, s_end) and
  // [w_start, p]; the state starts from the near set's softmax state
  int64_t p = 0, s_end = 0, w_start = 0;
  // several waves per row (the one-workgroup-per-row layout): no near state;
  // the near keys are gathered like the far ones, staged after the list's
  // entries. One wave per row: the state comes from the near kernel.
  constexpr bool kInlineNear = NEAR && NW > 1;
  int nn = 0;                                   // near keys appended
  if constexpr (NEAR) {
    p = a.q_start + (row - b * a.Tq);
    s_end = p + 1 < a.n_sink ? p + 1 : a.n_sink;
    w_start = p - a.window + 1 > 0 ? p - a.window + 1 : 0;
    if constexpr (kInlineNear) nn = (int)(w_start <= s_end ? p + 1 : s_end + (p - w_start + 1));
    if (!kInlineNear && r16 < a.G) {
      const int64_t slot = (row - a.row0) * a.Hq + (int64_t)kvh * a.G + r16;
      const float4* po = reinterpret_cast<const float4*>(a.near_o + slot * kHeadDim + 4 * u);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float4 x = po[4 * j];
        o[j] = f32x4{x.x, x.y, x.z, x.w};
      }
      m = a.near_m[slot];
      lp = u == 0 ? a.near_l[slot] : 0.f;
      mth = (m + kLazy) * inv_sl;
    }
  }

  const int vi = lane >> 4, vc = lane & 15;    // V loads: token 4 vi + j, chunk vc
  // transposing V reads: source lane s of a 16-lane group points at key row
  // 4u + (s >> 2), dims 16j + 4 (s & 3) .. +3 (byte 8 (s & 1) of chunk 2j + cv);
  // lane (r16, u) receives dim 16j + r16 of keys 4u .. 4u + 3
  const int sk = 4 * u + (r16 >> 2), cv = (r16 & 3) >> 1, sw = 2 * (sk & 7);
  const char* vrd = vt + 256 * sk + 8 * (r16 & 1);

  u32x4_t kr[kRing4][4], vr[kRing4][4];
  uint32_t kval[kRing4];                       // bit i: key 4u + i of the tile is real
  // slot i of a stage holding cn entries: the entry if it is valid, else -1
  auto put = [&](int i, int32_t e, int cn) {
    slist[i] = (i < cn && (uint32_t)e < tlim) ? e : -1;
  };
  // list entries [c0 + from, c0 + m) into slist, slots up to the next
  // multiple of 16: every load of a batch is issued before the stores, one
  // memory latency per NT * kB entries
  auto stage = [&](int c0, int from, int m, int cn) {
    const int m16 = (m + 15) & ~15;
    for (int base = from; base < m16; base += NT * kB) {
      int32_t t[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int i = base + tid + NT * u;
        t[u] = i < m ? lst[c0 + i] : -1;
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int i = base + tid + NT * u;
        if (i < m16) put(i, t[u], cn);
      }
    }
  };
  // far-key mode: entries [c0, c0 + cn) that are valid and outside the near
  // set, compacted into the stage in list order (each wave takes a
  // contiguous run of a batch; the runs' counts give the waves' offsets);
  // returns the number kept and pads the last tile with -1
  __shared__ int s_wcnt[NW];
  // far-key mode reads each list from its end in every other round of
  // workgroups (and every other launch): lists are sorted by position, so the
  // rows in flight sweep K/V together, and a round that starts where the last
  // one ended finds those rows still in the caches
  const bool rev = NEAR && ((((int64_t)blockIdx.x * 2 >= gridDim.x) ? 1 : 0) ^
                            (int)((a.row0 / a.nrows_launch) & 1));
  auto stage_far = [&](int c0, int cn) -> int {
    // a list entry is kept when valid and outside the near set; appended near
    // keys are always kept
    auto far = [&](int32_t x) {
      const int64_t e = x;
      return (uint32_t)x < tlim && !(e < s_end || (e >= w_start && e <= p));
    };
    int kept = 0;
    for (int base = 0; base < cn; base += NT * kB) {
      int32_t t[kB];
      uint64_t km = 0;                                     // inline near: bit u, t[u] is kept
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int v = c0 + base + wave * 64 * kB + 64 * u + lane;   // staged entry
        const bool in = v < c0 + cn;
        if constexpr (kInlineNear) {
          // the list's entries (from the end with rev), then near key v - n
          const int j = v - n;
          if (!in) t[u] = -1;
          else if (v < n) t[u] = lst[rev ? n - 1 - v : v];
          else t[u] = (int32_t)(w_start <= s_end || j < s_end ? j : w_start + (j - s_end));
          km |= (uint64_t)(in && (v >= n || far(t[u]))) << u;
        } else {
          t[u] = in ? lst[rev ? n - 1 - v : v] : -1;
        }
      }
      auto keep = [&](int u) {
        if constexpr (kInlineNear) return ((km >> u) & 1ull) != 0;
        else return far(t[u]);
      };
      int off = kept, total = 0;
      if constexpr (NW > 1) {
        // the waves' counts first (the ballots are taken again for the stores)
        int wc = 0;
#pragma unroll
        for (int u = 0; u < kB; ++u) wc += __popcll(__ballot(keep(u)));
        if (lane == 0) s_wcnt[wave] = wc;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          off += w < wave ? s_wcnt[w] : 0;
          total += s_wcnt[w];
        }
        __syncthreads();
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const bool k = keep(u);
        const uint64_t bal = __ballot(k);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
        if (k) slist[off + (int)below] = t[u];
        off += __popcll(bal);
      }
      kept += NW > 1 ? total : off - kept;
    }
    for (int i = kept + tid; i < ((kept + 15) & ~15); i += NT) slist[i] = -1;
    return kept;
  };
  if (tid < 16) slist[kList + tid] = -1;
  // the first chunk's loads do not wait for the count (the stores do)
  if constexpr (!NEAR) {
    const int cn = n < kList ? n : kList;
    const int m16 = (m0 + 15) & ~15;
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int i = tid + NT * u;
      if (i < m16) put(i, t0[u], cn);
    }
    stage(0, NT * kB, m0, cn);
  }
  stage_sync();
  const int nv = n + nn;                          // staged entries (list, then near keys)
  for (int c0 = 0; c0 < nv; c0 += kList) {
    int cn = (nv - c0) < kList ? (nv - c0) : kList;
    if constexpr (NEAR) {
      stage_sync();                            // every wave is done with the previous chunk
      cn = stage_far(c0, cn);
      stage_sync();
    } else if (c0 > 0) {
      stage_sync();                            // every wave is done with the previous chunk
      stage(c0, 0, cn, cn);
      stage_sync();
    }
    const int nt = (cn + 15) >> 4;

    // tile T into one ring buffer; kv: which of keys 4u .. 4u + 3 are real
    // (the entries this lane also loads V rows for: vi = u)
    auto issue = [&](int T, u32x4_t (&k)[4], u32x4_t (&v)[4], uint32_t& kv) {
      const int tr = T < nt ? T << 4 : kList;  // padding tiles read the -1 entries
      const int4 p4 = *reinterpret_cast<const int4*>(slist + tr + 4 * vi);
      kv = (p4.x >= 0 ? 1u : 0u) | (p4.y >= 0 ? 2u : 0u) | (p4.z >= 0 ? 4u : 0u) |
           (p4.w >= 0 ? 8u : 0u);
      // load j: token 4 vi + j, chunk vc of its K and V head rows
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = j == 0 ? p4.x : (j == 1 ? p4.y : (j == 2 ? p4.z : p4.w));
        const uint64_t off = (uint64_t)(uint32_t)(p > 0 ? p : 0) * tok + 16 * vc;
        k[j] = *reinterpret_cast<const u32x4_t*>(kb + off);
        v[j] = *reinterpret_cast<const u32x4_t*>(vb + off);
      }
    };
    auto compute = [&](const u32x4_t (&k)[4], const u32x4_t (&v)[4], uint32_t kv) {
      // the K tile's reads enter the LDS queue right behind its writes, and
      // the V tile is written while the K Q^T products run
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = 4 * vi + j;
        *reinterpret_cast<u32x4_t*>(kt + 256 * rr + 16 * (vc ^ rr)) = k[j];
      }
      wave_fence();
      // S^T = K Q^T: row = key 4u + i, column = head r16
      u32x4_t kf[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        kf[j] = *reinterpret_cast<const u32x4_t*>(kt + 256 * r16 + 16 * ((4 * j + u) ^ r16));
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[j]), qf[j], sacc, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = 4 * vi + j;
        *reinterpret_cast<u32x4_t*>(vt + 256 * rr + 16 * (vc ^ (2 * (rr & 7)))) = v[j];
      }
      bool grow = false;
#pragma unroll
      for (int i = 0; i < 4; ++i) grow |= ((kv >> i) & 1u) && sacc[i] > mth;
      if (__ballot(grow)) {
        // the head's max over the tile: this lane's keys, then its 4 lanes
        float x = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if ((kv >> i) & 1u) x = fmaxf(x, sacc[i] * sl);
        x = fmaxf(x, __shfl_xor(x, 16, 64));
        x = fmaxf(x, __shfl_xor(x, 32, 64));
        const float mn = fmaxf(m, x);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        lp *= alpha;
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[j][i] *= alpha;
        m = mn;
        mth = (mn + kLazy) * inv_sl;
      }
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = ((kv >> i) & 1u) ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], sl, -m)) : 0.f;
        lp += pv[i];
      }
      // P^T as the B operand of 16x16x16 MFMAs: lane (head r16, u), keys 4u .. 4u + 3
      uint2 w2;
      w2.x = pack_bf16x2(pv[0], pv[1]);
      w2.y = pack_bf16x2(pv[2], pv[3]);
      const v4s_t pb4 = __builtin_bit_cast(v4s_t, w2);
      // O^T += V^T P^T: A = V^T (dim 16j + r16, keys 4u .. 4u + 3)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const v4s_t va4 = __builtin_bit_cast(
            v4s_t, ds_read_tr16(reinterpret_cast<const uint16_t*>(vrd + 16 * ((2 * j + cv) ^ sw))));
        o[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va4, pb4, o[j], 0, 0, 0);
      }
      wave_fence();
    };

    // The compiler derives each wait from the load order, so the prologue's
    // tiles are pinned in ring order; every cycle then issues tile t + 2 and
    // computes tile t, with two tiles (16 loads per lane) still in flight.
    static_assert(kRing4 == 3, "the ring cycle below is written out for three buffers");
    issue(0, kr[0], vr[0], kval[0]);
    __builtin_amdgcn_sched_barrier(0);
    issue(1, kr[1], vr[1], kval[1]);
    __builtin_amdgcn_sched_barrier(0);
    for (int t0 = 0; t0 < nt; t0 += kRing4) {
      issue(t0 + 2, kr[2], vr[2], kval[2]);
      compute(kr[0], vr[0], kval[0]);
      issue(t0 + 3, kr[0], vr[0], kval[0]);
      compute(kr[1], vr[1], kval[1]);
      issue(t0 + 4, kr[1], vr[1], kval[1]);
      compute(kr[2], vr[2], kval[2]);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);        // vmcnt(0): the padding tiles' loads retired
  }
  // the head's sum over its four lanes
  float l = lp;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  // write: lane (head r16 < G, u) holds O^T rows 16j + 4u + i, i = 0..3
  if (r16 < a.G) {
    const int64_t h = (int64_t)kvh * a.G + r16;
    if (a.splits == 1) {
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t* orow = a.out + (row * a.Hq + h) * kHeadDim + 4 * u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint2 w;
        w.x = pack_bf16x2(o[j][0] * inv, o[j][1] * inv);
        w.y = pack_bf16x2(o[j][2] * inv, o[j][3] * inv);
        *reinterpret_cast<uint2*>(orow + 16 * j) = w;
      }
    } else {
      const int64_t slot = row * a.splits + split;
      float* ob = a.ws;
      float* mb = a.ws + a.rows * a.splits * a.Hq * kHeadDim;
      float* lb = mb + a.rows * a.splits * a.Hq;
      float* orow = ob + (slot * a.Hq + h) * kHeadDim + 4 * u;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        *reinterpret_cast<float4*>(orow + 16 * j) = make_float4(o[j][0], o[j][1], o[j][2], o[j][3]);
      // running max back to natural-log units for the combine step
      if (u == 0) { mb[slot * a.Hq + h] = m * 0.6931471805599453f; lb[slot * a.Hq + h] = l; }
    }
  }
}

// fp32 path: one wave per (query row, head).  Lane j scores key t0 + j; the
// output dims are split two per lane.
struct AttnArgsF32 {
  const float* q;
  const float* k;
  const float* v;
  const int32_t* idx;
  const int32_t* count;
  float* out;
  float* ws;
  int64_t rows, Tq, Tmax;
  int32_t Hq, Hkv, L, splits;
  float scale;
};

__global__ __launch_bounds__(64) void k_attn_f32(AttnArgsF32 a) {
  __shared__ float qs[kHeadDim];
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x / a.Hq;
  const int h = blockIdx.x % a.Hq;
  const int split = blockIdx.y;
  const int kvh = h * a.Hkv / a.Hq;
  const int64_t b = row / a.Tq;
  int cnt = a.count[row];
  cnt = cnt < 0 ? 0 : (cnt > a.L ? a.L : cnt);
  const int per = (cnt + a.splits - 1) / a.splits;
  const int k0 = split * per;
  const int k1 = (k0 + per) < cnt ? (k0 + per) : cnt;
  const int32_t* lst = a.idx + row * (int64_t)a.L;
  const float* qrow = a.q + (row * a.Hq + h) * kHeadDim;
  qs[lane] = qrow[lane];
  qs[lane + 64] = qrow[lane + 64];
  __syncthreads();
  float m = -__builtin_inff(), l = 0.f, o0 = 0.f, o1 = 0.f;
  for (int t0 = k0; t0 < k1; t0 += 64) {
    const int i = t0 + lane;
    int32_t pj = i < k1 ? lst[i] : -1;
    pj = pj < a.Tmax ? pj : -1;
    float s = -__builtin_inff();
    if (pj >= 0) {
      const float4* kr = reinterpret_cast<const float4*>(a.k + ((b * a.Tmax + pj) * a.Hkv + kvh) * kHeadDim);
      float acc = 0.f;
#pragma unroll 8
      for (int d = 0; d < kHeadDim / 4; ++d) {
        const float4 kv = kr[d];
        acc = __builtin_fmaf(qs[4 * d], kv.x, acc);
        acc = __builtin_fmaf(qs[4 * d + 1], kv.y, acc);
        acc = __builtin_fmaf(qs[4 * d + 2], kv.z, acc);
        acc = __builtin_fmaf(qs[4 * d + 3], kv.w, acc);
      }
      s = acc * a.scale;
    }
    float mx = s;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    const float mn = fmaxf(m, mx);
    const float alpha = mn == -__builtin_inff() ? 1.f : __expf(m - mn);
    const float p = pj >= 0 ? __expf(s - mn) : 0.f;
    float rs = p;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) rs += __shfl_xor(rs, off, 64);
    l = l * alpha + rs;
    m = mn;
    o0 *= alpha;
    o1 *= alpha;
    const int nk = (k1 - t0) < 64 ? (k1 - t0) : 64;
    for (int j = 0; j < nk; ++j) {
      const float pjv = __shfl(p, j, 64);
      const int32_t pos = __shfl(pj, j, 64);
      if (pos < 0) continue;
      const float2 vv = reinterpret_cast<const float2*>(a.v + ((b * a.Tmax + pos) * a.Hkv + kvh) * kHeadDim)[lane];
      o0 = __builtin_fmaf(pjv, vv.x, o0);
      o1 = __builtin_fmaf(pjv, vv.y, o1);
    }
  }
  if (a.splits == 1) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    reinterpret_cast<float2*>(a.out + (row * a.Hq + h) * kHeadDim)[lane] = make_float2(o0 * inv, o1 * inv);
  } else {
    const int64_t slot = row * a.splits + split;
    float* ob = a.ws;
    float* mb = a.ws + a.rows * a.splits * a.Hq * kHeadDim;
    float* lb = mb + a.rows * a.splits * a.Hq;
    reinterpret_cast<float2*>(ob + (slot * a.Hq + h) * kHeadDim)[lane] = make_float2(o0, o1);
    if (lane == 0) { mb[slot * a.Hq + h] = m; lb[slot * a.Hq + h] = l; }
  }
}

// Combine split partials: out = sum_s e^(m_s - M) O_s / sum_s e^(m_s - M) l_s.
// One workgroup per (row, head, 64-dim half): thread t owns dims
// 4 (t % 16) .. +3 of the half and splits t / 16, t / 16 + 16, ...; each
// thread keeps its sums relative to its own running max (loads of four
// splits in flight at a time), and the 16 split groups meet in LDS.
template <int DT>
__global__ __launch_bounds__(256) void k_attn_combine(const float* __restrict__ ws, void* out,
                                                      int64_t rows, int32_t Hq, int32_t splits) {
  __shared__ float s_m[16];
  __shared__ float s_den[16];
  __shared__ float4 s_num[16][16];
  const int64_t rhh = blockIdx.x;          // (row * Hq + h) * 2 + half
  const int64_t rh = rhh >> 1;
  const int hf = (int)(rhh & 1);
  const int64_t row = rh / Hq;
  const int h = (int)(rh % Hq);
  const int c = threadIdx.x & 15, g = threadIdx.x >> 4;
  const float* ob = ws;
  const float* mb = ws + rows * splits * Hq * kHeadDim;
  const float* lb = mb + rows * splits * Hq;
  float mg = -__builtin_inff(), den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = g; s0 < splits; s0 += 64) {
    float m[4], lv[4];
    float4 o[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sp = s0 + 16 * u;
      const int64_t slot = row * splits + (sp < splits ? sp : 0);
      m[u] = sp < splits ? mb[slot * Hq + h] : -__builtin_inff();
      lv[u] = lb[slot * Hq + h];
      o[u] = reinterpret_cast<const float4*>(ob + (slot * Hq + h) * kHeadDim + 64 * hf)[c];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (m[u] == -__builtin_inff()) continue;   // no keys in this split
      const float mn = fmaxf(mg, m[u]);
      const float a = __expf(mg - mn), w = __expf(m[u] - mn);   // mg = -inf gives a = 0
      num.x = num.x * a + w * o[u].x;
      num.y = num.y * a + w * o[u].y;
      num.z = num.z * a + w * o[u].z;
      num.w = num.w * a + w * o[u].w;
      den = den * a + w * lv[u];
      mg = mn;
    }
  }
  if (c == 0) { s_m[g] = mg; s_den[g] = den; }
  s_num[g][c] = num;
  __syncthreads();
  if (threadIdx.x < 64) {
    const int cc = threadIdx.x >> 2, e = threadIdx.x & 3;
    float M = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < 16; ++i) M = fmaxf(M, s_m[i]);
    float nn = 0.f, dd = 0.f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float w = s_m[i] == -__builtin_inff() ? 0.f : __expf(s_m[i] - M);
        const float4 v = s_num[i][cc];
        nn = __builtin_fmaf(w, e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w)), nn);
        dd = __builtin_fmaf(w, s_den[i], dd);
      }
    }
    const float r = dd > 0.f ? nn / dd : 0.f;
    const int64_t oi = rh * kHeadDim + 64 * hf + threadIdx.x;
    if (DT == LSA_BF16) reinterpret_cast<uint16_t*>(out)[oi] = f32_to_bf16_rne(r);
    else reinterpret_cast<float*>(out)[oi] = r;
  }
}

}  // namespace

int64_t attention_launch_rows() { return kRowsPerLaunch; }

bool attention_head_major(int32_t B, int64_t Tmax, int32_t Hkv, int32_t D, int dtype) {
  if (dtype != LSA_BF16 || Hkv <= 0 || D != kHeadDim || B < 0 || Tmax < 0) return false;
  // one workgroup per row exists for four KV heads only
  if (Hkv != 4 || B == 0 || Tmax == 0) return true;
  const int64_t per_token = (int64_t)Hkv * D * 2;   // bytes of one token's row
  return Tmax <= kHeadMajorMaxKvBytes / per_token / B;
}

hipError_t launch_attention(const void* q, const void* k, const void* v, int32_t B, int64_t Tq,
                            int64_t Tmax, int32_t Hq, int32_t Hkv, const int32_t* idx,
                            const int32_t* count, int32_t L_max, float scale, int dtype,
                            int32_t splits, void* out, float* ws, hipStream_t s) {
  const int64_t rows = (int64_t)B * Tq;
  if (rows <= 0) return hipSuccess;
  if (dtype == LSA_BF16) {
    AttnArgs a;
    a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
    a.idx = idx; a.count = count; a.out = (uint16_t*)out; a.ws = ws;
    a.rows = rows; a.Tq = Tq; a.Tmax = Tmax; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
    a.L = L_max; a.splits = splits; a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.near_o = a.near_m = a.near_l = nullptr;
    a.q_start = a.n_sink = a.window = 0;
    a.nrows_launch = kRowsPerLaunch;
    static bool attr_set = false;
    if (!attr_set) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_attn_bf16<4, 4>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, kLds4<4>);
      (void)hipGetLastError();  // advisory; never report it as a launch failure
      attr_set = true;
    }
    const bool head_major = attention_head_major(B, Tmax, Hkv, kHeadDim, dtype);
    for (int64_t r0 = 0; r0 < rows; r0 += kRowsPerLaunch) {
      a.row0 = r0;
      a.nrows = (rows - r0) < kRowsPerLaunch ? (rows - r0) : kRowsPerLaunch;
      if (Hkv != 4)
        hipLaunchKernelGGL((k_attn_bf16<1, 0>), dim3((unsigned)attn_grid<1>(Hkv, a.nrows),
                           (unsigned)splits), dim3(64), (size_t)kLds4<1>, s, a);
      else if (head_major)
        hipLaunchKernelGGL((k_attn_bf16<1, 4>), dim3((unsigned)attn_grid<1>(4, a.nrows),
                           (unsigned)splits), dim3(64), (size_t)kLds4<1>, s, a);
      else
        hipLaunchKernelGGL((k_attn_bf16<4, 4>), dim3((unsigned)attn_grid<4>(4, a.nrows),
                           (unsigned)splits), dim3(256), (size_t)kLds4<4>, s, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  } else {
    AttnArgsF32 a;
    a.q = (const float*)q; a.k = (const float*)k; a.v = (const float*)v;
    a.idx = idx; a.count = count; a.out = (float*)out; a.ws = ws;
    a.rows = rows; a.Tq = Tq; a.Tmax = Tmax; a.Hq = Hq; a.Hkv = Hkv; a.L = L_max;
    a.splits = splits; a.scale = scale;
    hipLaunchKernelGGL(k_attn_f32, dim3((unsigned)(rows * Hq), (unsigned)splits), dim3(64), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  if (dtype == LSA_BF16)
    hipLaunchKernelGGL(k_attn_combine<LSA_BF16>, dim3((unsigned)(rows * Hq * 2)), dim3(256), 0, s,
                       ws, out, rows, Hq, splits);
  else
    hipLaunchKernelGGL(k_attn_combine<LSA_F32>, dim3((unsigned)(rows * Hq * 2)), dim3(256), 0, s,
                       ws, out, rows, Hq, splits);
  return hipGetLastError();
}

// the near kernel runs over groups of this many rows (launches of the gather
// kernel), so that it fills the chip; its state for a group stays in the
// workspace until the group's gathers have read it
constexpr int64_t kNearGroupLaunches = 4;

int64_t near_state_bytes(int64_t rows, int32_t Hq) {
  const int64_t g = kRowsPerLaunch * kNearGroupLaunches;
  const int64_t r = rows < g ? rows : g;
  return r * Hq * ((int64_t)kHeadDim + 2) * 4;
}

hipError_t launch_attention_prefill(const void* q, const void* k, const void* v, int32_t B,
                                    int64_t Tq, int64_t q_start, int64_t Tmax, int32_t Hq,
                                    int32_t Hkv, const int32_t* idx, const int32_t* count,
                                    int32_t L_max, int64_t n_sink, int64_t window, float scale,
                                    void* out, float* ws, hipStream_t s) {
  const int64_t rows = (int64_t)B * Tq;
  if (rows <= 0) return hipSuccess;
  const int64_t group = kRowsPerLaunch * kNearGroupLaunches;
  const int64_t grows = rows < group ? rows : group;   // rows of the near state
  AttnArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.idx = idx; a.count = count; a.out = (uint16_t*)out; a.ws = nullptr;
  a.rows = rows; a.Tq = Tq; a.Tmax = Tmax; a.Hq = Hq; a.Hkv = Hkv; a.G = Hq / Hkv;
  a.L = L_max; a.splits = 1; a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  // near state of a group's rows: O [grows, Hq, 128], then m, then l
  float* po = ws;
  float* pm = po + grows * Hq * kHeadDim;
  float* pl = pm + grows * Hq;
  a.q_start = q_start; a.n_sink = n_sink; a.window = window;
  a.nrows_launch = kRowsPerLaunch;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_attn_bf16<4, 4, true>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kLds4<4>);
    (void)hipGetLastError();  // advisory; never report it as a launch failure
    attr_set = true;
  }
  const bool head_major = attention_head_major(B, Tmax, Hkv, kHeadDim, LSA_BF16);
  // One workgroup per row (K/V beyond the Infinity Cache): the near keys are
  // gathered with the far ones (the window's rows are cache hits either way,
  // and a separate near pass measured slower there); otherwise the near
  // kernel takes them dense per tile of rows.
  const bool near_pass = Hkv != 4 || head_major;
  for (int64_t g0 = 0; g0 < rows; g0 += group) {
    const int64_t gn = (rows - g0) < group ? (rows - g0) : group;
    hipError_t e = hipSuccess;
    if (near_pass) {
      e = launch_near_attention(q, k, v, g0, gn, Tq, q_start, Tmax, Hq, Hkv, n_sink, window, scale,
                                po, pm, pl, s);
      if (e != hipSuccess) return e;
    }
    for (int64_t r0 = g0; r0 < g0 + gn; r0 += kRowsPerLaunch) {
      a.row0 = r0;
      a.nrows = (g0 + gn - r0) < kRowsPerLaunch ? (g0 + gn - r0) : kRowsPerLaunch;
      // the launch's rows start (r0 - g0) rows into the group's state
      const int64_t off = (r0 - g0) * Hq;
      a.near_o = near_pass ? po + off * kHeadDim : nullptr;
      a.near_m = near_pass ? pm + off : nullptr;
      a.near_l = near_pass ? pl + off : nullptr;
      if (Hkv != 4)
        hipLaunchKernelGGL((k_attn_bf16<1, 0, true>), dim3((unsigned)attn_grid<1>(Hkv, a.nrows)),
                           dim3(64), (size_t)kLds4<1>, s, a);
      else if (head_major)
        hipLaunchKernelGGL((k_attn_bf16<1, 4, true>), dim3((unsigned)attn_grid<1>(4, a.nrows)),
                           dim3(64), (size_t)kLds4<1>, s, a);
      else
        hipLaunchKernelGGL((k_attn_bf16<4, 4, true>), dim3((unsigned)attn_grid<4>(4, a.nrows)),
                           dim3(256), (size_t)kLds4<4>, s, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace lsa
