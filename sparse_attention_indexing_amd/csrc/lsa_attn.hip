// Gather softmax attention over per-query key lists.
//
// [visual "Intro", "What one query actually does"]: after selection,
// ordinary attention runs over the sinks, the selected keys and the window,
// and one index list per query is shared by all of its attention heads.
//
// bf16 path: one workgroup per query row (and split), one wave per KV head.
// The GQA group of G <= 16 query heads forms the M side of 16x16x32 bf16
// MFMAs, so every gathered K/V row (256 B per KV head) is read once for the
// whole group.  Keys are processed 32 at a time: K rows are loaded straight
// into MFMA operand registers (64 contiguous bytes per lane), V rows are
// staged in LDS and read back with keys along the reduction dimension.
// Online softmax in fp32; P is rounded to bf16 for the PV product.
#include "lsa_internal.h"

namespace lsa {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kKT = 32;          // keys per tile
constexpr int kVStride = 136;    // LDS row stride (bf16) of the staged V tile
constexpr int kPStride = 40;     // LDS row stride (bf16) of P
constexpr int kMaxWaves = 4;

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
  int64_t Tq, Tmax;
  int32_t Hq, Hkv, G, L, splits;
  float scale;
};

constexpr int kWaveLds = kKT * kVStride + 16 * kPStride;  // bf16 elements per wave

// K fragment of one key row for 16x16x32 MFMAs: dims [32u, 32u + 32) (64 B)
__device__ __forceinline__ void load_krow(uint4* w, const uint16_t* base, int u) {
  const uint4* src = reinterpret_cast<const uint4*>(base + 32 * u);
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = src[j];
}
// half a V row: dims [64h, 64h + 64) (128 B), kept in eight named registers
struct VHalf {
  uint4 r0, r1, r2, r3, r4, r5, r6, r7;
};
__device__ __forceinline__ VHalf load_vhalf(const uint16_t* base, int h) {
  const uint4* src = reinterpret_cast<const uint4*>(base + 64 * h);
  VHalf v;
  v.r0 = src[0]; v.r1 = src[1]; v.r2 = src[2]; v.r3 = src[3];
  v.r4 = src[4]; v.r5 = src[5]; v.r6 = src[6]; v.r7 = src[7];
  return v;
}
__device__ __forceinline__ void store_vhalf(uint16_t* dst, const VHalf& v) {
  uint4* d = reinterpret_cast<uint4*>(dst);
  d[0] = v.r0; d[1] = v.r1; d[2] = v.r2; d[3] = v.r3;
  d[4] = v.r4; d[5] = v.r5; d[6] = v.r6; d[7] = v.r7;
}

// One workgroup per (query row, split); wave w handles KV heads w, w + nwaves, ...
// The row's index list is staged in LDS once.  Gathers are software
// pipelined: the K and V rows of tile t+1 are requested right after the QK^T
// products of tile t, so their latency overlaps the softmax and PV of tile t.
// Positions outside [0, Tmax) are skipped (masked to zero weight).
__global__ __launch_bounds__(64 * kMaxWaves, 3) void k_attn_bf16(AttnArgs a) {
  extern __shared__ uint16_t attn_lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int64_t row = blockIdx.x;
  const int split = blockIdx.y;
  const int64_t b = row / a.Tq;
  int cnt = a.count[row];
  cnt = cnt < 0 ? 0 : (cnt > a.L ? a.L : cnt);
  const int per = (cnt + a.splits - 1) / a.splits;
  const int k0 = split * per;
  const int k1 = (k0 + per) < cnt ? (k0 + per) : cnt;
  const int n = k1 > k0 ? k1 - k0 : 0;
  const int32_t* lst = a.idx + row * (int64_t)a.L + k0;
  int32_t* lst_s = reinterpret_cast<int32_t*>(attn_lds + nwaves * kWaveLds);
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int32_t v = lst[i];
    lst_s[i] = (v >= 0 && v < a.Tmax) ? v : -1;
  }
  __syncthreads();
  const int r16 = lane & 15, u = lane >> 4;
  const int kk = lane >> 1, hv = lane & 1;       // V staging: key kk, dims half hv
  uint16_t* vs = attn_lds + wave * kWaveLds;
  uint16_t* ps = vs + kKT * kVStride;
  const uint16_t* kbase = a.k + b * a.Tmax * a.Hkv * kHeadDim;
  const uint16_t* vbase = a.v + b * a.Tmax * a.Hkv * kHeadDim;

  for (int kvh = wave; kvh < a.Hkv; kvh += nwaves) {
    // Q fragment: head row r16 of the group, dims [32u + 8j, +8)
    bf16x8 qf[4];
    {
      const bool ok = r16 < a.G;
      const uint16_t* qrow = a.q + (row * a.Hq + (int64_t)kvh * a.G + (ok ? r16 : 0)) * kHeadDim + 32 * u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4 w = ok ? reinterpret_cast<const uint4*>(qrow)[j] : make_uint4(0, 0, 0, 0);
        qf[j] = __builtin_bit_cast(bf16x8, w);
      }
    }
    f32x4 o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) { m[i] = -__builtin_inff(); l[i] = 0.f; }

    auto pos_at = [&](int i) -> int32_t { return i < n ? lst_s[i] : -1; };
    auto row_of = [&](const uint16_t* base, int32_t p) {
      return base + ((int64_t)(p >= 0 ? p : 0) * a.Hkv + kvh) * kHeadDim;
    };
    int32_t pa = pos_at(r16), pb = pos_at(16 + r16), pv = pos_at(kk);
    uint4 wa[4], wb[4];
    load_krow(wa, row_of(kbase, pa), u);
    load_krow(wb, row_of(kbase, pb), u);
    VHalf vr = load_vhalf(row_of(vbase, pv), hv);
    for (int t = 0; t < n; t += kKT) {
      // stage this tile's V rows (registers -> LDS)
      store_vhalf(vs + kk * kVStride + 64 * hv, vr);
      // S = Q K^T for keys t + r16 (A) and t + 16 + r16 (B)
      f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[j], __builtin_bit_cast(bf16x8, wa[j]), sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[j], __builtin_bit_cast(bf16x8, wb[j]), sb, 0, 0, 0);
      }
      const bool va = pa >= 0, vb = pb >= 0;
      // request the next tile now
      if (t + kKT < n) {
        pa = pos_at(t + kKT + r16);
        pb = pos_at(t + kKT + 16 + r16);
        pv = pos_at(t + kKT + kk);
        load_krow(wa, row_of(kbase, pa), u);
        load_krow(wb, row_of(kbase, pb), u);
        vr = load_vhalf(row_of(vbase, pv), hv);
      }
      // online softmax; lane holds rows 4u + i for key column r16
      float pA[4], pB[4], alpha[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float xa = va ? sa[i] * a.scale : -__builtin_inff();
        const float xb = vb ? sb[i] * a.scale : -__builtin_inff();
        float mx = fmaxf(xa, xb);
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        const float mn = fmaxf(m[i], mx);
        const bool empty = mn == -__builtin_inff();
        alpha[i] = empty ? 1.f : __expf(m[i] - mn);
        pA[i] = empty ? 0.f : __expf(xa - mn);
        pB[i] = empty ? 0.f : __expf(xb - mn);
        float rs = pA[i] + pB[i];
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) rs += __shfl_xor(rs, off, 64);
        l[i] = l[i] * alpha[i] + rs;
        m[i] = mn;
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[j][i] *= alpha[i];
      // P (bf16) to LDS as [head row][key]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ps[(4 * u + i) * kPStride + r16] = f32_to_bf16_rne(pA[i]);
        ps[(4 * u + i) * kPStride + 16 + r16] = f32_to_bf16_rne(pB[i]);
      }
      wave_fence();
      // O += P V: A = P rows r16, keys [8u, +8); B = V keys [8u, +8), dim 16j + r16
      const bf16x8 pf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(ps + r16 * kPStride + 8 * u));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t lo = vs[(8 * u + 2 * e) * kVStride + 16 * j + r16];
          const uint32_t hi = vs[(8 * u + 2 * e + 1) * kVStride + 16 * j + r16];
          w[e] = lo | (hi << 16);
        }
        const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
        o[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, vf, o[j], 0, 0, 0);
      }
      wave_fence();
    }
    // write: rows 4u + i < G, dims 16j + r16
    if (a.splits == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hr = 4 * u + i;
        if (hr < a.G) {
          const float inv = l[i] > 0.f ? 1.f / l[i] : 0.f;
          uint16_t* orow = a.out + (row * a.Hq + (int64_t)kvh * a.G + hr) * kHeadDim;
#pragma unroll
          for (int j = 0; j < 8; ++j) orow[16 * j + r16] = f32_to_bf16_rne(o[j][i] * inv);
        }
      }
    } else {
      const int64_t slot = row * a.splits + split;
      float* ob = a.ws;
      float* mb = a.ws + a.rows * a.splits * a.Hq * kHeadDim;
      float* lb = mb + a.rows * a.splits * a.Hq;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hr = 4 * u + i;
        if (hr < a.G) {
          const int64_t h = (int64_t)kvh * a.G + hr;
          float* orow = ob + (slot * a.Hq + h) * kHeadDim;
#pragma unroll
          for (int j = 0; j < 8; ++j) orow[16 * j + r16] = o[j][i];
          if (r16 == 0) { mb[slot * a.Hq + h] = m[i]; lb[slot * a.Hq + h] = l[i]; }
        }
      }
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
template <int DT>
__global__ __launch_bounds__(128) void k_attn_combine(const float* __restrict__ ws, void* out,
                                                      int64_t rows, int32_t Hq, int32_t splits) {
  const int64_t rh = blockIdx.x;           // row * Hq + h
  const int64_t row = rh / Hq;
  const int h = (int)(rh % Hq);
  const int d = threadIdx.x;
  const float* ob = ws;
  const float* mb = ws + rows * splits * Hq * kHeadDim;
  const float* lb = mb + rows * splits * Hq;
  float M = -__builtin_inff();
  for (int s = 0; s < splits; ++s) M = fmaxf(M, mb[(row * splits + s) * Hq + h]);
  float num = 0.f, den = 0.f;
  if (M != -__builtin_inff()) {
    for (int s = 0; s < splits; ++s) {
      const int64_t slot = row * splits + s;
      const float ms = mb[slot * Hq + h];
      if (ms == -__builtin_inff()) continue;
      const float w = __expf(ms - M);
      num = __builtin_fmaf(w, ob[(slot * Hq + h) * kHeadDim + d], num);
      den = __builtin_fmaf(w, lb[slot * Hq + h], den);
    }
  }
  const float r = den > 0.f ? num / den : 0.f;
  if (DT == LSA_BF16) reinterpret_cast<uint16_t*>(out)[rh * kHeadDim + d] = f32_to_bf16_rne(r);
  else reinterpret_cast<float*>(out)[rh * kHeadDim + d] = r;
}

}  // namespace

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
    const int nw = Hkv < kMaxWaves ? Hkv : kMaxWaves;
    static bool attr_set = false;
    if (!attr_set) {
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(k_attn_bf16),
                                hipFuncAttributeMaxDynamicSharedMemorySize, 128 * 1024);
      (void)hipGetLastError();  // advisory; never report it as a launch failure
      attr_set = true;
    }
    const int per = (L_max + splits - 1) / splits;
    const size_t smem = (size_t)nw * kWaveLds * sizeof(uint16_t) + (size_t)per * sizeof(int32_t);
    hipLaunchKernelGGL(k_attn_bf16, dim3((unsigned)rows, (unsigned)splits), dim3(64 * nw), smem, s, a);
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
    hipLaunchKernelGGL(k_attn_combine<LSA_BF16>, dim3((unsigned)(rows * Hq)), dim3(kHeadDim), 0, s,
                       ws, out, rows, Hq, splits);
  else
    hipLaunchKernelGGL(k_attn_combine<LSA_F32>, dim3((unsigned)(rows * Hq)), dim3(kHeadDim), 0, s,
                       ws, out, rows, Hq, splits);
  return hipGetLastError();
}

}  // namespace lsa
