// Device-side fill of N(0,1) inputs for the synthetic workloads.
//
// Same definition as the host generator in lsa_synth/__init__.py: the
// counter-based Philox4x32-10 generator (Salmon, Moraes, Dror, Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011), element e uses
// counter (e/4 low word, e/4 high word, 0, 0); words (0,1) feed elements
// 4m, 4m+1 and words (2,3) elements 4m+2, 4m+3 through the Box-Muller
// transform in fp64; values are then rounded to nearest even in the storage
// type.  Harness code only: it holds none of the indexing method.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ void philox10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    const uint64_t p0 = (uint64_t)M0 * c[0];
    const uint64_t p1 = (uint64_t)M1 * c[2];
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0; c[1] = lo1; c[2] = n2; c[3] = lo0;
  }
}

// fp64 -> bf16 bits, nearest even on 8 significant bits (subnormal quantum 2^-133)
__device__ __forceinline__ uint16_t to_bf16(double x) {
  int e;
  (void)frexp(x, &e);
  if (e < -125) e = -125;
  const double q = ldexp(rint(ldexp(x, 8 - e)), e - 8);
  const float f = (float)q;  // exact: q has at most 8 significant bits
  return (uint16_t)(__float_as_uint(f) >> 16);
}

__device__ __forceinline__ void fill_one(void* out, int64_t i, int64_t off, uint32_t k0, uint32_t k1,
                                         int is_bf16) {
  const uint64_t e = (uint64_t)(off + i);
  const uint64_t m = e >> 2;
  const int slot = (int)(e & 3);
  uint32_t c[4] = {(uint32_t)m, (uint32_t)(m >> 32), 0u, 0u};
  philox10(c, k0, k1);
  const uint32_t wa = slot < 2 ? c[0] : c[2];
  const uint32_t wb = slot < 2 ? c[1] : c[3];
  const double u1 = ((double)wa + 0.5) * 0x1p-32;
  const double u2 = ((double)wb + 0.5) * 0x1p-32;
  const double r = sqrt(-2.0 * log(u1));
  const double th = 6.283185307179586 * u2;
  const double z = (slot % 2 == 0) ? r * cos(th) : r * sin(th);
  if (is_bf16) reinterpret_cast<uint16_t*>(out)[i] = to_bf16(z);
  else reinterpret_cast<float*>(out)[i] = (float)z;
}

// Grid-stride loop: a dispatch's total work-item count must stay below 2^32,
// and the 10M-token K/V tensors have 5.12e9 elements.
__global__ void k_fill_normal(void* out, int64_t n, int64_t off, uint32_t k0, uint32_t k1,
                              int is_bf16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    fill_one(out, i, off, k0, k1, is_bf16);
}

}  // namespace

extern "C" int synth_fill_normal(void* ptr, int64_t n, int64_t elem_offset, uint32_t k0,
                                 uint32_t k1, int is_bf16, void* stream) {
  if (n <= 0) return 0;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 262144) blocks = 262144;
  hipLaunchKernelGGL(k_fill_normal, dim3((unsigned)blocks), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), ptr, n, elem_offset, k0, k1, is_bf16);
  return (int)hipGetLastError();
}
