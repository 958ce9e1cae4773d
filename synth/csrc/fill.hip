// fill.hip -- device twin of synth/philox.py: seeded N(0, sigma^2) bf16 tensors.
//
// Input preparation only (no attention, cache or quantisation arithmetic).  Philox4x32-10
// (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11):
// element i takes 32-bit word i mod 4 of the block with counter (i div 4 mod 2^32,
// i div 2^34, 0, 0) under the 64-bit key split into two words; the word's top 16 bits
// index a 65536-entry float32 table of standard-normal quantiles made on the host; the
// value is float32(table[j] * sigma) rounded to bf16 (nearest, ties to even).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = uint64_t(0xD2511F53u) * c[0];
    const uint64_t p1 = uint64_t(0xCD9E8D57u) * c[2];
    const uint32_t n0 = uint32_t(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n1 = uint32_t(p1);
    const uint32_t n2 = uint32_t(p0 >> 32) ^ c[3] ^ k1;
    const uint32_t n3 = uint32_t(p0);
    c[0] = n0;
    c[1] = n1;
    c[2] = n2;
    c[3] = n3;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
}

__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// One thread per block of four elements.
__global__ __launch_bounds__(256) void fill_normal_kernel(uint16_t* out, int64_t n, uint32_t k0, uint32_t k1,
                                                          const float* table, float sigma) {
  const int64_t b = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t i0 = b * 4;
  if (i0 >= n) return;
  uint32_t c[4] = {uint32_t(uint64_t(b)), uint32_t(uint64_t(b) >> 32), 0u, 0u};
  philox4x32_10(c, k0, k1);
#pragma unroll
  for (int w = 0; w < 4; ++w)
    if (i0 + w < n) out[i0 + w] = bf16_rne(table[c[w] >> 16] * sigma);
}

}  // namespace

// out: n bf16 values (device); table: 65536 floats (device); returns a hipError_t.
extern "C" int synth_fill_normal_bf16(void* out, int64_t n, uint32_t k0, uint32_t k1, const void* table,
                                      float sigma, void* stream) {
  if (n <= 0) return 0;
  const int64_t blocks = (n + 3) / 4;
  const int64_t grid = (blocks + 255) / 256;
  hipLaunchKernelGGL(fill_normal_kernel, dim3(unsigned(grid)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint16_t*>(out), n, k0, k1, static_cast<const float*>(table), sigma);
  return int(hipGetLastError());
}
