// ceiling.hip -- the measured bf16 MFMA ceiling of the device, for the roofline that the
// attention kernel is quoted against (a measurement kernel, built into a library of its
// own; not part of the cache library or its interface).
//
// Every wave runs independent chains of the 32x32x16 bf16 MFMA the attention uses (four
// accumulators, so no MFMA waits for the one before it), nothing else in the loop: the
// rate at which the matrix cores retire that instruction at the clock the device holds
// under that load, which the nominal 2.5 PFLOP/s (at 2.4 GHz) does not show.
//
// The matrix cores' power, and so the clock the device can hold, depends on the operand
// bits.  Two forms: operands with few mantissa bits set, the same pair in every MFMA
// (a best case), or operands taken from a buffer of random values, a different pair in
// each MFMA of a group of four, as in attention where every MFMA reads new fragments.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void finish(float* out, const f32x16& c0, const f32x16& c1, const f32x16& c2,
                                       const f32x16& c3) {
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = s;   // keeps the chains live
}

__global__ __launch_bounds__(256) void mfma_loop_kernel(float* out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float((threadIdx.x + i) & 7) * 0.125f);
    b[i] = (__bf16)(float((threadIdx.x * 3 + i) & 7) * 0.0625f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = mfma(a, b, c0);
    c1 = mfma(b, a, c1);
    c2 = mfma(a, a, c2);
    c3 = mfma(b, b, c3);
  }
  finish(out, c0, c1, c2, c3);
}

// data: 256 lanes x 8 fragments of 8 bf16 (32 KB), the same for every workgroup; lane t
// holds fragments data[t*64 .. t*64+63].  Each iteration issues 16 MFMAs on 16 distinct
// (A, B) fragment pairs, four per accumulator.
__global__ __launch_bounds__(256) void mfma_loop_data_kernel(float* out, const bf16x8* data, int iters) {
  bf16x8 f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = data[threadIdx.x * 8 + i];
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; it += 4) {
    c0 = mfma(f[0], f[4], c0);
    c1 = mfma(f[1], f[5], c1);
    c2 = mfma(f[2], f[6], c2);
    c3 = mfma(f[3], f[7], c3);
    c0 = mfma(f[1], f[6], c0);
    c1 = mfma(f[2], f[7], c1);
    c2 = mfma(f[3], f[4], c2);
    c3 = mfma(f[0], f[5], c3);
    c0 = mfma(f[2], f[5], c0);
    c1 = mfma(f[3], f[6], c1);
    c2 = mfma(f[0], f[7], c2);
    c3 = mfma(f[1], f[4], c3);
    c0 = mfma(f[3], f[7], c0);
    c1 = mfma(f[0], f[4], c1);
    c2 = mfma(f[1], f[5], c2);
    c3 = mfma(f[2], f[6], c3);
  }
  finish(out, c0, c1, c2, c3);
}

}  // namespace

extern "C" {

// Launch `blocks` workgroups of 256 threads (4 waves), each wave issuing 4 * iters MFMAs
// of 32x32x16 (32768 flop each); out: device float[blocks * 256].  Returns a hipError_t.
int llc_mfma_loop(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks <= 0 || iters <= 0) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream), out,
                     iters);
  return int(hipGetLastError());
}

// The same count of MFMAs on operands read from `data` (device bf16[256 * 64], 16-byte
// aligned, read only); iters must be a multiple of 4.  Returns a hipError_t.
int llc_mfma_loop_data(float* out, const void* data, int blocks, int iters, void* stream) {
  if (!out || !data || blocks <= 0 || iters <= 0 || iters % 4 != 0 || (reinterpret_cast<uintptr_t>(data) & 15))
    return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(mfma_loop_data_kernel, dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     out, static_cast<const bf16x8*>(data), iters);
  return int(hipGetLastError());
}

}  // extern "C"
