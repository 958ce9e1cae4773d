// ceiling.hip -- the measured bf16 MFMA ceiling of the device, for the roofline that the
// attention kernel is quoted against (a measurement kernel, built into a library of its
// own; not part of the cache library or its interface).
//
// Every wave runs independent chains of the 32x32x16 bf16 MFMA the attention uses (four
// accumulators, so no MFMA waits for the one before it), nothing else in the loop: the
// rate at which the matrix cores retire that instruction at the clock the device holds
// under that load, which the nominal 2.5 PFLOP/s (at 2.4 GHz) does not show.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_loop_kernel(float* out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float((threadIdx.x + i) & 7) * 0.125f);
    b[i] = (__bf16)(float((threadIdx.x * 3 + i) & 7) * 0.0625f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  out[int64_t(blockIdx.x) * blockDim.x + threadIdx.x] = s;   // keeps the chains live
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

}  // extern "C"
