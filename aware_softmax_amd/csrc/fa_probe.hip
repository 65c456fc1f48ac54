// MFMA-only ceiling: back-to-back v_mfma_f32_32x32x16_bf16 with no memory
// traffic, no LDS and no VALU work in the loop.  Timed beside the attention
// forward, it gives the dense bf16 rate the chip sustains at the clock it
// actually runs under matrix load, next to the nominal 2.4 GHz peak.
#include <hip/hip_runtime.h>

#include "fa_internal.h"

namespace fa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Integer hash (a multiply-xorshift mix) mapped to a float in [-2, 2).
__device__ inline float hash_unit(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return (float)(x >> 8) * (4.0f / 16777216.0f) - 2.0f;
}

// Four independent accumulator chains per wave, each with its own operand
// pair of pseudo-random bf16 values (so the multipliers switch as they do
// on real data; constant operands draw less power and let the clock run
// higher than any real workload would).  The result is stored only when
// `store` is set, which the compiler cannot know, so no MFMA is dropped.
__global__ __launch_bounds__(256) void mfma_ceiling_kernel(float* sink, int iters, int store) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8 a[4], b[4];
  for (int j = 0; j < 4; ++j)
    for (int i = 0; i < 8; ++i) {
      a[j][i] = (__bf16)hash_unit(t * 64u + j * 16u + i);
      b[j][i] = (__bf16)hash_unit(t * 64u + j * 16u + 8u + i);
    }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[2], c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], b[3], c3, 0, 0, 0);
  }
  if (store) {
    float s = 0.f;
    for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
    sink[t] = s;
  }
}

}  // namespace

hipError_t launch_mfma_ceiling(float* sink, int iters, int blocks, int store, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(blocks), dim3(256), 0, stream, sink, iters, store);
  return hipGetLastError();
}

}  // namespace fa
