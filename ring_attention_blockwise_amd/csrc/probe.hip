// Matrix-core probe (gfx950): the dense bf16 MFMA rate and the shader clock
// on this device, measured with the instruction the step kernels use
// (v_mfma_f32_32x32x16_bf16), as the reference point beside the published
// peak. Not part of the attention path.
#include "bf16_tiles.h"

namespace ra {
namespace {

using namespace bf16k;

__global__ void __launch_bounds__(256) mfma_probe_kernel(int32_t iters, float* sink, uint64_t* stamps) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.0078125f * (float)((lane + i) & 7));
    b[i] = (__bf16)(0.0078125f * (float)((3 * lane + i) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  // the operands are "produced" after the first stamps, so the loop cannot be
  // hoisted above them
  asm volatile("" : "+v"(a), "+v"(b));
  for (int32_t it = 0; it < iters; ++it) {  // four independent accumulation chains
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c3, 0, 0, 0);
  }
  // ... and consumed before the last stamps
  asm volatile("" ::"v"(c0[0]), "v"(c1[0]), "v"(c2[0]), "v"(c3[0]));
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) s += c0[j] + c1[j] + c2[j] + c3[j];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (threadIdx.x == 0) {
    uint64_t* st = stamps + 4 * (size_t)blockIdx.x;
    st[0] = t0;
    st[1] = t1;
    st[2] = r0;
    st[3] = r1;
  }
}

}  // namespace

hipError_t launch_mfma_probe(int32_t blocks, int32_t iters, float* sink, uint64_t* stamps, hipStream_t s) {
  mfma_probe_kernel<<<dim3((unsigned)blocks), 256, 0, s>>>(iters, sink, stamps);
  return hipGetLastError();
}

}  // namespace ra
