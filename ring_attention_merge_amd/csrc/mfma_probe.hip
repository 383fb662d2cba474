// Dense bf16 MFMA rate probe: the ceiling the attention kernels are measured
// against on real data. Each wave keeps four 32x32 fp32 accumulators and runs
// eight v_mfma_f32_32x32x16_bf16 into each per iteration from operands held in
// registers (no memory traffic), eight waves per workgroup. The matrix cores'
// clock depends on the switching activity of the operands, so the rate with
// all-zero operands (the spec figure's condition) and with pseudo-random ones
// (what attention inputs look like) differ; the caller times both.
#include <hip/hip_runtime.h>

#include "ram.h"

namespace ram {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 512;

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(int32_t iters, int32_t operands, float* out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[4], b[8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      // a multiplicative hash of (lane, i, e) mapped to [-1, 1)
      const uint32_t h = ((uint32_t)lane * 2654435761u) ^ ((uint32_t)i * 40503u) ^ ((uint32_t)e * 2246822519u);
      const float r = operands ? (float)((h >> 8) & 0xffffu) * (1.0f / 32768.0f) - 1.0f : 0.0f;
      if (i < 4) a[i][e] = (__bf16)r;
      b[i][e] = (__bf16)(-0.5f * r);
    }
  f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c], b[j], acc[c], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int c = 0; c < 4; ++c) s += acc[c][0] + acc[c][15];
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

}  // namespace
}  // namespace ram

extern "C" ram_status ram_mfma_probe(int32_t n_blocks, int32_t iters, int32_t operands, float* out,
                                     hipStream_t stream) {
  if (n_blocks < 1 || iters < 1 || (operands != 0 && operands != 1) || !out) return RAM_ERR_INVALID;
  hipLaunchKernelGGL(ram::mfma_probe_kernel, dim3(n_blocks), dim3(ram::kProbeThreads), 0, stream, iters, operands,
                     out);
  return hipGetLastError() == hipSuccess ? RAM_OK : RAM_ERR_HIP;
}
