// Standalone LSE merge and the final cast of the float32 accumulator.
//
// The merge is _update_out_and_lse of the ejkernel ring-splash source page:
// a row whose running lse is -inf takes the block's (out, lse); otherwise,
// with x = block_lse - lse, out moves toward block_out by sigmoid(x) and lse
// grows by softplus(x). A block row with lse = -inf leaves the row unchanged
// (sigmoid(-inf) = 0, softplus(-inf) = 0); that case is skipped so that
// -inf - -inf is never formed.
//
// One row (D floats) is handled by D/4 consecutive lanes of one wave with
// 16-byte accesses; every lane reads the row's running lse before the one
// lane that writes it, all inside the same wave, so no other lane can see a
// half-updated row.
#include <hip/hip_runtime.h>

#include "ram_internal.h"

namespace ram {
namespace {

constexpr int kThreads = 256;

// With out_bf16 set, the merged rows (and the rows the block leaves unchanged) are written there
// in bf16 instead of back into out_acc: the merge and the final cast in one pass.
__global__ __launch_bounds__(kThreads) void merge_kernel(int B, int Sq, int H, int D, float* out_acc,
                                                         float* lse_acc, const float* out_blk,
                                                         const float* lse_blk, __bf16* out_bf16) {
  const int lpr = D / 4;                      // lanes per row (16 or 32)
  const int rows_per_block = kThreads / lpr;
  const int64_t row = (int64_t)blockIdx.x * rows_per_block + threadIdx.x / lpr;
  const int part = threadIdx.x % lpr;
  const int64_t n_rows = (int64_t)B * Sq * H;
  if (row >= n_rows) return;
  const int h = (int)(row % H);
  const int64_t bq = row / H;
  const int q = (int)(bq % Sq);
  const int b = (int)(bq / Sq);
  const int64_t li = ((int64_t)b * H + h) * Sq + q;
  const float la = lse_acc[li];
  const float lb = lse_blk[li];
  if (lb == -__builtin_inff() && !out_bf16) return;
  float4* pa = reinterpret_cast<float4*>(out_acc + row * D) + part;
  float4 o;
  float nl = la;
  if (lb == -__builtin_inff()) {
    o = *pa;
  } else if (la == -__builtin_inff()) {
    o = reinterpret_cast<const float4*>(out_blk + row * D)[part];
    nl = lb;
  } else {
    const float4 ob = reinterpret_cast<const float4*>(out_blk + row * D)[part];
    const float x = lb - la;
    const float sig = 1.0f / (1.0f + expf(-x));
    nl = la + (fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x))));
    const float4 a = *pa;
    o.x = a.x - sig * (a.x - ob.x);
    o.y = a.y - sig * (a.y - ob.y);
    o.z = a.z - sig * (a.z - ob.z);
    o.w = a.w - sig * (a.w - ob.w);
  }
  if (out_bf16) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 v = {o.x, o.y, o.z, o.w};
    reinterpret_cast<bf16x4*>(out_bf16 + row * D)[part] = __builtin_convertvector(v, bf16x4);
  } else {
    *pa = o;
  }
  if (part == 0) lse_acc[li] = nl;
}

__global__ __launch_bounds__(kThreads) void cast_bf16_kernel(const float* src, __bf16* dst, int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n8) return;
  const float4 a = reinterpret_cast<const float4*>(src)[2 * i];
  const float4 b = reinterpret_cast<const float4*>(src)[2 * i + 1];
  typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
  typedef float f32x8 __attribute__((ext_vector_type(8)));
  f32x8 v = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  reinterpret_cast<bf16x8*>(dst)[i] = __builtin_convertvector(v, bf16x8);
}

}  // namespace

hipError_t launch_merge(int B, int Sq, int H, int D, float* out_acc, float* lse_acc,
                        const float* out_blk, const float* lse_blk, hipStream_t s, void* out_bf16) {
  const int64_t n_rows = (int64_t)B * Sq * H;
  if (n_rows == 0) return hipSuccess;
  const int rows_per_block = kThreads / (D / 4);
  const int64_t grid = (n_rows + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, B, Sq, H, D, out_acc,
                     lse_acc, out_blk, lse_blk, static_cast<__bf16*>(out_bf16));
  return hipGetLastError();
}

hipError_t launch_cast_bf16(const float* src, void* dst, int64_t n, hipStream_t s) {
  const int64_t n8 = n / 8;   // n is a multiple of 8 (D is 64 or 128)
  if (n8 == 0) return hipSuccess;
  const int64_t grid = (n8 + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(cast_bf16_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, src,
                     reinterpret_cast<__bf16*>(dst), n8);
  return hipGetLastError();
}

}  // namespace ram
