// ring_attn_fwd_1gpu without a workspace argument, for callers that cannot allocate device memory:
// its scratch (the float32 running output, the chunks' block masks and, for a split ring, the
// second half's running state) lives in a static device array of kScratchBytes, one per GPU,
// held until the process ends. Every call on a GPU uses that GPU's array; the ring writes every
// byte of it that it reads, so nothing needs clearing between calls, and calls that overlap on
// one GPU race on it.
#include <cstdio>
#include <mutex>

#include <hip/hip_runtime.h>

#include "ram_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB
constexpr int kMaxDevices = 64;

}  // namespace

// The array itself. In host code this name is the host-side handle of the variable, not a device
// address: kernels get the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

std::mutex g_mu;
void* g_scratch[kMaxDevices];   // per device: the address of `scratch` there, once looked up

// The current device's address of `scratch`, looked up on the first call on that device (with it
// current).
ram_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return ram::api_fail(RAM_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return ram::api_fail(RAM_ERR_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return ram::api_fail(RAM_ERR_HIP, "hipGetSymbolAddress of the static scratch failed");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return RAM_OK;
}

}  // namespace

extern "C" ram_status ring_attn_fwd_1gpu_noalloc(const ram_attn_desc* desc, int32_t n_chunks, int32_t q_shard,
                                                 const void* q, const void* k_all, const void* v_all,
                                                 const ram_mask_src* src, const float* sinks, void* out, float* lse,
                                                 hipStream_t stream) {
  if (!desc) return ram::api_fail(RAM_ERR_INVALID, "desc is null");
  const size_t need = ring_attn_workspace_bytes(desc, n_chunks, src);
  if (need > kScratchBytes) {
    char msg[160];
    snprintf(msg, sizeof(msg), "this ring needs %zu bytes of scratch; the static scratch holds %zu", need,
             kScratchBytes);
    return ram::api_fail(RAM_ERR_UNSUPPORTED, msg);
  }
  void* ws = nullptr;
  const ram_status st = scratch_ptr(&ws);
  if (st != RAM_OK) return st;
  return ring_attn_fwd_1gpu(desc, n_chunks, q_shard, q, k_all, v_all, src, sinks, out, lse, ws, kScratchBytes,
                            stream);
}
