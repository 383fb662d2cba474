// Host-only stand-ins for everything ram_api.cpp calls outside itself: the kernel launchers
// (defined in the .hip files) and the three HIP runtime calls it makes. Linked with ram_api.cpp
// under the address and undefined-behaviour sanitizers, so that the C ABI's argument checking
// runs on the CPU. A launch that is reached reports hipErrorNoDevice (so a case that should have
// been rejected before any launch shows up as RAM_ERR_HIP).
#include "../../ring_attention_merge_amd/csrc/ram_internal.h"

namespace ram {
hipError_t launch_attn(const AttnParams&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_bwd(const BwdParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_bwd_dq(const BwdParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_bwd_dkv(const BwdParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_bwd_f32(const BwdParams&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_bwd_prep(int, int, int, int, int, const void*, const void*, const float*, const float*, float*,
                           float*, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_col_lists(const MaskParams&, int, int32_t*, int32_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_alt(const AttnParams&, const RingSplit*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_pack_v(const void*, int64_t, int, int, int, int, void*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_block_mask(const MaskParams&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_row_order(const int32_t*, int, int64_t, int, int32_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_merge(int, int, int, int, float*, float*, const float*, const float*, hipStream_t, void*) {
  return hipErrorNoDevice;
}
hipError_t launch_cast_bf16(const float*, void*, int64_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_sum_parts(const float*, int, int64_t, int, int64_t, float*, int64_t, hipStream_t) {
  return hipErrorNoDevice;
}
}  // namespace ram

extern "C" {
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipErrorNoDevice; }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) { return hipErrorNoDevice; }
const char* hipGetErrorString(hipError_t) { return "no device (host-only build)"; }
}
