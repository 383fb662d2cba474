// Block-mask builder: tile classes (EMPTY / PARTIAL / FULL) and, per row of
// tiles, the compacted ascending list of non-EMPTY kv tiles.
//
// What it computes: the block-sparse metadata the ejkernel ring-splash page
// passes to its kernel (MaskInfo: a block mask plus the lists of blocks to
// visit), built the way the Kvax page's create_attention_mask builds its
// block-wise masks: from positions and segment IDs, skipping blocks with
// nothing to attend. A tile is EMPTY when none of its (query, key) pairs is
// allowed, FULL when all are, else PARTIAL; pairs past the sequence ends do
// not count.
//
// One workgroup per (row of tiles, batch, chunk). With sequential positions
// and no segments a tile's class follows from its position ranges alone:
// FULL iff min q_pos >= max kv_pos, EMPTY iff max q_pos < min kv_pos. With
// explicit positions but no segments the same test runs on the tile's
// position minima and maxima. With segments every pair of the tile is
// checked. Classes are staged in LDS, then compacted in order with wave
// ballots and a running offset.
#include <hip/hip_runtime.h>

#include "ram_internal.h"

namespace ram {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ int wave_min(int v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ int wave_max(int v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// Block-wide min and max of one value per thread (all threads must call).
__device__ __forceinline__ void block_minmax(int vmin, int vmax, int* red, int& omin, int& omax) {
  vmin = wave_min(vmin);
  vmax = wave_max(vmax);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[w] = vmin;
    red[kWaves + w] = vmax;
  }
  __syncthreads();
  omin = red[0];
  omax = red[kWaves];
  for (int i = 1; i < kWaves; ++i) {
    omin = min(omin, red[i]);
    omax = max(omax, red[kWaves + i]);
  }
  __syncthreads();
}

__global__ __launch_bounds__(kThreads) void block_mask_kernel(MaskParams p) {
  __shared__ uint8_t cls_s[kMaxMaskCols];
  __shared__ int qpos_s[kMaxMaskTile], qseg_s[kMaxMaskTile];
  __shared__ int kpos_s[kMaxMaskTile], kseg_s[kMaxMaskTile];
  __shared__ int red[2 * kWaves];
  __shared__ int wsum[kWaves];

  const int qb = blockIdx.x, b = blockIdx.y, c = blockIdx.z;
  const int tid = threadIdx.x;
  const int q0 = qb * p.bq;
  const int nq = min(p.Sq, q0 + p.bq) - q0;
  const int kv_base = p.kv_pos_base + c * p.kv_base_step;
  const int32_t* qpos = p.q_pos ? p.q_pos + (int64_t)b * p.qm_stride_b + q0 : nullptr;
  const int32_t* qseg = p.q_seg ? p.q_seg + (int64_t)b * p.qm_stride_b + q0 : nullptr;
  const int64_t kvoff = (int64_t)b * p.kvm_stride_b + (int64_t)c * p.kv_chunk_off;
  const int32_t* kvpos = p.kv_pos ? p.kv_pos + kvoff : nullptr;
  const int32_t* kvseg = p.kv_seg ? p.kv_seg + kvoff : nullptr;
  const int64_t crow = ((int64_t)c * p.B + b) * p.nQb + qb;   // row index over (chunk, batch, q tile)

  if (qseg == nullptr) {
    // No segments: classes from position ranges (exact: all pairs allowed iff
    // max kv <= min q; none iff max q < min kv).
    int qmin, qmax;
    if (qpos) {
      int lo = 0x7fffffff, hi = -0x7fffffff - 1;
      for (int i = tid; i < nq; i += kThreads) {
        lo = min(lo, qpos[i]);
        hi = max(hi, qpos[i]);
      }
      block_minmax(lo, hi, red, qmin, qmax);
    } else {
      qmin = p.q_pos_base + q0;
      qmax = p.q_pos_base + q0 + nq - 1;
    }
    if (kvpos == nullptr) {
      for (int kb = tid; kb < p.nKb; kb += kThreads) {
        const int k0 = kb * p.bk;
        const int nk = min(p.Skv, k0 + p.bk) - k0;
        const int kmin = kv_base + k0, kmax = kv_base + k0 + nk - 1;
        uint8_t cl = 2;
        if (p.causal) cl = (qmin >= kmax) ? 2 : ((qmax < kmin) ? 0 : 1);
        cls_s[kb] = cl;
      }
    } else {
      for (int kb = 0; kb < p.nKb; ++kb) {
        const int k0 = kb * p.bk;
        const int nk = min(p.Skv, k0 + p.bk) - k0;
        int lo = 0x7fffffff, hi = -0x7fffffff - 1;
        for (int j = tid; j < nk; j += kThreads) {
          lo = min(lo, kvpos[k0 + j]);
          hi = max(hi, kvpos[k0 + j]);
        }
        int kmin, kmax;
        block_minmax(lo, hi, red, kmin, kmax);
        if (tid == 0) {
          uint8_t cl = 2;
          if (p.causal) cl = (qmin >= kmax) ? 2 : ((qmax < kmin) ? 0 : 1);
          cls_s[kb] = cl;
        }
      }
    }
  } else {
    // Segments: check every pair of each tile.
    for (int i = tid; i < nq; i += kThreads) {
      qpos_s[i] = qpos ? qpos[i] : p.q_pos_base + q0 + i;
      qseg_s[i] = qseg[i];
    }
    for (int kb = 0; kb < p.nKb; ++kb) {
      const int k0 = kb * p.bk;
      const int nk = min(p.Skv, k0 + p.bk) - k0;
      for (int j = tid; j < nk; j += kThreads) {
        kpos_s[j] = kvpos ? kvpos[k0 + j] : kv_base + k0 + j;
        kseg_s[j] = kvseg[k0 + j];
      }
      __syncthreads();
      int any_ok = 0, any_bad = 0;
      const int npair = nq * nk;
      for (int t = tid; t < npair; t += kThreads) {
        const int i = t / nk, j = t - (t / nk) * nk;
        bool ok = qseg_s[i] != -1 && qseg_s[i] == kseg_s[j];
        if (p.causal) ok = ok && kpos_s[j] <= qpos_s[i];
        any_ok |= ok;
        any_bad |= !ok;
      }
      any_ok = __syncthreads_or(any_ok);
      any_bad = __syncthreads_or(any_bad);
      if (tid == 0) cls_s[kb] = any_ok ? (any_bad ? 1 : 2) : 0;
    }
  }
  __syncthreads();

  // Write classes and compact the non-EMPTY tiles in ascending order.
  uint8_t* cls_out = p.tile_class + crow * p.nKb;
  int32_t* col_out = p.col_idx + crow * p.nKb;
  for (int kb = tid; kb < p.nKb; kb += kThreads) cls_out[kb] = cls_s[kb];
  const int lane = tid & 63, w = tid >> 6;
  int running = 0;
  for (int base = 0; base < p.nKb; base += kThreads) {
    const int kb = base + tid;
    const bool f = kb < p.nKb && cls_s[kb] != 0;
    const uint64_t bal = __ballot(f);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[w] = __popcll(bal);
    __syncthreads();
    int off = running;
    int total = 0;
    for (int i = 0; i < kWaves; ++i) {
      if (i < w) off += wsum[i];
      total += wsum[i];
    }
    if (f) col_out[off + before] = kb;
    running += total;
    __syncthreads();
  }
  for (int j = running + tid; j < p.nKb; j += kThreads) col_out[j] = -1;
  if (tid == 0) p.row_cnt[crow] = running;
}

}  // namespace

hipError_t launch_block_mask(const MaskParams& p, int n_chunks, hipStream_t s) {
  if (p.B == 0 || p.nQb == 0 || n_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(block_mask_kernel, dim3(p.nQb, p.B, n_chunks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace ram
