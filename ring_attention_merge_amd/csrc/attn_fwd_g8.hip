// Block-sparse attention forward for one KV chunk: 8-wave, 3-stage variant.
//
// Computes exactly what attn_fwd.hip computes (the per-ring-step kernel call of
// the ejkernel ring-splash source page, _ring_attention_forward, with the
// _update_out_and_lse merge as epilogue). What changes is how the tiles are
// fed, after measurement showed the 4-wave kernel losing most of its time
// waiting at the end of each tile for K/V loads issued at its start:
//
//  * One workgroup = 8 waves = two groups of 4 waves, each group one 128-row
//    q tile of the same head; both groups consume the same K/V tiles, so a
//    tile loaded once serves 256 query rows. Two waves share each SIMD (one
//    per group) and overlap each other's MFMA and softmax phases.
//  * K and V go from HBM straight to LDS (global_load_lds_dwordx4, no VGPR
//    staging) through 3 stages: tile j+2 is issued while tile j is computed,
//    so each load has two iterations to arrive. Only tile j+1's loads are
//    waited for (s_waitcnt vmcnt with the count of the loads issued after
//    them) before the one barrier per tile.
//  * LDS rows are dense 256-byte rows with XOR-swizzled 16-byte chunks:
//    chunk ^ (row & 15) for K (conflict-free A-operand reads of 16
//    consecutive rows) and chunk ^ 4*(row & 3) for V (conflict-free
//    transposing reads of 4 rows x 64 bytes).
//  * Per wave the math is the 4-wave kernel's: S^T = K Q^T and O^T = V^T P^T
//    with v_mfma_f32_32x32x16_bf16, a lane per query row, P kept in registers,
//    V read with ds_read_b64_tr_b16.
//  * The block mask stays at the 128 x 64 kernel tile: the workgroup walks
//    the union of its two tile rows and a group skips tiles EMPTY for it.
#include "attn_common.h"

namespace ram {
namespace {

using namespace attn;

constexpr int kGWaves = 8;
constexpr int kGThreads = 64 * kGWaves;
constexpr int kGD = 128;
constexpr int kStages = 3;
constexpr int kTileElems = kBlockKV * kGD;      // one K or V tile (16 KB)

__device__ __forceinline__ bool decode_work_g(const AttnParams& p, int nQp, int& b, int& h, int& qp) {
  const int G = p.H / p.Hkv;
  const int64_t T = (int64_t)p.B * p.Hkv * nQp * G;
  const int64_t per = (T + 7) / 8;
  const int64_t id = blockIdx.x;
  const int64_t item = (id & 7) * per + (id >> 3);
  if (item >= T) return false;
  const int hg = (int)(item % G);
  const int64_t r = item / G;
  const int qrev = (int)(r % nQp);
  const int64_t bg = r / nQp;
  const int g = (int)(bg % p.Hkv);
  b = (int)(bg / p.Hkv);
  h = g * G + hg;
  qp = nQp - 1 - qrev;
  return true;
}

// Tile kb of K (is_v = false) or V into LDS: wave w fills rows [8w, 8w+8) with
// two 4-row (1 KB) slabs; lane l writes physical chunk l & 15 of row l >> 4.
__device__ __forceinline__ void dma_tile(const __bf16* gbase, int64_t krs, int kb, int skv, __bf16* tile, int w,
                                         int lane, bool is_v) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * w + 4 * i + (lane >> 4);
    const int phys = lane & 15;
    const int logical = is_v ? (phys ^ (4 * (r & 3))) : (phys ^ (r & 15));
    const int row = min(kb * kBlockKV + r, skv - 1);     // rows past the end are masked later
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(gbase + row * krs + logical * 8),
                                     (void __attribute__((address_space(3)))*)(tile + (8 * w + 4 * i) * kGD), 16, 0, 0);
  }
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

template <bool CAP>
__global__ __launch_bounds__(kGThreads, 1) void attn_fwd_bf16_g8(AttnParams p) {
  constexpr int D = kGD;
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) __bf16 kst[kStages * kTileElems];
  __shared__ __attribute__((aligned(16))) __bf16 vst[kStages * kTileElems];
  __shared__ uint32_t ulist[kMaxMaskCols];
  __shared__ int wsum[kGWaves];

  const int nQp = (p.nQb + 1) >> 1;
  int b, h, qp;
  if (!decode_work_g(p, nQp, b, h, qp)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int grp = w >> 2, wi = w & 3;
  const int ln = lane & 31, lg = lane >> 5;
  const int G = p.H / p.Hkv;
  const int g = h / G;
  const int qb = 2 * qp + grp;
  const int q_row = qb * kBlockQ + wi * 32 + ln;
  const bool q_ok = qb < p.nQb && q_row < p.Sq;

  // ---- union of the two q tiles' non-EMPTY kv tiles
  const int64_t rowA = (int64_t)b * p.nQb + 2 * qp;
  const bool hasB = 2 * qp + 1 < p.nQb;
  int n = 0;
  for (int base = 0; base < p.nKb; base += kGThreads) {
    const int kb = base + tid;
    uint32_t ca = 0, cb = 0;
    if (kb < p.nKb) {
      ca = p.tile_class[rowA * p.nKb + kb];
      if (hasB) cb = p.tile_class[(rowA + 1) * p.nKb + kb];
    }
    const bool f = (ca | cb) != 0;
    const uint64_t bal = __ballot(f);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[w] = __popcll(bal);
    __syncthreads();
    int off = n, total = 0;
#pragma unroll
    for (int i = 0; i < kGWaves; ++i) {
      off += (i < w) ? wsum[i] : 0;
      total += wsum[i];
    }
    if (f) ulist[off + before] = (uint32_t)kb | (ca << 16) | (cb << 24);
    n += total;
    __syncthreads();
  }
  if (n == 0 && p.mode == 1 && p.sinks == nullptr) return;

  // ---- per-lane query state
  bf16x8 qf[NDS];
  {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.q_stride_b +
                         ((int64_t)(q_ok ? q_row : 0) * p.H + h) * D;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      bf16x8 t = *reinterpret_cast<const bf16x8*>(qrow + ds * 16 + lg * 8);
      qf[ds] = q_ok ? t : bf16x8{};
    }
  }
  const int qrow_c = q_ok ? q_row : p.Sq - 1;
  const int qpos = p.q_pos ? p.q_pos[(int64_t)b * p.qm_stride_b + qrow_c] : p.q_pos_base + q_row;
  const int qseg = p.q_seg ? p.q_seg[(int64_t)b * p.qm_stride_b + qrow_c] : 0;

  float m_ref = neg_inf(), l_acc = 0.0f;
  if (p.sinks) {
    m_ref = p.sinks[h] * kLog2e;
    l_acc = (lg == 0) ? 1.0f : 0.0f;
  }
  f32x16 O[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) O[db] = f32x16{};

  const int64_t krs = (int64_t)p.Hkv * D;
  const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + (int64_t)b * p.kv_stride_b + g * D;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.kv_stride_b + g * D;
  auto tile_kb = [&](int j) { return (int)(ulist[j] & 0xffffu); };
  auto tile_cls = [&](int j) { return (int)((ulist[j] >> (16 + 8 * grp)) & 0xffu); };

  // LDS byte offsets of this lane's operands inside a tile.
  int k_off[2][NDS];                  // K: row kb2*32 + ln, logical chunk 2*ds + lg
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) k_off[kb2][ds] = (kb2 * 32 + ln) * 256 + (((2 * ds + lg) ^ (ln & 15)) * 16);
  // V (transposing reads): row ks*16 + 8*r + 4*lg + r4, column db*32 + 16*hs + 4*(lane&3)
  const int r4 = (lane & 15) >> 2, hs = (lane >> 4) & 1;
  const int v_row = 4 * lg + r4;
  int v_col[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    v_col[db] = (((db * 4 + 2 * hs + ((lane & 3) >> 1)) ^ (4 * r4)) * 16) + (lane & 1) * 8;

  // ---- prologue: tiles 0 and 1 in flight, wait for tile 0
  if (n > 0) {
    dma_tile(kbase, krs, tile_kb(0), p.Skv, kst, w, lane, false);
    dma_tile(vbase, krs, tile_kb(0), p.Skv, vst, w, lane, true);
  }
  if (n > 1) {
    dma_tile(kbase, krs, tile_kb(1), p.Skv, kst + kTileElems, w, lane, false);
    dma_tile(vbase, krs, tile_kb(1), p.Skv, vst + kTileElems, w, lane, true);
    wait_vmcnt<4>();
  } else {
    wait_vmcnt<0>();
  }
  __syncthreads();

  int stage = 0;
  for (int j = 0; j < n; ++j) {
    // issue tile j+2 into the stage tile j-1 used (all waves passed the barrier after it)
    const int st2 = stage == 0 ? 2 : stage - 1;
    const bool pre = j + 2 < n;
    if (pre) {
      dma_tile(kbase, krs, tile_kb(j + 2), p.Skv, kst + st2 * kTileElems, w, lane, false);
      dma_tile(vbase, krs, tile_kb(j + 2), p.Skv, vst + st2 * kTileElems, w, lane, true);
    }
    const int cls = tile_cls(j);
    if (cls != 0) {
      const char* Kt = reinterpret_cast<const char*>(kst + stage * kTileElems);
      const char* Vt = reinterpret_cast<const char*>(vst + stage * kTileElems);
      const int kb = tile_kb(j);
      f32x16 S[2];
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ds = 0; ds < NDS; ++ds) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kt + k_off[kb2][ds]);
          S[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ds], ds == 0 ? f32x16{} : S[kb2], 0, 0, 0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (CAP) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int i = 0; i < 16; ++i) S[kb2][i] = capped_log2(S[kb2][i], p.cap_k2, p.cap_log2);
      }
      if (cls != 2 || (kb + 1) * kBlockKV > p.Skv) apply_mask(S, p, b, kb * kBlockKV, lg, qpos, qseg);
      softmax_step<NDB, CAP>(S, O, m_ref, l_acc, p);
      bf16x8 P[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          f32x2 two = {S[ks >> 1][(ks & 1) * 8 + 2 * jj], S[ks >> 1][(ks & 1) * 8 + 2 * jj + 1]};
          bf16x2 pk = __builtin_convertvector(two, bf16x2);
          P[ks][2 * jj] = pk[0];
          P[ks][2 * jj + 1] = pk[1];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const char* vp = Vt + (ks * 16 + v_row) * 256 + v_col[db];
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp));
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp + 8 * 256));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[ks], O[db], 0, 0, 0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // tile j+1 must have landed before the barrier; tile j+2's loads may stay in flight
    if (pre) wait_vmcnt<4>();
    else wait_vmcnt<0>();
    __syncthreads();
    stage = stage == 2 ? 0 : stage + 1;
  }
  epilogue<NDB>(O, m_ref, l_acc, p, b, h, q_ok ? q_row : p.Sq, lg);
}

template <typename K>
hipError_t launch_g(K kernel, const AttnParams& p, hipStream_t s) {
  const int nQp = (p.nQb + 1) / 2;
  const int64_t T = (int64_t)p.B * p.H * nQp;
  const int64_t grid = 8 * ((T + 7) / 8);
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kGThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_g8(const AttnParams& p, hipStream_t s) {
  if (p.softcap_on) return launch_g(attn_fwd_bf16_g8<true>, p, s);
  return launch_g(attn_fwd_bf16_g8<false>, p, s);
}

}  // namespace ram
