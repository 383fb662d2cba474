// Block-sparse attention forward for one KV chunk: 8-wave, software-pipelined variant.
//
// Computes exactly what attn_fwd.hip computes (the per-ring-step kernel call of
// the ejkernel ring-splash source page, _ring_attention_forward, with the
// _update_out_and_lse merge as epilogue). The schedule overlaps the matrix
// core and the vector ALU inside every wave, and across the two waves that
// share each SIMD:
//
//  * One workgroup = 8 waves = two groups of 4 waves, each group one 128-row
//    q tile of the same head; a wave owns 32 query rows. Both groups consume
//    the same K/V tiles.
//  * Loop iteration j issues one interleaved block: the MFMA stream
//    O += P_{j-1} V_{j-1} and S_{j+1} = Q K_{j+1}^T (32 MFMAs) runs alongside
//    the VALU stream of the online softmax of S_j. The block is 8 chunks of
//    (next chunk's LDS operand reads, 4 MFMAs, one softmax slice), fenced with
//    sched_barrier. The rare O rescale (when a row's running max grows by
//    more than 2^8) follows the block, after PV(j-1) has landed in O.
//  * K and V go from HBM straight to LDS (global_load_lds_dwordx4) two
//    iterations ahead of use: iteration j issues K_{j+3} and V_{j+1} into
//    3-stage rings and waits only for the loads of iteration j-1.
//  * LDS rows are dense 256-byte rows with XOR-swizzled 16-byte chunks:
//    chunk ^ (row & 15) for K (conflict-free A-operand reads) and
//    chunk ^ 4*(row & 3) for V (conflict-free ds_read_b64_tr_b16).
//  * The block mask stays at the 128 x 64 kernel tile: the workgroup walks
//    the union of its two tile rows. A group's EMPTY tiles are computed as
//    fully masked (zero weights), which keeps the block branch-free.
#include "attn_common.h"

namespace ram {
namespace {

using namespace attn;

constexpr int kPWaves = 8;
constexpr int kPThreads = 64 * kPWaves;
constexpr int kPD = 128;
constexpr int kPStages = 3;
constexpr int kPTile = kBlockKV * kPD;      // one K or V tile (16 KB)

__device__ __forceinline__ bool decode_work_p(const AttnParams& p, int nQp, int& b, int& h, int& qp) {
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

// Tile kb of K or V into LDS: wave w fills rows [8w, 8w+8) with two 4-row
// (1 KB) slabs; lane l writes physical chunk l & 15 of row l >> 4.
__device__ __forceinline__ void dma_tile_p(const __bf16* gbase, int64_t krs, int kb, int skv, __bf16* tile, int w,
                                           int lane, bool is_v) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * w + 4 * i + (lane >> 4);
    const int phys = lane & 15;
    const int logical = is_v ? (phys ^ (4 * (r & 3))) : (phys ^ (r & 15));
    const int row = min(kb * kBlockKV + r, skv - 1);
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(gbase + row * krs + logical * 8),
                                     (void __attribute__((address_space(3)))*)(tile + (8 * w + 4 * i) * kPD), 16, 0, 0);
  }
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

template <bool CAP>
__device__ __forceinline__ void block(const char* Vt, const char* Kt, int lane, const bf16x8 (&qf)[8],
                                      f32x16 (&O)[4], f32x16 (&Sc)[2], f32x16 (&Sn)[2], bf16x8 (&P)[4],
                                      float& m_ref, float& l_acc, float& alpha, float scale_log2) {
  const int ln = lane & 31, lg = lane >> 5;
  const int r4 = (lane & 15) >> 2, hs = (lane >> 4) & 1;
  // operands of MFMA group gi: 0-3 PV (ks = gi, db = 0..3), 4-7 QK (ds = 2*(gi-4) + u, kb2 = 0, 1)
  bf16x8 fr[2][4];
  auto frag = [&](int gi, bf16x8 (&dst)[4]) {
    if (gi < 4) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int c = ((db * 4 + 2 * hs + ((lane & 3) >> 1)) ^ (4 * r4)) * 16 + (lane & 1) * 8;
        const char* vp = Vt + (gi * 16 + 4 * lg + r4) * 256 + c;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp + 8 * 256));
        dst[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const int ds = 2 * (gi - 4) + u;
          dst[2 * u + kb2] = *reinterpret_cast<const bf16x8*>(Kt + (kb2 * 32 + ln) * 256 + (((2 * ds + lg) ^ (ln & 15)) * 16));
        }
    }
  };
  auto mfma = [&](int gi, const bf16x8 (&src)[4]) {
    if (gi < 4) {
#pragma unroll
      for (int db = 0; db < 4; ++db) O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(src[db], P[gi], O[db], 0, 0, 0);
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const int ds = 2 * (gi - 4) + u;
          Sn[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(src[2 * u + kb2], qf[ds], ds == 0 ? f32x16{} : Sn[kb2], 0, 0, 0);
        }
    }
  };
  float mx, msub;
  auto slice = [&](int sl) {
    if (sl == 0) {
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        t[u] = fmaxf(fmaxf(Sc[u >> 2][(u & 3) * 4 + 0], Sc[u >> 2][(u & 3) * 4 + 1]),
                     fmaxf(Sc[u >> 2][(u & 3) * 4 + 2], Sc[u >> 2][(u & 3) * 4 + 3]));
      mx = fmaxf(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])), fmaxf(fmaxf(t[4], t[5]), fmaxf(t[6], t[7])));
    } else if (sl == 1) {
      const float m = pair_max(mx);
      const float umax = CAP ? m : m * scale_log2;
      const bool need = umax > m_ref + kRescaleThreshold;
      const float m_new = need ? umax : m_ref;
      alpha = need ? fast_exp2(m_ref - m_new) : 1.0f;
      m_ref = m_new;
      msub = (m_new == neg_inf()) ? 0.0f : m_new;
    } else if (sl < 6) {
      const int e = sl - 2;                  // 8 scores per slice
      const int kb2 = e >> 1, i0 = (e & 1) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float s = Sc[kb2][i0 + i];
        Sc[kb2][i0 + i] = CAP ? fast_exp2(s - msub) : fast_exp2(__builtin_fmaf(s, scale_log2, -msub));
      }
    } else if (sl == 6) {
      float t[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        t[u] = (Sc[u >> 2][(u & 3) * 4 + 0] + Sc[u >> 2][(u & 3) * 4 + 1]) +
               (Sc[u >> 2][(u & 3) * 4 + 2] + Sc[u >> 2][(u & 3) * 4 + 3]);
      l_acc = l_acc * alpha + (((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7])));
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          f32x2 two = {Sc[ks >> 1][(ks & 1) * 8 + 2 * jj], Sc[ks >> 1][(ks & 1) * 8 + 2 * jj + 1]};
          bf16x2 pk = __builtin_convertvector(two, bf16x2);
          P[ks][2 * jj] = pk[0];
          P[ks][2 * jj + 1] = pk[1];
        }
    }
  };
  __builtin_amdgcn_sched_barrier(0);
  frag(0, fr[0]);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    if (c + 1 < 8) frag(c + 1, fr[(c + 1) & 1]);
    mfma(c, fr[c & 1]);
    slice(c);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <bool CAP>
__global__ __launch_bounds__(kPThreads, 1) void attn_fwd_bf16_g8p(AttnParams p) {
  constexpr int NDS = kPD / 16;
  __shared__ __attribute__((aligned(16))) __bf16 kst[kPStages * kPTile];
  __shared__ __attribute__((aligned(16))) __bf16 vst[kPStages * kPTile];
  __shared__ uint32_t ulist[kMaxMaskCols];
  __shared__ int wsum[kPWaves];

  const int nQp = (p.nQb + 1) >> 1;
  int b, h, qp;
  if (!decode_work_p(p, nQp, b, h, qp)) return;
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
  for (int base = 0; base < p.nKb; base += kPThreads) {
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
    for (int i = 0; i < kPWaves; ++i) {
      off += (i < w) ? wsum[i] : 0;
      total += wsum[i];
    }
    if (f) ulist[off + before] = (uint32_t)kb | (ca << 16) | (cb << 24);
    n += total;
    __syncthreads();
  }
  if (n == 0 && p.mode == 1 && p.sinks == nullptr) return;

  bf16x8 qf[NDS];
  {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.q_stride_b +
                         ((int64_t)(q_ok ? q_row : 0) * p.H + h) * kPD;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      bf16x8 t = *reinterpret_cast<const bf16x8*>(qrow + ds * 16 + lg * 8);
      qf[ds] = q_ok ? t : bf16x8{};
    }
  }
  const int qrow_c = q_ok ? q_row : p.Sq - 1;
  const int qpos = p.q_pos ? p.q_pos[(int64_t)b * p.qm_stride_b + qrow_c] : p.q_pos_base + q_row;
  const int qseg = p.q_seg ? p.q_seg[(int64_t)b * p.qm_stride_b + qrow_c] : 0;
  float m_ref = neg_inf(), l_acc = 0.0f, alpha = 1.0f;
  if (p.sinks) {
    m_ref = p.sinks[h] * kLog2e;
    l_acc = (lg == 0) ? 1.0f : 0.0f;
  }
  f32x16 O[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) O[db] = f32x16{};
  bf16x8 P[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) P[ks] = bf16x8{};

  const int64_t krs = (int64_t)p.Hkv * kPD;
  const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + (int64_t)b * p.kv_stride_b + g * kPD;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.kv_stride_b + g * kPD;
  auto tile_kb = [&](int j) { return (int)(ulist[j] & 0xffffu); };
  auto tile_cls = [&](int j) { return (int)((ulist[j] >> (16 + 8 * grp)) & 0xffu); };

  // ---- prologue: K_0, K_1 resident; S_0; then K_2 and V_0 in flight.
  // V stage 2 (read with zero weights by iteration 0) is cleared first.
  for (int i = tid; i < kPTile / 8; i += kPThreads)
    reinterpret_cast<uint4*>(vst + 2 * kPTile)[i] = make_uint4(0, 0, 0, 0);
  if (n > 0) dma_tile_p(kbase, krs, tile_kb(0), p.Skv, kst, w, lane, false);
  if (n > 1) dma_tile_p(kbase, krs, tile_kb(1), p.Skv, kst + kPTile, w, lane, false);
  wait_vm<0>();
  __syncthreads();
  f32x16 Sa[2], Sb[2];
  {
    const char* Kt = reinterpret_cast<const char*>(kst);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kt + (kb2 * 32 + ln) * 256 + (((2 * ds + lg) ^ (ln & 15)) * 16));
        Sa[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ds], ds == 0 ? f32x16{} : Sa[kb2], 0, 0, 0);
      }
  }
  __syncthreads();   // every wave is done reading K_0 before iteration 0 loads K_3 over it
  if (n > 2) dma_tile_p(kbase, krs, tile_kb(2), p.Skv, kst + 2 * kPTile, w, lane, false);
  if (n > 0) dma_tile_p(vbase, krs, tile_kb(0), p.Skv, vst, w, lane, true);

  // stage of tile t in each 3-stage ring: t % 3 (tracked incrementally)
  int st_j = 0;   // tile j
  auto step = [&](int j, f32x16 (&S_cur)[2], f32x16 (&S_next)[2]) {
    const int st_n = st_j == 2 ? 0 : st_j + 1;     // tile j+1
    const int st_p = st_j == 0 ? 2 : st_j - 1;     // tile j-1 (== tile j+2 == tile j+3 - 1 ... ring of 3)
    // loads two iterations ahead: K_{j+3} into the stage of K_j, V_{j+1} into the stage of V_{j-2} (== tile j+1)
    const bool ldk = j + 3 < n, ldv = j + 1 < n;
    if (ldk) dma_tile_p(kbase, krs, tile_kb(j + 3), p.Skv, kst + st_j * kPTile, w, lane, false);
    if (ldv) dma_tile_p(vbase, krs, tile_kb(j + 1), p.Skv, vst + st_n * kPTile, w, lane, true);
    const int cls = tile_cls(j);
    const int kb = tile_kb(j);
    if constexpr (CAP) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) S_cur[kb2][i] = capped_log2(S_cur[kb2][i], p.cap_k2, p.cap_log2);
    }
    if (cls == 0) {
      S_cur[0] = f32x16{} + neg_inf();
      S_cur[1] = f32x16{} + neg_inf();
    } else if (cls != 2 || (kb + 1) * kBlockKV > p.Skv) {
      apply_mask(S_cur, p, b, kb * kBlockKV, lg, qpos, qseg);
    }
    const char* Vt = reinterpret_cast<const char*>(vst + st_p * kPTile);   // V_{j-1}
    const char* Kt = reinterpret_cast<const char*>(kst + st_n * kPTile);   // K_{j+1}
    block<CAP>(Vt, Kt, lane, qf, O, S_cur, S_next, P, m_ref, l_acc, alpha, p.scale_log2);
    if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
      for (int db = 0; db < 4; ++db) O[db] *= alpha;
    }
    // K_{j+2} and V_j (issued one iteration ago) must land before the barrier
    if (ldk) wait_vm<4>();
    else if (ldv) wait_vm<2>();
    else wait_vm<0>();
    __syncthreads();
    st_j = st_n;
  };

  int j = 0;
  for (; j + 1 < n; j += 2) {
    step(j, Sa, Sb);
    step(j + 1, Sb, Sa);
  }
  if (j < n) step(j, Sa, Sb);

  // last PV: O += P_{n-1} V_{n-1}; V_{n-1} is in the stage before st_j
  if (n > 0) {
    const int st_p = st_j == 0 ? 2 : st_j - 1;
    const char* Vt = reinterpret_cast<const char*>(vst + st_p * kPTile);
    const int r4 = (lane & 15) >> 2, hs = (lane >> 4) & 1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int c = ((db * 4 + 2 * hs + ((lane & 3) >> 1)) ^ (4 * r4)) * 16 + (lane & 1) * 8;
        const char* vp = Vt + (ks * 16 + 4 * lg + r4) * 256 + c;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp + 8 * 256));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[ks], O[db], 0, 0, 0);
      }
  }
  epilogue<4>(O, m_ref, l_acc, p, b, h, q_ok ? q_row : p.Sq, lg);
}

template <typename K>
hipError_t launch_gp(K kernel, const AttnParams& p, hipStream_t s) {
  const int nQp = (p.nQb + 1) / 2;
  const int64_t T = (int64_t)p.B * p.H * nQp;
  const int64_t grid = 8 * ((T + 7) / 8);
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kPThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_g8p(const AttnParams& p, hipStream_t s) {
  if (p.softcap_on) return launch_gp(attn_fwd_bf16_g8p<true>, p, s);
  return launch_gp(attn_fwd_bf16_g8p<false>, p, s);
}

}  // namespace ram
