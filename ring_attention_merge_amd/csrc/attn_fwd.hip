// Block-sparse attention forward for one KV chunk, with a fused LSE-merge epilogue.
//
// What it computes: the per-ring-step kernel call of the ejkernel ring-splash
// source page (_ring_attention_forward): attention of q over one KV chunk,
// returning the chunk output and log-sum-exp, then (merge mode) the fold of
// _update_out_and_lse into the running state. Masking follows the Kvax
// flash_attention arguments (positions, segment IDs, padding segment).
//
// Design for gfx950 (CDNA4):
//  * One workgroup = 4 waves = 128 query rows of one head; each wave owns 32
//    rows. The workgroup walks the compacted list of non-EMPTY kv tiles of
//    its row of tiles (64 keys each); FULL tiles skip all mask arithmetic.
//  * Scores are computed transposed, S^T = K * Q^T, with
//    v_mfma_f32_32x32x16_bf16: A = K tile from LDS (32 keys x 16 dims), B = Q
//    held in registers for the whole loop. In the 32x32 accumulator layout a
//    lane owns one query row (lane & 31) and 16 keys, so row max / row sum
//    are in-lane plus one v_permlane32_swap with the partner lane.
//  * O^T = V^T * P^T with the same instruction: P leaves the S accumulator as
//    packed bf16 and feeds the B operand directly (no LDS round trip). V is
//    stored row-major in LDS like K and its A operand is read with gfx950's
//    transposing LDS read (ds_read_b64_tr_b16): two reads give each lane 8
//    keys of one head-dim column, in the key order P arrives in.
//  * LDS pitches keep every access conflict-free: K rows are 272 B (16 lanes
//    reading 16 B from 16 consecutive rows hit 16 distinct bank quads), V rows
//    are 320 B (a transposing read covers 4 rows x 64 B, i.e. all 64 banks).
//  * K / V tiles are double-buffered in LDS; the next tile's global loads are
//    issued before the current tile's math, one barrier per tile.
//  * Online softmax in base 2 with the scale folded into one FMA; the running
//    max is only raised when a row's max grows by more than 2^8 (the weights
//    stay <= 256, exact in the final normalisation), so most tiles skip the
//    O rescale.
//  * Workgroup ids are mapped so that each XCD (ids are dealt round-robin over
//    the 8 XCDs) gets a contiguous range of (batch, kv head) groups, keeping
//    their K/V in that XCD's L2, and within it heavier (later) q tiles first.
#include <cstdlib>
#include <cstring>

#include "attn_common.h"

namespace ram {
namespace {

using namespace attn;

// ------------------------------------------------------------------------------ bf16
template <int D, bool CAP, bool BITS>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16(AttnParams p) {
  constexpr int BK = kBlockKV;
  constexpr int NDS = D / 16;      // k-steps of S^T = K Q^T
  constexpr int NDB = D / 32;      // 32-row blocks of O^T
  constexpr int KP = D + 8;        // K row pitch (elements): 272 B for D = 128
  constexpr int VP = D + 32;       // V row pitch (elements): 320 B for D = 128
  constexpr int K_ELEMS = BK * KP;
  constexpr int V_ELEMS = BK * VP;
  constexpr int CH = D / 8;               // 16-byte chunks per row
  constexpr int RPP = kThreads / CH;      // rows per load pass
  constexpr int NPK = BK / RPP;           // load passes per tensor
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * (K_ELEMS + V_ELEMS)];

  int b, h, qb;
  if (!decode_work(p, b, h, qb)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int ln = lane & 31, lg = lane >> 5;
  const int G = p.H / p.Hkv;
  const int g = h / G;
  const int q_row = qb * kBlockQ + w * 32 + ln;
  const bool q_ok = q_row < p.Sq;

  const int64_t mrow = (int64_t)b * p.nQb + qb;
  const int cnt = p.row_cnt[mrow];
  // a merge with nothing to add is the identity (unless the result must be
  // converted to its final type, which the epilogue does for empty rows)
  if (cnt == 0 && p.mode == 1 && p.sinks == nullptr && p.out_final == nullptr) return;
  const auto cols = as_const_space(p.col_idx + mrow * p.nKb);
  const auto cls = as_const_space(p.tile_class + mrow * p.nKb);

  // Q fragments (B operand): lane holds row q_row, dims ds*16 + lg*8 .. +7.
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

  const int64_t krs = (int64_t)p.Hkv * D;  // key row stride
  const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + (int64_t)b * p.kv_stride_b + g * D;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.kv_stride_b + g * D;
  const int kc = tid % CH, kr0 = tid / CH;
  uint4 kreg[NPK], vreg[NPK];
  // Transposing-read address of this lane inside a V tile (see lds_read_tr16):
  // row 4*lg + (i >> 2), column 16*half + 4*(i & 3), i = lane & 15, half = (lane >> 4) & 1.
  const int vtr_off = (4 * lg + ((lane & 15) >> 2)) * VP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // K / V tiles come in through buffer loads whose resource covers exactly the
  // tile's rows that exist: rows past Skv read as zero, with no branches.
  const uint32_t row_bytes = (uint32_t)krs * 2;
  uint32_t voff[NPK];
#pragma unroll
  for (int i = 0; i < NPK; ++i) voff[i] = (uint32_t)(kr0 + i * RPP) * row_bytes + kc * 16;
  auto gload = [&](int kb) {
    const int k0 = kb * BK;
    const uint32_t bytes = (uint32_t)min(p.Skv - k0, BK) * row_bytes;
    const auto kr = tile_rsrc(kbase + (int64_t)k0 * krs, bytes);
    const auto vr = tile_rsrc(vbase + (int64_t)k0 * krs, bytes);
#pragma unroll
    for (int i = 0; i < NPK; ++i) kreg[i] = buffer_load_16(kr, voff[i]);
#pragma unroll
    for (int i = 0; i < NPK; ++i) vreg[i] = buffer_load_16(vr, voff[i]);
  };
  auto lstore = [&](int buf) {
    __bf16* Ks = smem + buf * (K_ELEMS + V_ELEMS);
    __bf16* Vs = Ks + K_ELEMS;
#pragma unroll
    for (int i = 0; i < NPK; ++i) {
      *reinterpret_cast<uint4*>(Ks + (kr0 + i * RPP) * KP + kc * 8) = kreg[i];
      *reinterpret_cast<uint4*>(Vs + (kr0 + i * RPP) * VP + kc * 8) = vreg[i];
    }
  };

  // The tile list is read ahead: entry it+2 and the mask flag of tile it+1
  // are loaded while tile it is processed, so no iteration waits on them.
  // mask kind of a tile: 0 none, 1 from positions / segments, 2 from its stored bits
  auto needs_mask = [&](int kb) {
    const int c = cls[kb];
    if constexpr (BITS)
      if (c == 1) return 2;
    return (c != 2 || (kb + 1) * BK > p.Skv) ? 1 : 0;
  };
  int kb_cur = cnt > 0 ? cols[0] : 0;
  int kb_nxt = cnt > 1 ? cols[1] : kb_cur;
  int mk_cur = cnt > 0 ? needs_mask(kb_cur) : 0;   // no class array to read when the row is empty
  if (cnt > 0) {
    gload(kb_cur);
    lstore(0);
  }
  __syncthreads();

  for (int it = 0; it < cnt; ++it) {
    const int kb = kb_cur;
    const int need_mask = mk_cur;
    const int buf = it & 1;
    const bool has_next = it + 1 < cnt;
    const int kb_nn = cols[min(it + 2, cnt - 1)];
    const int mk_nxt = needs_mask(kb_nxt);
    if (has_next) gload(kb_nxt);
    const __bf16* Ks = smem + buf * (K_ELEMS + V_ELEMS);
    const __bf16* Vs = Ks + K_ELEMS;

    f32x16 S[2];
    S[0] = f32x16{};
    S[1] = f32x16{};
    // MFMA sections run at raised wave priority so that the other wave on
    // this SIMD fills the matrix core's shadow with its softmax arithmetic.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + (kb2 * 32 + ln) * KP + ds * 16 + lg * 8);
        S[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ds], S[kb2], 0, 0, 0);
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
    if (BITS && need_mask == 2)
      apply_bits(S, p.mask_bits + ((mrow * p.nKb + kb) * kBlockQ + w * 32 + ln) * 2, lg);
    else if (need_mask)
      apply_mask(S, p, b, kb * BK, lg, qpos, qseg);
    softmax_step<NDB, CAP>(S, O, m_ref, l_acc, p);

    bf16x8 P[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x2 two = {S[ks >> 1][(ks & 1) * 8 + 2 * j], S[ks >> 1][(ks & 1) * 8 + 2 * j + 1]};
        bf16x2 pk = __builtin_convertvector(two, bf16x2);
        P[ks][2 * j] = pk[0];
        P[ks][2 * j + 1] = pk[1];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        // keys ks*16 + 4*lg + 0..3 and ks*16 + 8 + 4*lg + 0..3 of column db*32 + (lane & 31)
        const __bf16* vp = Vs + ks * 16 * VP + db * 32 + vtr_off;
        const s16x4 lo = lds_read_tr16(vp);
        const s16x4 hi = lds_read_tr16(vp + 8 * VP);
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[ks], O[db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    if (has_next) lstore(buf ^ 1);
    __syncthreads();
    kb_cur = kb_nxt;
    kb_nxt = kb_nn;
    mk_cur = mk_nxt;
  }
  epilogue<NDB>(O, m_ref, l_acc, p, b, h, q_row, lg);
}

// ------------------------------------------------------------------------------ fp32
// Same structure with v_mfma_f32_32x32x2_f32: one fp32 per lane per operand,
// K and V kept row-major in LDS, the fp32 weights feed PV directly.
template <int D, bool CAP, bool BITS>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_f32(AttnParams p) {
  constexpr int BK = kBlockKV;
  constexpr int NDB = D / 32;
  constexpr int NDS = D / 2;
  constexpr int KP = D + 4;                 // row pitch (floats), keeps float4 stores aligned
  constexpr int ELEMS = BK * KP;
  constexpr int CH = D / 4;                 // float4 chunks per row
  constexpr int NLD = BK * CH / kThreads;   // float4 loads per thread per tensor
  __shared__ __attribute__((aligned(16))) float smem[2 * 2 * ELEMS];

  int b, h, qb;
  if (!decode_work(p, b, h, qb)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int ln = lane & 31, lg = lane >> 5;
  const int G = p.H / p.Hkv;
  const int g = h / G;
  const int q_row = qb * kBlockQ + w * 32 + ln;
  const bool q_ok = q_row < p.Sq;

  const int64_t mrow = (int64_t)b * p.nQb + qb;
  const int cnt = p.row_cnt[mrow];
  if (cnt == 0 && p.mode == 1 && p.sinks == nullptr) return;
  const auto cols = as_const_space(p.col_idx + mrow * p.nKb);
  const auto cls = as_const_space(p.tile_class + mrow * p.nKb);

  float qf[NDS];
  {
    const float* qrow = reinterpret_cast<const float*>(p.q) + (int64_t)b * p.q_stride_b +
                        ((int64_t)(q_ok ? q_row : 0) * p.H + h) * D;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qf[ds] = q_ok ? qrow[ds * 2 + lg] : 0.0f;
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
  const float* kbase = reinterpret_cast<const float*>(p.k) + (int64_t)b * p.kv_stride_b + g * D;
  const float* vbase = reinterpret_cast<const float*>(p.v) + (int64_t)b * p.kv_stride_b + g * D;
  float4 kreg[NLD], vreg[NLD];

  auto gload = [&](int kb) {
    const int k0 = kb * BK;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tid + i * kThreads;
      const int row = k0 + idx / CH, c = idx % CH;
      const bool ok = row < p.Skv;
      kreg[i] = ok ? *reinterpret_cast<const float4*>(kbase + row * krs + c * 4) : make_float4(0, 0, 0, 0);
      vreg[i] = ok ? *reinterpret_cast<const float4*>(vbase + row * krs + c * 4) : make_float4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
    float* Ks = smem + buf * 2 * ELEMS;
    float* Vs = Ks + ELEMS;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int idx = tid + i * kThreads;
      const int row = idx / CH, c = idx % CH;
      *reinterpret_cast<float4*>(Ks + row * KP + c * 4) = kreg[i];
      *reinterpret_cast<float4*>(Vs + row * KP + c * 4) = vreg[i];
    }
  };

  // The tile list is read ahead: entry it+2 and the mask flag of tile it+1
  // are loaded while tile it is processed, so no iteration waits on them.
  // mask kind of a tile: 0 none, 1 from positions / segments, 2 from its stored bits
  auto needs_mask = [&](int kb) {
    const int c = cls[kb];
    if constexpr (BITS)
      if (c == 1) return 2;
    return (c != 2 || (kb + 1) * BK > p.Skv) ? 1 : 0;
  };
  int kb_cur = cnt > 0 ? cols[0] : 0;
  int kb_nxt = cnt > 1 ? cols[1] : kb_cur;
  int mk_cur = cnt > 0 ? needs_mask(kb_cur) : 0;   // no class array to read when the row is empty
  if (cnt > 0) {
    gload(kb_cur);
    lstore(0);
  }
  __syncthreads();

  for (int it = 0; it < cnt; ++it) {
    const int kb = kb_cur;
    const int need_mask = mk_cur;
    const int buf = it & 1;
    const bool has_next = it + 1 < cnt;
    const int kb_nn = cols[min(it + 2, cnt - 1)];
    const int mk_nxt = needs_mask(kb_nxt);
    if (has_next) gload(kb_nxt);
    const float* Ks = smem + buf * 2 * ELEMS;
    const float* Vs = Ks + ELEMS;

    f32x16 S[2];
    S[0] = f32x16{};
    S[1] = f32x16{};
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const float a = Ks[(kb2 * 32 + ln) * KP + ds * 2 + lg];
        S[kb2] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf[ds], S[kb2], 0, 0, 0);
      }
    }
    if constexpr (CAP) {
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int i = 0; i < 16; ++i) S[kb2][i] = capped_log2(S[kb2][i], p.cap_k2, p.cap_log2);
    }
    if (BITS && need_mask == 2)
      apply_bits(S, p.mask_bits + ((mrow * p.nKb + kb) * kBlockQ + w * 32 + ln) * 2, lg);
    else if (need_mask)
      apply_mask(S, p, b, kb * BK, lg, qpos, qseg);
    softmax_step<NDB, CAP>(S, O, m_ref, l_acc, p);

#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb2 * 32 + 8 * (i >> 2) + 4 * lg + (i & 3);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const float a = Vs[key * KP + db * 32 + ln];
          O[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, S[kb2][i], O[db], 0, 0, 0);
        }
      }
    }
    if (has_next) lstore(buf ^ 1);
    __syncthreads();
    kb_cur = kb_nxt;
    kb_nxt = kb_nn;
    mk_cur = mk_nxt;
  }
  epilogue<NDB>(O, m_ref, l_acc, p, b, h, q_row, lg);
}

template <typename K>
hipError_t launch(K kernel, const AttnParams& p, hipStream_t s) {
  const int64_t T = (int64_t)p.B * p.H * p.nQb;
  const int64_t grid = 8 * ((T + 7) / 8);
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

// Instantiations by (soft cap, tile bits); BITS kernels mask PARTIAL tiles by their stored bits.
template <template <bool, bool> class K>
hipError_t launch_cb(const AttnParams& p, hipStream_t s) {
  const bool cap = p.softcap_on != 0, bits = p.mask_bits != nullptr;
  if (cap) return bits ? launch(K<true, true>::fn, p, s) : launch(K<true, false>::fn, p, s);
  return bits ? launch(K<false, true>::fn, p, s) : launch(K<false, false>::fn, p, s);
}
template <int D>
struct Bf16Staged {
  template <bool CAP, bool BITS>
  struct K {
    static constexpr auto fn = attn_fwd_bf16<D, CAP, BITS>;
  };
};
template <int D>
struct F32 {
  template <bool CAP, bool BITS>
  struct K {
    static constexpr auto fn = attn_fwd_f32<D, CAP, BITS>;
  };
};

}  // namespace

hipError_t launch_attn(const AttnParams& p, int dtype, hipStream_t s) {
  if (dtype == 1) {
    if (p.D != 64) return hipErrorInvalidValue;   // bf16 D = 128 runs launch_attn_alt
    return launch_cb<Bf16Staged<64>::K>(p, s);
  }
  if (p.D == 128) return launch_cb<F32<128>::K>(p, s);
  return launch_cb<F32<64>::K>(p, s);
}

}  // namespace ram
