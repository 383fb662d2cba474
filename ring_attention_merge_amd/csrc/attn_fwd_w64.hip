// Block-sparse attention forward for one KV chunk: wide-wave variant.
//
// Computes exactly what attn_fwd.hip computes (the per-ring-step kernel call of
// the ejkernel ring-splash source page, _ring_attention_forward, with the
// _update_out_and_lse merge as epilogue). The schedule is built around two
// measured limits of gfx950: LDS operand bandwidth (a wave of 32 query rows
// needs 1 KB of LDS operand per 32x32x16 MFMA; the transposing LDS read
// sustains only ~56 B/clk/CU) and the serial phases of a wave
// (QK -> softmax -> PV):
//
//  * One workgroup = 4 waves, one per SIMD; each wave owns 64 query rows (two
//    32-row blocks), so every K or V operand read from LDS feeds two MFMAs.
//  * Keys advance 32 at a time (half of a 64-key mask tile). Iteration t
//    interleaves, inside one wave, an MFMA stream (O += P_{t-1} V_{t-1} and
//    S_{t+1} = Q K_{t+1}^T: 32 MFMAs) with the VALU stream of the online
//    softmax of S_t. The streams are written as 8 chunks (4 MFMAs + one
//    softmax slice each) fenced with sched_barrier; each chunk reads the next
//    chunk's LDS operands first.
//  * The running max only moves when a row's max grows by more than 2^8, so
//    the O rescale (which must follow PV(t-1)) is rare and runs after the
//    interleaved block.
//  * K and V go from HBM straight to LDS (global_load_lds_dwordx4, no VGPR
//    staging) into dense 256-byte rows with XOR-swizzled 16-byte chunks:
//    chunk ^ (row & 15) for K (conflict-free A-operand reads of 16 rows) and
//    chunk ^ 4*(row & 3) for V (conflict-free transposing reads of 4 rows x
//    64 bytes). K_{t+2} and V_t load during iteration t.
//  * The block mask stays at the 128 x 64 kernel tile: the workgroup walks
//    the union of its two 128-row tile rows; waves 0-1 take their tile
//    classes from the first row, waves 2-3 from the second.
#include "attn_common.h"

namespace ram {
namespace {

using namespace attn;

constexpr int kWWaves = 4;
constexpr int kWThreads = 64 * kWWaves;
constexpr int kSub = 32;                 // keys per step
constexpr int kD = 128;
constexpr int kSubElems = kSub * kD;     // one K or V step in LDS (8 KB)

__device__ __forceinline__ bool decode_work_w(const AttnParams& p, int nQt, int& b, int& h, int& qt) {
  const int G = p.H / p.Hkv;
  const int64_t T = (int64_t)p.B * p.Hkv * nQt * G;
  const int64_t per = (T + 7) / 8;
  const int64_t id = blockIdx.x;
  const int64_t item = (id & 7) * per + (id >> 3);
  if (item >= T) return false;
  const int hg = (int)(item % G);
  const int64_t r = item / G;
  const int qrev = (int)(r % nQt);
  const int64_t bg = r / nQt;
  const int g = (int)(bg % p.Hkv);
  b = (int)(bg / p.Hkv);
  h = g * G + hg;
  qt = nQt - 1 - qrev;
  return true;
}

// One 32-key step of K or V: wave w fills rows [8w, 8w+8), one 4-row (1 KB)
// slab per instruction; lane l writes physical chunk l & 15 of row l >> 4.
__device__ __forceinline__ void load_step(const __bf16* gbase, int64_t krs, int k0, int skv, __bf16* tile,
                                          int w, int lane, bool is_v) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * w + 4 * i + (lane >> 4);
    const int phys = lane & 15;
    const int logical = is_v ? (phys ^ (4 * (r & 3))) : (phys ^ (r & 15));
    const int row = min(k0 + r, skv - 1);                 // rows past the end are masked
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(gbase + row * krs + logical * 8),
                                     (void __attribute__((address_space(3)))*)(tile + (8 * w + 4 * i) * kD), 16, 0, 0);
  }
}

struct Wave {
  // LDS byte offsets of this lane's operands inside a step
  int k_off[8];        // K A operand for ds = 0..7: row ln, logical chunk 2*ds + lg
  int v_off[2][2][4];  // V transposing reads [ks][r][db]
};

__device__ __forceinline__ void wave_offsets(Wave& wv, int lane) {
  const int ln = lane & 31, lg = lane >> 5;
#pragma unroll
  for (int ds = 0; ds < 8; ++ds) wv.k_off[ds] = ln * 256 + (((2 * ds + lg) ^ (ln & 15)) * 16);
  const int r4 = (lane & 15) >> 2;
  const int hs = (lane >> 4) & 1;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int row = ks * 16 + 8 * r + 4 * lg + r4;
        const int c = (db * 4 + 2 * hs + ((lane & 3) >> 1)) ^ (4 * r4);
        wv.v_off[ks][r][db] = row * 256 + c * 16 + (lane & 1) * 8;
      }
}

__device__ __forceinline__ bf16x8 read_v(const char* Vt, const Wave& wv, int ks, int db) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(Vt + wv.v_off[ks][0][db]));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(Vt + wv.v_off[ks][1][db]));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Masking of one 32-key step for a 32-row block: keys k0 + 8*(i>>2) + 4*lg + (i&3).
__device__ __forceinline__ void mask_step(f32x16& S, const AttnParams& p, int b, int k0, int lg, int qpos, int qseg) {
  const int32_t* kvp = p.kv_pos ? p.kv_pos + (int64_t)b * p.kvm_stride_b : nullptr;
  const int32_t* kvs = p.kv_seg ? p.kv_seg + (int64_t)b * p.kvm_stride_b : nullptr;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int key = k0 + 8 * (i >> 2) + 4 * lg + (i & 3);
    bool ok = key < p.Skv;
    if (ok && p.causal) ok = (kvp ? kvp[key] : p.kv_pos_base + key) <= qpos;
    if (ok && kvs) ok = (kvs[key] == qseg) && (qseg != -1);
    if (!ok) S[i] = neg_inf();
  }
}

template <bool CAP>
__device__ __forceinline__ void step_body(const char* Vt, const char* Kt, const Wave& wv, const bf16x8 (&qf)[2][8],
                                          f32x16 (&O)[2][4], f32x16 (&Sc)[2], f32x16 (&Sn)[2], bf16x8 (&P)[2][2],
                                          float (&m_ref)[2], float (&l_acc)[2], float (&alpha)[2], float scale_log2) {
  // operands of MFMA group gi: 0-3 PV (ks = gi >> 1, db = 2*(gi&1) + u), 4-7 QK (ds = 2*(gi-4) + u)
  bf16x8 fr[2][2];
  auto frag = [&](int gi, bf16x8 (&dst)[2]) {
    if (gi < 4) {
#pragma unroll
      for (int u = 0; u < 2; ++u) dst[u] = read_v(Vt, wv, gi >> 1, 2 * (gi & 1) + u);
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u) dst[u] = *reinterpret_cast<const bf16x8*>(Kt + wv.k_off[2 * (gi - 4) + u]);
    }
  };
  auto mfma = [&](int gi, const bf16x8 (&src)[2]) {
    if (gi < 4) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
          const int db = 2 * (gi & 1) + u;
          O[qh][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(src[u], P[qh][gi >> 1], O[qh][db], 0, 0, 0);
        }
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
          const int ds = 2 * (gi - 4) + u;
          Sn[qh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(src[u], qf[qh][ds], ds == 0 ? f32x16{} : Sn[qh], 0, 0, 0);
        }
    }
  };
  float mx[2], msub[2], ls[2];
  auto slice = [&](int sl) {
    if (sl == 0) {                                   // row max (tree)
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        float t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) t[u] = fmaxf(fmaxf(Sc[qh][4 * u], Sc[qh][4 * u + 1]), fmaxf(Sc[qh][4 * u + 2], Sc[qh][4 * u + 3]));
        mx[qh] = fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3]));
      }
    } else if (sl == 1) {                            // reference max, rescale factor
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        const float m = pair_max(mx[qh]);
        const float umax = CAP ? m : m * scale_log2;
        const bool need = umax > m_ref[qh] + kRescaleThreshold;
        const float m_new = need ? umax : m_ref[qh];
        alpha[qh] = need ? fast_exp2(m_ref[qh] - m_new) : 1.0f;
        m_ref[qh] = m_new;
        msub[qh] = (m_new == neg_inf()) ? 0.0f : m_new;
      }
    } else if (sl < 6) {                             // exponentials, 8 per slice
      const int e = sl - 2;
      const int qh = e >> 1, i0 = (e & 1) * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float s = Sc[qh][i0 + i];
        Sc[qh][i0 + i] = CAP ? fast_exp2(s - msub[qh]) : fast_exp2(__builtin_fmaf(s, scale_log2, -msub[qh]));
      }
    } else if (sl == 6) {                            // row sums (tree), running sums
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        float t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) t[u] = (Sc[qh][4 * u] + Sc[qh][4 * u + 1]) + (Sc[qh][4 * u + 2] + Sc[qh][4 * u + 3]);
        ls[qh] = (t[0] + t[1]) + (t[2] + t[3]);
        l_acc[qh] = l_acc[qh] * alpha[qh] + ls[qh];
      }
    } else {                                         // weights to bf16: B operand of the next PV
#pragma unroll
      for (int qh = 0; qh < 2; ++qh)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            f32x2 two = {Sc[qh][ks * 8 + 2 * jj], Sc[qh][ks * 8 + 2 * jj + 1]};
            bf16x2 pk = __builtin_convertvector(two, bf16x2);
            P[qh][ks][2 * jj] = pk[0];
            P[qh][ks][2 * jj + 1] = pk[1];
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
__global__ __launch_bounds__(kWThreads, 1) void attn_fwd_bf16_w64(AttnParams p) {
  constexpr int NDS = kD / 16;
  __shared__ __attribute__((aligned(16))) __bf16 kbuf[2 * kSubElems];
  __shared__ __attribute__((aligned(16))) __bf16 vbuf[2 * kSubElems];
  __shared__ uint32_t ulist[kMaxMaskCols];
  __shared__ int wsum[kWWaves];

  const int nQt = (p.nQb + 1) >> 1;             // 256-row q tiles
  int b, h, qt;
  if (!decode_work_w(p, nQt, b, h, qt)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int ln = lane & 31, lg = lane >> 5;
  const int G = p.H / p.Hkv;
  const int g = h / G;
  const int half = w >> 1;
  const int row0 = qt * 2 * kBlockQ + w * 64;

  // ---- union of the two 128-row tile rows' non-EMPTY 64-key tiles
  const int64_t rowA = (int64_t)b * p.nQb + 2 * qt;
  const bool hasB = 2 * qt + 1 < p.nQb;
  int n = 0;
  for (int base = 0; base < p.nKb; base += kWThreads) {
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
    for (int i = 0; i < kWWaves; ++i) {
      off += (i < w) ? wsum[i] : 0;
      total += wsum[i];
    }
    if (f) ulist[off + before] = (uint32_t)kb | (ca << 16) | (cb << 24);
    n += total;
    __syncthreads();
  }
  if (n == 0 && p.mode == 1 && p.sinks == nullptr) return;
  const int nt = 2 * n;                          // 32-key steps

  // ---- query fragments and row state of the wave's two 32-row blocks
  bf16x8 qf[2][NDS];
  float m_ref[2], l_acc[2], alpha[2];
  int qpos[2], qseg[2];
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const int q_row = row0 + 32 * qh + ln;
    const bool q_ok = q_row < p.Sq;
    const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.q_stride_b +
                         ((int64_t)(q_ok ? q_row : 0) * p.H + h) * kD;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      bf16x8 t = *reinterpret_cast<const bf16x8*>(qrow + ds * 16 + lg * 8);
      qf[qh][ds] = q_ok ? t : bf16x8{};
    }
    const int qc = q_ok ? q_row : p.Sq - 1;
    qpos[qh] = p.q_pos ? p.q_pos[(int64_t)b * p.qm_stride_b + qc] : p.q_pos_base + q_row;
    qseg[qh] = p.q_seg ? p.q_seg[(int64_t)b * p.qm_stride_b + qc] : 0;
    m_ref[qh] = p.sinks ? p.sinks[h] * kLog2e : neg_inf();
    l_acc[qh] = (p.sinks && lg == 0) ? 1.0f : 0.0f;
    alpha[qh] = 1.0f;
  }
  f32x16 O[2][4];
#pragma unroll
  for (int qh = 0; qh < 2; ++qh)
#pragma unroll
    for (int db = 0; db < 4; ++db) O[qh][db] = f32x16{};

  Wave wv;
  wave_offsets(wv, lane);
  const int64_t krs = (int64_t)p.Hkv * kD;
  const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + (int64_t)b * p.kv_stride_b + g * kD;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.kv_stride_b + g * kD;
  // key offset of 32-key step t (the mask tile of step t is ulist[t >> 1])
  auto step_k0 = [&](int t) { return (int)(ulist[t >> 1] & 0xffffu) * kBlockKV + (t & 1) * kSub; };
  auto step_cls = [&](int t) { return (int)((ulist[t >> 1] >> (16 + 8 * half)) & 0xffu); };

  // ---- prologue: K_0, K_1 in LDS; S_0 = Q K_0^T. Step 0's PV reads V buffer 1
  // with zero weights; it is cleared so that no stale NaN can enter O.
  for (int i = tid; i < kSubElems / 8; i += kWThreads)
    reinterpret_cast<uint4*>(vbuf + kSubElems)[i] = make_uint4(0, 0, 0, 0);
  f32x16 Sa[2], Sb[2];
  bf16x8 P[2][2];
#pragma unroll
  for (int qh = 0; qh < 2; ++qh)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) P[qh][ks] = bf16x8{};
  if (nt > 0) load_step(kbase, krs, step_k0(0), p.Skv, kbuf, w, lane, false);
  if (nt > 1) load_step(kbase, krs, step_k0(1), p.Skv, kbuf + kSubElems, w, lane, false);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (nt > 0) {
    const char* Kt = reinterpret_cast<const char*>(kbuf);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(Kt + wv.k_off[ds]);
#pragma unroll
      for (int qh = 0; qh < 2; ++qh)
        Sa[qh] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qh][ds], ds == 0 ? f32x16{} : Sa[qh], 0, 0, 0);
    }
  }
  __syncthreads();

  // one step t: S_cur = S_t, P = P_{t-1}; leaves S_next = S_{t+1}, P = P_t
  auto step = [&](int t, f32x16 (&S_cur)[2], f32x16 (&S_next)[2]) {
    if (t + 2 < nt) load_step(kbase, krs, step_k0(t + 2), p.Skv, kbuf + (t & 1) * kSubElems, w, lane, false);
    load_step(vbase, krs, step_k0(t), p.Skv, vbuf + (t & 1) * kSubElems, w, lane, true);
    const int cls = step_cls(t);
    const int k0 = step_k0(t);
    if constexpr (CAP) {
#pragma unroll
      for (int qh = 0; qh < 2; ++qh)
#pragma unroll
        for (int i = 0; i < 16; ++i) S_cur[qh][i] = capped_log2(S_cur[qh][i], p.cap_k2, p.cap_log2);
    }
    if (cls == 0) {
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) S_cur[qh] = f32x16{} + neg_inf();
    } else if (cls != 2 || k0 + kSub > p.Skv) {
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) mask_step(S_cur[qh], p, b, k0, lg, qpos[qh], qseg[qh]);
    }
    const char* Vt = reinterpret_cast<const char*>(vbuf + ((t + 1) & 1) * kSubElems);   // V_{t-1}
    const char* Kt = reinterpret_cast<const char*>(kbuf + ((t + 1) & 1) * kSubElems);   // K_{t+1}
    // always both streams: at t = 0 the weights P are zero, and after the last
    // step the S_next it computes from a stale K buffer is never used
    step_body<CAP>(Vt, Kt, wv, qf, O, S_cur, S_next, P, m_ref, l_acc, alpha, p.scale_log2);
    // rare: some row's running max moved; O (now holding P_{t-1} V_{t-1}) follows it
    if (__builtin_amdgcn_ballot_w64(alpha[0] != 1.0f || alpha[1] != 1.0f) != 0) {
#pragma unroll
      for (int qh = 0; qh < 2; ++qh)
#pragma unroll
        for (int db = 0; db < 4; ++db) O[qh][db] *= alpha[qh];
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  for (int t = 0; t < nt; t += 2) {      // nt is even: two 32-key steps per 64-key tile
    step(t, Sa, Sb);
    step(t + 1, Sb, Sa);
  }

  // last PV: O += P_{nt-1} V_{nt-1}
  if (nt > 0) {
    const char* Vt = reinterpret_cast<const char*>(vbuf + ((nt - 1) & 1) * kSubElems);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 a = read_v(Vt, wv, ks, db);
#pragma unroll
        for (int qh = 0; qh < 2; ++qh)
          O[qh][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[qh][ks], O[qh][db], 0, 0, 0);
      }
  }
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const int q_row = row0 + 32 * qh + ln;
    epilogue<4>(O[qh], m_ref[qh], l_acc[qh], p, b, h, q_row < p.Sq ? q_row : p.Sq, lg);
  }
}

template <typename K>
hipError_t launch_w(K kernel, const AttnParams& p, hipStream_t s) {
  const int nQt = (p.nQb + 1) / 2;
  const int64_t T = (int64_t)p.B * p.H * nQt;
  const int64_t grid = 8 * ((T + 7) / 8);
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kWThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_w64(const AttnParams& p, hipStream_t s) {
  if (p.softcap_on) return launch_w(attn_fwd_bf16_w64<true>, p, s);
  return launch_w(attn_fwd_bf16_w64<false>, p, s);
}

}  // namespace ram
