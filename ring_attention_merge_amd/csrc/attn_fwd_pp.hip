// Block-sparse attention forward for one KV chunk: 8-wave ping-pong variant.
//
// Computes exactly what attn_fwd.hip computes (the per-ring-step kernel call of
// the ejkernel ring-splash source page, _ring_attention_forward, with the
// _update_out_and_lse merge as epilogue), with a schedule built for CDNA4's
// split between the matrix core and the vector ALU:
//
//  * One workgroup = 8 waves = two 128-row q tiles of one head (256 rows).
//    Waves 0-3 form group 0 and waves 4-7 group 1; wave w and wave w+4 share
//    a SIMD, so every SIMD hosts one wave of each group.
//  * Each group alternates an M phase (O += P_{j-1} V_{j-1}, then
//    S_j = Q K_j^T: 32 MFMAs for a 64-key tile) and an S phase (online
//    softmax of S_j into P_j: VALU and transcendental work). Group 1 runs one
//    phase behind group 0 and a workgroup barrier closes every phase, so on
//    each SIMD one wave keeps the matrix core busy while the other runs its
//    softmax. MFMA phases run at raised wave priority.
//  * K and V are double-buffered separately: the loads of K_{j+1} and V_j are
//    issued at the start of slot 2j and stored to LDS at the end of slot 2j+1,
//    two phases after issue; each buffer is rewritten only after both groups
//    have finished reading it.
//  * The workgroup visits the union of its two q tiles' non-EMPTY kv tiles
//    (block mask at the 128 x 64 kernel tile); a group skips every tile that
//    is EMPTY for its own q tile and masks only its PARTIAL tiles.
//  * Operand layouts (transposed S, transposing LDS reads for V, conflict-free
//    LDS pitches) are those of attn_fwd.hip.
#include "attn_common.h"

namespace ram {
namespace {

using namespace attn;

constexpr int kPPWaves = 8;
constexpr int kPPThreads = 64 * kPPWaves;

// Work decode over (batch*Hkv + kv head, q-tile pair descending, head in group);
// XCD x = id % 8 takes the contiguous item range [x*per, (x+1)*per).
__device__ __forceinline__ bool decode_work_pairs(const AttnParams& p, int nQp, int& b, int& h, int& qp) {
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

// The M phase as 8 steps of 4 MFMAs: steps 0-3 are PV (one 16-key slice of
// V_{j-1} against P_{j-1}, A operands from transposing LDS reads), steps 4-7
// are QK (two 16-dim slices of K_j against Q). Operands of step t+1 are read
// from LDS before the MFMAs of step t are issued, so LDS latency hides under
// the matrix core. [T0, T1) selects the steps to run.
template <int D, int T0, int T1>
__device__ __forceinline__ void m_phase(const __bf16* Vs, const __bf16* Ks, int vtr_off, int ln, int lg,
                                        const bf16x8 (&P)[4], const bf16x8 (&qf)[D / 16],
                                        f32x16 (&O)[D / 32], f32x16 (&S)[2]) {
  constexpr int NDB = D / 32;
  constexpr int KP = D + 8;
  constexpr int VP = D + 32;
  static_assert(NDB == 4 || NDB == 2, "head dim");
  bf16x8 a[2][4];
  auto load = [&](int t, bf16x8 (&dst)[4]) {
    if (t < 4) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const __bf16* vp = Vs + t * 16 * VP + db * 32 + vtr_off;
        const s16x4 lo = lds_read_tr16(vp);
        const s16x4 hi = lds_read_tr16(vp + 8 * VP);
        dst[db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    } else {
      constexpr int PER = NDB;                 // MFMAs per QK step: 4 (D=128) or 2 (D=64)
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int ds = (t - 4) * (PER / 2) + (i >> 1);
        const int kb2 = i & 1;
        dst[i] = *reinterpret_cast<const bf16x8*>(Ks + (kb2 * 32 + ln) * KP + ds * 16 + lg * 8);
      }
    }
  };
  auto mma = [&](int t, const bf16x8 (&src)[4]) {
    if (t < 4) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) O[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(src[db], P[t], O[db], 0, 0, 0);
    } else {
      constexpr int PER = NDB;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int ds = (t - 4) * (PER / 2) + (i >> 1);
        const int kb2 = i & 1;
        S[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(src[i], qf[ds], S[kb2], 0, 0, 0);
      }
    }
  };
  load(T0, a[0]);
#pragma unroll
  for (int t = T0; t < T1; ++t) {
    if (t + 1 < T1) load(t + 1, a[(t + 1 - T0) & 1]);
    __builtin_amdgcn_sched_barrier(0);
    mma(t, a[(t - T0) & 1]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D, bool CAP>
__global__ __launch_bounds__(kPPThreads, 1) void attn_fwd_bf16_pp(AttnParams p) {
  constexpr int BK = kBlockKV;
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  constexpr int KP = D + 8;          // K row pitch (elements): 272 B for D = 128
  constexpr int VP = D + 32;         // V row pitch (elements): 320 B for D = 128
  constexpr int K_ELEMS = BK * KP;
  constexpr int V_ELEMS = BK * VP;
  constexpr int CH = D / 8;                  // 16-byte chunks per row
  constexpr int RPP = kPPThreads / CH;       // rows per load pass
  constexpr int NPK = BK / RPP;              // load passes per tensor
  static_assert(NPK >= 1 && BK % RPP == 0, "tile split");
  __shared__ __attribute__((aligned(16))) __bf16 kbuf[2 * K_ELEMS];
  __shared__ __attribute__((aligned(16))) __bf16 vbuf[2 * V_ELEMS];
  __shared__ uint32_t ulist[kMaxMaskCols];   // kb | class(q tile 0) << 16 | class(q tile 1) << 24
  __shared__ int wsum[kPPWaves];

  const int nQp = (p.nQb + 1) >> 1;
  int b, h, qp;
  if (!decode_work_pairs(p, nQp, b, h, qp)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int grp = w >> 2, wi = w & 3;
  const int ln = lane & 31, lg = lane >> 5;
  const int G = p.H / p.Hkv;
  const int g = h / G;
  const int qb = 2 * qp + grp;                 // this group's 128-row q tile
  const int q_row = qb * kBlockQ + wi * 32 + ln;
  const bool q_ok = qb < p.nQb && q_row < p.Sq;

  // ---- union of the two q tiles' non-EMPTY kv tiles, in ascending order
  const int64_t rowA = (int64_t)b * p.nQb + 2 * qp;
  const bool hasB = 2 * qp + 1 < p.nQb;
  int n = 0;
  for (int base = 0; base < p.nKb; base += kPPThreads) {
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
    for (int i = 0; i < kPPWaves; ++i) {
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

  // ---- tile loads (all 512 threads; global -> registers -> LDS)
  const int64_t krs = (int64_t)p.Hkv * D;
  const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + (int64_t)b * p.kv_stride_b + g * D;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.kv_stride_b + g * D;
  const int kc = tid % CH, kr0 = tid / CH;
  uint4 kreg[NPK], vreg[NPK];
  auto gload = [&](uint4 (&reg)[NPK], const __bf16* base, int kb) {
    const int k0 = kb * BK;
#pragma unroll
    for (int i = 0; i < NPK; ++i) {
      const int row = k0 + kr0 + i * RPP;
      reg[i] = row < p.Skv ? *reinterpret_cast<const uint4*>(base + row * krs + kc * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](const uint4 (&reg)[NPK], __bf16* dst, int pitch) {
#pragma unroll
    for (int i = 0; i < NPK; ++i) *reinterpret_cast<uint4*>(dst + (kr0 + i * RPP) * pitch + kc * 8) = reg[i];
  };
  const int vtr_off = (4 * lg + ((lane & 15) >> 2)) * VP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  auto tile_kb = [&](int j) { return (int)(ulist[j] & 0xffffu); };
  auto tile_cls = [&](int j) { return (int)((ulist[j] >> (16 + 8 * grp)) & 0xffu); };

  if (n > 0) {
    gload(kreg, kbase, tile_kb(0));
    lstore(kreg, kbuf, KP);
  }
  __syncthreads();

  f32x16 S[2];
  S[0] = f32x16{};
  S[1] = f32x16{};
  bf16x8 P[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) P[ks] = bf16x8{};

  const int n_slots = 2 * n + 2;
  for (int s = 0; s < n_slots; ++s) {
    const int jl = s >> 1;
    if (!(s & 1)) {   // slot 2j starts: fetch K_{j+1} and V_j
      if (jl + 1 < n) gload(kreg, kbase, tile_kb(jl + 1));
      if (jl < n) gload(vreg, vbase, tile_kb(jl));
    }
    const int ph = s - grp;
    if (ph >= 0 && ph <= 2 * n) {
      const int jj = ph >> 1;
      if (!(ph & 1)) {
        // ---- M phase: O += P_{jj-1} V_{jj-1}; S = Q K_{jj}^T
        const bool do_pv = jj >= 1 && tile_cls(jj - 1) != 0;
        const bool do_qk = jj < n && tile_cls(jj) != 0;
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(1);
        if (do_qk) {
          S[0] = f32x16{};
          S[1] = f32x16{};
        }
        const __bf16* Vs = vbuf + ((jj + 1) & 1) * V_ELEMS;   // V_{jj-1}
        const __bf16* Ks = kbuf + (jj & 1) * K_ELEMS;         // K_{jj}
        if (do_pv && do_qk) m_phase<D, 0, 8>(Vs, Ks, vtr_off, ln, lg, P, qf, O, S);
        else if (do_pv) m_phase<D, 0, 4>(Vs, Ks, vtr_off, ln, lg, P, qf, O, S);
        else if (do_qk) m_phase<D, 4, 8>(Vs, Ks, vtr_off, ln, lg, P, qf, O, S);
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // ---- S phase: online softmax of S_{jj} into P_{jj}
        const int cls = tile_cls(jj);
        if (cls != 0) {
          const int kb = tile_kb(jj);
          if constexpr (CAP) {
#pragma unroll
            for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
              for (int i = 0; i < 16; ++i) S[kb2][i] = capped_log2(S[kb2][i], p.cap_k2, p.cap_log2);
          }
          if (cls != 2 || (kb + 1) * BK > p.Skv) apply_mask(S, p, b, kb * BK, lg, qpos, qseg);
          softmax_step<NDB, CAP>(S, O, m_ref, l_acc, p);
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
        }
      }
    }
    if (s & 1) {      // slot 2j+1 ends: K_{j+1} and V_j go to LDS
      if (jl + 1 < n) lstore(kreg, kbuf + ((jl + 1) & 1) * K_ELEMS, KP);
      if (jl < n) lstore(vreg, vbuf + (jl & 1) * V_ELEMS, VP);
    }
    __syncthreads();
  }
  epilogue<NDB>(O, m_ref, l_acc, p, b, h, q_ok ? q_row : p.Sq, lg);
}

template <typename K>
hipError_t launch_pp(K kernel, const AttnParams& p, hipStream_t s) {
  const int nQp = (p.nQb + 1) / 2;
  const int64_t T = (int64_t)p.B * p.H * nQp;
  const int64_t grid = 8 * ((T + 7) / 8);
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kPPThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_pp(const AttnParams& p, hipStream_t s) {
  const bool cap = p.softcap_on != 0;
  if (p.D == 128) return cap ? launch_pp(attn_fwd_bf16_pp<128, true>, p, s) : launch_pp(attn_fwd_bf16_pp<128, false>, p, s);
  return cap ? launch_pp(attn_fwd_bf16_pp<64, true>, p, s) : launch_pp(attn_fwd_bf16_pp<64, false>, p, s);
}

}  // namespace ram
