// Block-sparse attention forward for one KV chunk: wide-wave variant.
//
// Computes exactly what attn_fwd.hip computes (the per-ring-step kernel call of
// the ejkernel ring-splash source page, _ring_attention_forward, with the
// _update_out_and_lse merge as epilogue). The layout targets the LDS operand
// traffic of the 4-wave kernel: with 32 query rows per wave every
// v_mfma_f32_32x32x16_bf16 needs 1 KB of K or V from LDS, so LDS bandwidth and
// latency, not the matrix cores, set the pace. Here:
//
//  * One workgroup = 4 waves, one per SIMD, 256 query rows (two 128-row mask
//    tile rows of one head); each wave owns 64 rows as two 32-row blocks, so
//    every K or V operand read from LDS feeds two MFMAs.
//  * Registers: O^T (64 rows x 128 dims, fp32) and the Q operands live in the
//    accumulation registers (AGPRs), scores and weights in VGPRs. The MFMAs
//    are written with explicit operand classes so the compiler never copies
//    between the two files; the MFMA-to-VALU result latency, which the
//    hardware does not interlock, is waited out explicitly (settle_*).
//  * K and V go from HBM straight to LDS (buffer_load_dwordx4 ... lds, rows
//    past the chunk read as zero) into a 3-stage ring of dense 256-byte rows
//    with XOR-swizzled 16-byte chunks:
//    chunk ^ (row & 15) for K, chunk ^ 4*(row & 3) for V (conflict-free
//    operand reads, V through ds_read_b64_tr_b16). Tile j+2 loads while tile
//    j is computed.
//  * The workgroup walks the union of its two tile rows' non-EMPTY kv tiles;
//    a wave skips tiles EMPTY for its own row and masks only PARTIAL ones.
#include "attn_common.h"

namespace ram {
namespace {

using namespace attn;

constexpr int kWWaves = 4;
constexpr int kWThreads = 64 * kWWaves;
constexpr int kWD = 128;
constexpr int kWStages = 3;
constexpr int kWTile = kBlockKV * kWD;   // one K or V tile (16 KB)

__device__ __forceinline__ bool decode_work_w(const AttnParams& p, int nQp, int& b, int& h, int& qp) {
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

// Lane offsets (bytes, inside a tile of global rows) of the four 1 KB slabs
// a wave moves per tile: wave w fills LDS rows [16w, 16w+16); lane l of slab i
// writes physical chunk l & 15 of row 16w + 4i + (l >> 4), which holds logical
// chunk (l & 15) ^ (row & 15) for K and (l & 15) ^ 4*(row & 3) for V.
__device__ __forceinline__ void dma_offsets(uint32_t (&off)[4], uint32_t row_bytes, int w, int lane, bool is_v) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * w + 4 * i + (lane >> 4);
    const int phys = lane & 15;
    const int logical = is_v ? (phys ^ (4 * (r & 3))) : (phys ^ (r & 15));
    off[i] = (uint32_t)r * row_bytes + logical * 16;
  }
}

// Tile kb of K or V into LDS through a buffer resource covering the tile's
// rows that exist (rows past Skv read as zero).
__device__ __forceinline__ void dma_tile_w(const __bf16* gbase, int64_t krs, int kb, int skv, __bf16* tile,
                                           int w, const uint32_t (&off)[4]) {
  const int k0 = kb * kBlockKV;
  const auto rs = tile_rsrc(gbase + (int64_t)k0 * krs, (uint32_t)min(skv - k0, kBlockKV) * (uint32_t)krs * 2);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(tile + (16 * w + 4 * i) * kWD),
                                             16, off[i], 0, 0, 0);
}

// Slab i (rows 16w + 4i .. +3) of tile kb, as one instruction.
__device__ __forceinline__ void dma_slab_w(const __bf16* gbase, int64_t krs, int kb, int skv, __bf16* tile,
                                           int w, uint32_t off, int i) {
  const int k0 = kb * kBlockKV;
  const auto rs = tile_rsrc(gbase + (int64_t)k0 * krs, (uint32_t)min(skv - k0, kBlockKV) * (uint32_t)krs * 2);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(tile + (16 * w + 4 * i) * kWD),
                                           16, off, 0, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_w() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// ---- MFMAs with explicit register files
// S (VGPR) = K (VGPR) x Q (AGPR), first k-step / accumulate
__device__ __forceinline__ void mfma_qk0(f32x16& d, const bf16x8& a, const bf16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(q));
}
__device__ __forceinline__ void mfma_qk(f32x16& d, const bf16x8& a, const bf16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(q));
}
// O (AGPR) += V^T (VGPR) x P (VGPR)
__device__ __forceinline__ void mfma_pv(f32x16& o, const bf16x8& a, const bf16x8& pw) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(pw));
}
// Wait states between an MFMA writing registers and the first VALU or
// accumulator-move access to them (covers the longest MFMA pipeline); the
// operands tie the wait to the values so no access is scheduled above it.
__device__ __forceinline__ void settle_s(f32x16 (&S)[2][2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(S[0][0]), "+v"(S[0][1]), "+v"(S[1][0]), "+v"(S[1][1]));
}
__device__ __forceinline__ void settle_o(f32x16 (&O)[4]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+a"(O[0]), "+a"(O[1]), "+a"(O[2]), "+a"(O[3]));
}
__device__ __forceinline__ void settle_s2(f32x16 (&S)[2]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+v"(S[0]), "+v"(S[1]));
}
__device__ __forceinline__ void settle_p2(bf16x8 (&P)[2][2]) {
  asm volatile("s_nop 3" : "+v"(P[0][0]), "+v"(P[0][1]), "+v"(P[1][0]), "+v"(P[1][1]));
}
// VALU writes (weights, rescaled accumulators) ahead of MFMA reads
__device__ __forceinline__ void settle_p(bf16x8 (&P)[2][4]) {
  asm volatile("s_nop 3" : "+v"(P[0][0]), "+v"(P[0][1]), "+v"(P[0][2]), "+v"(P[0][3]), "+v"(P[1][0]),
               "+v"(P[1][1]), "+v"(P[1][2]), "+v"(P[1][3]));
}

template <bool CAP>
__global__ __launch_bounds__(kWThreads, 1) void attn_fwd_bf16_w64(AttnParams p) {
  constexpr int D = kWD;
  constexpr int NDS = D / 16;
  constexpr int NDB = D / 32;
  __shared__ __attribute__((aligned(16))) __bf16 kst[kWStages * kWTile];
  __shared__ __attribute__((aligned(16))) __bf16 vst[kWStages * kWTile];
  __shared__ uint32_t ulist[kMaxMaskCols];
  __shared__ int wsum[kWWaves];

  const int nQp = (p.nQb + 1) >> 1;
  int b, h, qp;
  if (!decode_work_w(p, nQp, b, h, qp)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int grp = w >> 1;                 // mask tile row of this wave
  const int ln = lane & 31, lg = lane >> 5;
  const int G = p.H / p.Hkv;
  const int g = h / G;
  const int qb = 2 * qp + grp;

  // ---- union of the two q tiles' non-EMPTY kv tiles
  const int64_t rowA = (int64_t)b * p.nQb + 2 * qp;
  const bool hasB = 2 * qp + 1 < p.nQb;
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

  // ---- per-lane query state: rows q_row[r] for the two 32-row blocks
  int q_row[2], qpos[2];
  bool q_ok[2];
  bf16x8 qf[2][NDS];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    q_row[r] = qb * kBlockQ + (w & 1) * 64 + r * 32 + ln;
    q_ok[r] = qb < p.nQb && q_row[r] < p.Sq;
    const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.q_stride_b +
                         ((int64_t)(q_ok[r] ? q_row[r] : 0) * p.H + h) * D;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      bf16x8 t = *reinterpret_cast<const bf16x8*>(qrow + ds * 16 + lg * 8);
      qf[r][ds] = q_ok[r] ? t : bf16x8{};
    }
    const int qrow_c = q_ok[r] ? q_row[r] : p.Sq - 1;
    qpos[r] = p.q_pos ? p.q_pos[(int64_t)b * p.qm_stride_b + qrow_c] : p.q_pos_base + q_row[r];
  }

  // Q operands move to the accumulation registers once, for the whole loop
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) asm volatile("" : "+a"(qf[r][ds]));

  float m_ref[2], l_acc[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    m_ref[r] = neg_inf();
    l_acc[r] = 0.0f;
    if (p.sinks) {
      m_ref[r] = p.sinks[h] * kLog2e;
      l_acc[r] = (lg == 0) ? 1.0f : 0.0f;
    }
  }
  f32x16 O[2][NDB];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int db = 0; db < NDB; ++db) O[r][db] = f32x16{};

  const int64_t krs = (int64_t)p.Hkv * D;
  const __bf16* kbase = reinterpret_cast<const __bf16*>(p.k) + (int64_t)b * p.kv_stride_b + g * D;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(p.v) + (int64_t)b * p.kv_stride_b + g * D;
  // list entries are the same for every lane: keep them in scalar registers
  auto tile_kb = [&](int j) { return __builtin_amdgcn_readfirstlane((int)(ulist[j] & 0xffffu)); };
  auto tile_cls = [&](int j) { return __builtin_amdgcn_readfirstlane((int)((ulist[j] >> (16 + 8 * grp)) & 0xffu)); };

  // LDS byte offsets of this lane's operands inside a tile half (32 keys).
  int k_off[NDS];                     // K: row ln, logical chunk 2*ds + lg
#pragma unroll
  for (int ds = 0; ds < NDS; ++ds) k_off[ds] = ln * 256 + (((2 * ds + lg) ^ (ln & 15)) * 16);
  // V (transposing reads): row ks*16 + 8*part + 4*lg + r4, column db*32 + 16*hs + 4*(lane&3)
  const int r4 = (lane & 15) >> 2, hs = (lane >> 4) & 1;
  const int v_row = 4 * lg + r4;
  int v_col[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    v_col[db] = (((db * 4 + 2 * hs + ((lane & 3) >> 1)) ^ (4 * r4)) * 16) + (lane & 1) * 8;

  uint32_t koff[4], voff[4];
  dma_offsets(koff, (uint32_t)krs * 2, w, lane, false);
  dma_offsets(voff, (uint32_t)krs * 2, w, lane, true);
  if (p.Skv % kBlockKV) {
    // A ragged last tile leaves rows of its stage unwritten; start from zeros
    // so that those rows (masked, weight 0) hold finite values.
    for (int i = tid; i < kWStages * kWTile / 8; i += kWThreads) {
      reinterpret_cast<uint4*>(kst)[i] = make_uint4(0, 0, 0, 0);
      reinterpret_cast<uint4*>(vst)[i] = make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- schedule
  // Keys go in 32-key steps s = 0 .. 2n-1 (step s = half s & 1 of list tile
  // s >> 1). Block s interleaves, inside this wave, the softmax of step s
  // (VALU) with the MFMAs of PV(s-1) and QK(s+1). K is read one step ahead
  // and V one step behind, so they have separate 3-stage rings (list tile j
  // in stage j % 3): during tile j's two blocks the workgroup reads K(j),
  // K(j+1), V(j-1), V(j) and loads K(j+2), V(j+1), waited for before the
  // barrier that closes tile j.
  auto k_at = [&](int s2) {   // K rows of step s2
    return reinterpret_cast<const char*>(kst + ((s2 >> 1) % kWStages) * kWTile) + (s2 & 1) * 32 * 256;
  };
  auto v_at = [&](int s2) {
    return reinterpret_cast<const char*>(vst + ((s2 >> 1) % kWStages) * kWTile) + (s2 & 1) * 32 * 256;
  };
  auto kread = [&](const char* Kt, int ds) { return *reinterpret_cast<const bf16x8*>(Kt + k_off[ds]); };
  auto vread = [&](const char* Vt, int f) {   // f = 4*ks + db
    const char* vp = Vt + ((f >> 2) * 16 + v_row) * 256 + v_col[f & 3];
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(vp + 8 * 256));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  if (n > 0) {
    dma_tile_w(kbase, krs, tile_kb(0), p.Skv, kst, w, koff);
    dma_tile_w(vbase, krs, tile_kb(0), p.Skv, vst, w, voff);
  }
  if (n > 1) dma_tile_w(kbase, krs, tile_kb(1), p.Skv, kst + kWTile, w, koff);
  wait_vmcnt_w<0>();
  __syncthreads();

  // Scores and weights ping-pong between two register sets from step to step:
  // step s works on set s & 1 (softmax) and fills set (s + 1) & 1 (QK).
  f32x16 SA[2], SB[2];        // [row block]
  bf16x8 PA[2][2], PB[2][2];  // [row block][16-key slice]
  if (n > 0) {
    const char* Kt = k_at(0);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const bf16x8 a = kread(Kt, ds);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        if (ds == 0) mfma_qk0(SA[r], a, qf[r][0]);
        else mfma_qk(SA[r], a, qf[r][ds]);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) PB[r][0] = PB[r][1] = bf16x8{};

  const int nsteps = 2 * n;
  // One 32-key step: softmax of Sc (step s2) interleaved with PV(s2-1) (weights
  // Pp) and QK(s2+1) (into Sn); the new weights go to Pc. The MFMA / VALU
  // sequence is one basic block, cut into eight MFMA groups and eight VALU
  // chunks by scheduling barriers, so that the matrix core runs while the
  // softmax issues. The first step's PV multiplies zero weights with V of
  // tile 0, the last step's QK fills scores nobody reads: both stay in bounds
  // and keep the block free of branches.
  auto step = [&](int s2, int kb, int cls, f32x16 (&Sc)[2], f32x16 (&Sn)[2], bf16x8 (&Pp)[2][2],
                  bf16x8 (&Pc)[2][2], auto&& dma_piece) {
    const char* Vt = v_at(s2 > 0 ? s2 - 1 : 0);
    const char* Kt = k_at(s2 + 1 < nsteps ? s2 + 1 : s2);

    // ---- scores of step s2: wait out the MFMA pipeline, then cap / mask
    settle_s2(Sc);
    if constexpr (CAP) {
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) Sc[r][i] = capped_log2(Sc[r][i], p.cap_k2, p.cap_log2);
    }
    if (cls == 0) {   // EMPTY for this wave's tile row: weight 0 everywhere
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) Sc[r][i] = neg_inf();
    } else if (cls != 2 || (kb + 1) * kBlockKV > p.Skv) {
      // positions kv_pos_base + key (this kernel runs without position or
      // segment arrays): exactly the keys below `lim` are kept
      const int k0 = kb * kBlockKV + (s2 & 1) * 32 + 4 * lg;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int64_t reach = (int64_t)qpos[r] - p.kv_pos_base + 1;
        int thr = (p.causal ? (int)max<int64_t>(-1, min<int64_t>(p.Skv, reach)) : p.Skv) - k0;
        asm volatile("" : "+v"(thr));
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i >> 2) + (i & 3) >= thr) Sc[r][i] = neg_inf();
      }
    }
    asm volatile("" : "+v"(Sc[0]), "+v"(Sc[1]));

    // ---- operand groups: 0-3 PV(s2-1) (V operands 2g, 2g+1), 4-7 QK(s2+1)
    // (k-steps 2(g-4), 2(g-4)+1); each operand feeds both row blocks.
    // Operands are read two groups ahead of their MFMAs.
    bf16x8 fr[8][2];
    auto gread = [&](int g) {
      if (g < 4) {
        fr[g][0] = vread(Vt, 2 * g);
        fr[g][1] = vread(Vt, 2 * g + 1);
      } else {
        fr[g][0] = kread(Kt, 2 * (g - 4));
        fr[g][1] = kread(Kt, 2 * (g - 4) + 1);
      }
    };
    auto gmfma = [&](int g) {
      if (g < 4) {
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 2; ++r) mfma_pv(O[r][(2 * g + u) & 3], fr[g][u], Pp[r][(2 * g + u) >> 2]);
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int ds = 2 * (g - 4) + u;
#pragma unroll
          for (int r = 0; r < 2; ++r) {
            if (ds == 0) mfma_qk0(Sn[r], fr[g][u], qf[r][0]);
            else mfma_qk(Sn[r], fr[g][u], qf[r][ds]);
          }
        }
      }
    };

    // ---- softmax of step s2 in eight VALU chunks (no branches: the rescale
    // decision is a wave-uniform select; O itself is rescaled after the block)
    float mx[2], alpha[2], msub[2];
    bool resc = false;
    auto vchunk = [&](int c) {
      if (c == 0) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          float t[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            t[u] = fmaxf(fmaxf(Sc[r][4 * u], Sc[r][4 * u + 1]), fmaxf(Sc[r][4 * u + 2], Sc[r][4 * u + 3]));
          mx[r] = pair_max(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])));
        }
        asm volatile("" : "+v"(mx[0]), "+v"(mx[1]));
      } else if (c == 1) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const float umax = CAP ? mx[r] : mx[r] * p.scale_log2;
          const bool any = __builtin_amdgcn_ballot_w64(umax > m_ref[r] + kRescaleThreshold) != 0;
          const float m_new = any ? fmaxf(m_ref[r], umax) : m_ref[r];
          const float a = fast_exp2(m_ref[r] - m_new);
          alpha[r] = (any && m_new != neg_inf()) ? a : 1.0f;
          l_acc[r] *= alpha[r];
          m_ref[r] = m_new;
          resc |= any;
          msub[r] = (m_ref[r] == neg_inf()) ? 0.0f : m_ref[r];
        }
        asm volatile("" : "+v"(msub[0]), "+v"(msub[1]));
      } else if (c < 6) {
        const int r = (c - 2) >> 1, i0 = ((c - 2) & 1) * 8;
#pragma unroll
        for (int i = i0; i < i0 + 8; ++i)
          Sc[r][i] = CAP ? fast_exp2(Sc[r][i] - msub[r]) : fast_exp2(__builtin_fmaf(Sc[r][i], p.scale_log2, -msub[r]));
        if (i0 == 8) asm volatile("" : "+v"(Sc[r]));
      } else if (c == 6) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          float t[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) t[u] = (Sc[r][4 * u] + Sc[r][4 * u + 1]) + (Sc[r][4 * u + 2] + Sc[r][4 * u + 3]);
          l_acc[r] += (t[0] + t[1]) + (t[2] + t[3]);
        }
        asm volatile("" : "+v"(l_acc[0]), "+v"(l_acc[1]));
      } else {
        // B operand of PV for slice ks: keys 16*ks + 8*((i>>2) & 1) + 4*lg + (i&3), i = 8*ks .. 8*ks+7
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              f32x2 two = {Sc[r][ks * 8 + 2 * jj], Sc[r][ks * 8 + 2 * jj + 1]};
              bf16x2 pk = __builtin_convertvector(two, bf16x2);
              Pc[r][ks][2 * jj] = pk[0];
              Pc[r][ks][2 * jj + 1] = pk[1];
            }
        asm volatile("" : "+v"(Pc[0][0]), "+v"(Pc[0][1]), "+v"(Pc[1][0]), "+v"(Pc[1][1]));
      }
    };

    gread(0);
    gread(1);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if (g + 2 < 8) gread(g + 2);
      gmfma(g);
      if (g & 1) dma_piece(g >> 1);   // the tile's loads go out between MFMA groups
      __builtin_amdgcn_sched_barrier(0);
      vchunk(g);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (resc) {   // after PV(s2-1): bring O to the new reference max
      settle_o(O[0]);
      settle_o(O[1]);
#pragma unroll
      for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) O[r][db][i] *= alpha[r];
      settle_o(O[0]);
      settle_o(O[1]);
    }
  };

  for (int j = 0; j < n; ++j) {
    // K(j+2) and V(j+1) go out slab by slab inside the two steps. Near the
    // end of the list they repeat the last tile into a free stage, which
    // keeps the steps free of branches.
    const int kb_k = tile_kb(min(j + 2, n - 1)), kb_v = tile_kb(min(j + 1, n - 1));
    __bf16* kdst = kst + ((j + 2) % kWStages) * kWTile;
    __bf16* vdst = vst + ((j + 1) % kWStages) * kWTile;
    const int kb = tile_kb(j);
    const int cls = tile_cls(j);
    // even steps: softmax set A, weights into A; odd steps: set B
    step(2 * j, kb, cls, SA, SB, PB, PA,
         [&](int i) { dma_slab_w(kbase, krs, kb_k, p.Skv, kdst, w, koff[i], i); });
    step(2 * j + 1, kb, cls, SB, SA, PA, PB,
         [&](int i) { dma_slab_w(vbase, krs, kb_v, p.Skv, vdst, w, voff[i], i); });
    // K(j+2) and V(j+1) must have landed before the barrier
    wait_vmcnt_w<0>();
    __syncthreads();
  }
  bf16x8 (&Pp)[2][2] = PB;   // weights of the last (odd) step
  // ---- PV of the last step
  if (n > 0) {
    settle_p2(Pp);
    const char* Vt = v_at(nsteps - 1);
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const bf16x8 a = vread(Vt, f);
#pragma unroll
      for (int r = 0; r < 2; ++r) mfma_pv(O[r][f & 3], a, Pp[r][f >> 2]);
    }
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    settle_o(O[r]);
    epilogue<NDB>(O[r], m_ref[r], l_acc[r], p, b, h, q_ok[r] ? q_row[r] : p.Sq, lg);
  }
}

template <typename K>
hipError_t launch_w(K kernel, const AttnParams& p, hipStream_t s) {
  const int nQp = (p.nQb + 1) / 2;
  const int64_t T = (int64_t)p.B * p.H * nQp;
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
