// Block-sparse attention forward for bf16, D = 128, with a deep DMA pipeline and operands read a
// step ahead into registers. Serves attn_fwd_chunk (one visit) and the one-launch ring of
// ring_attn_fwd_1gpu (one visit per KV chunk).
//
// What it computes: the per-ring-step kernel call of the ejkernel ring-splash source page
// (_ring_attention_forward): attention of q over one KV chunk, returning the chunk output and
// log-sum-exp, folded into the running state with _update_out_and_lse (sigmoid weight,
// softplus lse) on every visit after the first. Masking follows the Kvax flash_attention
// arguments.
//
// Design for gfx950 (CDNA4):
//  * One workgroup = 4 waves = 128 query rows of one head, wave w owning rows 32w..32w+31; two
//    workgroups per CU, so each SIMD holds two waves of different workgroups that run freely
//    past each other: one wave's softmax arithmetic issues in the other's matrix-product
//    shadow.
//  * The workgroup walks the compacted list of its row of 128x64 mask tiles in steps of 32
//    keys. Step j of a wave: S(j+1) = K(j+1) Q^T (v_mfma_f32_32x32x16_bf16, K from registers,
//    Q held for the whole launch) in fenced groups of one product beside two exponentials of
//    S(j); then O^T += V(j)^T P(j)^T beside the bf16 packing and row sum of S(j); one barrier;
//    then the LDS reads of the next operands (K(j+2), V(j+1)), and the mask and row max of
//    S(j+1). The DMA of step j+kAltStages-1 goes out one instruction beside each of the last
//    four products of S(j+1) (with a soft cap: of the second half of O^T += V^T P^T, and step
//    j reads V(j) itself halfway through the products of S(j+1)).
//    The loop is unrolled by the ring depth, so stage offsets are immediates of the reads and
//    the two score register sets alternate. Scores are transposed, so a lane owns one query
//    row: row max and row sum are in-lane plus one v_permlane32_swap with the partner lane.
//  * K / V step tiles (32 keys x 256 B each, 16-byte chunks XOR-swizzled so the operand reads
//    are free of bank conflicts) come into a ring of kAltStages LDS stages by LDS DMA. The DMA
//    is issued from inline assembly, so the compiler does not see its LDS writes and places
//    its own waits only for the LDS reads it issues; the kernel orders the DMA with vmcnt waits
//    (only for the tile the next reads need) and barriers, both compiler memory barriers.
//  * V operands: read with transposing LDS reads from V's own rows, or (VP instantiations, the
//    rings that repack V with pack_v_kernel) with row reads like K's, from tiles that already
//    hold each lane's eight keys in the order the weights feed the product. A transposing read
//    moves under half the bytes per cycle of a row read.
//  * Soft cap: a step keeps u = -1 / (1 + exp2(2 scale log2(e) s / cap)); the capped logit is
//    cap log2(e) (1 + 2u), an affine map folded into the row maximum and the exponentials.
//  * Masks: FULL tiles run no mask code. PARTIAL tiles are masked either by one compare per
//    score against a per-row key limit (sequential key positions, no segments, no dense mask)
//    or, in the BITS instantiations, from the tile's stored element bits, which come into LDS
//    with the step's DMA. A FULL tile cut by the end of the chunk masks the keys past it.
//  * Online softmax in base 2 with the scale folded into one FMA; the running max is raised
//    only when a row's max grows by more than 2^8.
#include <type_traits>

#include "attn_common.h"

namespace ram {
namespace {

using namespace attn;

constexpr int kAltWaves = kAltRows / 32;                    // one wave per 32 query rows
constexpr int kAltThreads = 64 * kAltWaves;
constexpr int kAltKeys = 32;                                // keys per step
constexpr int kAltStages = 4;                               // LDS ring depth (steps)
constexpr int kAltTile = kAltKeys * 256;                    // bytes of one K or V step tile
constexpr int kDmaPerTile = kAltKeys / (4 * kAltWaves);     // 1 KiB DMA instructions per wave and tile
constexpr int kAltBitsBytes = kAltWaves * 256;              // one step's tile bits: 32 rows x 2 words per wave

template <bool BITS>
constexpr int alt_stage_bytes() {
  return 2 * kAltTile + (BITS ? kAltBitsBytes : 0);
}
static_assert(kPackKeys == kAltKeys && kPackTileBytes == kAltTile, "repacked V tiles are the kernel's steps");
// the stages and the longest tile list (one 8-byte record per tile) fit a CU's 160 KiB of LDS
static_assert(kAltStages * alt_stage_bytes<true>() + 8 * kMaxMaskCols <= 160 * 1024, "LDS budget");

// LDS DMA issued from inline assembly: 16 bytes per lane (4 for dma4) from the buffer at byte
// offset `voff` into LDS at m0 + 16 * lane (4 * lane). The compiler does not see these writes to
// LDS, so it never waits for them before its own LDS reads; the kernel orders them itself with
// vmcnt waits and barriers that are also compiler memory barriers (the "memory" clobber). m0 is
// set by every DMA statement and read by nothing else in this kernel.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds_byte, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_byte), "v"(voff), "s"(r)
               : "memory");
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t lds_byte, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds_byte), "v"(voff), "s"(r)
               : "memory");
}

// Wait until at most N vector-memory loads of this wave (the DMA included) are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// Wait until at most PER * k vector loads are outstanding, k in [0, K] (a runtime value picks
// among compile-time immediates).
template <int PER, int K>
__device__ __forceinline__ void wait_vm_steps(int k) {
  if constexpr (K == 0) {
    wait_vm<0>();
  } else {
    if (k >= K) wait_vm<PER * K>();
    else wait_vm_steps<PER, K - 1>(k);
  }
}
// Workgroup barrier that is also a compiler memory barrier (LDS written by DMA is read after it).
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" : : : "memory"); }

__device__ __forceinline__ bf16x8 lds_b128(uint32_t byte) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>((uintptr_t)byte);
}
__device__ __forceinline__ uint32_t lds_b32(uint32_t byte) {
  return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>((uintptr_t)byte);
}
// One V operand: two transposing reads, 8 rows (2048 bytes) apart, joined.
__device__ __forceinline__ bf16x8 lds_v_operand(uint32_t byte) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) s16x4*>((uintptr_t)byte));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      reinterpret_cast<__attribute__((address_space(3))) s16x4*>((uintptr_t)(byte + 2048)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Mask of one step's scores. kind: 0 no mask, 1 keys at or past `thr` (lane-relative key
// offset) masked, 2 from bits `bw` (key 8*(i>>2) + 4*lg + (i&3) at bit 8*(i>>2) + 4*lg + (i&3)).
template <bool BITS>
__device__ __forceinline__ void step_mask(f32x16& S, int kind, int thr, uint32_t bw, int lg) {
  if constexpr (!BITS) {
    if (kind == 1) {
      asm volatile("" : "+v"(thr));   // keep the compares next to their use
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + (i & 3) >= thr) S[i] = neg_inf();
    }
  } else if (kind != 0) {
    // Both kinds as one word whose bit 8*(i>>2) + (i&3) keeps score i: one masking pass over the
    // scores (two separately masked copies of them would not fit the register budget).
    const uint32_t below = thr <= 0 ? 0u : (thr >= 32 ? ~0u : (1u << thr) - 1u);
    const uint32_t keep = kind == 1 ? below : (bw >> (4 * lg));
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (((keep >> (8 * (i >> 2) + (i & 3))) & 1u) == 0u) S[i] = neg_inf();
  }
}

// Row max of one step's (capped, masked) scores in the running max's units: whether some row
// grew by more than 2^8 over m_ref (wave-uniform), and the new max and the factor for O and l.
template <bool CAP>
__device__ __forceinline__ bool step_max(const f32x16& S, float m_ref, float& m_new, float& alpha,
                                         const AttnParams& p) {
  float all[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) all[i] = S[i];
  const float mx = pair_max(max_tree3(all));
  const float umax = CAP ? __builtin_fmaf(mx, 2.0f * p.cap_log2, p.cap_log2) : mx * p.scale_log2;
  m_new = fmaxf(m_ref, umax);
  alpha = (m_new == neg_inf()) ? 1.0f : fast_exp2(m_ref - m_new);
  return __builtin_amdgcn_ballot_w64(umax > m_ref + kRescaleThreshold) != 0;
}

// With a soft cap the step's scores are kept as u = -1 / (1 + exp2(k2 * s)), k2 = 2 scale log2(e) /
// cap, in [-1, 0] and increasing in s: the capped logit in log2 units, cap log2(e) tanh(scale s /
// cap), is c (1 + 2u) with c = cap log2(e). That affine map is folded into the products that use
// it (the row maximum, one value per lane, and the exponentials' FMA), which saves two VALU
// operations per score over forming the capped logit itself. Masked scores are -inf in either
// form.
template <bool CAP>
__device__ __forceinline__ void step_cap(f32x16& S, const AttnParams& p) {
  if constexpr (CAP) {
#pragma unroll
    for (int i = 0; i < 16; ++i) S[i] = __builtin_amdgcn_rcpf(-1.0f - fast_exp2(S[i] * p.cap_k2));
  }
}

template <bool CAP, bool BITS, bool SPLIT, bool VP>
__global__ __launch_bounds__(kAltThreads, 2) void attn_fwd_bf16_alt(AttnParams p, RingSplit rs) {
  constexpr int D = 128;
  constexpr int NS = kAltStages;
  constexpr int SB = alt_stage_bytes<BITS>();
  constexpr int NDMA = 2 * kDmaPerTile + (BITS ? 1 : 0);   // DMA instructions per wave and step
  // Step j issues the DMA of step j + NS - 1 one instruction at a time beside its products (the
  // last four of S(j+1), or with a soft cap the second half of O += V P): a burst of LDS-DMA
  // instructions from every wave right after the barrier holds each wave for tens of cycles per
  // instruction.
  // LATE_V: with a soft cap, step j reads its V operands itself, halfway through the products of
  // S(j+1), instead of the step before reading them after its barrier (measured faster for the
  // cap kernels only, whose step is longer).
  constexpr bool LATE_V = CAP;
  // EARLY_MAX: with a soft cap, the mask, row max and rescale of S(j+1) run before step j's
  // barrier (after its products) instead of after it (measured faster for the cap kernels only).
  constexpr bool EARLY_MAX = CAP;
  // NS stages of SB bytes, then the visit's tile list (AltTile records, p.nKb of them), staged
  // once per visit so that the loop reads it from LDS instead of waiting on scalar loads
  extern __shared__ __attribute__((aligned(16))) char smem[];
  uint2* tinfo = reinterpret_cast<uint2*>(smem + NS * SB);

  // SPLIT: two workgroups per row, each with half the visits (an instantiation of its own)
  int b, h, qb, sp = 0;
  if (!decode_work(p, b, h, qb, SPLIT ? 2 : 1, SPLIT ? &sp : nullptr)) return;
  // wave-uniform: keep them (and the addresses made from them) in scalar registers
  b = __builtin_amdgcn_readfirstlane(b);
  h = __builtin_amdgcn_readfirstlane(h);
  qb = __builtin_amdgcn_readfirstlane(qb);
  sp = __builtin_amdgcn_readfirstlane(sp);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, lg = lane >> 5;
  const int G = p.H / p.Hkv;
  const int g = h / G;
  const int q_row = qb * kAltRows + w * 32 + ln;
  const bool q_ok = q_row < p.Sq;
  const int64_t mrow = (int64_t)b * p.nQb + qb;

  // Q fragments (B operand of S^T = K Q^T): lane holds row q_row, dims 16*ds + 8*lg .. +7.
  bf16x8 qf[8];
  {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.q_stride_b +
                         ((int64_t)(q_ok ? q_row : 0) * p.H + h) * D;
#pragma unroll
    for (int ds = 0; ds < 8; ++ds) {
      const bf16x8 t = *reinterpret_cast<const bf16x8*>(qrow + ds * 16 + lg * 8);
      qf[ds] = q_ok ? t : bf16x8{};
    }
  }
  const int qrow_c = q_ok ? q_row : p.Sq - 1;
  const int qpos = p.q_pos ? p.q_pos[(int64_t)b * p.qm_stride_b + qrow_c] : p.q_pos_base + q_row;

  const uint32_t row_bytes = (uint32_t)p.Hkv * D * 2;   // bytes between key rows
  const uint32_t half_bytes = kAltKeys * row_bytes;      // second step of a 64-key tile
  // DMA: wave w fills rows 4*(w + kAltWaves*i) .. +3 of a step tile (i < kDmaPerTile); lane l
  // writes physical 16-byte chunk l & 15 of row 4*(w + kAltWaves*i) + (l >> 4), i.e. 1 KiB of
  // consecutive LDS bytes per instruction.
  // VP: V comes repacked (launch_pack_v), each step tile the 8 KiB LDS image itself, so the same
  // wave copies the same 1 KiB pieces of it linearly.
  uint32_t koff[kDmaPerTile], voff[kDmaPerTile];
#pragma unroll
  for (int i = 0; i < kDmaPerTile; ++i) {
    const int dr = 4 * (w + kAltWaves * i) + (lane >> 4), phys = lane & 15;
    koff[i] = (uint32_t)dr * row_bytes + (uint32_t)((phys ^ (dr & 15)) * 16);
    voff[i] = VP ? (uint32_t)(w + kAltWaves * i) * 1024 + (uint32_t)lane * 16
                 : (uint32_t)dr * row_bytes + (uint32_t)((phys ^ (4 * (dr & 3))) * 16);
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  // Operand read offsets inside a stage. K: row ln, logical chunk 2*ds + lg.
  uint32_t k_rd[8];
#pragma unroll
  for (int ds = 0; ds < 8; ++ds) k_rd[ds] = ln * 256 + (((2 * ds + lg) ^ (ln & 15)) * 16);
  // V (transposing reads, see lds_read_tr16): row 4*lg + r4 (+8, +16, +24), head dims
  // db*32 + 16*hs + 4*(lane&3) .. +3, r4 = (lane&15)>>2, hs = (lane>>4)&1.
  const int r4 = (lane & 15) >> 2, hs = (lane >> 4) & 1;
  uint32_t v_rd[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
    v_rd[db] = kAltTile + (4 * lg + r4) * 256 + ((((db * 4 + 2 * hs + ((lane & 3) >> 1)) ^ (4 * r4)) * 16) +
                                                 (lane & 1) * 8);
  const uint32_t b_rd = 2 * kAltTile + w * 256 + ln * 8;   // + 4 * (step parity)

  // this workgroup's visits (all of them, or one of the two halves of a split ring)
  const int t_half = (p.n_chunks + 1) / 2;
  const int t_begin = (SPLIT && sp == 1) ? t_half : 0;
  const int t_end = (SPLIT && sp == 0) ? t_half : p.n_chunks;
  for (int t = t_begin; t < t_end; ++t) {
    AttnParams pc = p;   // this visit's chunk
    ring_chunk_view(pc, p, t);
    if (SPLIT && sp == 1) {
      // the second half runs its own ring into out2 / lse2, starting as a first visit does
      pc.out = rs.out2;
      pc.lse = rs.lse2;
      if (t == t_begin) pc.mode = p.mode;
    }
    const int cnt = pc.row_cnt[mrow];
    // a merge with nothing to add is the identity (unless the result must be converted to its
    // final type, which the epilogue does for empty rows)
    if (cnt == 0 && pc.mode == 1 && pc.sinks == nullptr && pc.out_final == nullptr) continue;
    const int n = 2 * cnt;   // steps of 32 keys
    const int32_t* cols = pc.col_idx + mrow * p.nKb;
    const uint8_t* cls = pc.tile_class + mrow * p.nKb;

    float m_ref = neg_inf(), l_acc = 0.0f;
    if (pc.sinks) {
      m_ref = pc.sinks[h] * kLog2e;
      l_acc = (lg == 0) ? 1.0f : 0.0f;
    }
    f32x16 O[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) O[db] = f32x16{};
    // keys at or past lim (chunk-relative) are masked in PARTIAL tiles of the positional kernels,
    // keys at or past Skv in FULL tiles cut by the chunk end
    int lim = p.Skv;
    if (!BITS && p.causal) {
      const int64_t reach = (int64_t)qpos - pc.kv_pos_base + 1;
      lim = (int)max<int64_t>(-1, min<int64_t>(p.Skv, reach));
    }

    // K / V of this (batch, kv head) in this chunk: one buffer resource each, spanning the
    // chunk's Skv key rows, so that rows past the chunk end read as zeros (their scores are
    // masked). Byte offsets into it fit 32 bits (the host checks Skv * row_bytes).
    const auto krs = tile_rsrc(reinterpret_cast<const __bf16*>(pc.k) + (int64_t)b * p.kv_stride_b + g * D,
                               (uint32_t)p.Skv * row_bytes);
    const int n_vt = (p.Skv + kAltKeys - 1) / kAltKeys;   // packed V tiles of the chunk
    const auto vrs = VP ? tile_rsrc(static_cast<const char*>(pc.vt) + ((int64_t)b * p.Hkv + g) * n_vt * kAltTile,
                                    (uint32_t)n_vt * kAltTile)
                        : tile_rsrc(reinterpret_cast<const __bf16*>(pc.v) + (int64_t)b * p.kv_stride_b + g * D,
                                    (uint32_t)p.Skv * row_bytes);
    // DMA of step s (parity PAR, tile record `tr`) into stage st: this wave's rows of K and V
    // (dma_piece, instruction i: K rows of piece i / 2 for even i, V rows for odd i) and (BITS,
    // dma_bits) its 32 rows' bit words of the tile when it is PARTIAL.
    auto dma_piece = [&](auto PAR_, int st, uint2 tr, int i) {
      constexpr int PAR = decltype(PAR_)::value;
      const uint32_t soff = (tr.x & ~63u) + (PAR ? half_bytes : 0u);
      // packed V: tile (first key / 32 + PAR) of the chunk
      const uint32_t soff_v = VP ? tr.y * (kAltTile / kAltKeys) + (PAR ? (uint32_t)kAltTile : 0u) : soff;
      const uint32_t sb = lds0 + st * SB;
      const int t = i >> 1;
      if ((i & 1) == 0) dma16(krs, sb + 4 * (w + kAltWaves * t) * 256, koff[t] + soff);
      else dma16(vrs, sb + kAltTile + 4 * (w + kAltWaves * t) * 256, voff[t] + soff_v);
    };
    auto dma_bits = [&](auto PAR_, int st, uint2 tr) {
      constexpr int PAR = decltype(PAR_)::value;
      if constexpr (BITS) {
        const uint32_t sb = lds0 + st * SB;
        const int kb = (int)(tr.y >> 6);
        const bool partial = ((tr.x >> (2 * PAR)) & 3u) == 2u;
        const uint32_t* words = pc.mask_bits + ((mrow * p.nKb + kb) * kAltRows + w * 32) * 2;
        const auto br = tile_rsrc(words, partial ? 256u : 0u);
        dma4(br, sb + 2 * kAltTile + w * 256, (uint32_t)lane * 4);
      }
    };
    auto dma_step = [&](auto PAR_, int st, uint2 tr) {   // all of it
#pragma unroll
      for (int i = 0; i < 2 * kDmaPerTile; ++i) dma_piece(PAR_, st, tr, i);
      dma_bits(PAR_, st, tr);
    };
    // mask kind (0 none, 1 key limit, 2 bits) and lane-relative key limit of a step of parity PAR
    auto step_info = [&](auto PAR_, uint2 tr, int& kind, int& thr) {
      constexpr int PAR = decltype(PAR_)::value;
      kind = (int)((tr.x >> (2 * PAR)) & 3u);
      thr = lim - ((int)tr.y + PAR * kAltKeys + 4 * lg);
    };
    // tile record of step s (clamped to the list), read from LDS
    auto info = [&](int s) { return tinfo[min(s >> 1, cnt - 1)]; };
    auto uniform = [](uint2 t) {
      return make_uint2(__builtin_amdgcn_readfirstlane(t.x), __builtin_amdgcn_readfirstlane(t.y));
    };

    // Every wave is done with the previous visit's stages and list; then this visit's list. A
    // tile's record: x = byte offset of its first key row, with the mask kinds of its two steps
    // in bits 0-1 and 2-3 (the offset is a multiple of 64); y = its first key.
    __syncthreads();
    for (int i = tid; i < cnt; i += kAltThreads) {
      const int kb = cols[i];
      const int c = cls[kb];
      const int k0 = kb * kBlockKV;
      uint32_t kinds = 0;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const bool cut = k0 + (hf + 1) * kAltKeys > p.Skv;
        const uint32_t kind = (BITS && c == 1) ? 2u : ((c != 2 || cut) ? 1u : 0u);
        kinds |= kind << (2 * hf);
      }
      tinfo[i] = make_uint2((uint32_t)k0 * row_bytes | kinds, (uint32_t)k0);
    }
    __syncthreads();
    if (n > 0) {
      const int pre = min(NS - 1, n);
      {
        uint2 inf[(NS + 1) / 2];
#pragma unroll
        for (int e = 0; e < (NS + 1) / 2; ++e) inf[e] = uniform(tinfo[min(e, cnt - 1)]);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          if (s < pre) {
            if (s & 1) dma_step(std::integral_constant<int, 1>{}, s, inf[s >> 1]);
            else dma_step(std::integral_constant<int, 0>{}, s, inf[s >> 1]);
          }
        }
      }
      // steps 0 and 1 must have landed (n is even, so n >= 2)
      wait_vm_steps<NDMA, NS - 2>(pre - 2);
      barrier();

      bf16x8 kf[8], vf[8];
      bf16x8 P[2];
      // scores of the step being exponentiated and of the next one, alternating between the two
      // registers sets with the step's parity (the loop is unrolled by NS, which is even)
      f32x16 S2[2];
      // S(0), its mask and row max
      S2[0] = f32x16{};
#pragma unroll
      for (int ds = 0; ds < 8; ++ds)
        S2[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_b128(lds0 + k_rd[ds]), qf[ds], S2[0], 0, 0, 0);
      {
        int kind, thr;
        step_info(std::integral_constant<int, 0>{}, uniform(info(0)), kind, thr);
        step_cap<CAP>(S2[0], p);
        step_mask<BITS>(S2[0], kind, thr, BITS ? lds_b32(lds0 + b_rd) : 0u, lg);
        float m_new, alpha;
        if (step_max<CAP>(S2[0], m_ref, m_new, alpha, p)) {
          l_acc *= alpha;
          m_ref = m_new;
        }
      }
      // operands of step 1 (K) and step 0 (V); list entries a step ahead. Operand addresses are
      // a per-lane base plus compile-time offsets (stage, key block), folded into the reads.
      uint32_t kad[8], vad[4];
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) kad[ds] = lds0 + k_rd[ds];
#pragma unroll
      for (int db = 0; db < 4; ++db) vad[db] = lds0 + v_rd[db];
#pragma unroll
      for (int ds = 0; ds < 8; ++ds) kf[ds] = lds_b128(kad[ds] + SB);
      if constexpr (!LATE_V) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          vf[i] = VP ? lds_b128(kad[i] + kAltTile) : lds_v_operand(vad[i & 3] + (i >> 2) * 4096);
      }
      uint2 inf_dma = info(NS - 1), inf_msk = info(1);

      // Step j (stage j % NS == JS): products, barrier, loads. STEADY: a step at least 2 NS - 1
      // steps before the end, which issues its DMA and reads the next operands unconditionally
      // and waits for a fixed number of DMA steps.
      auto step = [&](auto JS_, auto STEADY_, int j) {
        constexpr int JS = decltype(JS_)::value;
        constexpr bool STEADY = decltype(STEADY_)::value;
        constexpr int CUR = JS & 1, NXT = CUR ^ 1;
        constexpr int ST1 = (JS + 1) % NS, ST2 = (JS + 2) % NS;
        f32x16& Sc = S2[CUR];
        f32x16& Sn = S2[NXT];
        // mask and row max of S(j+1) (tile record inf_m) and, when a row's max grew by more than
        // 2^8, the rescale of O and l (after the products of step j, which used the previous max)
        auto next_max = [&](uint2 inf_m) {
          int kind, thr;
          step_info(std::integral_constant<int, NXT>{}, inf_m, kind, thr);
          step_cap<CAP>(Sn, p);
          step_mask<BITS>(Sn, kind, thr, BITS ? lds_b32(lds0 + ST1 * SB + b_rd + 4 * ((JS + 1) & 1)) : 0u, lg);
          float m_new, alpha;
          if (step_max<CAP>(Sn, m_ref, m_new, alpha, p)) {
            l_acc *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
              for (int i = 0; i < 16; ++i) O[db][i] *= alpha;
            m_ref = m_new;
          }
        };
        // ---------------------------------------------------------------- products of step j
        // S(j+1) = K(j+1) Q^T in fenced groups of one product and two exponentials of S(j), then
        // O^T += V(j)^T P(j)^T beside the bf16 packing. On the last step the first product runs
        // on stale operands and its result is not used.
        // The products run at raised wave priority: with two workgroups per CU, the wave whose
        // matrix products are ready issues first and the other fills the slots between them.
        __builtin_amdgcn_s_setprio(1);
        Sn = f32x16{};
        // the DMA of step j + NS - 1, into the stage of step j - 1 (every wave is past the barrier
        // that followed its last reads)
        const bool dma_now = STEADY || j + NS - 1 < n;
        using PD = std::integral_constant<int, (JS + 1) & 1>;
        constexpr int STD = (JS + NS - 1) % NS;
        const uint2 inf_ds = uniform(inf_dma);
        {
          const float msub = (m_ref == neg_inf()) ? 0.0f : m_ref;
          // weight = exp2(logit - m): the logit is sc * s without a cap, c (1 + 2u) with one
          const float sc = CAP ? 2.0f * p.cap_log2 : p.scale_log2;
          const float sub = CAP ? p.cap_log2 - msub : -msub;
#pragma unroll
          for (int ds = 0; ds < 8; ++ds) {
            if (LATE_V && ds == 4) {
              // V(j): its tile landed before the barrier of step j - 2, and the barrier of step j
              // follows the products that use it
              __builtin_amdgcn_sched_barrier(0);
#pragma unroll
              for (int i = 0; i < 8; ++i)
                vf[i] = VP ? lds_b128(kad[i] + kAltTile + JS * SB) : lds_v_operand(vad[i & 3] + JS * SB + (i >> 2) * 4096);
            }
            Sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ds], qf[ds], Sn, 0, 0, 0);
            float e0 = fast_exp2(__builtin_fmaf(Sc[2 * ds], sc, sub));
            float e1 = fast_exp2(__builtin_fmaf(Sc[2 * ds + 1], sc, sub));
            // pin the product and the two exponentials to this group (the compiler would
            // otherwise move the products next to their use)
            asm volatile("" : "+v"(Sn), "+v"(e0), "+v"(e1));
            Sc[2 * ds] = e0;
            Sc[2 * ds + 1] = e1;
            if (!CAP && ds >= 8 - 2 * kDmaPerTile && dma_now) dma_piece(PD{}, STD, inf_ds, ds - (8 - 2 * kDmaPerTile));
          }
          if (dma_now) dma_bits(PD{}, STD, inf_ds);
        }
#pragma unroll
        for (int j2 = 0; j2 < 4; ++j2) {
          f32x2 two = {Sc[2 * j2], Sc[2 * j2 + 1]};
          const bf16x2 pk = __builtin_convertvector(two, bf16x2);
          P[0][2 * j2] = pk[0];
          P[0][2 * j2 + 1] = pk[1];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          O[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], P[0], O[i], 0, 0, 0);
          if (i == 0) {
#pragma unroll
            for (int j2 = 0; j2 < 4; ++j2) {
              f32x2 two = {Sc[8 + 2 * j2], Sc[8 + 2 * j2 + 1]};
              const bf16x2 pk = __builtin_convertvector(two, bf16x2);
              P[1][2 * j2] = pk[0];
              P[1][2 * j2 + 1] = pk[1];
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          O[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[4 + i], P[1], O[i], 0, 0, 0);
          if (CAP && dma_now) dma_piece(PD{}, STD, inf_ds, i);
          if (CAP) __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        {
          // row sum as a tree, in fp32 (bf16 weights would put up to 2^-9 into the lse of a row
          // with few keys)
          const float t0 = (Sc[0] + Sc[1]) + (Sc[2] + Sc[3]);
          const float t1 = (Sc[4] + Sc[5]) + (Sc[6] + Sc[7]);
          const float t2 = (Sc[8] + Sc[9]) + (Sc[10] + Sc[11]);
          const float t3 = (Sc[12] + Sc[13]) + (Sc[14] + Sc[15]);
          l_acc += (t0 + t1) + (t2 + t3);
        }
        if (EARLY_MAX && (STEADY || j + 1 < n)) next_max(uniform(inf_msk));
        // step j+2's tile (read below) has landed: this wave issued its DMA through step
        // min(n, j+NS)-1, the tile's being at most NS-3 steps before the newest; the barrier
        // makes every wave's share visible and shows that every wave is done with step j's
        // stage (its last reads fed this step's products)
        if (STEADY) wait_vm<NDMA * (NS - 3)>();
        else if (j + 2 < n) wait_vm_steps<NDMA, NS - 3>(min(n, j + NS) - 1 - (j + 2));
        barrier();

        // ---------------------------------------------------------------- loads of step j
        // The operand reads for the next products (K(j+2), and V(j+1) unless LATE_V) and the
        // list reads, then (unless EARLY_MAX) the mask and row max of S(j+1) and, when a row's
        // max grew by more than 2^8, the rescale of O and l.
        const bool has_next = STEADY || j + 1 < n;
        const uint2 inf_m = EARLY_MAX ? uint2{} : uniform(inf_msk);   // S(j+1)'s record
        if (STEADY || j + 2 < n) {
#pragma unroll
          for (int ds = 0; ds < 8; ++ds) kf[ds] = lds_b128(kad[ds] + ST2 * SB);
        }
        if (has_next) {
          if constexpr (!LATE_V) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
              vf[i] = VP ? lds_b128(kad[i] + kAltTile + ST1 * SB)
                         : lds_v_operand(vad[i & 3] + ST1 * SB + (i >> 2) * 4096);
          }
          inf_dma = info(j + NS);
          inf_msk = info(j + 2);
          if constexpr (!EARLY_MAX) next_max(inf_m);
        }
      };
      static_assert(NS == 4, "the step loop is unrolled by the ring depth");
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      using I3 = std::integral_constant<int, 3>;
      using Steady = std::true_type;
      using Tail = std::false_type;
      int j = 0;
      for (; j + 2 * NS <= n; j += NS) {
        step(I0{}, Steady{}, j);
        step(I1{}, Steady{}, j + 1);
        step(I2{}, Steady{}, j + 2);
        step(I3{}, Steady{}, j + 3);
      }
      // the last 2 NS - 1 steps or fewer; n is even: groups of four steps, then possibly two
      for (; j < n; j += NS) {
        step(I0{}, Tail{}, j);
        step(I1{}, Tail{}, j + 1);
        if (j + 2 >= n) break;
        step(I2{}, Tail{}, j + 2);
        step(I3{}, Tail{}, j + 3);
      }
    }
    epilogue<4>(O, m_ref, l_acc, pc, b, h, q_row, lg);
  }
}

template <bool CAP, bool BITS, bool SPLIT, bool VP>
hipError_t launch_alt(const AttnParams& p, const RingSplit& rs, hipStream_t s) {
  const int S = SPLIT ? 2 : 1;
  const int64_t T = (int64_t)p.B * p.H * p.nQb * S;
  const size_t lds = (size_t)kAltStages * alt_stage_bytes<BITS>() + sizeof(uint2) * (size_t)max(1, p.nKb);
  hipLaunchKernelGGL((attn_fwd_bf16_alt<CAP, BITS, SPLIT, VP>), dim3((unsigned)(8 * ((T + 7) / 8))),
                     dim3(kAltThreads), lds, s, p, rs);
  return hipGetLastError();
}

// Repacked V (VP) is built without the soft cap only: the host repacks V for rings without one.
template <bool VP>
hipError_t launch_alt_v(const AttnParams& p, const RingSplit* split, hipStream_t s) {
  const bool cap = p.softcap_on != 0, bits = p.mask_bits != nullptr;
  const RingSplit rs = split ? *split : RingSplit{nullptr, nullptr};
  if constexpr (VP) {
    if (cap) return hipErrorInvalidValue;
    if (split) return bits ? launch_alt<false, true, true, true>(p, rs, s) : launch_alt<false, false, true, true>(p, rs, s);
    return bits ? launch_alt<false, true, false, true>(p, rs, s) : launch_alt<false, false, false, true>(p, rs, s);
  } else {
    if (split) {
      if (cap) return bits ? launch_alt<true, true, true, false>(p, rs, s) : launch_alt<true, false, true, false>(p, rs, s);
      return bits ? launch_alt<false, true, true, false>(p, rs, s) : launch_alt<false, false, true, false>(p, rs, s);
    }
    if (cap) return bits ? launch_alt<true, true, false, false>(p, rs, s) : launch_alt<true, false, false, false>(p, rs, s);
    return bits ? launch_alt<false, true, false, false>(p, rs, s) : launch_alt<false, false, false, false>(p, rs, s);
  }
}

// V repacked for row reads. Workgroup = one 32-key step tile of one (chunk, batch, kv head): the
// tile's 32 key rows of 128 dims come into LDS with coalesced 16-byte loads (rows past Skv as
// zeros), then each thread writes two 16-byte chunks of the tile's LDS image. Image chunk
// o = 16 r + p holds logical chunk c = p ^ (r & 15) of row r (the kernel's swizzle for row
// reads), and logical chunk c = 2 i + g of row r is what lane (r, g) reads as V operand i:
// dim 32 (i & 3) + r of the keys 16 (i >> 2) + 8 (m >> 2) + 4 g + (m & 3), m = 0..7, the key
// order in which the weights' accumulator hands its 16 values to the product.
__global__ __launch_bounds__(256) void pack_v_kernel(const __bf16* v_all, int64_t kv_stride_b, int B, int Skv,
                                                     int Hkv, int n_vt, char* vt) {
  constexpr int D = 128;
  __shared__ __attribute__((aligned(16))) __bf16 tile[kAltKeys * D];
  const int g = blockIdx.x / n_vt, t = blockIdx.x - g * n_vt;
  const int b = blockIdx.y, c = blockIdx.z;
  const int tid = threadIdx.x;
  const __bf16* src = v_all + (int64_t)b * kv_stride_b + ((int64_t)c * Skv * Hkv + g) * D;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int e = tid + 256 * r;              // 16-byte piece: key e / 16, dims 8 (e % 16) ..
    const int key = t * kAltKeys + e / 16;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (key < Skv) x = *reinterpret_cast<const uint4*>(src + (int64_t)key * Hkv * D + (e % 16) * 8);
    *reinterpret_cast<uint4*>(tile + (e / 16) * D + (e % 16) * 8) = x;
  }
  __syncthreads();
  char* dst = vt + (((int64_t)c * B + b) * Hkv + g) * n_vt * kAltTile + (int64_t)t * kAltTile;
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int o = tid + 256 * r;
    const int row = o / 16, lc = (o % 16) ^ (row & 15);
    const int i = lc >> 1, lg = lc & 1;
    const int dim = 32 * (i & 3) + row;
    __bf16 out[8];
#pragma unroll
    for (int m = 0; m < 8; ++m) out[m] = tile[(16 * (i >> 2) + 8 * (m >> 2) + 4 * lg + (m & 3)) * D + dim];
    *reinterpret_cast<uint4*>(dst + o * 16) = *reinterpret_cast<const uint4*>(out);
  }
}

}  // namespace

hipError_t launch_pack_v(const void* v_all, int64_t kv_stride_b, int B, int n_chunks, int Skv, int Hkv, void* vt,
                         hipStream_t s) {
  const int n_vt = (Skv + kAltKeys - 1) / kAltKeys;
  if ((int64_t)B * n_chunks * n_vt * Hkv == 0) return hipSuccess;
  if (B > 65535 || n_chunks > 65535 || (int64_t)n_vt * Hkv > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pack_v_kernel, dim3((unsigned)(n_vt * Hkv), (unsigned)B, (unsigned)n_chunks), dim3(256), 0, s,
                     static_cast<const __bf16*>(v_all), kv_stride_b, B, Skv, Hkv, n_vt, static_cast<char*>(vt));
  return hipGetLastError();
}

hipError_t launch_attn_alt(const AttnParams& p, const RingSplit* split, hipStream_t s) {
  if (p.n_chunks < 1) return hipErrorInvalidValue;
  return p.vt ? launch_alt_v<true>(p, split, s) : launch_alt_v<false>(p, split, s);
}

}  // namespace ram
