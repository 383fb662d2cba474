// Block-sparse attention backward for one KV chunk, and its helpers.
//
// What it computes: the per-step call of the ejkernel ring-splash page's
// _ring_attention_backward: the gradients of one chunk's attention given the
// final out and logsumexp of the whole ring (so the chunk's weights are its
// share of the global softmax). For query row i, allowed key j:
//   p_ij = exp(u_ij - lse_i),  dp_ij = dout_i . v_j,  D_i = dout_i . out_i,
//   ds_ij = p_ij (dp_ij - D_i) (1 - t_ij^2 with the soft cap, t = u / cap),
//   dq_i += scale * sum_j ds_ij k_j,  dk_j = scale * sum_i ds_ij q_i,
//   dv_j = sum_i p_ij dout_i   (dk, dv summed over the heads sharing a KV head).
//
// Design for gfx950 (bf16, D = 128 or 64; v_mfma_f32_32x32x16_bf16 throughout):
//  * dq: one workgroup per (batch, head, 128-row q tile), the forward's layout:
//    S^T = K Q^T and dP^T = V dO^T with Q and dO held in registers as B
//    operands (a lane owns one query row), then dQ^T += K^T dS^T with dS^T
//    going from the accumulator to the B operand in registers and K^T read
//    from LDS with the transposing read. Walks the row's non-EMPTY kv tiles.
//  * dk / dv: one workgroup per (batch, kv head, 64-key tile); a wave owns 32
//    keys and one half of every 64-row q step, with K and V held in registers
//    as B operands (a lane owns one key): S = Q K^T, dP = dO V^T, then
//    dV^T += dO^T P and dK^T += Q^T dS with Q^T and dO^T read transposed from
//    LDS. Walks the kv tile's non-EMPTY q tiles (the transposed tile lists)
//    and every head of the KV group; the two waves of a key block add their
//    halves through LDS at the end. No atomics anywhere: results are
//    deterministic.
//  * Tiles move HBM -> LDS by DMA. Every tile is read both row-wise and with
//    the transposing read, so 16-byte chunks are swizzled: with 256-byte rows
//    (D = 128) by chunk ^ (4*(row & 3) + ((row >> 2) & 3)), with 128-byte rows
//    (D = 64) by chunk ^ (4*((row >> 1) & 1) + ((row >> 2) & 3)). Either way
//    16 consecutive rows put one logical chunk in 16 distinct bank groups,
//    and the 4 rows x 64 bytes of a transposing read cover all 64 banks.
//  * Row values (lse, D) of rows past Sq or with lse = -inf become +inf / 0,
//    so their weights are exactly 0.
#include <cstdlib>
#include <cstring>

#include "attn_common.h"

namespace ram {
namespace {

using namespace attn;

// Tile geometry for head dim D: 64-row tiles of D bf16 (2D-byte rows, D/8 chunks of 16 bytes).
template <int D>
struct Geo {
  static constexpr int NDS = D / 16;            // 16-deep MFMA steps over D
  static constexpr int NDB = D / 32;            // 32-wide blocks of D
  static constexpr int kTileElems = 64 * D;     // one 64-row tile (elements)
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kChunks = D / 8;         // 16-byte chunks per row
  static constexpr int kSlabRows = 64 / kChunks;  // rows one 16-byte DMA of a wave fills
};

template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return 4 * (row & 3) + ((row >> 2) & 3);
  else return 4 * ((row >> 1) & 1) + ((row >> 2) & 3);
}

// Byte offsets of this lane's DMA chunks: wave w fills rows [16w, 16w + 16) of
// a 64-row tile in slabs of kSlabRows rows; lane l of slab i writes physical
// chunk l % kChunks of row 16w + kSlabRows*i + l / kChunks, fetched from the
// logical chunk at that position. `row_bytes` is the global row stride.
template <int D, int N>
__device__ __forceinline__ void dma_offsets(uint32_t (&off)[N], int w, int lane, uint32_t row_bytes) {
  using Gm = Geo<D>;
  static_assert(N == 16 / Gm::kSlabRows, "one offset per slab");
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const int r = 16 * w + Gm::kSlabRows * i + lane / Gm::kChunks;
    off[i] = (uint32_t)r * row_bytes + ((lane % Gm::kChunks) ^ swz<D>(r)) * 16;
  }
}
// LDS-DMA of 16 / 4 bytes per lane. Kernel lambdas reach the builtin only
// through these plain functions: a builtin call whose arguments depend on a
// template parameter inside a lambda (which the host pass also compiles) makes
// the host pass drop the kernel's launch stub without a diagnostic.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, const void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, const void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, off, 0, 0, 0);
}
// (D is a constant once inlined)
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t r, __bf16* tile, const uint32_t* off, int w, int D) {
  const int slab_rows = 512 / D, n = 16 / slab_rows;
#pragma unroll
  for (int i = 0; i < n; ++i) dma16(r, tile + (16 * w + slab_rows * i) * D, off[i]);
}

// Row read (16 bytes): row `row`, logical chunk c.
template <int D>
__device__ __forceinline__ bf16x8 lds_row(const char* tile, int row, int c) {
  return *reinterpret_cast<const bf16x8*>(tile + row * (2 * D) + ((c ^ swz<D>(row)) * 16));
}
// Transposed operand of 32 columns x 16 rows starting at row r0, column block db:
// lane receives column db*32 + (lane & 31) at rows r0 + 4*lg + 0..3 and r0 + 8 + 4*lg + 0..3.
// Issued from assembly (see lds_tr_pair_issue): the value must pass lds_settle().
template <int D>
__device__ __forceinline__ TrPair lds_tr(const char* tile, int r0, int db, int lane) {
  const int lg = lane >> 5, r4 = (lane & 15) >> 2, hs = (lane >> 4) & 1;
  const int c = 4 * db + 2 * hs + ((lane & 3) >> 1);
  const int ra = r0 + 4 * lg + r4, rb = ra + 8;
  const char* pa = tile + ra * (2 * D) + ((c ^ swz<D>(ra)) * 16) + (lane & 1) * 8;
  const char* pb = tile + rb * (2 * D) + ((c ^ swz<D>(rb)) * 16) + (lane & 1) * 8;
  return lds_tr_pair_issue2(pa, pb);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// The 16 accumulator values of a 32x32 block as two 16-deep bf16 B operands
// (K index order matching lds_tr: 4*lg + 0..3, then 8 + 4*lg + 0..3).
__device__ __forceinline__ void pack_b(const f32x16& S, bf16x8 (&P)[2]) {
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f32x2 two = {S[ks * 8 + 2 * j], S[ks * 8 + 2 * j + 1]};
      bf16x2 pk = __builtin_convertvector(two, bf16x2);
      P[ks][2 * j] = pk[0];
      P[ks][2 * j + 1] = pk[1];
    }
}

// Weights and score gradients of one 32x32 block in place: S (raw q.k, masked
// entries -inf after capping) becomes dS = P (dP - D) (1 - t^2), and P is
// returned in Pout. lse2 / dl per element (log2 units / D of the element's row).
template <bool CAP>
__device__ __forceinline__ void weights_and_grads(f32x16& S, const f32x16& dP, f32x16& Pout, const float (&lse2)[16],
                                                  const float (&dl)[16], const AttnParams& p) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float pw, g = 1.0f;
    if constexpr (CAP) {
      pw = fast_exp2(S[i] - lse2[i]);
      const float t = fmaxf(S[i], -p.cap_log2) * (1.0f / p.cap_log2);
      g = __builtin_fmaf(-t, t, 1.0f);
    } else {
      pw = fast_exp2(__builtin_fmaf(S[i], p.scale_log2, -lse2[i]));
    }
    Pout[i] = pw;
    S[i] = pw * (dP[i] - dl[i]) * g;
  }
}

// ------------------------------------------------------------------------------ dq
// One workgroup per (batch, head, q tile). A chunk call (n_chunks <= 1) walks one chunk's tiles
// and writes or adds float32 dq. A ring (n_chunks > 1) visits every chunk in ring order with dQ
// held in registers across the visits (dq is the sum of the chunks' terms), and writes the
// result once, in bf16, to dq_out.
template <int D, bool CAP, bool BITS>
__global__ __launch_bounds__(kThreads, 2) void attn_bwd_dq(BwdParams bp) {
  const AttnParams& p = bp.a;
  using Gm = Geo<D>;
  constexpr int NDS = Gm::NDS, NDB = Gm::NDB, kTileElems = Gm::kTileElems;
  constexpr int BK = kBlockKV;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * 2 * kTileElems];   // [stage][K, V]

  int b, h, qb;
  if (!decode_work(p, b, h, qb)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, lg = lane >> 5;
  const int G = p.H / p.Hkv;
  const int g = h / G;
  const int q_row = qb * kBlockQ + w * 32 + ln;
  const bool q_ok = q_row < p.Sq;
  const bool ring = p.n_chunks > 1;
  const int64_t mrow = (int64_t)b * p.nQb + qb;
  if (!ring && p.row_cnt[mrow] == 0 && bp.dq_mode == 1) return;   // adds nothing

  // q and dout rows as B operands: lane holds row q_row, dims ds*16 + lg*8 .. +7
  bf16x8 qf[NDS], dof[NDS];
  {
    const int64_t rq = (q_ok ? q_row : 0) * (int64_t)p.H + h;
    const __bf16* qrow = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.q_stride_b + rq * D;
    const __bf16* drow = reinterpret_cast<const __bf16*>(bp.dout) + ((int64_t)b * p.Sq * p.H + rq) * D;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(qrow + ds * 16 + lg * 8);
      const bf16x8 c = *reinterpret_cast<const bf16x8*>(drow + ds * 16 + lg * 8);
      qf[ds] = q_ok ? a : bf16x8{};
      dof[ds] = q_ok ? c : bf16x8{};
    }
  }
  const int qrow_c = q_ok ? q_row : p.Sq - 1;
  const int qpos = p.q_pos ? p.q_pos[(int64_t)b * p.qm_stride_b + qrow_c] : p.q_pos_base + q_row;
  const int qseg = p.q_seg ? p.q_seg[(int64_t)b * p.qm_stride_b + qrow_c] : 0;
  float lse2 = __builtin_inff(), dl = 0.0f;
  if (q_ok) {
    const int64_t li = ((int64_t)b * p.H + h) * p.Sq + q_row;
    const float l = p.lse[li];
    if (l != neg_inf()) {
      lse2 = l * kLog2e;
      dl = bp.delta[li];
    }
  }
  float lse2v[16], dlv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    lse2v[i] = lse2;
    dlv[i] = dl;
  }

  f32x16 dQ[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dQ[db] = f32x16{};

  const int64_t krs = (int64_t)p.Hkv * D;
  const uint32_t row_bytes = (uint32_t)krs * 2;
  uint32_t off[16 / Gm::kSlabRows];
  dma_offsets<D>(off, w, lane, row_bytes);
  if (p.Skv % BK) {
    // a ragged last tile leaves rows unwritten: start from zeros (finite, masked)
    for (int i = tid; i < 2 * 2 * kTileElems / 8; i += kThreads)
      reinterpret_cast<uint4*>(smem)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
  }

  const int n_vis = ring ? p.n_chunks : 1;
  for (int t = 0; t < n_vis; ++t) {
    AttnParams pc = p;   // this visit's chunk
    if (ring) ring_chunk_view(pc, p, t);
    const int cnt = pc.row_cnt[mrow];
    if (cnt == 0) continue;
    const auto cols = as_const_space(pc.col_idx + mrow * p.nKb);
    const auto cls = as_const_space(pc.tile_class + mrow * p.nKb);
    const __bf16* kbase = reinterpret_cast<const __bf16*>(pc.k) + (int64_t)b * p.kv_stride_b + g * D;
    const __bf16* vbase = reinterpret_cast<const __bf16*>(pc.v) + (int64_t)b * p.kv_stride_b + g * D;
    auto dma = [&](int kb, int buf) {
      const int k0 = kb * BK;
      const uint32_t bytes = (uint32_t)min(p.Skv - k0, BK) * row_bytes;
      __bf16* Ks = smem + buf * 2 * kTileElems;
      dma_tile(tile_rsrc(kbase + (int64_t)k0 * krs, bytes), Ks, off, w, D);
      dma_tile(tile_rsrc(vbase + (int64_t)k0 * krs, bytes), Ks + kTileElems, off, w, D);
    };
    auto needs_mask = [&](int kb) {
      const int c = cls[kb];
      if constexpr (BITS)
        if (c == 1) return 2;
      return (c != 2 || (kb + 1) * BK > p.Skv) ? 1 : 0;
    };
    int kb_cur = cols[0];
    int kb_nxt = cnt > 1 ? cols[1] : kb_cur;
    int mk_cur = needs_mask(kb_cur);
    // every wave is done with both stages (the previous visit's last step ended in a barrier)
    dma(kb_cur, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int it = 0; it < cnt; ++it) {
      const int kb = kb_cur;
      const int need_mask = mk_cur;
      const int buf = it & 1;
      if (it + 1 < cnt) dma(kb_nxt, buf ^ 1);
      const char* Kt = reinterpret_cast<const char*>(smem + buf * 2 * kTileElems);
      const char* Vt = Kt + kTileElems * 2;

      // S^T = K Q^T and dP^T = V dO^T: A = key rows of K / V, B = q / dout in registers
      f32x16 S[2], dP[2];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        S[kb2] = f32x16{};
        dP[kb2] = f32x16{};
      }
      // in phases of 8 operands each (NDS / 4 per product), so that few operands are live at once
      constexpr int kPh = NDS / 4;
#pragma unroll
      for (int ph = 0; ph < 2 * kPh; ++ph) {
        const char* T = (ph < kPh) ? Kt : Vt;
        bf16x8 a[4][2];
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2) a[d4][kb2] = lds_row<D>(T, kb2 * 32 + ln, 2 * ((ph % kPh) * 4 + d4) + lg);
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4)
#pragma unroll
          for (int kb2 = 0; kb2 < 2; ++kb2) {
            const int ds = (ph % kPh) * 4 + d4;
            if (ph < kPh) S[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[d4][kb2], qf[ds], S[kb2], 0, 0, 0);
            else dP[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[d4][kb2], dof[ds], dP[kb2], 0, 0, 0);
          }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (CAP) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int i = 0; i < 16; ++i) S[kb2][i] = capped_log2(S[kb2][i], p.cap_k2, p.cap_log2);
      }
      if (BITS && need_mask == 2)
        apply_bits(S, pc.mask_bits + ((mrow * p.nKb + kb) * kBlockQ + w * 32 + ln) * 2, lg);
      else if (need_mask)
        apply_mask(S, pc, b, kb * BK, lg, qpos, qseg);
      bf16x8 DS[4];
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        f32x16 Pw;
        weights_and_grads<CAP>(S[kb2], dP[kb2], Pw, lse2v, dlv, p);
        bf16x8 two[2];
        pack_b(S[kb2], two);
        DS[2 * kb2] = two[0];
        DS[2 * kb2 + 1] = two[1];
      }
      // dQ^T += K^T dS^T: A = K read transposed (lane = dim), B = dS^T (lane = query);
      // 4 * NDB products in batches of 8
      constexpr int kKsPer = 8 / NDB;
#pragma unroll
      for (int half = 0; half < 4 / kKsPer; ++half) {
        TrPair kt8[8];
#pragma unroll
        for (int f = 0; f < 8; ++f) kt8[f] = lds_tr<D>(Kt, (half * kKsPer + f / NDB) * 16, f % NDB, lane);
        lds_settle(kt8);
#pragma unroll
        for (int f = 0; f < 8; ++f) {
          const int ks = half * kKsPer + f / NDB, db = f % NDB;
          dQ[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_join(kt8[f]), DS[ks], dQ[db], 0, 0, 0);
        }
      }

      const int kb_nn = cols[min(it + 2, cnt - 1)];
      const int mk_nxt = needs_mask(kb_nxt);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      kb_cur = kb_nxt;
      kb_nxt = kb_nn;
      mk_cur = mk_nxt;
    }
  }

  if (!q_ok) return;
  const float sc = p.scale_log2 * kLn2;   // the score scale
  const int64_t o = (((int64_t)b * p.Sq + q_row) * p.H + h) * D;
  if (ring) {
    __bf16* dq = reinterpret_cast<__bf16*>(bp.dq_out) + o;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int col = db * 32 + 8 * i4 + 4 * lg;
        f32x2 lo = {dQ[db][4 * i4] * sc, dQ[db][4 * i4 + 1] * sc};
        f32x2 hi = {dQ[db][4 * i4 + 2] * sc, dQ[db][4 * i4 + 3] * sc};
        const bf16x2 a = __builtin_convertvector(lo, bf16x2), c = __builtin_convertvector(hi, bf16x2);
        *reinterpret_cast<uint2*>(dq + col) =
            make_uint2(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, c));
      }
    return;
  }
  float* dq = bp.dq + o;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int col = db * 32 + 8 * i4 + 4 * lg;
      float4 v = make_float4(dQ[db][4 * i4] * sc, dQ[db][4 * i4 + 1] * sc, dQ[db][4 * i4 + 2] * sc,
                             dQ[db][4 * i4 + 3] * sc);
      float4* ptr = reinterpret_cast<float4*>(dq + col);
      if (bp.dq_mode == 1) {
        const float4 a = *ptr;
        v.x += a.x;
        v.y += a.y;
        v.z += a.z;
        v.w += a.w;
      }
      *ptr = v;
    }
}

// ------------------------------------------------------------------------------ dk, dv
// Work decode: item order (batch * Hkv + kv head, kv tile ascending); XCD x =
// id % 8 takes the contiguous item range [x*per, (x+1)*per).
__device__ __forceinline__ bool decode_kv_work(const AttnParams& p, int S, int& b, int& g, int& kb, int& s) {
  const int64_t T = (int64_t)p.B * p.Hkv * p.nKb * S;
  const int64_t id = blockIdx.x;
  // as decode_work: whole (batch, kv head) groups per XCD when they divide evenly, else round
  // robin (causal kv tiles differ in work)
  int64_t item = id;
  if (((int64_t)p.B * p.Hkv) % 8 == 0) item = (id & 7) * (T / 8) + (id >> 3);
  if (item >= T) return false;
  s = (int)(item % S);
  kb = (int)((item / S) % p.nKb);
  const int64_t bg = item / S / p.nKb;
  g = (int)(bg % p.Hkv);
  b = (int)(bg / p.Hkv);
  return true;
}

// Element mask of a 32-query x 32-key block with the key per lane and
// sequential positions: query of register i is row q0 + 8*(i>>2) + 4*lg + (i&3)
// of the step (rows of the step at qrow0 in the sequence).
__device__ __forceinline__ void mask_kv_seq(f32x16& S, const AttnParams& p, int key, int qrow0, int q0, int lg) {
  {
    // sequential positions: a query row r keeps the key iff r >= key + kv_base - q_base
    const int64_t t64 = (int64_t)key + p.kv_pos_base - p.q_pos_base - (qrow0 + q0 + 4 * lg);
    int thr = key < p.Skv ? (p.causal ? (int)max<int64_t>(-64, min<int64_t>(64, t64)) : -64) : 64;
    asm volatile("" : "+v"(thr));
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (8 * (i >> 2) + (i & 3) < thr) S[i] = neg_inf();
  }
}

// Eight waves in two roles, two waves per SIMD. For key block kbw (32 keys)
// and query half qh (32 rows of the 64-row step):
//   P wave  (waves 0-3), step t: S = Q K^T, mask, P = exp2(S' - lse), hands
//                                G = P (1 - t^2) (G = P without a cap) to its
//                                partner, then dV^T += dO^T P
//   dS wave (waves 4-7), step t: dS = G (dP - D) and dK^T += Q^T dS of step
//                                t-1, then dP = dO V^T of step t (kept in
//                                registers for the next step)
// Each wave runs 16 products per step and holds one accumulator (64
// registers) and one of K / V (32), so two waves fit a SIMD and each hides
// the other's latency. The dS waves use the hand-off one step after it is
// written (bf16, 32 bytes per lane, double-buffered in LDS), so it needs no
// barrier of its own: one barrier per step. The step data (Q, dO tiles and the rows' lse, D,
// positions, segments) comes through a 4-stage LDS-DMA ring filled two steps
// ahead (the dS waves still read the previous stage), 5 loads per wave and
// step (3 at D = 64), with one fixed vmcnt wait per step. Every LDS access in the loop is
// issued from assembly (see lds_tr_pair_issue), and the loop's barrier is a
// bare s_barrier for the same reason.
constexpr int kDkvWaves = 8;
constexpr int kDkvThreads = 64 * kDkvWaves;
constexpr int kStages = 4;
// s_waitcnt immediate: vmcnt <= n, expcnt and lgkmcnt not waited on (gfx9 encoding).
constexpr int vmcnt_wait(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

__device__ __forceinline__ void lds_settle_v(bf16x8 (&t)[8]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]), "+v"(t[6]), "+v"(t[7]));
}
__device__ __forceinline__ void lds_settle(TrPair (&t)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(t[0].lo), "+v"(t[0].hi), "+v"(t[1].lo), "+v"(t[1].hi), "+v"(t[2].lo), "+v"(t[2].hi),
                 "+v"(t[3].lo), "+v"(t[3].hi));
}
__device__ __forceinline__ void lds_settle_v(bf16x8 (&t)[4]) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]));
}
// Hand-off of 16 bf16 values per lane: two 16-byte halves, 1 KB apart.
__device__ __forceinline__ void lds_put32(char* a, const bf16x8& lo, const bf16x8& hi) {
  asm volatile("ds_write_b128 %0, %1\n\tds_write_b128 %0, %2 offset:1024" : : "v"(lds_addr(a)), "v"(lo), "v"(hi));
}
// Reads issued without a wait; the values must pass lds_tie() after a later wait.
__device__ __forceinline__ void lds_rows4_issue(const char* a, f32x4 (&x)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:32\n\t"
      "ds_read_b128 %2, %4 offset:64\n\t"
      "ds_read_b128 %3, %4 offset:96"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
      : "v"(lds_addr(a)));
}
__device__ __forceinline__ void lds_get32_issue(const char* a, bf16x8& lo, bf16x8& hi) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:1024" : "=&v"(lo), "=&v"(hi) : "v"(lds_addr(a)));
}
// Ties values read without a wait to the point after an `s_waitcnt lgkmcnt(0)` issued before it.
__device__ __forceinline__ void lds_tie(f32x4 (&x)[4]) { asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3])); }
__device__ __forceinline__ void lds_tie(bf16x8& lo, bf16x8& hi) { asm volatile("" : "+v"(lo), "+v"(hi)); }
// Two 16-byte reads (a and b) and their wait.
__device__ __forceinline__ void lds_pair4(const char* a, const char* b, f32x4& x, f32x4& y) {
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
               : "=&v"(x), "=&v"(y)
               : "v"(lds_addr(a)), "v"(lds_addr(b)));
}

template <int D, bool CAP, bool BITS>
__global__ __launch_bounds__(kDkvThreads, 1) void attn_bwd_dkv(BwdParams bp) {
  const AttnParams& p = bp.a;
  using Gm = Geo<D>;
  constexpr int NDS = Gm::NDS, NDB = Gm::NDB, kTileElems = Gm::kTileElems;
  constexpr int kSlabs = 8 / Gm::kSlabRows;        // DMA slabs per wave and tile (8 rows)
  constexpr int kDmaPerStep = 2 * kSlabs + 1;      // Q, dO slabs and one row array
  // [stage][Q, dO] tiles, then [stage][8][64] row floats (lse, D, pos, seg, 4 unused),
  // then the hand-off: [step parity][kbw*2 + qh][half][64 lanes][16 bytes]
  constexpr int kRowsBytes = kStages * 8 * 64 * 4;
  constexpr int kXBytes = 2 * 4 * 2 * 64 * 16;
  __shared__ __attribute__((aligned(16))) __bf16 smem[kStages * 2 * kTileElems + (kRowsBytes + kXBytes) / 2];
  char* const rows_lds = reinterpret_cast<char*>(smem + kStages * 2 * kTileElems);
  char* const xch = rows_lds + kRowsBytes;
  auto row_at = [&](int buf, int arr, int r) { return rows_lds + ((buf * 8 + arr) * 64 + r) * 4; };

  int b, g, kb, hs;
  const int S = bp.head_split;
  if (!decode_kv_work(p, S, b, g, kb, hs)) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, lg = lane >> 5;
  const bool pw = w < 4;                     // P wave (else dS wave)
  const int kbw = w & 1, qh = (w >> 1) & 1;  // key block and query half
  const int G = p.H / p.Hkv / S;   // heads of the group this workgroup walks
  const int h0 = g * (p.H / p.Hkv) + hs * G;   // the first of them
  const int key = kb * kBlockKV + 32 * kbw + ln;
  const bool key_ok = key < p.Skv;
  char* const my_x = xch + (kbw * 2 + qh) * 2 * 1024 + lane * 16;   // parity 0; parity 1 at + 8 KB

  // K (P waves) or V (dS waves) rows as B operands: lane holds key `key`, dims ds*16 + lg*8 .. +7
  bf16x8 kv[NDS];
  {
    const int64_t ro = (int64_t)b * p.kv_stride_b + ((int64_t)(key_ok ? key : 0) * p.Hkv + g) * D;
    const __bf16* row = reinterpret_cast<const __bf16*>(pw ? p.k : p.v) + ro;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(row + ds * 16 + lg * 8);
      kv[ds] = key_ok ? a : bf16x8{};
    }
  }
  const int key_c = key_ok ? key : 0;
  const int kpos = p.kv_pos ? p.kv_pos[(int64_t)b * p.kvm_stride_b + key_c] : p.kv_pos_base + key;
  const int kseg = p.kv_seg ? p.kv_seg[(int64_t)b * p.kvm_stride_b + key_c] : 0;

  f32x16 acc[NDB];   // dV^T (P waves) or dK^T (dS waves): [dim][key]
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  const int64_t kcol = (int64_t)b * p.nKb + kb;
  const int ccnt = bp.col_cnt[kcol];
  const auto rows = as_const_space(bp.row_idx + kcol * p.nQb);
  const int n_steps = ccnt * 2 * G;          // (q tile, 64-row half, head in group)
  auto tile_class_of = [&](int qb) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p.tile_class + ((int64_t)b * p.nQb + qb) * p.nKb + kb);
    const uint32_t word = *as_const_space(reinterpret_cast<const uint32_t*>(a & ~uintptr_t(3)));
    return (int)((word >> (8 * (a & 3))) & 0xffu);
  };

  const uint32_t row_bytes = (uint32_t)p.H * D * 2;
  // DMA: wave w fills rows [8w, 8w + 8) of the Q and dO tiles (kSlabs slabs each)
  uint32_t off[kSlabs];
#pragma unroll
  for (int i = 0; i < kSlabs; ++i) {
    const int r = 8 * w + Gm::kSlabRows * i + lane / Gm::kChunks;
    off[i] = (uint32_t)r * row_bytes + ((lane % Gm::kChunks) ^ swz<D>(r)) * 16;
  }
  // Step t covers q tile rows[t / 2G], 64-row half (t / G) & 1 and head g*G + t % G. Both
  // the DMA stage and the work step advance one step at a time, so each keeps a cursor
  // (tile index, half, head in group) instead of dividing by G every step.
  struct Cursor {
    int qi, half, hi;
  };
  auto advance = [&](Cursor& c) {
    if (++c.hi == G) {
      c.hi = 0;
      c.half ^= 1;
      c.qi += c.half == 0;
    }
  };
  // The row array this wave moves: waves 0-3 the base-2 lse and D (both written by the
  // prep kernel), positions, segments (empty when absent); waves 4-7 an empty load into
  // an unused array, so every wave issues the same count.
  const float* row_src =
      w == 0 ? bp.delta + (int64_t)p.B * p.H * p.Sq : (w == 1 ? bp.delta : (w == 2 ? reinterpret_cast<const float*>(p.q_pos)
                                                   : (w == 3 ? reinterpret_cast<const float*>(p.q_seg) : nullptr)));
  const bool row_per_head = w < 2;
  // Staging: bases at head g*G of this workgroup's batch; the values that change only with
  // the staged q tile or half (first row, byte counts, row offset) are recomputed only then,
  // and a step adds its head's stride (steps past the last stage empty loads).
  const __bf16* q_wg = reinterpret_cast<const __bf16*>(p.q) + (int64_t)b * p.q_stride_b + (int64_t)h0 * D;
  const __bf16* o_wg = reinterpret_cast<const __bf16*>(bp.dout) + ((int64_t)b * p.Sq * p.H + h0) * D;
  const float* r_wg =
      row_src ? row_src + (row_per_head ? ((int64_t)b * p.H + h0) * p.Sq : (int64_t)b * p.qm_stride_b) : p.lse;
  const int r_step = row_per_head ? p.Sq : 0;   // row-array elements per head
  Cursor stc{0, 0, 0};                          // the next step to stage
  int64_t st_off = 0;                           // elements to its first row at head g*G
  int st_r0 = 0;
  uint32_t st_bytes = 0, st_rbytes = 0;
  auto stage_rows = [&]() {
    const int r0 = stc.qi < ccnt ? rows[stc.qi] * kBlockQ + stc.half * 64 : p.Sq;
    const int nrows = max(0, min(64, p.Sq - r0));
    st_r0 = min(r0, p.Sq);
    st_off = (int64_t)st_r0 * p.H * D;
    st_bytes = nrows > 0 ? (uint32_t)(nrows - 1) * row_bytes + D * 2 : 0u;
    st_rbytes = row_src ? (uint32_t)nrows * 4u : 0u;
  };
  stage_rows();
  auto stage = [&](int buf) {
    const int64_t eoff = st_off + (int64_t)stc.hi * D;
    __bf16* Qs = smem + buf * 2 * kTileElems;
    const auto qr = tile_rsrc(q_wg + eoff, st_bytes);
    const auto orr = tile_rsrc(o_wg + eoff, st_bytes);
#pragma unroll
    for (int i = 0; i < kSlabs; ++i) {
      const int r = 8 * w + Gm::kSlabRows * i;
      dma16(qr, Qs + r * D, off[i]);
      dma16(orr, Qs + kTileElems + r * D, off[i]);
    }
    const float* rs = row_src ? r_wg + stc.hi * r_step + st_r0 : p.lse;
    dma4(tile_rsrc(rs, st_rbytes), row_at(buf, w, 0), (uint32_t)lane * 4u);
    if (++stc.hi == G) {
      stc.hi = 0;
      stc.half ^= 1;
      stc.qi += stc.half == 0;
      stage_rows();
    }
  };

  constexpr int kAhead = 2;   // stages in flight beyond the next one
  stage(0);
  stage(1);
  __builtin_amdgcn_s_waitcnt(vmcnt_wait(kDmaPerStep * (kAhead - 1)));
  __syncthreads();

  const int q0 = 32 * qh;                    // this wave's first row in a step
  Cursor wc{0, 0, 0};                        // the step this wave works on next
  // The P waves' q tile of that step and its mask kind (0 none, 1 positions / segments,
  // 2 stored bits), looked up when the cursor enters a q tile (every 2G steps).
  auto tile_mask_kind = [&](int qb) {
    const int cl = tile_class_of(qb);
    return (BITS && cl == 1) ? 2 : ((cl != 2 || (kb + 1) * kBlockKV > p.Skv) ? 1 : 0);
  };
  int w_qb = 0, w_mask = 0;
  if (pw && ccnt > 0) {
    w_qb = rows[0];
    w_mask = tile_mask_kind(w_qb);
  }
  // The dS waves run half a step behind the P waves: in step t a dS wave first finishes
  // step t-1 (dS from the dP it computed at the end of step t-1 and the partner's G, then
  // dK^T += Q^T dS) and then computes dP of step t, which it keeps in registers. Its
  // products thus fall in the P wave's softmax phase, and its VALU work in the P wave's
  // wait for its first operands. Step t reads buffers t (P waves, and dO for the dS
  // waves' dP) and t-1 (the dS waves' Q^T, D and G); the stage writes buffer t+2.
  // The two roles run separate loops (the same number of barriers), so that neither
  // role's registers count against the other's.
  // Step t+1 has landed once at most the loads of step t+2 are outstanding (every LDS
  // access of a step has been waited for before its barrier).
  auto step_end = [&]() {
    __builtin_amdgcn_s_waitcnt(vmcnt_wait(kDmaPerStep * (kAhead - 1)));
    __builtin_amdgcn_s_barrier();
  };
  if (pw) {
    for (int t = 0; t <= n_steps; ++t) {
      const int buf = t & (kStages - 1);
      const char* Qt = reinterpret_cast<const char*>(smem + buf * 2 * kTileElems);
      const char* Ot = Qt + kTileElems * 2;
      if (t == n_steps) {
        stage((t + kAhead) & (kStages - 1));
      } else {
        char* const x_t = my_x + (t & 1) * 8192;
        // the first product's A operands (Q rows) and the rows' base-2 lse, one wait for both
        f32x4 rv[4];
        lds_rows4_issue(row_at(buf, 0, q0 + 4 * lg), rv);
        f32x16 X = f32x16{};
        {
          bf16x8 a[NDS];
#pragma unroll
          for (int ds = 0; ds < NDS; ++ds) {
            const int r = q0 + ln, c = 2 * ds + lg;
            a[ds] = lds_b128_issue(Qt + r * (2 * D) + ((c ^ swz<D>(r)) * 16));
          }
          // the stage's loads issue while these reads are served
          stage((t + kAhead) & (kStages - 1));
          lds_settle_v(a);
          lds_tie(rv);
#pragma unroll
          for (int ds = 0; ds < NDS; ++ds) X = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ds], kv[ds], X, 0, 0, 0);
        }
        // dO^T operands of dV load while the weights are computed
        TrPair tr[2 * NDB];
#pragma unroll
        for (int f = 0; f < 2 * NDB; ++f) tr[f] = lds_tr<D>(Ot, q0 + (f / NDB) * 16, f % NDB, lane);
        const int qb = w_qb;
        const int r0 = qb * kBlockQ + wc.half * 64;
        const int need_mask = w_mask;
        if constexpr (CAP) {
#pragma unroll
          for (int i = 0; i < 16; ++i) X[i] = capped_log2(X[i], p.cap_k2, p.cap_log2);
        }
        if (BITS && need_mask == 2) {
          // bits of the tile: row (step half * 64 + q0 + r), word kbw, bit ln
          const uint32_t* tb = p.mask_bits + (((int64_t)b * p.nQb + qb) * p.nKb + kb) * kBlockQ * 2 +
                               (int64_t)((r0 - qb * kBlockQ) + q0 + 4 * lg) * 2 + kbw;
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (((tb[(8 * (i >> 2) + (i & 3)) * 2] >> ln) & 1u) == 0u) X[i] = neg_inf();
        } else if (need_mask) {
          if (!p.q_pos && !p.kv_pos && !p.q_seg) {
            mask_kv_seq(X, p, key, r0, q0, lg);
          } else {
            // explicit positions / segments: the rows' values four at a time
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              f32x4 qpv, qsv;
              lds_pair4(row_at(buf, 2, q0 + 8 * j + 4 * lg), row_at(buf, 3, q0 + 8 * j + 4 * lg), qpv, qsv);
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = q0 + 8 * j + 4 * lg + e;
                bool ok = key < p.Skv;
                if (p.causal) ok = ok && kpos <= (p.q_pos ? __float_as_int(qpv[e]) : p.q_pos_base + r0 + r);
                if (p.q_seg) ok = ok && __float_as_int(qsv[e]) == kseg && kseg != -1;
                if (!ok) X[4 * j + e] = neg_inf();
              }
            }
          }
        }
        // P in place of S; G = P (1 - t^2) goes to the partner (G = P without a cap)
        f32x16 Gw;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float l2 = rv[i >> 2][i & 3];   // lse * log2(e), +inf for a row with no allowed key
          if constexpr (CAP) {
            const float tt = fmaxf(X[i], -p.cap_log2) * (1.0f / p.cap_log2);
            X[i] = fast_exp2(X[i] - l2);
            Gw[i] = X[i] * __builtin_fmaf(-tt, tt, 1.0f);
          } else {
            X[i] = fast_exp2(__builtin_fmaf(X[i], p.scale_log2, -l2));
          }
        }
        bf16x8 Pb[2];
        pack_b(X, Pb);
        if constexpr (CAP) {
          bf16x8 Gb[2];
          pack_b(Gw, Gb);
          lds_put32(x_t, Gb[0], Gb[1]);
        } else {
          lds_put32(x_t, Pb[0], Pb[1]);
        }
        // dV^T += dO^T P
        lds_settle(tr);
#pragma unroll
        for (int f = 0; f < 2 * NDB; ++f)
          acc[f % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_join(tr[f]), Pb[f / NDB], acc[f % NDB], 0, 0, 0);
        advance(wc);
        if (wc.hi == 0 && wc.half == 0 && wc.qi < ccnt) {
          w_qb = rows[wc.qi];
          w_mask = tile_mask_kind(w_qb);
        }
      }
      step_end();
    }
  } else {
    f32x16 dp_keep = f32x16{};   // dP of the step the wave finishes next
    for (int t = 0; t <= n_steps; ++t) {
      const char* Ot = reinterpret_cast<const char*>(smem + (t & (kStages - 1)) * 2 * kTileElems) + kTileElems * 2;
      if (t > 0) {
        // finish step t-1: dS = G (dP - D), dK^T += Q^T dS
        const int pb = (t - 1) & (kStages - 1);
        const char* Qp = reinterpret_cast<const char*>(smem + pb * 2 * kTileElems);
        char* const x_p = my_x + ((t - 1) & 1) * 8192;
        TrPair tr[2 * NDB];
#pragma unroll
        for (int f = 0; f < 2 * NDB; ++f) tr[f] = lds_tr<D>(Qp, q0 + (f / NDB) * 16, f % NDB, lane);
        bf16x8 gb[2];
        f32x4 rv[4];   // D of rows q0 + 8j + 4*lg + 0..3
        lds_get32_issue(x_p, gb[0], gb[1]);
        lds_rows4_issue(row_at(pb, 1, q0 + 4 * lg), rv);
        if (t == n_steps) stage((t + kAhead) & (kStages - 1));
        lds_settle(tr);
        lds_tie(rv);
        lds_tie(gb[0], gb[1]);
        f32x16 dS;
#pragma unroll
        for (int i = 0; i < 16; ++i) dS[i] = (float)gb[i >> 3][i & 7] * (dp_keep[i] - rv[i >> 2][i & 3]);
        bf16x8 DSb[2];
        pack_b(dS, DSb);
#pragma unroll
        for (int f = 0; f < 2 * NDB; ++f)
          acc[f % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_join(tr[f]), DSb[f / NDB], acc[f % NDB], 0, 0, 0);
      }
      if (t < n_steps) {
        // dP of step t = dO V^T
        bf16x8 a[NDS];
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
          const int r = q0 + ln, c = 2 * ds + lg;
          a[ds] = lds_b128_issue(Ot + r * (2 * D) + ((c ^ swz<D>(r)) * 16));
        }
        stage((t + kAhead) & (kStages - 1));
        lds_settle_v(a);
        f32x16 X = f32x16{};
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) X = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ds], kv[ds], X, 0, 0, 0);
        dp_keep = X;
      }
      step_end();
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // the empty loads of the last stages
  __syncthreads();

  // The two query halves of each (role, key block): qh = 1 hands its sum to qh = 0.
  float* red = reinterpret_cast<float*>(smem);   // [role][key block][NDB][16][64 lanes]
  const int slot = (pw ? 0 : 2) + kbw;
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) red[((slot * NDB + db) * 16 + i) * 64 + lane] = acc[db][i];
  }
  __syncthreads();
  if (qh == 1 || !key_ok) return;
  const float sc = pw ? 1.0f : p.scale_log2 * kLn2;   // dk carries the score scale
  float* dst = (pw ? bp.dv : bp.dk) + hs * bp.part_stride + (int64_t)b * bp.dkv_stride_b + ((int64_t)key * p.Hkv + g) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int col = db * 32 + 8 * i4 + 4 * lg;
      float a[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * i4 + e;
        a[e] = (acc[db][i] + red[((slot * NDB + db) * 16 + i) * 64 + lane]) * sc;
      }
      *reinterpret_cast<float4*>(dst + col) = make_float4(a[0], a[1], a[2], a[3]);
    }
}

// ------------------------------------------------------------------------------ helpers
// delta[b,h,i] = dout[b,i,h,:] . out[b,i,h,:]; 16 lanes per (row, head), 8 elements each.
template <typename T>
__global__ __launch_bounds__(256) void bwd_delta_kernel(int64_t n_rows, int H, int Sq, int Dd, const T* out,
                                                        const T* dout, const float* lse, float* delta) {
  const int64_t pair = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int part = threadIdx.x & 15;
  float acc = 0.0f;
  if (pair < n_rows) {
    const T* o = out + pair * Dd;
    const T* d = dout + pair * Dd;
    for (int e = part * 8; e < Dd; e += 128)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += (float)o[e + j] * (float)d[e + j];
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 16);
  if (pair < n_rows && part == 0) {
    // pair = (b*Sq + i)*H + h  ->  [b, h, i]
    const int h = (int)(pair % H);
    const int64_t bi = pair / H;
    const int i = (int)(bi % Sq);
    const int64_t bb = bi / Sq;
    const int64_t at = (bb * H + h) * Sq + i;
    delta[at] = acc;
    // the row's logsumexp in base 2; +inf for a row with no allowed key, whose weights
    // exp2(s * scale * log2(e) - that) are then exactly 0
    const float l = lse[at];
    delta[n_rows + at] = l == -__builtin_inff() ? __builtin_inff() : l * kLog2e;
  }
}

// dst[b * dst_stride + i] = sum over s of src[s * part_stride + b * n + i], four floats per thread.
__global__ __launch_bounds__(256) void sum_parts_kernel(const float* src, int S, int64_t part_stride, int64_t n4,
                                                        float* dst, int64_t dst_stride) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int b = blockIdx.y;
  if (i >= n4) return;
  const float4* sp = reinterpret_cast<const float4*>(src + (int64_t)b * n4 * 4) + i;
  float4 a = sp[0];
  for (int s = 1; s < S; ++s) {
    const float4 c = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(sp) + s * part_stride);
    a.x += c.x;
    a.y += c.y;
    a.z += c.z;
    a.w += c.w;
  }
  reinterpret_cast<float4*>(dst + (int64_t)b * dst_stride)[i] = a;
}

// dsinks[h] = -sum over (b, i) of exp(sink_h - lse[b,h,i]) * delta[b,h,i] (rows
// with lse = -inf have no weight); one workgroup per head, a fixed-order tree.
__global__ __launch_bounds__(256) void bwd_dsinks_kernel(int B, int H, int Sq, const float* sinks, const float* lse,
                                                         const float* delta, float* dsinks) {
  __shared__ float red[256];
  const int h = blockIdx.x;
  const float s = sinks[h];
  float acc = 0.0f;
  for (int b = 0; b < B; ++b) {
    const int64_t base = ((int64_t)b * H + h) * Sq;
    for (int i = threadIdx.x; i < Sq; i += 256) {
      const float l = lse[base + i];
      if (l != neg_inf()) acc += expf(s - l) * delta[base + i];
    }
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) dsinks[h] = -red[0];
}

// Transposed tile lists: for every kv tile, the q tiles whose class is not
// EMPTY, ascending, then -1. One workgroup per (kv tile, batch, chunk).
__global__ __launch_bounds__(256) void col_lists_kernel(MaskParams p, int32_t* col_cnt, int32_t* row_idx) {
  __shared__ int wsum[4];
  const int kb = blockIdx.x, b = blockIdx.y, c = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t chunk_tiles = (int64_t)p.B * p.nQb * p.nKb;
  const uint8_t* cls = p.tile_class + c * chunk_tiles + (int64_t)b * p.nQb * p.nKb + kb;
  const int64_t col = ((int64_t)c * p.B + b) * p.nKb + kb;
  int32_t* out = row_idx + col * p.nQb;
  int running = 0;
  for (int base = 0; base < p.nQb; base += 256) {
    const int qb = base + tid;
    const bool f = qb < p.nQb && cls[(int64_t)qb * p.nKb] != 0;
    const uint64_t bal = __ballot(f);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[w] = __popcll(bal);
    __syncthreads();
    int o = running, total = 0;
    for (int i = 0; i < 4; ++i) {
      if (i < w) o += wsum[i];
      total += wsum[i];
    }
    if (f) out[o + before] = qb;
    running += total;
    __syncthreads();
  }
  for (int j = running + tid; j < p.nQb; j += 256) out[j] = -1;
  if (tid == 0) col_cnt[col] = running;
}

template <typename K>
hipError_t launch_grid(K kernel, int64_t items, int threads, const BwdParams& p, hipStream_t s) {
  const int64_t grid = 8 * ((items + 7) / 8);
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(threads), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_bwd_dq_d(const BwdParams& p, hipStream_t s) {
  const AttnParams& a = p.a;
  const bool cap = a.softcap_on != 0, bits = a.mask_bits != nullptr;
  const int64_t q_items = (int64_t)a.B * a.H * a.nQb;
  if (q_items == 0) return hipSuccess;
  const int t = kThreads;
  if (cap) return bits ? launch_grid(attn_bwd_dq<D, true, true>, q_items, t, p, s) : launch_grid(attn_bwd_dq<D, true, false>, q_items, t, p, s);
  return bits ? launch_grid(attn_bwd_dq<D, false, true>, q_items, t, p, s) : launch_grid(attn_bwd_dq<D, false, false>, q_items, t, p, s);
}

template <int D>
hipError_t launch_bwd_dkv_d(const BwdParams& p, hipStream_t s) {
  const AttnParams& a = p.a;
  const bool cap = a.softcap_on != 0, bits = a.mask_bits != nullptr;
  const int64_t kv_items = (int64_t)a.B * a.Hkv * a.nKb * p.head_split;
  if (kv_items == 0) return hipSuccess;
  const int t = kDkvThreads;
  if (cap) return bits ? launch_grid(attn_bwd_dkv<D, true, true>, kv_items, t, p, s) : launch_grid(attn_bwd_dkv<D, true, false>, kv_items, t, p, s);
  return bits ? launch_grid(attn_bwd_dkv<D, false, true>, kv_items, t, p, s) : launch_grid(attn_bwd_dkv<D, false, false>, kv_items, t, p, s);
}

}  // namespace

hipError_t launch_attn_bwd_dq(const BwdParams& p, hipStream_t s) {
  return p.a.D == 64 ? launch_bwd_dq_d<64>(p, s) : launch_bwd_dq_d<128>(p, s);
}

hipError_t launch_attn_bwd_dkv(const BwdParams& p, hipStream_t s) {
  return p.a.D == 64 ? launch_bwd_dkv_d<64>(p, s) : launch_bwd_dkv_d<128>(p, s);
}

hipError_t launch_attn_bwd(const BwdParams& p, hipStream_t s) {
  const hipError_t e = launch_attn_bwd_dq(p, s);
  return e != hipSuccess ? e : launch_attn_bwd_dkv(p, s);
}

hipError_t launch_bwd_prep(int dtype, int B, int Sq, int H, int Dd, const void* out, const void* dout,
                           const float* lse, const float* sinks, float* delta, float* dsinks, hipStream_t s) {
  const int64_t n_rows = (int64_t)B * Sq * H;
  if (n_rows > 0) {
    const int64_t grid = (n_rows * 16 + 255) / 256;
    if (dtype == 1)
      hipLaunchKernelGGL(bwd_delta_kernel<__bf16>, dim3((unsigned)grid), dim3(256), 0, s, n_rows, H, Sq, Dd,
                         reinterpret_cast<const __bf16*>(out), reinterpret_cast<const __bf16*>(dout), lse, delta);
    else
      hipLaunchKernelGGL(bwd_delta_kernel<float>, dim3((unsigned)grid), dim3(256), 0, s, n_rows, H, Sq, Dd,
                         reinterpret_cast<const float*>(out), reinterpret_cast<const float*>(dout), lse, delta);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (sinks && H > 0) {
    hipLaunchKernelGGL(bwd_dsinks_kernel, dim3(H), dim3(256), 0, s, B, H, Sq, sinks, lse, delta, dsinks);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_sum_parts(const float* src, int S, int64_t part_stride, int B, int64_t n, float* dst,
                            int64_t dst_stride, hipStream_t s) {
  const int64_t n4 = n / 4;   // n is a multiple of 4 (rows of D floats)
  if (n4 == 0 || B == 0) return hipSuccess;
  hipLaunchKernelGGL(sum_parts_kernel, dim3((unsigned)((n4 + 255) / 256), (unsigned)B), dim3(256), 0, s, src, S,
                     part_stride, n4, dst, dst_stride);
  return hipGetLastError();
}

hipError_t launch_col_lists(const MaskParams& p, int n_chunks, int32_t* col_cnt, int32_t* row_idx, hipStream_t s) {
  if (p.B == 0 || p.nKb == 0 || n_chunks == 0) return hipSuccess;
  hipLaunchKernelGGL(col_lists_kernel, dim3(p.nKb, p.B, n_chunks), dim3(256), 0, s, p, col_cnt, row_idx);
  return hipGetLastError();
}

}  // namespace ram
