// Device helpers shared by the attention kernels (internal).
//
// Layout conventions (v_mfma_f32_32x32x16_bf16, scores computed transposed as
// S^T = K * Q^T): lane l owns query row (l & 31); accumulator register i of a
// 32-key block holds key 8*(i>>2) + 4*(l>>5) + (i&3). Lanes l and l^32 hold
// the same query row.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>

#include "ram_internal.h"

namespace ram {
namespace attn {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleThreshold = 8.0f;  // log2 units
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// The tile lists are read-only for the whole launch: reading them through the
// constant address space lets uniform loads go through the scalar cache.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(4))) T* as_const_space(const T* p) {
  return (const __attribute__((address_space(4))) T*)p;
}

// Work decode: item order is (batch*Hkv + kv head, q tile descending, head in group);
// XCD x = id % 8 takes the contiguous item range [x*per, (x+1)*per).
// With S > 1 each (batch, head, q tile) is S items, *s_out the index among them.
__device__ __forceinline__ bool decode_work(const AttnParams& p, int& b, int& h, int& qb, int S = 1,
                                            int* s_out = nullptr) {
  const int G = p.H / p.Hkv;
  const int64_t T = (int64_t)p.B * p.Hkv * p.nQb * G * S;
  const int64_t id = blockIdx.x;
  // Workgroups go to the 8 XCDs round robin (block id mod 8). With whole (batch, kv head)
  // groups per XCD, a group's K / V stay in one XCD's L2. With fewer groups than that (MQA,
  // small batches) a contiguous share would give one XCD the heaviest causal rows: there
  // the items go round robin too, so that each XCD gets some heads of every q tile.
  int64_t item = id;
  if (p.row_order) {
    // rows most tiles first, every head of a row before the next row, round robin over XCDs
    if (item >= T) return false;
    if (s_out) *s_out = (int)(item % S);
    item /= S;
    h = (int)(item % p.H);
    const int row = p.row_order[item / p.H];
    b = row / p.nQb;
    qb = row - b * p.nQb;
    return true;
  }
  if (((int64_t)p.B * p.Hkv) % 8 == 0) item = (id & 7) * (T / 8) + (id >> 3);
  if (item >= T) return false;
  if (s_out) *s_out = (int)(item % S);
  item /= S;
  const int hg = (int)(item % G);
  const int64_t r = item / G;
  const int qrev = (int)(r % p.nQb);
  const int64_t bg = r / p.nQb;
  const int g = (int)(bg % p.Hkv);
  b = (int)(bg / p.Hkv);
  h = g * G + hg;
  qb = p.nQb - 1 - qrev;
  return true;
}

// Lanes l and l^32 hold the same query row. v_permlane32_swap exchanges the
// upper half of its first operand with the lower half of its second; with x
// passed as both, the two results of each lane are {own value, partner value}
// (in an order that depends on the lane half), so max / sum over the pair is
// the reduction over both lanes.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Element mask for the keys a lane holds of NK 32-key blocks starting at k0.
// Key of accumulator register i of block kb2: k0 + kb2*32 + 8*(i>>2) + 4*lg + (i&3).
template <int NK>
__device__ __forceinline__ void apply_mask(f32x16 (&S)[NK], const AttnParams& p, int b, int k0,
                                           int lg, int qpos, int qseg) {
  if (!p.kv_pos && !p.kv_seg) {
    // positions kv_pos_base + key: exactly the keys below `lim` are kept
    const int64_t reach = (int64_t)qpos - p.kv_pos_base + 1;
    const int lim = p.causal ? (int)max<int64_t>(-1, min<int64_t>(p.Skv, reach)) : p.Skv;
    int thr = lim - (k0 + 4 * lg);
    // keep the per-element compares next to their use (hoisted, they pin one
    // scalar register pair per score across the MFMA block)
    asm volatile("" : "+v"(thr));
#pragma unroll
    for (int kb2 = 0; kb2 < NK; ++kb2)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (kb2 * 32 + 8 * (i >> 2) + (i & 3) >= thr) S[kb2][i] = neg_inf();
    return;
  }
  const int32_t* kvp = p.kv_pos ? p.kv_pos + (int64_t)b * p.kvm_stride_b : nullptr;
  const int32_t* kvs = p.kv_seg ? p.kv_seg + (int64_t)b * p.kvm_stride_b : nullptr;
  int key0 = k0 + 4 * lg;
  asm volatile("" : "+v"(key0));   // as above: no hoisting of the compares
#pragma unroll
  for (int kb2 = 0; kb2 < NK; ++kb2) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key0 + kb2 * 32 + 8 * (i >> 2) + (i & 3);
      bool ok = key < p.Skv;
      if (ok && p.causal) {
        const int kp = kvp ? kvp[key] : p.kv_pos_base + key;
        ok = kp <= qpos;
      }
      if (ok && kvs) ok = (kvs[key] == qseg) && (qseg != -1);
      if (!ok) S[kb2][i] = neg_inf();
    }
  }
}

// Element mask of a PARTIAL tile from its stored bits: `row` holds NK words
// for this lane's query row, key j of the tile at bit j % 32 of word j / 32.
template <int NK>
__device__ __forceinline__ void apply_bits(f32x16 (&S)[NK], const uint32_t* row, int lg) {
  uint32_t wv[NK];
  if constexpr (NK == 2) {
    const uint2 t = *reinterpret_cast<const uint2*>(row);
    wv[0] = t.x;
    wv[1] = t.y;
  } else {
#pragma unroll
    for (int kb2 = 0; kb2 < NK; ++kb2) wv[kb2] = row[kb2];
  }
#pragma unroll
  for (int kb2 = 0; kb2 < NK; ++kb2) {
    const uint32_t x = wv[kb2] >> (4 * lg);   // key 8*(i>>2) + 4*lg + (i&3) of the block
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (((x >> (8 * (i >> 2) + (i & 3))) & 1u) == 0u) S[kb2][i] = neg_inf();
  }
}

// Soft cap in log2 units: u = cap*log2(e) * tanh(s*scale/cap), tanh(x) = 1 - 2/(1+e^{2x}).
__device__ __forceinline__ float capped_log2(float s, float k2, float cap_log2) {
  const float e = fast_exp2(s * k2);
  const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e);
  return cap_log2 * t;
}

// Maximum of N values by a tree of three-input maxima (v_max3_f32).
template <int N>
__device__ __forceinline__ float max_tree3(const float (&v)[N]) {
  if constexpr (N == 1) {
    return v[0];
  } else if constexpr (N == 2) {
    return fmaxf(v[0], v[1]);
  } else {
    constexpr int M = (N + 2) / 3;
    float u[M];
#pragma unroll
    for (int j = 0; j < N / 3; ++j) u[j] = fmaxf(fmaxf(v[3 * j], v[3 * j + 1]), v[3 * j + 2]);
    if constexpr (N % 3 == 1) u[M - 1] = v[N - 1];
    if constexpr (N % 3 == 2) u[M - 1] = fmaxf(v[N - 2], v[N - 1]);
    return max_tree3<M>(u);
  }
}

// Online-softmax step on the NK*16 scores a lane holds. Updates m_ref / l_acc
// / O and leaves the weights in S.
template <int NDB, bool CAP, int NK>
__device__ __forceinline__ void softmax_step(f32x16 (&S)[NK], f32x16 (&O)[NDB], float& m_ref,
                                             float& l_acc, const AttnParams& p) {
  constexpr int NG = NK * 4;
  float t[NG];
  float all[NK * 16];
#pragma unroll
  for (int kb2 = 0; kb2 < NK; ++kb2)
#pragma unroll
    for (int i = 0; i < 16; ++i) all[kb2 * 16 + i] = S[kb2][i];
  const float mx = pair_max(max_tree3(all));
  const float umax = CAP ? mx : mx * p.scale_log2;
  const bool need = umax > m_ref + kRescaleThreshold;
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
    const float m_new = fmaxf(m_ref, umax);
    const float alpha = (m_new == neg_inf()) ? 1.0f : fast_exp2(m_ref - m_new);
    l_acc *= alpha;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[db][i] *= alpha;
    m_ref = m_new;
  }
  const float msub = (m_ref == neg_inf()) ? 0.0f : m_ref;
#pragma unroll
  for (int kb2 = 0; kb2 < NK; ++kb2)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      S[kb2][i] = CAP ? fast_exp2(S[kb2][i] - msub) : fast_exp2(__builtin_fmaf(S[kb2][i], p.scale_log2, -msub));
  // row sum: a tree (short dependency chains), in fp32: the weights' bf16
  // rounding would put up to 2^-9 into the logsumexp of a row with few keys
#pragma unroll
  for (int u = 0; u < NG; ++u)
    t[u] = (S[u >> 2][(u & 3) * 4 + 0] + S[u >> 2][(u & 3) * 4 + 1]) +
           (S[u >> 2][(u & 3) * 4 + 2] + S[u >> 2][(u & 3) * 4 + 3]);
#pragma unroll
  for (int w = NG / 2; w >= 1; w /= 2)
#pragma unroll
    for (int u = 0; u < w; ++u) t[u] += t[u + w];
  l_acc += t[0];
}

// Four consecutive floats of a row as bf16, one 8-byte store.
__device__ __forceinline__ void store_bf16x4(void* base, int64_t idx, float4 v) {
  f32x2 lo = {v.x, v.y}, hi = {v.z, v.w};
  const bf16x2 a = __builtin_convertvector(lo, bf16x2), c = __builtin_convertvector(hi, bf16x2);
  uint2 u;
  u.x = __builtin_bit_cast(uint32_t, a);
  u.y = __builtin_bit_cast(uint32_t, c);
  *reinterpret_cast<uint2*>(reinterpret_cast<__bf16*>(base) + idx) = u;
}

// Epilogue: normalise, then write (mode 0) or merge into (mode 1) the running
// state. With p.out_final set the result goes there as bf16 instead of back
// into p.out (rows this chunk does not reach are converted unchanged).
template <int NDB>
__device__ __forceinline__ void epilogue(const f32x16 (&O)[NDB], float m_ref, float l_acc,
                                         const AttnParams& p, int b, int h, int q_row, int lg) {
  constexpr int D = NDB * 32;
  const float l_row = pair_sum(l_acc);
  if (q_row >= p.Sq) return;
  const float inv = l_row > 0.0f ? 1.0f / l_row : 0.0f;
  const float lse_c = l_row > 0.0f ? (m_ref + log2f(l_row)) * kLn2 : neg_inf();
  const int64_t row0 = (((int64_t)b * p.Sq + q_row) * p.H + h) * D;
  float* orow = p.out + row0;
  float* lptr = p.lse + ((int64_t)b * p.H + h) * p.Sq + q_row;
  if (p.mode == 0) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float4 o;
        o.x = O[db][4 * i4 + 0] * inv;
        o.y = O[db][4 * i4 + 1] * inv;
        o.z = O[db][4 * i4 + 2] * inv;
        o.w = O[db][4 * i4 + 3] * inv;
        const int col = db * 32 + 8 * i4 + 4 * lg;
        if (p.out_final) store_bf16x4(p.out_final, row0 + col, o);
        else *reinterpret_cast<float4*>(orow + col) = o;
      }
    if (lg == 0) *lptr = lse_c;
    return;
  }
  // merge (ring-splash _update_out_and_lse). The running row is read whole, before any store
  // (one round trip to memory, not one per 16 bytes).
  float4 run[NDB * 4];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      run[4 * db + i4] = *reinterpret_cast<const float4*>(orow + db * 32 + 8 * i4 + 4 * lg);
  const float acc_lse = *lptr;
  if (lse_c == neg_inf()) {   // nothing attended in this chunk: identity
    if (p.out_final) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) store_bf16x4(p.out_final, row0 + db * 32 + 8 * i4 + 4 * lg, run[4 * db + i4]);
    }
    return;
  }
  float sig = 1.0f, new_lse = lse_c;
  if (acc_lse != neg_inf()) {
    const float x = lse_c - acc_lse;
    sig = 1.0f / (1.0f + expf(-x));
    new_lse = acc_lse + (fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x))));
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int col = db * 32 + 8 * i4 + 4 * lg;
      float4* ptr = reinterpret_cast<float4*>(orow + col);
      const float4 a = (acc_lse == neg_inf()) ? make_float4(0.f, 0.f, 0.f, 0.f) : run[4 * db + i4];
      float4 o;
      o.x = a.x - sig * (a.x - O[db][4 * i4 + 0] * inv);
      o.y = a.y - sig * (a.y - O[db][4 * i4 + 1] * inv);
      o.z = a.z - sig * (a.z - O[db][4 * i4 + 2] * inv);
      o.w = a.w - sig * (a.w - O[db][4 * i4 + 3] * inv);
      if (p.out_final) store_bf16x4(p.out_final, row0 + col, o);
      else *ptr = o;
    }
  if (lg == 0) *lptr = new_lse;
}

// The chunk of visit t of a one-launch ring: a copy of the launch's parameters pointing at
// chunk c = (ring_shard - t) mod n_chunks (or t for natural order), its K / V, masks, key
// positions and segments; sinks and the launch's `mode` belong to the first visit, out_final
// to the last.
__device__ __forceinline__ void ring_chunk_view(AttnParams& pc, const AttnParams& p, int t) {
  const int n = p.n_chunks;
  const int c = p.ring_shard >= 0 ? ((p.ring_shard - t) % n + n) % n : t;
  pc.k = reinterpret_cast<const __bf16*>(p.k) + c * p.kv_chunk_elems;
  pc.v = reinterpret_cast<const __bf16*>(p.v) + c * p.kv_chunk_elems;
  pc.tile_class = p.tile_class + c * p.mask_chunk_tiles;
  pc.col_idx = p.col_idx + c * p.mask_chunk_tiles;
  pc.row_cnt = p.row_cnt + c * p.mask_chunk_rows;
  pc.mask_bits = p.mask_bits ? p.mask_bits + c * p.mask_chunk_tiles * p.tile_words : nullptr;
  pc.kv_pos = p.kv_pos ? p.kv_pos + (int64_t)c * p.Skv : nullptr;
  pc.kv_seg = p.kv_seg ? p.kv_seg + (int64_t)c * p.Skv : nullptr;
  pc.kv_pos_base = p.kv_pos_base + c * p.Skv;
  pc.sinks = t == 0 ? p.sinks : nullptr;
  pc.mode = t == 0 ? p.mode : 1;
  pc.out_final = t == n - 1 ? p.out_final : nullptr;
  pc.vt = p.vt ? static_cast<const char*>(p.vt) + c * p.vt_chunk_bytes : nullptr;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + bytes): loads at offsets >= bytes return
// zero (raw buffer, stride 0; 0x00020000 is the gfx9 word-3 default format).
// `base` and `bytes` must be wave-uniform; they are read from the first lane
// so that the resource stays in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(lo | (hi << 32)), 0,
                                           __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 buffer_load_16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Transposing LDS read: within each group of 16 lanes, lane i receives element
// (i % 4) of the 8-byte chunks addressed by lanes i/4, i/4+4, i/4+8, i/4+12.
__device__ __forceinline__ s16x4 lds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// Transposing LDS reads issued from inline assembly. The compiler cannot tell
// a ds_read_b64_tr_b16 address from LDS that an LDS-DMA in flight is writing,
// so its own form waits for every outstanding DMA first, including the one
// filling the next tile. Kernels that prefetch by DMA issue these instead and
// wait for the next tile explicitly. A value read this way may not be touched
// (not even moved) before lds_settle(): the hardware does not interlock LDS
// results, so the wait ties every pending register.
struct TrPair {
  s16x4 lo, hi;
};
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}
// reads at p and p + OFF bytes
template <int OFF>
__device__ __forceinline__ TrPair lds_tr_pair_issue(const void* p) {
  TrPair r;
  asm volatile("ds_read_b64_tr_b16 %0, %2\n\tds_read_b64_tr_b16 %1, %2 offset:%3"
               : "=&v"(r.lo), "=&v"(r.hi)
               : "v"(lds_addr(p)), "i"(OFF));
  return r;
}
// reads at two addresses
__device__ __forceinline__ TrPair lds_tr_pair_issue2(const void* pa, const void* pb) {
  TrPair r;
  asm volatile("ds_read_b64_tr_b16 %0, %2\n\tds_read_b64_tr_b16 %1, %3"
               : "=&v"(r.lo), "=&v"(r.hi)
               : "v"(lds_addr(pa)), "v"(lds_addr(pb)));
  return r;
}
// A 16-byte LDS read issued from assembly, for the same reason; settle with lds_settle16.
__device__ __forceinline__ bf16x8 lds_b128_issue(const void* p) {
  bf16x8 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(lds_addr(p)));
  return r;
}
__device__ __forceinline__ void lds_settle16(bf16x8 (&t)[16]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(t[0]), "+v"(t[1]), "+v"(t[2]), "+v"(t[3]), "+v"(t[4]), "+v"(t[5]), "+v"(t[6]), "+v"(t[7]),
                 "+v"(t[8]), "+v"(t[9]), "+v"(t[10]), "+v"(t[11]), "+v"(t[12]), "+v"(t[13]), "+v"(t[14]), "+v"(t[15]));
}
// Waits for all LDS reads of this wave (lgkmcnt(0)) and ties eight pairs.
__device__ __forceinline__ void lds_settle(TrPair (&t)[8]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(t[0].lo), "+v"(t[0].hi), "+v"(t[1].lo), "+v"(t[1].hi), "+v"(t[2].lo), "+v"(t[2].hi),
                 "+v"(t[3].lo), "+v"(t[3].hi), "+v"(t[4].lo), "+v"(t[4].hi), "+v"(t[5].lo), "+v"(t[5].hi),
                 "+v"(t[6].lo), "+v"(t[6].hi), "+v"(t[7].lo), "+v"(t[7].hi));
}
__device__ __forceinline__ bf16x8 tr_join(const TrPair& t) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(t.lo, t.hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

}  // namespace attn
}  // namespace ram
