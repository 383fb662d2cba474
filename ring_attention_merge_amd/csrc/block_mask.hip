// Block-mask builder: tile classes (EMPTY / PARTIAL / FULL), per row of tiles
// the compacted ascending list of non-EMPTY kv tiles, and optionally the
// element mask of every PARTIAL tile as bits.
//
// What it computes: the block-sparse metadata the ejkernel ring-splash page
// passes to its kernel (MaskInfo: a block mask, the lists of blocks to visit
// and, for a caller-given two-dimensional mask, the contents of the partial
// blocks), built the way the Kvax page's create_attention_mask builds its
// block-wise masks: from positions and segment IDs, skipping blocks with
// nothing to attend. A tile is EMPTY when none of its (query, key) pairs is
// allowed, FULL when all are, else PARTIAL; pairs past the sequence ends do
// not count.
//
// One workgroup per (row of tiles, batch, chunk), or, where the pairs are checked, one per group
// of key tiles of a row, which then leave the compaction of the row's list to a second kernel
// (block_mask_compact). With sequential positions,
// no segments, no dense mask and no bits requested, a tile's class follows
// from its position ranges alone: FULL iff min q_pos >= max kv_pos, EMPTY iff
// max q_pos < min kv_pos; with explicit positions the same test runs on the
// tile's position minima and maxima. Otherwise every pair is checked, a
// group of tiles per round: each thread builds 32-pair words of the tiles' bit
// rows (key j of a tile at bit j % 32 of word j / 32) from a closed-form causal
// prefix (sequential keys), the segment IDs and 16-byte reads of the dense
// mask, skipping the reads for words the other tests already cleared; the
// words are staged in LDS and stored for PARTIAL tiles. Classes are staged in
// LDS, then compacted in order with wave ballots and a running offset.
#include <algorithm>

#include <hip/hip_runtime.h>

#include "ram_internal.h"

namespace ram {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// Pairwise rounds cover up to kGroupKeys keys and kGroupWords bit words.
constexpr int kGroupKeys = 1024;
constexpr int kGroupWords = 8192;
constexpr int kGroupTiles = 8;   // at most this many tiles per round (and per workgroup of a split row)

// One bit per byte of 4 bytes (nonzero -> 1), byte k to bit k: OR-fold each
// byte onto its lowest bit, then one multiply moves the four bits next to each
// other at bits 21..24 (the 16 partial products land on distinct bits).
__device__ __forceinline__ uint32_t nonzero_bytes4(uint32_t x) {
  uint32_t y = x | (x >> 4);
  y |= y >> 2;
  y |= y >> 1;
  y &= 0x01010101u;
  return ((y * 0x00204081u) >> 21) & 0xFu;
}

// Bits of 32 dense-mask bytes held in two 16-byte values, byte j at bit j.
__device__ __forceinline__ uint32_t bits_of_bytes32(const uint4& a, const uint4& b) {
  return nonzero_bytes4(a.x) | nonzero_bytes4(a.y) << 4 | nonzero_bytes4(a.z) << 8 | nonzero_bytes4(a.w) << 12 |
         nonzero_bytes4(b.x) << 16 | nonzero_bytes4(b.y) << 20 | nonzero_bytes4(b.z) << 24 | nonzero_bytes4(b.w) << 28;
}

// Bits of `n` (<= 32) consecutive dense-mask bytes, byte j at bit j.
__device__ __forceinline__ uint32_t dense_word(const uint8_t* d, int n) {
  if (n == 32 && (reinterpret_cast<uintptr_t>(d) & 15) == 0)
    return bits_of_bytes32(*reinterpret_cast<const uint4*>(d), *reinterpret_cast<const uint4*>(d + 16));
  uint32_t m = 0;
  for (int j = 0; j < n; ++j) m |= (uint32_t)(d[j] != 0) << j;
  return m;
}

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

// Bit jj of the result: keys[j0 + jj] <= v (EQ false) or == v (EQ true), jj < n. A full,
// 16-byte aligned word reads its 32 values with eight 16-byte LDS reads issued together.
template <bool EQ>
__device__ __forceinline__ uint32_t key_bits(const int* keys, int j0, int n, int v) {
  uint32_t m = 0;
  if (n == 32 && (j0 & 3) == 0) {
    const int4* k4 = reinterpret_cast<const int4*>(keys + j0);
    int4 a[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) a[q] = k4[q];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e[4] = {a[q].x, a[q].y, a[q].z, a[q].w};
#pragma unroll
      for (int r = 0; r < 4; ++r) m |= (uint32_t)(EQ ? e[r] == v : e[r] <= v) << (4 * q + r);
    }
    return m;
  }
  for (int jj = 0; jj < n; ++jj) m |= (uint32_t)(EQ ? keys[j0 + jj] == v : keys[j0 + jj] <= v) << jj;
  return m;
}

// n / d for n < 2^14 and d < 2^13 by one high multiply (exact on that range: m = floor(2^32/d) + 1).
struct FastDiv {
  uint32_t d, m;
  __device__ explicit FastDiv(uint32_t d_) : d(d_), m(d_ > 1 ? (uint32_t)(0xFFFFFFFFu / d_) + 1u : 0u) {}
  __device__ uint32_t div(uint32_t n) const { return d > 1 ? __umulhi(n, m) : n; }
};

// Key tiles per pairwise round (and per workgroup of a split row): bounded by the keys staged
// and by the bit words held in LDS.
__host__ __device__ inline int group_tiles(int bq, int bk) {
  const int tw = bq * ((bk + 31) >> 5);
  return max(1, min(kGroupTiles, min(kGroupKeys / bk, kGroupWords / tw)));
}

__device__ __forceinline__ void compact_row_impl(const MaskParams& p, int64_t crow, const uint8_t* cls_s, int* wsum);
__device__ __forceinline__ void compact_row(const MaskParams& p, int64_t crow, const uint8_t* cls_s, int* wsum) {
  compact_row_impl(p, crow, cls_s, wsum);
}

// The parts of a workgroup's dynamic LDS, 16-byte aligned byte offsets: the bit words of a
// round, the keys' positions and segments of a round, the rows' positions and segments, and the
// row's tile classes. A part that a variant does not read has size 0.
struct MaskLds {
  int bits, kpos, kseg, qpos, qseg, cls, total;
};
__host__ __device__ inline int lds_round16(int b) { return (b + 15) & ~15; }
__host__ __device__ inline MaskLds mask_lds(const MaskParams& p, bool pair, bool kpos, bool segs) {
  const int tg = group_tiles(p.bq, p.bk);
  MaskLds l;
  int o = 0;
  l.bits = o;
  o += pair ? lds_round16(tg * p.bq * ((p.bk + 31) >> 5) * 4) : 0;
  l.kpos = o;
  o += pair && kpos ? lds_round16(tg * p.bk * 4) : 0;
  l.kseg = o;
  o += pair && segs ? lds_round16(tg * p.bk * 4) : 0;
  l.qpos = o;
  o += pair ? lds_round16(p.bq * 4) : 0;
  l.qseg = o;
  o += pair && segs ? lds_round16(p.bq * 4) : 0;
  l.cls = o;
  o += lds_round16(p.nKb);
  l.total = o;
  return l;
}

// PAIR: pairs are checked (segments, a dense mask or bits requested), else classes from ranges.
// KPOS: explicit key positions (else sequential from kv_pos_base). SEGS: segment IDs on both
// sides. DENSE: a dense mask. Each combination is its own kernel, so that one holds only the
// registers and LDS its tests need; the dense mask alone fits 8 workgroups per CU (64 VGPRs).
template <bool PAIR, bool KPOS, bool SEGS, bool DENSE>
__global__ __launch_bounds__(kThreads, DENSE && !SEGS && !KPOS ? 8 : 4) void block_mask_kernel(MaskParams p) {
  static_assert(2 * kGroupTiles <= 32, "two flag bits per tile of a round in one word");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ int red[2 * kWaves];
  __shared__ int wsum[kWaves];
  __shared__ int open_s[kGroupTiles];
  __shared__ int n_open_s;
  // per tile t of the round, bits 2t (a pair allowed) and 2t+1 (a pair excluded)
  __shared__ uint32_t flags_s;
  const MaskLds L = mask_lds(p, PAIR, KPOS, SEGS);
  uint8_t* cls_s = lds + L.cls;

  const int qb = blockIdx.x / p.kv_split, b = blockIdx.y, c = blockIdx.z;
  const int split = blockIdx.x - qb * p.kv_split;   // this workgroup's group of key tiles
  const int tid = threadIdx.x;
  const int q0 = qb * p.bq;
  const int nq = min(p.Sq, q0 + p.bq) - q0;
  const int kv_base = p.kv_pos_base + c * p.kv_base_step;
  const int32_t* qpos = p.q_pos ? p.q_pos + (int64_t)b * p.qm_stride_b + q0 : nullptr;
  const int32_t* qseg = SEGS ? p.q_seg + (int64_t)b * p.qm_stride_b + q0 : nullptr;
  const int64_t kvoff = (int64_t)b * p.kvm_stride_b + (int64_t)c * p.kv_chunk_off;
  const int32_t* kvpos = KPOS ? p.kv_pos + kvoff : nullptr;
  const int32_t* kvseg = SEGS ? p.kv_seg + kvoff : nullptr;
  const int64_t crow = ((int64_t)c * p.B + b) * p.nQb + qb;   // row index over (chunk, batch, q tile)

  if constexpr (!PAIR) {
    // No segments or dense mask: classes from position ranges (exact: all pairs allowed iff
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
    if constexpr (!KPOS) {
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
    // Pairwise: positions, segments and the dense mask of every pair, a group
    // of tiles per round. Each thread builds 32-pair words of the tiles' bit
    // rows; per-tile flags (a pair allowed, a pair excluded) give the classes.
    uint32_t* bits_s = reinterpret_cast<uint32_t*>(lds + L.bits);
    int* kpos_s = reinterpret_cast<int*>(lds + L.kpos);
    int* kseg_s = reinterpret_cast<int*>(lds + L.kseg);
    int* qpos_s = reinterpret_cast<int*>(lds + L.qpos);
    int* qseg_s = reinterpret_cast<int*>(lds + L.qseg);
    const int tg = group_tiles(p.bq, p.bk);
    // a split row: this workgroup's group only
    const int kb_first = p.kv_split > 1 ? split * tg : 0;
    const int kb_end = p.kv_split > 1 ? min(p.nKb, kb_first + tg) : p.nKb;
    // The keys of a group into LDS, all of a thread's loads issued before the first store
    // (a group holds at most kGroupKeys keys), and the flags cleared. The first group's loads
    // are issued here, beside the rows' (the barriers below cover them).
    auto stage_group = [&](int kbg) {
      if constexpr (KPOS || SEGS) {
        const int ng = min(tg, p.nKb - kbg);
        const int g0 = kbg * p.bk;
        const int gk = min(p.Skv, (kbg + ng) * p.bk) - g0;
        constexpr int R = kGroupKeys / kThreads;
        int pv[R] = {}, sv[R] = {};
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int j = tid + r * kThreads;
          if (j < gk) {
            if constexpr (KPOS) pv[r] = kvpos[g0 + j];
            if constexpr (SEGS) sv[r] = kvseg[g0 + j];
          }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int j = tid + r * kThreads;
          if (j < gk) {
            if constexpr (KPOS) kpos_s[j] = pv[r];
            if constexpr (SEGS) kseg_s[j] = sv[r];
          }
        }
      }
      if (tid == 0) flags_s = 0;
    };
    if (kb_first < kb_end) stage_group(kb_first);
    // ranges over the rows that can have an allowed key (padding rows have none)
    int qpl = 0x7fffffff, qph = -0x7fffffff - 1, qsl = 0x7fffffff, qsh = -0x7fffffff - 1;
    bool qpad = false;
    for (int i = tid; i < nq; i += kThreads) {
      qpos_s[i] = qpos ? qpos[i] : p.q_pos_base + q0 + i;
      if constexpr (SEGS) {
        qseg_s[i] = qseg[i];
        if (qseg_s[i] == -1) {
          qpad = true;
          continue;
        }
        qsl = min(qsl, qseg_s[i]);
        qsh = max(qsh, qseg_s[i]);
      }
      qpl = min(qpl, qpos_s[i]);
      qph = max(qph, qpos_s[i]);
    }
    // Tiles whose class follows from the rows' and keys' position and segment ranges are
    // decided before their pairs are checked (exactly: these are sufficient conditions); the
    // rest (class 3 until then) go through the pairwise words. Ranges leave out padding rows
    // and keys (segment -1), which have no allowed pair. EMPTY: every key after every row
    // (causal), disjoint segment ranges, or all rows or all keys padding. FULL (without a
    // dense mask, which can clear any pair): every key at or before every row, no padding,
    // and one segment on both sides.
    int qpmin, qpmax, qsmin = 0, qsmax = 0;
    block_minmax(qpl, qph, red, qpmin, qpmax);
    if constexpr (SEGS) block_minmax(qsl, qsh, red, qsmin, qsmax);
    const bool any_qpad = SEGS ? __syncthreads_or(qpad) : false;
    const int W = (p.bk + 31) >> 5;   // words per tile row
    const int tw = p.bq * W;          // words per tile
    const uint8_t* drow0 = DENSE ? p.dense + (int64_t)q0 * p.dense_ld + (int64_t)c * p.dense_col_step : nullptr;
    for (int kbg = kb_first; kbg < kb_end; kbg += tg) {
      const int ng = min(tg, p.nKb - kbg);
      const int g0 = kbg * p.bk;                           // first key of the group
      const int gk = min(p.Skv, (kbg + ng) * p.bk) - g0;   // keys of the group
      if (kbg != kb_first) stage_group(kbg);
      __syncthreads();
      // the group's tiles by their ranges, 16 threads per tile
      bool open = false;
      for (int t0 = 0; t0 < ng; t0 += kThreads / 16) {
        const int t = t0 + (tid >> 4), l = tid & 15;
        const int nk = t < ng ? min(p.bk, gk - t * p.bk) : 0;
        int kpl = 0x7fffffff, kph = -0x7fffffff - 1, ksl = 0x7fffffff, ksh = -0x7fffffff - 1, kpad = 0;
        if constexpr (KPOS || SEGS) {
          for (int j = l; j < nk; j += 16) {
            int sg = 0;
            if constexpr (SEGS) {
              sg = kseg_s[t * p.bk + j];
              if (sg == -1) {
                kpad = 1;
                continue;
              }
            }
            const int kp = KPOS ? kpos_s[t * p.bk + j] : kv_base + g0 + t * p.bk + j;
            kpl = min(kpl, kp);
            kph = max(kph, kp);
            ksl = min(ksl, sg);
            ksh = max(ksh, sg);
          }
#pragma unroll
          for (int o = 8; o > 0; o >>= 1) {
            kpl = min(kpl, __shfl_xor(kpl, o, 16));
            kph = max(kph, __shfl_xor(kph, o, 16));
            ksl = min(ksl, __shfl_xor(ksl, o, 16));
            ksh = max(ksh, __shfl_xor(ksh, o, 16));
            kpad |= __shfl_xor(kpad, o, 16);
          }
        } else if (nk > 0) {
          // sequential keys, no padding
          kpl = kv_base + g0 + t * p.bk;
          kph = kpl + nk - 1;
        }
        if (t < ng) {
          // (with no non-padding rows or keys the ranges are empty: min > max)
          const bool empty = nk <= 0 || qpmin > qpmax || kpl > kph || (p.causal && kpl > qpmax) ||
                             (SEGS && (ksh < qsmin || ksl > qsmax));
          const bool full = !DENSE && !any_qpad && !kpad && (!p.causal || kph <= qpmin) &&
                            (!SEGS || (qsmin == qsmax && ksl == ksh && qsmin == ksl));
          const uint8_t cl = empty ? 0 : (full ? 2 : 3);
          if (l == 0) cls_s[kbg + t] = cl;
          open = open || cl == 3;
        }
      }
      if (!__syncthreads_or(open)) continue;   // every tile of the group decided
      // the tiles left open, in order: only their words are checked
      if (tid == 0) {
        int no = 0;
        for (int t = 0; t < ng; ++t)
          if (cls_s[kbg + t] == 3) open_s[no++] = t;
        n_open_s = no;
      }
      __syncthreads();
      const int nw = n_open_s * tw;   // words of the open tiles
      const int gw = n_open_s * W;    // words per query row across them
      const FastDiv div_gw((uint32_t)gw), div_w((uint32_t)W), div_tw((uint32_t)tw), div_bq((uint32_t)p.bq);
      // With a dense mask, words are taken row by row (consecutive threads:
      // consecutive 32-key words of one query row), so that the mask is read in
      // long contiguous runs; without one, column by column (consecutive threads:
      // one word of consecutive rows), so that a wave's key reads are LDS
      // broadcasts (the builder 9% faster on the packed-document workload).
      // kBatch words per thread at a time: their positions and segments first,
      // then all their dense-mask loads together. A thread's flags stay in a
      // register until the round ends. With a dense mask, one word per thread:
      // the rate follows the workgroups resident per CU, not the loads each
      // thread keeps in flight (over a 32k x 32k causal mask, 4.0 TB/s at one
      // word and 8 waves per SIMD; 3.5 at two words and 5 waves; 3.1 at four).
      constexpr int kBatch = DENSE ? 1 : 2;
      uint32_t fl = 0;
      for (int u0 = tid; u0 < nw; u0 += kBatch * kThreads) {
        uint32_t wv[kBatch], valv[kBatch];
        int tv[kBatch], tlv[kBatch], iv[kBatch], j0v[kBatch], jnv[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int u = u0 + k * kThreads;
          int i, oi, wi;
          if constexpr (DENSE) {
            i = (int)div_gw.div((uint32_t)u);
            const int jw = u - i * gw;
            oi = (int)div_w.div((uint32_t)jw);
            wi = jw - oi * W;
          } else {
            const int col = (int)div_bq.div((uint32_t)u);
            i = u - col * p.bq;
            oi = (int)div_w.div((uint32_t)col);
            wi = col - oi * W;
          }
          const int tl = u < nw ? open_s[oi] : 0;
          const int j0 = tl * p.bk + wi * 32;                // first key of the word within the group
          const int jn = u < nw ? min(min(32, gk - j0), (tl + 1) * p.bk - j0) : 0;
          tv[k] = tl * tw + i * W + wi;                      // the word's place in bits_s (tile-major)
          tlv[k] = tl;
          iv[k] = i;
          j0v[k] = j0;
          jnv[k] = jn;
          uint32_t w = 0, valid = 0;
          if (u < nw && i < nq && jn > 0) {
            valid = jn == 32 ? ~0u : ((1u << jn) - 1u);
            w = valid;
            if (p.causal) {
              if constexpr (!KPOS) {
                // sequential keys: the allowed ones are a prefix of the word
                const int64_t lim = (int64_t)qpos_s[i] - ((int64_t)kv_base + g0 + j0);
                w &= lim < 0 ? 0u : (lim >= 31 ? ~0u : ((2u << lim) - 1u));
              } else {
                w &= key_bits<false>(kpos_s, j0, jn, qpos_s[i]);
              }
            }
            if constexpr (SEGS) {
              if (w) {
                const int qs = qseg_s[i];
                w &= qs != -1 ? key_bits<true>(kseg_s, j0, jn, qs) : 0u;
              }
            }
          }
          wv[k] = w;
          valv[k] = valid;
        }
        if constexpr (DENSE) {
          uint4 lo[kBatch], hi[kBatch];
#pragma unroll
          for (int k = 0; k < kBatch; ++k) {
            const uint8_t* d = drow0 + (int64_t)iv[k] * p.dense_ld + g0 + j0v[k];
            lo[k] = hi[k] = make_uint4(0, 0, 0, 0);
            if (wv[k] && jnv[k] == 32 && (reinterpret_cast<uintptr_t>(d) & 15) == 0) {
              lo[k] = *reinterpret_cast<const uint4*>(d);
              hi[k] = *reinterpret_cast<const uint4*>(d + 16);
            }
          }
#pragma unroll
          for (int k = 0; k < kBatch; ++k) {
            if (!wv[k]) continue;
            const uint8_t* d = drow0 + (int64_t)iv[k] * p.dense_ld + g0 + j0v[k];
            wv[k] &= (jnv[k] == 32 && (reinterpret_cast<uintptr_t>(d) & 15) == 0) ? bits_of_bytes32(lo[k], hi[k])
                                                                                   : dense_word(d, jnv[k]);
          }
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          if (u0 + k * kThreads >= nw) continue;
          const uint32_t w = wv[k];
          const uint32_t f = valv[k] ? ((w != 0 ? 1u : 0u) | (w != valv[k] ? 2u : 0u)) : 0u;
          fl |= f << (2 * tlv[k]);
          bits_s[tv[k]] = w;
        }
      }
      // the round's flags: OR over the wave, then one LDS atomic per wave
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) fl |= __shfl_xor(fl, o);
      if ((tid & 63) == 0 && fl) atomicOr(&flags_s, fl);
      __syncthreads();
      const uint32_t flags = flags_s;
      for (int t = tid; t < ng; t += kThreads) {
        const uint32_t f = (flags >> (2 * t)) & 3u;
        if (cls_s[kbg + t] == 3) cls_s[kbg + t] = (f & 1) ? ((f & 2) ? 1 : 2) : 0;
      }
      if (p.bits) {
        // the bits of the open tiles that came out PARTIAL
        uint32_t* dst = p.bits + ((size_t)crow * p.nKb + kbg) * tw;
        for (int u = tid; u < nw; u += kThreads) {
          const int oi = (int)div_tw.div((uint32_t)u);
          const int t = open_s[oi], o = t * tw + (u - oi * tw);
          if (((flags >> (2 * t)) & 3u) == 3u) dst[o] = bits_s[o];
        }
      }
      __syncthreads();   // the next group rewrites kpos_s / kseg_s / bits_s / flags_s
    }
  }
  __syncthreads();

  uint8_t* cls_out = p.tile_class + crow * p.nKb;
  if (p.kv_split > 1) {
    // a split row: this group's classes; block_mask_compact makes the list
    const int tg = group_tiles(p.bq, p.bk);
    const int kb_first = split * tg, kb_end = min(p.nKb, kb_first + tg);
    for (int kb = kb_first + tid; kb < kb_end; kb += kThreads) cls_out[kb] = cls_s[kb];
    return;
  }
  // Write classes and compact the non-EMPTY tiles in ascending order.
  for (int kb = tid; kb < p.nKb; kb += kThreads) cls_out[kb] = cls_s[kb];
  compact_row(p, crow, cls_s, wsum);
}

// The compacted list and count of one row of tiles from its classes in LDS.
__device__ __forceinline__ void compact_row_impl(const MaskParams& p, int64_t crow, const uint8_t* cls_s, int* wsum) {
  const int tid = threadIdx.x;
  int32_t* col_out = p.col_idx + crow * p.nKb;
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

// Lists of the rows block_mask_kernel classified in split groups: one workgroup per row.
__global__ __launch_bounds__(kThreads) void block_mask_compact(MaskParams p) {
  __shared__ uint8_t cls_s[kMaxMaskCols];
  __shared__ int wsum[kWaves];
  const int64_t crow = ((int64_t)blockIdx.z * p.B + blockIdx.y) * p.nQb + blockIdx.x;
  const uint8_t* cls_in = p.tile_class + crow * p.nKb;
  for (int kb = threadIdx.x; kb < p.nKb; kb += kThreads) cls_s[kb] = cls_in[kb];
  __syncthreads();
  compact_row_impl(p, crow, cls_s, wsum);
}

// Counting sort of the rows by their total tile count, most first (one workgroup).
constexpr int kOrderThreads = 1024;
constexpr int kOrderKeys = 4096;
__global__ __launch_bounds__(kOrderThreads) void row_order_kernel(const int32_t* row_cnt, int n_chunks, int64_t rows,
                                                                  int max_key, int32_t* order) {
  __shared__ int hist[kOrderKeys];
  const int tid = threadIdx.x;
  const int nk = max_key + 1;   // keys 0 .. max_key, histogram slot max_key - key (most first)
  for (int i = tid; i < nk; i += kOrderThreads) hist[i] = 0;
  __syncthreads();
  auto key = [&](int64_t r) {
    int64_t t = 0;
    for (int c = 0; c < n_chunks; ++c) t += row_cnt[c * rows + r];
    return (int)min<int64_t>(t, max_key);
  };
  for (int64_t r = tid; r < rows; r += kOrderThreads) atomicAdd(&hist[max_key - key(r)], 1);
  __syncthreads();
  // exclusive prefix sum over the slots, by one wave (each lane a contiguous run of slots)
  if (tid < 64) {
    const int per = (nk + 63) / 64;
    const int s0 = min(nk, tid * per), s1 = min(nk, s0 + per);
    int run = 0;
    for (int i = s0; i < s1; ++i) run += hist[i];
    int incl = run;
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (tid >= o) incl += v;
    }
    int base = incl - run;
    for (int i = s0; i < s1; ++i) {
      const int c = hist[i];
      hist[i] = base;
      base += c;
    }
  }
  __syncthreads();
  for (int64_t r = tid; r < rows; r += kOrderThreads) order[atomicAdd(&hist[max_key - key(r)], 1)] = (int32_t)r;
}

}  // namespace

hipError_t launch_row_order(const int32_t* row_cnt, int n_chunks, int64_t rows, int max_tiles, int32_t* order,
                            hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const int max_key = (int)std::min<int64_t>((int64_t)max_tiles * n_chunks, kOrderKeys - 1);
  hipLaunchKernelGGL(row_order_kernel, dim3(1), dim3(kOrderThreads), 0, s, row_cnt, n_chunks, rows, max_key, order);
  return hipGetLastError();
}

hipError_t launch_block_mask(const MaskParams& p_in, int n_chunks, hipStream_t s) {
  if (p_in.B == 0 || p_in.nQb == 0 || n_chunks == 0) return hipSuccess;
  MaskParams p = p_in;
  // Rows checked pair by pair (segments, a dense mask or stored bits) take one workgroup per
  // group of key tiles when a row has several groups, so that a row's rounds run side by side.
  const bool segs = p.q_seg != nullptr, dense = p.dense != nullptr, kpos = p.kv_pos != nullptr;
  const bool pair = segs || dense || p.bits != nullptr;
  const int tg = group_tiles(p.bq, p.bk);
  p.kv_split = pair ? (p.nKb + tg - 1) / tg : 1;
  if (p.kv_split < 1) p.kv_split = 1;
  using Kernel = void (*)(MaskParams);
  static constexpr Kernel kRange[2] = {block_mask_kernel<false, false, false, false>,
                                       block_mask_kernel<false, true, false, false>};
  static constexpr Kernel kPair[8] = {
      block_mask_kernel<true, false, false, false>, block_mask_kernel<true, false, false, true>,
      block_mask_kernel<true, false, true, false>,  block_mask_kernel<true, false, true, true>,
      block_mask_kernel<true, true, false, false>,  block_mask_kernel<true, true, false, true>,
      block_mask_kernel<true, true, true, false>,   block_mask_kernel<true, true, true, true>};
  const Kernel k = pair ? kPair[(kpos ? 4 : 0) | (segs ? 2 : 0) | (dense ? 1 : 0)] : kRange[kpos ? 1 : 0];
  const size_t lds = (size_t)mask_lds(p, pair, kpos, segs).total;
  hipLaunchKernelGGL(k, dim3(p.nQb * p.kv_split, p.B, n_chunks), dim3(kThreads), lds, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.kv_split == 1) return e;
  hipLaunchKernelGGL(block_mask_compact, dim3(p.nQb, p.B, n_chunks), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace ram
