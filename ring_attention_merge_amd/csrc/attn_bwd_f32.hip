// Block-sparse attention backward for one KV chunk with float32 inputs.
//
// The same gradients as the bf16 kernels (the per-step chunk backward of the
// ejkernel ring-splash page's _ring_attention_backward, against the ring's
// final out and logsumexp): for query row i and allowed key j,
//   p = exp(u_ij - lse_i) with u the scaled (and capped) logit, dp = dout_i . v_j,
//   ds = p (dp - D_i) (1 - t^2 with a soft cap), dq_i += scale ds k_j,
//   dk_j += scale ds q_i, dv_j += p dout_i   (dk, dv summed over the KV group).
//
// Float32 is the exact-reference dtype here, not a throughput path: plain
// float32 VALU arithmetic, 16 lanes per row (or key), each holding D/16
// dimensions, dot products finished by a 16-lane butterfly. The tiles visited
// are the non-EMPTY ones of the block mask (per q tile for dq, per kv tile via
// the transposed lists for dk/dv); PARTIAL tiles are masked from positions and
// segments, or from the stored bits of a dense mask.
#include "attn_common.h"

namespace ram {
namespace {

using namespace attn;

constexpr int kLanes = 16;                 // lanes per row / key
constexpr int kRowsPerWg = 256 / kLanes;   // 16

__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) x += __shfl_xor(x, o, 16);
  return x;
}

// Whether query row i (position qpos, segment qseg) may attend key j of the chunk,
// inside the tile (qb, kb) of class cls (never EMPTY here).
__device__ __forceinline__ bool pair_allowed(const AttnParams& p, int b, int qb, int kb, int cls, int i, int j,
                                             int qpos, int qseg) {
  if (j >= p.Skv || i >= p.Sq) return false;
  if (cls == 2) return true;   // FULL
  if (p.mask_bits) {
    const uint32_t* tb = p.mask_bits + (((int64_t)b * p.nQb + qb) * p.nKb + kb) * kBlockQ * 2;
    const int r = i - qb * kBlockQ, c = j - kb * kBlockKV;
    return (tb[r * 2 + (c >> 5)] >> (c & 31)) & 1u;
  }
  const int64_t km = (int64_t)b * p.kvm_stride_b + j;
  const int kpos = p.kv_pos ? p.kv_pos[km] : p.kv_pos_base + j;
  if (p.causal && kpos > qpos) return false;
  if (p.q_seg) {
    const int kseg = p.kv_seg ? p.kv_seg[km] : 0;
    if (kseg != qseg || qseg == -1) return false;
  }
  return true;
}

// Weight and score gradient of one allowed pair: raw dot s, dout . v = dp.
__device__ __forceinline__ void pair_grads(const AttnParams& p, float s, float dp, float lse, float dl, float& pw,
                                           float& ds) {
  const float scale = p.scale_log2 * kLn2;
  float u = s * scale, g = 1.0f;
  if (p.softcap_on) {
    const float cap = p.cap_log2 * kLn2;
    const float t = tanhf(u / cap);
    u = cap * t;
    g = 1.0f - t * t;
  }
  pw = lse == neg_inf() ? 0.0f : expf(u - lse);
  ds = pw * (dp - dl) * g;
}

// dq: one workgroup per (batch, head, 16 rows of a 128-row q tile); K / V tiles through LDS.
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_f32(BwdParams bp) {
  const AttnParams& p = bp.a;
  constexpr int NP = D / kLanes;   // dimensions per lane
  __shared__ __attribute__((aligned(16))) float kv_s[2][kBlockKV][D];
  const int64_t item = blockIdx.x;
  const int sub = (int)(item % (kBlockQ / kRowsPerWg));
  const int64_t r1 = item / (kBlockQ / kRowsPerWg);
  const int qb = (int)(r1 % p.nQb);
  const int64_t r2 = r1 / p.nQb;
  const int h = (int)(r2 % p.H);
  const int b = (int)(r2 / p.H);
  const int G = p.H / p.Hkv, g = h / G;
  const int tid = threadIdx.x, part = tid % kLanes;
  const int i = qb * kBlockQ + sub * kRowsPerWg + tid / kLanes;
  const bool row_ok = i < p.Sq;
  const int ic = row_ok ? i : 0;

  const float* qrow = reinterpret_cast<const float*>(p.q) + (int64_t)b * p.q_stride_b + ((int64_t)ic * p.H + h) * D;
  const float* drow = reinterpret_cast<const float*>(bp.dout) + (((int64_t)b * p.Sq + ic) * p.H + h) * D;
  float qv[NP], dv[NP], acc[NP];
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    qv[e] = qrow[part * NP + e];
    dv[e] = drow[part * NP + e];
    acc[e] = 0.0f;
  }
  const int64_t li = ((int64_t)b * p.H + h) * p.Sq + ic;
  const float lse = p.lse[li], dl = bp.delta[li];
  const int qpos = p.q_pos ? p.q_pos[(int64_t)b * p.qm_stride_b + ic] : p.q_pos_base + i;
  const int qseg = p.q_seg ? p.q_seg[(int64_t)b * p.qm_stride_b + ic] : 0;

  const int64_t mrow = (int64_t)b * p.nQb + qb;
  const int cnt = p.row_cnt[mrow];
  const int64_t krs = (int64_t)p.Hkv * D;
  const float* kbase = reinterpret_cast<const float*>(p.k) + (int64_t)b * p.kv_stride_b + g * D;
  const float* vbase = reinterpret_cast<const float*>(p.v) + (int64_t)b * p.kv_stride_b + g * D;
  for (int it = 0; it < cnt; ++it) {
    const int kb = p.col_idx[mrow * p.nKb + it];
    const int cls = p.tile_class[mrow * p.nKb + kb];
    __syncthreads();   // the previous tile's readers are done
    for (int x = tid; x < kBlockKV * D / 4; x += 256) {
      const int r = x / (D / 4), c4 = x % (D / 4);
      const int j = kb * kBlockKV + r;
      float4 kk = make_float4(0.f, 0.f, 0.f, 0.f), vv = kk;
      if (j < p.Skv) {
        kk = *reinterpret_cast<const float4*>(kbase + j * krs + c4 * 4);
        vv = *reinterpret_cast<const float4*>(vbase + j * krs + c4 * 4);
      }
      *reinterpret_cast<float4*>(&kv_s[0][r][c4 * 4]) = kk;
      *reinterpret_cast<float4*>(&kv_s[1][r][c4 * 4]) = vv;
    }
    __syncthreads();
    for (int r = 0; r < kBlockKV; ++r) {
      const int j = kb * kBlockKV + r;
      float s = 0.0f, dp = 0.0f;
#pragma unroll
      for (int e = 0; e < NP; ++e) {
        s += qv[e] * kv_s[0][r][part * NP + e];
        dp += dv[e] * kv_s[1][r][part * NP + e];
      }
      s = sum16(s);
      dp = sum16(dp);
      if (!pair_allowed(p, b, qb, kb, cls, i, j, qpos, qseg)) continue;
      float pw, ds;
      pair_grads(p, s, dp, lse, dl, pw, ds);
#pragma unroll
      for (int e = 0; e < NP; ++e) acc[e] += ds * kv_s[0][r][part * NP + e];
    }
  }
  if (!row_ok) return;
  const float scale = p.scale_log2 * kLn2;
  float* dq = bp.dq + (((int64_t)b * p.Sq + i) * p.H + h) * D + part * NP;
#pragma unroll
  for (int e = 0; e < NP; ++e) dq[e] = acc[e] * scale + (bp.dq_mode == 1 ? dq[e] : 0.0f);
}

// dk, dv: one workgroup per (batch, kv head, 16 keys of a 64-key tile); the q and
// dout rows of each (q tile, head) through LDS.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkv_f32(BwdParams bp) {
  const AttnParams& p = bp.a;
  constexpr int NP = D / kLanes;
  constexpr int kRowsStage = 32;   // q rows staged at a time
  __shared__ __attribute__((aligned(16))) float qd_s[2][kRowsStage][D];
  __shared__ float row_s[4][kRowsStage];   // lse, D, position, segment
  const int64_t item = blockIdx.x;
  const int sub = (int)(item % (kBlockKV / kRowsPerWg));
  const int64_t r1 = item / (kBlockKV / kRowsPerWg);
  const int kb = (int)(r1 % p.nKb);
  const int64_t r2 = r1 / p.nKb;
  const int g = (int)(r2 % p.Hkv);
  const int b = (int)(r2 / p.Hkv);
  const int G = p.H / p.Hkv;
  const int tid = threadIdx.x, part = tid % kLanes;
  const int j = kb * kBlockKV + sub * kRowsPerWg + tid / kLanes;
  const bool key_ok = j < p.Skv;
  const int jc = key_ok ? j : 0;

  const int64_t krs = (int64_t)p.Hkv * D;
  const float* krow = reinterpret_cast<const float*>(p.k) + (int64_t)b * p.kv_stride_b + jc * krs + g * D;
  const float* vrow = reinterpret_cast<const float*>(p.v) + (int64_t)b * p.kv_stride_b + jc * krs + g * D;
  float kv_[NP], vv_[NP], dk[NP], dvv[NP];
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    kv_[e] = krow[part * NP + e];
    vv_[e] = vrow[part * NP + e];
    dk[e] = 0.0f;
    dvv[e] = 0.0f;
  }

  const int64_t kcol = (int64_t)b * p.nKb + kb;
  const int ccnt = bp.col_cnt[kcol];
  for (int ci = 0; ci < ccnt; ++ci) {
    const int qb = bp.row_idx[kcol * p.nQb + ci];
    const int cls = p.tile_class[((int64_t)b * p.nQb + qb) * p.nKb + kb];
    for (int hg = 0; hg < G; ++hg) {
      const int h = g * G + hg;
      for (int r0 = qb * kBlockQ; r0 < min(p.Sq, (qb + 1) * kBlockQ); r0 += kRowsStage) {
        __syncthreads();   // the previous rows' readers are done
        for (int x = tid; x < kRowsStage * D / 4; x += 256) {
          const int r = x / (D / 4), c4 = x % (D / 4);
          const int i = r0 + r;
          float4 qq = make_float4(0.f, 0.f, 0.f, 0.f), oo = qq;
          if (i < p.Sq) {
            qq = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p.q) + (int64_t)b * p.q_stride_b +
                                                  ((int64_t)i * p.H + h) * D + c4 * 4);
            oo = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(bp.dout) +
                                                  (((int64_t)b * p.Sq + i) * p.H + h) * D + c4 * 4);
          }
          *reinterpret_cast<float4*>(&qd_s[0][r][c4 * 4]) = qq;
          *reinterpret_cast<float4*>(&qd_s[1][r][c4 * 4]) = oo;
        }
        if (tid < kRowsStage) {
          const int i = r0 + tid;
          const int ic = i < p.Sq ? i : 0;
          const int64_t li = ((int64_t)b * p.H + h) * p.Sq + ic;
          row_s[0][tid] = i < p.Sq ? p.lse[li] : neg_inf();
          row_s[1][tid] = i < p.Sq ? bp.delta[li] : 0.0f;
          row_s[2][tid] = __int_as_float(p.q_pos ? p.q_pos[(int64_t)b * p.qm_stride_b + ic] : p.q_pos_base + i);
          row_s[3][tid] = __int_as_float(p.q_seg ? p.q_seg[(int64_t)b * p.qm_stride_b + ic] : 0);
        }
        __syncthreads();
        const int nr = min(kRowsStage, p.Sq - r0);
        for (int r = 0; r < nr; ++r) {
          const int i = r0 + r;
          float s = 0.0f, dp = 0.0f;
#pragma unroll
          for (int e = 0; e < NP; ++e) {
            s += qd_s[0][r][part * NP + e] * kv_[e];
            dp += qd_s[1][r][part * NP + e] * vv_[e];
          }
          s = sum16(s);
          dp = sum16(dp);
          if (!pair_allowed(p, b, qb, kb, cls, i, j, __float_as_int(row_s[2][r]), __float_as_int(row_s[3][r])))
            continue;
          float pw, ds;
          pair_grads(p, s, dp, row_s[0][r], row_s[1][r], pw, ds);
#pragma unroll
          for (int e = 0; e < NP; ++e) {
            dvv[e] += pw * qd_s[1][r][part * NP + e];
            dk[e] += ds * qd_s[0][r][part * NP + e];
          }
        }
      }
    }
  }
  if (!key_ok) return;
  const float scale = p.scale_log2 * kLn2;
  const int64_t o = (int64_t)b * bp.dkv_stride_b + ((int64_t)j * p.Hkv + g) * D + part * NP;
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    bp.dk[o + e] = dk[e] * scale;
    bp.dv[o + e] = dvv[e];
  }
}

template <int D>
hipError_t launch_f32(const BwdParams& p, hipStream_t s) {
  const AttnParams& a = p.a;
  const int64_t q_items = (int64_t)a.B * a.H * a.nQb * (kBlockQ / kRowsPerWg);
  const int64_t kv_items = (int64_t)a.B * a.Hkv * a.nKb * (kBlockKV / kRowsPerWg);
  if (q_items > 0) {
    hipLaunchKernelGGL(bwd_dq_f32<D>, dim3((unsigned)q_items), dim3(256), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (kv_items > 0) {
    hipLaunchKernelGGL(bwd_dkv_f32<D>, dim3((unsigned)kv_items), dim3(256), 0, s, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_attn_bwd_f32(const BwdParams& p, hipStream_t s) {
  return p.a.D == 64 ? launch_f32<64>(p, s) : launch_f32<128>(p, s);
}

}  // namespace ram
