// C ABI of libram: host-side validation, launches and the one-GPU ring loop.
//
// Every entry point checks all of its arguments before it enqueues anything
// (the ring-splash page likewise raises before any compute), so on a non-OK
// status no kernel ran and no output changed.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include <hip/hip_runtime_api.h>

#include "../../include/ram.h"
#include "ram_internal.h"

namespace {

thread_local std::string g_err;
// Events the rings record around their attention launches (ram_set_kernel_events).
thread_local hipEvent_t g_ev_start = nullptr, g_ev_stop = nullptr;

ram_status fail(ram_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

ram_status ok() {
  g_err.clear();
  return RAM_OK;
}

ram_status hip_fail(hipError_t e, const char* what) {
  return fail(RAM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr int64_t kMaxSeq = int64_t(1) << 30;
constexpr int32_t kMaxGridYZ = 65535;
constexpr int kMaxHeads = 1 << 16;

// Which tile a call needs its block masks at.
enum TileUse { kMaskTile = 0, kFwdTile = 1, kBwdTile = 2 };

// Checks the fields every call reads. kFwdTile / kBwdTile also require the
// forward / backward kernels' mask tile; kMaskTile only the builder's limits.
ram_status check_desc(const ram_attn_desc* d, TileUse tile, bool need_heads) {
  if (!d) return fail(RAM_ERR_INVALID, "desc is null");
  if (d->B < 0 || d->Sq < 0 || d->Skv < 0)
    return fail(RAM_ERR_INVALID, "negative size: B=%d Sq=%d Skv=%d", d->B, d->Sq, d->Skv);
  if (d->Sq > kMaxSeq || d->Skv > kMaxSeq)
    return fail(RAM_ERR_INVALID, "sequence too long: Sq=%d Skv=%d", d->Sq, d->Skv);
  if (d->causal != 0 && d->causal != 1) return fail(RAM_ERR_INVALID, "causal must be 0 or 1");
  if (need_heads) {
    if (d->H < 1 || d->Hkv < 1) return fail(RAM_ERR_INVALID, "H=%d Hkv=%d must be >= 1", d->H, d->Hkv);
    if (d->H % d->Hkv) return fail(RAM_ERR_INVALID, "H=%d is not a multiple of Hkv=%d", d->H, d->Hkv);
    // K/V tiles are read through 32-bit buffer offsets: one tile of key rows
    // (64 x Hkv x D elements) must stay well inside 4 GiB.
    if (d->H > kMaxHeads) return fail(RAM_ERR_UNSUPPORTED, "H=%d above %d", d->H, kMaxHeads);
    if (d->D != 64 && d->D != 128) return fail(RAM_ERR_UNSUPPORTED, "head dim D=%d (built: 64, 128)", d->D);
    if (d->dtype != RAM_F32 && d->dtype != RAM_BF16) return fail(RAM_ERR_UNSUPPORTED, "dtype %d", d->dtype);
    if (!std::isfinite(d->scale) || !(d->scale > 0.0f))
      return fail(RAM_ERR_INVALID, "scale must be finite and > 0");
    if (!std::isfinite(d->softcap)) return fail(RAM_ERR_INVALID, "softcap must be finite");
    const int64_t esz = d->dtype == RAM_BF16 ? 2 : 4;
    const int64_t qmin = (int64_t)d->Sq * d->H * d->D;
    if (d->q_stride_b != 0 && (d->q_stride_b < qmin || (d->q_stride_b * esz) % 16))
      return fail(RAM_ERR_INVALID, "q_stride_b=%lld (>= %lld, 16-byte multiple)", (long long)d->q_stride_b,
                  (long long)qmin);
  }
  if (tile != kMaskTile) {
    const int bq = tile == kFwdTile ? ram::fwd_block_q(d->dtype, d->D) : ram::kBlockQ;
    if (d->block_q != bq || d->block_kv != ram::kBlockKV)
      return fail(RAM_ERR_INVALID, "block mask tile %dx%d differs from the kernel tile %dx%d", d->block_q,
                  d->block_kv, bq, ram::kBlockKV);
  } else {
    if (d->block_q < 16 || d->block_q > ram::kMaxMaskTile || d->block_kv < 16 || d->block_kv > ram::kMaxMaskTile)
      return fail(RAM_ERR_INVALID, "tile %dx%d outside [16, %d]", d->block_q, d->block_kv, ram::kMaxMaskTile);
  }
  if (cdiv(d->Skv, d->block_kv) > ram::kMaxMaskCols)
    return fail(RAM_ERR_UNSUPPORTED, "more than %d kv tiles in a row", ram::kMaxMaskCols);
  // the bf16 D = 128 forward reads a chunk's key rows (of one batch) through 32-bit byte offsets
  if (tile == kFwdTile && need_heads && d->dtype == RAM_BF16 && d->D == 128 &&
      (int64_t)d->Skv * d->Hkv * d->D * 2 > (int64_t)UINT32_MAX)
    return fail(RAM_ERR_UNSUPPORTED, "one KV chunk of Skv=%d x Hkv=%d rows spans 4 GiB or more", d->Skv, d->Hkv);
  return RAM_OK;
}

ram_status check_kv_stride(const ram_attn_desc* d, int64_t keys) {
  const int64_t esz = d->dtype == RAM_BF16 ? 2 : 4;
  const int64_t kmin = keys * d->Hkv * d->D;
  if (d->kv_stride_b != 0 && (d->kv_stride_b < kmin || (d->kv_stride_b * esz) % 16))
    return fail(RAM_ERR_INVALID, "kv_stride_b=%lld (>= %lld, 16-byte multiple)", (long long)d->kv_stride_b,
                (long long)kmin);
  return RAM_OK;
}

// Positions / segments of one call whose KV spans `kv_len` keys; a dense mask
// is read over `dense_cols` columns per row.
ram_status check_src(const ram_mask_src* m, const ram_attn_desc* d, int64_t kv_len, int64_t q_base_extra,
                     int64_t dense_cols) {
  if (!m) return fail(RAM_ERR_INVALID, "mask source is null");
  if (m->dense) {
    if (m->dense_chunk_step < 0) return fail(RAM_ERR_INVALID, "dense_chunk_step=%lld < 0", (long long)m->dense_chunk_step);
    if (m->dense_ld != 0 && m->dense_ld < dense_cols)
      return fail(RAM_ERR_INVALID, "dense_ld=%lld < %lld columns read", (long long)m->dense_ld, (long long)dense_cols);
  }
  if ((m->q_seg == nullptr) != (m->kv_seg == nullptr))
    return fail(RAM_ERR_INVALID, "q_seg and kv_seg must both be set or both be null");
  if (m->q_meta_stride_b != 0 && m->q_meta_stride_b < d->Sq)
    return fail(RAM_ERR_INVALID, "q_meta_stride_b=%lld < Sq", (long long)m->q_meta_stride_b);
  if (m->kv_meta_stride_b != 0 && m->kv_meta_stride_b < kv_len)
    return fail(RAM_ERR_INVALID, "kv_meta_stride_b=%lld < %lld", (long long)m->kv_meta_stride_b, (long long)kv_len);
  const void* arrs[4] = {m->q_pos, m->kv_pos, m->q_seg, m->kv_seg};
  for (const void* a : arrs)
    if (a && !aligned(a, 4)) return fail(RAM_ERR_INVALID, "position / segment arrays must be 4-byte aligned");
  if (!m->q_pos) {
    const int64_t hi = (int64_t)m->q_pos_base + q_base_extra + d->Sq;
    if (hi > INT32_MAX || (int64_t)m->q_pos_base + q_base_extra < INT32_MIN)
      return fail(RAM_ERR_INVALID, "sequential q positions overflow int32");
  }
  if (!m->kv_pos) {
    const int64_t hi = (int64_t)m->kv_pos_base + kv_len;
    if (hi > INT32_MAX || m->kv_pos_base < INT32_MIN / 2)
      return fail(RAM_ERR_INVALID, "sequential kv positions overflow int32");
  }
  return RAM_OK;
}

ram_status check_mask_arrays(const ram_block_mask* bm, const ram_attn_desc* d, bool need_bits) {
  if (!bm) return fail(RAM_ERR_INVALID, "block mask is null");
  if (bm->bits && !aligned(bm->bits, 8)) return fail(RAM_ERR_INVALID, "bits not 8-byte aligned");
  if (need_bits && !bm->bits && cdiv(d->Skv, d->block_kv) > 0)
    return fail(RAM_ERR_INVALID, "a dense mask needs the tile bits (block mask bits is null)");
  const int64_t rows = (int64_t)d->B * cdiv(d->Sq, d->block_q);
  if (rows == 0) return RAM_OK;
  if (!bm->row_cnt || !aligned(bm->row_cnt, 4)) return fail(RAM_ERR_INVALID, "row_cnt null or misaligned");
  if (cdiv(d->Skv, d->block_kv) > 0) {
    if (!bm->tile_class) return fail(RAM_ERR_INVALID, "tile_class is null");
    if (!bm->col_idx || !aligned(bm->col_idx, 4)) return fail(RAM_ERR_INVALID, "col_idx null or misaligned");
  }
  return RAM_OK;
}

ram_status check_col_lists(const ram_block_mask* bm, const ram_attn_desc* d, bool need) {
  if ((bm->col_cnt == nullptr) != (bm->row_idx == nullptr))
    return fail(RAM_ERR_INVALID, "col_cnt and row_idx must both be set or both be null");
  if (bm->col_cnt && (!aligned(bm->col_cnt, 4) || !aligned(bm->row_idx, 4)))
    return fail(RAM_ERR_INVALID, "col_cnt / row_idx misaligned");
  if (need && !bm->col_cnt && (int64_t)d->B * cdiv(d->Skv, d->block_kv) > 0)
    return fail(RAM_ERR_INVALID, "the backward needs the transposed lists (col_cnt, row_idx)");
  return RAM_OK;
}

// What the backward kernels are built for.
ram_status check_bwd_support(const ram_attn_desc* d) {
  if (d->dtype != RAM_BF16 && d->dtype != RAM_F32)
    return fail(RAM_ERR_UNSUPPORTED, "backward dtype %d (built: bf16, float32)", d->dtype);
  if (d->D != 128 && d->D != 64) return fail(RAM_ERR_UNSUPPORTED, "backward head dim D=%d (built: 64, 128)", d->D);
  return RAM_OK;
}

ram_status check_tensor(const void* p, const char* name) {
  if (!p) return fail(RAM_ERR_INVALID, "%s is null", name);
  if (!aligned(p, 16)) return fail(RAM_ERR_UNSUPPORTED, "%s is not 16-byte aligned", name);
  return RAM_OK;
}

#define RAM_TRY(x)                      \
  do {                                  \
    ram_status _s = (x);                \
    if (_s != RAM_OK) return _s;        \
  } while (0)

ram::MaskParams mask_params(const ram_attn_desc* d, const ram_mask_src* m, const ram_block_mask* bm,
                            int64_t dense_cols) {
  ram::MaskParams p{};
  p.dense = m->dense;
  p.dense_ld = m->dense_ld ? m->dense_ld : dense_cols;
  p.dense_col_step = 0;
  p.bits = bm->bits;
  p.q_pos = m->q_pos;
  p.kv_pos = m->kv_pos;
  p.q_seg = m->q_seg;
  p.kv_seg = m->kv_seg;
  p.qm_stride_b = m->q_meta_stride_b ? m->q_meta_stride_b : d->Sq;
  p.kvm_stride_b = m->kv_meta_stride_b ? m->kv_meta_stride_b : d->Skv;
  p.kv_chunk_off = 0;
  p.q_pos_base = m->q_pos_base;
  p.kv_pos_base = m->kv_pos_base;
  p.kv_base_step = 0;
  p.B = d->B;
  p.Sq = d->Sq;
  p.Skv = d->Skv;
  p.bq = d->block_q;
  p.bk = d->block_kv;
  p.nQb = (int)cdiv(d->Sq, d->block_q);
  p.nKb = (int)cdiv(d->Skv, d->block_kv);
  p.causal = d->causal;
  p.tile_class = bm->tile_class;
  p.row_cnt = bm->row_cnt;
  p.col_idx = bm->col_idx;
  return p;
}

ram::AttnParams attn_params(const ram_attn_desc* d, const void* q, const void* k, const void* v,
                            const ram_mask_src* m, const ram_block_mask* bm, const float* sinks, int mode,
                            float* out, float* lse, int block_q) {
  ram::AttnParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.out = out;
  p.lse = lse;
  p.sinks = sinks;
  p.tile_class = bm->tile_class;
  p.row_cnt = bm->row_cnt;
  p.col_idx = bm->col_idx;
  p.mask_bits = bm->bits;
  p.q_pos = m->q_pos;
  p.kv_pos = m->kv_pos;
  p.q_seg = m->q_seg;
  p.kv_seg = m->kv_seg;
  p.q_stride_b = d->q_stride_b ? d->q_stride_b : (int64_t)d->Sq * d->H * d->D;
  p.kv_stride_b = d->kv_stride_b ? d->kv_stride_b : (int64_t)d->Skv * d->Hkv * d->D;
  p.qm_stride_b = m->q_meta_stride_b ? m->q_meta_stride_b : d->Sq;
  p.kvm_stride_b = m->kv_meta_stride_b ? m->kv_meta_stride_b : d->Skv;
  p.q_pos_base = m->q_pos_base;
  p.kv_pos_base = m->kv_pos_base;
  p.B = d->B;
  p.Sq = d->Sq;
  p.Skv = d->Skv;
  p.H = d->H;
  p.Hkv = d->Hkv;
  p.D = d->D;
  p.nQb = (int)cdiv(d->Sq, block_q);
  p.nKb = (int)cdiv(d->Skv, ram::kBlockKV);
  p.tile_words = block_q * (ram::kBlockKV / 32);
  const float log2e = 1.4426950408889634f;
  p.scale_log2 = d->scale * log2e;
  p.softcap_on = d->softcap > 0.0f;
  p.cap_k2 = p.softcap_on ? 2.0f * d->scale * log2e / d->softcap : 0.0f;
  p.cap_log2 = p.softcap_on ? d->softcap * log2e : 0.0f;
  p.causal = d->causal;
  p.mode = mode;
  return p;
}

struct RingLayout {
  size_t acc_off, cls_off, cnt_off, col_off, bits_off, order_off, acc2_off, lse2_off, vt_off, total;
};

// The bf16 kernel for D = 128 runs a whole ring in one launch; the others run one chunk per launch.
bool alt_kernel(const ram_attn_desc* d) { return d->dtype == RAM_BF16 && d->D == 128; }

// Whether a forward call's PARTIAL tiles are masked from tile bits: always with a dense mask,
// and in the bf16 D = 128 kernel also with key positions or segment IDs (its only other mask is
// the positional one).
bool fwd_needs_bits(const ram_attn_desc* d, const ram_mask_src* m) {
  return m && (m->dense || (alt_kernel(d) && (m->kv_pos || m->kv_seg || m->q_seg)));
}

// Workgroups of the bf16 D = 128 kernel one launch should have: two per CU (256 CUs).
constexpr int64_t kAltFill = 512;

// Whether the one-launch ring splits each row of q tiles' visits over two workgroups: when its
// rows give fewer workgroups than CUs, two halves of the ring run side by side and their
// results are merged afterwards (this changes the merge order, so the result differs from
// chunk-by-chunk calls in rounding).
bool ring_split_shape(const ram_attn_desc* d, int32_t n_chunks) {
  return alt_kernel(d) && n_chunks >= 2 && (int64_t)d->B * d->H * cdiv(d->Sq, ram::kAltRows) < kAltFill;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Whether the one-launch ring reads V repacked for row reads (ram::launch_pack_v). The repack
// reads and writes V once (2 bytes read and written per element); it saves about 3% of the
// kernel's time, whose work per V element grows with the query rows that attend a key times the
// query heads per kv head. It pays when that product is in the tens of thousands, which
// Sq * (H / Hkv) >= 32768 stands for (half of it for a causal ring). Not with a soft cap: that
// kernel is bound by its vector arithmetic, not its LDS reads.
constexpr int64_t kPackMinRowsPerKey = 32768;
bool ring_packs_v(const ram_attn_desc* d) {
  return alt_kernel(d) && !(d->softcap > 0.0f) && d->Skv > 0 &&
         (int64_t)d->Sq * (d->H / d->Hkv) >= kPackMinRowsPerKey;
}

// Words of tile bits per backward mask tile (block_q rows of block_kv / 32 words).
constexpr int64_t kBwdTileWords = (int64_t)ram::kBlockQ * (ram::kBlockKV / 32);

// Whether the one-launch ring takes its rows of q tiles most tiles first (an order it sorts on the
// GPU): when positions, segment IDs or a dense mask make a row's work unrelated to its index. With
// sequential positions the natural order (last q tile first) already is.
bool ring_row_order(const ram_attn_desc* d, const ram_mask_src* m) {
  return alt_kernel(d) && m && (m->q_pos || m->kv_pos || m->q_seg || m->kv_seg || m->dense);
}

RingLayout ring_layout(const ram_attn_desc* d, int32_t n_chunks, bool with_bits, bool with_order) {
  RingLayout L{};
  const int bq = ram::fwd_block_q(d->dtype, d->D);
  const int64_t nQb = cdiv(d->Sq, bq), nKb = cdiv(d->Skv, ram::kBlockKV);
  const int64_t tiles = (int64_t)n_chunks * d->B * nQb * nKb;
  const int64_t rows = (int64_t)n_chunks * d->B * nQb;
  size_t off = 0;
  L.acc_off = off;
  if (d->dtype == RAM_BF16) off += align256((size_t)d->B * d->Sq * d->H * d->D * sizeof(float));
  L.cls_off = off;
  off += align256((size_t)tiles);
  L.cnt_off = off;
  off += align256((size_t)rows * sizeof(int32_t));
  L.col_off = off;
  off += align256((size_t)tiles * sizeof(int32_t));
  L.bits_off = off;
  if (with_bits) off += align256((size_t)tiles * bq * (ram::kBlockKV / 32) * sizeof(uint32_t));
  L.order_off = off;
  if (with_order) off += align256((size_t)d->B * nQb * sizeof(int32_t));
  const bool split = ring_split_shape(d, n_chunks);
  L.acc2_off = off;
  if (split) off += align256((size_t)d->B * d->Sq * d->H * d->D * sizeof(float));
  L.lse2_off = off;
  if (split) off += align256((size_t)d->B * d->H * d->Sq * sizeof(float));
  // the one-launch ring reads V repacked for row reads (ram::launch_pack_v)
  L.vt_off = off;
  if (ring_packs_v(d)) off += align256(ram::pack_v_bytes(d->B, n_chunks, d->Skv, d->Hkv));
  L.total = off;
  return L;
}

// How many workgroups share the heads of a KV group in the ring's dk / dv launches: enough that a
// chunk's launch has 512 of them (two per CU), within the group size. Only the bf16 kernels split.
int bwd_head_split(const ram_attn_desc* d) {
  if (d->dtype != RAM_BF16) return 1;
  const int G = d->H / d->Hkv;
  const int64_t items = (int64_t)d->B * d->Hkv * cdiv(d->Skv, ram::kBlockKV);
  int S = 1;
  while (items * S < 512 && G % (2 * S) == 0) S *= 2;
  return S;
}

struct BwdLayout {
  size_t dq_off, dk_off, dv_off, delta_off, cls_off, cnt_off, col_off, bits_off, ccnt_off, ridx_off, kpart_off,
      vpart_off, total;
};
BwdLayout bwd_layout(const ram_attn_desc* d, int32_t n_chunks, bool with_bits) {
  BwdLayout L{};
  const int64_t nQb = cdiv(d->Sq, ram::kBlockQ), nKb = cdiv(d->Skv, ram::kBlockKV);
  const int64_t tiles = (int64_t)n_chunks * d->B * nQb * nKb;
  const int64_t kv_elems = (int64_t)d->B * n_chunks * d->Skv * d->Hkv * d->D;
  size_t off = 0;
  auto take = [&](size_t& at, size_t bytes) {
    at = off;
    off += align256(bytes);
  };
  take(L.dq_off, (size_t)d->B * d->Sq * d->H * d->D * sizeof(float));
  take(L.dk_off, (size_t)kv_elems * sizeof(float));
  take(L.dv_off, (size_t)kv_elems * sizeof(float));
  take(L.delta_off, (size_t)2 * d->B * d->H * d->Sq * sizeof(float));
  take(L.cls_off, (size_t)tiles);
  take(L.cnt_off, (size_t)n_chunks * d->B * nQb * sizeof(int32_t));
  take(L.col_off, (size_t)tiles * sizeof(int32_t));
  take(L.bits_off, with_bits ? (size_t)tiles * kBwdTileWords * sizeof(uint32_t) : 0);
  take(L.ccnt_off, (size_t)n_chunks * d->B * nKb * sizeof(int32_t));
  take(L.ridx_off, (size_t)tiles * sizeof(int32_t));
  // one chunk's partial dk / dv per head split (reused by every chunk)
  const int S = bwd_head_split(d);
  const size_t part = S > 1 ? (size_t)S * d->B * d->Skv * d->Hkv * d->D * sizeof(float) : 0;
  take(L.kpart_off, part);
  take(L.vpart_off, part);
  L.total = off;
  return L;
}

}  // namespace

namespace ram {
ram_status api_fail(ram_status s, const char* msg) { return fail(s, "%s", msg); }
}  // namespace ram

extern "C" {

const char* ram_last_error(void) { return g_err.c_str(); }

ram_status ram_set_kernel_events(hipEvent_t start, hipEvent_t stop) {
  if ((start == nullptr) != (stop == nullptr)) return fail(RAM_ERR_INVALID, "set both events or neither");
  g_ev_start = start;
  g_ev_stop = stop;
  return ok();
}

ram_status ram_kernel_tile(int32_t dtype, int32_t D, int32_t* block_q, int32_t* block_kv) {
  if (!block_q || !block_kv) return fail(RAM_ERR_INVALID, "null output pointer");
  if (dtype != RAM_F32 && dtype != RAM_BF16) return fail(RAM_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (D != 64 && D != 128) return fail(RAM_ERR_UNSUPPORTED, "head dim D=%d (built: 64, 128)", D);
  *block_q = ram::fwd_block_q(dtype, D);
  *block_kv = ram::kBlockKV;
  return ok();
}

ram_status ram_bwd_kernel_tile(int32_t dtype, int32_t D, int32_t* block_q, int32_t* block_kv) {
  if (!block_q || !block_kv) return fail(RAM_ERR_INVALID, "null output pointer");
  if (dtype != RAM_F32 && dtype != RAM_BF16) return fail(RAM_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (D != 64 && D != 128) return fail(RAM_ERR_UNSUPPORTED, "head dim D=%d (built: 64, 128)", D);
  *block_q = ram::kBlockQ;
  *block_kv = ram::kBlockKV;
  return ok();
}

ram_status build_block_mask(const ram_attn_desc* desc, const ram_mask_src* src, const ram_block_mask* out,
                            hipStream_t stream) {
  RAM_TRY(check_desc(desc, kMaskTile, false));
  RAM_TRY(check_src(src, desc, desc->Skv, 0, desc->Skv));
  RAM_TRY(check_mask_arrays(out, desc, false));
  RAM_TRY(check_col_lists(out, desc, false));
  if (desc->B == 0 || desc->Sq == 0) return ok();
  ram::MaskParams p = mask_params(desc, src, out, desc->Skv);
  hipError_t e = ram::launch_block_mask(p, 1, stream);
  if (e != hipSuccess) return hip_fail(e, "build_block_mask launch");
  if (out->col_cnt) {
    e = ram::launch_col_lists(p, 1, out->col_cnt, out->row_idx, stream);
    if (e != hipSuccess) return hip_fail(e, "build_block_mask transposed lists launch");
  }
  return ok();
}

ram_status attn_fwd_chunk(const ram_attn_desc* desc, const void* q, const void* k, const void* v,
                          const ram_mask_src* src, const ram_block_mask* mask, const float* sinks, int32_t mode,
                          float* out, float* lse, hipStream_t stream) {
  RAM_TRY(check_desc(desc, kFwdTile, true));
  RAM_TRY(check_kv_stride(desc, desc->Skv));
  RAM_TRY(check_src(src, desc, desc->Skv, 0, desc->Skv));
  const bool need_bits = fwd_needs_bits(desc, src);
  if (need_bits && !mask->bits && cdiv(desc->Skv, desc->block_kv) > 0 && !src->dense)
    return fail(RAM_ERR_INVALID, "with key positions or segment IDs this kernel masks PARTIAL tiles from their bits: "
                                 "build the block mask with bits");
  RAM_TRY(check_mask_arrays(mask, desc, need_bits));
  if (mode != RAM_OUT_WRITE && mode != RAM_OUT_MERGE) return fail(RAM_ERR_INVALID, "mode %d", mode);
  if (desc->B == 0 || desc->Sq == 0) return ok();
  RAM_TRY(check_tensor(q, "q"));
  if (desc->Skv > 0) {
    RAM_TRY(check_tensor(k, "k"));
    RAM_TRY(check_tensor(v, "v"));
  }
  RAM_TRY(check_tensor(out, "out"));
  if (!lse || !aligned(lse, 4)) return fail(RAM_ERR_INVALID, "lse null or misaligned");
  if (sinks && !aligned(sinks, 4)) return fail(RAM_ERR_INVALID, "sinks misaligned");
  ram::AttnParams p = attn_params(desc, q, k, v, src, mask, sinks, mode, out, lse, desc->block_q);
  hipError_t e;
  if (alt_kernel(desc)) {
    p.n_chunks = 1;
    p.ring_shard = -1;
    if (!need_bits) p.mask_bits = nullptr;
    e = ram::launch_attn_alt(p, nullptr, stream);
  } else {
    e = ram::launch_attn(p, desc->dtype, stream);
  }
  if (e != hipSuccess) return hip_fail(e, "attn_fwd_chunk launch");
  return ok();
}

ram_status lse_merge(int32_t B, int32_t Sq, int32_t H, int32_t D, float* out_acc, float* lse_acc,
                     const float* out_blk, const float* lse_blk, hipStream_t stream) {
  if (B < 0 || Sq < 0 || H < 0) return fail(RAM_ERR_INVALID, "negative size");
  if (D != 64 && D != 128) return fail(RAM_ERR_UNSUPPORTED, "head dim D=%d (built: 64, 128)", D);
  if ((int64_t)B * Sq * H == 0) return ok();
  RAM_TRY(check_tensor(out_acc, "out_acc"));
  RAM_TRY(check_tensor(out_blk, "out_blk"));
  if (!lse_acc || !lse_blk || !aligned(lse_acc, 4) || !aligned(lse_blk, 4))
    return fail(RAM_ERR_INVALID, "lse null or misaligned");
  if (out_acc == out_blk) return fail(RAM_ERR_INVALID, "out_blk aliases out_acc");
  hipError_t e = ram::launch_merge(B, Sq, H, D, out_acc, lse_acc, out_blk, lse_blk, stream);
  if (e != hipSuccess) return hip_fail(e, "lse_merge launch");
  return ok();
}

size_t ring_attn_workspace_bytes(const ram_attn_desc* desc, int32_t n_chunks, const ram_mask_src* src) {
  if (!desc || n_chunks < 1 || desc->B < 0 || desc->Sq < 0 || desc->Skv < 0 || desc->H < 1 ||
      (desc->D != 64 && desc->D != 128))
    return 0;
  ram_attn_desc dt = *desc;
  dt.block_q = ram::fwd_block_q(desc->dtype, desc->D);
  dt.block_kv = ram::kBlockKV;
  return ring_layout(&dt, n_chunks, fwd_needs_bits(&dt, src), ring_row_order(&dt, src)).total;
}

ram_status ring_attn_fwd_masks(const ram_attn_desc* desc, int32_t n_chunks, const ram_mask_src* src,
                               ram_ring_masks* out) {
  if (!desc || !out) return fail(RAM_ERR_INVALID, "desc or out is null");
  ram_attn_desc dt = *desc;
  dt.block_q = ram::fwd_block_q(desc->dtype, desc->D);
  dt.block_kv = ram::kBlockKV;
  RAM_TRY(check_desc(&dt, kFwdTile, true));
  if (n_chunks < 1) return fail(RAM_ERR_INVALID, "n_chunks=%d must be >= 1", n_chunks);
  // the rings' per-chunk launches put batch rows and chunks in the grid's y and z (at most 65535)
  if (n_chunks > kMaxGridYZ || desc->B > kMaxGridYZ)
    return fail(RAM_ERR_UNSUPPORTED, "n_chunks=%d or B=%d above %d", n_chunks, desc->B, kMaxGridYZ);
  const bool with_bits = fwd_needs_bits(&dt, src);
  const bool with_order = ring_row_order(&dt, src);
  const RingLayout L = ring_layout(&dt, n_chunks, with_bits, with_order);
  out->cls_off = (int64_t)L.cls_off;
  out->cnt_off = (int64_t)L.cnt_off;
  out->col_off = (int64_t)L.col_off;
  out->bits_off = with_bits ? (int64_t)L.bits_off : -1;
  out->order_off = with_order ? (int64_t)L.order_off : -1;
  out->block_q = dt.block_q;
  out->block_kv = dt.block_kv;
  out->nQb = (int32_t)cdiv(dt.Sq, dt.block_q);
  out->nKb = (int32_t)cdiv(dt.Skv, dt.block_kv);
  out->tile_words = dt.block_q * (dt.block_kv / 32);
  return ok();
}

ram_status ring_attn_bwd_masks(const ram_attn_desc* desc, int32_t n_chunks, const ram_mask_src* src,
                               ram_ring_masks* out) {
  if (!desc || !out) return fail(RAM_ERR_INVALID, "desc or out is null");
  ram_attn_desc dt = *desc;
  dt.block_q = ram::kBlockQ;
  dt.block_kv = ram::kBlockKV;
  RAM_TRY(check_desc(&dt, kBwdTile, true));
  if (n_chunks < 1) return fail(RAM_ERR_INVALID, "n_chunks=%d must be >= 1", n_chunks);
  // the rings' per-chunk launches put batch rows and chunks in the grid's y and z (at most 65535)
  if (n_chunks > kMaxGridYZ || desc->B > kMaxGridYZ)
    return fail(RAM_ERR_UNSUPPORTED, "n_chunks=%d or B=%d above %d", n_chunks, desc->B, kMaxGridYZ);
  const bool with_bits = src && src->dense;
  const BwdLayout L = bwd_layout(&dt, n_chunks, with_bits);
  out->cls_off = (int64_t)L.cls_off;
  out->cnt_off = (int64_t)L.cnt_off;
  out->col_off = (int64_t)L.col_off;
  out->bits_off = with_bits ? (int64_t)L.bits_off : -1;
  out->order_off = -1;
  out->block_q = dt.block_q;
  out->block_kv = dt.block_kv;
  out->nQb = (int32_t)cdiv(dt.Sq, dt.block_q);
  out->nKb = (int32_t)cdiv(dt.Skv, dt.block_kv);
  out->tile_words = (int32_t)kBwdTileWords;
  return ok();
}

ram_status ring_attn_fwd_1gpu(const ram_attn_desc* desc, int32_t n_chunks, int32_t q_shard, const void* q,
                              const void* k_all, const void* v_all, const ram_mask_src* src, const float* sinks,
                              void* out, float* lse, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  if (!desc) return fail(RAM_ERR_INVALID, "desc is null");
  ram_attn_desc dt = *desc;  // the ring builds its own masks at the kernel tile
  dt.block_q = ram::fwd_block_q(desc->dtype, desc->D);
  dt.block_kv = ram::kBlockKV;
  desc = &dt;
  RAM_TRY(check_desc(desc, kFwdTile, true));
  if (n_chunks < 1) return fail(RAM_ERR_INVALID, "n_chunks=%d must be >= 1", n_chunks);
  // the rings' per-chunk launches put batch rows and chunks in the grid's y and z (at most 65535)
  if (n_chunks > kMaxGridYZ || desc->B > kMaxGridYZ)
    return fail(RAM_ERR_UNSUPPORTED, "n_chunks=%d or B=%d above %d", n_chunks, desc->B, kMaxGridYZ);
  if (q_shard < -1 || q_shard >= n_chunks)
    return fail(RAM_ERR_INVALID, "q_shard=%d outside [-1, %d)", q_shard, n_chunks);
  const int64_t kv_total = (int64_t)n_chunks * desc->Skv;
  if (kv_total > kMaxSeq) return fail(RAM_ERR_INVALID, "total KV too long");
  RAM_TRY(check_kv_stride(desc, kv_total));
  const int64_t q_extra = q_shard >= 0 ? (int64_t)q_shard * desc->Sq : 0;
  if (!src) return fail(RAM_ERR_INVALID, "mask source is null");
  const int64_t dense_cols = desc->Skv + (int64_t)(n_chunks - 1) * (src->dense ? src->dense_chunk_step : 0);
  RAM_TRY(check_src(src, desc, kv_total, q_extra, dense_cols));
  if (desc->B == 0 || desc->Sq == 0) return ok();
  RAM_TRY(check_tensor(q, "q"));
  if (desc->Skv > 0) {
    RAM_TRY(check_tensor(k_all, "k_all"));
    RAM_TRY(check_tensor(v_all, "v_all"));
  }
  RAM_TRY(check_tensor(out, "out"));
  if (!lse || !aligned(lse, 4)) return fail(RAM_ERR_INVALID, "lse null or misaligned");
  if (sinks && !aligned(sinks, 4)) return fail(RAM_ERR_INVALID, "sinks misaligned");
  const bool with_bits = fwd_needs_bits(desc, src);
  const bool with_order = ring_row_order(desc, src);
  const RingLayout L = ring_layout(desc, n_chunks, with_bits, with_order);
  if (!workspace || !aligned(workspace, 256))
    return fail(RAM_ERR_WORKSPACE, "workspace null or not 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(RAM_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, L.total);

  char* ws = static_cast<char*>(workspace);
  ram_block_mask bm{reinterpret_cast<uint8_t*>(ws + L.cls_off), reinterpret_cast<int32_t*>(ws + L.cnt_off),
                    reinterpret_cast<int32_t*>(ws + L.col_off),
                    with_bits ? reinterpret_cast<uint32_t*>(ws + L.bits_off) : nullptr};
  float* acc = desc->dtype == RAM_BF16 ? reinterpret_cast<float*>(ws + L.acc_off) : static_cast<float*>(out);
  const int64_t nQb = cdiv(desc->Sq, desc->block_q), nKb = cdiv(desc->Skv, ram::kBlockKV);
  const int64_t tile_words = (int64_t)desc->block_q * (ram::kBlockKV / 32);
  const int64_t kv_full_stride = desc->kv_stride_b ? desc->kv_stride_b : kv_total * desc->Hkv * desc->D;
  const int64_t kvm_full = src->kv_meta_stride_b ? src->kv_meta_stride_b : kv_total;
  const int32_t q_base = (int32_t)(src->q_pos_base + q_extra);

  // Block masks of every chunk in one launch (chunk c in blockIdx.z).
  ram_attn_desc dm = *desc;
  ram_mask_src sm = *src;
  sm.q_pos_base = q_base;
  sm.kv_meta_stride_b = kvm_full;
  ram::MaskParams mp = mask_params(&dm, &sm, &bm, dense_cols);
  mp.kv_chunk_off = desc->Skv;
  mp.kv_base_step = desc->Skv;
  mp.dense_col_step = src->dense_chunk_step;
  hipError_t e = ram::launch_block_mask(mp, n_chunks, stream);
  if (e != hipSuccess) return hip_fail(e, "ring block mask launch");

  const int64_t esz = desc->dtype == RAM_BF16 ? 2 : 4;
  if (alt_kernel(desc)) {
    // The whole ring as one launch: a workgroup visits every chunk in ring order, each visit
    // exactly a chunk call's work (same tiles, epilogue and merge).
    ram_attn_desc dc = *desc;
    dc.kv_stride_b = kv_full_stride;
    ram_mask_src sc = *src;
    sc.q_pos_base = q_base;
    sc.kv_meta_stride_b = kvm_full;
    ram::AttnParams p = attn_params(&dc, q, k_all, v_all, &sc, &bm, sinks, RAM_OUT_WRITE, acc, lse, desc->block_q);
    p.n_chunks = n_chunks;
    p.ring_shard = q_shard;
    p.kv_chunk_elems = (int64_t)desc->Skv * desc->Hkv * desc->D;
    p.mask_chunk_tiles = (int64_t)desc->B * nQb * nKb;
    p.mask_chunk_rows = (int64_t)desc->B * nQb;
    if (with_order) {
      int32_t* order = reinterpret_cast<int32_t*>(ws + L.order_off);
      e = ram::launch_row_order(bm.row_cnt, n_chunks, (int64_t)desc->B * nQb, (int)nKb, order, stream);
      if (e != hipSuccess) return hip_fail(e, "ring row order launch");
      p.row_order = order;
    }
    const bool split = ring_split_shape(desc, n_chunks);
    float* acc2 = reinterpret_cast<float*>(ws + L.acc2_off);
    float* lse2 = reinterpret_cast<float*>(ws + L.lse2_off);
    const ram::RingSplit halves{acc2, lse2};
    if (!split) p.out_final = out;   // the last visit writes the bf16 result
    if (ring_packs_v(desc)) {
      // V of every chunk repacked so that the kernel reads its operands with row reads
      e = ram::launch_pack_v(v_all, kv_full_stride, desc->B, n_chunks, desc->Skv, desc->Hkv, ws + L.vt_off, stream);
      if (e != hipSuccess) return hip_fail(e, "ring V pack launch");
      p.vt = ws + L.vt_off;
      p.vt_chunk_bytes = (int64_t)ram::pack_v_bytes(desc->B, 1, desc->Skv, desc->Hkv);
    }
    if (g_ev_start && (e = hipEventRecord(g_ev_start, stream)) != hipSuccess) return hip_fail(e, "event record");
    e = ram::launch_attn_alt(p, split ? &halves : nullptr, stream);
    if (e != hipSuccess) return hip_fail(e, "ring launch");
    if (g_ev_stop && (e = hipEventRecord(g_ev_stop, stream)) != hipSuccess) return hip_fail(e, "event record");
    if (split) {
      // the second half's running result merged into the first's, written as the bf16 result
      e = ram::launch_merge(desc->B, desc->Sq, desc->H, desc->D, acc, lse, acc2, lse2, stream, out);
      if (e != hipSuccess) return hip_fail(e, "split ring merge launch");
    }
    return ok();
  }
  // The four-wave kernels: one launch per chunk, in ring order.
  if (g_ev_start && (e = hipEventRecord(g_ev_start, stream)) != hipSuccess) return hip_fail(e, "event record");
  for (int t = 0; t < n_chunks; ++t) {
    const int c = q_shard >= 0 ? ((q_shard - t) % n_chunks + n_chunks) % n_chunks : t;
    ram_attn_desc dc = *desc;
    dc.kv_stride_b = kv_full_stride;
    ram_mask_src sc = *src;
    sc.q_pos_base = q_base;
    sc.kv_meta_stride_b = kvm_full;
    sc.kv_pos = src->kv_pos ? src->kv_pos + (int64_t)c * desc->Skv : nullptr;
    sc.kv_seg = src->kv_seg ? src->kv_seg + (int64_t)c * desc->Skv : nullptr;
    sc.kv_pos_base = src->kv_pos_base + c * desc->Skv;
    const int64_t tiles_c = (int64_t)c * desc->B * nQb * nKb;
    const ram_block_mask bc{bm.tile_class + tiles_c, bm.row_cnt + (int64_t)c * desc->B * nQb,
                            bm.col_idx + tiles_c, with_bits ? bm.bits + tiles_c * tile_words : nullptr};
    const char* kc = static_cast<const char*>(k_all) + (int64_t)c * desc->Skv * desc->Hkv * desc->D * esz;
    const char* vc = static_cast<const char*>(v_all) + (int64_t)c * desc->Skv * desc->Hkv * desc->D * esz;
    ram::AttnParams p = attn_params(&dc, q, kc, vc, &sc, &bc, t == 0 ? sinks : nullptr,
                                    t == 0 ? RAM_OUT_WRITE : RAM_OUT_MERGE, acc, lse, desc->block_q);
    // the last visit writes the bf16 result itself
    if (t == n_chunks - 1 && desc->dtype == RAM_BF16) p.out_final = out;
    e = ram::launch_attn(p, desc->dtype, stream);
    if (e != hipSuccess) return hip_fail(e, "ring chunk launch");
  }
  if (g_ev_stop && (e = hipEventRecord(g_ev_stop, stream)) != hipSuccess) return hip_fail(e, "event record");
  return ok();
}

// ------------------------------------------------------------------------------ backward
ram_status attn_bwd_prep(const ram_attn_desc* desc, const void* out, const void* dout, const float* lse,
                         const float* sinks, float* delta, float* dsinks, hipStream_t stream) {
  if (!desc) return fail(RAM_ERR_INVALID, "desc is null");
  if (desc->B < 0 || desc->Sq < 0) return fail(RAM_ERR_INVALID, "negative size: B=%d Sq=%d", desc->B, desc->Sq);
  if (desc->H < 1 || desc->H > kMaxHeads) return fail(RAM_ERR_INVALID, "H=%d outside [1, %d]", desc->H, kMaxHeads);
  RAM_TRY(check_bwd_support(desc));
  if (desc->B == 0 || desc->Sq == 0) {
    if (!sinks) return ok();
  } else {
    RAM_TRY(check_tensor(out, "out"));
    RAM_TRY(check_tensor(dout, "dout"));
    if (!delta || !aligned(delta, 4)) return fail(RAM_ERR_INVALID, "delta null or misaligned");
  }
  if (!lse && desc->B * (int64_t)desc->Sq > 0) return fail(RAM_ERR_INVALID, "lse is null");
  if (lse && !aligned(lse, 4)) return fail(RAM_ERR_INVALID, "lse misaligned");
  if (sinks && (!aligned(sinks, 4) || !dsinks || !aligned(dsinks, 4)))
    return fail(RAM_ERR_INVALID, "sinks given: dsinks must be set, both 4-byte aligned");
  hipError_t e = ram::launch_bwd_prep(desc->dtype, desc->B, desc->Sq, desc->H, desc->D, out, dout, lse, sinks, delta, dsinks,
                                      stream);
  if (e != hipSuccess) return hip_fail(e, "attn_bwd_prep launch");
  return ok();
}

ram_status attn_bwd_chunk(const ram_attn_desc* desc, const void* q, const void* k, const void* v,
                          const void* dout, const float* lse, const float* delta, const ram_mask_src* src,
                          const ram_block_mask* mask, int32_t dq_mode, float* dq, float* dk, float* dv,
                          hipStream_t stream) {
  RAM_TRY(check_desc(desc, kBwdTile, true));
  RAM_TRY(check_bwd_support(desc));
  RAM_TRY(check_kv_stride(desc, desc->Skv));
  RAM_TRY(check_src(src, desc, desc->Skv, 0, desc->Skv));
  RAM_TRY(check_mask_arrays(mask, desc, src->dense != nullptr));
  RAM_TRY(check_col_lists(mask, desc, true));
  if (dq_mode != RAM_OUT_WRITE && dq_mode != RAM_OUT_MERGE) return fail(RAM_ERR_INVALID, "dq_mode %d", dq_mode);
  if (desc->B == 0) return ok();
  if (desc->Sq > 0) {
    RAM_TRY(check_tensor(q, "q"));
    RAM_TRY(check_tensor(dout, "dout"));
    RAM_TRY(check_tensor(dq, "dq"));
    if (!lse || !aligned(lse, 4) || !delta || !aligned(delta, 4))
      return fail(RAM_ERR_INVALID, "lse / delta null or misaligned");
  }
  if (desc->Skv > 0) {
    RAM_TRY(check_tensor(k, "k"));
    RAM_TRY(check_tensor(v, "v"));
    RAM_TRY(check_tensor(dk, "dk"));
    RAM_TRY(check_tensor(dv, "dv"));
  }
  if (desc->Sq == 0 && desc->Skv == 0) return ok();
  ram::BwdParams bp{};
  bp.a = attn_params(desc, q, k, v, src, mask, nullptr, 0, nullptr, const_cast<float*>(lse), ram::kBlockQ);
  bp.dout = dout;
  bp.delta = delta;
  bp.dq = dq;
  bp.dk = dk;
  bp.dv = dv;
  bp.dkv_stride_b = bp.a.kv_stride_b;
  bp.col_cnt = mask->col_cnt;
  bp.row_idx = mask->row_idx;
  bp.dq_mode = dq_mode;
  bp.head_split = 1;
  hipError_t e = desc->dtype == RAM_F32 ? ram::launch_attn_bwd_f32(bp, stream) : ram::launch_attn_bwd(bp, stream);
  if (e != hipSuccess) return hip_fail(e, "attn_bwd_chunk launch");
  return ok();
}


size_t ring_attn_bwd_workspace_bytes(const ram_attn_desc* desc, int32_t n_chunks, const ram_mask_src* src) {
  if (!desc || n_chunks < 1 || desc->B < 0 || desc->Sq < 0 || desc->Skv < 0 || desc->H < 1 || desc->Hkv < 1 ||
      (desc->D != 64 && desc->D != 128))
    return 0;
  ram_attn_desc dt = *desc;
  dt.block_q = ram::kBlockQ;
  dt.block_kv = ram::kBlockKV;
  return bwd_layout(&dt, n_chunks, src && src->dense).total;
}

ram_status ring_attn_bwd_1gpu(const ram_attn_desc* desc, int32_t n_chunks, int32_t q_shard, const void* q,
                              const void* k_all, const void* v_all, const void* out, const float* lse,
                              const void* dout, const ram_mask_src* src, const float* sinks, void* dq,
                              void* dk_all, void* dv_all, float* dsinks, void* workspace, size_t workspace_bytes,
                              hipStream_t stream) {
  if (!desc) return fail(RAM_ERR_INVALID, "desc is null");
  ram_attn_desc dt = *desc;
  dt.block_q = ram::kBlockQ;
  dt.block_kv = ram::kBlockKV;
  desc = &dt;
  RAM_TRY(check_desc(desc, kBwdTile, true));
  RAM_TRY(check_bwd_support(desc));
  if (n_chunks < 1) return fail(RAM_ERR_INVALID, "n_chunks=%d must be >= 1", n_chunks);
  // the rings' per-chunk launches put batch rows and chunks in the grid's y and z (at most 65535)
  if (n_chunks > kMaxGridYZ || desc->B > kMaxGridYZ)
    return fail(RAM_ERR_UNSUPPORTED, "n_chunks=%d or B=%d above %d", n_chunks, desc->B, kMaxGridYZ);
  if (q_shard < -1 || q_shard >= n_chunks)
    return fail(RAM_ERR_INVALID, "q_shard=%d outside [-1, %d)", q_shard, n_chunks);
  const int64_t kv_total = (int64_t)n_chunks * desc->Skv;
  if (kv_total > kMaxSeq) return fail(RAM_ERR_INVALID, "total KV too long");
  RAM_TRY(check_kv_stride(desc, kv_total));
  const int64_t q_extra = q_shard >= 0 ? (int64_t)q_shard * desc->Sq : 0;
  if (!src) return fail(RAM_ERR_INVALID, "mask source is null");
  const int64_t dense_cols = desc->Skv + (int64_t)(n_chunks - 1) * (src->dense ? src->dense_chunk_step : 0);
  RAM_TRY(check_src(src, desc, kv_total, q_extra, dense_cols));
  if (sinks && (!aligned(sinks, 4) || !dsinks || !aligned(dsinks, 4)))
    return fail(RAM_ERR_INVALID, "sinks given: dsinks must be set, both 4-byte aligned");
  if (desc->B == 0) return ok();
  if (desc->Sq > 0) {
    RAM_TRY(check_tensor(q, "q"));
    RAM_TRY(check_tensor(out, "out"));
    RAM_TRY(check_tensor(dout, "dout"));
    RAM_TRY(check_tensor(dq, "dq"));
    if (!lse || !aligned(lse, 4)) return fail(RAM_ERR_INVALID, "lse null or misaligned");
  }
  if (desc->Skv > 0) {
    RAM_TRY(check_tensor(k_all, "k_all"));
    RAM_TRY(check_tensor(v_all, "v_all"));
    RAM_TRY(check_tensor(dk_all, "dk_all"));
    RAM_TRY(check_tensor(dv_all, "dv_all"));
  }
  const bool with_bits = src->dense != nullptr;
  const BwdLayout L = bwd_layout(desc, n_chunks, with_bits);
  if (!workspace || !aligned(workspace, 256))
    return fail(RAM_ERR_WORKSPACE, "workspace null or not 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(RAM_ERR_WORKSPACE, "workspace of %zu bytes, need %zu", workspace_bytes, L.total);

  char* ws = static_cast<char*>(workspace);
  float* dq_acc = reinterpret_cast<float*>(ws + L.dq_off);
  float* dk_acc = reinterpret_cast<float*>(ws + L.dk_off);
  float* dv_acc = reinterpret_cast<float*>(ws + L.dv_off);
  float* delta = reinterpret_cast<float*>(ws + L.delta_off);
  const int head_split = bwd_head_split(desc);
  float* k_part = reinterpret_cast<float*>(ws + L.kpart_off);
  float* v_part = reinterpret_cast<float*>(ws + L.vpart_off);
  ram_block_mask bm{reinterpret_cast<uint8_t*>(ws + L.cls_off), reinterpret_cast<int32_t*>(ws + L.cnt_off),
                    reinterpret_cast<int32_t*>(ws + L.col_off),
                    with_bits ? reinterpret_cast<uint32_t*>(ws + L.bits_off) : nullptr,
                    reinterpret_cast<int32_t*>(ws + L.ccnt_off), reinterpret_cast<int32_t*>(ws + L.ridx_off)};
  const int64_t nQb = cdiv(desc->Sq, ram::kBlockQ), nKb = cdiv(desc->Skv, ram::kBlockKV);
  const int64_t kv_full_stride = desc->kv_stride_b ? desc->kv_stride_b : kv_total * desc->Hkv * desc->D;
  const int64_t kv_acc_stride = kv_total * desc->Hkv * desc->D;
  const int64_t kvm_full = src->kv_meta_stride_b ? src->kv_meta_stride_b : kv_total;
  const int32_t q_base = (int32_t)(src->q_pos_base + q_extra);

  hipError_t e = ram::launch_bwd_prep(desc->dtype, desc->B, desc->Sq, desc->H, desc->D, out, dout, lse, sinks, delta, dsinks,
                                      stream);
  if (e != hipSuccess) return hip_fail(e, "ring backward prep launch");
  ram_mask_src sm = *src;
  sm.q_pos_base = q_base;
  sm.kv_meta_stride_b = kvm_full;
  ram::MaskParams mp = mask_params(desc, &sm, &bm, dense_cols);
  mp.kv_chunk_off = desc->Skv;
  mp.kv_base_step = desc->Skv;
  mp.dense_col_step = src->dense_chunk_step;
  e = ram::launch_block_mask(mp, n_chunks, stream);
  if (e != hipSuccess) return hip_fail(e, "ring backward block mask launch");
  e = ram::launch_col_lists(mp, n_chunks, bm.col_cnt, bm.row_idx, stream);
  if (e != hipSuccess) return hip_fail(e, "ring backward transposed lists launch");

  const int64_t esz = desc->dtype == RAM_BF16 ? 2 : 4;
  // bf16 with several chunks: dq of all chunks in one launch, each workgroup visiting every chunk
  // with its dq in registers and writing the bf16 result once; the chunk loop below then runs
  // the dk / dv kernel alone
  const bool dq_ring = desc->dtype == RAM_BF16 && n_chunks > 1 && desc->Sq > 0;
  if (g_ev_start && (e = hipEventRecord(g_ev_start, stream)) != hipSuccess) return hip_fail(e, "event record");
  if (dq_ring) {
    ram_attn_desc dc = *desc;
    dc.kv_stride_b = kv_full_stride;
    ram_mask_src sc = *src;
    sc.q_pos_base = q_base;
    sc.kv_meta_stride_b = kvm_full;
    ram::BwdParams bp{};
    bp.a = attn_params(&dc, q, k_all, v_all, &sc, &bm, nullptr, 0, nullptr, const_cast<float*>(lse), ram::kBlockQ);
    bp.a.n_chunks = n_chunks;
    bp.a.ring_shard = q_shard;
    bp.a.kv_chunk_elems = (int64_t)desc->Skv * desc->Hkv * desc->D;
    bp.a.mask_chunk_tiles = (int64_t)desc->B * nQb * nKb;
    bp.a.mask_chunk_rows = (int64_t)desc->B * nQb;
    bp.dout = dout;
    bp.delta = delta;
    bp.dq_out = dq;
    bp.head_split = 1;
    e = ram::launch_attn_bwd_dq(bp, stream);
    if (e != hipSuccess) return hip_fail(e, "ring backward dq launch");
  }
  for (int t = 0; t < n_chunks; ++t) {
    const int c = q_shard >= 0 ? ((q_shard - t) % n_chunks + n_chunks) % n_chunks : t;
    ram_attn_desc dc = *desc;
    dc.kv_stride_b = kv_full_stride;
    ram_mask_src sc = *src;
    sc.q_pos_base = q_base;
    sc.kv_meta_stride_b = kvm_full;
    sc.kv_pos = src->kv_pos ? src->kv_pos + (int64_t)c * desc->Skv : nullptr;
    sc.kv_seg = src->kv_seg ? src->kv_seg + (int64_t)c * desc->Skv : nullptr;
    sc.kv_pos_base = src->kv_pos_base + c * desc->Skv;
    const int64_t tiles_c = (int64_t)c * desc->B * nQb * nKb;
    const ram_block_mask bc{bm.tile_class + tiles_c, bm.row_cnt + (int64_t)c * desc->B * nQb, bm.col_idx + tiles_c,
                            with_bits ? bm.bits + tiles_c * kBwdTileWords : nullptr,
                            bm.col_cnt + (int64_t)c * desc->B * nKb, bm.row_idx + tiles_c};
    const int64_t kv_off = (int64_t)c * desc->Skv * desc->Hkv * desc->D;
    ram::BwdParams bp{};
    bp.a = attn_params(&dc, q, static_cast<const char*>(k_all) + kv_off * esz,
                       static_cast<const char*>(v_all) + kv_off * esz, &sc, &bc, nullptr, 0, nullptr,
                       const_cast<float*>(lse), ram::kBlockQ);
    bp.dout = dout;
    bp.delta = delta;
    bp.dq = dq_acc;
    bp.dk = dk_acc + kv_off;
    bp.dv = dv_acc + kv_off;
    bp.dkv_stride_b = kv_acc_stride;
    bp.col_cnt = bc.col_cnt;
    bp.row_idx = bc.row_idx;
    bp.dq_mode = t == 0 ? RAM_OUT_WRITE : RAM_OUT_MERGE;
    bp.head_split = head_split;
    if (head_split > 1) {
      // partial sums per head split, [S][B][Skv][Hkv][D], added into the chunk's accumulators below
      bp.dk = k_part;
      bp.dv = v_part;
      bp.dkv_stride_b = (int64_t)desc->Skv * desc->Hkv * desc->D;
      bp.part_stride = (int64_t)desc->B * bp.dkv_stride_b;
    }
    if (desc->dtype == RAM_F32) e = ram::launch_attn_bwd_f32(bp, stream);
    else e = dq_ring ? ram::launch_attn_bwd_dkv(bp, stream) : ram::launch_attn_bwd(bp, stream);
    if (e != hipSuccess) return hip_fail(e, "ring backward chunk launch");
    if (head_split > 1) {
      const int64_t n = (int64_t)desc->Skv * desc->Hkv * desc->D;
      e = ram::launch_sum_parts(k_part, head_split, bp.part_stride, desc->B, n, dk_acc + kv_off, kv_acc_stride, stream);
      if (e == hipSuccess)
        e = ram::launch_sum_parts(v_part, head_split, bp.part_stride, desc->B, n, dv_acc + kv_off, kv_acc_stride,
                                  stream);
      if (e != hipSuccess) return hip_fail(e, "ring backward partial sums launch");
    }
  }
  if (g_ev_stop && (e = hipEventRecord(g_ev_stop, stream)) != hipSuccess) return hip_fail(e, "event record");
  if (desc->dtype == RAM_F32) {
    // float32 results: the accumulators are the answer, copied into the caller's layout
    const size_t dq_bytes = (size_t)desc->B * desc->Sq * desc->H * desc->D * 4;
    e = hipMemcpyAsync(dq, dq_acc, dq_bytes, hipMemcpyDeviceToDevice, stream);
    for (int b = 0; b < desc->B && e == hipSuccess; ++b) {
      e = hipMemcpyAsync(static_cast<char*>(dk_all) + b * kv_full_stride * esz, dk_acc + b * kv_acc_stride,
                         kv_acc_stride * 4, hipMemcpyDeviceToDevice, stream);
      if (e == hipSuccess)
        e = hipMemcpyAsync(static_cast<char*>(dv_all) + b * kv_full_stride * esz, dv_acc + b * kv_acc_stride,
                           kv_acc_stride * 4, hipMemcpyDeviceToDevice, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "dq / dk / dv copy");
    return ok();
  }
  if (!dq_ring) {
    e = ram::launch_cast_bf16(dq_acc, dq, (int64_t)desc->B * desc->Sq * desc->H * desc->D, stream);
    if (e != hipSuccess) return hip_fail(e, "dq cast launch");
  }
  for (int b = 0; b < desc->B; ++b) {
    e = ram::launch_cast_bf16(dk_acc + b * kv_acc_stride, static_cast<char*>(dk_all) + b * kv_full_stride * esz,
                              kv_acc_stride, stream);
    if (e == hipSuccess)
      e = ram::launch_cast_bf16(dv_acc + b * kv_acc_stride, static_cast<char*>(dv_all) + b * kv_full_stride * esz,
                                kv_acc_stride, stream);
    if (e != hipSuccess) return hip_fail(e, "dk / dv cast launch");
  }
  return ok();
}

}  // extern "C"
