// Internal parameter blocks and launchers shared by the HIP sources of libram.
// Not part of the C ABI (include/ram.h is).
#pragma once

#include <cstdint>
#include <hip/hip_runtime_api.h>

#include "../../include/ram.h"

namespace ram {

// Mask tiles the kernels walk: 128 query rows by 64 keys (the forward kernels, the backward).
constexpr int kBlockQ = 128;
constexpr int kAltRows = 128;
constexpr int kBlockKV = 64;
// Query rows of the forward mask tile for a dtype code (1 = bf16) and head dim.
constexpr int fwd_block_q(int dtype, int D) { return (dtype == 1 && D == 128) ? kAltRows : kBlockQ; }
// Largest number of kv tiles in one block-mask row (classes are staged in LDS).
constexpr int kMaxMaskCols = 8192;
constexpr int kMaxMaskTile = 512;

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  float* out;         // float32 [B,Sq,H,D], dense
  void* out_final;    // bf16 [B,Sq,H,D] or null: when set, the final result goes
                      // here in bf16 (the last chunk of a ring) and `out` is only read
  float* lse;         // float32 [B,H,Sq], dense
  const float* sinks; // [H] or null
  const uint8_t* tile_class;
  const int32_t* row_cnt;
  const int32_t* col_idx;
  const int32_t* q_pos;
  const int32_t* kv_pos;
  const int32_t* q_seg;
  const int32_t* kv_seg;
  const uint32_t* mask_bits;  // bits of the PARTIAL tiles (tile rows x 2 words per tile) or null
  int64_t q_stride_b, kv_stride_b;   // elements
  int64_t qm_stride_b, kvm_stride_b; // elements of the position / segment arrays
  int32_t q_pos_base, kv_pos_base;
  int32_t B, Sq, Skv, H, Hkv, D;
  int32_t nQb, nKb;       // mask tiles of the call
  int32_t tile_words;     // bit words per mask tile: rows x (block_kv / 32)
  float scale_log2;   // scale * log2(e)
  float cap_k2;       // 2 * scale * log2(e) / softcap   (soft cap on)
  float cap_log2;     // softcap * log2(e)               (soft cap on)
  int32_t softcap_on;
  int32_t causal;
  int32_t mode;       // 0 write, 1 merge
  // One launch for a whole ring (launch_attn_alt): k, v, the mask arrays and
  // kv_pos / kv_seg / kv_pos_base describe chunk 0, chunk c lies kv_chunk_elems
  // elements (k, v), mask_chunk_tiles tiles and mask_chunk_rows rows (masks)
  // and c*Skv keys (kv arrays, kv_pos_base) further. Visit t takes chunk
  // (ring_shard - t) mod n_chunks, or t when ring_shard < 0; sinks and `mode`
  // apply to visit 0, out_final to the last.
  int32_t n_chunks;
  int32_t ring_shard;
  int64_t kv_chunk_elems;
  int64_t mask_chunk_tiles;
  int64_t mask_chunk_rows;
  // or null: the rows (b * nQb + qb) in the order workgroups take them (most tiles first, made by
  // launch_row_order); heads are the inner index, workgroups go to the XCDs round robin
  const int32_t* row_order;
  // or null (bf16, D = 128 kernel only): V repacked by launch_pack_v, read with row reads instead
  // of transposing ones; chunk c at + c * vt_chunk_bytes, then [B][Hkv][ceil(Skv / 32)] tiles
  const void* vt;
  int64_t vt_chunk_bytes;
};

// A split ring (launch_attn_alt with this given): each q tile row's visits go to two
// workgroups, visits [0, h) and [h, n_chunks) with h = (n_chunks + 1) / 2; the second writes
// its own running result to out2 / lse2 (its first visit in `mode`), to be merged into
// out / lse afterwards.
struct RingSplit {
  float* out2;
  float* lse2;
};

struct MaskParams {
  const int32_t* q_pos;
  const int32_t* kv_pos;
  const int32_t* q_seg;
  const int32_t* kv_seg;
  int64_t qm_stride_b, kvm_stride_b;
  int64_t kv_chunk_off;    // elements added to kv_pos / kv_seg per chunk (blockIdx.z)
  int32_t q_pos_base, kv_pos_base;
  int32_t kv_base_step;    // added to kv_pos_base per chunk
  const uint8_t* dense;    // [Sq, dense_ld] or null; chunk c reads from column c * dense_col_step
  int64_t dense_ld, dense_col_step;
  int32_t B, Sq, Skv, bq, bk, nQb, nKb, causal;
  uint8_t* tile_class;     // chunk c at + c * B*nQb*nKb
  int32_t* row_cnt;        // chunk c at + c * B*nQb
  int32_t* col_idx;        // chunk c at + c * B*nQb*nKb
  uint32_t* bits;          // or null; tile t at + t * bq*ceil(bk/32), t counted like tile_class
  int32_t kv_split;        // workgroups per row of tiles (set by the launcher; 1: one does it all)
};

// Backward of one chunk: `a` carries q, k, v, lse, the masks and sizes of the
// forward call (a.out, a.out_final, a.sinks and a.mode are not read).
struct BwdParams {
  AttnParams a;
  const void* dout;        // [B,Sq,H,D] in the q dtype
  const float* delta;      // [B,H,Sq]: rowsum(dout * out)
  float* dq;               // float32 [B,Sq,H,D], written (dq_mode 0) or added to (1)
  // ring (a.n_chunks > 1, bf16): dq over all chunks, written once as bf16 [B,Sq,H,D]
  void* dq_out;
  float* dk;               // float32 [B, Skv, Hkv, D] rows, batch stride dkv_stride_b
  float* dv;
  int64_t dkv_stride_b;    // elements
  const int32_t* col_cnt;  // [B, nKb]: non-EMPTY q tiles per kv tile
  const int32_t* row_idx;  // [B, nKb, nQb]: those q tiles, ascending
  int32_t dq_mode;
  // dk / dv over the heads of a KV group split into head_split workgroups (a divisor of the
  // group size; 1 = one workgroup per kv tile): split s writes its partial sums at
  // dk / dv + s * part_stride, to be added up by launch_sum_parts.
  int32_t head_split;
  int64_t part_stride;     // elements
};

// float32 (D = 64 / 128) and bf16 D = 64: the four-wave kernels, one chunk per launch.
hipError_t launch_attn(const AttnParams& p, int dtype, hipStream_t s);
hipError_t launch_attn_bwd(const BwdParams& p, hipStream_t s);       // bf16, D = 64 / 128: dq, then dk / dv
hipError_t launch_attn_bwd_dq(const BwdParams& p, hipStream_t s);    // bf16: dq alone (a ring if a.n_chunks > 1)
hipError_t launch_attn_bwd_dkv(const BwdParams& p, hipStream_t s);   // bf16: dk / dv alone
hipError_t launch_attn_bwd_f32(const BwdParams& p, hipStream_t s);   // float32, D = 64 / 128
// delta (and dsinks) from out and dout in `dtype` (RAM_BF16 / RAM_F32 codes)
hipError_t launch_bwd_prep(int dtype, int B, int Sq, int H, int D, const void* out, const void* dout,
                           const float* lse, const float* sinks, float* delta, float* dsinks, hipStream_t s);
hipError_t launch_col_lists(const MaskParams& p, int n_chunks, int32_t* col_cnt, int32_t* row_idx,
                            hipStream_t s);
// bf16, D = 128, mask tiles of kAltRows rows: one visit per chunk (n_chunks = 1 for a single chunk).
// Kernels without kv positions, kv segments or tile bits mask PARTIAL tiles by positions;
// with any of them, PARTIAL tiles are masked from mask_bits, which must then be set.
// V of every chunk of a ring [B, kv_stride_b (elements), keys n_chunks * Skv, Hkv, D = 128], bf16,
// repacked for the bf16 D = 128 kernel: per (chunk, batch, kv head) ceil(Skv / 32) tiles of 8 KiB,
// each the LDS image of one 32-key step of V in the order of the weights' operand (keys past Skv
// zero).
constexpr int kPackKeys = 32;                   // keys per repacked V tile (one kernel step)
constexpr int kPackTileBytes = kPackKeys * 256; // 32 keys x 128 dims x 2 bytes
inline size_t pack_v_bytes(int B, int n_chunks, int Skv, int Hkv) {
  return (size_t)n_chunks * B * Hkv * ((Skv + kPackKeys - 1) / kPackKeys) * kPackTileBytes;
}
hipError_t launch_pack_v(const void* v_all, int64_t kv_stride_b, int B, int n_chunks, int Skv, int Hkv, void* vt,
                         hipStream_t s);
hipError_t launch_attn_alt(const AttnParams& p, const RingSplit* split, hipStream_t s);
hipError_t launch_block_mask(const MaskParams& p, int n_chunks, hipStream_t s);
// order[0 .. rows): the rows of tiles sorted by their non-EMPTY tiles summed over the n_chunks
// chunks' counts (row_cnt + c * rows, each at most max_tiles), most first (totals above 4095
// count as 4095; rows with equal totals in any order).
hipError_t launch_row_order(const int32_t* row_cnt, int n_chunks, int64_t rows, int max_tiles, int32_t* order,
                            hipStream_t s);
// lse merge of a block's (out, lse) into the running ones; with out_bf16 set, the merged rows go
// there in bf16 (bf16 [B,Sq,H,D]) instead of back into out_acc
hipError_t launch_merge(int B, int Sq, int H, int D, float* out_acc, float* lse_acc,
                        const float* out_blk, const float* lse_blk, hipStream_t s, void* out_bf16 = nullptr);
hipError_t launch_cast_bf16(const float* src, void* dst, int64_t n, hipStream_t s);
// dst[b * dst_stride + i] = sum over s < S of src[s * part_stride + b * n + i], i < n, b < B
// (a fixed order: deterministic).
// Sets the message ram_last_error() returns and returns s (for entry points outside ram_api.cpp).
ram_status api_fail(ram_status s, const char* msg);
hipError_t launch_sum_parts(const float* src, int S, int64_t part_stride, int B, int64_t n, float* dst,
                            int64_t dst_stride, hipStream_t s);

}  // namespace ram
