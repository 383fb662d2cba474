/*
 * ram.h - C ABI of the chunked (ring) attention forward for MI355X (gfx950).
 *
 * What it computes. The ejkernel ring-splash source page (module
 * ejkernel.kernels._pallas.tpu.ring_attention._ring_splash) runs, once per
 * KV chunk of a ring, a block-sparse flash-attention forward that returns the
 * chunk output and its per-row log-sum-exp, and folds each chunk into a
 * running (out, lse) with the sigmoid/softplus merge of _update_out_and_lse.
 * The Kvax page ("Kvax: Flash Attention for JAX", flash_attention and
 * create_attention_mask) fixes the tensor layouts and the position /
 * segment-ID masking; the ring-splash page's make_ring_attention adds a
 * caller-given two-dimensional mask. On one GPU the ring is a sequential
 * loop over chunks.
 *
 * Conventions shared by every call:
 *  - Tensor pointers are DEVICE pointers, allocated and owned by the caller.
 *    The library allocates nothing and keeps no state besides a thread-local
 *    error message.
 *  - Layouts (row-major, innermost last): q and out [B, Sq, H, D];
 *    k and v [B, Skv, Hkv, D]; lse [B, H, Sq] float32; positions and segment
 *    IDs [B, S] int32. Within a batch, rows are dense (row stride H*D or
 *    Hkv*D elements); the batch stride may be larger (a chunk view of a
 *    longer KV), given in elements, 0 meaning dense.
 *  - Every call validates all arguments on the host before it enqueues
 *    anything. On a non-OK status nothing was launched and no output was
 *    written; ram_last_error() describes the failure.
 *  - Calls are asynchronous on `stream` (0 = the null stream).
 *  - Query head h reads KV head h / (H / Hkv) (contiguous groups; Hkv == 1
 *    is MQA).
 *  - Scores: s = scale * q.k; with softcap > 0, s = softcap * tanh(s / softcap).
 *    A pair (i, j) takes part iff (!causal || kv_pos[j] <= q_pos[i]) and,
 *    with segment IDs, q_seg[i] == kv_seg[j] != RAM_PAD_SEGMENT_ID and, with
 *    a dense mask, its byte for (i, j) is nonzero. Excluded
 *    pairs get weight exactly 0 (the pages' finite mask value gives the same
 *    result on every row that attends to at least one key).
 *  - A sink (float32 [H], raw logit, neither scaled nor capped) adds
 *    exp(sink[h]) to the softmax normaliser with no value row.
 *  - A row with no allowed key (and no sink) has out = 0 and lse = -inf.
 *  - lse is the natural log of the normaliser.
 */
#ifndef RAM_H
#define RAM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Segment ID of padding tokens. The Kvax page names the constant without a value. */
#define RAM_PAD_SEGMENT_ID (-1)

typedef enum {
  RAM_OK = 0,
  RAM_ERR_INVALID = 1,     /* bad argument: null pointer, bad shape, mismatched tiles */
  RAM_ERR_UNSUPPORTED = 2, /* valid but not built: head dim, dtype, alignment */
  RAM_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  RAM_ERR_HIP = 4          /* a HIP launch failed; message holds hipGetErrorString */
} ram_status;

typedef enum { RAM_F32 = 0, RAM_BF16 = 1 } ram_dtype;

/* Tile classes: the ring-splash page names a block mask without codes. */
typedef enum { RAM_TILE_EMPTY = 0, RAM_TILE_PARTIAL = 1, RAM_TILE_FULL = 2 } ram_tile_class;

/* WRITE stores the chunk's (out, lse); MERGE folds them into (out, lse). */
typedef enum { RAM_OUT_WRITE = 0, RAM_OUT_MERGE = 1 } ram_out_mode;

typedef struct {
  int32_t B, Sq, Skv, H, Hkv, D; /* Skv: keys of one chunk; H % Hkv == 0, H <= 65536; D in {64, 128} */
  int32_t dtype;                 /* ram_dtype of q, k, v (and of the final out) */
  int64_t q_stride_b;            /* elements between batches of q; 0 = Sq*H*D */
  int64_t kv_stride_b;           /* elements between batches of k and v; 0 = Skv*Hkv*D */
  float scale;                   /* score scale (Kvax default is 1.0) */
  float softcap;                 /* <= 0: off */
  int32_t causal;                /* 0 or 1 */
  int32_t block_q, block_kv;     /* tile of the block mask; attention needs ram_kernel_tile() (forward)
                                    or ram_bwd_kernel_tile() (backward) */
} ram_attn_desc;

/* Positions, segment IDs and an optional dense mask for one (q, KV-chunk)
 * pair (Kvax flash_attention arguments; the two-dimensional mask of the
 * ring-splash make_ring_attention). A NULL position array means sequential
 * positions base + index. Segment arrays are both NULL (no segment masking)
 * or both set.
 *
 * Dense mask: uint8 [Sq, dense_ld], row i for query row i of this call, one
 * mask for every batch row and head; nonzero allows the pair. Key j of a
 * single-chunk call reads column j. In ring_attn_fwd_1gpu key j of chunk c
 * reads column c * dense_chunk_step + j: dense_chunk_step = Skv gives one mask
 * over all n_chunks*Skv keys, 0 reuses one [Sq, Skv] mask for every chunk (the
 * non-causal ring of the ring-splash page keeps one mask info for all steps).
 * dense_ld 0 means the columns the call reads: Skv, or Skv + (n_chunks - 1) *
 * dense_chunk_step in the ring. A dense mask needs tile bits (ram_block_mask). */
typedef struct {
  const int32_t* q_pos;   /* [B, Sq] or NULL => q_pos_base + i */
  const int32_t* kv_pos;  /* [B, Skv] or NULL => kv_pos_base + j */
  int32_t q_pos_base, kv_pos_base;
  const int32_t* q_seg;   /* [B, Sq] or NULL */
  const int32_t* kv_seg;  /* [B, Skv] or NULL */
  int64_t q_meta_stride_b;  /* elements between batches of q_pos/q_seg; 0 = Sq */
  int64_t kv_meta_stride_b; /* elements between batches of kv_pos/kv_seg; 0 = Skv */
  const uint8_t* dense;     /* [Sq, dense_ld] or NULL */
  int64_t dense_ld;         /* bytes between dense rows; 0 = the columns the call reads */
  int64_t dense_chunk_step; /* ring only: dense columns per chunk index, >= 0 */
} ram_mask_src;

/* Block mask of one (q, KV-chunk) pair at tile (block_q, block_kv), with
 * nQb = ceil(Sq/block_q), nKb = ceil(Skv/block_kv):
 *   tile_class uint8 [B, nQb, nKb]: ram_tile_class of each tile; pairs past
 *              the sequence ends do not count;
 *   row_cnt    int32 [B, nQb]: number of non-EMPTY tiles in the tile row;
 *   col_idx    int32 [B, nQb, nKb]: the row's non-EMPTY kv-tile indices in
 *              ascending order, then -1 in the remaining slots;
 *   bits       uint32 [B, nQb, nKb, block_q, ceil(block_kv/32)] or NULL: the
 *              element mask of each PARTIAL tile (MaskInfo partial_mask_blocks
 *              of the ring-splash page), one row of words per query row, key
 *              j of the tile at bit j % 32 of word j / 32, 0 past the
 *              sequence ends. Only PARTIAL tiles are written; the words of
 *              other tiles are left as they were. 8-byte aligned;
 *   col_cnt    int32 [B, nKb] or NULL, and
 *   row_idx    int32 [B, nKb, nQb] or NULL (both or neither): the transposed
 *              lists the backward walks (the ring-splash dkv MaskInfo): for
 *              each kv tile, its non-EMPTY q tiles ascending, then -1. */
typedef struct {
  uint8_t* tile_class;
  int32_t* row_cnt;
  int32_t* col_idx;
  uint32_t* bits;
  int32_t* col_cnt;
  int32_t* row_idx;
} ram_block_mask;

/* Tile classes and compacted non-empty tile lists from positions, segment
 * IDs and the dense mask (Kvax create_attention_mask; ring-splash MaskInfo
 * block_mask, the lists of blocks to visit and, when out->bits is set, the
 * partial blocks). Only desc->B, Sq, Skv, causal, block_q and block_kv are
 * read; block_q and block_kv must lie in [16, 512]. Exact for every tile. */
ram_status build_block_mask(const ram_attn_desc* desc, const ram_mask_src* src,
                            const ram_block_mask* out, hipStream_t stream);

/* One chunk of block-sparse attention forward (ring-splash
 * _ring_attention_forward, the per-step kernel call), visiting only the
 * non-EMPTY tiles of `mask` (built by build_block_mask at ram_kernel_tile()).
 * PARTIAL tiles are masked from mask->bits when they are needed: with a dense
 * mask, and for bf16 with D = 128 also with kv positions or segment IDs (that
 * kernel's only other mask is the positional one); mask->bits must then be
 * set, else the call returns RAM_ERR_INVALID. Otherwise they are masked by
 * positions and segment IDs (and bits, if given, by them).
 *   q [B,Sq,H,D], k and v [B,Skv,Hkv,D] in desc->dtype; sinks float32 [H] or NULL.
 *   mode RAM_OUT_WRITE: out <- chunk output (float32 [B,Sq,H,D]), lse <- chunk
 *        lse (float32 [B,H,Sq]), for every row (empty rows get 0 / -inf).
 *   mode RAM_OUT_MERGE: (out, lse) hold a running state and are updated in
 *        place with the merge of _update_out_and_lse: a row whose running lse
 *        is -inf takes the chunk's values; otherwise, with x = chunk_lse - lse,
 *        out -= sigmoid(x) * (out - chunk_out) and lse += softplus(x).
 * `src` gives the masking data of this chunk (it must match the one the mask
 * was built from). */
ram_status attn_fwd_chunk(const ram_attn_desc* desc, const void* q, const void* k, const void* v,
                          const ram_mask_src* src, const ram_block_mask* mask, const float* sinks,
                          int32_t mode, float* out, float* lse, hipStream_t stream);

/* Standalone merge of one chunk's (out_blk, lse_blk) into (out_acc, lse_acc),
 * in place, by _update_out_and_lse of the ring-splash page. All float32;
 * out_* [B,Sq,H,D], lse_* [B,H,Sq]. out_blk may not alias out_acc. */
ram_status lse_merge(int32_t B, int32_t Sq, int32_t H, int32_t D, float* out_acc, float* lse_acc,
                     const float* out_blk, const float* lse_blk, hipStream_t stream);

/* The ring of _ring_attention_forward on one GPU: n_chunks KV chunks of
 * desc->Skv keys each, k_all and v_all [B, n_chunks*Skv, Hkv, D], visited in
 * sequence and merged by LSE into float32 accumulators; the result is cast to
 * the q dtype (out [B,Sq,H,D]) with lse float32 [B,H,Sq].
 *   q_shard >= 0: this q shard is ring index r = q_shard of n_chunks; step t
 *     visits chunk (r - t) mod n_chunks, and sequential q positions start at
 *     r * Sq + src->q_pos_base.
 *   q_shard == -1: chunks are visited in order 0..n_chunks-1 and sequential q
 *     positions start at src->q_pos_base.
 *   Sequential KV positions are global: chunk c key j is c*Skv + j +
 *     src->kv_pos_base. Explicit kv_pos / kv_seg arrays span all
 *     n_chunks*Skv keys and travel with their chunk.
 *   Sinks enter on the first visited chunk only.
 *   A dense mask (src->dense) is read per chunk as ram_mask_src describes.
 * bf16 with D = 128 runs the whole ring as one launch in which each workgroup
 * keeps its q tile and visits every chunk; when the rows of q tiles are fewer
 * than the GPU's compute units, each row's visits are split over two
 * workgroups (the first and second half of the ring order) whose running
 * results are merged by lse afterwards: the same result up to the rounding of
 * the merge order.
 * workspace: device memory of at least ring_attn_workspace_bytes(), 256-byte
 * aligned; it holds the float32 output accumulator (bf16 only), the block
 * masks of every chunk (with their tile bits when the forward call would need
 * them, see attn_fwd_chunk), for a split ring the second half's running
 * result, and, when the ring reads V repacked (bf16, D = 128, no soft cap and
 * Sq * H / Hkv >= 32768), a copy of v_all rearranged for the kernel (the same
 * size as v_all, rounded up to 32 keys per chunk).
 * The call only launches kernels on `stream` (no allocation, memset or host
 * synchronisation), so a caller may capture it in a HIP graph and replay it.
 * RAM_ERR_UNSUPPORTED for n_chunks or B above 65535. */
ram_status ring_attn_fwd_1gpu(const ram_attn_desc* desc, int32_t n_chunks, int32_t q_shard,
                              const void* q, const void* k_all, const void* v_all,
                              const ram_mask_src* src, const float* sinks, void* out, float* lse,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- backward
 * The ring-splash page's _ring_attention_backward: every ring step runs the
 * chunk backward with the final out and logsumexp of the whole ring as
 * residuals and sums the chunk gradients. For query row i and allowed key j:
 *   p_ij = exp(s'_ij - lse_i) (s' the scaled, capped logit), D_i = dout_i . out_i,
 *   ds_ij = p_ij (dout_i . v_j - D_i) (1 - t_ij^2 with a soft cap, t = s' / cap),
 *   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,  dv_j = sum_i p_ij dout_i
 * (dk, dv summed over the query heads sharing a KV head), and for a sink
 *   dsink_h = - sum over batch rows and queries of exp(sink_h - lse_i) D_i,
 * counted once (the sink enters the forward once). Built for bf16 and
 * float32 with D = 64 or 128; other dtypes and head dims return
 * RAM_ERR_UNSUPPORTED.
 * out, dout: [B, Sq, H, D] dense in desc->dtype; lse: float32 [B, H, Sq] (as
 * the forward wrote them). */

/* delta: float32 [2, B, H, Sq], the row values the chunk backward reads:
 * delta[0,b,h,i] = dout[b,i,h,:] . out[b,i,h,:] and delta[1,b,h,i] =
 * lse[b,h,i] * log2(e) (+inf where lse is -inf); and, when sinks is not NULL,
 * dsinks (float32 [H]) as above. */
ram_status attn_bwd_prep(const ram_attn_desc* desc, const void* out, const void* dout, const float* lse,
                         const float* sinks, float* delta, float* dsinks, hipStream_t stream);

/* Gradients of one chunk (the per-step call of _ring_attention_backward) with
 * mask built by build_block_mask at ram_bwd_kernel_tile() including the transposed
 * lists (and the bits when src->dense is set).
 *   dq: float32 [B, Sq, H, D] dense; dq_mode RAM_OUT_WRITE stores the chunk's
 *       dq, RAM_OUT_MERGE adds it to dq.
 *   dk, dv: float32 with the layout and strides of k and v; written.
 * Deterministic: no atomics. */
ram_status attn_bwd_chunk(const ram_attn_desc* desc, const void* q, const void* k, const void* v,
                          const void* dout, const float* lse, const float* delta, const ram_mask_src* src,
                          const ram_block_mask* mask, int32_t dq_mode, float* dq, float* dk, float* dv,
                          hipStream_t stream);

/* The backward of ring_attn_fwd_1gpu with the same desc, n_chunks, q_shard,
 * src and sinks: dq [B, Sq, H, D] dense, dk_all and dv_all with the layout of
 * k_all and v_all, all in desc->dtype; dsinks float32 [H] (NULL when sinks is
 * NULL). workspace: at least ring_attn_bwd_workspace_bytes(), 256-byte
 * aligned (float32 accumulators, delta, and the block masks of every chunk). */
ram_status ring_attn_bwd_1gpu(const ram_attn_desc* desc, int32_t n_chunks, int32_t q_shard, const void* q,
                              const void* k_all, const void* v_all, const void* out, const float* lse,
                              const void* dout, const ram_mask_src* src, const float* sinks, void* dq,
                              void* dk_all, void* dv_all, float* dsinks, void* workspace, size_t workspace_bytes,
                              hipStream_t stream);

/* Workspace bytes ring_attn_bwd_1gpu needs (0 on bad input); src may be NULL. */
size_t ring_attn_bwd_workspace_bytes(const ram_attn_desc* desc, int32_t n_chunks, const ram_mask_src* src);

/* ring_attn_fwd_1gpu for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, results and errors without the workspace. Its scratch is a
 * static device array of 64 MiB that each GPU the library runs on holds until
 * the process ends (looked up on the first call on a device); shapes whose
 * ring_attn_workspace_bytes() exceeds it fail with RAM_ERR_UNSUPPORTED before
 * anything runs. All calls on one GPU share that GPU's array: calls that
 * overlap on a GPU (on different streams or threads) race. Allocates nothing. */
ram_status ring_attn_fwd_1gpu_noalloc(const ram_attn_desc* desc, int32_t n_chunks, int32_t q_shard, const void* q,
                                      const void* k_all, const void* v_all, const ram_mask_src* src,
                                      const float* sinks, void* out, float* lse, hipStream_t stream);

/* Workspace bytes ring_attn_fwd_1gpu needs for this shape (0 on bad input).
 * src may be NULL; a source whose forward needs tile bits needs room for them. */
size_t ring_attn_workspace_bytes(const ram_attn_desc* desc, int32_t n_chunks, const ram_mask_src* src);

/* Where ring_attn_fwd_1gpu (ring_attn_fwd_masks) and ring_attn_bwd_1gpu
 * (ring_attn_bwd_masks) keep, inside their workspace, the block masks they
 * build for every chunk (at the tile their kernels walk), so that a caller can
 * read them back after a call: byte offsets of
 *   tile classes  uint8 [n_chunks][B][nQb][nKb] (RAM_TILE_*),
 *   tile counts   int32 [n_chunks][B][nQb],
 *   tile lists    int32 [n_chunks][B][nQb][nKb] (ascending, -1 padded),
 *   tile bits     uint32 [n_chunks][B][nQb][nKb][tile_words] as in
 *                 ram_block_mask, or -1 when the call stores none,
 *   row order     int32 [B * nQb] (forward only, else -1): the rows of q tiles
 *                 (b * nQb + qb) in the order the one-launch ring takes them,
 *                 most non-EMPTY tiles over all chunks first (made when
 *                 positions, segment IDs or a dense mask are given),
 * chunk c being the chunk at index c of k_all (not the visit order). The mask
 * of a chunk is what build_block_mask makes for that chunk's keys (see
 * ring_attn_fwd_1gpu for their positions and dense-mask columns). Same
 * arguments as the workspace-size calls; RAM_ERR_INVALID on bad input. */
typedef struct ram_ring_masks {
  int64_t cls_off, cnt_off, col_off, bits_off, order_off;
  int32_t block_q, block_kv, nQb, nKb, tile_words;
} ram_ring_masks;
ram_status ring_attn_fwd_masks(const ram_attn_desc* desc, int32_t n_chunks, const ram_mask_src* src,
                               ram_ring_masks* out);
ram_status ring_attn_bwd_masks(const ram_attn_desc* desc, int32_t n_chunks, const ram_mask_src* src,
                               ram_ring_masks* out);

/* The tile (block_q, block_kv) the forward kernel of (dtype, D) walks: block
 * masks passed to attn_fwd_chunk must be built at this tile (128 x 64 for
 * every built dtype and head dim). */
ram_status ram_kernel_tile(int32_t dtype, int32_t D, int32_t* block_q, int32_t* block_kv);

/* The tile the backward kernels walk (128 x 64): block masks passed to
 * attn_bwd_chunk must be built at this tile. */
ram_status ram_bwd_kernel_tile(int32_t dtype, int32_t D, int32_t* block_q, int32_t* block_kv);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* ram_last_error(void);

/* Measurement aid: until called again with (NULL, NULL), ring_attn_fwd_1gpu
 * and ring_attn_bwd_1gpu calls made on this thread record `start` on their
 * stream right before their first attention-kernel launch and `stop` right
 * after the last one (the block-mask build, the backward's row dots and the
 * final casts fall outside), so a caller can time the attention kernels alone.
 * The events stay owned by the caller. Returns RAM_ERR_INVALID if exactly one
 * of them is NULL. */
ram_status ram_set_kernel_events(hipEvent_t start, hipEvent_t stop);

/* Measurement aid, not part of the attention path: n_blocks workgroups of 8
 * waves, each wave running iters x 32 v_mfma_f32_32x32x16_bf16 (32768 FLOP
 * each) from operands held in registers, all zero
 * (operands = 0) or pseudo-random in [-1, 1) (operands = 1): the dense bf16
 * MFMA rate the chip sustains, which depends on the operands' values. out:
 * device float32 [n_blocks * 512], written (a checksum per thread). Returns
 * RAM_ERR_INVALID for bad arguments (nothing launched), RAM_ERR_HIP if the
 * launch fails; ram_last_error() is not set by this call. */
ram_status ram_mfma_probe(int32_t n_blocks, int32_t iters, int32_t operands, float* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RAM_H */
