// The C ABI's argument checking, run on the CPU against a host-only build of ram_api.cpp (kernel
// launchers stubbed) under the address and undefined-behaviour sanitizers. Each case calls an
// entry point with arguments it must reject (or accept as a no-op without launching) and checks
// the status and the message; the pointers are fake, aligned, and never dereferenced on these
// paths. Prints one line per failed case and exits with the number of failures.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <limits>

#include "../../include/ram.h"

namespace {

int g_fail = 0, g_cases = 0;

void expect(const char* what, ram_status got, ram_status want, const char* msg = nullptr) {
  ++g_cases;
  const char* err = ram_last_error();
  if (got != want || (msg && !std::strstr(err, msg))) {
    ++g_fail;
    std::printf("FAIL %s: status %d (want %d), message \"%s\" (want \"%s\")\n", what, (int)got, (int)want, err,
                msg ? msg : "");
  }
}
void expect_size(const char* what, size_t got, size_t want) {
  ++g_cases;
  if (got != want) {
    ++g_fail;
    std::printf("FAIL %s: %zu (want %zu)\n", what, got, want);
  }
}

void* const FAKE = reinterpret_cast<void*>(0x100000);   // 256-byte aligned, never dereferenced
void* const FAKE2 = reinterpret_cast<void*>(0x200000);
template <typename T>
T* fake(uintptr_t add = 0) {
  return reinterpret_cast<T*>(reinterpret_cast<uintptr_t>(FAKE) + add);
}

ram_attn_desc desc(int B = 1, int Sq = 256, int Skv = 256, int H = 4, int Hkv = 2, int D = 128,
                   int dtype = RAM_BF16) {
  ram_attn_desc d{};
  d.B = B;
  d.Sq = Sq;
  d.Skv = Skv;
  d.H = H;
  d.Hkv = Hkv;
  d.D = D;
  d.dtype = dtype;
  d.scale = 0.125f;
  d.causal = 1;
  d.block_q = 128;
  d.block_kv = 64;
  return d;
}
ram_block_mask mask() {
  return ram_block_mask{fake<uint8_t>(), fake<int32_t>(), fake<int32_t>(), nullptr, nullptr, nullptr};
}
ram_status chunk(const ram_attn_desc& d, const ram_mask_src& s, const ram_block_mask& m, int mode = 0,
                 const void* q = FAKE, const void* k = FAKE, float* out = fake<float>(), float* lse = fake<float>()) {
  return attn_fwd_chunk(&d, q, k, FAKE, &s, &m, nullptr, mode, out, lse, nullptr);
}
ram_status ring(const ram_attn_desc& d, int n, int r, const ram_mask_src& s, void* ws = FAKE,
                size_t ws_bytes = size_t(1) << 40) {
  return ring_attn_fwd_1gpu(&d, n, r, FAKE, FAKE, FAKE, &s, nullptr, FAKE, fake<float>(), ws, ws_bytes, nullptr);
}

}  // namespace

int main() {
  const ram_mask_src none{};
  const ram_block_mask m = mask();

  // descriptor checks
  {
    ram_attn_desc d = desc();
    d.Hkv = 3;
    expect("H not a multiple of Hkv", chunk(d, none, m), RAM_ERR_INVALID, "multiple");
    d = desc(1, 256, 256, 4, 2, 96);
    expect("head dim", chunk(d, none, m), RAM_ERR_UNSUPPORTED, "head dim");
    d = desc();
    d.dtype = 5;
    expect("dtype", chunk(d, none, m), RAM_ERR_UNSUPPORTED, "dtype");
    d = desc();
    d.scale = 0.0f;
    expect("scale 0", chunk(d, none, m), RAM_ERR_INVALID, "scale");
    d.scale = std::numeric_limits<float>::quiet_NaN();
    expect("scale NaN", chunk(d, none, m), RAM_ERR_INVALID, "scale");
    d = desc();
    d.softcap = std::numeric_limits<float>::infinity();
    expect("softcap inf", chunk(d, none, m), RAM_ERR_INVALID, "softcap");
    d = desc();
    d.causal = 2;
    expect("causal 2", chunk(d, none, m), RAM_ERR_INVALID, "causal");
    d = desc();
    d.block_q = 64;
    expect("tile rows", chunk(d, none, m), RAM_ERR_INVALID, "tile");
    d = desc();
    d.B = -1;
    expect("negative B", chunk(d, none, m), RAM_ERR_INVALID, "negative");
    d = desc(1, 256, 256, 1 << 17, 1);
    expect("too many heads", chunk(d, none, m), RAM_ERR_UNSUPPORTED, "above");
    d = desc();
    d.q_stride_b = 100;
    expect("q_stride_b", chunk(d, none, m), RAM_ERR_INVALID, "q_stride_b");
    d = desc();
    d.kv_stride_b = 256 * 2 * 128 + 3;
    expect("kv_stride_b", chunk(d, none, m), RAM_ERR_INVALID, "kv_stride_b");
    d = desc(1, 4096, 524288, 32, 32);
    expect("chunk of 4 GiB", chunk(d, none, m), RAM_ERR_UNSUPPORTED, "4 GiB");
    expect("null desc", attn_fwd_chunk(nullptr, FAKE, FAKE, FAKE, &none, &m, nullptr, 0, fake<float>(), fake<float>(), nullptr),
           RAM_ERR_INVALID);
  }
  // pointers, modes, mask arrays
  {
    const ram_attn_desc d = desc();
    expect("null q", chunk(d, none, m, 0, nullptr), RAM_ERR_INVALID, "q is null");
    expect("misaligned k", chunk(d, none, m, 0, FAKE, fake<char>(2)), RAM_ERR_UNSUPPORTED, "aligned");
    expect("null out", chunk(d, none, m, 0, FAKE, FAKE, nullptr), RAM_ERR_INVALID);
    expect("misaligned lse", chunk(d, none, m, 0, FAKE, FAKE, fake<float>(), fake<float>(2)), RAM_ERR_INVALID);
    expect("bad mode", chunk(d, none, m, 3), RAM_ERR_INVALID, "mode");
    ram_mask_src s{};
    s.q_seg = fake<int32_t>();
    expect("one segment array", chunk(d, s, m), RAM_ERR_INVALID, "both");
    s = ram_mask_src{};
    s.q_pos = fake<int32_t>(1);
    expect("misaligned q_pos", chunk(d, s, m), RAM_ERR_INVALID);
    s = ram_mask_src{};
    s.q_pos_base = 2147483647 - 10;
    expect("position overflow", chunk(d, s, m), RAM_ERR_INVALID, "overflow");
    s = ram_mask_src{};
    s.kv_meta_stride_b = 10;
    expect("kv_meta_stride_b", chunk(d, s, m), RAM_ERR_INVALID);
    ram_block_mask bm = m;
    bm.row_cnt = nullptr;
    expect("null row_cnt", chunk(d, none, bm), RAM_ERR_INVALID, "row_cnt");
    bm = m;
    bm.tile_class = nullptr;
    expect("null tile_class", chunk(d, none, bm), RAM_ERR_INVALID, "tile_class");
    bm = m;
    bm.col_idx = nullptr;
    expect("null col_idx", chunk(d, none, bm), RAM_ERR_INVALID, "col_idx");
    expect("null mask source", attn_fwd_chunk(&d, FAKE, FAKE, FAKE, nullptr, &m, nullptr, 0, fake<float>(), fake<float>(), nullptr),
           RAM_ERR_INVALID);
  }
  // dense masks
  {
    const ram_attn_desc d = desc();
    ram_mask_src s{};
    s.dense = fake<uint8_t>(0x100000);
    expect("dense without bits", chunk(d, s, m), RAM_ERR_INVALID, "tile bits");
    ram_block_mask bm = m;
    bm.bits = fake<uint32_t>(4);
    expect("misaligned bits", chunk(d, s, bm), RAM_ERR_INVALID, "8-byte");
    bm.bits = fake<uint32_t>(0x100000);
    s.dense_ld = 255;
    expect("dense_ld short", chunk(d, s, bm), RAM_ERR_INVALID, "dense_ld");
    s.dense_ld = 0;
    s.dense_chunk_step = -1;
    expect("negative dense step", chunk(d, s, bm), RAM_ERR_INVALID);
    ram_attn_desc dm = desc();
    dm.block_q = 64;
    dm.block_kv = 48;
    ram_mask_src sd{};
    sd.dense = fake<uint8_t>(0x100000);
    sd.dense_ld = 100;
    expect("builder dense_ld", build_block_mask(&dm, &sd, &m, nullptr), RAM_ERR_INVALID);
    dm.block_q = 8;
    expect("builder tile", build_block_mask(&dm, &none, &m, nullptr), RAM_ERR_INVALID);
    expect("builder null source", build_block_mask(&dm, nullptr, &m, nullptr), RAM_ERR_INVALID);
  }
  // the ring
  {
    const ram_attn_desc d = desc(1, 4096, 4096, 8, 8);
    const size_t need = ring_attn_workspace_bytes(&d, 4, nullptr);
    expect_size("workspace with no chunks", ring_attn_workspace_bytes(&d, 0, nullptr), 0);
    expect("no chunks", ring(d, 0, -1, none), RAM_ERR_INVALID);
    expect("q_shard past the end", ring(d, 4, 4, none), RAM_ERR_INVALID, "q_shard");
    expect("q_shard below -1", ring(d, 4, -2, none), RAM_ERR_INVALID);
    expect("workspace short", ring(d, 4, 3, none, FAKE, need - 1), RAM_ERR_WORKSPACE, "need");
    expect("workspace misaligned", ring(d, 4, 3, none, fake<char>(16)), RAM_ERR_WORKSPACE);
    expect("workspace null", ring(d, 4, 3, none, nullptr), RAM_ERR_WORKSPACE);
    ram_mask_src s{};
    s.q_pos_base = 2147483647 - 5000;
    expect("ring position overflow", ring(d, 4, 3, s), RAM_ERR_INVALID);
    s = ram_mask_src{};
    s.kv_meta_stride_b = 4096;
    expect("kv arrays span one chunk", ring(d, 4, 3, s), RAM_ERR_INVALID);
    const ram_attn_desc dr = desc(1, 512, 512, 4, 4);
    s = ram_mask_src{};
    s.dense = fake<uint8_t>(0x100000);
    s.dense_chunk_step = 512;
    s.dense_ld = 4 * 512 - 1;
    expect("ring dense_ld", ring(dr, 4, 3, s), RAM_ERR_INVALID, "dense_ld");
    ram_ring_masks rm{};
    expect("mask layout", ring_attn_fwd_masks(&d, 4, nullptr, &rm), RAM_OK);
    expect_size("mask layout bits", (size_t)(rm.bits_off == -1), 1);
    expect("mask layout no chunks", ring_attn_fwd_masks(&d, 0, nullptr, &rm), RAM_ERR_INVALID);
    expect("mask layout null out", ring_attn_bwd_masks(&d, 2, nullptr, nullptr), RAM_ERR_INVALID);
  }
  // merge, backward, tiles
  {
    expect("merge head dim", lse_merge(1, 4, 2, 96, fake<float>(), fake<float>(), fake<float>(0x100000),
                                       fake<float>(0x100000), nullptr),
           RAM_ERR_UNSUPPORTED);
    expect("merge aliasing", lse_merge(1, 4, 2, 128, fake<float>(), fake<float>(), fake<float>(), fake<float>(0x100000),
                                       nullptr),
           RAM_ERR_INVALID, "alias");
    expect("merge negative", lse_merge(-1, 4, 2, 128, fake<float>(), fake<float>(), fake<float>(0x100000),
                                       fake<float>(0x100000), nullptr),
           RAM_ERR_INVALID);
    int32_t bq = 0, bk = 0;
    expect("kernel tile", ram_kernel_tile(RAM_BF16, 128, &bq, &bk), RAM_OK);
    expect_size("kernel tile rows", (size_t)bq, 128);
    expect("kernel tile head dim", ram_kernel_tile(RAM_BF16, 96, &bq, &bk), RAM_ERR_UNSUPPORTED);
    expect("bwd kernel tile dtype", ram_bwd_kernel_tile(7, 128, &bq, &bk), RAM_ERR_UNSUPPORTED);
    const ram_attn_desc d = desc();
    ram_block_mask bm = m;
    expect("bwd without transposed lists",
           attn_bwd_chunk(&d, FAKE, FAKE, FAKE, FAKE, fake<float>(), fake<float>(), &none, &bm, 0, fake<float>(),
                          fake<float>(), fake<float>(), nullptr),
           RAM_ERR_INVALID, "transposed");
    bm.col_cnt = fake<int32_t>();
    expect("bwd one transposed array",
           attn_bwd_chunk(&d, FAKE, FAKE, FAKE, FAKE, fake<float>(), fake<float>(), &none, &bm, 0, fake<float>(),
                          fake<float>(), fake<float>(), nullptr),
           RAM_ERR_INVALID, "both");
  }
  // empty inputs: valid, nothing launched
  {
    ram_attn_desc d = desc(0);
    expect("B = 0", chunk(d, none, m, 0, nullptr, FAKE, nullptr, nullptr), RAM_OK);
    d = desc(1, 0);
    expect("Sq = 0", chunk(d, none, m, 0, nullptr, FAKE, nullptr, nullptr), RAM_OK);
    expect("builder Sq = 0", build_block_mask(&d, &none, &m, nullptr), RAM_OK);
    expect("merge of nothing", lse_merge(0, 5, 2, 128, nullptr, nullptr, nullptr, nullptr, nullptr), RAM_OK);
    d = desc(0);
    expect("ring B = 0", ring_attn_fwd_1gpu(&d, 4, 3, nullptr, FAKE, FAKE, &none, nullptr, nullptr, fake<float>(), FAKE,
                                            size_t(1) << 40, nullptr),
           RAM_OK);
  }
  std::printf("%d of %d cases as expected\n", g_cases - g_fail, g_cases);
  return g_fail;
}
