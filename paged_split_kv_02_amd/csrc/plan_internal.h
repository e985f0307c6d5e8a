// Internal constants and helpers shared by the host plan and the launchers.
#pragma once

#include <stdint.h>

#include "../../include/attn_decode.h"

namespace attn {

constexpr uint64_t kPlanMagic = 0x5041474544534b56ull;  // "PAGEDSKV"
constexpr int kTile = 16;            // keys per tile = rows of one 16x16 MFMA block
constexpr int kWavesPerBlock = 4;    // one chunk per workgroup, one quarter per wave
constexpr int64_t kXcdSkewDiv = 20;    // even/odd chunks: +-1/20 of a quarter's tiles
constexpr int64_t kTargetWaves = 1024;  // 256 CUs x 4 SIMDs: one chunk-wave per SIMD
constexpr int kMergeGroups = 8;      // level-1 groups per (request, head) in the merge
constexpr int64_t kMaxRows = 64;     // query rows per request (multi-row windows)
// Key positions are 32-bit in the kernels, which add tile and lookahead offsets (at most a
// few hundred) to them: every position a plan admits stays this far below 2^31.
constexpr int64_t kPosMargin = 1024;
constexpr uint64_t kPrefillMagic = 0x4c4c494645525050ull;  // "PPREFILL"
constexpr int kPrefillKeys = 32;     // keys per prefill tile (one page holds whole tiles)
constexpr int kPrefillColumns = 64;  // (query row, head) columns per prefill workgroup (x2 at D=256)

// Bytes of one pool element of the given type, 0 for an unknown type.
int kv_elem_bytes(int kv_dtype);
// Element types the partial kernels read.
bool kv_dtype_served(int kv_dtype);
bool shape_supported(const attn_decode_desc& d);
int64_t row_extent(const attn_decode_desc& d);
int make_plan(const attn_decode_desc* desc, const int32_t* lens, attn_decode_plan_t* plan);
int check_desc(const attn_decode_desc& d);
bool prefill_shape_supported(const attn_decode_desc& d);
int make_prefill_plan(const attn_decode_desc* desc, const int32_t* lens, const int32_t* q_starts,
                      attn_prefill_plan_t* plan);
int check_prefill_plan(const attn_prefill_plan_t* plan);
// Decode windows of several rows at head dim 512 over bf16 or FP8 pages of whole 32-key tiles
// (with in-row offsets below 2^31 bytes) run on the 32-key MFMA tile kernel, in chunks
// of whole 32-key tiles; other shapes on the 16-key rows kernel.
bool rows_on_tiles(const attn_decode_desc& d, int64_t rows);
// row_masks: null for causal rows, else one 64-bit mask per (request, row) (tree attention).
void launch_rows_tiles(const attn_decode_plan_t& p, const float* q, const void* kv_pool,
                       const int32_t* page_table, const int32_t* seq_lens,
                       const uint64_t* row_masks, float* part_m, float* part_l, float* part_o,
                       void* stream);
// Prefill over an f32 pool on the f32 decode kernel's prefill mode.
void launch_f32_prefill(const attn_prefill_plan_t& p, const float* q, const void* kv_pool,
                        const int32_t* page_table, const int32_t* seq_lens, const int32_t* q_starts,
                        float* out, void* stream);
int check_plan(const attn_decode_plan_t* plan);
int check_workspace(const attn_decode_plan_t* plan, const void* ws, size_t bytes);

// Device buffers the kernels move in 16-byte vectors (query, pool, output, K/V rows), and
// the natural alignment of the 4- and 8-byte words they read (table, lengths, masks).
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline bool aligned_to(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

}  // namespace attn
