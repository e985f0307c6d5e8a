// Rows on 32-key MFMA tiles for gfx950 (MI355X): paged prefill (prompt rows attending
// causally to their request's keys through the page table, the normalised output written
// directly), and, in a chunked mode, decode windows of several rows at head dim 512 (each
// workgroup one key chunk of four rows, writing chunk states for the decode merge).
//
// pegainfer PR #1055 ("Description") runs the global family's prompt rows through a
// prefill over the split or folded pool; pegainfer PR #1057 ("Description") runs the
// sliding family's prompt rows through a varlen kernel with a window lower bound over
// pages of 64; TensorFold PR #1619 ("body") reads prompt rows through the slot's
// page-table row.  A row at position p sees the keys lo .. p (lo = p + 1 - window with a
// window): it is a decode token at length p + 1.
//
// One workgroup = row_tile consecutive prompt rows of one (request, KV head), as four
// waves.  A column block of 32 MFMA columns = (32 / G) rows x the G query heads of the KV
// head belongs to a pair of waves at head dim 512, which split the head dimension (256
// dims each: each holds half of the columns' query operand and half of their output), and
// to a single wave at head dim 256 (decode windows: to all four waves, 128 dims each).  Per 32-key tile (whole tiles inside one page: the
// page id is read once per tile):
//   * the tile's stored rows are copied from the pool straight into LDS with 16-byte
//     global->LDS loads (no registers involved), one kilobyte of one row per
//     instruction; the next tile is requested as soon as its buffer is free, so it lands
//     while the current one is used (decode windows stage through registers instead,
//     two tiles ahead).  Staged rows are 16 bytes apart beyond their length,
//     which keeps every LDS read pattern below free of bank conflicts and lets every
//     read address be a per-lane base plus a constant;
//   * each wave forms S^T = K Q^T over its dims on the 32x32x16 MFMA (keys as rows, (row,
//     head) as columns), K fragments read three steps ahead; the fp32 query, with
//     scale * log2(e) folded in, enters as a high and a low bf16 part, both multiplied
//     against each K fragment, so the scores keep ~16 mantissa bits.  Where waves split
//     the dims, their partial scores are added through LDS in a fixed order, so all waves
//     of a block hold the same scores bit for bit;
//   * causal and window masks by select (skipped on interior tiles); online softmax in
//     base 2;
//   * O^T += V^T P^T on the same MFMA for the wave's dims, the probabilities
//     again as high and low bf16 parts taken straight from the score registers; V^T is
//     assembled from LDS row reads with byte permutes.  V rows of keys no row of the
//     workgroup may see are zeroed on the way, so padding (NaN or huge) never reaches
//     the sums.
// The hot loop never rescales the accumulators (that would move them through the vector
// registers every tile): a column's reference maximum is fixed by its first tile with a
// visible key, when nothing has been accumulated yet, and probabilities may then grow to
// 2^kHeadroom (64 for bf16 operands, 15 for f16).  A larger score only raises a flag, and the workgroup recomputes its rows in
// a second loop that does rescale.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "plan_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescaleSlack = 8.0f;  // slow path: log2 units a tile may exceed the reference
constexpr int kKeys = kPrefillKeys;    // keys per tile: the 32 rows of one MFMA block
constexpr int kCols = 32;              // MFMA columns of a column block
// Buffer resource word 3 for raw (untyped) buffer loads on gfx9-family parts, and the
// loads' cache policy: non-temporal (bit 1 on gfx94x / gfx950) for decode windows, whose
// rows are read once; the default for prompts, whose neighbouring row tiles read the same
// keys again from L2 (measured on FP8 prompts: 10,602 rows 9.44 -> 9.36 ms, the 16 sliding
// prompts 2.80 -> 2.71 ms).
constexpr int kBufferWord3 = 0x00020000;
constexpr int kStreamLoad = 2;
constexpr int kReuseLoad = 0;
// Decode windows: tiles staged in registers ahead of the math.  Two keep the stream
// going; a third spills registers and measured slower.
constexpr int kStageSets = 2;

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

struct PrefillArgs {
  const float* q;
  float* out;
  const char* pool;
  const int32_t* table;
  const int32_t* seq_lens;
  const int32_t* q_starts;
  // Pool strides and column offsets in bytes; num_pages in pages.
  int64_t page_stride, head_stride, row_stride, k_offset, v_offset, num_pages;
  int32_t num_q_heads, page_size, max_pages, window, total_rows, max_rows, row_tiles;
  int32_t num_kv_heads, items;  // work items: row_tiles per (request, KV head)
  float qscale_k;  // scale * log2(e) * k_scale: query dims that meet K columns
  float qscale_v;  // scale * log2(e) * v_scale: folded query dims that meet V columns
  float vscale;    // v_scale, applied to the output
  // Decode windows (chunked): chunk states [request, row, head, chunk] (m, l) and
  // [.., D] (O), the chunking of the plan, rows per request, groups of four rows.
  float* part_m;
  float* part_l;
  float* part_o;
  int32_t chunk_len, num_chunks, num_rows, row_groups;
  int32_t chunk_len_odd;      // keys of odd-numbered chunks
  const uint64_t* row_masks;  // decode windows: per (request, row) window masks, or null
};

// Staged tile of kKeys stored rows (whole rows: K and V columns of the row format).
template <int D, bool FOLDED>
struct PStage {
  static constexpr int ROT = FOLDED ? 128 : 0;
  static constexpr int COLS = FOLDED ? ROT + D : 2 * D;  // staged elements per row
  static constexpr int ROW_BYTES = 2 * COLS;
  static constexpr int PITCH = ROW_BYTES + 16;            // staged row pitch in LDS
  static constexpr int TILE_BYTES = kKeys * PITCH;
  static constexpr int TV = FOLDED ? ROT : D;            // staged column of V[0]
  static constexpr int WAVES = 4;                        // waves per workgroup
  static constexpr int ROWS_PER_WAVE = kKeys / WAVES;    // staged rows a wave loads
  static constexpr int FULL_KB = ROW_BYTES / 1024;       // whole kilobytes of a row
  static constexpr int TAIL = ROW_BYTES % 1024;          // 0 or 256 bytes
  static_assert(TAIL == 0 || TAIL == 256, "a row is whole kilobytes plus at most 256 bytes");
};

// SPLIT waves share a column block, each holding D / SPLIT dims of its query operand,
// accumulators and K / V reads.
template <int D, bool FOLDED, int SPLIT>
struct PShape : PStage<D, FOLDED> {
  static constexpr int HALF = D / SPLIT;   // dims per wave
  static constexpr int KSTEPS = HALF / 16;  // 16-dim MFMA steps of QK
  static constexpr int DPR = HALF / 32;     // dims per lane per V row read
  static_assert(DPR == 8 || DPR == 4, "V reads of 16 or 8 bytes");
};

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ unsigned perm(unsigned hi, unsigned lo, unsigned sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// MFMA operand type of a pool element type: bf16 for bf16 and FP8 E4M3 rows (every E4M3
// value is a bf16 value), f16 for f16 rows; fp32 accumulation either way.
// D = A B + C on the 32x32x16 MFMA.  Lane l holds A[l % 32][8(l / 32) + j] and
// B[8(l / 32) + j][l % 32] (j = 0..7); element r of D is D[8(r / 4) + 4(l / 32) + r % 4][l % 32].
template <bool F16>
struct POps;

template <>
struct POps<false> {
  typedef __bf16 T;
  typedef bf16x8 T8;
  // Largest log2 distance a probability may sit above its column's reference in the
  // loop that never rescales (fp32 and bf16 reach 2^127).
  static constexpr float kHeadroom = 64.0f;
  static __device__ __forceinline__ floatx16 mma(u32x4 a, T8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(T8, a), b, c, 0, 0, 0);
  }
};

template <>
struct POps<true> {
  typedef _Float16 T;
  typedef halfx8 T8;
  static constexpr float kHeadroom = 15.0f;  // f16 reaches 65504 < 2^16
  static __device__ __forceinline__ floatx16 mma(u32x4 a, T8 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(T8, a), b, c, 0, 0, 0);
  }
};

// Two E4M3 codes (bytes 2HI, 2HI + 1 of w) to a packed bf16 pair: exact, since every E4M3
// value is a bf16 value.
template <int HI>
__device__ __forceinline__ unsigned widen8(unsigned w) {
  return __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI != 0));
}

// Page-table entry through the scalar cache (uniform index; the table is only read).
__device__ __forceinline__ int32_t table_entry(const int32_t* row, int idx) {
  typedef const int32_t __attribute__((address_space(4))) cint;
  return *(cint*)(row + __builtin_amdgcn_readfirstlane(idx));
}

// Byte offset inside the stored row of staged 256-byte piece sb (128 elements).
template <int D, bool FOLDED>
__device__ __forceinline__ int64_t piece_col(const PrefillArgs& a, int sb) {
  constexpr int VG = D / 128;
  if (FOLDED) return sb == 0 ? a.k_offset : a.v_offset + 256 * (sb - 1);
  return sb < VG ? a.k_offset + 256 * sb : a.v_offset + 256 * (sb - VG);
}

// Request one tile into `lds`.  `base` is the pool address of the tile's first row (page,
// KV head, slot).  Wave w stages rows w, w + WAVES, ...; each kilobyte of a row is one load
// instruction whose lane l brings the row's 16-byte chunk 64k + l (lanes 0..15 for a
// 256-byte tail), landing at M0 + 16l.  `off[k]` is this lane's byte offset of that chunk
// in the stored row, fixed for the whole kernel.
template <int D, bool FOLDED>
__device__ __forceinline__ void issue_tile(const PrefillArgs& a, const char* base, char* lds,
                                           int wave, int lane, const uint32_t (&off)[2]) {
  using S = PStage<D, FOLDED>;
#pragma unroll
  for (int i = 0; i < S::ROWS_PER_WAVE; ++i) {
    const int row = i * S::WAVES + wave;
    const char* rb = base + int64_t(row) * a.row_stride;
    char* lb = lds + row * S::PITCH;
#pragma unroll
    for (int k = 0; k < S::FULL_KB; ++k)
      __builtin_amdgcn_global_load_lds(rb + off[k], (lds_void*)(lb + 1024 * k), 16, 0, 0);
    if constexpr (S::TAIL != 0) {
      if (lane < 16)
        __builtin_amdgcn_global_load_lds(rb + off[1], (lds_void*)(lb + 1024), 16, 0, 0);
    }
  }
}

// Key (inside a tile) of k index 8 * hh + j of PV MFMA t: the scores of MFMA rows
// 8(r / 4) + 4hh + r % 4 with r = 8t + j, as they sit in the score registers.
__device__ __forceinline__ int pv_key(int t, int hh, int j) {
  return 16 * t + 8 * (j >> 2) + 4 * hh + (j & 3);
}

// Rows of one (request, KV head) against their keys, over the staged tiles.  Two uses:
//   * prefill (CHUNKED false): a work item is row_tile consecutive prompt rows; its keys
//     run from the first row's window start to the last row's position, and the
//     normalised output is written;
//   * a decode window of several rows (CHUNKED true, head dim 512): a work item is one key
//     chunk of one group of four rows (32 columns = 4 rows x 8 heads, each of the four
//     waves holding a quarter of the dims), and the chunk's unnormalised state (m in
//     natural-log units, l, O) is written for the merge, as by the one-row decode kernels.
template <int D, int G, bool FOLDED, bool CHUNKED, int KV>
__global__ __launch_bounds__(256, 1) void rows_tile_kernel(PrefillArgs a) {
  constexpr bool FP8 = KV == ATTN_KV_FP8_E4M3;
  using O = POps<KV == ATTN_KV_F16>;
  using T = typename O::T;
  using T8 = typename O::T8;
  constexpr int SPLIT = CHUNKED ? 4 : (D == 512 ? 2 : 1);  // waves sharing a column block
  // Staged through registers: decode windows (to keep tiles in flight) and FP8 pools (to
  // widen the codes to bf16 on their way into LDS).  Prefill keeps one tile ahead.
  constexpr bool REGS = CHUNKED || FP8;
  using S = PShape<D, FOLDED, SPLIT>;
  constexpr int P = S::PITCH;
  constexpr int HALF = S::HALF;
  constexpr int DPR = S::DPR;
  constexpr int RPP = kCols / G;               // rows per column block
  constexpr int W = S::WAVES;
  constexpr int QT = W / SPLIT * RPP;          // rows per workgroup
  static_assert(kCols % G == 0, "a column block holds whole rows");
  static_assert(!CHUNKED || D == 512, "decode windows on tiles: head dim 512");
  __shared__ __attribute__((aligned(1024))) char buf0[S::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char buf1[S::TILE_BYTES];
  __shared__ floatx4 xs[W][4][64];  // partial scores, one slot per wave
  __shared__ floatx4 ys[SPLIT == 4 ? W : 1][64];  // four-way exchange: summed score groups

  const int lane = threadIdx.x & 63;
  const int n = lane & 31;   // MFMA column: (row, head) of the block / key row of a K fragment
  const int hh = lane >> 5;  // k half of the MFMA operands / row group of the results
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int block = wave / SPLIT;  // column block
  const int half = wave % SPLIT;   // dims [half * HALF, (half + 1) * HALF)

  int g, r, qs0, nrows, row0, chunk = 0;
  if constexpr (CHUNKED) {
    // Launch order of the decode plan: the row groups of a chunk 8 slots apart, i.e. on
    // one XCD, so a later group finds the chunk's rows in that XCD's L2.
    const int lo8 = blockIdx.x % 8;
    const int hi8 = blockIdx.x / 8;
    chunk = (hi8 / a.row_groups) * 8 + lo8;
    if (chunk >= a.num_chunks) return;  // padding of the launch order (whole workgroup)
    g = blockIdx.y;
    r = blockIdx.z;
    nrows = a.num_rows;
    qs0 = r * nrows;
    row0 = (hi8 % a.row_groups) * QT;
  } else {
    // Launch slot -> work item.  Workgroups are handed to the eight XCDs in turn (slot w
    // runs on XCD w % 8), so runs of 32 consecutive items, i.e. neighbouring row tiles of
    // one (request, KV head) whose key ranges overlap, are given to one XCD and share its
    // L2; successive runs rotate over the XCDs.  The launch is padded to whole rounds of 256.
    const int w = blockIdx.x;
    const int slot = w >> 3;
    const int item = ((slot >> 5) * 8 + (w & 7)) * 32 + (slot & 31);
    if (item >= a.items) return;
    g = (item / a.row_tiles) % a.num_kv_heads;
    r = item / a.row_tiles / a.num_kv_heads;
    const int tile = a.row_tiles - 1 - item % a.row_tiles;  // the longest rows start first
    // Offsets the plan cannot serve are not followed: nothing is read or written.
    qs0 = a.q_starts[r];
    const int qs1 = a.q_starts[r + 1];
    nrows = qs1 - qs0;
    if (qs0 < 0 || nrows < 0 || nrows > a.max_rows || qs1 > a.total_rows) return;
    row0 = tile * QT;
    if (row0 >= nrows) return;
  }
  const int L = a.seq_lens[r];
  bool poison = L < nrows || int64_t(L) > int64_t(a.max_pages) * a.page_size;
  // Decode windows: chunks partition the keys from the request's first row's window start
  // (rounded down to a tile); they must cover the keys up to L.
  int64_t origin = 0;
  if constexpr (CHUNKED) {
    const int first_hi = L - nrows + 1;
    origin = (a.window > 0 ? max(0, first_hi - a.window) : 0) & ~(kKeys - 1);
    const int64_t pair = int64_t(a.chunk_len) + a.chunk_len_odd;
    const int64_t cover =
        int64_t(a.num_chunks >> 1) * pair + (a.num_chunks & 1) * int64_t(a.chunk_len);
    poison = poison || int64_t(L) - origin > cover;
  }

  // This lane's column: row qrow of the request, query head `head`; it sees keys lo_c .. pos
  // (none for an idle or poisoned column).  Decode windows: of the window's own keys
  // [wstart, L), only those whose bit key - wstart is set in the row's mask (causal rows:
  // bits 0 .. qrow, the same keys).
  const int qrow = row0 + block * RPP + n / G;
  const bool active = qrow < nrows;
  const int head = g * G + n % G;
  const int pos = (active && !poison) ? L - nrows + qrow : -1;
  const int lo_c = pos < 0 ? INT32_MAX : a.window > 0 ? max(0, pos + 1 - a.window) : 0;
  const int wstart = L - nrows;
  uint64_t mask = 0;
  if constexpr (CHUNKED) {
    if (active)
      mask = a.row_masks ? a.row_masks[int64_t(qs0) + qrow]
                         : (qrow >= 63 ? ~uint64_t(0) : (uint64_t(2) << qrow) - 1);
  }

  // Keys of the workgroup: the first row's window start .. the last row's position (a
  // decode window with masks: .. the last key; and inside the chunk).
  const int pos_first = L - nrows + row0;
  const int pos_last =
      (CHUNKED && a.row_masks) ? L - 1 : L - nrows + min(row0 + QT, nrows) - 1;
  const int lo_first = a.window > 0 ? max(0, pos_first + 1 - a.window) : 0;
  int start, ntiles;
  if constexpr (CHUNKED) {
    const int64_t c0 = origin + int64_t(chunk >> 1) * (int64_t(a.chunk_len) + a.chunk_len_odd) +
                       (chunk & 1) * int64_t(a.chunk_len);
    const int64_t c1 =
        min(c0 + ((chunk & 1) ? a.chunk_len_odd : a.chunk_len), int64_t(pos_last) + 1);
    start = int(min(c0, int64_t(L)));
    ntiles = (poison || c1 <= c0) ? 0 : int((c1 - c0 + kKeys - 1) / kKeys);
  } else {
    start = lo_first & ~(kKeys - 1);
    ntiles = poison ? 0 : (pos_last + 1 - start + kKeys - 1) / kKeys;
  }

  const int32_t* trow = a.table + int64_t(r) * a.max_pages;
  const char* head_base = a.pool + int64_t(g) * a.head_stride;
  // Pool address of the tile starting at key k0, or null if its page id is outside the pool.
  auto tile_base = [&](int k0) -> const char* {
    const int32_t pid = table_entry(trow, k0 / a.page_size);
    if (pid < 0 || int64_t(pid) >= a.num_pages) return nullptr;
    return head_base + int64_t(pid) * a.page_stride + int64_t(k0 % a.page_size) * a.row_stride;
  };

  // This lane's chunk of each staged kilobyte: chunk 64k + lane of the row, i.e. piece
  // 4k + lane / 16 (a tail of 256 bytes is piece 4 read by lanes 0..15).
  uint32_t off[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    off[k] = uint32_t(piece_col<D, FOLDED>(a, 4 * k + (S::TAIL != 0 && k == 1 ? 0 : lane >> 4))) +
             uint32_t((lane & 15) << 4);

  // Decode windows stage tiles through registers, kStageSets ahead of the math: each wave
  // loads its rows of a tile (the same 16-byte chunks per lane as the direct loads below)
  // and copies them into the tile's LDS buffer when its turn comes.  With the whole tile in
  // two 66 KB buffers, direct loads could keep only one tile in flight per CU.
  // The loads are buffer loads over the tile's rows, issued on every step whether or not
  // the tile is wanted: a tile past the end (or on a page outside the pool) gets an empty
  // range, so its loads return zeros without touching memory.  Every step then issues
  // the same loads, and the compiler's wait before a copy keeps the newer tile in flight.
  // FP8 rows: lane l < COLS / 16 holds stored codes 16l .. 16l + 15 of the staged row (K
  // or rotated K columns first, then V), widened to the bf16 of staged columns 16l ..
  constexpr int RW = S::ROWS_PER_WAVE;
  constexpr int NS = CHUNKED ? kStageSets : 1;  // register sets: tiles ahead of the math
  constexpr int KC = FOLDED ? S::ROT : D;        // staged K columns
  constexpr int FP8_LANES = S::COLS / 16;
  const uint32_t off8 = lane >= FP8_LANES ? 0x80000000u  // past the range: zeros, no access
                        : 16 * lane < KC ? uint32_t(a.k_offset) + 16 * lane
                                         : uint32_t(a.v_offset) + 16 * lane - KC;
  constexpr int kPolicy = CHUNKED ? kStreamLoad : kReuseLoad;
  u32x4 stg[NS][RW][2];
  auto fetch = [&](u32x4 (&st)[RW][2], int k0, bool want) -> bool {  // false: bad page
    const char* b = want ? tile_base(k0) : nullptr;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(b ? b : a.pool), 0, b ? 0x7fffffff : 0, kBufferWord3);
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const uint32_t ro = uint32_t(i * S::WAVES + wave) * uint32_t(a.row_stride);
      if constexpr (FP8) {
        st[i][0] = __builtin_amdgcn_raw_buffer_load_b128(
            rs, lane < FP8_LANES ? ro + off8 : 0x80000000u, 0, kPolicy);
        continue;
      }
#pragma unroll
      for (int k = 0; k < S::FULL_KB; ++k)
        st[i][k] = __builtin_amdgcn_raw_buffer_load_b128(rs, ro + off[k], 0, kPolicy);
      if constexpr (S::TAIL != 0)  // lanes 16.. ask past the range: zeros, no access
        st[i][1] = __builtin_amdgcn_raw_buffer_load_b128(rs, lane < 16 ? ro + off[1] : 0x80000000u,
                                                        0, kPolicy);
    }
    return b || !want;
  };
  auto stash = [&](const u32x4 (&st)[RW][2], char* lds) {
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      if constexpr (FP8) {
        if (lane < FP8_LANES) {
          char* lb = lds + (i * S::WAVES + wave) * P + 32 * lane;
          const u32x4 x = st[i][0];
          *reinterpret_cast<u32x4*>(lb) =
              u32x4{widen8<0>(x[0]), widen8<1>(x[0]), widen8<0>(x[1]), widen8<1>(x[1])};
          *reinterpret_cast<u32x4*>(lb + 16) =
              u32x4{widen8<0>(x[2]), widen8<1>(x[2]), widen8<0>(x[3]), widen8<1>(x[3])};
        }
        continue;
      }
      char* lb = lds + (i * S::WAVES + wave) * P + 16 * lane;
#pragma unroll
      for (int k = 0; k < S::FULL_KB; ++k) *reinterpret_cast<u32x4*>(lb + 1024 * k) = st[i][k];
      if constexpr (S::TAIL != 0) {
        if (lane < 16) *reinterpret_cast<u32x4*>(lb + 1024) = st[i][1];
      }
    }
  };
  // The first tiles (prefill: one, by direct loads) are requested before the query
  // operand is prepared, so they stream meanwhile.
  int count0 = ntiles;  // tiles whose pages were found (a missing page poisons the rest)
  auto prologue = [&]() {
    if constexpr (REGS) {
#pragma unroll
      for (int u = 0; u < NS; ++u)
        if (!fetch(stg[u], start + u * kKeys, count0 > u)) count0 = min(count0, u);
    } else {
      if (count0 > 0) {
        const char* b = tile_base(start);
        if (b)
          issue_tile<D, FOLDED>(a, b, buf0, wave, lane, off);
        else
          count0 = 0;
      }
    }
    if (count0 < ntiles) poison = true;
  };
  if constexpr (!CHUNKED) prologue();

  // Query operand (B of the QK MFMA): lane (n, hh), step s holds dims
  // half * HALF + 16s + 8hh + [0, 8) of column n, as a high and a low bf16 part.
  T8 qhi[S::KSTEPS], qlo[S::KSTEPS];
  {
    // Inactive columns read row 0 (always present) and use zeros.
    const float* qp = a.q + (int64_t(qs0) + (active ? qrow : 0)) * a.num_q_heads * D +
                      int64_t(head) * D + half * HALF + 8 * hh;
    floatx4 xq[S::KSTEPS][2];
#pragma unroll
    for (int s = 0; s < S::KSTEPS; ++s) {
      xq[s][0] = *reinterpret_cast<const floatx4*>(qp + 16 * s);
      xq[s][1] = *reinterpret_cast<const floatx4*>(qp + 16 * s + 4);
    }
    // Decode windows request their first tiles after the query loads, so that waiting
    // for the query leaves the tiles in flight.
    if constexpr (CHUNKED) prologue();
#pragma unroll
    for (int s = 0; s < S::KSTEPS; ++s) {
      const float qs = (FOLDED && half * HALF + 16 * s >= S::ROT) ? a.qscale_v : a.qscale_k;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = active ? xq[s][e >> 2][e & 3] * qs : 0.0f;
        const T h = (T)x;
        qhi[s][e] = h;
        qlo[s][e] = (T)(x - (float)h);
      }
      // Park the query operand in the accumulation registers, leaving the vector registers
      // to the output accumulators and the tile work (the QK products take their B operands
      // from there).
      asm volatile("" : "+a"(qhi[s]), "+a"(qlo[s]));
    }
  }

  // LDS read bases of this lane: K fragments of row n at dims half*HALF + 8hh (+ the step),
  // V of row 4hh at dims half*HALF + DPR*n (+ the key row).
  const int kbase = n * P + 16 * hh;
  const int vbase = 4 * hh * P + 2 * (S::TV + half * HALF + DPR * n);
  // Interior tiles: all rows of the workgroup present and every key of the tile visible to
  // all of them (at or after the last row's window start, at or before the first row;
  // decode windows: before the window's own keys).
  const bool full_tile = row0 + QT <= nrows;
  const int vis_end = CHUNKED ? wstart - 1 : pos_first;
  const int lo_last = a.window > 0 ? max(0, pos_last + 1 - a.window) : 0;

  float m_run, l_run;
  float m_top;              // decode windows: the largest score seen (the state's final m)
  floatx16 acc[DPR];        // step jj: element r <-> dim half*HALF + DPR*(8(r/4) + 4hh + r%4) + jj
  bool overflow = false;    // a score exceeded the reference by more than O::kHeadroom

  // One staged tile (keys k0 .. k0 + 31) for this wave's dims of its block's 32 columns.
  auto compute = [&](const char* t, int k0, auto rescale) {
    constexpr bool RESCALE = decltype(rescale)::value;
    // Partial scores over this wave's dims; the K fragments of step s + 1 are read while
    // step s multiplies.  Element e holds key 8(e/4) + 4hh + e%4 of column n.
    floatx16 sp = {}, sq = {};  // high and low query parts: two independent chains
    auto kfrag = [&](int s) {  // row n, dims half*HALF + 16s + 8hh .. + 8
      const int kd = half * HALF + 16 * s;
      const int col = (FOLDED && kd >= S::ROT) ? S::TV + kd : kd;
      return *reinterpret_cast<const u32x4*>(t + kbase + 2 * col);
    };
    constexpr int KA = 3;  // K fragments in flight ahead of the MFMAs
    u32x4 kq[KA];
#pragma unroll
    for (int s = 0; s < KA; ++s) kq[s] = kfrag(s);
#pragma unroll
    for (int s = 0; s < S::KSTEPS; ++s) {
      const u32x4 kf = kq[s % KA];
      if (s + KA < S::KSTEPS) kq[s % KA] = kfrag(s + KA);
      __builtin_amdgcn_sched_barrier(0);
      sp = O::mma(kf, qhi[s], sp);
      sq = O::mma(kf, qlo[s], sq);
      __builtin_amdgcn_sched_barrier(0);
    }
    sp += sq;
    float sc[16];
    if constexpr (SPLIT == 2) {
      // Add the pair's two halves in a fixed order (half 0 first): identical in both waves.
#pragma unroll
      for (int e = 0; e < 4; ++e)
        xs[wave][e][lane] = floatx4{sp[4 * e], sp[4 * e + 1], sp[4 * e + 2], sp[4 * e + 3]};
      __syncthreads();
      floatx4 other[4];  // all reads issued before the first add
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) other[e4] = xs[wave ^ 1][e4][lane];
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
#pragma unroll
        for (int i = 0; i < 4; ++i)  // (IEEE addition commutes: the same sum in both waves)
          sc[4 * e4 + i] = sp[4 * e4 + i] + other[e4][i];
    } else if constexpr (SPLIT == 4) {
      // Reduce-scatter, then all-gather, through LDS: wave `half` adds score group `half`
      // of the four quarters as (q0 + q1) + (q2 + q3) and publishes it; every wave then
      // reads the four sums, so all hold the same scores bit for bit (and each wave reads
      // 8 KB per tile instead of all 16 KB of partials).
#pragma unroll
      for (int e = 0; e < 4; ++e)
        xs[wave][e][lane] = floatx4{sp[4 * e], sp[4 * e + 1], sp[4 * e + 2], sp[4 * e + 3]};
      __syncthreads();
      const int w0 = block * SPLIT;
      floatx4 x[4];  // all reads issued before the first add
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = xs[w0 + u][half][lane];
      ys[wave][lane] = (x[0] + x[1]) + (x[2] + x[3]);
      __syncthreads();
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const floatx4 y = ys[w0 + e4][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[4 * e4 + i] = y[i];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[e] = sp[e];
    }
    // Tiles whose every key every row of the workgroup sees need no mask (uniform branch).
    if (!(full_tile && k0 >= lo_last && k0 + kKeys - 1 <= vis_end)) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = k0 + 8 * (e >> 2) + 4 * hh + (e & 3);
        bool vis;
        if constexpr (CHUNKED)
          vis = (key >= lo_c) & (key < L) &
                ((key < wstart) | bool((mask >> ((key - wstart) & 63)) & 1));
        else
          vis = (key >= lo_c) & (key <= pos);
        sc[e] = vis ? sc[e] : -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[e]);
    mx = fmaxf(mx, shfl_xor(mx, 32));
    if constexpr (CHUNKED) m_top = fmaxf(m_top, mx);
    if constexpr (RESCALE) {
      const bool grow = mx > m_run + kRescaleSlack;
      if (__builtin_expect(__any(grow), 0)) {
        // Columns of one wave see different key ranges: a column that keeps its maximum
        // keeps its sums (exp2(-inf - -inf) would be NaN for one with no visible key yet).
        const float m_new = grow ? mx : m_run;
        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // 0 from -inf
        l_run *= alpha;
#pragma unroll
        for (int jj = 0; jj < DPR; ++jj) acc[jj] *= alpha;
        m_run = m_new;
      }
    } else {
      if (m_run == -INFINITY) m_run = mx;  // first visible tile: nothing accumulated yet
      overflow |= mx > m_run + O::kHeadroom;
    }
    // Probabilities as the PV B operands: MFMA t takes elements 8t .. 8t + 7.
    // A reference still unset means every score of the column so far is -inf: any finite
    // stand-in gives the zero probabilities.
    T8 phi[2], plo[2];
    float psum = 0.0f;
    const float m_ref = m_run == -INFINITY ? 0.0f : m_run;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(sc[e] - m_ref);
      psum += p;
      const T h = (T)p;
      phi[e >> 3][e & 7] = h;
      plo[e >> 3][e & 7] = (T)(p - (float)h);
    }
    l_run += psum;

    // PV: A of MFMA t, step jj = V^T: lane (n, hh) holds dim half*HALF + DPR*n + jj of the
    // keys pv_key(t, hh, j).  Eight row reads of DPR dims, then byte permutes.
    const bool edge = k0 < lo_first || k0 + kKeys - 1 > pos_last;  // uniform
    auto vrows = [&](int tt, u32x4 (&w)[8]) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int o = (pv_key(tt, hh, j) - 4 * hh) * P;  // vbase: row 4hh, the lane's dims
        if constexpr (DPR == 8) {
          w[j] = *reinterpret_cast<const u32x4*>(t + vbase + o);
        } else {
          const u32x2 x = *reinterpret_cast<const u32x2*>(t + vbase + o);
          w[j] = u32x4{x[0], x[1], 0u, 0u};
        }
      }
    };
    // The V rows of MFMA 1 are read while MFMA 0's products run.
    u32x4 wv[2][8];
    vrows(0, wv[0]);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (tt == 0) vrows(1, wv[1]);
      u32x4 (&w)[8] = wv[tt];
      if (__builtin_expect(edge, 0)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int key = k0 + pv_key(tt, hh, j);
          const unsigned keep = ((key >= lo_first) & (key <= pos_last)) ? ~0u : 0u;
          w[j] &= u32x4{keep, keep, keep, keep};
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dd = 0; dd < DPR / 2; ++dd) {
        u32x4 ev, od;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          ev[u] = perm(w[2 * u + 1][dd], w[2 * u][dd], 0x05040100u);
          od[u] = perm(w[2 * u + 1][dd], w[2 * u][dd], 0x07060302u);
        }
        acc[2 * dd] = O::mma(ev, phi[tt], acc[2 * dd]);
        acc[2 * dd + 1] = O::mma(od, phi[tt], acc[2 * dd + 1]);
        acc[2 * dd] = O::mma(ev, plo[tt], acc[2 * dd]);
        acc[2 * dd + 1] = O::mma(od, plo[tt], acc[2 * dd + 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // All tiles of the work item through the two LDS buffers.
  auto run = [&](auto rescale) {
    m_run = -INFINITY;
    m_top = -INFINITY;
    l_run = 0.0f;
#pragma unroll
    for (int jj = 0; jj < DPR; ++jj) acc[jj] = floatx16{};
    int count = count0;
    if constexpr (REGS) {
      // Tile it sits in registers (fetched two steps earlier): copy it into its buffer
      // (free: every wave passed the last barrier after using it two tiles ago), refill
      // the registers with tile it + 2, wait for all waves' copies, use the buffer.
      auto step = [&](u32x4 (&st)[RW][2], int it) {
        char* cur = (it & 1) ? buf1 : buf0;
        stash(st, cur);
        if (!fetch(st, start + (it + NS) * kKeys, it + NS < count)) {
          poison = true;
          count = it + NS;
        }
        __syncthreads();
        compute(cur, start + it * kKeys, rescale);
      };
      // Whole rounds in the loop (every pass refills all register sets, in order), the
      // last tiles after it.
      int it = 0;
      for (; it + NS - 1 < count; it += NS) {
#pragma unroll
        for (int u = 0; u < NS; ++u) step(stg[u], it + u);
      }
#pragma unroll
      for (int u = 0; u < NS - 1; ++u)
        if (it + u < count) step(stg[u], it + u);
    } else {
      // Wait for this tile's loads (own, then everyone's via the barrier, which also frees
      // the other buffer and the score slots), request the next tile into the other
      // buffer, use this one.
      auto step = [&](const char* cur, char* nxt, int it) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        const int k0 = start + it * kKeys;
        if (it + 1 < count) {
          const char* b = tile_base(k0 + kKeys);
          if (b) {
            issue_tile<D, FOLDED>(a, b, nxt, wave, lane, off);
          } else {
            poison = true;
            count = it + 1;
          }
        }
        compute(cur, k0, rescale);
      };
      for (int it = 0; it < count; it += 2) {
        step(buf0, buf1, it);
        if (it + 1 < count) step(buf1, buf0, it + 1);
      }
    }
  };
  run(Flag<false>{});

  // Workgroup-wide OR of the overflow flags through the score slots.  The wave's vote is
  // taken with every lane active, before lane 0 stores it.
  const bool wave_overflow = __any(overflow);
  __syncthreads();
  if (lane == 0) xs[wave][0][0][0] = wave_overflow ? 1.0f : 0.0f;
  __syncthreads();
  bool any_overflow = false;
#pragma unroll
  for (int w = 0; w < W; ++w) any_overflow |= xs[w][0][0][0] != 0.0f;
  if (any_overflow) {  // uniform: every wave of the workgroup takes it
    __syncthreads();   // the flags have been read
    count0 = ntiles;
    prologue();
    run(Flag<true>{});
  }

  if (!active) return;
  if constexpr (CHUNKED) {
    // State relative to the chunk's largest score (the reference may lie below it).
    if (m_top > m_run) {
      const float al = __builtin_amdgcn_exp2f(m_run - m_top);
      l_run *= al;
#pragma unroll
      for (int jj = 0; jj < DPR; ++jj) acc[jj] *= al;
      m_run = m_top;
    }
  }
  l_run += shfl_xor(l_run, 32);
  const float qnan = __builtin_nanf("");
  // Prefill: O / l into the row.  Decode window: the chunk state; an empty one is
  // (-inf, 0, 0), a poisoned one NaN.
  float* o;
  float f;
  if constexpr (CHUNKED) {
    const int64_t st = ((int64_t(qs0) + qrow) * a.num_q_heads + head) * a.num_chunks + chunk;
    if (half == 0 && hh == 0) {
      a.part_m[st] = poison ? qnan : (m_run == -INFINITY ? -INFINITY : m_run * kLn2);
      a.part_l[st] = poison ? qnan : l_run;
    }
    o = a.part_o + st * D + half * HALF;
    f = a.vscale;
  } else {
    o = a.out + (int64_t(qs0) + qrow) * a.num_q_heads * D + int64_t(head) * D + half * HALF;
    f = a.vscale / l_run;
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int mrow = 8 * (e >> 2) + 4 * hh + (e & 3);
    float v[DPR];
#pragma unroll
    for (int jj = 0; jj < DPR; ++jj) v[jj] = poison ? qnan : acc[jj][e] * f;
    float* dst = o + DPR * mrow;
    *reinterpret_cast<floatx4*>(dst) = floatx4{v[0], v[1], v[2], v[3]};
    if constexpr (DPR == 8) *reinterpret_cast<floatx4*>(dst + 4) = floatx4{v[4], v[5], v[6], v[7]};
  }
}

template <int D, int G, bool FOLDED, bool CHUNKED>
void launch_rows_tile(const PrefillArgs& args, int kv_dtype, dim3 grid, hipStream_t s) {
  if (kv_dtype == ATTN_KV_FP8_E4M3)
    hipLaunchKernelGGL((rows_tile_kernel<D, G, FOLDED, CHUNKED, ATTN_KV_FP8_E4M3>), grid, dim3(256),
                       0, s, args);
  else if (kv_dtype == ATTN_KV_F16) {
    if constexpr (!CHUNKED)  // prompts only: decode windows over f16 rows run elsewhere
      hipLaunchKernelGGL((rows_tile_kernel<D, G, FOLDED, CHUNKED, ATTN_KV_F16>), grid, dim3(256),
                         0, s, args);
  } else {
    hipLaunchKernelGGL((rows_tile_kernel<D, G, FOLDED, CHUNKED, ATTN_KV_BF16>), grid, dim3(256),
                       0, s, args);
  }
}

// Pool geometry and query scaling shared by both uses.
void fill_common(PrefillArgs& args, const attn_decode_desc& d, const float* q,
                 const void* kv_pool, const int32_t* page_table, const int32_t* seq_lens) {
  const int64_t eb = kv_elem_bytes(d.kv_dtype);
  args = PrefillArgs{};
  args.q = q;
  args.pool = static_cast<const char*>(kv_pool);
  args.table = page_table;
  args.seq_lens = seq_lens;
  args.page_stride = d.page_stride * eb;
  args.head_stride = d.head_stride * eb;
  args.row_stride = d.row_stride * eb;
  args.k_offset = d.k_offset * eb;
  args.v_offset = d.v_offset * eb;
  args.num_pages = d.num_pages;
  args.num_q_heads = d.num_q_heads;
  args.num_kv_heads = d.num_kv_heads;
  args.page_size = d.page_size;
  args.max_pages = d.max_pages_per_seq;
  args.window = d.window;
  args.qscale_k = d.scale * kLog2e * d.k_scale;
  args.qscale_v = d.scale * kLog2e * d.v_scale;
  args.vscale = d.v_scale;
}

}  // namespace
}  // namespace attn

extern "C" int attn_prefill(const attn_prefill_plan_t* plan, const float* q, const void* kv_pool,
                            const int32_t* page_table, const int32_t* seq_lens,
                            const int32_t* q_starts, float* out, void* stream) {
  using namespace attn;
  int rc = check_prefill_plan(plan);
  if (rc != ATTN_OK) return rc;
  if (!q || !kv_pool || !page_table || !seq_lens || !q_starts || !out) return ATTN_E_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kv_pool) || !aligned16(out) || !aligned_to(page_table, 4) ||
      !aligned_to(seq_lens, 4) || !aligned_to(q_starts, 4))
    return ATTN_E_INVALID_ARG;
  const attn_decode_desc& d = plan->desc;
  if (!prefill_shape_supported(d)) return ATTN_E_UNSUPPORTED;
  if (plan->total_rows == 0) return ATTN_OK;

  if (d.kv_dtype == ATTN_KV_F32) {
    (void)hipGetLastError();
    launch_f32_prefill(*plan, q, kv_pool, page_table, seq_lens, q_starts, out, stream);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
  }
  PrefillArgs args;
  fill_common(args, d, q, kv_pool, page_table, seq_lens);
  args.out = out;
  args.q_starts = q_starts;
  args.total_rows = plan->total_rows;
  args.max_rows = plan->max_rows;
  args.row_tiles = plan->grid_x;
  args.items = plan->grid_x * d.num_kv_heads * d.batch;  // bounded by the plan

  const dim3 grid((args.items + 255) / 256 * 256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (d.head_dim == 512 && d.format == ATTN_KV_SPLIT)
    launch_rows_tile<512, 8, false, false>(args, d.kv_dtype, grid, s);
  else if (d.head_dim == 512 && d.format == ATTN_KV_FOLDED)
    launch_rows_tile<512, 8, true, false>(args, d.kv_dtype, grid, s);
  else
    launch_rows_tile<256, 2, false, false>(args, d.kv_dtype, grid, s);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

namespace attn {

void launch_rows_tiles(const attn_decode_plan_t& p, const float* q, const void* kv_pool,
                       const int32_t* page_table, const int32_t* seq_lens,
                       const uint64_t* row_masks, float* part_m, float* part_l, float* part_o,
                       void* stream) {
  const attn_decode_desc& d = p.desc;
  PrefillArgs args;
  fill_common(args, d, q, kv_pool, page_table, seq_lens);
  args.row_masks = row_masks;
  args.part_m = part_m;
  args.part_l = part_l;
  args.part_o = part_o;
  args.chunk_len = p.chunk_len;
  args.chunk_len_odd = p.chunk_len_odd;
  args.num_chunks = p.num_chunks;
  args.num_rows = p.num_rows;
  args.row_groups = p.row_groups;
  const dim3 grid(p.grid_x, d.num_kv_heads, d.batch);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d.format == ATTN_KV_FOLDED)
    launch_rows_tile<512, 8, true, true>(args, d.kv_dtype, grid, s);
  else
    launch_rows_tile<512, 8, false, true>(args, d.kv_dtype, grid, s);
}

}  // namespace attn
