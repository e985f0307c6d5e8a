// Paged split-KV decode attention for gfx950 (MI355X): partial and merge kernels
// and the C-ABI entry points that launch them.
//
// Partial kernel (one workgroup = one key chunk of one (request, KV head); each of
// its four waves streams a quarter of the chunk and the quarters are merged in LDS):
//   * the G query heads of a KV head share every K/V byte the wave streams; each
//     row is fetched from HBM once (gem design note, "Candidate ownership and
//     storage": stage each K row once for the eight query heads);
//   * the page id is resolved once per 16-key tile, never per key (TensorFold
//     PR #1619, review thread: per-tile lookup instead of per-key);
//   * QK^T and PV run on MFMA.  The 16 output columns of a 16x16 MFMA hold the G
//     heads twice: a high and a low bf16 part of the fp32 query (and of the fp32
//     probabilities), so the products keep ~16 mantissa bits while the inputs
//     stay bf16, and no column is padding when G = 8;
//   * online softmax in base 2 with scale*log2(e) folded into the query; the
//     reference maximum moves only when a tile exceeds it by 2^8, so the
//     accumulators are rarely rescaled; the stored reference is converted back
//     to natural-log units (any reference <= the chunk maximum is a valid state);
//   * masked keys (past L, before the window, padding slots of the last page)
//     are excluded by select, and their V rows are zeroed before PV, so NaN or
//     huge padding never reaches the sums;
//   * pool element types: bf16 and f16 rows are staged as stored and multiplied on
//     the MFMA of their own type; FP8 E4M3 rows are fetched at half the bytes and
//     widened to bf16 (exactly): for one query row by a kernel of their own that stages
//     the codes in LDS as stored and widens them as it reads its operands, for several
//     rows on their way into LDS.  The dequantisation factors fold into the query (K)
//     and into the written state (V).
// Merge (one launch): level 1 folds runs of consecutive chunk states into group
// states held in LDS, out of place; level 2 folds the group states in order and
// divides (pegainfer PR #1055, "Description": merge in two levels; gem design note,
// "Candidate ownership and storage" for the identity).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "plan_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef _Float16 halfx4 __attribute__((ext_vector_type(4)));
typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

struct SplitArgs {
  const float* q;
  const char* pool;
  const int32_t* table;
  const int32_t* seq_lens;
  float* part_m;
  float* part_l;
  float* part_o;
  // Pool strides and column offsets in bytes.
  int64_t page_stride, head_stride, row_stride, k_offset, v_offset, num_pages;
  int32_t num_q_heads, page_size, max_pages, window, chunk_len, num_chunks;
  int32_t chunk_len_odd;  // keys of odd-numbered chunks (one row; else == chunk_len)
  int32_t num_rows, row_groups;  // query rows per request; groups of 4 rows (multi-row kernel)
  // Several rows: bit j of row_masks[r * num_rows + i] lets row i see the key of window
  // row j (tree attention); null means causal rows.
  const uint64_t* row_masks;
  float qscale_k;  // scale * log2(e) * k_scale: the query dims that meet K columns
  float qscale_v;  // scale * log2(e) * v_scale: folded query dims that meet V columns
  float vscale;    // v_scale, applied to the written numerators
  // Prompt rows (the f32 kernel's prefill mode): request r's new rows are q_starts[r] ..
  // q_starts[r + 1] of q and out; normalised rows are written to out.
  const int32_t* q_starts;
  float* out;
  int32_t total_rows, max_rows;
  int32_t row_tiles, items, num_kv_heads;  // prompt rows: work items (row tiles x KV heads x requests)
};

// Keys covered by the first c chunks (even chunks chunk_len, odd ones chunk_len_odd).
__device__ __forceinline__ int64_t chunk_cover(const SplitArgs& a, int c) {
  return int64_t(c >> 1) * (a.chunk_len + a.chunk_len_odd) + (c & 1) * int64_t(a.chunk_len);
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// Value of the lane holding the other bf16 part of the same head: column c ^ G
// inside each 16-lane row (row rotation by 8 for G = 8, quad swap for G = 2).
template <int G>
__device__ __forceinline__ float partner(float v) {
  static_assert(G == 8 || G == 2, "pairing defined for 8 or 2 heads per KV head");
  const int x = __builtin_bit_cast(int, v);
  const int y = G == 8 ? __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false)   // row_ror:8
                       : __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
  return __builtin_bit_cast(float, y);
}

// Uniform read of a page-table entry through the scalar cache (the table is never
// written by these kernels).
__device__ __forceinline__ int32_t load_page_id(const int32_t* row, int idx) {
  typedef const int32_t __attribute__((address_space(4))) cint;
  return *(cint*)(row + __builtin_amdgcn_readfirstlane(idx));
}

// The running maximum of a chunk is only moved when a tile's maximum exceeds it
// by more than this (log2 units); until then probabilities stay below 2^8.  Any
// reference at or below the true maximum gives a valid state for the merge.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ unsigned perm(unsigned hi, unsigned lo, unsigned sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Stored element types.  A lane fetches 8 consecutive elements of a row at a time
// (16 bytes of bf16/f16, 8 bytes of FP8) with a streaming load that does not keep the
// line in the caches, and widens them to 8 MFMA operand elements (16 bytes) before
// they are written to LDS.  kAhead = key tiles a wave of the single-row kernel keeps
// in flight (32 KB per wave at head dim 512).
template <int KV>
struct Elem;

template <>
struct Elem<ATTN_KV_BF16> {
  static constexpr int kBytes = 2;
  static constexpr bool kF16 = false;  // operand type: bf16
  static constexpr int kAhead = 1;
  typedef u32x4 Raw;
  static __device__ __forceinline__ Raw load(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  static __device__ __forceinline__ u32x4 widen(Raw r) { return r; }
};

template <>
struct Elem<ATTN_KV_F16> : Elem<ATTN_KV_BF16> {
  static constexpr bool kF16 = true;  // operand type: f16
};

// FP8 E4M3 (OCP): every E4M3 value (subnormals included) is exactly a bf16 value, and
// gfx950's v_cvt_scalef32_pk_bf16_fp8 with scale 1 converts two codes straight to a
// packed bf16 pair.
template <>
struct Elem<ATTN_KV_FP8_E4M3> {
  static constexpr int kBytes = 1;
  static constexpr bool kF16 = false;
  typedef u32x2 Raw;
  static __device__ __forceinline__ Raw load(const char* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  }
  static __device__ __forceinline__ u32x4 widen(Raw r) {
    u32x4 out;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      out[2 * i] = __builtin_bit_cast(                                       // bytes 0, 1
          unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[i], 1.0f, false));
      out[2 * i + 1] = __builtin_bit_cast(                                   // bytes 2, 3
          unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[i], 1.0f, true));
    }
    return out;
  }
};

// MFMA operand type: bf16 or f16, with fp32 accumulation either way.
template <bool F16>
struct Ops;

template <>
struct Ops<false> {
  typedef __bf16 T;
  typedef bf16x8 T8;
  typedef bf16x4 T4;
  static __device__ __forceinline__ floatx4 mma32(T8 a, T8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ floatx4 mma16(T4 a, T4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
  }
};

template <>
struct Ops<true> {
  typedef _Float16 T;
  typedef halfx8 T8;
  typedef halfx4 T4;
  static __device__ __forceinline__ floatx4 mma32(T8 a, T8 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ floatx4 mma16(T4 a, T4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
};

// LDS tile: the 16 stored rows of one key tile, padded by 16 bytes per row.
// Staging writes (one row, 16 consecutive 16-byte pieces per 16-lane pass) and the
// QK reads (16 rows, one column per pass) both fall in distinct banks.
template <int COLS>
struct alignas(16) RowTile {
  static constexpr int kPitch = COLS + 8;  // elements
  uint16_t v[kTile * kPitch];
};

// Compile-time shape of one partial kernel instance.
template <int D, bool FOLDED>
struct Shape {
  static constexpr int KSTEPS = D / 32;    // 16x16x32 MFMA steps over the key dimension
  static constexpr int VGROUPS = D / 128;  // 128-dim slabs of V per tile
  static constexpr int ROT = FOLDED ? 128 : 0;
  // Columns staged per row: split K | V (2D), folded rotated K | V (ROT + D).
  static constexpr int COLS = FOLDED ? ROT + D : 2 * D;
  static constexpr int SLABS = COLS / 128;  // 256-byte pieces per row
  static constexpr int P = RowTile<COLS>::kPitch;
  static constexpr int TV = FOLDED ? ROT : D;  // staged column of V[0]
};

// Query operand of lane (c, qg) for one query row: column c holds head (c % G) of KV
// head g, the high operand-type part of q*scale*log2(e)*factor for c < G, the low
// remainder for G <= c < 2G, zero beyond; k-step j covers dims 32j + 8qg + [0, 8).
// Dims below kdims meet K columns (factor k_scale), the others V columns (v_scale).
template <int D, int G, bool F16>
__device__ __forceinline__ void make_query_operand(const float* qrow_heads, int g, int c, int qg,
                                                   float qscale_k, float qscale_v, int kdims,
                                                   typename Ops<F16>::T8 (&qop)[D / 32]) {
  using T = typename Ops<F16>::T;
  const int part = c / G;
  const float* qrow = qrow_heads + int64_t(g * G + c % G) * D;
#pragma unroll
  for (int j = 0; j < D / 32; ++j) {
    typename Ops<F16>::T8 v;
    const float qs = 32 * j < kdims ? qscale_k : qscale_v;
    if (part < 2) {
      const floatx4 x0 = *reinterpret_cast<const floatx4*>(qrow + 32 * j + 8 * qg);
      const floatx4 x1 = *reinterpret_cast<const floatx4*>(qrow + 32 * j + 8 * qg + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (e < 4 ? x0[e & 3] : x1[e & 3]) * qs;
        const T h = (T)x;
        v[e] = part == 0 ? h : (T)(x - (float)h);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (T)0.0f;
    }
    qop[j] = v;
  }
}

// One staged tile of 16 keys for one query row: QK^T on MFMA, online softmax over the
// keys tok0 + 4qg + i visible to the row (lo <= key < hi, and with MASKED, a key at or
// past wstart, i.e. a key of the row window, only if its bit key - wstart of `mask` is
// set), PV on MFMA.  The caller has zeroed the V rows of keys no row may see.
template <int D, int G, bool FOLDED, bool F16, bool MASKED = false>
__device__ __forceinline__ void tile_math(const uint16_t* tile, int tok0, int lo, int hi,
                                          const typename Ops<F16>::T8 (&qop)[D / 32], int c,
                                          int qg, float& m_run, float& l_run,
                                          floatx4 (&acc)[D / 128][8], int wstart = 0,
                                          uint64_t mask = 0) {
  using S = Shape<D, FOLDED>;
  using O = Ops<F16>;
  using T = typename O::T;
  const int part = c / G;
  // Scores of 16 keys x 16 columns (hi/lo parts of the G heads).  Key dim kd sits at
  // staged column kd (split / rotated part) or TV + kd (folded, kd >= ROT).
  floatx4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < S::KSTEPS; ++j) {
    const int kd = 32 * j + 8 * qg;
    const int col = (FOLDED && kd >= S::ROT) ? S::TV + kd : kd;
    const u32x4 kv = *reinterpret_cast<const u32x4*>(tile + c * S::P + col);
    s = O::mma32(__builtin_bit_cast(typename O::T8, kv), qop[j], s);
  }

  // Online softmax (base 2); lane holds keys tok0 + 4qg + i.
  float sc[4];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float full = s[i] + partner<G>(s[i]);
    const int t = tok0 + 4 * qg + i;
    bool vis = t >= lo && t < hi;
    if constexpr (MASKED) vis = vis && (t < wstart || ((mask >> ((t - wstart) & 63)) & 1));
    sc[i] = vis ? full : -INFINITY;
    mx = fmaxf(mx, sc[i]);
  }
  mx = fmaxf(mx, shfl_xor(mx, 16));
  mx = fmaxf(mx, shfl_xor(mx, 32));
  // Move the reference maximum only when this tile exceeds it by the slack.
  const bool grow = mx > m_run + kRescaleSlack;
  if (__builtin_expect(__any(grow), 0)) {
    const float m_new = grow ? mx : m_run;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 from -inf
    l_run *= alpha;
#pragma unroll
    for (int b = 0; b < S::VGROUPS; ++b)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) acc[b][jj] *= alpha;
    m_run = m_new;
  }
  float p[4] = {0.f, 0.f, 0.f, 0.f};
  if (m_run != -INFINITY) {
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] - m_run);
  }
  l_run += (p[0] + p[1]) + (p[2] + p[3]);
  typename O::T4 pop;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const T h = (T)p[i];
    const T l = (T)(p[i] - (float)h);
    pop[i] = part == 0 ? h : (part == 1 ? l : (T)0.0f);
  }

  // PV: lane row c of slab b, step jj <-> dim 128b + 8c + jj; keys 4qg + [0, 4).  The
  // transposed V operand is built from four 16-byte row reads with byte permutes
  // (on gfx950 this measured faster than the LDS transpose load for this tile).
#pragma unroll
  for (int b = 0; b < S::VGROUPS; ++b) {
    u32x4 w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = *reinterpret_cast<const u32x4*>(tile + (4 * qg + e) * S::P + S::TV + 128 * b + 8 * c);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x2 even = {perm(w[1][u], w[0][u], 0x05040100u), perm(w[3][u], w[2][u], 0x05040100u)};
      const u32x2 odd = {perm(w[1][u], w[0][u], 0x07060302u), perm(w[3][u], w[2][u], 0x07060302u)};
      acc[b][2 * u] = O::mma16(__builtin_bit_cast(typename O::T4, even), pop, acc[b][2 * u]);
      acc[b][2 * u + 1] = O::mma16(__builtin_bit_cast(typename O::T4, odd), pop, acc[b][2 * u + 1]);
    }
  }
}

// Zero the V rows of a staged tile whose keys lie outside [lo, hi), for the 4 rows
// 4qg + e this lane group owns, so padding cannot leak through 0 * NaN.
template <int D, bool FOLDED>
__device__ __forceinline__ void zero_dead_rows(uint16_t* tile, int tok0, int lo, int hi, int c,
                                               int qg, int e0, int e1) {
  using S = Shape<D, FOLDED>;
#pragma unroll
  for (int e = e0; e < e1; ++e) {
    const int t = tok0 + 4 * qg + e;
    if (t < lo || t >= hi) {
#pragma unroll
      for (int b = 0; b < S::VGROUPS; ++b)
        *reinterpret_cast<u32x4*>(tile + (4 * qg + e) * S::P + S::TV + 128 * b + 8 * c) =
            u32x4{0u, 0u, 0u, 0u};
    }
  }
}

// Byte offset in the stored row of staged piece sb (128 elements each).
template <int D, bool FOLDED, int EB>
__device__ __forceinline__ int64_t src_col(const SplitArgs& a, int sb) {
  constexpr int VG = D / 128;
  if (FOLDED) return sb == 0 ? a.k_offset : a.v_offset + 128 * EB * (sb - 1);
  return sb < VG ? a.k_offset + 128 * EB * sb : a.v_offset + 128 * EB * (sb - VG);
}

// Page ids of one table row, read once per page through the scalar cache with the next
// page's id fetched a page ahead.  Lookups must be monotone in position.
struct PageWalker {
  const int32_t* trow;
  int64_t num_pages;
  int page_size, max_pages, cur_page;
  int32_t cur_pid, next_pid;
  __device__ __forceinline__ void start(int tok) {  // tok inside the table row
    cur_page = tok / page_size;
    cur_pid = load_page_id(trow, cur_page);
    const int32_t nxt = load_page_id(trow, min(cur_page + 1, max_pages - 1));  // no branch
    next_pid = cur_page + 1 < max_pages ? nxt : -1;
  }
  // Page id of position tok (a tile never straddles two pages), -1 if outside the pool.
  __device__ __forceinline__ int32_t page_of(int tok) {
    const int page = tok / page_size;
    if (page != cur_page) {
      cur_page = page;
      cur_pid = next_pid;
      next_pid = page + 1 < max_pages ? load_page_id(trow, page + 1) : -1;
    }
    return (cur_pid < 0 || int64_t(cur_pid) >= num_pages) ? -1 : cur_pid;
  }
};

// (m, l, O) of the G heads of one wave's quarter of a chunk, parked in LDS for the
// workgroup merge (m in log2 units, NaN for a poisoned quarter).
template <int D, int G>
struct QuarterState {
  float m[G], l[G];
  floatx4 o[G][D / 4];
};

// Workgroup merge of the four quarter states (fixed order) into the chunk's state,
// head by head, 4 dims per thread; written in natural-log units with O times v_scale.
template <int D, int G>
__device__ __forceinline__ void write_chunk_state(const SplitArgs& a,
                                                  const QuarterState<D, G>* const (&parked)[kWavesPerBlock],
                                                  int r, int g, int chunk) {
  const float qnan = __builtin_nanf("");
  for (int idx = threadIdx.x; idx < G * (D / 4); idx += 64 * kWavesPerBlock) {
    const int h = idx / (D / 4);
    const int d4 = idx % (D / 4);
    float M = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
      const float x = parked[w]->m[h];
      nan |= x != x;
      M = fmaxf(M, x);
    }
    float S = 0.0f;
    floatx4 O = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWavesPerBlock; ++w) {
        const float x = parked[w]->m[h];
        const float wt = x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x - M);
        S += wt * parked[w]->l[h];
        O += wt * parked[w]->o[h][d4];
      }
    }
    const int64_t st = (int64_t(r) * a.num_q_heads + g * G + h) * a.num_chunks + chunk;
    if (nan) {
      M = S = qnan;
      O = floatx4{qnan, qnan, qnan, qnan};
    }
    if (d4 == 0) {
      a.part_m[st] = M == -INFINITY ? -INFINITY : M * kLn2;
      a.part_l[st] = S;
    }
    *reinterpret_cast<floatx4*>(a.part_o + st * D + 4 * d4) = O * a.vscale;
  }
}

template <int D, int G, bool FOLDED, int KV>
__global__ __launch_bounds__(256, 1) void split_partial_kernel(SplitArgs a) {
  using S = Shape<D, FOLDED>;
  using E = Elem<KV>;
  constexpr int KSTEPS = S::KSTEPS;
  constexpr int COLS = S::COLS;
  constexpr int SLABS = S::SLABS;
  constexpr int P = S::P;
  constexpr int EB = E::kBytes;
  // Tiles staged ahead in registers (one query row over FP8 rows: fp8_ring_kernel).
  constexpr int kAhead = E::kAhead;
  static_assert(KV != ATTN_KV_FP8_E4M3, "FP8 rows take the ring kernel");
  static_assert(2 * G <= 16, "hi/lo columns must fit one 16-wide MFMA block");
  __shared__ RowTile<COLS> tiles[kWavesPerBlock];

  const int lane = threadIdx.x & 63;
  const int c = lane & 15;   // MFMA row/column index inside a 16-block
  const int qg = lane >> 4;  // lane group: selects k sub-range / output rows
  const int wave = threadIdx.x >> 6;
  const int chunk = blockIdx.x;  // one chunk per workgroup, one quarter per wave
  const int g = blockIdx.y;
  const int r = blockIdx.z;
  uint16_t* tile = tiles[wave].v;

  const int64_t cap = int64_t(a.max_pages) * a.page_size;
  const int quarter = ((chunk & 1) ? a.chunk_len_odd : a.chunk_len) / kWavesPerBlock;
  PageWalker pw{a.table + int64_t(r) * a.max_pages, a.num_pages, a.page_size, a.max_pages, 0, -1, -1};
  // Without a window the quarter's first position does not depend on the length, so its
  // page ids are requested before the length is read (the two loads overlap).
  const int c0_nw = int(chunk_cover(a, chunk)) + wave * quarter;
  const bool early = a.window == 0 && c0_nw < cap;
  pw.start(early ? c0_nw : 0);  // unconditional: no wait before the length is requested

  const int L = a.seq_lens[r];
  const int lo = (a.window > 0 && L > a.window) ? L - a.window : 0;
  const int start = lo & ~(kTile - 1);
  bool poison = L < 1 || int64_t(L) > cap ||
                int64_t(L) - start > chunk_cover(a, a.num_chunks);
  const int c0 = start + int(chunk_cover(a, chunk)) + wave * quarter;
  const int c1 = min(c0 + quarter, L);
  int end = (!poison && c0 < c1) ? c1 : c0;  // tiles from `end` on are not processed
  const char* head_base = a.pool + int64_t(g) * a.head_stride;
  typename E::Raw stage[kAhead][4][SLABS];

  // Fetch one tile into a register set.  Lane (c, qg) reads rows 4qg + e, 8 elements at
  // 128 sb + 8c: every instruction covers four whole row pieces, so each line is
  // requested once.  A table entry outside the pool poisons the chunk and ends it.
  auto fetch = [&](typename E::Raw (&buf)[4][SLABS], int tok0) {
    const int32_t pid = pw.page_of(tok0);
    if (pid < 0) {
      poison = true;
      end = tok0;
      return;
    }
    const char* base = head_base + int64_t(pid) * a.page_stride +
                       int64_t(tok0 % a.page_size) * a.row_stride + 8 * EB * c;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const char* row = base + int64_t(4 * qg + e) * a.row_stride;
#pragma unroll
      for (int sb = 0; sb < SLABS; ++sb) buf[e][sb] = E::load(row + src_col<D, FOLDED, EB>(a, sb));
    }
  };

  // Start streaming the first tiles before the query is prepared.
  if (c0 < end) {
    if (!early) pw.start(c0);
#pragma unroll
    for (int k = 0; k < kAhead; ++k)
      if (c0 + k * kTile < end) fetch(stage[k], c0 + k * kTile);
  }

  typename Ops<E::kF16>::T8 qop[KSTEPS];
  make_query_operand<D, G, E::kF16>(a.q + int64_t(r) * a.num_q_heads * D, g, c, qg, a.qscale_k,
                                    a.qscale_v, FOLDED ? S::ROT : D, qop);

  float m_run = -INFINITY;
  float l_run = 0.0f;
  floatx4 acc[D / 128][8];  // slab b, step jj: lane (c, qg) rows 4qg + i <-> dims 128b + 8(4qg+i) + jj
#pragma unroll
  for (int b = 0; b < D / 128; ++b)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc[b][jj] = floatx4{0.f, 0.f, 0.f, 0.f};

  // One tile: widen and stage it, refill its registers kAhead tiles ahead, mask, math.
  auto step = [&](typename E::Raw (&regs)[4][SLABS], int tok0) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int sb = 0; sb < SLABS; ++sb)
        *reinterpret_cast<u32x4*>(tile + (4 * qg + e) * P + 128 * sb + 8 * c) = E::widen(regs[e][sb]);
    if (tok0 + kAhead * kTile < end) fetch(regs, tok0 + kAhead * kTile);
    // Keys outside [lo, L): first tile of a window, tail of the last page.
    if (__builtin_expect(tok0 < lo || tok0 + kTile > L, 0))
      zero_dead_rows<D, FOLDED>(tile, tok0, lo, L, c, qg, 0, 4);
    tile_math<D, G, FOLDED, E::kF16>(tile, tok0, lo, L, qop, c, qg, m_run, l_run, acc);
  };
  for (int tok0 = c0; tok0 < end; tok0 += kAhead * kTile) {
#pragma unroll
    for (int k = 0; k < kAhead; ++k) {
      if (tok0 + k * kTile >= end) break;
      step(stage[k], tok0 + k * kTile);
    }
  }

  // Quarter state: sum l over the lane groups, add the low columns onto the high ones.
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
#pragma unroll
  for (int b = 0; b < D / 128; ++b)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[b][jj][i] += partner<G>(acc[b][jj][i]);

  // Workgroup merge of the four quarters (fixed order) into the chunk's state.  Each
  // wave parks (m, l, O) of its G heads in its own LDS tile; after the barrier the
  // workgroup folds them.
  using Parked = QuarterState<D, G>;
  static_assert(sizeof(Parked) <= sizeof(RowTile<COLS>), "parked state must fit the tile");
  Parked* mine = reinterpret_cast<Parked*>(tile);
  const float qnan = __builtin_nanf("");
  if (c < G) {
    if (qg == 0) {
      mine->m[c] = poison ? qnan : m_run;  // log2 units, -inf when empty
      mine->l[c] = l_run;
    }
#pragma unroll
    for (int b = 0; b < D / 128; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 128 * b + 32 * qg + 8 * i;  // dims d .. d + 7
        mine->o[c][d / 4] = floatx4{acc[b][0][i], acc[b][1][i], acc[b][2][i], acc[b][3][i]};
        mine->o[c][d / 4 + 1] = floatx4{acc[b][4][i], acc[b][5][i], acc[b][6][i], acc[b][7][i]};
      }
  }
  __syncthreads();
  const Parked* parked[kWavesPerBlock];
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) parked[w] = reinterpret_cast<const Parked*>(tiles[w].v);
  write_chunk_state<D, G>(a, parked, r, g, chunk);
}

// ---------------------------------------------------------------------------------------
// FP32 pools (the KV type of the gem design note's "Fixed production shape"): products in
// full fp32 on v_mfma_f32_16x16x4_f32, so nothing is split into parts.  A wave copies the
// K half, then the V half, of a 16-key tile of whole rows into its own LDS region with
// non-temporal 16-byte global->LDS loads (no registers carry them); at head dim 512
// through a ring of eight slots, seven pieces in flight while it computes on the eighth.
// Each wave works alone until the workgroup merge of the quarter states.
//   A (16 x 4): lane l holds A[l % 16][l / 16];  B (4 x 16): B[l / 16][l % 16];
//   C (16 x 16): element i of lane l is C[4(l / 16) + i][l % 16].
typedef __attribute__((address_space(3))) void lds_void;
// Cache policy of the rows' global->LDS loads: non-temporal, as for the streaming loads of
// the other decode kernels (each row is read once per launch).  With the default policy
// the f32 kernel streamed at ~5.1 TB/s at 163,336 tokens and ~3.1 TB/s on the sliding
// batch; non-temporal, ~6.4 and ~5.4 TB/s.
constexpr int kStreamLds = 2;

__device__ __forceinline__ floatx4 mma_f32(float a, float b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// A compile-time int for the loop bounds of the per-tile lambdas.
template <int N>
struct Int {
  static constexpr int value = N;
};

// Wait until at most N vector memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void vm_wait_lt() {
  static_assert(N >= 0 && N <= 28 && N % 4 == 0, "counts of whole 4-load pieces");
  if constexpr (N == 28) asm volatile("s_waitcnt vmcnt(28)" ::: "memory");
  else if constexpr (N == 24) asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
  else if constexpr (N == 20) asm volatile("s_waitcnt vmcnt(20)" ::: "memory");
  else if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if constexpr (N == 12) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Wait until at most N vector memory operations of this wave are outstanding (any N the
// counter holds).
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N <= 63, "the counter holds 0 .. 63");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(Int<I>{});
    static_for<I + 1, N>(f);
  }
}

// ---------------------------------------------------------------------------------------
// FP8 E4M3 rows, one query row per request.  The stored codes are staged in LDS as they
// are, with 16-byte global->LDS loads (half the LDS bytes of a widened tile and no
// registers in flight), and widened to bf16 as each lane reads its MFMA operands; the
// math is the bf16 kernel's (QK^T on the 16x16x32 MFMA, base-2 online softmax with the
// lazy rescale, PV on the 16x16x16 MFMA with V^T from byte permutes), so the results are
// those of a bf16 pool holding the same values.  A tile's 16 rows stream in pieces: a
// piece is the same span of codes (PW per row) of all 16 rows, one load instruction
// brings 1024 / PW rows of it, and within a row 16-byte chunk x lands at position
// x ^ (row % (PW / 16)), so the score reads (16 rows, 8 bytes each) and the PV reads (one
// row per 16 lanes) spread over the banks.  The score of tile s is interleaved with the
// output (PV) of tile s - 1, piece by piece (see the step loop), so each wave has two
// independent MFMA streams and its LDS reads of one overlap the other's products.
//   * split rows: pieces of 256 codes (whole 256-byte segments per row, as the bf16
//     kernel's loads), K pieces then V pieces, slots of two tiles;
//   * folded rows: pieces of 128 codes: the rotated-K piece and the four V pieces (load
//     order K0, V1, V2, V3, V0); the score reads K0, V1, V2, V3 and the output V0 .. V3,
//     so slots free a tile at a time: three sets of five slots.
template <int D, bool FOLDED>
struct Fp8Ring {
  // Codes (bytes) of a row per piece: 256 for split rows (whole 256-byte row segments per
  // load, as the bf16 kernel's); 128 for folded rows, whose rotated K part is 128 codes.
  static constexpr int PW = FOLDED ? 128 : 256;
  static constexpr int CH = PW / 16;               // 16-byte chunks of a row piece
  static constexpr int KP = FOLDED ? 1 : D / PW;   // K pieces of a tile
  static constexpr int VP = D / PW;                // V pieces of a tile
  static constexpr int SPP = PW / 128;             // PV slabs (128 dims) per V piece
  static constexpr int NPT = KP + VP;              // pieces per tile
  static constexpr int RPI = 1024 / PW;            // rows per load instruction
  static constexpr int IPP = kTile / RPI;          // load instructions per piece
  // LDS bytes per load block: 128-code pieces pad 64 bytes, so rows 8 apart (same chunk
  // positions) fall in other banks.
  static constexpr int BLOCK = PW == 128 ? 1024 + 64 : 1024;
  static constexpr int SLOT = IPP * BLOCK;
  static constexpr int SETS = FOLDED ? 3 : 2;      // tiles of slots
  static constexpr int SLOTS = SETS * NPT;
  static constexpr int REGION = SLOTS * SLOT;      // one wave's LDS
  // Most load instructions a wave has outstanding (less the awaited piece's).
  static constexpr int MAXOUT = FOLDED ? (2 * NPT - 1) * IPP : (2 * KP + VP - 1) * IPP;
  static_assert(MAXOUT <= 63, "outstanding loads fit the counter");
  static_assert(REGION * kWavesPerBlock <= 160 * 1024, "four waves' slots fit the LDS");
};

// LDS offset of staged row kr inside a slot.
template <class R>
__device__ __forceinline__ int ring_row(int kr) {
  return (kr / R::RPI) * R::BLOCK + (kr % R::RPI) * R::PW;
}

template <int D, int G, bool FOLDED>
__global__ __launch_bounds__(256, 1) void fp8_ring_kernel(SplitArgs a) {
  using S = Shape<D, FOLDED>;
  using R = Fp8Ring<D, FOLDED>;
  using O = Ops<false>;
  using E = Elem<ATTN_KV_FP8_E4M3>;
  constexpr int KSTEPS = S::KSTEPS;
  static_assert(2 * G <= 16, "hi/lo columns must fit one 16-wide MFMA block");
  static_assert(!FOLDED || D == 512, "folded rows: head dim 512");
  static_assert(R::PW % 128 == 0 && R::CH * 16 == R::PW, "whole 16-byte chunks per row piece");
  static_assert(sizeof(QuarterState<D, G>) <= R::REGION, "parked state must fit the region");
  static_assert(R::KP + (FOLDED ? 3 : 0) == R::VP, "score piece i pairs with PV slab i");
  __shared__ __attribute__((aligned(16))) char region[kWavesPerBlock][R::REGION];

  const int lane = threadIdx.x & 63;
  const int c = lane & 15;   // MFMA row/column index inside a 16-block
  const int qg = lane >> 4;  // lane group: selects k sub-range / output rows
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int chunk = blockIdx.x;  // one chunk per workgroup, one quarter per wave
  const int g = blockIdx.y;
  const int r = blockIdx.z;
  char* lds = region[wave];

  const int64_t cap = int64_t(a.max_pages) * a.page_size;
  const int quarter = ((chunk & 1) ? a.chunk_len_odd : a.chunk_len) / kWavesPerBlock;
  PageWalker pw{a.table + int64_t(r) * a.max_pages, a.num_pages, a.page_size, a.max_pages, 0, -1, -1};
  const int c0_nw = int(chunk_cover(a, chunk)) + wave * quarter;
  const bool early = a.window == 0 && c0_nw < cap;
  pw.start(early ? c0_nw : 0);

  const int L = a.seq_lens[r];
  const int lo = (a.window > 0 && L > a.window) ? L - a.window : 0;
  const int start = lo & ~(kTile - 1);
  bool poison = L < 1 || int64_t(L) > cap ||
                int64_t(L) - start > chunk_cover(a, a.num_chunks);
  const int c0 = start + int(chunk_cover(a, chunk)) + wave * quarter;
  const int c1 = min(c0 + quarter, L);
  int ntiles = (!poison && c0 < c1) ? (c1 - c0 + kTile - 1) / kTile : 0;
  const char* head_base = a.pool + int64_t(g) * a.head_stride;

  // Pool address of tile t's first row, or null (and the quarter poisoned and cut there)
  // if its page id is outside the pool.  Called for t = 0, 1, 2, ... in order.
  auto tile_base = [&](int t) -> const char* {
    const int tok0 = c0 + t * kTile;
    const int32_t pid = pw.page_of(tok0);
    if (pid < 0) {
      poison = true;
      ntiles = t;
      return nullptr;
    }
    return head_base + int64_t(pid) * a.page_stride + int64_t(tok0 % a.page_size) * a.row_stride;
  };
  // Byte offset in the stored row of load-order piece j of a tile.
  auto piece_col = [&](int j) -> int64_t {
    if constexpr (FOLDED) return j == 0 ? a.k_offset : a.v_offset + R::PW * (j < 4 ? j : 0);
    return j < R::KP ? a.k_offset + R::PW * j : a.v_offset + R::PW * (j - R::KP);
  };
  // Request piece j of the tile at `tb` into `slot`: lane l of instruction i fetches row
  // 8i + l / 8, chunk (l % 8) ^ (row % 8), landing at 16 l of the instruction's block.
  auto issue = [&](const char* tb, int j, int slot) {
    const char* base = tb + piece_col(j);
    char* dst = lds + R::SLOT * slot;
#pragma unroll
    for (int i = 0; i < R::IPP; ++i) {
      const int row = R::RPI * i + lane / R::CH;
      const int64_t off = int64_t(row) * a.row_stride + 16 * ((lane % R::CH) ^ (row % R::CH));
      __builtin_amdgcn_global_load_lds(base + off, (lds_void*)(dst + R::BLOCK * i), 16, 0, kStreamLds);
    }
  };
  auto reads_done = [] { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };

  // Tile 0 and the first pieces of tile 1 stream while the query operand is prepared.
  const char* tb1 = nullptr;  // base of tile 1
  if (ntiles > 0) {
    if (!early) pw.start(c0);
    const char* tb0 = tile_base(0);
    if (tb0) {
      if constexpr (FOLDED) {
#pragma unroll
        for (int j = 0; j < R::NPT; ++j) issue(tb0, j, j);
        if (ntiles > 1) tb1 = tile_base(1);
        if (tb1) {
#pragma unroll
          for (int j = 0; j < R::NPT; ++j) issue(tb1, j, R::NPT + j);
        }
      } else {
        // tile 0, then tile 1's K pieces (its V pieces follow during step 0)
#pragma unroll
        for (int j = 0; j < R::NPT; ++j) issue(tb0, j, j);
        if (ntiles > 1) tb1 = tile_base(1);
        if (tb1) {
#pragma unroll
          for (int j = 0; j < R::KP; ++j) issue(tb1, j, R::NPT + j);
        }
      }
    }
  }
  typename O::T8 qop[KSTEPS];
  make_query_operand<D, G, false>(a.q + int64_t(r) * a.num_q_heads * D, g, c, qg, a.qscale_k,
                                  a.qscale_v, FOLDED ? S::ROT : D, qop);

  float m_run = -INFINITY;
  float l_run = 0.0f;
  floatx4 acc[D / 128][8];  // slab b, step jj: lane (c, qg) rows 4qg + i <-> dims 128b + 8(4qg+i) + jj
#pragma unroll
  for (int b = 0; b < D / 128; ++b)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc[b][jj] = floatx4{0.f, 0.f, 0.f, 0.f};
  floatx4 sacc;             // scores of the tile in progress
  typename O::T4 pop;       // its probabilities (high or low part per column)
  const int part = c / G;

  // Score steps of piece p (dims PW p .. PW (p + 1)) from the piece in `slot`: lane (c, qg),
  // step u of the piece reads row c, codes 32u + 8qg .. + 8.
  auto qk_piece = [&](const char* slot, auto pc) {
    constexpr int SPIECE = R::PW / 32;  // score steps per piece
    constexpr int P0 = SPIECE * decltype(pc)::value;
    const char* rowp = slot + ring_row<R>(c);
#pragma unroll
    for (int u = 0; u < SPIECE; ++u) {
      const int x = 2 * u + (qg >> 1);
      const u32x2 raw = *reinterpret_cast<const u32x2*>(rowp + 16 * (x ^ (c % R::CH)) + 8 * (qg & 1));
      sacc = O::mma32(__builtin_bit_cast(typename O::T8, E::widen(raw)), qop[P0 + u], sacc);
    }
  };
  // Online softmax over keys tok0 + 4qg + i (as the bf16 kernel's tile math).
  auto softmax = [&](int tok0) {
    float sc[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float full = sacc[i] + partner<G>(sacc[i]);
      const int t = tok0 + 4 * qg + i;
      sc[i] = (t >= lo && t < L) ? full : -INFINITY;
      mx = fmaxf(mx, sc[i]);
    }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const bool grow = mx > m_run + kRescaleSlack;
    if (__builtin_expect(__any(grow), 0)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 from -inf
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < D / 128; ++b)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) acc[b][jj] *= alpha;
      m_run = m_new;
    }
    float p[4] = {0.f, 0.f, 0.f, 0.f};
    if (m_run != -INFINITY) {
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] - m_run);
    }
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 h = (__bf16)p[i];
      const __bf16 l = (__bf16)(p[i] - (float)h);
      pop[i] = part == 0 ? h : (part == 1 ? l : (__bf16)0.0f);
    }
  };
  // PV for slab b (dims 128b ..), part bb of the V piece in `slot`: lane (c, qg) reads rows
  // 4qg + e, codes 128bb + 8c .. + 8; rows of keys outside [lo, L) are zeroed after widening.
  auto pv_slab = [&](const char* slot, auto bc, auto bbc, int tok0) {
    constexpr int B = decltype(bc)::value;
    constexpr int BB = decltype(bbc)::value;
    const bool edge = tok0 < lo || tok0 + kTile > L;  // uniform
    u32x2 raw[4];  // all four reads issued before any is used
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kr = 4 * qg + e;
      raw[e] = *reinterpret_cast<const u32x2*>(slot + ring_row<R>(kr) +
                                               16 * ((8 * BB + (c >> 1)) ^ (kr % R::CH)) + 8 * (c & 1));
    }
    u32x4 w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = E::widen(raw[e]);
    if (__builtin_expect(edge, 0)) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = tok0 + 4 * qg + e;
        const unsigned keep = (key >= lo && key < L) ? ~0u : 0u;
        w[e] &= u32x4{keep, keep, keep, keep};
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const u32x2 even = {perm(w[1][u], w[0][u], 0x05040100u), perm(w[3][u], w[2][u], 0x05040100u)};
      const u32x2 odd = {perm(w[1][u], w[0][u], 0x07060302u), perm(w[3][u], w[2][u], 0x07060302u)};
      acc[B][2 * u] = O::mma16(__builtin_bit_cast(typename O::T4, even), pop, acc[B][2 * u]);
      acc[B][2 * u + 1] = O::mma16(__builtin_bit_cast(typename O::T4, odd), pop, acc[B][2 * u + 1]);
    }
  };
  // PV for V piece v (slabs SPP v .. SPP v + SPP - 1) from `slot`.
  auto pv_piece = [&](const char* slot, auto vc, int tok0) {
    constexpr int V = decltype(vc)::value;
    static_for<0, R::SPP>([&](auto bbc) {
      constexpr int BB = decltype(bbc)::value;
      pv_slab(slot, Int<R::SPP * V + BB>{}, bbc, tok0);
    });
  };

  // Step s interleaves the score of tile s with the output of tile s - 1: score piece i,
  // then the PV of tile s - 1's V piece i (with the probabilities step s - 1 produced); then
  // tile s's softmax (which may rescale the accumulators, after the PV of tile s - 1).  A
  // last step does the PV of the last tile.  Every accumulator sees its terms in the same
  // order as tile after tile.
  if constexpr (!FOLDED) {
    // Split rows: the slots of tile t are set t % 2 (K pieces, then V pieces).  Step s
    // first requests tile s + 1's K pieces (into the slots tile s - 1's K pieces left in
    // step s - 1), and after the PV of tile s - 1's V piece i, tile s + 1's V piece i (into
    // its slot).  Before score piece i, the pieces requested after it are tile s's later K
    // pieces, its V pieces, and tile s + 1's K pieces and first i V pieces: 2 KP + VP - 1
    // of them while a tile s + 1 exists.  Tile s - 1's V pieces were requested before.
    if (ntiles > 0) {
      const char* tbn = tb1;  // base of tile s + 1
      for (int s = 0; s < ntiles; ++s) {
        const int tok0 = c0 + s * kTile;
        const int set = s & 1;
        reads_done();
        if (s >= 1 && s + 1 < ntiles) {
          tbn = tile_base(s + 1);  // null (and ntiles cut) for a bad page
          if (tbn) {
#pragma unroll
            for (int j = 0; j < R::KP; ++j) issue(tbn, j, (set ^ 1) * R::NPT + j);
          }
        }
        const bool more = s + 1 < ntiles;
        const char* ks = lds + R::SLOT * (set * R::NPT);
        const char* vs = lds + R::SLOT * ((set ^ 1) * R::NPT + R::KP);  // tiles s - 1, s + 1
        sacc = floatx4{0.f, 0.f, 0.f, 0.f};
        static_for<0, R::KP>([&](auto ic) {
          constexpr int I = decltype(ic)::value;
          if (more)
            vm_wait<(2 * R::KP + R::VP - 1) * R::IPP>();
          else
            vm_wait<(R::KP - 1 - I + R::VP) * R::IPP>();
          qk_piece(ks + R::SLOT * I, Int<I>{});
          if (s >= 1) pv_piece(vs + R::SLOT * I, Int<I>{}, tok0 - kTile);
          if (more && tbn) {
            reads_done();
            issue(tbn, R::KP + I, (set ^ 1) * R::NPT + R::KP + I);
          }
        });
        softmax(tok0);
      }
      // The output of the last tile.
      vm_wait<0>();
      const char* vs = lds + R::SLOT * (((ntiles - 1) & 1) * R::NPT + R::KP);
      const int ptok = c0 + (ntiles - 1) * kTile;
      static_for<0, R::VP>([&](auto vc) {
        constexpr int V = decltype(vc)::value;
        pv_piece(vs + R::SLOT * V, vc, ptok);
      });
    }
  } else {
    // Folded rows: tile t's five pieces (K0, V1, V2, V3, V0) are set t % 3, all requested
    // as step t - 1 starts (tiles 0 and 1 first); the score of tile t reads its first four
    // pieces, the output V0 .. V3.  Before score piece i of tile s, the loads of the rest of
    // tile s and all of tile s + 1 (if any) may stay in flight.
    if (ntiles > 0) {
      int kset = 0;  // set of tile s
      int pset = 0;  // set of tile s - 1
      for (int s = 0; s < ntiles; ++s) {
        const int tok0 = c0 + s * kTile;
        reads_done();
        if (s >= 1 && s + 1 < ntiles) {
          const char* tbn = tile_base(s + 1);  // null (and ntiles cut) for a bad page
          if (tbn) {
            const int nset = kset == 2 ? 0 : kset + 1;
#pragma unroll
            for (int j = 0; j < R::NPT; ++j) issue(tbn, j, nset * R::NPT + j);
          }
        }
        const bool more = s + 1 < ntiles;
        const char* ks = lds + R::SLOT * (kset * R::NPT);
        const char* ps = lds + R::SLOT * (pset * R::NPT);
        sacc = floatx4{0.f, 0.f, 0.f, 0.f};
        static_for<0, 4>([&](auto ic) {
          constexpr int I = decltype(ic)::value;  // score piece: K0, V1, V2, V3
          if (more)
            vm_wait<(2 * R::NPT - 1 - I) * R::IPP>();
          else
            vm_wait<(R::NPT - 1 - I) * R::IPP>();
          qk_piece(ks + R::SLOT * I, Int<I>{});
          if (s >= 1) pv_piece(ps + R::SLOT * (I == 0 ? 4 : I), Int<I>{}, tok0 - kTile);
        });
        softmax(tok0);
        pset = kset;
        kset = kset == 2 ? 0 : kset + 1;
      }
      vm_wait<0>();
      const char* ps = lds + R::SLOT * (pset * R::NPT);
      const int ptok = c0 + (ntiles - 1) * kTile;
      static_for<0, R::VP>([&](auto vc) {
        constexpr int V = decltype(vc)::value;
        pv_piece(ps + R::SLOT * (V == 0 ? 4 : V), vc, ptok);
      });
    }
  }
  // Every load has landed and been read before the region is reused for the quarter state.
  vm_wait<0>();
  reads_done();

  // Quarter state: sum l over the lane groups, add the low columns onto the high ones.
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
#pragma unroll
  for (int b = 0; b < D / 128; ++b)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[b][jj][i] += partner<G>(acc[b][jj][i]);

  using Parked = QuarterState<D, G>;
  Parked* mine = reinterpret_cast<Parked*>(lds);
  const float qnan = __builtin_nanf("");
  if (c < G) {
    if (qg == 0) {
      mine->m[c] = poison ? qnan : m_run;  // log2 units, -inf when empty
      mine->l[c] = l_run;
    }
#pragma unroll
    for (int b = 0; b < D / 128; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d = 128 * b + 32 * qg + 8 * i;  // dims d .. d + 7
        mine->o[c][d / 4] = floatx4{acc[b][0][i], acc[b][1][i], acc[b][2][i], acc[b][3][i]};
        mine->o[c][d / 4 + 1] = floatx4{acc[b][4][i], acc[b][5][i], acc[b][6][i], acc[b][7][i]};
      }
  }
  __syncthreads();
  const Parked* parked[kWavesPerBlock];
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) parked[w] = reinterpret_cast<const Parked*>(region[w]);
  write_chunk_state<D, G>(a, parked, r, g, chunk);
}

template <int D>
struct F32Shape {
  static constexpr int HALF_BYTES = 4 * D;        // the K or the V half of a row
  static constexpr int PITCH = HALF_BYTES + 16;   // staged row pitch: conflict-free reads
  static constexpr int REGION = kTile * PITCH;    // one wave's LDS region
  static constexpr int LOADS = HALF_BYTES / 1024; // 1-KB load instructions per row half
  static constexpr int QSTEPS = D / 16;           // 16-dim groups of QK (4 MFMA steps each)
  static constexpr int VBLOCKS = D / 64;          // 64-dim blocks of PV
  static_assert(HALF_BYTES % 1024 == 0, "whole kilobytes per row half");
};

// The head-dim-512 ring of the f32 kernel: each half (K or V) of a staged row streams in
// NP pieces of PW bytes; one load instruction brings RPI rows of a piece.
template <int D>
struct F32Ring {
  static constexpr int NP = 8;                                // pieces per row half
  static constexpr int PW = F32Shape<D>::HALF_BYTES / NP;     // bytes of a row per piece
  static constexpr int CH = PW / 16;                          // 16-byte chunks of a row per piece
  static constexpr int RPI = 1024 / PW;                       // rows per load instruction
  static constexpr int IPP = kTile / RPI;                     // load instructions per piece
  static constexpr int SLOT = kTile * PW;                     // LDS bytes per slot
  static constexpr int AHEAD = NP - 1;                        // pieces in flight behind the one in use
};

// Merge of the four waves' quarter states of the f32 kernel (fixed order), 4 dims per
// thread, for the 16 MFMA columns: column h is row row0 + h / G of the work item, head
// h % G.  Decode: the chunk state of each active column (natural-log m, O times v_scale).
// Prefill: the normalised row O * v_scale / S into out.
template <int D, int G, bool PREFILL>
__device__ __forceinline__ void write_f32_states(const SplitArgs& a,
                                                 const QuarterState<D, 16>* const (&parked)[kWavesPerBlock],
                                                 int g, int chunk, int64_t qs0, int row0, int rows) {
  const float qnan = __builtin_nanf("");
  for (int idx = threadIdx.x; idx < 16 * (D / 4); idx += 64 * kWavesPerBlock) {
    const int h = idx / (D / 4);
    const int d4 = idx % (D / 4);
    const int row = row0 + h / G;
    if (row >= rows) continue;
    float M = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int w = 0; w < kWavesPerBlock; ++w) {
      const float x = parked[w]->m[h];
      nan |= x != x;
      M = fmaxf(M, x);
    }
    float S = 0.0f;
    floatx4 O = {0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kWavesPerBlock; ++w) {
        const float x = parked[w]->m[h];
        const float wt = x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(x - M);
        S += wt * parked[w]->l[h];
        O += wt * parked[w]->o[h][d4];
      }
    }
    if (nan) {
      M = S = qnan;
      O = floatx4{qnan, qnan, qnan, qnan};
    }
    const int64_t hq = (qs0 + row) * a.num_q_heads + g * G + h % G;
    if constexpr (PREFILL) {
      *reinterpret_cast<floatx4*>(a.out + hq * D + 4 * d4) = O * (a.vscale / S);
    } else {
      const int64_t st = hq * a.num_chunks + chunk;
      if (d4 == 0) {
        a.part_m[st] = M == -INFINITY ? -INFINITY : M * kLn2;
        a.part_l[st] = S;
      }
      *reinterpret_cast<floatx4*>(a.part_o + st * D + 4 * d4) = O * a.vscale;
    }
  }
}

// The f32 kernel.  Its 16 MFMA columns hold R = 16 / G query rows of the KV head's G heads
// (column c: row c / G of the work item, head c % G): one decode row uses the first G
// columns; a window of rows is cut into groups of R rows, each a workgroup per chunk; in
// prefill mode (PREFILL) a workgroup is R consecutive prompt rows of one request, whose
// keys (from the first row's window start to the last row's position) are cut into four
// quarters, one per wave, and whose normalised rows are written directly.
template <int D, int G, bool FOLDED, bool PREFILL>
__global__ __launch_bounds__(256, 1) void f32_partial_kernel(SplitArgs a) {
  using S = F32Shape<D>;
  constexpr int R = 16 / G;  // query rows per work item
  static_assert(!FOLDED || D == 512, "folded rows: head dim 512");
  static_assert(G <= 16 && 16 % G == 0, "whole rows of heads fill the 16 MFMA columns");
  static_assert(sizeof(QuarterState<D, 16>) <= S::REGION, "parked state must fit the region");
  __shared__ __attribute__((aligned(16))) char region[kWavesPerBlock][S::REGION];

  const int lane = threadIdx.x & 63;
  const int c = lane & 15;   // MFMA column ((row, head) pair) / K row inside the tile
  const int qg = lane >> 4;  // lane group: k index of the MFMA operands / output rows
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  char* lds = region[wave];

  // Prompt rows: a 1-D launch over the work items.  Workgroups go to the eight XCDs in
  // turn (slot w on XCD w % 8), so runs of 32 consecutive items, i.e. neighbouring row
  // tiles of one (request, KV head) whose key ranges nearly coincide, are given to one XCD
  // and start together, longest rows first: they stream the same keys through that XCD's
  // L2 at about the same time.  The launch is padded to whole rounds of 256.
  int g, r, tile = 0;
  if constexpr (PREFILL) {
    const int w = blockIdx.x;
    const int slot = w >> 3;
    const int item = ((slot >> 5) * 8 + (w & 7)) * 32 + (slot & 31);
    if (item >= a.items) return;
    g = (item / a.row_tiles) % a.num_kv_heads;
    r = item / a.row_tiles / a.num_kv_heads;
    tile = a.row_tiles - 1 - item % a.row_tiles;
  } else {
    g = blockIdx.y;
    r = blockIdx.z;
  }

  const int L = a.seq_lens[r];
  const int64_t cap = int64_t(a.max_pages) * a.page_size;
  int chunk = 0, rows, row0;
  int64_t qs0;
  if constexpr (PREFILL) {
    // Offsets the plan cannot serve are not followed: nothing is read or written.
    qs0 = a.q_starts[r];
    const int qs1 = a.q_starts[r + 1];
    rows = qs1 - int(qs0);
    if (qs0 < 0 || rows < 0 || rows > a.max_rows || qs1 > a.total_rows) return;
    row0 = tile * R;
    if (row0 >= rows) return;
  } else {
    // Launch order of several row groups: the groups of a chunk 8 workgroups apart (one XCD).
    const int lo8 = blockIdx.x % 8;
    const int hi8 = blockIdx.x / 8;
    chunk = (hi8 / a.row_groups) * 8 + lo8;
    if (chunk >= a.num_chunks) return;  // padding of the launch order (whole workgroup)
    rows = a.num_rows;
    qs0 = int64_t(r) * rows;
    row0 = (hi8 % a.row_groups) * R;
  }
  bool poison = L < max(rows, 1) || int64_t(L) > cap;

  // This lane's column: row `row` of the request's rows (position L - rows + row), head
  // c % G.  It sees keys lo_c <= t < hi_c, and with row masks (tree windows) of the window's
  // own keys [wstart, L) only those whose bit t - wstart is set.  An idle column sees none.
  const int row = row0 + c / G;
  const bool active = row < rows;
  const int hi_row = L - rows + row + 1;
  int lo_c = a.window > 0 ? max(0, hi_row - a.window) : 0;
  int hi_c = hi_row;
  int wstart = INT32_MAX;
  uint64_t mask_c = ~uint64_t(0);
  if constexpr (!PREFILL) {
    if (a.row_masks && active) {
      hi_c = L;
      wstart = L - rows;
      mask_c = a.row_masks[qs0 + row];
    }
  }
  if (!active) {
    lo_c = INT32_MAX;
    hi_c = 0;
  }
  // Keys some column of the work item may see: [kv_lo, kv_hi); V rows outside are zeroed.
  // Decode chunks partition the keys from the request's first row's window start.
  const int last = min(row0 + R, rows) - 1;
  const int hi_first = L - rows + (PREFILL ? row0 : 0) + 1;
  const int kv_lo = a.window > 0 ? max(0, hi_first - a.window) : 0;
  const int kv_hi = (PREFILL || !a.row_masks) ? L - rows + last + 1 : L;
  const int start = kv_lo & ~(kTile - 1);
  int c0, c1;
  if constexpr (PREFILL) {
    const int quarter = (kv_hi - start + 4 * kTile - 1) / (4 * kTile) * kTile;
    c0 = start + wave * quarter;
    c1 = min(c0 + quarter, kv_hi);
  } else {
    poison = poison || int64_t(L) - start > chunk_cover(a, a.num_chunks);
    const int quarter = ((chunk & 1) ? a.chunk_len_odd : a.chunk_len) / kWavesPerBlock;
    c0 = start + int(chunk_cover(a, chunk)) + wave * quarter;
    c1 = min(c0 + quarter, kv_hi);
  }
  const int end = (!poison && c0 < c1) ? c1 : c0;
  const char* head_base = a.pool + int64_t(g) * a.head_stride;
  PageWalker pw{a.table + int64_t(r) * a.max_pages, a.num_pages, a.page_size, a.max_pages, 0, -1, -1};
  // Cache policy of the row loads: decode streams each row once (non-temporal); the row
  // tiles of a prompt read their keys again from L2 (default policy: the 16 sliding f32
  // prompts 13.1 -> 9.3 ms, the 10,602-row prompt 41.8 -> 41.7 ms).
  constexpr int kPolicy = PREFILL ? 0 : kStreamLds;

  // Query operand: lane (c, qg), group s, step j holds q[row][head][16s + 4qg + j] times
  // scale * log2(e) * k_scale (folded rows: v_scale for the dims from 128 on, which meet V
  // columns; zero for an idle column).  Parked in the accumulation registers, so the
  // vector registers hold the output accumulators.
  floatx4 qv[S::QSTEPS];
  {
    const float* qrow =
        a.q + ((qs0 + (active ? row : 0)) * a.num_q_heads + g * G + c % G) * int64_t(D) + 4 * qg;
#pragma unroll
    for (int s = 0; s < S::QSTEPS; ++s) {
      const float f = (FOLDED && 16 * s >= 128) ? a.qscale_v : a.qscale_k;
      qv[s] = active ? *reinterpret_cast<const floatx4*>(qrow + 16 * s) * f
                     : floatx4{0.f, 0.f, 0.f, 0.f};
      asm volatile("" : "+a"(qv[s]));
    }
  }

  float m_run = -INFINITY;
  float l_run = 0.0f;
  floatx4 acc[S::VBLOCKS][4];  // block b, step jj: lane (c, qg) element i <-> dim 64b + 4(4qg+i) + jj
#pragma unroll
  for (int b = 0; b < S::VBLOCKS; ++b)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) acc[b][jj] = floatx4{0.f, 0.f, 0.f, 0.f};
  floatx4 sj[4];  // score chains (step j) of the current tile
  float p[4];     // probabilities of keys tok0 + 4qg + i for head c

  // Scores of keys tok0 + 4qg + i for head c over 16-dim groups [S0, S1): four
  // independent chains (step j), summed by the softmax.
  auto qk = [&](auto s_begin, auto s_end) {
#pragma unroll
    for (int s = decltype(s_begin)::value; s < decltype(s_end)::value; ++s) {
      const floatx4 kv = *reinterpret_cast<const floatx4*>(lds + c * S::PITCH + 64 * s + 16 * qg);
      const floatx4 qq = qv[s];
#pragma unroll
      for (int j = 0; j < 4; ++j) sj[j] = mma_f32(kv[j], qq[j], sj[j]);
    }
  };
  // Online softmax (base 2), masked keys by select, lazy rescale as in the bf16 kernel.
  auto softmax = [&](int tok0) {
    const floatx4 sc4 = (sj[0] + sj[1]) + (sj[2] + sj[3]);
    float sc[4];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = tok0 + 4 * qg + i;
      const bool vis = t >= lo_c && t < hi_c && (t < wstart || ((mask_c >> ((t - wstart) & 63)) & 1));
      sc[i] = vis ? sc4[i] : -INFINITY;
      mx = fmaxf(mx, sc[i]);
    }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const bool grow = mx > m_run + kRescaleSlack;
    if (__builtin_expect(__any(grow), 0)) {
      const float m_new = grow ? mx : m_run;
      // Columns see different keys (rows, windows): one that keeps its maximum keeps its
      // sums (exp2(-inf - -inf) would be NaN for a column with no visible key yet).
      const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // 0 from -inf
      l_run *= alpha;
#pragma unroll
      for (int b = 0; b < S::VBLOCKS; ++b)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[b][jj] *= alpha;
      m_run = m_new;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = 0.0f;
    if (m_run != -INFINITY) {
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(sc[i] - m_run);
    }
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
  };
  // PV over 64-dim blocks [B0, B1).  MFMA t takes keys 4qg + t, so lane (c, qg) supplies
  // its own p[t] as B; A = V^T: lane (m, qg) holds dims 64b + 4m + jj of key 4qg + t.
  auto pv = [&](int tok0, auto b_begin, auto b_end) {
    const bool edge = tok0 < kv_lo || tok0 + kTile > kv_hi;  // uniform
#pragma unroll
    for (int b = decltype(b_begin)::value; b < decltype(b_end)::value; ++b)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kr = 4 * qg + t;
        floatx4 vv = *reinterpret_cast<const floatx4*>(lds + kr * S::PITCH + 256 * b + 16 * c);
        if (__builtin_expect(edge, 0)) {
          const int key = tok0 + kr;
          if (key < kv_lo || key >= kv_hi) vv = floatx4{0.f, 0.f, 0.f, 0.f};  // padding never reaches O
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[b][jj] = mma_f32(vv[jj], p[t], acc[b][jj]);
      }
  };
  auto clear_scores = [&] {
#pragma unroll
    for (int j = 0; j < 4; ++j) sj[j] = floatx4{0.f, 0.f, 0.f, 0.f};
  };

  if constexpr (S::LOADS == 2) {
    // Head dim 512: the tile's K half, then its V half, streams through a ring of eight
    // 4 KB LDS slots in pieces of 256 bytes per row (64 dims of the 16 rows), seven pieces
    // in flight while the wave computes on the eighth: piece j of a tile (K pieces 0-7,
    // then V pieces 0-7) goes to slot j % 8, and phase j first requests piece j + 7 (of the
    // next tile from phase 9 on) into the slot that phase j - 1 has finished reading, then
    // waits only for piece j.  One load instruction brings four rows' 256 bytes; within a
    // row, 16-byte chunk x sits at position x ^ row, so the score reads (16 rows, one chunk
    // each) and the PV reads (one row, 16 chunks) both touch distinct banks, and each
    // aligned group of eight lanes still fetches one whole 128-byte line.
    using R = F32Ring<D>;
    static_assert(R::PW == 256 && R::CH == kTile && R::NP * R::SLOT <= S::REGION, "ring of 4 KB slots");
    static_assert(R::AHEAD * R::IPP <= 63, "outstanding loads fit the counter");
    static_assert(S::QSTEPS == 4 * R::NP && S::VBLOCKS == R::NP, "one piece = 4 score steps = 1 PV block");

    // Folded rows (rotated K: 2 pieces, V: 8 pieces): the score takes K pieces 0-1 and V
    // pieces 2-7, the output V pieces 0-7, so a tile loads 10 pieces into the same eight
    // slots: K0, K1, V2 .. V7 for the score phases 0-7 (slots 0-7), and V0 / V1 into slots
    // 0 / 1 once phases 0 / 1 have read K0 / K1; the output phases 8-15 read slots 0-7.  A
    // slot is refilled with the next tile's piece after its last read (K0' after phase 8,
    // K1' after 9, V2' .. V6' after 10 .. 14, V7' at the next tile's phase 0), so every
    // piece is requested about seven phases before it is used.
    // Lane l of load instruction i fetches row R::RPI*i + l / R::CH, chunk (l % R::CH) ^ row.
    auto issue_at = [&](int32_t pid, int tok0, int64_t col, int slot) {  // 256 B per row at col
      const char* base = head_base + int64_t(pid) * a.page_stride +
                         int64_t(tok0 % a.page_size) * a.row_stride + col;
      char* dst = lds + R::SLOT * slot;
#pragma unroll
      for (int i = 0; i < R::IPP; ++i) {
        const int row = R::RPI * i + lane / R::CH;
        const int64_t off = int64_t(row) * a.row_stride + 16 * ((lane % R::CH) ^ row);
        __builtin_amdgcn_global_load_lds(base + off, (lds_void*)(dst + 1024 * i), 16, 0, kPolicy);
      }
    };
    // Split rows: piece j (0-15) of the tile: K pieces 0-7, then V pieces 0-7, slot j % 8.
    // Folded rows: piece j of the load order K0, K1, V2 .. V7, V0, V1 (slots 0-7, 0, 1).
    auto issue = [&](int32_t pid, int tok0, int j) {
      if constexpr (FOLDED) {
        const int64_t col = j < 2 ? a.k_offset + R::PW * j
                                  : a.v_offset + R::PW * (j < R::NP ? j : j - R::NP);
        issue_at(pid, tok0, col, j % R::NP);
      } else {
        issue_at(pid, tok0, (j >= R::NP ? a.v_offset : a.k_offset) + R::PW * (j % R::NP), j % R::NP);
      }
    };
    auto reads_done = [] { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };

    auto phase = [&](auto jc, int32_t pid, int tok0, int32_t npid, int next, bool more) {
      constexpr int J = decltype(jc)::value;
      reads_done();
      if constexpr (FOLDED) {
        // Requests: V7 at phase 0, V0 / V1 at 1 / 2, the next tile's K0, K1, V2 .. V6 at
        // 9 .. 15.  Wait for the piece this phase reads (phases 10-15 read V pieces the
        // score phases already waited for): pieces requested after it may stay in flight.
        if constexpr (J == 0) issue(pid, tok0, 7);
        if constexpr (J == 1 || J == 2) issue(pid, tok0, 7 + J);
        if constexpr (J >= 9) {
          if (more) issue(npid, next, J - 9);
        }
        if constexpr (J <= 2) {
          vm_wait_lt<R::AHEAD * R::IPP>();
        } else if constexpr (J <= 8) {
          vm_wait_lt<(9 - J) * R::IPP>();
        } else if constexpr (J == 9) {
          if (more)
            vm_wait_lt<R::IPP>();
          else
            vm_wait_lt<0>();
        }
      } else {
        if constexpr (J + R::AHEAD < 2 * R::NP) {
          issue(pid, tok0, J + R::AHEAD);
        } else {
          if (more) issue(npid, next, J + R::AHEAD - 2 * R::NP);
        }
        // Wait for piece J: the loads issued after it may stay in flight.
        if constexpr (J + R::AHEAD < 2 * R::NP) {
          vm_wait_lt<R::AHEAD * R::IPP>();
        } else {
          if (more)
            vm_wait_lt<R::AHEAD * R::IPP>();
          else
            vm_wait_lt<(2 * R::NP - 1 - J) * R::IPP>();
        }
      }
      const char* slot = lds + R::SLOT * (J % R::NP);
      if constexpr (J < R::NP) {
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          const int x = 4 * sl + qg;
          const floatx4 kv = *reinterpret_cast<const floatx4*>(slot + R::PW * c + 16 * (x ^ c));
          const floatx4 qq = qv[4 * J + sl];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) sj[jj] = mma_f32(kv[jj], qq[jj], sj[jj]);
        }
        if constexpr (J == R::NP - 1) softmax(tok0);
      } else {
        constexpr int B = J - R::NP;
        const bool edge = tok0 < kv_lo || tok0 + kTile > kv_hi;  // uniform
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int kr = 4 * qg + t;
          floatx4 vv = *reinterpret_cast<const floatx4*>(slot + R::PW * kr + 16 * (c ^ kr));
          if (__builtin_expect(edge, 0)) {
            const int key = tok0 + kr;
            if (key < kv_lo || key >= kv_hi) vv = floatx4{0.f, 0.f, 0.f, 0.f};  // padding never reaches O
          }
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) acc[B][jj] = mma_f32(vv[jj], p[t], acc[B][jj]);
        }
      }
    };
    int32_t pid = -1;
    if (c0 < end) {
      pw.start(c0);
      pid = pw.page_of(c0);
      if (pid < 0) {  // a table entry outside the pool poisons the quarter
        poison = true;
      } else {
#pragma unroll
        for (int j = 0; j < R::AHEAD; ++j) issue(pid, c0, j);
      }
    }
    for (int tok0 = c0; pid >= 0 && tok0 < end; tok0 += kTile) {
      const int next = tok0 + kTile;
      const int32_t npid = next < end ? pw.page_of(next) : -1;
      const bool more = npid >= 0;  // uniform
      if (next < end && !more) poison = true;
      clear_scores();
      phase(Int<0>{}, pid, tok0, npid, next, more);
      phase(Int<1>{}, pid, tok0, npid, next, more);
      phase(Int<2>{}, pid, tok0, npid, next, more);
      phase(Int<3>{}, pid, tok0, npid, next, more);
      phase(Int<4>{}, pid, tok0, npid, next, more);
      phase(Int<5>{}, pid, tok0, npid, next, more);
      phase(Int<6>{}, pid, tok0, npid, next, more);
      phase(Int<7>{}, pid, tok0, npid, next, more);
      phase(Int<8>{}, pid, tok0, npid, next, more);
      phase(Int<9>{}, pid, tok0, npid, next, more);
      phase(Int<10>{}, pid, tok0, npid, next, more);
      phase(Int<11>{}, pid, tok0, npid, next, more);
      phase(Int<12>{}, pid, tok0, npid, next, more);
      phase(Int<13>{}, pid, tok0, npid, next, more);
      phase(Int<14>{}, pid, tok0, npid, next, more);
      phase(Int<15>{}, pid, tok0, npid, next, more);
      pid = npid;
    }
  } else {
    // Head dim 256: a row half is one kilobyte, so the K half is staged whole, then the V
    // half into the same region: instruction (row, k) brings one kilobyte of the row, lane
    // l its 16-byte chunk 64k + l.
    auto stage = [&](int32_t pid, int tok0, int part) {
      const char* base = head_base + int64_t(pid) * a.page_stride +
                         int64_t(tok0 % a.page_size) * a.row_stride + (part ? a.v_offset : a.k_offset) +
                         16 * lane;
#pragma unroll
      for (int row = 0; row < kTile; ++row)
#pragma unroll
        for (int k = 0; k < S::LOADS; ++k)
          __builtin_amdgcn_global_load_lds(base + int64_t(row) * a.row_stride + 1024 * k,
                                           (lds_void*)(lds + row * S::PITCH + 1024 * k), 16, 0, kPolicy);
    };
    if (c0 < end) pw.start(c0);
    for (int tok0 = c0; tok0 < end; tok0 += kTile) {
      const int32_t pid = pw.page_of(tok0);
      if (pid < 0) {  // a table entry outside the pool poisons the quarter
        poison = true;
        break;
      }
      stage(pid, tok0, 0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      clear_scores();
      qk(Int<0>{}, Int<S::QSTEPS>{});
      softmax(tok0);
      // V half into the same region (the K reads above have all returned: they fed the
      // scores), then PV.
      stage(pid, tok0, 1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      pv(tok0, Int<0>{}, Int<S::VBLOCKS>{});
    }
  }

  // Quarter state: sum l over the lane groups; park (m, l, O) of all 16 columns for the
  // workgroup merge (an idle column parks the empty state).  Each wave parks in its own
  // region, which only it has used.
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  using Parked = QuarterState<D, 16>;
  Parked* mine = reinterpret_cast<Parked*>(lds);
  if (qg == 0) {
    mine->m[c] = poison ? __builtin_nanf("") : m_run;
    mine->l[c] = l_run;
  }
#pragma unroll
  for (int b = 0; b < S::VBLOCKS; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      mine->o[c][(64 * b + 16 * qg + 4 * i) / 4] =
          floatx4{acc[b][0][i], acc[b][1][i], acc[b][2][i], acc[b][3][i]};
  __syncthreads();
  const Parked* parked[kWavesPerBlock];
#pragma unroll
  for (int w = 0; w < kWavesPerBlock; ++w) parked[w] = reinterpret_cast<const Parked*>(region[w]);
  write_f32_states<D, G, PREFILL>(a, parked, g, chunk, qs0, row0, rows);
}

// Write one query row's chunk state: low columns added onto the high ones, maximum in
// natural-log units, NaN everywhere if the chunk was poisoned.
template <int D, int G>
__device__ __forceinline__ void write_row_state(const SplitArgs& a, int64_t st, int c, int qg,
                                                bool poison, float m_run, float l_run,
                                                floatx4 (&acc)[D / 128][8]) {
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
#pragma unroll
  for (int b = 0; b < D / 128; ++b)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[b][jj][i] += partner<G>(acc[b][jj][i]);
  if (c >= G) return;
  const float qnan = __builtin_nanf("");
  if (qg == 0) {
    a.part_m[st] = poison ? qnan : (m_run == -INFINITY ? -INFINITY : m_run * kLn2);
    a.part_l[st] = poison ? qnan : l_run;
  }
  float* o = a.part_o + st * D;
#pragma unroll
  for (int b = 0; b < D / 128; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      floatx4 w0 = floatx4{acc[b][0][i], acc[b][1][i], acc[b][2][i], acc[b][3][i]} * a.vscale;
      floatx4 w1 = floatx4{acc[b][4][i], acc[b][5][i], acc[b][6][i], acc[b][7][i]} * a.vscale;
      if (poison) w0 = w1 = floatx4{qnan, qnan, qnan, qnan};
      float* dst = o + 128 * b + 32 * qg + 8 * i;
      *reinterpret_cast<floatx4*>(dst) = w0;
      *reinterpret_cast<floatx4*>(dst + 4) = w1;
    }
}

// Several query rows per request (a verify window): row i sits at position
// L - rows + i and attends causally, or with row masks (tree attention) to the keys before
// the window and the window rows its mask names.  One workgroup = one key chunk of one (request,
// KV head, group of up to four rows); wave w serves row 4*group + w.  The four waves
// fetch each tile together (wave w the rows 4qg + w) into a double-buffered LDS tile,
// so every K/V byte is read once for all the rows of the group.  Workgroups of the
// same chunk and different row groups are 8 apart in launch order, i.e. on the same
// XCD, so the later group finds the rows in that XCD's L2.
template <int D, int G, bool FOLDED, int KV>
__global__ __launch_bounds__(256, 1) void rows_partial_kernel(SplitArgs a) {
  using S = Shape<D, FOLDED>;
  using E = Elem<KV>;
  constexpr int EB = E::kBytes;
  static_assert(2 * G <= 16, "hi/lo columns must fit one 16-wide MFMA block");
  __shared__ RowTile<S::COLS> tiles[2];

  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int qg = lane >> 4;
  const int wave = threadIdx.x >> 6;
  const int lo8 = blockIdx.x % 8;
  const int hi8 = blockIdx.x / 8;
  const int rg = hi8 % a.row_groups;
  const int chunk = (hi8 / a.row_groups) * 8 + lo8;
  const int g = blockIdx.y;
  const int r = blockIdx.z;
  if (chunk >= a.num_chunks) return;  // padding of the launch order (whole workgroup)

  const int rows = a.num_rows;
  const int row = rg * kWavesPerBlock + wave;
  const bool row_active = row < rows;
  const int L = a.seq_lens[r];
  const int first_hi = L - rows + 1;  // keys the first row sees: [.., first_hi)
  const int lo_all = (a.window > 0 && first_hi > a.window) ? first_hi - a.window : 0;
  const int hi = L - rows + row + 1;  // a causal row's keys: [lo, hi)
  const int lo = (a.window > 0 && hi > a.window) ? hi - a.window : 0;
  // Keys of the window [L - rows, L) this row sees: its mask, or (causal) rows 0 .. row.
  const uint64_t mask = !row_active ? 0
                        : a.row_masks ? a.row_masks[int64_t(r) * rows + row]
                        : (row >= 63 ? ~uint64_t(0) : (uint64_t(2) << row) - 1);
  const int start = lo_all & ~(kTile - 1);
  const int64_t cap = int64_t(a.max_pages) * a.page_size;
  bool poison = L < rows || int64_t(L) > cap ||
                int64_t(L) - start > chunk_cover(a, a.num_chunks);
  const int c0 = start + int(chunk_cover(a, chunk));
  const int c1 = min(c0 + ((chunk & 1) ? a.chunk_len_odd : a.chunk_len), L);
  const char* head_base = a.pool + int64_t(g) * a.head_stride;

  PageWalker pw{a.table + int64_t(r) * a.max_pages, a.num_pages, a.page_size, a.max_pages, 0, -1, -1};
  // Tiles stream ahead of the math (three of 16-bit rows, six of FP8 rows: the same
  // bytes); each register set holds this wave's quarter of one tile (rows 4qg + wave,
  // 8 elements at 128 sb + 8c).
  constexpr int kAhead = 6 / EB;
  typename E::Raw stage[kAhead][S::SLABS];
  int end = (!poison && c0 < c1) ? c1 : c0;  // tiles from `end` on are not processed
  auto fetch = [&](typename E::Raw (&buf)[S::SLABS], int tok0) {
    const int32_t pid = pw.page_of(tok0);
    if (pid < 0) {
      poison = true;
      end = tok0;
      return;
    }
    const char* row_ptr = head_base + int64_t(pid) * a.page_stride +
                          int64_t(tok0 % a.page_size + 4 * qg + wave) * a.row_stride + 8 * EB * c;
#pragma unroll
    for (int sb = 0; sb < S::SLABS; ++sb) buf[sb] = E::load(row_ptr + src_col<D, FOLDED, EB>(a, sb));
  };
  if (c0 < end) {
    pw.start(c0);
#pragma unroll
    for (int k = 0; k < kAhead; ++k)
      if (c0 + k * kTile < end) fetch(stage[k], c0 + k * kTile);
  }
  typename Ops<E::kF16>::T8 qop[S::KSTEPS];
  if (row_active)
    make_query_operand<D, G, E::kF16>(a.q + (int64_t(r) * rows + row) * a.num_q_heads * D, g, c, qg,
                                      a.qscale_k, a.qscale_v, FOLDED ? S::ROT : D, qop);
  float m_run = -INFINITY;
  float l_run = 0.0f;
  floatx4 acc[D / 128][8];  // slab b, step jj: lane (c, qg) rows 4qg + i <-> dims 128b + 8(4qg+i) + jj
#pragma unroll
  for (int b = 0; b < D / 128; ++b)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) acc[b][jj] = floatx4{0.f, 0.f, 0.f, 0.f};

  // One tile: stage this wave's quarter into the shared buffer, refill the registers
  // kAhead tiles ahead, wait for the whole tile, then this wave's row does the math.
  // Every wave runs the same tiles, so the barrier is uniform over the workgroup.
  int buf = 0;
  auto step = [&](typename E::Raw (&regs)[S::SLABS], int tok0) {
    uint16_t* tile = tiles[buf].v;
#pragma unroll
    for (int sb = 0; sb < S::SLABS; ++sb)
      *reinterpret_cast<u32x4*>(tile + (4 * qg + wave) * S::P + 128 * sb + 8 * c) = E::widen(regs[sb]);
    if (tok0 + kAhead * kTile < end) fetch(regs, tok0 + kAhead * kTile);
    if (__builtin_expect(tok0 < lo_all || tok0 + kTile > L, 0))
      zero_dead_rows<D, FOLDED>(tile, tok0, lo_all, L, c, qg, wave, wave + 1);
    __syncthreads();  // the tile is complete; the other buffer is free again
    if (row_active)
      tile_math<D, G, FOLDED, E::kF16, true>(tile, tok0, lo, L, qop, c, qg, m_run, l_run, acc,
                                             L - rows, mask);
    buf ^= 1;
  };
  for (int tok0 = c0; tok0 < end; tok0 += kAhead * kTile) {
#pragma unroll
    for (int k = 0; k < kAhead; ++k) {
      if (tok0 + k * kTile >= end) break;
      step(stage[k], tok0 + k * kTile);
    }
  }
  if (row_active) {
    const int hq = g * G + (c % G);
    const int64_t st = ((int64_t(r) * rows + row) * a.num_q_heads + hq) * a.num_chunks + chunk;
    write_row_state<D, G>(a, st, c, qg, poison, m_run, l_run, acc);
  }
}

struct MergeArgs {
  const float* part_m;
  const float* part_l;
  const float* part_o;
  float* out;
  int32_t n;      // chunk states per (request, head)
  int32_t group;  // consecutive chunk states folded by one level-1 group
};

// Fold states [k0, k1) of one (request, head) over 4 dims: the maximum first, then
// every state weighted by e^(m_k - M) (0 for an empty state) in ascending k.
// Returns false if a maximum is NaN (a poisoned chunk).
__device__ __forceinline__ bool fold_states(const float* m, const float* l, const float* o,
                                            int64_t stride, int k0, int k1, float& M, float& S,
                                            floatx4& O) {
  if (k1 - k0 <= 8) {
    // Up to eight states: every load is issued before any arithmetic (one memory round
    // trip); the same order of operations as below.
    float mk[8], lk[8];
    floatx4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (k0 + u < k1) {
        mk[u] = m[k0 + u];
        lk[u] = l[k0 + u];
        v[u] = *reinterpret_cast<const floatx4*>(o + int64_t(k0 + u) * stride);
      }
    }
    M = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k0 + u < k1) {
        nan |= mk[u] != mk[u];
        M = fmaxf(M, mk[u]);
      }
    S = 0.0f;
    O = floatx4{0.f, 0.f, 0.f, 0.f};
    if (nan || M == -INFINITY) return !nan;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k0 + u < k1) {
        const float w = mk[u] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((mk[u] - M) * kLog2e);
        S += w * lk[u];
        O += w * v[u];
      }
    return true;
  }
  M = -INFINITY;
  bool nan = false;
  for (int k = k0; k < k1; ++k) {
    const float x = m[k];
    nan |= x != x;
    M = fmaxf(M, x);
  }
  S = 0.0f;
  O = floatx4{0.f, 0.f, 0.f, 0.f};
  if (nan || M == -INFINITY) return !nan;
  int k = k0;
  for (; k + 4 <= k1; k += 4) {  // four independent loads in flight
    floatx4 v[4];
    float w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[u] = *reinterpret_cast<const floatx4*>(o + int64_t(k + u) * stride);
      const float x = m[k + u];
      w[u] = x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((x - M) * kLog2e);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      S += w[u] * l[k + u];
      O += w[u] * v[u];
    }
  }
  for (; k < k1; ++k) {
    const float x = m[k];
    const float w = x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((x - M) * kLog2e);
    S += w * l[k];
    O += w * *reinterpret_cast<const floatx4*>(o + int64_t(k) * stride);
  }
  return true;
}

// One workgroup per (128-dim slab, request*head).  Level 1: thread group gi (32
// threads, 4 dims each) folds chunk states [gi*group, (gi+1)*group) into a group
// state kept in LDS (out of place: chunk states are only read).  Level 2: group 0
// folds the group states in ascending order and writes O / S.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  __shared__ float sm[kMergeGroups], sl[kMergeGroups];
  __shared__ floatx4 so[kMergeGroups][32];
  const int t = threadIdx.x;
  const int gi = t >> 5;
  const int d4 = t & 31;
  const int64_t bh = blockIdx.y;
  const int dim = blockIdx.x * 128 + 4 * d4;
  const float qnan = __builtin_nanf("");

  float M, S;
  floatx4 O;
  const int k0 = gi * a.group;
  const int k1 = min(k0 + a.group, a.n);
  if (!fold_states(a.part_m + bh * a.n, a.part_l + bh * a.n, a.part_o + bh * a.n * D + dim, D, k0,
                   k1, M, S, O)) {
    M = S = qnan;
    O = floatx4{qnan, qnan, qnan, qnan};
  }
  if (d4 == 0) {
    sm[gi] = M;
    sl[gi] = S;
  }
  so[gi][d4] = O;
  __syncthreads();
  if (gi == 0) {
    float M2, S2;
    floatx4 O2;
    if (!fold_states(sm, sl, reinterpret_cast<const float*>(&so[0][d4]), 32 * 4, 0, kMergeGroups,
                     M2, S2, O2)) {
      S2 = qnan;
      O2 = floatx4{qnan, qnan, qnan, qnan};
    }
    *reinterpret_cast<floatx4*>(a.out + bh * D + dim) = O2 / S2;
  }
}

struct WriteArgs {
  const float* k;
  const float* v;
  const int32_t* start_pos;
  char* pool;
  const int32_t* table;
  int32_t* bad_rows;
  // Pool strides and column offsets in bytes.
  int64_t page_stride, head_stride, row_stride, k_offset, v_offset, num_pages;
  int32_t num_kv_heads, head_dim, kcols, num_new, page_size, max_pages;
  float k_scale, v_scale;  // written value = x / factor (the decode multiplies back)
};

// One stored element type's encoding of 8 consecutive float32 values (16 bytes of bf16 or
// f16, 8 of FP8, 32 of f32), stored at dst.
template <int KV>
struct Writer;

template <>
struct Writer<ATTN_KV_BF16> {  // nearest, ties to even (v_cvt_pk_bf16_f32)
  static __device__ __forceinline__ void put(char* dst, floatx4 x0, floatx4 x1) {
    bf16x8 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[e] = (__bf16)x0[e];
      y[e + 4] = (__bf16)x1[e];
    }
    *reinterpret_cast<bf16x8*>(dst) = y;
  }
};

template <>
struct Writer<ATTN_KV_F16> {  // IEEE binary16, nearest, ties to even; overflow to infinity
  static __device__ __forceinline__ void put(char* dst, floatx4 x0, floatx4 x1) {
    halfx8 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      y[e] = (_Float16)x0[e];
      y[e + 4] = (_Float16)x1[e];
    }
    *reinterpret_cast<halfx8*>(dst) = y;
  }
};

template <>
struct Writer<ATTN_KV_F32> {
  static __device__ __forceinline__ void put(char* dst, floatx4 x0, floatx4 x1) {
    *reinterpret_cast<floatx4*>(dst) = x0;
    *reinterpret_cast<floatx4*>(dst + 16) = x1;
  }
};

// OCP E4M3 code of a float32: nearest representable value, a tie to the even mantissa;
// magnitudes from 448 up (infinity included) saturate to 448, NaN gives S.1111.111, and
// the sign of a result that rounds to zero is kept.
__device__ __forceinline__ unsigned e4m3_code(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const unsigned sgn = (u >> 24) & 0x80u;
  const unsigned a = u & 0x7FFFFFFFu;
  unsigned mag;
  if (a > 0x7F800000u) {
    mag = 0x7Fu;                                            // NaN
  } else if (a >= 0x43E00000u) {
    mag = 0x7Eu;                                            // >= 448: saturate
  } else if (a < 0x3C800000u) {
    // below the smallest normal 2^-6: subnormal steps of 2^-9 (exact scaling, then round
    // half to even); 8 steps is the smallest normal, code 0x08
    mag = unsigned(__builtin_rintf(__builtin_fabsf(x) * 512.0f));
  } else {
    // keep 3 of the 23 mantissa bits, rounding half to even (a carry moves the exponent);
    // the exponent bias goes from 127 to 7
    mag = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  }
  return sgn | mag;
}

template <>
struct Writer<ATTN_KV_FP8_E4M3> {
  static __device__ __forceinline__ void put(char* dst, floatx4 x0, floatx4 x1) {
    u32x2 y;
    y[0] = e4m3_code(x0[0]) | (e4m3_code(x0[1]) << 8) | (e4m3_code(x0[2]) << 16) |
           (e4m3_code(x0[3]) << 24);
    y[1] = e4m3_code(x1[0]) | (e4m3_code(x1[1]) << 8) | (e4m3_code(x1[2]) << 16) |
           (e4m3_code(x1[3]) << 24);
    *reinterpret_cast<u32x2*>(dst) = y;
  }
};

// New K/V rows into their pages: one workgroup per (request, token, KV head) row, one
// thread per 8 values (read as two 16-byte fp32 loads, divided by the tensor's factor
// unless it is 1, encoded as the pool's element type).  The row's position and page are
// workgroup-uniform.  Rows whose position or page is outside the table / pool are
// skipped and flagged.
template <int KV>
__global__ __launch_bounds__(128) void kv_write_kernel(WriteArgs a) {
  constexpr int EB = KV == ATTN_KV_FP8_E4M3 ? 1 : KV == ATTN_KV_F32 ? 4 : 2;  // bytes per element
  const int64_t row = blockIdx.x;  // ((r * num_new) + i) * num_kv_heads + g
  const int g = int(row % a.num_kv_heads);
  const int64_t ri = row / a.num_kv_heads;
  const int i = int(ri % a.num_new);
  const int r = int(ri / a.num_new);
  const int pc = threadIdx.x;
  const int kp = a.kcols / 8;
  if (pc >= kp + a.head_dim / 8) return;
  const int64_t pos = int64_t(a.start_pos[r]) + i;
  bool ok = pos >= 0 && pos < int64_t(a.max_pages) * a.page_size;
  int32_t pid = -1;
  if (ok) {
    pid = a.table[int64_t(r) * a.max_pages + pos / a.page_size];
    ok = pid >= 0 && int64_t(pid) < a.num_pages;
  }
  if (!ok) {
    if (a.bad_rows && pc == 0) *a.bad_rows = 1;
    return;
  }
  const float* src;
  int64_t col;
  float fac;
  if (pc < kp) {
    src = a.k + row * a.kcols + 8 * pc;
    col = a.k_offset + 8 * EB * pc;
    fac = a.k_scale;
  } else {
    src = a.v + row * a.head_dim + 8 * (pc - kp);
    col = a.v_offset + 8 * EB * (pc - kp);
    fac = a.v_scale;
  }
  floatx4 x0 = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(src));
  floatx4 x1 = __builtin_nontemporal_load(reinterpret_cast<const floatx4*>(src + 4));
  if (fac != 1.0f) {  // x / factor, one correctly rounded division each (exact for 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x0[e] = __fdiv_rn(x0[e], fac);
      x1[e] = __fdiv_rn(x1[e], fac);
    }
  }
  char* dst = a.pool + int64_t(pid) * a.page_stride + int64_t(g) * a.head_stride +
              (pos % a.page_size) * a.row_stride + col;
  Writer<KV>::put(dst, x0, x1);
}

// q' = q with columns rot.. multiplied by the norm weight (one float32 product each).
__global__ __launch_bounds__(256) void query_fold_kernel(const float* q, const float* w, float* out,
                                                          int64_t quads, int head_dim, int rot) {
  const int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (t >= quads) return;
  const int d = int((4 * t) % head_dim);
  floatx4 x = *reinterpret_cast<const floatx4*>(q + 4 * t);
  if (d >= rot) x *= *reinterpret_cast<const floatx4*>(w + (d - rot));
  *reinterpret_cast<floatx4*>(out + 4 * t) = x;
}

template <int D, int G, bool FOLDED, int KV>
void launch_split(const SplitArgs& args, dim3 grid, hipStream_t s) {
  if (args.num_rows > 1)
    hipLaunchKernelGGL((rows_partial_kernel<D, G, FOLDED, KV>), grid, dim3(64 * kWavesPerBlock), 0,
                       s, args);
  else if constexpr (KV == ATTN_KV_FP8_E4M3)
    hipLaunchKernelGGL((fp8_ring_kernel<D, G, FOLDED>), grid, dim3(64 * kWavesPerBlock), 0, s, args);
  else
    hipLaunchKernelGGL((split_partial_kernel<D, G, FOLDED, KV>), grid, dim3(64 * kWavesPerBlock), 0,
                       s, args);
}

template <int D, int G, bool FOLDED>
void launch_split_kv(int kv_dtype, const SplitArgs& args, dim3 grid, hipStream_t s) {
  if (kv_dtype == ATTN_KV_F32) {  // any number of rows; folded rows at head dim 512
    hipLaunchKernelGGL((f32_partial_kernel<D, G, FOLDED, false>), grid, dim3(64 * kWavesPerBlock),
                       0, s, args);
    return;
  }
  switch (kv_dtype) {
    case ATTN_KV_F16: launch_split<D, G, FOLDED, ATTN_KV_F16>(args, grid, s); break;
    case ATTN_KV_FP8_E4M3: launch_split<D, G, FOLDED, ATTN_KV_FP8_E4M3>(args, grid, s); break;
    default: launch_split<D, G, FOLDED, ATTN_KV_BF16>(args, grid, s); break;
  }
}

template <int D>
void launch_merge(const attn_decode_plan_t& p, char* ws, float* out, hipStream_t s) {
  const int64_t bh = int64_t(p.desc.batch) * p.num_rows * p.desc.num_q_heads;
  MergeArgs m{reinterpret_cast<const float*>(ws + p.off_part_m),
              reinterpret_cast<const float*>(ws + p.off_part_l),
              reinterpret_cast<const float*>(ws + p.off_part_o), out, p.num_chunks, p.merge_group};
  hipLaunchKernelGGL((merge_kernel<D>), dim3(D / 128, bh), dim3(256), 0, s, m);
}

}  // namespace

// Prefill over an f32 pool: the f32 kernel in its prefill mode, one workgroup
// per R = 16 / G consecutive prompt rows of one (request, KV head).
void launch_f32_prefill(const attn_prefill_plan_t& p, const float* q, const void* kv_pool,
                        const int32_t* page_table, const int32_t* seq_lens, const int32_t* q_starts,
                        float* out, void* stream) {
  const attn_decode_desc& d = p.desc;
  SplitArgs args{};
  const int64_t eb = kv_elem_bytes(d.kv_dtype);
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
  args.page_size = d.page_size;
  args.max_pages = d.max_pages_per_seq;
  args.window = d.window;
  args.qscale_k = d.scale * kLog2e * d.k_scale;
  args.qscale_v = d.scale * kLog2e * d.v_scale;
  args.vscale = d.v_scale;
  args.q_starts = q_starts;
  args.out = out;
  args.total_rows = p.total_rows;
  args.max_rows = p.max_rows;
  args.row_tiles = p.grid_x;
  args.num_kv_heads = d.num_kv_heads;
  args.items = p.grid_x * d.num_kv_heads * d.batch;  // bounded by the plan
  const dim3 grid((args.items + 255) / 256 * 256);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (d.head_dim == 512 && d.format == ATTN_KV_FOLDED)
    hipLaunchKernelGGL((f32_partial_kernel<512, 8, true, true>), grid, dim3(64 * kWavesPerBlock), 0,
                       s, args);
  else if (d.head_dim == 512)
    hipLaunchKernelGGL((f32_partial_kernel<512, 8, false, true>), grid, dim3(64 * kWavesPerBlock), 0,
                       s, args);
  else
    hipLaunchKernelGGL((f32_partial_kernel<256, 2, false, true>), grid, dim3(64 * kWavesPerBlock), 0,
                       s, args);
}

namespace {

int launch_status() {
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

}  // namespace
}  // namespace attn

namespace attn {
namespace {

// The split launch of attn_decode_split (row_masks null: causal rows) and
// attn_decode_split_tree.
int split_launch(const attn_decode_plan_t* plan, const float* q, const void* kv_pool,
                 const int32_t* page_table, const int32_t* seq_lens, const uint64_t* row_masks,
                 void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_plan(plan);
  if (rc != ATTN_OK) return rc;
  if (!q || !kv_pool || !page_table || !seq_lens) return ATTN_E_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kv_pool) || !aligned_to(page_table, 4) || !aligned_to(seq_lens, 4) ||
      !aligned_to(row_masks, 8))
    return ATTN_E_INVALID_ARG;
  rc = check_workspace(plan, workspace, workspace_bytes);
  if (rc != ATTN_OK) return rc;
  const attn_decode_desc& d = plan->desc;
  if (!shape_supported(d)) return ATTN_E_UNSUPPORTED;

  char* ws = static_cast<char*>(workspace);
  SplitArgs args;
  const int64_t eb = kv_elem_bytes(d.kv_dtype);
  args.q = q;
  args.pool = static_cast<const char*>(kv_pool);
  args.table = page_table;
  args.seq_lens = seq_lens;
  args.part_m = reinterpret_cast<float*>(ws + plan->off_part_m);
  args.part_l = reinterpret_cast<float*>(ws + plan->off_part_l);
  args.part_o = reinterpret_cast<float*>(ws + plan->off_part_o);
  args.page_stride = d.page_stride * eb;
  args.head_stride = d.head_stride * eb;
  args.row_stride = d.row_stride * eb;
  args.k_offset = d.k_offset * eb;
  args.v_offset = d.v_offset * eb;
  args.num_pages = d.num_pages;
  args.num_q_heads = d.num_q_heads;
  args.page_size = d.page_size;
  args.max_pages = d.max_pages_per_seq;
  args.window = d.window;
  args.chunk_len = plan->chunk_len;
  args.chunk_len_odd = plan->chunk_len_odd;
  args.num_chunks = plan->num_chunks;
  args.num_rows = plan->num_rows;
  args.row_groups = plan->row_groups;
  args.row_masks = row_masks;
  args.qscale_k = d.scale * kLog2e * d.k_scale;
  args.qscale_v = d.scale * kLog2e * d.v_scale;
  args.vscale = d.v_scale;

  const dim3 grid(plan->grid_x, d.num_kv_heads, d.batch);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (rows_on_tiles(d, plan->num_rows))
    launch_rows_tiles(*plan, q, kv_pool, page_table, seq_lens, row_masks, args.part_m,
                      args.part_l, args.part_o, stream);
  else if (d.head_dim == 512 && d.format == ATTN_KV_SPLIT)
    launch_split_kv<512, 8, false>(d.kv_dtype, args, grid, s);
  else if (d.head_dim == 512 && d.format == ATTN_KV_FOLDED)
    launch_split_kv<512, 8, true>(d.kv_dtype, args, grid, s);
  else
    launch_split_kv<256, 2, false>(d.kv_dtype, args, grid, s);
  return launch_status();
}

}  // namespace
}  // namespace attn

extern "C" int attn_decode_split(const attn_decode_plan_t* plan, const float* q, const void* kv_pool,
                                 const int32_t* page_table, const int32_t* seq_lens, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  return attn::split_launch(plan, q, kv_pool, page_table, seq_lens, nullptr, workspace,
                            workspace_bytes, stream);
}

extern "C" int attn_decode_split_tree(const attn_decode_plan_t* plan, const float* q,
                                      const void* kv_pool, const int32_t* page_table,
                                      const int32_t* seq_lens, const uint64_t* row_masks,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = attn::check_plan(plan);
  if (rc != ATTN_OK) return rc;
  if (!row_masks || plan->num_rows < 2) return ATTN_E_INVALID_ARG;
  return attn::split_launch(plan, q, kv_pool, page_table, seq_lens, row_masks, workspace,
                            workspace_bytes, stream);
}

extern "C" int attn_decode_merge(const attn_decode_plan_t* plan, void* workspace,
                                 size_t workspace_bytes, float* out, void* stream) {
  using namespace attn;
  int rc = check_plan(plan);
  if (rc != ATTN_OK) return rc;
  if (!out || !aligned16(out)) return ATTN_E_INVALID_ARG;
  rc = check_workspace(plan, workspace, workspace_bytes);
  if (rc != ATTN_OK) return rc;
  if (!shape_supported(plan->desc)) return ATTN_E_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (plan->desc.head_dim == 512)
    launch_merge<512>(*plan, static_cast<char*>(workspace), out, s);
  else
    launch_merge<256>(*plan, static_cast<char*>(workspace), out, s);
  return launch_status();
}

extern "C" int attn_kv_write(const attn_decode_plan_t* plan, const float* k, const float* v,
                             int32_t num_new, const int32_t* start_pos, void* kv_pool,
                             const int32_t* page_table, int32_t* bad_rows, void* stream) {
  using namespace attn;
  int rc = check_plan(plan);
  if (rc != ATTN_OK) return rc;
  if (!k || !v || !start_pos || !kv_pool || !page_table || num_new < 1) return ATTN_E_INVALID_ARG;
  if (!aligned16(k) || !aligned16(v) || !aligned16(kv_pool) || !aligned_to(start_pos, 4) ||
      !aligned_to(page_table, 4) || !aligned_to(bad_rows, 4))
    return ATTN_E_INVALID_ARG;
  const attn_decode_desc& d = plan->desc;
  if (!kv_dtype_served(d.kv_dtype)) return ATTN_E_UNSUPPORTED;
  const int64_t eb = kv_elem_bytes(d.kv_dtype);
  const int kcols = d.format == ATTN_KV_FOLDED ? d.rot_cols : d.head_dim;
  const int row_pieces = (kcols + d.head_dim) / 8;  // at most 128 for the supported shapes
  int64_t rows;
  if (__builtin_mul_overflow(int64_t(d.batch) * d.num_kv_heads, int64_t(num_new), &rows))
    return ATTN_E_OVERFLOW;
  if (rows > INT32_MAX || row_pieces > 128) return ATTN_E_OVERFLOW;
  WriteArgs a;
  a.k = k;
  a.v = v;
  a.start_pos = start_pos;
  a.pool = static_cast<char*>(kv_pool);
  a.table = page_table;
  a.bad_rows = bad_rows;
  a.page_stride = d.page_stride * eb;
  a.head_stride = d.head_stride * eb;
  a.row_stride = d.row_stride * eb;
  a.k_offset = d.k_offset * eb;
  a.v_offset = d.v_offset * eb;
  a.k_scale = d.k_scale;
  a.v_scale = d.v_scale;
  a.num_pages = d.num_pages;
  a.num_kv_heads = d.num_kv_heads;
  a.head_dim = d.head_dim;
  a.kcols = kcols;
  a.num_new = num_new;
  a.page_size = d.page_size;
  a.max_pages = d.max_pages_per_seq;
  (void)hipGetLastError();
  const dim3 grid{unsigned(rows)}, block{unsigned(row_pieces)};
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (d.kv_dtype) {
    case ATTN_KV_F16: hipLaunchKernelGGL(kv_write_kernel<ATTN_KV_F16>, grid, block, 0, s, a); break;
    case ATTN_KV_FP8_E4M3: hipLaunchKernelGGL(kv_write_kernel<ATTN_KV_FP8_E4M3>, grid, block, 0, s, a); break;
    case ATTN_KV_F32: hipLaunchKernelGGL(kv_write_kernel<ATTN_KV_F32>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(kv_write_kernel<ATTN_KV_BF16>, grid, block, 0, s, a); break;
  }
  return launch_status();
}

extern "C" int attn_query_fold(const attn_decode_plan_t* plan, const float* q, const float* norm_w,
                               float* q_out, void* stream) {
  using namespace attn;
  int rc = check_plan(plan);
  if (rc != ATTN_OK) return rc;
  if (!q || !norm_w || !q_out) return ATTN_E_INVALID_ARG;
  if (!aligned16(q) || !aligned16(norm_w) || !aligned16(q_out)) return ATTN_E_INVALID_ARG;
  const attn_decode_desc& d = plan->desc;
  if (d.format != ATTN_KV_FOLDED) return ATTN_E_UNSUPPORTED;
  const int64_t quads = int64_t(d.batch) * d.num_q_heads * d.head_dim / 4;
  (void)hipGetLastError();
  hipLaunchKernelGGL(query_fold_kernel, dim3(unsigned((quads + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), q, norm_w, q_out, quads, d.head_dim, d.rot_cols);
  return launch_status();
}


// ---------------------------------------------------------------------------------------
// Allocation-free decode step, for callers that cannot allocate device memory.  The chunk
// states (the workspace of attn_decode_split / attn_decode_merge) live in one static device
// array per GPU.  In host code `scratch` names a host-side stand-in, not device memory:
// its device address is taken once per device with hipGetSymbolAddress and only that
// address is ever handed to a kernel.
namespace attn {

__device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (looked up on the first call
// on that device, with it current).
int scratch_of_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_E_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return ATTN_E_LAUNCH;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = static_cast<char*>(g_scratch_ptr[dev]);
  return ATTN_OK;
}

}  // namespace
}  // namespace attn

extern "C" int attn_decode_step_noalloc(const attn_decode_plan_t* plan, const float* q,
                                        const void* kv_pool, const int32_t* page_table,
                                        const int32_t* seq_lens, const uint64_t* row_masks,
                                        float* out, void* stream) {
  using namespace attn;
  int rc = check_plan(plan);
  if (rc != ATTN_OK) return rc;
  if (row_masks && plan->num_rows < 2) return ATTN_E_INVALID_ARG;
  if (!q || !kv_pool || !page_table || !seq_lens || !out) return ATTN_E_INVALID_ARG;
  if (!aligned16(q) || !aligned16(kv_pool) || !aligned16(out) || !aligned_to(page_table, 4) ||
      !aligned_to(seq_lens, 4) || !aligned_to(row_masks, 8))
    return ATTN_E_INVALID_ARG;
  if (!shape_supported(plan->desc)) return ATTN_E_UNSUPPORTED;
  if (plan->workspace_bytes > uint64_t(ATTN_NOALLOC_SCRATCH_BYTES)) return ATTN_E_SCRATCH;
  char* ws = nullptr;
  rc = scratch_of_current_device(&ws);
  if (rc != ATTN_OK) return rc;
  // The same launches as attn_decode_split (or _split_tree) and attn_decode_merge, with
  // the static array as their workspace; every state the merge reads is written first,
  // so nothing needs clearing.
  rc = split_launch(plan, q, kv_pool, page_table, seq_lens, row_masks, ws,
                    ATTN_NOALLOC_SCRATCH_BYTES, stream);
  if (rc != ATTN_OK) return rc;
  return attn_decode_merge(plan, ws, ATTN_NOALLOC_SCRATCH_BYTES, out, stream);
}
