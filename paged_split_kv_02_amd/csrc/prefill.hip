// Paged prefill for gfx950 (MI355X): prompt rows attending causally to their request's
// keys through the page table, the normalised output written directly.
//
// pegainfer PR #1055 ("Description") runs the global family's prompt rows through a
// prefill over the split or folded pool; pegainfer PR #1057 ("Description") runs the
// sliding family's prompt rows through a varlen kernel with a window lower bound over
// pages of 64; TensorFold PR #1619 ("body") reads prompt rows through the slot's
// page-table row.  A row at position p sees the keys lo .. p (lo = p + 1 - window with a
// window): it is a decode token at length p + 1.
//
// One workgroup = row_tile consecutive prompt rows of one (request, KV head).  Each of its
// four waves owns 16 MFMA columns: (16 / G) rows x the G query heads of the KV head.
// Per 32-key tile (whole tiles inside one page: the page id is read once per tile):
//   * the tile's stored rows are copied from the pool straight into LDS with 16-byte
//     global->LDS loads (no registers involved); the next tile is requested as soon as
//     its buffer is free, so it lands while the current one is used.  The 16-byte chunks
//     of a row are XOR-swizzled inside each 256-byte group (chunk lc of row k sits at
//     lc ^ (k & 15)), which keeps both LDS read patterns below free of bank conflicts
//     without padding, so every 1-KB load instruction fills one contiguous kilobyte;
//   * S^T = K Q^T on MFMA (keys as rows, (row, head) as columns).  The fp32 query, with
//     scale * log2(e) folded in, is split into a high and a low bf16 part and both are
//     multiplied against each K fragment, so the scores keep ~16 mantissa bits;
//   * causal and window masks by select; online softmax in base 2 with the reference
//     maximum moved only when a tile exceeds it by 2^8 (rare rescales);
//   * O^T += V^T P^T on MFMA with the probabilities again as high and low bf16 parts,
//     taken straight from the score registers; V^T is assembled from 16-byte LDS row
//     reads with byte permutes.  V rows of keys no row of the workgroup may see are
//     zeroed on the way, so padding (NaN or huge) never reaches the sums.
// The fp32 output accumulators (128 per lane at head dim 512) live in the accumulation
// registers, the split query operand (128) in the vector registers.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "plan_internal.h"

namespace attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kRescaleSlack = 8.0f;  // log2 units; probabilities stay below 2^8
constexpr int kKeys = kPrefillKeys;    // keys per tile: two 16-key MFMA blocks
// Without rescaling, probabilities may reach 2^kHeadroom (log2 units above a column's
// reference): far inside fp32 and bf16 range, with room for any sum of them.
constexpr float kHeadroom = 64.0f;

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
  float qscale_k;  // scale * log2(e) * k_scale: query dims that meet K columns
  float qscale_v;  // scale * log2(e) * v_scale: folded query dims that meet V columns
  float vscale;    // v_scale, applied to the output
};

template <int D, bool FOLDED>
struct PShape {
  static constexpr int ROT = FOLDED ? 128 : 0;
  static constexpr int COLS = FOLDED ? ROT + D : 2 * D;  // staged elements per row
  static constexpr int ROW_BYTES = 2 * COLS;
  static constexpr int TILE_BYTES = kKeys * ROW_BYTES;
  static constexpr int TV = FOLDED ? ROT : D;            // staged column of V[0]
  static constexpr int KSTEPS = D / 32;                  // 32-dim MFMA steps of QK
  static constexpr int SLABS = D / 128;                  // 128-dim slabs of PV
  static constexpr int LOADS = TILE_BYTES / (1024 * kWavesPerBlock);  // 1-KB loads per wave
  static_assert(TILE_BYTES % (1024 * kWavesPerBlock) == 0, "whole 1-KB loads per wave");
  static_assert(ROW_BYTES % 256 == 0, "rows are whole 256-byte swizzle groups");
};

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ unsigned perm(unsigned hi, unsigned lo, unsigned sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ floatx4 mma(u32x4 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b, c, 0, 0, 0);
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

// LDS byte offset of logical 16-byte chunk lc of staged row k.
template <int ROW_BYTES>
__device__ __forceinline__ int lds_off(int k, int lc) {
  return k * ROW_BYTES + ((lc ^ (k & 15)) << 4);
}

// Request one tile into `lds`.  `base` is the pool address of the tile's first row (page,
// KV head, slot).  Load instruction u = k * 4 + wave fills LDS bytes [1024u, 1024u + 1024):
// lane l's 16 bytes land at 1024u + 16l, i.e. physical chunk pc of staged row k, which
// holds logical chunk pc ^ (k & 15) of that row.  `lane` is passed through an opaque
// move first, so the per-lane offsets are recomputed here rather than kept live.
template <int D, bool FOLDED>
__device__ __forceinline__ void issue_tile(const PrefillArgs& a, const char* base, char* lds,
                                           int wave, int lane) {
  using S = PShape<D, FOLDED>;
  asm volatile("" : "+v"(lane));
#pragma unroll
  for (int k = 0; k < S::LOADS; ++k) {
    const int u = k * kWavesPerBlock + wave;
    const int o = u * 1024 + lane * 16;
    const int row = o / S::ROW_BYTES;
    const int lc = ((o % S::ROW_BYTES) >> 4) ^ (row & 15);
    const uint32_t off = uint32_t(row * int32_t(a.row_stride)) +
                         uint32_t(piece_col<D, FOLDED>(a, lc >> 4)) + uint32_t((lc & 15) << 4);
    __builtin_amdgcn_global_load_lds(base + off, (lds_void*)(lds + u * 1024), 16, 0, 0);
  }
}

template <int D, int G, bool FOLDED>
__global__ __launch_bounds__(256, D == 256 ? 2 : 1) void prefill_kernel(PrefillArgs a) {
  using S = PShape<D, FOLDED>;
  constexpr int RB = S::ROW_BYTES;
  constexpr int RPC = kPrefillColumns / G;     // rows per wave
  constexpr int QT = RPC * kWavesPerBlock;     // rows per workgroup
  static_assert(kPrefillColumns % G == 0, "a wave holds whole rows");
  __shared__ __attribute__((aligned(1024))) char buf0[S::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char buf1[S::TILE_BYTES];

  const int lane = threadIdx.x & 63;
  const int c = lane & 15;   // MFMA column (row, head) / K row inside a 16-key block
  const int qg = lane >> 4;  // lane group: k sub-range / output rows
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int g = blockIdx.y;
  const int r = blockIdx.z;
  const int tile = a.row_tiles - 1 - int(blockIdx.x);  // the longest rows start first

  // Offsets the plan cannot serve are not followed: nothing is read or written.
  const int qs0 = a.q_starts[r];
  const int qs1 = a.q_starts[r + 1];
  const int n = qs1 - qs0;
  if (qs0 < 0 || n < 0 || n > a.max_rows || qs1 > a.total_rows) return;
  const int row0 = tile * QT;
  if (row0 >= n) return;
  const int L = a.seq_lens[r];
  bool poison = L < n || int64_t(L) > int64_t(a.max_pages) * a.page_size;

  // This lane's column: row qrow of the request, query head `head`; it sees keys lo_c .. pos.
  const int qrow = row0 + wave * RPC + c / G;
  const bool active = qrow < n;
  const int head = g * G + c % G;
  const int pos = (active && !poison) ? L - n + qrow : -1;
  const int lo_c = a.window > 0 ? max(0, pos + 1 - a.window) : 0;

  // Keys of the workgroup: the first row's window start .. the last row's position.
  const int pos_first = L - n + row0;
  const int pos_last = L - n + min(row0 + QT, n) - 1;
  const int lo_first = a.window > 0 ? max(0, pos_first + 1 - a.window) : 0;
  const int start = lo_first & ~(kKeys - 1);
  int ntiles = poison ? 0 : (pos_last + 1 - start + kKeys - 1) / kKeys;

  const int32_t* trow = a.table + int64_t(r) * a.max_pages;
  const char* head_base = a.pool + int64_t(g) * a.head_stride;
  // Pool address of the tile starting at key k0, or null if its page id is outside the pool.
  auto tile_base = [&](int k0) -> const char* {
    const int32_t pid = table_entry(trow, k0 / a.page_size);
    if (pid < 0 || int64_t(pid) >= a.num_pages) return nullptr;
    return head_base + int64_t(pid) * a.page_stride + int64_t(k0 % a.page_size) * a.row_stride;
  };

  // Request the first tile, then prepare the query operand while it streams.
  if (ntiles > 0) {
    const char* b = tile_base(start);
    if (b) {
      issue_tile<D, FOLDED>(a, b, buf0, wave, lane);
    } else {
      poison = true;
      ntiles = 0;
    }
  }

  // Query operand (B of the QK MFMA): lane (c, qg), k-step j holds dims 32j + 8qg + [0, 8)
  // of column c, as a high and a low bf16 part.
  bf16x8 qhi[S::KSTEPS], qlo[S::KSTEPS];
  {
    const float* qp = a.q + (int64_t(qs0) + (active ? qrow : 0)) * a.num_q_heads * D +
                      int64_t(head) * D;
#pragma unroll
    for (int j = 0; j < S::KSTEPS; ++j) {
      const float qs = (FOLDED && 32 * j >= S::ROT) ? a.qscale_v : a.qscale_k;
      floatx4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
      if (active) {
        x0 = *reinterpret_cast<const floatx4*>(qp + 32 * j + 8 * qg);
        x1 = *reinterpret_cast<const floatx4*>(qp + 32 * j + 8 * qg + 4);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = (e < 4 ? x0[e & 3] : x1[e & 3]) * qs;
        const __bf16 h = (__bf16)x;
        qhi[j][e] = h;
        qlo[j][e] = (__bf16)(x - (float)h);
      }
    }
  }

  float m_run, l_run;
  floatx4 acc[S::SLABS][8];  // slab b, step jj: lane (c, qg) rows 4qg + i <-> dims 128b + 8(4qg+i) + jj
  bool overflow = false;     // a score exceeded the reference by more than kHeadroom

  // One staged tile (keys k0 .. k0 + 31) for this wave's 16 columns.  Without RESCALE the
  // reference maximum of a column is fixed by its first tile with a visible key (the
  // accumulators are still zero then, so nothing is rescaled) and probabilities may grow
  // to 2^kHeadroom; a larger score only raises `overflow`.  With RESCALE (the slow path
  // for such workgroups) the reference follows the running maximum as in decode.
  auto compute = [&](const char* t, int k0, auto rescale) {
    constexpr bool RESCALE = decltype(rescale)::value;
    // Scores: block kb holds keys k0 + 16kb + 4qg + i (lane (c, qg), i = 0..3) of column c.
    // The K fragments of step j + 1 are read while step j multiplies.
    floatx4 sh0 = {0.f, 0.f, 0.f, 0.f}, sl0 = sh0, sh1 = sh0, sl1 = sh0;
    auto kfrag = [&](int j, int blk) {
      const int kd = 32 * j + 8 * qg;
      const int lc = ((FOLDED && kd >= S::ROT) ? S::TV + kd : kd) >> 3;
      return *reinterpret_cast<const u32x4*>(t + lds_off<RB>(16 * blk + c, lc));
    };
    u32x4 ka = kfrag(0, 0), kb = kfrag(0, 1);
#pragma unroll
    for (int j = 0; j < S::KSTEPS; ++j) {
      u32x4 na = ka, nb = kb;
      if (j + 1 < S::KSTEPS) {
        na = kfrag(j + 1, 0);
        nb = kfrag(j + 1, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      sh0 = mma(ka, qhi[j], sh0);
      sh1 = mma(kb, qhi[j], sh1);
      sl0 = mma(ka, qlo[j], sl0);
      sl1 = mma(kb, qlo[j], sl1);
      __builtin_amdgcn_sched_barrier(0);
      ka = na;
      kb = nb;
    }
    const floatx4 s0 = sh0 + sl0, s1 = sh1 + sl1;

    float sc[8];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = k0 + (e < 4 ? 4 * qg + e : 16 + 4 * qg + (e - 4));
      const float v = e < 4 ? s0[e] : s1[e - 4];
      sc[e] = (key >= lo_c && key <= pos) ? v : -INFINITY;
      mx = fmaxf(mx, sc[e]);
    }
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    if constexpr (RESCALE) {
      const bool grow = mx > m_run + kRescaleSlack;
      if (__builtin_expect(__any(grow), 0)) {
        const float m_new = grow ? mx : m_run;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 from -inf
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < S::SLABS; ++b)
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) acc[b][jj] *= alpha;
        m_run = m_new;
      }
    } else {
      if (m_run == -INFINITY) m_run = mx;  // first visible tile: nothing accumulated yet
      overflow |= mx > m_run + kHeadroom;
    }
    // Probabilities as the PV B operand: k index 8qg + e <-> key of sc[e].
    bf16x8 phi, plo;
    float psum = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p = m_run == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sc[e] - m_run);
      psum += p;
      const __bf16 h = (__bf16)p;
      phi[e] = h;
      plo[e] = (__bf16)(p - (float)h);
    }
    l_run += psum;

    // PV: A = V^T of slab b, step jj: lane (c, qg) dims 128b + 8c + jj, keys of sc[0..7].
    // Each slab's eight 16-byte V row reads are issued before its MFMAs.
    const bool edge = k0 < lo_first || k0 + kKeys - 1 > pos_last;  // uniform
#pragma unroll
    for (int b = 0; b < S::SLABS; ++b) {
      u32x4 w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kr = e < 4 ? 4 * qg + e : 16 + 4 * qg + (e - 4);
        w[e] = *reinterpret_cast<const u32x4*>(t + lds_off<RB>(kr, (S::TV >> 3) + 16 * b + c));
        if (__builtin_expect(edge, 0)) {
          const int key = k0 + kr;
          if (key < lo_first || key > pos_last) w[e] = u32x4{0u, 0u, 0u, 0u};
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        u32x4 ev, od;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          ev[u] = perm(w[2 * u + 1][dd], w[2 * u][dd], 0x05040100u);
          od[u] = perm(w[2 * u + 1][dd], w[2 * u][dd], 0x07060302u);
        }
        acc[b][2 * dd] = mma(ev, phi, acc[b][2 * dd]);
        acc[b][2 * dd + 1] = mma(od, phi, acc[b][2 * dd + 1]);
        acc[b][2 * dd] = mma(ev, plo, acc[b][2 * dd]);
        acc[b][2 * dd + 1] = mma(od, plo, acc[b][2 * dd + 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // All tiles of the workgroup, double-buffered: wait for this tile's loads (own, then
  // everyone's via the barrier, which also frees the other buffer), request the next tile
  // into the other buffer, use this one.
  auto run = [&](auto rescale) {
    m_run = -INFINITY;
    l_run = 0.0f;
#pragma unroll
    for (int b = 0; b < S::SLABS; ++b)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) acc[b][jj] = floatx4{0.f, 0.f, 0.f, 0.f};
    int count = ntiles;
    auto step = [&](const char* cur, char* nxt, int it) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      const int k0 = start + it * kKeys;
      if (it + 1 < count) {
        const char* b = tile_base(k0 + kKeys);
        if (b) {
          issue_tile<D, FOLDED>(a, b, nxt, wave, lane);
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
  };
  run(Flag<false>{});
  if (__syncthreads_or(overflow)) {  // uniform: every wave of the workgroup takes it
    __syncthreads();                 // the last tile's buffer is no longer read
    if (ntiles > 0) issue_tile<D, FOLDED>(a, tile_base(start), buf0, wave, lane);
    run(Flag<true>{});
  }

  if (!active) return;
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  float* o = a.out + (int64_t(qs0) + qrow) * a.num_q_heads * D + int64_t(head) * D;
  const float qnan = __builtin_nanf("");
#pragma unroll
  for (int b = 0; b < S::SLABS; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      floatx4 w0 = floatx4{acc[b][0][i], acc[b][1][i], acc[b][2][i], acc[b][3][i]} * a.vscale / l_run;
      floatx4 w1 = floatx4{acc[b][4][i], acc[b][5][i], acc[b][6][i], acc[b][7][i]} * a.vscale / l_run;
      if (poison) w0 = w1 = floatx4{qnan, qnan, qnan, qnan};
      float* dst = o + 128 * b + 32 * qg + 8 * i;
      *reinterpret_cast<floatx4*>(dst) = w0;
      *reinterpret_cast<floatx4*>(dst + 4) = w1;
    }
}

template <int D, int G, bool FOLDED>
void launch_prefill(const PrefillArgs& args, dim3 grid, hipStream_t s) {
  hipLaunchKernelGGL((prefill_kernel<D, G, FOLDED>), grid, dim3(64 * kWavesPerBlock), 0, s, args);
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
  const attn_decode_desc& d = plan->desc;
  if (!prefill_shape_supported(d)) return ATTN_E_UNSUPPORTED;
  if (plan->total_rows == 0) return ATTN_OK;

  const int64_t eb = kv_elem_bytes(d.kv_dtype);
  PrefillArgs args;
  args.q = q;
  args.out = out;
  args.pool = static_cast<const char*>(kv_pool);
  args.table = page_table;
  args.seq_lens = seq_lens;
  args.q_starts = q_starts;
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
  args.total_rows = plan->total_rows;
  args.max_rows = plan->max_rows;
  args.row_tiles = plan->grid_x;
  args.qscale_k = d.scale * kLog2e * d.k_scale;
  args.qscale_v = d.scale * kLog2e * d.v_scale;
  args.vscale = d.v_scale;

  const dim3 grid(plan->grid_x, d.num_kv_heads, d.batch);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (d.head_dim == 512 && d.format == ATTN_KV_SPLIT)
    launch_prefill<512, 8, false>(args, grid, s);
  else if (d.head_dim == 512 && d.format == ATTN_KV_FOLDED)
    launch_prefill<512, 8, true>(args, grid, s);
  else
    launch_prefill<256, 2, false>(args, grid, s);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}
