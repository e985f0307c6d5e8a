// Host-side planning for paged split-KV decode attention: validation, chunking
// and the workspace layout.  No device call is made here, so the plan can be
// built (and tested) on a machine without a GPU.
#include "plan_internal.h"

#include <cmath>
#include <cstring>

namespace {

constexpr uint64_t kAlign = 256;

bool mul_ok(uint64_t a, uint64_t b, uint64_t* out) { return !__builtin_mul_overflow(a, b, out); }
bool add_ok(uint64_t a, uint64_t b, uint64_t* out) { return !__builtin_add_overflow(a, b, out); }

bool align_up(uint64_t v, uint64_t* out) {
  uint64_t t;
  if (!add_ok(v, kAlign - 1, &t)) return false;
  *out = t / kAlign * kAlign;
  return true;
}

// Place a float32 region of `count` elements at *cursor (aligned), advance the cursor.
bool place(uint64_t* cursor, uint64_t count, uint64_t* offset) {
  uint64_t bytes, start, end;
  if (!mul_ok(count, 4, &bytes)) return false;
  if (!align_up(*cursor, &start)) return false;
  if (!add_ok(start, bytes, &end)) return false;
  *offset = start;
  *cursor = end;
  return true;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

namespace attn {

int kv_elem_bytes(int kv_dtype) {
  switch (kv_dtype) {
    case ATTN_KV_BF16: return 2;
    case ATTN_KV_F16: return 2;
    case ATTN_KV_FP8_E4M3: return 1;
    case ATTN_KV_F32: return 4;
    default: return 0;
  }
}

bool kv_dtype_served(int kv_dtype) {
  return kv_dtype == ATTN_KV_BF16 || kv_dtype == ATTN_KV_F16 || kv_dtype == ATTN_KV_FP8_E4M3 ||
         kv_dtype == ATTN_KV_F32;
}

bool shape_supported(const attn_decode_desc& d) {
  if (!kv_dtype_served(d.kv_dtype)) return false;
  const int g = d.num_q_heads / d.num_kv_heads;
  if (d.head_dim == 512 && g == 8) {
    if (d.format == ATTN_KV_SPLIT) return d.rot_cols == 0;
    if (d.format == ATTN_KV_FOLDED) return d.rot_cols == 128;
    return false;
  }
  if (d.head_dim == 256 && g == 2) return d.format == ATTN_KV_SPLIT && d.rot_cols == 0;
  return false;
}

// Last column (exclusive) a row read touches.
int64_t row_extent(const attn_decode_desc& d) {
  int64_t k_end = d.k_offset + (d.format == ATTN_KV_FOLDED ? d.rot_cols : d.head_dim);
  int64_t v_end = d.v_offset + d.head_dim;
  return k_end > v_end ? k_end : v_end;
}

// Checks shared by the decode and prefill plans: sizes, format, element type, scale
// factors, 16-byte aligned strides and offsets, rows inside their page, pool size.
int check_desc(const attn_decode_desc& d) {
  if (d.batch < 1 || d.num_q_heads < 1 || d.num_kv_heads < 1 || d.head_dim < 1 ||
      d.page_size < 1 || d.max_pages_per_seq < 1 || d.window < 0 || d.num_chunks < 0 ||
      d.merge_group < 0 || d.num_pages < 1 || d.num_rows < 0)
    return ATTN_E_INVALID_ARG;
  if (d.num_q_heads % d.num_kv_heads != 0) return ATTN_E_UNSUPPORTED;
  if (d.format != ATTN_KV_SPLIT && d.format != ATTN_KV_FOLDED) return ATTN_E_INVALID_ARG;
  const int eb = kv_elem_bytes(d.kv_dtype);
  if (eb == 0) return ATTN_E_INVALID_ARG;
  if (!shape_supported(d)) return ATTN_E_UNSUPPORTED;
  if (!std::isfinite(d.scale)) return ATTN_E_INVALID_ARG;
  if (!(std::isfinite(d.k_scale) && d.k_scale > 0.0f) ||
      !(std::isfinite(d.v_scale) && d.v_scale > 0.0f))
    return ATTN_E_INVALID_ARG;
  if (d.page_size % kTile != 0) return ATTN_E_UNSUPPORTED;

  // Layout: 16-byte aligned rows and columns, non-negative strides, rows inside their page.
  const int64_t v[] = {d.page_stride, d.head_stride, d.row_stride, d.k_offset, d.v_offset};
  for (int64_t x : v)
    if (x < 0 || x % (16 / eb) != 0) return ATTN_E_INVALID_ARG;
  {
    uint64_t a, b, c, e;
    if (!mul_ok(uint64_t(d.num_kv_heads - 1), uint64_t(d.head_stride), &a) ||
        !mul_ok(uint64_t(d.page_size - 1), uint64_t(d.row_stride), &b) || !add_ok(a, b, &c) ||
        !add_ok(c, uint64_t(row_extent(d)), &e))
      return ATTN_E_OVERFLOW;
    if (e > uint64_t(d.page_stride)) return ATTN_E_INVALID_ARG;
    uint64_t pool_elems;
    if (!mul_ok(uint64_t(d.num_pages), uint64_t(d.page_stride), &pool_elems) ||
        pool_elems > (uint64_t(1) << 60))
      return ATTN_E_OVERFLOW;
  }
  return ATTN_OK;
}

int make_plan(const attn_decode_desc* desc, const int32_t* lens, attn_decode_plan_t* plan) {
  if (!desc || !lens || !plan) return ATTN_E_INVALID_ARG;
  const attn_decode_desc& d = *desc;
  const int rc0 = check_desc(d);
  if (rc0 != ATTN_OK) return rc0;

  // Query rows: 1 = ordinary decode; a window of n rows uses groups of four rows.
  const int64_t rows = d.num_rows < 1 ? 1 : d.num_rows;
  if (rows > kMaxRows) return ATTN_E_INVALID_ARG;
  // Row groups: four rows per workgroup on the 16-bit kernels (one per wave, or a quarter of
  // the dims each); f32 pools put 16 / G rows of the G heads in the 16 MFMA columns, and
  // every wave streams a quarter of the chunk for all of them.
  const bool f32 = d.kv_dtype == ATTN_KV_F32;
  const int64_t per_group = f32 ? 16 / (d.num_q_heads / d.num_kv_heads) : kWavesPerBlock;
  const int64_t groups = rows > 1 ? ceil_div(rows, per_group) : 1;

  // Keys per tile of the partial kernel the shape runs on.
  const int64_t T = rows_on_tiles(d, rows) ? kPrefillKeys : kTile;

  // Lengths: rows <= L <= pages in a table row * page size.
  const int64_t cap = int64_t(d.max_pages_per_seq) * d.page_size;
  int64_t max_span = 0, max_start = 0;
  for (int r = 0; r < d.batch; ++r) {
    const int64_t L = lens[r];
    if (L < 1 || L < rows) return ATTN_E_INVALID_ARG;
    if (L > cap) return ATTN_E_PAST_PAGES;
    const int64_t first_hi = L - rows + 1;  // keys the first row sees: [.., first_hi)
    const int64_t lo = d.window > 0 && first_hi > d.window ? first_hi - d.window : 0;
    const int64_t start = lo / T * T;
    if (L - start > max_span) max_span = L - start;
    if (start > max_start) max_start = start;
  }
  if (max_span > INT32_MAX) return ATTN_E_OVERFLOW;

  // Chunking.  One row: one chunk per workgroup, one quarter of it per wave, so that
  // every SIMD of the chip streams one quarter; a quarter is never shorter than a
  // tile.  Several rows: the four waves share each tile (one row each on the 16-key
  // kernel, a quarter of the dims each on the 32-key one), so a chunk is whole tiles.
  // An explicit count is honoured (trailing chunks may then be empty).
  const int64_t split = (rows > 1 && !f32) ? 1 : kWavesPerBlock;  // waves a chunk is cut into
  const int64_t tiles = ceil_div(max_span, T);
  int64_t n = d.num_chunks;
  if (n == 0) {
    const int64_t units = int64_t(d.batch) * d.num_kv_heads * groups;
    // One workgroup per CU in one round.  At head dim 256 the kernels' registers and LDS
    // allow two per CU; filling both slots pays only on the f32 kernel (16 sliding
    // requests: 89 against 94 us).  The 16-bit and FP8 kernels run faster with one
    // workgroup per CU and chunks twice as long (16 requests 47.3 against 48.9 us, 4
    // requests 22.1 against 25.7), their fixed cost per workgroup (query operand, state
    // write) weighing more than the second slot's overlap.
    const int64_t per_cu = (rows == 1 && d.head_dim == 256 && f32) ? 2 : 1;
    n = ceil_div(per_cu * kTargetWaves / kWavesPerBlock, units);
    const int64_t most = ceil_div(tiles, split);
    if (n > most) n = most;
    if (n < 1) n = 1;
  }
  if (n > (int64_t(1) << 24)) return ATTN_E_OVERFLOW;
  const int64_t piece_tiles = ceil_div(tiles, n * split);
  int64_t chunk_len = piece_tiles * T * split;
  int64_t chunk_len_odd = chunk_len;
  if (d.num_chunks == 0) n = ceil_div(max_span, chunk_len);
  // XCD balance (one row, the plan's own chunking): a launch hands workgroups to the
  // eight XCDs in turn, so with an even number of chunks (the grid's width) chunk c runs
  // on an XCD of c's parity.  On MI355X the odd XCDs stream HBM ~7-10 % slower (per-wave
  // timestamps on several parts, whatever the page placement), so even-numbered chunks
  // take ~5 % more keys and odd-numbered ones as many fewer, and all finish together.
  if (rows == 1 && d.num_chunks == 0) {
    const int64_t skew = piece_tiles / kXcdSkewDiv;
    const int64_t le = (piece_tiles + skew) * T * split, lo = (piece_tiles - skew) * T * split;
    const int64_t pairs = max_span / (le + lo), rest = max_span - pairs * (le + lo);
    const int64_t m = 2 * pairs + (rest > 0) + (rest > le);
    if (skew > 0 && m % 2 == 0) {
      chunk_len = le;
      chunk_len_odd = lo;
      n = m;
    }
  }
  // The kernels address chunk positions in 32 bits: every chunk must end a margin below
  // 2^31 (chunks are whole tiles, so near that size the rounding alone could cross it).
  const int64_t cover = (n / 2) * (chunk_len + chunk_len_odd) + (n % 2) * chunk_len;
  if (max_start + cover > INT32_MAX - kPosMargin) return ATTN_E_OVERFLOW;
  // Launch order of the multi-row kernel: row groups of a chunk 8 workgroups apart.
  const int64_t grid_x = groups > 1 ? ceil_div(n, 8) * 8 * groups : n;

  // Level-1 groups: at most kMergeGroups per (request, head), so the merge's second
  // level fits one workgroup.
  const int64_t gm_min = ceil_div(n, kMergeGroups);
  int64_t gm = d.merge_group == 0 ? gm_min : d.merge_group;
  if (gm < gm_min) return ATTN_E_UNSUPPORTED;
  if (gm > n) gm = n;
  const int64_t ng = ceil_div(n, gm);

  // Grid limits: blocks along x carry chunks (and row groups), y the KV heads, z the requests.
  if (grid_x > INT32_MAX || d.batch > 65535 || d.num_kv_heads > 65535 ||
      d.num_q_heads > 65535)
    return ATTN_E_OVERFLOW;

  attn_decode_plan_t p;
  std::memset(&p, 0, sizeof(p));
  p.magic = kPlanMagic;
  p.desc = d;
  p.group_size = d.num_q_heads / d.num_kv_heads;
  p.tile = int32_t(T);
  p.chunk_len = int32_t(chunk_len);
  p.chunk_len_odd = int32_t(chunk_len_odd);
  p.num_chunks = int32_t(n);
  p.merge_group = int32_t(gm);
  p.num_groups = int32_t(ng);
  p.max_span = int32_t(max_span);
  p.num_rows = int32_t(rows);
  p.row_groups = int32_t(groups);
  p.grid_x = int32_t(grid_x);

  uint64_t brows, bh, states, elems;
  if (!mul_ok(uint64_t(d.batch), uint64_t(rows), &brows) ||
      !mul_ok(brows, uint64_t(d.num_q_heads), &bh) ||
      !mul_ok(bh, uint64_t(n), &states) || !mul_ok(states, uint64_t(d.head_dim), &elems))
    return ATTN_E_OVERFLOW;
  if (bh > 65535) return ATTN_E_OVERFLOW;  // merge grid rows
  uint64_t cur = 0;
  if (!place(&cur, states, &p.off_part_m) || !place(&cur, states, &p.off_part_l) ||
      !place(&cur, elems, &p.off_part_o) || !align_up(cur, &p.workspace_bytes))
    return ATTN_E_OVERFLOW;

  *plan = p;
  return ATTN_OK;
}

// In-row byte offsets of a 32-key tile (rows and columns) fit 31 bits.
bool tile_offsets_fit(const attn_decode_desc& d) {
  const int64_t eb = kv_elem_bytes(d.kv_dtype);
  uint64_t a, b;
  return mul_ok(uint64_t(kPrefillKeys - 1), uint64_t(d.row_stride * eb), &a) &&
         add_ok(a, uint64_t(row_extent(d) * eb), &b) && b <= uint64_t(INT32_MAX);
}

// Element types the 32-key tile kernel stages: bf16 as stored, FP8 E4M3 widened to bf16.
bool tile_dtype(const attn_decode_desc& d) {
  return d.kv_dtype == ATTN_KV_BF16 || d.kv_dtype == ATTN_KV_FP8_E4M3;
}

bool rows_on_tiles(const attn_decode_desc& d, int64_t rows) {
  return rows > 1 && d.head_dim == 512 && tile_dtype(d) && d.page_size % kPrefillKeys == 0 &&
         tile_offsets_fit(d);
}

bool prefill_shape_supported(const attn_decode_desc& d) {
  if (!shape_supported(d)) return false;
  if (d.kv_dtype == ATTN_KV_F32) return true;  // the f32 kernel's 16-key tiles
  return (tile_dtype(d) || d.kv_dtype == ATTN_KV_F16) && d.page_size % kPrefillKeys == 0;
}

int make_prefill_plan(const attn_decode_desc* desc, const int32_t* lens, const int32_t* q_starts,
                      attn_prefill_plan_t* plan) {
  if (!desc || !lens || !q_starts || !plan) return ATTN_E_INVALID_ARG;
  const attn_decode_desc& d = *desc;
  const int rc0 = check_desc(d);
  if (rc0 != ATTN_OK) return rc0;
  if (!prefill_shape_supported(d)) return ATTN_E_UNSUPPORTED;
  const bool f32 = d.kv_dtype == ATTN_KV_F32;
  // A tile's rows are addressed with 32-bit byte offsets from its first row (the 32-key
  // tile kernel; the f32 kernel addresses in 64 bits).
  if (!f32 && !tile_offsets_fit(d)) return ATTN_E_OVERFLOW;

  // Rows of request r are q_starts[r] .. q_starts[r + 1] (0 allowed); they are its last
  // positions, so there are at most L_r of them, and L_r fits the table row.
  if (q_starts[0] != 0) return ATTN_E_INVALID_ARG;
  const int64_t cap = int64_t(d.max_pages_per_seq) * d.page_size;
  int64_t max_rows = 0;
  for (int r = 0; r < d.batch; ++r) {
    const int64_t n = int64_t(q_starts[r + 1]) - q_starts[r];
    const int64_t L = lens[r];
    if (n < 0 || L < n) return ATTN_E_INVALID_ARG;
    if (L > cap) return ATTN_E_PAST_PAGES;
    if (L > INT32_MAX - kPosMargin) return ATTN_E_OVERFLOW;  // 32-bit positions in the kernel
    if (n > max_rows) max_rows = n;
  }
  const int64_t total = q_starts[d.batch];
  // Rows per workgroup: the 32-key tile kernel's 64 (x2 at head dim 256) columns, or the f32
  // kernel's 16 MFMA columns, of (row, head) pairs.
  const int64_t row_tile = f32 ? 16 / (d.num_q_heads / d.num_kv_heads)
                               : (d.head_dim == 256 ? 2 : 1) * kPrefillColumns /
                                     (d.num_q_heads / d.num_kv_heads);
  const int64_t tiles = ceil_div(max_rows, row_tile);
  uint64_t elems;
  if (!mul_ok(uint64_t(total), uint64_t(d.num_q_heads) * uint64_t(d.head_dim), &elems) ||
      elems > (uint64_t(1) << 60))
    return ATTN_E_OVERFLOW;
  // One workgroup per (row tile, KV head, request), launched in whole rounds of 256.
  uint64_t heads, items;
  if (f32 && (d.batch > 65535 || d.num_kv_heads > 65535)) return ATTN_E_OVERFLOW;  // grid y, z
  if (!mul_ok(uint64_t(d.num_kv_heads), uint64_t(d.batch), &heads) ||
      !mul_ok(uint64_t(tiles), heads, &items) || items > uint64_t(INT32_MAX - 255))
    return ATTN_E_OVERFLOW;

  attn_prefill_plan_t p;
  std::memset(&p, 0, sizeof(p));
  p.magic = kPrefillMagic;
  p.desc = d;
  p.group_size = d.num_q_heads / d.num_kv_heads;
  p.key_tile = f32 ? kTile : kPrefillKeys;
  p.row_tile = int32_t(row_tile);
  p.total_rows = int32_t(total);
  p.max_rows = int32_t(max_rows);
  p.grid_x = int32_t(tiles);
  *plan = p;
  return ATTN_OK;
}

int check_prefill_plan(const attn_prefill_plan_t* plan) {
  if (!plan) return ATTN_E_INVALID_ARG;
  if (plan->magic != kPrefillMagic) return ATTN_E_PLAN;
  return ATTN_OK;
}

int check_plan(const attn_decode_plan_t* plan) {
  if (!plan) return ATTN_E_INVALID_ARG;
  if (plan->magic != kPlanMagic) return ATTN_E_PLAN;
  return ATTN_OK;
}

int check_workspace(const attn_decode_plan_t* plan, const void* ws, size_t bytes) {
  if (!ws) return ATTN_E_INVALID_ARG;
  if (bytes < plan->workspace_bytes) return ATTN_E_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return ATTN_E_WORKSPACE;
  return ATTN_OK;
}

}  // namespace attn

extern "C" int attn_decode_plan(const attn_decode_desc* desc, const int32_t* seq_lens_host,
                                attn_decode_plan_t* plan) {
  return attn::make_plan(desc, seq_lens_host, plan);
}

extern "C" int attn_prefill_plan(const attn_decode_desc* desc, const int32_t* seq_lens_host,
                                 const int32_t* q_starts_host, attn_prefill_plan_t* plan) {
  return attn::make_prefill_plan(desc, seq_lens_host, q_starts_host, plan);
}

extern "C" const char* attn_decode_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_E_INVALID_ARG: return "invalid argument";
    case ATTN_E_UNSUPPORTED: return "unsupported shape";
    case ATTN_E_PAST_PAGES: return "length past the pages of a table row";
    case ATTN_E_OVERFLOW: return "size overflow";
    case ATTN_E_WORKSPACE: return "workspace too small or misaligned";
    case ATTN_E_PLAN: return "not a plan made by attn_decode_plan";
    case ATTN_E_LAUNCH: return "kernel launch failed";
    case ATTN_E_SCRATCH: return "plan needs more chunk-state memory than the static scratch holds";
    default: return "unknown status";
  }
}
