// Host-only fuzz of the planning entry points (attn_decode_plan, attn_prefill_plan,
// attn_decode_status_string) for the sanitizer build: seeded random descriptors mixing
// valid, edge and hostile values, random request lengths and prompt offsets.  Every call
// must return without undefined behaviour; a successful decode plan must cover every
// request's keys with its chunks and give a positive workspace.  Exit status 0 on success.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <vector>

#include "../../include/attn_decode.h"

namespace {

uint64_t state = 0x9E3779B97F4A7C15ull;
uint64_t next() {  // xorshift64 (Marsaglia)
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return state;
}
template <class T, size_t N>
T pick(const T (&v)[N]) {
  return v[next() % N];
}

int fail(const char* what, int it) {
  std::fprintf(stderr, "plan_fuzz: %s at iteration %d\n", what, it);
  return 1;
}

}  // namespace

int main() {
  const int32_t I32MAX = std::numeric_limits<int32_t>::max();
  const float NaN = std::numeric_limits<float>::quiet_NaN();
  const float Inf = std::numeric_limits<float>::infinity();
  const int32_t batches[] = {1, 2, 16, 0, -1, 64, 100000};
  const int32_t hqs[] = {32, 32, 16, 8, 0, -32, 31};
  const int32_t hkvs[] = {4, 4, 16, 2, 0, 1, 5};
  const int32_t dims[] = {512, 512, 256, 128, 0, 511};
  const int32_t formats[] = {ATTN_KV_SPLIT, ATTN_KV_SPLIT, ATTN_KV_FOLDED, 2, -1};
  const int32_t pages[] = {256, 256, 64, 16, 32, 0, 15, 1 << 20};
  const int32_t maxp[] = {1, 42, 639, 640, 64, 0, I32MAX, 3};
  const int32_t windows[] = {0, 0, 1024, 700, -1, I32MAX};
  const int32_t chunks[] = {0, 0, 8, 64, 256, -1, 100000, 3};
  const int32_t groups[] = {0, 0, 1, 8, -1, 1000};
  const int32_t rows[] = {0, 1, 1, 4, 8, 64, 65, -1};
  const int32_t dtypes[] = {ATTN_KV_BF16, ATTN_KV_BF16, ATTN_KV_F16, ATTN_KV_FP8_E4M3, ATTN_KV_F32, 4, -1};
  const float scales[] = {0.0441941738f, 1.0f, 0.0f, NaN, Inf, -1.0f};
  const float dq[] = {1.0f, 1.0f, 0.0175f, 0.0f, NaN, -1.0f, Inf};
  const int64_t npages[] = {640, 8, 0, -1, int64_t(1) << 40, std::numeric_limits<int64_t>::max() / 2};
  const int64_t wild[] = {0, -1, 16, int64_t(1) << 40, std::numeric_limits<int64_t>::max()};
  int accepted = 0, refused = 0, p_accepted = 0;
  for (int it = 0; it < 200000; ++it) {
    attn_decode_desc d;
    std::memset(&d, 0, sizeof d);
    // a valid shape: global hd512 (split or folded rows) or sliding hd256, any element type
    const bool sliding = next() % 3 == 0;
    d.batch = sliding ? 16 : int32_t(1 + next() % 4);
    d.num_q_heads = 32;
    d.num_kv_heads = sliding ? 16 : 4;
    d.head_dim = sliding ? 256 : 512;
    d.format = !sliding && next() % 3 == 0 ? ATTN_KV_FOLDED : ATTN_KV_SPLIT;
    d.kv_dtype = int32_t(next() % 4);
    if (d.kv_dtype == ATTN_KV_F32) d.format = ATTN_KV_SPLIT;
    d.rot_cols = d.format == ATTN_KV_FOLDED ? 128 : 0;
    d.page_size = sliding ? 64 : (next() % 4 ? 256 : 16);
    d.max_pages_per_seq = sliding ? 64 : int32_t(1 + next() % 700);
    d.window = sliding ? 1024 : (next() % 5 ? 0 : int32_t(1 + next() % 4096));
    d.num_chunks = next() % 2 ? 0 : int32_t(1 + next() % 300);
    d.merge_group = next() % 2 ? 0 : int32_t(1 + next() % 64);
    d.num_rows = next() % 3 ? 0 : int32_t(1 + next() % 9);
    d.scale = 0.0441941738f;
    d.k_scale = d.kv_dtype == ATTN_KV_FP8_E4M3 ? 0.0175f : 1.0f;
    d.v_scale = d.kv_dtype == ATTN_KV_FP8_E4M3 ? 0.0225f : 1.0f;
    d.num_pages = int64_t(d.batch) * d.max_pages_per_seq + int64_t(next() % 8);
    const int64_t cols = d.format == ATTN_KV_FOLDED ? int64_t(d.rot_cols) + d.head_dim : 2 * int64_t(d.head_dim);
    d.row_stride = cols;
    d.head_stride = cols * d.page_size;
    d.page_stride = d.head_stride * d.num_kv_heads;
    d.k_offset = 0;
    d.v_offset = d.format == ATTN_KV_FOLDED ? d.rot_cols : d.head_dim;
    // then up to two fields replaced by edge or hostile values
    for (int m = int(next() % 4) - 1; m > 0; --m) {
      switch (next() % 20) {
        case 0: d.batch = pick(batches); break;
        case 1: d.num_q_heads = pick(hqs); break;
        case 2: d.num_kv_heads = pick(hkvs); break;
        case 3: d.head_dim = pick(dims); break;
        case 4: d.format = pick(formats); break;
        case 5: d.rot_cols = pick(windows); break;
        case 6: d.page_size = pick(pages); break;
        case 7: d.max_pages_per_seq = pick(maxp); break;
        case 8: d.window = pick(windows); break;
        case 9: d.num_chunks = pick(chunks); break;
        case 10: d.merge_group = pick(groups); break;
        case 11: d.num_rows = pick(rows); break;
        case 12: d.kv_dtype = pick(dtypes); break;
        case 13: d.scale = pick(scales); break;
        case 14: d.k_scale = pick(dq); break;
        case 15: d.v_scale = pick(dq); break;
        case 16: d.num_pages = pick(npages); break;
        case 17: d.row_stride = pick(wild); break;
        case 18: d.page_stride = pick(wild); break;
        default: d.v_offset = pick(wild); break;
      }
    }
    const int32_t nb = d.batch > 0 ? d.batch : 1;
    const int64_t cap = int64_t(d.max_pages_per_seq) * d.page_size;
    std::vector<int32_t> lens(nb);
    const int64_t lpick[] = {1, 16, 1024, 10602, 163336, 0, -5, I32MAX, cap, cap + 1, cap - 1};
    for (auto& L : lens) {
      // mostly valid lengths up to the table's capacity, sometimes an edge value
      const int64_t v = next() % 8 && cap > 0 ? int64_t(1 + next() % uint64_t(cap)) : pick(lpick);
      L = int32_t(v > I32MAX ? I32MAX : v < -I32MAX ? -I32MAX : v);
    }
    attn_decode_plan_t plan;
    const int rc = attn_decode_plan(&d, next() % 50 ? lens.data() : nullptr, &plan);
    if (rc == ATTN_OK) {
      ++accepted;
      if (plan.num_chunks < 1 || plan.chunk_len < 1 || plan.workspace_bytes <= 0) {
        std::fprintf(stderr, "batch %d hq %d hkv %d D %d fmt %d rot %d page %d maxp %d win %d chunks %d group %d rows %d dt %d\n",
                     d.batch, d.num_q_heads, d.num_kv_heads, d.head_dim, d.format, d.rot_cols, d.page_size,
                     d.max_pages_per_seq, d.window, d.num_chunks, d.merge_group, d.num_rows, d.kv_dtype);
        for (int32_t L : lens) std::fprintf(stderr, "  L %d\n", L);
        std::fprintf(stderr, "plan chunks %d len %d odd %d tile %d ws %lld\n", plan.num_chunks, plan.chunk_len,
                     plan.chunk_len_odd, plan.tile, (long long)plan.workspace_bytes);
        return fail("accepted plan without chunks or workspace", it);
      }
      if (plan.tile != 16 && plan.tile != 32) return fail("tile neither 16 nor 32", it);
      const int64_t pair = int64_t(plan.chunk_len) + plan.chunk_len_odd;
      const int64_t cover = int64_t(plan.num_chunks / 2) * pair + (plan.num_chunks % 2) * int64_t(plan.chunk_len);
      for (int32_t L : lens) {
        const int64_t rows = plan.num_rows > 1 ? plan.num_rows : 1;
        const int64_t first_hi = int64_t(L) - rows + 1;
        const int64_t lo = d.window > 0 && first_hi > d.window ? first_hi - d.window : 0;
        const int64_t start = lo / plan.tile * plan.tile;
        if (L - start > cover) return fail("chunks do not cover a request", it);
        if (start + cover > int64_t(I32MAX) - 1024) return fail("chunk positions near 2^31", it);
      }
    } else {
      ++refused;
      if (!attn_decode_status_string(rc)) return fail("no text for a status", it);
    }
    // prefill plan over the same descriptor: prompt rows 0 .. L per request
    std::vector<int32_t> starts(nb + 1, 0);
    for (int32_t r = 0; r < nb; ++r) {
      const int32_t L = lens[r];
      const int32_t n = L > 0 ? int32_t(next() % (uint64_t(L) + 1)) : int32_t(next() % 3);
      const int64_t s = int64_t(starts[r]) + (next() % 40 ? n : -n);
      starts[r + 1] = int32_t(s > I32MAX ? I32MAX : s < -I32MAX ? -I32MAX : s);
    }
    attn_prefill_plan_t pp;
    const int prc = attn_prefill_plan(&d, lens.data(), next() % 50 ? starts.data() : nullptr, &pp);
    if (prc == ATTN_OK) {
      ++p_accepted;
      for (int32_t L : lens)
        if (int64_t(L) > int64_t(I32MAX) - 1024) return fail("prefill length near 2^31", it);
      const int32_t key_tile = d.kv_dtype == ATTN_KV_F32 ? 16 : 32;
      if (pp.grid_x < 0 || pp.row_tile < 1 || pp.key_tile != key_tile)
        return fail("prefill plan fields", it);
    }
  }
  for (int s = -10; s <= 2; ++s)
    if (!attn_decode_status_string(s)) return fail("status text", s);
  std::printf("plan_fuzz: %d decode plans accepted, %d refused, %d prefill plans accepted\n",
              accepted, refused, p_accepted);
  return 0;
}
