/*
 * attn_decode.h -- C ABI of the paged split-KV decode-attention library (gfx950).
 *
 * One decode step of one attention layer: every query head of every request
 * attends, with an exact softmax, over its KV head's keys stored in a paged pool.
 * The keys are cut into chunks; each chunk yields an online-softmax partial
 * (running max M, sum S, unnormalised numerator O) and the partials are merged
 * with the exact rescaling identity in two levels (pegainfer PR #1055,
 * "Description": a split-KV decode kernel with a partial over key chunks and a
 * merge in two levels; gem "Parked D512 fused split-KV decode design", section
 * "Candidate ownership and storage": M = max(Ma, Mb), S = Sa e^(Ma-M) + Sb e^(Mb-M),
 * the numerator likewise, then O / S).
 *
 * Three calls make a step:
 *   attn_decode_plan   host only: validates the shape and the request lengths,
 *                      chooses the chunking and lays out the workspace.
 *   attn_decode_split  enqueues the partial kernel on a HIP stream.
 *   attn_decode_merge  enqueues the merge (level 1, level 2, O / S) on a stream.
 *   attn_decode_split_tree  the split step for a window of rows forming a tree.
 * Around the step: attn_kv_write stores new tokens' K/V rows into the pages,
 * attn_query_fold folds K's norm weight into the query for a folded pool, and
 * attn_prefill_plan / attn_prefill run a request's prompt rows (causal, several rows
 * per request) over the same pool and descriptor.
 *
 * Ownership: the caller owns every buffer (query, pool, page table, lengths,
 * workspace, output).  Buffers of floats or pool rows (q, kv_pool, out, the K/V rows of
 * attn_kv_write, attn_query_fold's q, norm_w and q_out) must be 16-byte aligned (the
 * kernels move them in 16-byte vectors); the workspace 256-byte aligned; int32 and uint64
 * arrays (page table, lengths, offsets, masks) to their element size.  The library allocates nothing, keeps no mutable global
 * state and is reentrant (attn_decode_step_noalloc aside: it uses a static per-GPU array
 * and remembers that array's address per device).  Launches are asynchronous; buffers must stay alive
 * until the stream has run them.  A plan is plain old data and may be copied.
 * The enqueuing calls neither synchronise nor allocate nor record memsets, and a
 * plan fixes their grids, so they can be captured into a HIP graph and replayed.
 *
 * Errors: every check runs before any launch, so a refused call enqueues
 * nothing.  Kernels write only the plan's workspace extent and `out`.
 */
#ifndef ATTN_DECODE_H
#define ATTN_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every call. */
enum {
  ATTN_OK = 0,
  ATTN_E_INVALID_ARG = -1,  /* null pointer, non-positive size, inconsistent layout */
  ATTN_E_UNSUPPORTED = -2,  /* shape with no kernel: see attn_decode_desc */
  ATTN_E_PAST_PAGES = -3,   /* a length needs more pages than a table row holds */
  ATTN_E_OVERFLOW = -4,     /* a size computation would overflow 64 bits / grid limits */
  ATTN_E_WORKSPACE = -5,    /* workspace smaller than the plan needs, or misaligned */
  ATTN_E_PLAN = -6,         /* plan not produced by attn_decode_plan (bad magic) */
  ATTN_E_LAUNCH = -7,       /* the HIP runtime refused a launch */
  ATTN_E_SCRATCH = -8       /* attn_decode_step_noalloc: the plan needs more chunk-state
                               memory than its static array holds */
};

/* Row formats of the pool, fixed for the pool's life (pegainfer PR #1055,
 * "Description": the page format is an axis of the layout). */
enum {
  ATTN_KV_SPLIT = 0,   /* row = K[0:D] at k_offset, V[0:D] at v_offset (1024 cols at D=512) */
  ATTN_KV_FOLDED = 1   /* row = rotated K[0:rot] at k_offset, V[0:D] at v_offset; the
                          unrotated part of the score is q'[rot:D] . V[rot:D], with K's norm
                          weight already folded into q' by the caller (640 cols at D=512) */
};

/* Element types of the pool (kv_dtype).  BF16 is the pages' row type; F32 is the
 * production KV type of the gem design note ("Fixed production shape"), where F16
 * and quantised KV are named as further axes.  The quantised type taken here is
 * FP8 E4M3 as the OCP 8-bit floating point specification defines it (bias 7,
 * subnormals, no infinity, S.1111.111 = NaN), the FP8 encoding gfx950 converts
 * natively.  Every type is widened exactly to the MFMA operand type (bf16 for BF16
 * and FP8, f16 for F16); F32 rows are multiplied in full fp32. */
enum {
  ATTN_KV_BF16 = 0,
  ATTN_KV_F16 = 1,
  ATTN_KV_FP8_E4M3 = 2,
  ATTN_KV_F32 = 3
};

/*
 * Shape and layout of one layer's paged pool and decode batch.
 *
 * Supported shapes (others give ATTN_E_UNSUPPORTED):
 *   head_dim 512, 8 query heads per KV head, SPLIT, or FOLDED with rot_cols 128
 *   head_dim 256, 2 query heads per KV head, SPLIT (sliding layers, any window)
 * Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * Element (page p, KV head g, slot s, column c) of the pool is the kv_dtype
 * element at
 *   pool[p * page_stride + g * head_stride + s * row_stride + c]
 * All strides and offsets count elements of kv_dtype and must be multiples of 16
 * bytes (8 BF16/F16 elements, 16 FP8 elements); every row of a page must lie
 * inside its page_stride.
 * The keys and values used are the stored values times k_scale and v_scale
 * (dequantisation factors, one per tensor; 1 for an unscaled pool).  In a FOLDED
 * row the unrotated part of the key is made of V columns, so it takes v_scale.
 * Logical key position j of request r lives in slot j % page_size of page
 * page_table[r * max_pages_per_seq + j / page_size] (TensorFold PR #1619, body).
 *
 * window > 0 makes a request of length L attend to positions [L - window, L)
 * only; older keys in resident pages are masked (pegainfer PR #1057,
 * "Description").  Page-table entries wholly before that range are never read.
 */
typedef struct attn_decode_desc {
  int32_t batch;              /* requests, one query token each */
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;           /* D: 512 or 256 */
  int32_t format;             /* ATTN_KV_SPLIT or ATTN_KV_FOLDED */
  int32_t rot_cols;           /* FOLDED: stored rotated K columns (128); SPLIT: 0 */
  int32_t page_size;          /* positions per page, a multiple of 16 */
  int32_t max_pages_per_seq;  /* length of one page-table row */
  int32_t window;             /* 0 = whole context */
  int32_t num_chunks;         /* key chunks per (request, KV head); 0 = choose automatically */
  int32_t merge_group;        /* chunk partials per level-1 group; 0 = choose automatically,
                                 else at least ceil(chunks / 8) (at most 8 groups) */
  int32_t num_rows;           /* query rows per request, 0 or 1 = ordinary decode; n > 1 is a
                                 window: row i is the token at position L - n + i and attends
                                 causally to the keys before L - n + i + 1 (drafted verify
                                 windows through the paged decode, TensorFold PR #1619, review
                                 thread); q and out are then [batch][n][num_q_heads][head_dim] */
  int32_t kv_dtype;           /* ATTN_KV_BF16, ATTN_KV_F16, ATTN_KV_FP8_E4M3 or ATTN_KV_F32 */
  float scale;                /* score = scale * q . k (1/sqrt(D) in the workloads) */
  float k_scale;              /* K = stored * k_scale; finite and > 0 */
  float v_scale;              /* V = stored * v_scale; finite and > 0 */
  int64_t num_pages;          /* pages in the pool; table entries outside [0, num_pages) poison */
  int64_t page_stride;        /* elements between pages */
  int64_t head_stride;        /* elements between KV heads inside a page */
  int64_t row_stride;         /* elements between consecutive slots */
  int64_t k_offset;           /* column of K[0] (split) or of the rotated K[0] (folded) */
  int64_t v_offset;           /* column of V[0] */
} attn_decode_desc;

/*
 * A validated plan (host-only POD).  Chunk c of request r covers the chunk_len (c even)
 * or chunk_len_odd (c odd) key positions from
 *   start_r + (c / 2) * (chunk_len + chunk_len_odd) + (c % 2) * chunk_len
 * intersected with the keys a query row sees, where
 * lo_r = max(0, L_r - rows + 1 - window) (0 without a window) is the oldest key any row
 * of the request sees and start_r = lo_r rounded down to a multiple of `tile`.  A chunk with no visible key yields the empty partial (-inf, 0, 0).
 *
 * Workspace layout (byte offsets from the workspace base, each region 256-byte
 * aligned, all float32, partition-major and contiguous in the output dimension;
 * gem design note, "Candidate ownership and storage"):
 * (with several query rows, B counts requests x rows: row i of request r is r*rows + i)
 *   part_m [B][Hq][num_chunks]        reference maxima, natural-log units: at most the
 *                                     chunk's largest score and at least that minus 8 ln 2
 *                                     (-inf for an empty chunk); part_l and part_o are
 *                                     taken relative to it, as the merge identity allows
 *   part_l [B][Hq][num_chunks]        denominators S
 *   part_o [B][Hq][num_chunks][D]     numerators O (unnormalised)
 * The merge's level-1 group states live in on-chip memory and need no workspace.
 */
typedef struct attn_decode_plan_t {
  uint64_t magic;
  attn_decode_desc desc;
  int32_t group_size;    /* query heads per KV head */
  int32_t tile;          /* keys per tile (16; 32 for several query rows at head dim 512
                            over bf16 or FP8 pages); chunk starts are multiples of it */
  int32_t chunk_len;     /* keys per even-numbered chunk: a multiple of 4 * tile for one
                            query row (one quarter per wave), of tile for several */
  int32_t chunk_len_odd; /* keys per odd-numbered chunk (the same multiple); equal to
                            chunk_len except for one query row with an automatic chunk
                            count, where even chunks run on the faster XCDs */
  int32_t num_chunks;    /* chunks per (request, KV head) */
  int32_t merge_group;   /* chunk partials folded per level-1 group */
  int32_t num_groups;    /* level-1 states per (request, query head), at most 8 */
  int32_t max_span;      /* max over requests of L_r - start_r */
  int32_t num_rows;      /* query rows per request (>= 1) */
  int32_t row_groups;    /* groups of up to 4 rows, one workgroup each (multi-row) */
  int32_t grid_x;        /* workgroups along the chunk axis of the partial launch */
  uint64_t off_part_m, off_part_l, off_part_o;
  uint64_t workspace_bytes; /* bytes attn_decode_split / attn_decode_merge need */
} attn_decode_plan_t;

/*
 * Validate `desc` and the host copy of the request lengths seq_lens_host[batch]
 * and fill `plan`.  No device call is made.
 * Refusals: null pointers or non-positive sizes (ATTN_E_INVALID_ARG); a shape
 * outside the supported list, or an element type without a kernel
 * (ATTN_E_UNSUPPORTED); an unknown element type, a dequantisation factor that is
 * not finite and positive, a stride or offset not a multiple of 16 bytes, or
 * rows overrunning their page (ATTN_E_INVALID_ARG); a length
 * below 1 or below num_rows, or num_rows above 64 (ATTN_E_INVALID_ARG); a length
 * above max_pages_per_seq * page_size
 * (ATTN_E_PAST_PAGES, TensorFold PR #1619, body: rows past a slot's pages are
 * refused); a merge_group below ceil(chunks / 8) (ATTN_E_UNSUPPORTED); any size
 * product that overflows, a grid beyond the launch limits, or chunks that would end
 * within 1024 positions of 2^31 (the kernels' key positions are 32-bit) (ATTN_E_OVERFLOW;
 * gem design note, "Candidate ownership and storage": all scratch products are
 * overflow-checked).
 */
int attn_decode_plan(const attn_decode_desc* desc, const int32_t* seq_lens_host,
                     attn_decode_plan_t* plan);

/*
 * Enqueue the partial kernel: one online-softmax state per (request, query
 * head, chunk) into the workspace's part_* regions.
 *   q          device, float32 [batch][num_q_heads][head_dim] (FOLDED: the folded q'),
 *              [batch][num_rows][num_q_heads][head_dim] with several query rows
 *   kv_pool    device, pool of kv_dtype elements laid out as described for
 *              attn_decode_desc
 *   page_table device, int32 [batch][max_pages_per_seq]
 *   seq_lens   device, int32 [batch]; must equal the lengths given to the plan.  A
 *              device length or page id the plan cannot serve is not read past:
 *              the affected request's partials become NaN.
 *   workspace  device, >= plan->workspace_bytes, 256-byte aligned
 *   stream     hipStream_t (NULL = the default stream)
 * Returns ATTN_E_PLAN on a bad plan, ATTN_E_WORKSPACE on a short or misaligned
 * workspace, ATTN_E_INVALID_ARG on null pointers, ATTN_E_LAUNCH if HIP refuses.
 */
int attn_decode_split(const attn_decode_plan_t* plan, const float* q, const void* kv_pool,
                      const int32_t* page_table, const int32_t* seq_lens, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * attn_decode_split for a window of several query rows whose rows form a tree
 * (speculative decoding's tree attention; TensorFold PR #1619, body and review thread,
 * names paged tree-attention decode kernels for its drafted verify windows, without
 * fixing a mask).  Row i of request r sees the keys before the window, L_r - num_rows,
 * that a causal row i sees, and of the window's own keys the key of row j exactly when
 * bit j of row_masks[r * num_rows + i] is set (a tree: row i and its ancestors; causal
 * rows are the masks 2^(i+1) - 1, which give attn_decode_split's result).  A window
 * lower bound applies to every key as for the causal row.  Bits at or past num_rows are
 * ignored; a row that sees no key gets NaN from the merge (0 / 0).
 *   row_masks  device, uint64 [batch][num_rows]
 * Other arguments and returns as attn_decode_split; ATTN_E_INVALID_ARG also for a null
 * row_masks or a plan of one query row.
 */
int attn_decode_split_tree(const attn_decode_plan_t* plan, const float* q, const void* kv_pool,
                           const int32_t* page_table, const int32_t* seq_lens,
                           const uint64_t* row_masks, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Enqueue the two-level merge as one kernel: level 1 folds each run of
 * merge_group consecutive chunk states into a group state (out of place: the
 * chunk states are only read); level 2 folds the group states in ascending
 * order and writes O / S.
 *   out   device, float32 [batch][num_q_heads][head_dim] ([batch][num_rows][...] with
 *         several query rows); nothing else is written.
 * Same error behaviour as attn_decode_split.
 */
int attn_decode_merge(const attn_decode_plan_t* plan, void* workspace, size_t workspace_bytes,
                      float* out, void* stream);

/*
 * Write new tokens' K/V rows into the pool: the step that feeds decode.  Each
 * forward's k/v rows are copied into the pages through the table (TensorFold PR
 * #1619, body), in the pool's row format (pegainfer PR #1055, "Description": the
 * hd512 prep writes either form).  Values arrive as float32; each is divided by its
 * tensor's factor (k_scale or v_scale: one float32 division rounded to nearest, skipped
 * when the factor is 1) and stored as the pool's element type:
 *   BF16, F16  rounded to nearest with ties to even (F16: overflow gives infinity)
 *   F32        as is
 *   FP8_E4M3   the nearest E4M3 value with ties to the even mantissa; magnitudes from 448
 *              up (infinity included) saturate to 448, NaN gives S.1111.111, and a value
 *              that rounds to zero keeps its sign (the decode path reads stored * factor;
 *              the pages name quantised KV as an axis without fixing the encoding, gem
 *              design note, "Fixed production shape").
 *   k          device float32 [batch][num_new][num_kv_heads][kc]; kc = head_dim for
 *              SPLIT (row columns k_offset..), rot_cols for FOLDED (the rotated part)
 *   v          device float32 [batch][num_new][num_kv_heads][head_dim] (columns v_offset..)
 *   start_pos  device int32 [batch]: logical position of each request's first new token;
 *              token i goes to position start_pos[r] + i (a decode step appends at L - 1)
 *   kv_pool    device pool of kv_dtype elements, written in place
 *   page_table device int32 [batch][max_pages_per_seq]
 *   bad_rows   device int32, may be NULL: set to 1 if any row was skipped because its
 *              position is past the table row or its page id is outside the pool (such
 *              rows are never written); the caller clears it beforehand
 * Only the addressed row columns are written.  Uses the plan's layout (its lengths are
 * not consulted).  ATTN_E_INVALID_ARG on null pointers or num_new < 1.
 */
int attn_kv_write(const attn_decode_plan_t* plan, const float* k, const float* v, int32_t num_new,
                  const int32_t* start_pos, void* kv_pool, const int32_t* page_table,
                  int32_t* bad_rows, void* stream);

/*
 * Fold K's norm weight into the query for a FOLDED pool (pegainfer PR #1055,
 * "Description"): q_out[r][h][d] = q[r][h][d] for d < rot_cols, else the float32
 * product q[r][h][d] * norm_w[d - rot_cols].  q and q_out are device float32
 * [batch][num_q_heads][head_dim] (may alias); norm_w is device float32
 * [head_dim - rot_cols].  ATTN_E_UNSUPPORTED for a SPLIT plan.
 */
int attn_query_fold(const attn_decode_plan_t* plan, const float* q, const float* norm_w,
                    float* q_out, void* stream);

/*
 * Paged prefill: the prompt rows of a batch of requests, each row attending causally to
 * its request's keys through the page table.  pegainfer PR #1055 ("Description") serves
 * the global family's prompt rows through a generated prefill over the split or folded
 * pool beside the split-KV decode; pegainfer PR #1057 ("Description") serves the sliding
 * family's prompt rows through a varlen kernel with a window lower bound over pages of
 * 64, and its "Verification" gates that kernel on crossing the window, ragged prompts, a
 * continuation and a tiny prompt; TensorFold PR #1619 ("body") reads prompt rows through
 * the slot's page-table row.
 *
 * Request r has q_starts[r + 1] - q_starts[r] = n_r new rows (0 allowed), packed in q
 * and out at rows q_starts[r] .. q_starts[r + 1] - 1, and L_r = seq_lens[r] keys in all
 * (its new rows' keys already written to the pool).  Its row i sits at position
 * p = L_r - n_r + i and attends to the keys at positions lo .. p, lo = 0 without a
 * window and max(0, p + 1 - window) with one: each row is a decode token at length
 * p + 1 (n_r < L_r is a continuation after L_r - n_r earlier keys).
 * The descriptor is the decode descriptor (num_chunks, merge_group and num_rows are not
 * used).  Supported: the decode shapes; bf16, f16 and FP8 E4M3 pools with page_size a
 * multiple of 32 (FP8 codes are widened to bf16 on their way on chip, f16 rows are
 * multiplied on the f16 MFMA, and the dequantisation factors are applied as in decode), and
 * f32 pools (full fp32 products on the f32 decode kernel, 16 / G rows per workgroup, each
 * wave a quarter of the keys).
 * The output is written directly (no workspace, no merge): one workgroup owns
 * row_tile consecutive rows of one (request, KV head) and walks their keys in
 * key_tile-key tiles, staged once in on-chip memory for all its rows and heads.
 */
typedef struct attn_prefill_plan_t {
  uint64_t magic;
  attn_decode_desc desc;
  int32_t group_size;  /* query heads per KV head */
  int32_t key_tile;    /* keys per tile (32; 16 for f32 pools) */
  int32_t row_tile;    /* query rows per workgroup (8 at head dim 512 / GQA 8, 64 at head dim 256 / GQA 2;
                          f32 pools: 2 and 8) */
  int32_t total_rows;  /* q_starts[batch] */
  int32_t max_rows;    /* largest n_r */
  int32_t grid_x;      /* row tiles per (request, KV head): ceil(max_rows / row_tile) */
} attn_prefill_plan_t;

/*
 * Validate `desc`, the host lengths seq_lens_host[batch] and the host row offsets
 * q_starts_host[batch + 1], and fill `plan`.  No device call is made.
 * Refusals as attn_decode_plan for the descriptor (ATTN_E_INVALID_ARG,
 * ATTN_E_UNSUPPORTED, ATTN_E_OVERFLOW); a page size not a multiple of 32 for a 16-bit or
 * FP8 pool (ATTN_E_UNSUPPORTED); q_starts[0] != 0, decreasing offsets, or
 * more rows than keys in a request (ATTN_E_INVALID_ARG); a length above
 * max_pages_per_seq * page_size (ATTN_E_PAST_PAGES); a length within 1024 of 2^31, or
 * more work items than one launch takes (ATTN_E_OVERFLOW).
 */
int attn_prefill_plan(const attn_decode_desc* desc, const int32_t* seq_lens_host,
                      const int32_t* q_starts_host, attn_prefill_plan_t* plan);

/*
 * Enqueue the prefill kernel.
 *   q          device, float32 [total_rows][num_q_heads][head_dim] (FOLDED: folded q')
 *   kv_pool    device, bf16 or FP8 E4M3 pool laid out as described for attn_decode_desc
 *   page_table device, int32 [batch][max_pages_per_seq]
 *   seq_lens   device, int32 [batch]; q_starts device, int32 [batch + 1]; both must equal
 *              what the plan was given.  A request whose device offsets the plan cannot
 *              serve is skipped (nothing written); one whose device length or page ids the
 *              plan cannot serve gets NaN rows.  Nothing is read past the pool or the rows.
 *   out        device, float32 [total_rows][num_q_heads][head_dim]; only rows of requests
 *              are written.
 * Returns ATTN_E_PLAN on a bad plan, ATTN_E_INVALID_ARG on null pointers,
 * ATTN_E_LAUNCH if HIP refuses.
 */
int attn_prefill(const attn_prefill_plan_t* plan, const float* q, const void* kv_pool,
                 const int32_t* page_table, const int32_t* seq_lens, const int32_t* q_starts,
                 float* out, void* stream);

/*
 * Allocation-free decode step, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).  It enqueues
 * exactly attn_decode_split (attn_decode_split_tree when row_masks is not NULL) followed
 * by attn_decode_merge, but the chunk states live in a static device array of
 * ATTN_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs on until the
 * process ends, instead of a caller's workspace.  Nothing is allocated: no hipMalloc, no
 * hipFree, no allocating library routine.  The first call on a device, with that device
 * current, looks up the array's device address (hipGetSymbolAddress) and keeps it.
 *   q, kv_pool, page_table, seq_lens, row_masks  as attn_decode_split / _split_tree
 *   out     device, float32 as attn_decode_merge
 *   stream  hipStream_t of the current device (NULL = its default stream)
 * Every call on one GPU shares that GPU's array and leaves the last call's states in it:
 * calls that overlap on one GPU (other streams, other threads) race and must be ordered by
 * the caller.  Returns ATTN_E_SCRATCH if plan->workspace_bytes exceeds
 * ATTN_NOALLOC_SCRATCH_BYTES (e.g. 163,336 tokens with one query row needs 4.2 MB, four
 * query rows 16.8 MB), ATTN_E_LAUNCH if the array's address cannot be obtained or HIP
 * refuses a launch, else the errors of attn_decode_split and attn_decode_merge.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
int attn_decode_step_noalloc(const attn_decode_plan_t* plan, const float* q, const void* kv_pool,
                             const int32_t* page_table, const int32_t* seq_lens,
                             const uint64_t* row_masks, float* out, void* stream);

/* Static, NUL-terminated text for a status code. */
const char* attn_decode_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_DECODE_H */
