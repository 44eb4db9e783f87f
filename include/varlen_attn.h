/*
 * varlen_attn.h -- C ABI of the MI355X (gfx950) varlen paged attention library.
 *
 * One call computes one attention layer of one serving iteration in which requests at
 * different stages share a flat Q tensor: uncached prefills, chunked-prefill chunks,
 * and decode steps.
 *
 *   Request r contributes q_rows = q_end[r] - q_start[r] new query rows (rows
 *   q_start[r] .. q_end[r]-1 of the flat Q tensor) and has kv_len[r] positions of
 *   context after this iteration's K/V were appended ("ORCA 和 chunked prefill",
 *   section 2: the (q_start, q_end, kv_length) triple).  With S0 = kv_len - q_rows,
 *   new row i (0-based within the request) reads the S0 cached positions and the new
 *   positions up to and including its own, i.e. positions 0 .. S0+i
 *   ("How To Scale Your Model 笔记(7-8)", section 2: the mask is zero on the first S0
 *   columns and hides only the strict upper triangle of the last q_rows columns).
 *
 *   out[t, h, :] = softmax_j( scale * <q[t, h, :], K_r[j, kvh, :]> ) . V_r[j, kvh, :]
 *   over the visible j, with kvh = h / g, g = num_q_heads / num_kv_heads (grouped-query
 *   attention: "How To Scale Your Model 笔记(7-8)", section 3, KV 容量与 GQA) and
 *   scale = 1/sqrt(head_dim) by default ("一次 forward 怎么塞下很多个 request",
 *   section 6: softmax(Q K^T / sqrt(d_head)) V, computed request by request).
 *
 *   K_r / V_r are reached through request r's block table: logical position j lives in
 *   physical page block_table[r][j / page_size], slot j % page_size ("How To Scale Your
 *   Model 笔记(7-8)", section 3, paging).
 *
 * Memory layouts (all row-major, element type given by va_params.dtype):
 *   q, out   [total_q_rows][num_q_heads][head_dim]
 *   k_pool   [num_pages][num_kv_heads][page_size][head_dim]
 *   v_pool   [num_pages][num_kv_heads][head_dim][page_size]   (V pages are transposed)
 *            Unlike K, a V page holds head_dim rows of page_size consecutive positions, so
 *            the P.V operand (8 consecutive keys of one d) is one 16-byte load.  V kept in
 *            K's layout must be transposed page by page before run(); the append entry
 *            points below write this layout directly.
 *   k_scale, v_scale  float32 [num_pages][num_kv_heads][page_size]   (fp8 pools only)
 *   block table  int32 [num_reqs][max_pages_per_req]; only the first
 *                ceil(kv_len[r] / page_size) entries of row r are read.
 *
 * Ownership: the caller owns every buffer passed in (device memory allocated by e.g.
 * PyTorch).  A plan owns its host metadata and one device buffer of work lists,
 * freed by varlen_attn_plan_destroy().  The library never frees or keeps caller memory.
 *
 * Errors: every entry point returns a va_status and never aborts; on failure
 * varlen_attn_last_error() returns a message describing the first problem found (per
 * calling thread).  varlen_attn_plan() validates all metadata on the host;
 * varlen_attn_run() checks pointers and the workspace size only and assumes the
 * device block table holds the same ids as the host one given to the plan.
 *
 * Streams: run() and debug_gather() only enqueue work on the given stream (NULL = the
 * null stream); they do not synchronise, allocate or copy from the host, so they can be
 * captured into a HIP graph.  A plan is immutable and can be reused by every layer of an
 * iteration and by concurrent runs on different streams (each with its own workspace).
 */
#ifndef VARLEN_ATTN_H
#define VARLEN_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VA_OK = 0,
  VA_ERR_INVALID_ARG = -1,          /* bad metadata, null pointer, bad sizes */
  VA_ERR_UNSUPPORTED = -2,          /* valid but not built for (head_dim, page_size, dtype) */
  VA_ERR_OUT_OF_MEMORY = -3,        /* host or device allocation of the plan failed */
  VA_ERR_HIP = -4,                  /* a HIP runtime call failed (message has hipGetErrorString) */
  VA_ERR_WORKSPACE_TOO_SMALL = -5   /* workspace_bytes below what the plan reported */
} va_status;

/* VA_DTYPE_FP8_E4M3: q and out are bf16; k_pool and v_pool hold OCP fp8 e4m3fn codes
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; S.1111.111 is NaN) in the
 * layouts above, and every position of every KV head has one float32 scale for its K row
 * and one for its V row: element d of that position is decode(code) * scale ("How To
 * Scale Your Model 笔记(7-8)", section 4: a storage format widened on chip, the arithmetic
 * in the wider format; "GLM-5.3 推理全链路(八)", on the costs outside the 656-byte
 * ledger: FP32 scales stored with each token's FP8 data, both read to dequantise).
 * Such plans run with varlen_attn_run_fp8 (codes are widened exactly to bf16 on chip and
 * the scales applied in fp32 to scores (K) and probabilities (V));
 * new rows are stored with varlen_attn_append_kv_fp8. */
typedef enum { VA_DTYPE_BF16 = 0, VA_DTYPE_F32 = 1, VA_DTYPE_FP8_E4M3 = 2 } va_dtype;

enum {
  /* Find requests whose block tables start with the same physical pages and read those
   * pages once per group for all the group's rows ("How To Scale Your Model 笔记(7-8)",
   * section 3: load one common KV block, let several requests' queries use it, each
   * request keeping its own running max and sum). */
  VA_FLAG_SHARED_PREFIX = 1u << 0,
  /* Route every row through the split-KV kernel (no MFMA prefill tiles). */
  VA_FLAG_NO_PREFILL_KERNEL = 1u << 1,
  /* Build the plan on the host only: no device buffer, run() refuses it.  Used to test
   * planning without a GPU. */
  VA_FLAG_HOST_ONLY = 1u << 2,
  /* Keep requests with few new rows (decodes, speculative-decode verify rows) on split-KV
   * items.  Without it, a bf16 plan runs them as MFMA prefill tiles (one per KV head, all
   * of the request's keys) when those tiles, with the prefill tiles, fill the GPU. */
  VA_FLAG_NO_DECODE_TILES = 1u << 3
};

typedef struct {
  int32_t num_q_heads;        /* Hq >= 1 */
  int32_t num_kv_heads;       /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;           /* 64 or 128 */
  int32_t page_size;          /* 16, 32, 64, 128 or 256 positions per page */
  int32_t num_pages;          /* pages in each pool */
  int32_t max_pages_per_req;  /* row stride of the block table */
  int32_t dtype;              /* va_dtype of q, k_pool, v_pool, out; accumulation is fp32 */
  float softmax_scale;        /* <= 0: 1/sqrt(head_dim) */
  uint32_t flags;             /* VA_FLAG_* */
  int32_t prefill_min_rows;   /* q_rows from which a request uses prefill tiles;
                                 <= 0: when q_rows * (Hq / Hkv) >= 64 */
  int32_t split_len;          /* kv positions per split-KV item; <= 0: chosen by the planner */
  int32_t prefill_split_len;  /* key chunk of a cut prefill tile (rounded up to 64): a tile whose
                                 keys visible to all its columns span more than one chunk is
                                 cut into one tile per chunk, their partial results merged by
                                 the combine pass; 0: the planner cuts tiles only when a few
                                 long tiles would leave most of the GPU idle; < 0: never */
} va_params;

typedef struct {
  int64_t num_reqs;
  int64_t total_q_rows;       /* max(q_end): rows q and out must hold */
  int64_t prefill_tiles;      /* MFMA tiles: prefill rows, decode rows run as tiles, key chunks */
  int64_t split_items;        /* split-KV work items (one wavefront each) */
  int64_t shared_items;       /* of which read a shared prefix for several requests */
  int64_t shared_groups;      /* groups of requests found sharing leading pages */
  int64_t partial_slots;      /* (m, 1/l, acc/l [head_dim]) partials in the workspace */
  int64_t combine_rows;       /* (row, head) outputs merged by the combine pass */
  int64_t visible_pairs;      /* sum over requests of m*S0 + m(m+1)/2 */
  double flops;               /* 4 * head_dim * num_q_heads * visible_pairs */
  int64_t logical_kv_bytes;   /* sum kv_len * Hkv * head_dim * 2 (K and V) * elem;
                                 fp8: sum kv_len * Hkv * 2 * (head_dim + 4) (codes + scales) */
  int64_t physical_kv_bytes;  /* distinct (page, slot) positions read, same units */
  int64_t q_bytes;            /* query rows read */
  int64_t o_bytes;            /* output rows written */
  int64_t table_bytes;        /* block-table entries read */
  int64_t workspace_bytes;    /* device scratch run() needs */
  double plan_host_us;        /* host time spent in varlen_attn_plan */
  double prefill_flops;       /* part of `flops` of the requests run on MFMA tiles */
  double split_flops;         /* part of `flops` of the requests run on split-KV items */
  int64_t prefill_kv_bytes;   /* distinct KV bytes the tile requests read */
  int64_t split_kv_bytes;     /* distinct KV bytes the split-KV requests read */
  int64_t split_q_bytes;      /* query bytes of the split-KV requests */
  int64_t direct_items;       /* split-KV items that write output rows directly (no combine) */
  int64_t shared_tiles;       /* MFMA tiles scoring shared-prefix chunks for stacked member rows
                                 (part of prefill_tiles) */
  double shared_tile_flops;   /* part of split_flops done by those tiles (in the prefill stage) */
  int64_t split_item_kv_bytes; /* distinct KV bytes the split-KV items read */
  int64_t prefill_split_tiles; /* of prefill_tiles, those scoring one key chunk of a cut tile */
  double split_item_flops;    /* part of `flops` done by the split-KV items */
} va_plan_stats;

typedef struct va_plan va_plan;   /* opaque, immutable after creation */

/* Build a plan for one iteration's metadata (all arrays are host memory, read during the
 * call only).  Validates: q_start <= q_end, q_rows <= kv_len, Q ranges do not overlap,
 * kv_len <= max_pages_per_req * page_size, the first ceil(kv_len/page_size) block-table ids
 * of every request in [0, num_pages),
 * Hq % Hkv == 0, supported head_dim / page_size / dtype.  Requests with q_rows == 0 are
 * skipped.  Unless VA_FLAG_HOST_ONLY is set, uploads the work lists to a device buffer on
 * the current HIP device (synchronously).  On success *plan_out is a new plan and
 * *workspace_bytes_out (if not NULL) the device workspace run() needs. */
va_status varlen_attn_plan(const va_params* params, int32_t num_reqs, const int32_t* q_start,
                           const int32_t* q_end, const int32_t* kv_len,
                           const int32_t* block_table_host, va_plan** plan_out,
                           size_t* workspace_bytes_out);

/* Enqueue the attention of the planned iteration on `stream` (a hipStream_t, NULL for the
 * null stream).  q, k_pool, v_pool, out: device buffers in the layouts above;
 * block_table_dev: device copy of the block table given to the plan; workspace: device
 * buffer of at least the plan's workspace bytes (contents need not be initialised; may be
 * NULL when the plan needs none).  Output rows outside every request are not written. */
va_status varlen_attn_run(const va_plan* plan, const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_table_dev, void* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/* varlen_attn_run for a plan built with dtype VA_DTYPE_FP8_E4M3: k_pool and v_pool hold
 * the fp8 codes, k_scale and v_scale (device float32 [num_pages][num_kv_heads][page_size],
 * 16-byte aligned) their scales; q and out are bf16.  events: NULL, or VA_RUN_EVENTS
 * events recorded as by varlen_attn_run_events.  Any other plan dtype is refused. */
va_status varlen_attn_run_fp8(const va_plan* plan, const void* q, const void* k_pool, const void* v_pool,
                              const float* k_scale, const float* v_scale, const int32_t* block_table_dev,
                              void* out, void* workspace, size_t workspace_bytes, void* stream,
                              void* const* events);

/* Same as varlen_attn_run, and also records the VA_RUN_EVENTS hipEvent_t handles in
 * `events` on `stream` around its kernel stages, for per-kernel timing:
 *   events[0] before the MFMA prefill kernel, events[1] after it (before the split-KV
 *   kernel), events[2] after the split-KV kernel (before combine), events[3] at the end.
 * A stage with no work leaves two consecutive events adjacent.  The events are created
 * by the caller (with timing enabled) and are only recorded here. */
/* varlen_attn_run without a workspace argument, for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that forbid
 * allocation): the library's own static scratch of VA_STATIC_SCRATCH_BYTES on each device
 * (a file-scope device array held from the library's load until the process ends) is the
 * workspace.  Nothing is allocated: no hipMalloc or other allocating call.  The caller
 * still owns q, k_pool, v_pool, block_table_dev and out (as in varlen_attn_run).  A plan
 * whose workspace exceeds VA_STATIC_SCRATCH_BYTES is refused with
 * VA_ERR_WORKSPACE_TOO_SMALL; fp8 plans are refused (use varlen_attn_run_fp8).  Every call
 * on one device shares that device's scratch, which keeps the last call's contents (every
 * partial result is written before it is read, so nothing needs clearing): calls that
 * overlap on one device -- on different streams, or on one stream while another thread
 * enqueues -- race on it and must be serialised by the caller.  The device address of the
 * scratch is looked up on the first call on each device (with that device current). */
#define VA_STATIC_SCRATCH_BYTES (64u << 20)
va_status varlen_attn_run_noalloc(const va_plan* plan, const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_table_dev, void* out, void* stream);

#define VA_RUN_EVENTS 4
va_status varlen_attn_run_events(const va_plan* plan, const void* q, const void* k_pool,
                                 const void* v_pool, const int32_t* block_table_dev, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* events);

/* Write one iteration's new K and V into the paged pools ("ORCA 和 chunked prefill",
 * section 3: the layer's K/V of the new rows are appended to each request's cache before
 * attention reads the whole prefix; "GLM-5.3 推理全链路(八)", stage 4: out_cache_loc gives
 * every new token the page and slot it is written to).
 *   params:        layout of the pools (num_kv_heads, head_dim, page_size, num_pages, dtype;
 *                  the other fields are ignored)
 *   num_tokens:    new tokens (>= 0)
 *   k_new, v_new:  device [num_tokens][num_kv_heads][head_dim], element type params->dtype
 *   out_cache_loc: device int64 [num_tokens]: token t goes to page loc / page_size, slot
 *                  loc % page_size of both pools; loc < 0 is padding and writes nothing
 *   k_pool, v_pool: device pools in the layouts above (K rows, V pages transposed)
 *   bad_loc_count: optional device int32 (NULL: not reported); every token whose loc is
 *                  >= num_pages * page_size is skipped and counted here (atomically added,
 *                  the caller zeroes it)
 * Values are copied bit for bit.  k_new, v_new, k_pool and v_pool must be 16-byte aligned
 * (VA_ERR_INVALID_ARG otherwise).  Enqueue only (no allocation, no synchronisation); two
 * tokens naming the same slot leave one of them, unspecified which. */
va_status varlen_attn_append_kv(const va_params* params, int64_t num_tokens, const void* k_new,
                                const void* v_new, const int64_t* out_cache_loc, void* k_pool,
                                void* v_pool, int32_t* bad_loc_count, void* stream);

/* varlen_attn_append_kv for fp8 pools (params->dtype VA_DTYPE_FP8_E4M3): k_new, v_new are
 * bf16 [num_tokens][num_kv_heads][head_dim] (finite values).  Each token's K vector and V
 * vector of each KV head is stored as e4m3fn codes with its own float32 scale: scale =
 * max|x| / 448 (float32 division; 1 for an all-zero vector) and code = x / scale rounded
 * to the nearest e4m3fn value, ties to even ("GLM-5.3 推理全链路(八)", on the costs outside
 * the 656-byte ledger: each token's FP8 data carries FP32 scales).  The codes go to
 * k_pool / v_pool and the scales to k_scale / v_scale ([num_pages][num_kv_heads][page_size])
 * at the token's out_cache_loc; padding, out-of-range entries, bad_loc_count and the
 * 16-byte alignment of k_new, v_new and the code pools are as in varlen_attn_append_kv.
 * Enqueue only. */
va_status varlen_attn_append_kv_fp8(const va_params* params, int64_t num_tokens, const void* k_new,
                                    const void* v_new, const int64_t* out_cache_loc, void* k_pool, void* v_pool,
                                    float* k_scale, float* v_scale, int32_t* bad_loc_count, void* stream);

/* The out_cache_loc of the planned iteration (host int64 [total_q_rows]): flat row
 * q_start[r] + i of request r is logical position kv_len[r] - q_rows + i, in page
 * block_table[r][pos / page_size], slot pos % page_size; rows outside every request get -1. */
va_status varlen_attn_plan_slots(const va_plan* plan, int64_t* out_cache_loc_host);

/* Counters of the planned work (no device access).  The distinct-position counters
 * (physical_kv_bytes, prefill_kv_bytes, split_kv_bytes, split_item_kv_bytes) walk every
 * block-table entry and are computed on the first call for a plan (thread-safe), so
 * plan_host_us does not include them. */
va_status varlen_attn_plan_stats(const va_plan* plan, va_plan_stats* out);

/* Measurement aid: reads `bytes` of device memory at `buf` once (16-byte loads, streaming)
 * and discards them, so a caller can time the device's achievable HBM read rate with the
 * same runtime and launch path as the attention kernels.  buf must be 16-byte aligned and
 * bytes a multiple of 16; sink is a device uint32 that the kernel overwrites only when the
 * XOR of a lane's words hits one fixed value (it keeps the loads from being optimised away;
 * its content is meaningless).  Enqueue only. */
va_status varlen_attn_debug_stream_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/* Copy every request's K and V into logical order through the same page-address code the
 * attention kernels use: k_out, v_out are device [sum_r kv_len[r]][num_kv_heads][head_dim]
 * (requests back to back).  Exists to test the page gather bit for bit. */
va_status varlen_attn_debug_gather(const va_plan* plan, const void* k_pool, const void* v_pool,
                                   const int32_t* block_table_dev, void* k_out, void* v_out,
                                   void* stream);

/* The same copy as varlen_attn_debug_gather, made by the MFMA attention kernel's own
 * staging of bf16 pools: one workgroup per (request, KV head) stages every 64-key tile of
 * the request into LDS with the page lookup, DMA addressing (buffer resources over page
 * slices, per-lane offsets) and tail handling the attention tiles use, then copies the staged
 * K rows and V^T slices out in logical order.  bf16 plans only (VA_ERR_UNSUPPORTED
 * otherwise); pools and outputs 16-byte aligned.  Exists to test that address path bit for
 * bit ("How To Scale Your Model 笔记(7-8)", section 3: paging changes where a position is
 * stored, not what is read). */
va_status varlen_attn_debug_stage_gather(const va_plan* plan, const void* k_pool, const void* v_pool,
                                         const int32_t* block_table_dev, void* k_out, void* v_out, void* stream);

/* Widen n fp8 e4m3fn codes (device, 8-byte aligned; n a multiple of 8) to bf16 bit
 * patterns (device uint16 [n], 16-byte aligned) with the converter the fp8 attention
 * kernel uses.  Exists to test that conversion against the format's definition. */
va_status varlen_attn_debug_fp8_to_bf16(const uint8_t* codes, uint16_t* out, int64_t n, void* stream);

/* Introspection for tests: the plan's host work lists as int32 records.
 * which = 0: split-KV items {req, kvh, col0, ncols, k0, k1, slot, flags}
 *            (flags bit 0: some column's causal limit falls inside [k0, k1); bit 1: the
 *            item writes its columns' output rows directly)
 *         1: query columns {q_row, q_head, limit, pbase}
 *         2: combine rows {q_row, q_head, pbase, nparts}
 *         3: MFMA tiles in launch order {req, kvh, c0, ncols, q0, S0, kv_end, kbeg, pbase,
 *            pstride, flags, group}: columns c0 .. c0+ncols of request req under KV head kvh
 *            (column c = new row c / g, head kvh*g + c % g, row i sees keys up to S0 + i),
 *            keys [kbeg, kv_end); pbase < 0: output rows written directly, else column c's
 *            partial to slot pbase + (c - c0) * pstride.  flags bit 0 (column list): the
 *            columns are cols[c0 .. c0+ncols) instead, their partials to slot pbase + q0
 *            (of each column); group = 1 marks a shared-prefix group tile
 *         4: the column-list tiles of 3 only
 * *data stays valid until the plan is destroyed. */
va_status varlen_attn_plan_export(const va_plan* plan, int32_t which, const int32_t** data,
                                  int64_t* count, int32_t* ints_per_entry);

void varlen_attn_plan_destroy(va_plan* plan);
const char* varlen_attn_status_string(va_status status);
const char* varlen_attn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* VARLEN_ATTN_H */
