/*
 * mla_decode.h — C ABI of the MI355X (gfx950) MLA paged-KV decode library.
 *
 * The library computes batched decode attention in the multi-head latent
 * attention (MLA) "absorbed" form over a paged latent cache, as the FlashMLA
 * attention backend page of SGLang drives it:
 *
 *   - q is [bs, q_len, H, 576] (kv_lora_rank 512 + rope 64), viewed that way
 *     in FlashMLABackend.forward_decode;
 *   - the cache is [num_pages, 64, 576] latent rows (64-token pages, the
 *     module's PAGE_SIZE; forward_decode views it as [-1, 64, 1, 576]);
 *     V is the first 512 columns of the same row (head_dim_v = kv_lora_rank);
 *   - pages are found through a per-request block table built from the
 *     req_to_token map (init_forward_metadata);
 *   - the KV sequence is split into pieces by a planner (the get_mla_metadata
 *     call: a [num_parts, 8] tile table and a bs+1 split vector), each piece
 *     produces a partial (o, lse) state, and the pieces are merged exactly
 *     (the merge_state step of the FlashInfer backend page's forward_extend).
 *
 * Conventions shared by every entry point
 *   - Every pointer is device memory unless its comment says "host".
 *   - The caller owns every buffer.  The library allocates no device memory
 *     at run time; its only device memory of its own is file-scope arrays
 *     (the static workspace of mla_decode_static; the debug build's error
 *     word), held per device until the process ends.
 *     State kept between calls: per host thread, the last error text and the
 *     events of mla_decode_time_next_launch (used by the next decode only);
 *     per device, whether the planner kernels' LDS limit was raised (set
 *     once, on their first launch there) and the static workspace's address;
 *     per process, whether MLA_TRACE is set (read once).
 *   - Calls are asynchronous on the given HIP stream (0 = the null stream),
 *     never synchronise and never read device memory on the host, so they can
 *     be captured in a HIP graph (the FlashMLA page prepares fixed-capacity
 *     buffers for graph replay in init_cuda_graph_state).  The debug build
 *     (libmla_decode_debug.so, compiled with -DMLA_DEBUG) is the exception:
 *     the table builders and the decodes check their preconditions on the
 *     device and synchronise the stream to read the result back.
 *   - With the environment variable MLA_TRACE set (not "0"), every launch
 *     writes one line to stderr ("[mla] entry point: sizes, grid, stream").
 *   - Argument errors are detected on the host before any launch and
 *     returned as a status; nothing is launched then.  No C++ exception
 *     crosses the ABI; no call aborts the process.
 *   - Row order inside a request is r = i*H + h (token i of q_len, head h).
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 2
#define MLA_PAGE_SIZE 64
#define MLA_LATENT_DIM 576
#define MLA_V_DIM 512
#define MLA_MAX_ROWS_PER_REQ 512   /* H * q_len */
#define MLA_MAX_BATCH 16384        /* planner limit */
#define MLA_MAX_PARTS 512          /* planner limit (also <= device CU count) */
#define MLA_MAX_DECODE_PARTS 65536 /* parts one mla_decode launch takes (fixed-tile plans) */

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARGUMENT = 1, /* null pointer, negative size, bad enum, non-finite scale */
  MLA_ERR_UNSUPPORTED = 2,      /* a shape or dtype this build has no kernel for */
  MLA_ERR_CAPACITY = 3,         /* a caller buffer is too small for the request */
  MLA_ERR_PRECONDITION = 4,     /* debug build only: a device-side precondition check failed */
  MLA_ERR_DEVICE = 5            /* a HIP runtime call failed; see mla_last_error_message */
} mla_status;

typedef enum mla_kv_dtype {
  MLA_KV_BF16 = 0,      /* latent rows are bf16 */
  MLA_KV_FP8_E4M3 = 1   /* latent rows are OCP float8 e4m3fn bytes, times a per-tensor descale */
} mla_kv_dtype;

/* Version of this ABI (MLA_ABI_VERSION of the build). */
int32_t mla_abi_version(void);

/* Static text for a status code; any int32 value is accepted ("unknown
 * status" for values that are not an mla_status). */
const char* mla_status_string(int32_t status);

/* Text describing the last non-OK status returned on this host thread
 * ("" if none).  Valid until the next library call on the thread. */
const char* mla_last_error_message(void);

/*
 * mla_build_block_table — per-request page table.
 *
 * The index kernel the FlashMLA page launches in init_forward_metadata
 * (create_flashmla_kv_indices_triton, body not on the page): for request b,
 * n_b = ceil(seq_lens[b] / 64) and, for p < n_b,
 *     block_table[b * bt_row_stride + p] = floor(req_to_token[rpi[b] * r2t_row_stride + 64*p] / 64)
 * i.e. the page holding token 64p.  Every other cell of the row, up to
 * bt_row_stride, is written with pad_value (the page pre-fills with -1).
 * Slots are assumed page-aligned (slot of token j = 64*page + j % 64); the
 * debug build checks every token of every request against the table it
 * built and returns PRECONDITION naming the first that differs (a table
 * narrower than a request counts as well).
 *
 *   req_to_token      int32 [r2t_rows, r2t_row_stride]
 *   req_pool_indices  int32 [bs], each in [0, r2t_rows)
 *   seq_lens          int32 [bs], KV lengths incl. the new tokens, >= 0
 *   page_size         must be 64
 *   block_table       int32 [bs, bt_row_stride], written in full
 *   max_seq_len_hint  host: an upper bound of seq_lens, or -1 if unknown
 *
 * Errors: INVALID_ARGUMENT for null pointers, bs <= 0, r2t_rows <= 0,
 * bt_row_stride <= 0 or r2t_row_stride <= 0; UNSUPPORTED for page_size != 64;
 * CAPACITY when the hint needs more than bt_row_stride pages or more than
 * r2t_row_stride slots.  Without a hint the device clamps a request that needs
 * more than bt_row_stride pages to bt_row_stride pages, and a cell whose
 * req_to_token read would fall outside the map gets pad_value.
 */
mla_status mla_build_block_table(const int32_t* req_to_token, int32_t r2t_rows,
                                 int64_t r2t_row_stride, const int32_t* req_pool_indices,
                                 const int32_t* seq_lens, int32_t bs, int32_t page_size,
                                 int32_t* block_table, int32_t bt_row_stride,
                                 int32_t pad_value, int32_t max_seq_len_hint,
                                 hipStream_t stream);

/*
 * mla_plan_splits — split the (request, page) sequence over num_parts
 * work-groups (the get_mla_metadata call of init_forward_metadata: a
 * [num_parts, 8] table and a bs+1 vector; num_parts at most the CU count).
 *
 * Rule (deterministic, depends only on seq_lens, rows_per_req, num_parts),
 * in quarter pages: request b has N_b = ceil(L_b/64) pages and costs
 * 4 N_b + c, with c = 4 + ceil(8 rows_per_req / 128) the per-piece overhead
 * (0 for an empty request).  With C the total cost, part p covers cost
 * positions [floor(pC/P), floor((p+1)C/P)); a position x inside request b
 * maps to the page boundary clamp(floor((x - cum_b - c + 2) / 4), 0, N_b).
 * Each part therefore costs at most ceil(C/P) + c + 4 units (counting c for
 * every piece it holds), every page lies in exactly one part, and the number
 * of pieces is at most bs + num_parts.
 *
 *   tile_plan     int32 [num_parts, 8]: begin_req, begin_page, end_req
 *                 (inclusive), end_page (exclusive, in end_req), piece index
 *                 of the first piece inside begin_req, number of pages, 0, 0.
 *                 An empty part is all zeros.
 *   split_indptr  int32 [bs + 1]: split_indptr[b] = pieces before request b;
 *                 request b's pieces use partial slots split_indptr[b] ..
 *                 split_indptr[b+1]-1, in part order.
 *   kv_dtype      MLA_KV_BF16 or MLA_KV_FP8_E4M3 (accepted for symmetry with
 *                 the page's is_fp8_kvcache flag; the rule does not use it).
 *
 * Errors: INVALID_ARGUMENT for null pointers, bs <= 0, num_parts <= 0 or a bad
 * dtype; UNSUPPORTED for rows_per_req outside 1..512 or a tile_plan that is
 * not 16-byte aligned (rows are written 16 bytes at a time); CAPACITY for
 * bs > MLA_MAX_BATCH, num_parts > MLA_MAX_PARTS or num_parts above the current
 * device's CU count (the page asserts num_sm_parts <= preallocated count).
 */
mla_status mla_plan_splits(const int32_t* seq_lens, int32_t bs, int32_t rows_per_req,
                           int32_t num_parts, int32_t kv_dtype, int32_t* tile_plan,
                           int32_t* split_indptr, hipStream_t stream);

/*
 * mla_plan_fixed_splits — deterministic plan with fixed-size tiles (the
 * FlashInfer backend page's deterministic mode: enable_deterministic splits
 * the decode KV into tiles of decode_split_tile_size = 2048 tokens, i.e. 32
 * pages, and switches graph-mode KV splitting off).
 *
 * Request b, with N_b = ceil(seq_lens[b] / 64) pages, is cut at the
 * multiples of tile_pages pages of its own sequence into
 * n_b = ceil(N_b / tile_pages) pieces.  Where a request is cut, and so every
 * floating-point step of its result, does not depend on the other requests
 * of the batch or on max_parts: a request decodes bit for bit the same alone
 * or in any batch.  Each part holds exactly one piece:
 *   split_indptr[b] = n_0 + ... + n_{b-1},
 *   part split_indptr[b] + k = {b, k*T, b, min((k+1)*T, N_b), k, pages, 0, 0}
 * (the mla_plan_splits row format), T = tile_pages; rows from
 * split_indptr[bs] to max_parts - 1 are zeros (parts with nothing to do).
 * Pass the plan to mla_decode with num_parts = max_parts and
 * partial_slots >= bs + max_parts.  Unlike mla_plan_splits, the number of
 * parts is not tied to the CU count, so short batches may leave CUs idle.
 *
 *   tile_plan         int32 [max_parts, 8], 16-byte aligned
 *   split_indptr      int32 [bs + 1]
 *   max_seq_len_hint  host: an upper bound of seq_lens, or -1
 *
 * If the pieces do not fit in max_parts rows (possible only without a
 * hint), nothing is planned: every row and every split_indptr entry is 0, so
 * decode and merge then write o = 0 and lse = -inf for every row.
 *
 * Errors: INVALID_ARGUMENT for null pointers or bs, tile_pages or max_parts
 * <= 0; UNSUPPORTED for a tile_plan that is not 16-byte aligned; CAPACITY for bs > MLA_MAX_BATCH, max_parts > MLA_MAX_DECODE_PARTS,
 * or when the hint allows more pieces than max_parts
 * (mla_fixed_split_parts_bound(bs, hint, tile_pages) > max_parts).
 */
mla_status mla_plan_fixed_splits(const int32_t* seq_lens, int32_t bs, int32_t tile_pages,
                                 int32_t max_parts, int32_t max_seq_len_hint,
                                 int32_t* tile_plan, int32_t* split_indptr, hipStream_t stream);
/* Host helper: bs * ceil(ceil(max_seq_len / 64) / tile_pages), the most
 * pieces a fixed-tile plan of such a batch can have (INT32_MAX if larger;
 * -1 for negative sizes or tile_pages <= 0). */
int32_t mla_fixed_split_parts_bound(int32_t bs, int32_t max_seq_len, int32_t tile_pages);
/*
 * mla_plan_fixed_packed — the fixed-size tiles of mla_plan_fixed_splits (the
 * same pieces: request b is cut at the multiples of tile_pages pages of its
 * own sequence, and split_indptr is the same), packed into num_parts parts
 * of about equal cost, as mla_plan_splits packs pages: so a deterministic
 * plan keeps every CU busy whether the batch has fewer or more tiles than
 * CUs.  Every tile stays a piece of its own wherever it lands (the decode
 * ends a piece at each multiple of tile_pages pages of a request, told so
 * by field 6 of the row), so a request still decodes bit for bit the same
 * alone or in any batch (FlashInfer backend page, __init__: the
 * deterministic mode's fixed decode_split_tile_size).
 *
 * The rule, in quarter pages: a tile of n pages costs 4 n + c, c the
 * per-piece overhead of mla_plan_splits for rows_per_req rows; with Q_t the
 * cost of the tiles before tile t (request order, then tile order), C the
 * total and x_p = floor(p C / num_parts), part p holds the tiles from the
 * boundary whose Q is nearest x_p (the lower one on a tie) to that of
 * x_{p+1} (part num_parts - 1 ends at the last tile).  Row p is
 *   {first request, its first page, last request, end page there,
 *    tile index of the first tile in its request, pages, tile_pages, 0}
 * (all zeros for an empty part).  Every part costs at most C / num_parts
 * plus one tile.
 *
 * Pass the plan to mla_decode with num_parts and partial_slots >= the
 * number of tiles, split_indptr[bs] (at most mla_fixed_split_parts_bound).
 *
 *   tile_plan     int32 [num_parts, 8], 16-byte aligned
 *   split_indptr  int32 [bs + 1]
 *
 * Errors: INVALID_ARGUMENT for null pointers or bs, tile_pages, num_parts
 * <= 0; UNSUPPORTED for rows_per_req outside 1..512 or a misaligned
 * tile_plan; CAPACITY for bs > MLA_MAX_BATCH or num_parts above the CU count
 * (or MLA_MAX_PARTS).  The total cost must stay below 2^31 quarter pages.
 */
mla_status mla_plan_fixed_packed(const int32_t* seq_lens, int32_t bs, int32_t tile_pages,
                                 int32_t rows_per_req, int32_t num_parts, int32_t* tile_plan,
                                 int32_t* split_indptr, hipStream_t stream);
/*
 * mla_build_table_and_plan — mla_build_block_table and mla_plan_splits in
 * one launch (init_forward_metadata of both page backends computes the block
 * table and the split metadata together, once per batch step).  One work-group
 * plans while the others fill the table, so the step pays for one small
 * launch instead of two.
 *
 * Arguments are those of the two calls (same meaning, same layouts), and the
 * results are bit for bit theirs.  Errors: those of mla_build_block_table,
 * then those of mla_plan_splits, checked before anything is launched;
 * UNSUPPORTED if the table needs more than 2^31 - 2 work-groups.
 */
mla_status mla_build_table_and_plan(const int32_t* req_to_token, int32_t r2t_rows,
                                    int64_t r2t_row_stride, const int32_t* req_pool_indices,
                                    const int32_t* seq_lens, int32_t bs, int32_t page_size,
                                    int32_t* block_table, int32_t bt_row_stride,
                                    int32_t pad_value, int32_t max_seq_len_hint,
                                    int32_t rows_per_req, int32_t num_parts, int32_t kv_dtype,
                                    int32_t* tile_plan, int32_t* split_indptr,
                                    hipStream_t stream);

/* Host helpers: upper bound of split_indptr[bs] (= bs + num_parts), and the
 * bytes of the decode workspace that bound needs: partial_o (bf16
 * [slots, rows_per_req, 512]) plus partial_lse (fp32 [slots, rows_per_req])
 * with slots = bs + num_parts (the page's backends take one preallocated
 * workspace buffer).  mla_partial_bytes is the same function under its
 * earlier name.  0 for negative sizes. */
int32_t mla_max_total_splits(int32_t bs, int32_t num_parts);
size_t mla_workspace_bytes(int32_t bs, int32_t rows_per_req, int32_t num_parts);
size_t mla_partial_bytes(int32_t bs, int32_t rows_per_req, int32_t num_parts);

/* Host helper: CU count of the current device (the default num_parts), or -1. */
int32_t mla_device_num_cus(void);

/*
 * mla_decode — split attention over the plan's pieces
 * (flash_mla_with_kvcache as forward_decode and the target-verify branch of
 * forward_extend call it).
 *
 * For request b, query row r = i*H + h (i < q_len) and visible keys
 * j <= L_b - q_len + i when causal (bottom-right aligned; all j < L_b
 * otherwise), with K_j the latent row of token j (times *kv_descale for fp8)
 * and V_j its first 512 columns:
 *     s_j = softmax_scale * <q_r, K_j>,  lse_r = ln sum_j exp(s_j),
 *     o_r = sum_j exp(s_j - lse_r) V_j.
 * A piece computes these sums over its own pages.  A request with exactly
 * one piece is final: o goes to out (bf16, round to nearest even) and lse to
 * lse.  Otherwise each piece writes its o (normalised by its own row sum,
 * rounded to bf16) and its lse (fp32) to partial slot split_indptr[b] + piece,
 * and mla_merge_states finishes the request.  A slot outside
 * [0, partial_slots) is not written.
 *
 *   q             bf16 [bs, q_len, num_heads, 576], contiguous
 *   kv_cache      [num_pages, 64, 576] bf16, or bytes for MLA_KV_FP8_E4M3
 *   block_table   int32 [bs, bt_row_stride] from mla_build_block_table
 *   seq_lens      int32 [bs], the lengths the plan was made from
 *   tile_plan, split_indptr, num_parts   from mla_plan_splits
 *   softmax_scale host, by value (passed as a host float so no device read is
 *                 needed, as the FlashInfer page notes for graph capture)
 *   kv_descale    device fp32 scalar delta for fp8 (ignored for bf16, may be
 *                 NULL): the latent value of a cache byte is e4m3fn(byte) * delta,
 *                 one scale for K and V (the page's descale_k).  delta must be
 *                 finite; it may be 0 or negative.  Read on the device, so a
 *                 captured graph picks up a new value without re-capture.
 *   partial_o     bf16 [partial_slots, q_len*num_heads, 512], 16-byte aligned
 *   partial_lse   fp32 [partial_slots, q_len*num_heads]
 *   partial_slots slots of the workspace (the decode's capacity argument;
 *                 the page's graph state preallocates fixed capacities)
 *   out           bf16 [bs, q_len, num_heads, 512] (rows of split requests
 *                 are written by mla_merge_states)
 *   lse           fp32 [bs, q_len, num_heads] natural-log LSE, or NULL
 *
 * Block-table entries outside [0, num_pages), or a page index at or past
 * bt_row_stride, are a caller error: such a page is never read, and its keys
 * are masked (they contribute nothing), so the kernel never leaves the pool.
 * The debug build checks the entries first and returns PRECONDITION naming
 * the first bad (request, page), launching nothing.
 *
 * Errors: INVALID_ARGUMENT for null pointers, non-positive sizes, a
 * negative or non-finite scale, or fp8 with a NULL kv_descale; UNSUPPORTED for
 * q_len*num_heads outside 1..512 or an unknown kv_dtype; CAPACITY when
 * partial_slots < bs + num_parts or num_parts > MLA_MAX_DECODE_PARTS.
 */
mla_status mla_decode(const void* q, int32_t bs, int32_t q_len, int32_t num_heads,
                      const void* kv_cache, int32_t kv_dtype, int64_t num_pages,
                      const int32_t* block_table, int32_t bt_row_stride,
                      const int32_t* seq_lens, const int32_t* tile_plan, int32_t num_parts,
                      const int32_t* split_indptr, float softmax_scale, int32_t causal,
                      const float* kv_descale, void* partial_o, float* partial_lse,
                      int32_t partial_slots, void* out, float* lse, hipStream_t stream);

/*
 * mla_decode_q8 — mla_decode with an e4m3 query over an e4m3 cache (the fp8
 * branch of forward_decode on the FlashMLA page: q quantised with
 * scaled_fp8_quant, here mla_quantize_q_fp8, and handed to the kernel with
 * descale_q and descale_k).
 *
 * Computes what mla_decode computes with the query row value
 * q_r = e4m3fn(q_fp8 code) * (*q_descale) and the cache value
 * e4m3fn(byte) * (*kv_descale).  The scores are sums of exact products of
 * e4m3 codes (matrix cores, fp32 accumulation) times
 * softmax_scale * q_descale * kv_descale; the output contraction also runs
 * on e4m3 operands, V as stored and each weight as the sum of two e4m3
 * numbers (about 2^-8 relative, against bf16's 2^-9 in mla_decode), scaled
 * by a power of two per page, accumulated in fp32.
 *
 *   q_fp8      uint8 e4m3fn codes [bs, q_len, num_heads, 576], contiguous,
 *              16-byte aligned
 *   q_descale  device fp32 scalar, finite (may be 0 or negative); read on
 *              the device
 *   kv_cache   [num_pages, 64, 576] e4m3fn bytes
 *   the rest   as for mla_decode (kv_descale is required)
 *
 * Errors: those of mla_decode for an MLA_KV_FP8_E4M3 cache, and
 * INVALID_ARGUMENT for a NULL q_descale.
 */
mla_status mla_decode_q8(const void* q_fp8, const float* q_descale, int32_t bs, int32_t q_len,
                         int32_t num_heads, const void* kv_cache, int64_t num_pages,
                         const int32_t* block_table, int32_t bt_row_stride,
                         const int32_t* seq_lens, const int32_t* tile_plan, int32_t num_parts,
                         const int32_t* split_indptr, float softmax_scale, int32_t causal,
                         const float* kv_descale, void* partial_o, float* partial_lse,
                         int32_t partial_slots, void* out, float* lse, hipStream_t stream);

/*
 * mla_decode_time_next_launch — measurement hook.  The next mla_decode call
 * on this host thread launches its kernel with hipExtLaunchKernel so that
 * `start` and `stop` (events the caller created; either may be NULL) take
 * the kernel's own begin and end times.  hipEventElapsedTime(start, stop)
 * is then the kernel's duration, without the dispatch and cache-flush time
 * that a separate event pair around the call also counts.  The hook is used
 * once and cleared, also when that mla_decode call fails.  Always MLA_OK.
 */
mla_status mla_decode_time_next_launch(hipEvent_t start, hipEvent_t stop);

/*
 * mla_merge_states — exact merge of partial (o, lse) states (merge_state of
 * the FlashInfer page's forward_extend, generalised to k pieces).
 *
 * For request b with k = split_indptr[b+1] - split_indptr[b] pieces and each
 * row r:  M = max_k lse_k,  LSE = M + ln sum_k exp(lse_k - M),
 *         o = sum_k exp(lse_k - LSE) * o_k.
 * Pieces with lse = -inf weigh 0, and so does a piece whose slot
 * split_indptr[b] + s lies outside [0, partial_slots) (it is not read); if all
 * do, o = 0 and LSE = -inf.
 * k == 1: the request is skipped (mla_decode already wrote it).
 * k == 0: o = 0 and LSE = -inf are written.
 * A two-way merge of arbitrary states is the case split_indptr = {0, 2, 4, ...}.
 *
 *   partial_o     bf16 [partial_slots, rows_per_req, dv], 16-byte aligned
 *   partial_lse   fp32 [partial_slots, rows_per_req]
 *   dv            value width; must be 512 (kv_lora_rank)
 *   out           bf16 [bs, rows_per_req, dv], 16-byte aligned
 *   lse           fp32 [bs, rows_per_req] or NULL
 *
 * Errors: INVALID_ARGUMENT for null pointers, bs <= 0 or partial_slots < 0;
 * UNSUPPORTED for rows_per_req outside 1..512, dv != 512 or misaligned
 * partial_o / out.
 */
mla_status mla_merge_states(const void* partial_o, const float* partial_lse,
                            int32_t partial_slots, const int32_t* split_indptr, int32_t bs,
                            int32_t rows_per_req, int32_t dv, void* out, float* lse,
                            hipStream_t stream);

/*
 * mla_decode_static — mla_decode and then mla_merge_states in one call that
 * allocates nothing and takes no workspace: for callers that cannot allocate
 * device memory or hand one in (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).
 *
 * Arguments and results are those of mla_decode without partial_o,
 * partial_lse and partial_slots: every request's final o goes to out and its
 * lse to lse (or nowhere if lse is NULL), whatever its number of pieces.
 * The split pieces' partial states live in a device array of the library,
 * MLA_STATIC_WORKSPACE_BYTES (64 MiB) per GPU, held from the first call on
 * that GPU until the process ends; a call needs
 * (bs + num_parts) * q_len * num_heads * 1028 bytes of it.
 *
 * Every call on one GPU uses that GPU's one array: calls that overlap on a
 * GPU (on different streams, or from several host threads) race and must be
 * ordered by the caller.  Nothing in the array needs to start at zero: each
 * slot the merge reads is written by the decode of the same call.
 *
 * Errors: those of mla_decode and mla_merge_states; CAPACITY when the
 * partial states would exceed MLA_STATIC_WORKSPACE_BYTES; DEVICE when the
 * array's address cannot be found on the current device.
 */
#define MLA_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
mla_status mla_decode_static(const void* q, int32_t bs, int32_t q_len, int32_t num_heads,
                             const void* kv_cache, int32_t kv_dtype, int64_t num_pages,
                             const int32_t* block_table, int32_t bt_row_stride,
                             const int32_t* seq_lens, const int32_t* tile_plan, int32_t num_parts,
                             const int32_t* split_indptr, float softmax_scale, int32_t causal,
                             const float* kv_descale, void* out, float* lse, hipStream_t stream);

/*
 * mla_set_kv_buffer — store the new tokens' latent rows in the paged cache
 * (token_to_kv_pool.set_kv_buffer(layer, cache_loc, k, v) with
 * cache_loc = out_cache_loc, which forward_decode and the target-verify
 * branch of forward_extend on the FlashMLA page call before attention).
 *
 * For i < num_tokens and s = out_cache_loc[i] with 0 <= s < 64*num_pages,
 * latent row i of k goes to row s % 64 of page s / 64.  In MLA V is the first
 * 512 columns of that row, so nothing else is stored.  Slots outside the pool
 * are skipped (never written).  Slots are expected to be distinct; if two
 * tokens name one slot, which row it ends up holding is unspecified.
 *
 *   k              bf16 [num_tokens, k_row_stride], the first 576 columns of a
 *                  row are its latent row; 16-byte aligned
 *   k_row_stride   elements between rows, >= 576 and a multiple of 8
 *   out_cache_loc  int64 [num_tokens] pool slots
 *   kv_cache       [num_pages, 64, 576] bf16, or e4m3fn bytes for
 *                  MLA_KV_FP8_E4M3; 16-byte aligned; updated in place
 *   kv_scale       fp8 only: device fp32 scalar (the page's k_scale).  The
 *                  stored byte is the e4m3fn value nearest to k / kv_scale
 *                  (the quotient rounded to fp32, ties to even, magnitudes
 *                  above 448 saturating to 448, NaN to 0x7F/0xFF), so that
 *                  byte * kv_scale, the value mla_decode reads with the same
 *                  scale as kv_descale, approximates k.  Expected positive
 *                  and finite.  Ignored for bf16 (may be NULL).
 *
 * num_tokens == 0 launches nothing (k and out_cache_loc may then be NULL).
 * Errors: INVALID_ARGUMENT for null pointers, num_tokens < 0, num_pages <= 0,
 * k_row_stride < 576, or fp8 with a NULL kv_scale; UNSUPPORTED for an unknown kv_dtype or misaligned k,
 * k_row_stride or kv_cache.
 */
mla_status mla_set_kv_buffer(const void* k, int64_t k_row_stride, const int64_t* out_cache_loc,
                             int32_t num_tokens, void* kv_cache, int32_t kv_dtype,
                             int64_t num_pages, const float* kv_scale, hipStream_t stream);

/*
 * mla_quantize_q_fp8 — quantise query rows to e4m3fn with a per-tensor scale
 * (the fp8 branch of forward_decode on the FlashMLA page runs
 * scaled_fp8_quant(q, q_scale) with q_scale = the cache's k_scale before the
 * attention call, and passes descale_q = k_scale).
 *
 * For every row i < num_rows and column c < 576:
 *     q_fp8[i * 576 + c] = e4m3fn(q[i * q_row_stride + c] / *q_scale)
 * with the quotient rounded to fp32, then to the nearest e4m3fn value (ties
 * to even), magnitudes above 448 saturating to 448 and NaN to 0x7F/0xFF: the
 * rounding of mla_set_kv_buffer's fp8 bytes.
 *
 *   q             bf16 rows of 576 (e.g. [bs, q_len, H, 576] seen as rows),
 *                 16-byte aligned
 *   q_row_stride  elements between rows, >= 576 and a multiple of 8
 *   q_scale       device fp32 scalar, expected positive and finite
 *   q_fp8         uint8 [num_rows, 576], contiguous, 8-byte aligned
 *
 * num_rows == 0 launches nothing (q may then be NULL).  Errors:
 * INVALID_ARGUMENT for null pointers, num_rows < 0 or q_row_stride < 576;
 * UNSUPPORTED for misaligned pointers or stride, or num_rows >= 2^31.
 */
mla_status mla_quantize_q_fp8(const void* q, int64_t q_row_stride, int64_t num_rows,
                              const float* q_scale, void* q_fp8, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
