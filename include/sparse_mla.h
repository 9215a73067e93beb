/*
 * sparse_mla.h - C ABI of the MI355X (gfx950) top-k sparse MLA decode library.
 *
 * What the library computes
 * -------------------------
 * Decode attention for DeepSeek-V4-style multi-head latent attention in which every
 * query row attends only to its own list of top-k cache positions.  One latent KV
 * "head" (576 wide = 512 latent + 64 rope) is shared by all query heads; the value
 * vector is the 512-wide latent part.  The serving engines on the source pages call
 * such a kernel from the sparse-MLA attention backend's forward_mqa, after
 * translating request-local top-k positions to global cache slots through the block
 * table, and allocate the output as [tokens, heads, kv_lora_rank=512] in the dtype
 * of q (prhub vllm#43477 "DSv4 and GLM-5.1 on Blackwell SM120", key code excerpts:
 * FlashInferMLASparseSM120Impl.forward_mqa).  Gathering and dequantizing the paged
 * entries, a tiled online softmax, the merge of split partial results and the
 * attention sink are the pieces of the Triton decode path described on prhub
 * sglang#24692 "SM120 support for DeepSeek-V4", implementation breakdown items 2-3.
 *
 * For query row r (request b = row_req[r]) and head h, with J the multiset of list
 * positions j whose index idx[r][j] != -1:
 *     s_j    = softmax_scale * sum_{d<576} q[r][h][d] * k_j[d]
 *     sigma  = sinks[h]   (or -inf when sinks == NULL)
 *     m      = max(max_j s_j, sigma)
 *     Z      = exp(sigma - m) + sum_j exp(s_j - m)
 *     out[r][h][:] = sum_j exp(s_j - m) * k_j[0:512] / Z        (bf16, round to nearest even)
 *     lse[r][h]    = m + ln Z                                    (fp32, natural log)
 * A row with no valid entry gives out = 0 and lse = sigma (-inf without a sink).
 * The sink adds exp(sigma) to the denominator and carries no value; it is applied once.
 *
 * Split-KV: with S splits, list positions [c*C, (c+1)*C), C = ceil(K/S), form chunk c.
 * A chunk's partial result is sink-free:
 *     o_c   = sum_{j in c} exp(s_j - m_c) k_j[0:512] / sum_{j in c} exp(s_j - m_c)
 *     lse_c = ln sum_{j in c} exp(s_j)          (o_c = 0, lse_c = -inf for an empty chunk)
 * and the merge is
 *     M = max(max_c lse_c, sigma), w_c = exp(lse_c - M), w_s = exp(sigma - M),
 *     out = sum_c w_c o_c / (sum_c w_c + w_s),  lse = M + ln(sum_c w_c + w_s).
 *
 * Cache byte layout (the library's own; the source pages describe one paged buffer
 * read through fp8 / uint8 / bf16 views with in-page addressing, prhub sglang#24692,
 * implementation breakdown items 2-3, and a bf16 cache of shape
 * (num_blocks, block_size, 576), prhub vllm#43477, key code excerpts: get_kv_cache_shape):
 *   SMLA_KV_BF16       page = bf16[page_size][576]; bytes per page 1152*page_size.
 *                      Dims 0..511 are the latent (= V), 512..575 the rope part.
 *   SMLA_KV_FP8_UE8M0  page = 648*page_size bytes, three regions:
 *                        latent  e4m3fn[page_size][512]  at byte 0
 *                        rope    bf16  [page_size][64]   at byte 512*page_size
 *                        scales  uint8 [page_size][8]    at byte 640*page_size
 *                      k[d] = e4m3fn(latent[d]) * 2^(scale[d/64] - 127) for d < 512,
 *                      k[512+i] = rope[i].  e4m3fn is OCP FP8 E4M3 (bias 7, max 448,
 *                      S.1111.111 = NaN); a scale byte is UE8M0 (power of two, 255 = NaN).
 *                      The dequantized value is exact in bf16 for scale bytes 10..246;
 *                      outside that range the kernel's bf16 rounding applies.
 *   SMLA_KV_FP8_TENSOR page = e4m3fn[page_size][576]; bytes per page 576*page_size.  The
 *                      contiguous per-tensor FP8 cache of prhub vllm#43827 (implementation
 *                      breakdown 1 and 4: a contiguous bf16 or fp8_e4m3 cache, bmm1 scale =
 *                      softmax scale * kv scale, bmm2 scale = kv scale): k[d] = e4m3fn(code[d])
 *                      * kv_scale for all 576 dims.  The kernel applies kv_scale as those
 *                      two scalar factors (scores and output); q stays bf16.
 * A cache slot s lives in page s / page_size at in-page row s % page_size.
 *
 * Conventions
 *   - All device pointers are caller-owned device memory; the library never allocates,
 *     frees or synchronises, and launches only on the stream passed in (a hipStream_t
 *     passed as void*; NULL = the null stream).
 *   - Shapes are row-major and contiguous unless a stride is named.
 *   - Every entry point checks its arguments on the host first and returns a status
 *     without launching anything when they are invalid.  A failed launch returns
 *     SMLA_ERR_HIP.
 *   - Index values outside the valid range (< -1, beyond the request's page table,
 *     or page ids outside [0, num_pages)) are never dereferenced: the kernel treats
 *     them as -1.  With SMLA_F_CHECK_INDICES the first such (row, position) is also
 *     recorded in the workspace and can be read with sparse_mla_read_index_error.
 *   - Non-finite q or cache values give unspecified output and LSE for the (row, head)
 *     pairs whose scores or values they reach; every call still completes, and the other
 *     pairs are unaffected.
 *   - The plan is plain host memory, independent of any data, and may be reused across
 *     calls and graph replays.  The library keeps no mutable global state beyond a
 *     per-device attribute cache filled once.
 */
#ifndef SPARSE_MLA_H_
#define SPARSE_MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SMLA_QK_DIM 576
#define SMLA_V_DIM 512
#define SMLA_ROPE_DIM 64
#define SMLA_SCALE_GROUP 64
#define SMLA_NUM_SCALE_GROUPS 8
#define SMLA_FP8_ENTRY_BYTES 648
#define SMLA_BF16_ENTRY_BYTES 1152
#define SMLA_MAX_HEADS 128
#define SMLA_MAX_SPLITS 256
/* Device scratch held by the library for sparse_mla_decode_run_noalloc, per GPU (16 MiB) */
#define SMLA_NOALLOC_SCRATCH_BYTES (16u << 20)

typedef enum {
  SMLA_OK = 0,
  SMLA_ERR_NULL_ARG = 1,             /* a required pointer is NULL */
  SMLA_ERR_BAD_SHAPE = 2,            /* a size is negative, zero where it must not be, or inconsistent */
  SMLA_ERR_UNSUPPORTED = 3,          /* valid but unsupported: head count, format, mode, flag */
  SMLA_ERR_MISALIGNED = 4,           /* a pointer or a row stride breaks the alignment rule */
  SMLA_ERR_WORKSPACE_TOO_SMALL = 5,  /* workspace_bytes below what the plan asks for */
  SMLA_ERR_HIP = 6,                  /* the HIP runtime reported an error (no device, launch failure) */
  SMLA_ERR_BAD_PLAN = 7              /* the plan was not produced by sparse_mla_decode_plan */
} smla_status;

typedef enum { SMLA_KV_BF16 = 0, SMLA_KV_FP8_UE8M0 = 1, SMLA_KV_FP8_TENSOR = 2 } smla_kv_format;

/* LOGICAL: idx is a request-local position t; slot = page_table[row_req[r]][t / page_size]
 * * page_size + t % page_size (the block-table translation that the vLLM SM120 backend
 * performs before its kernel, prhub vllm#43477, key code excerpts: forward_mqa).
 * GLOBAL: idx already is the cache slot. */
typedef enum { SMLA_IDX_LOGICAL = 0, SMLA_IDX_GLOBAL = 1 } smla_index_mode;

enum {
  /* Write the per-chunk sink-free partials (partial_o, partial_lse) instead of the merged
   * output; out/lse are not written.  For callers that merge elsewhere. */
  SMLA_F_PARTIALS_ONLY = 1,
  /* Record the first out-of-range index in the workspace (see sparse_mla_read_index_error). */
  SMLA_F_CHECK_INDICES = 2,
  /* For batches whose rows hold very different numbers of entries (short contexts padded
   * with -1).  The run first counts each row's valid entries (those the decode keeps), gives
   * each row its own split count (one for most rows; up to the plan's S for rows far longer
   * than an even share of the work) and orders the (row, split) jobs longest first (two
   * small launches; workspace for 3 + S int32 per row); the decode then takes the jobs in
   * that order, a split row's chunks hold equal numbers of its valid entries instead of
   * equal ranges of positions, rows of one split write their output directly and only split
   * rows are merged.  The result is the same attention; the rounding of a split row may
   * differ from the positional split (LOGICAL and GLOBAL mode over the same entries still
   * agree bit for bit).  On rows of equal length it only adds cost.  Not with
   * SMLA_F_PARTIALS_ONLY (UNSUPPORTED): the documented partials are ranges of positions;
   * num_rows must be below 2^24 (BAD_SHAPE). */
  SMLA_F_BALANCE_ROWS = 4
};

typedef struct {
  int32_t num_rows;          /* R query rows (decode tokens); >= 0 */
  int32_t num_requests;      /* B requests; rows map to requests through row_req; >= 1 in LOGICAL mode */
  int32_t num_heads;         /* H query heads: a multiple of 16 in [16, 128] */
  int32_t topk;              /* K = index row stride in int32 elements; >= 4 and a multiple of 4
                                (16-byte aligned rows, as the page prhub vllm#43827 notes for
                                the FlashInfer sparse kernels, review highlights item 2) */
  int32_t page_size;         /* tokens per page; a power of two in [1, 1024] (>= 2 for FP8) */
  int32_t num_pages;         /* pages in kv_cache; >= 1 */
  int32_t max_pages_per_req; /* page_table row stride; >= 1 in LOGICAL mode */
  int32_t kv_format;         /* smla_kv_format */
  int32_t index_mode;        /* smla_index_mode */
  int32_t num_splits;        /* 0: the planner chooses; > 0: forced S (chunks of ceil(K/S) positions) */
  int32_t flags;             /* SMLA_F_* */
  float softmax_scale;       /* multiplies q.k; the sink lives in the same (scaled) logit domain */
  float kv_scale;            /* SMLA_KV_FP8_TENSOR: the one scale of every cache value (finite,
                                > 0); ignored for the other formats */
} smla_problem;

/* Host-side plan.  Copyable plain bytes; contents are private to the library. */
typedef struct {
  uint8_t opaque[256];
} smla_plan;

/* Choose the split count and launch shape for a problem and report the workspace size.
 * This is the decode's scheduler metadata: built on the host from shapes alone, so one plan
 * serves every step and every graph replay of a batch shape, with the work split derived
 * inside the library from the literal compute-unit total (prhub vllm#52164 "[Attention][DSA]
 * Take the native decode path for MTP=3 on SM90", implementation breakdown step 4 and design
 * highlight 3: graph-stable, preallocated scheduler metadata whose slot count the wrapper
 * derives from the plain SM count itself).  The split-KV decode it plans and the merge that
 * follows are the split path of prhub sglang#24692, implementation breakdown items 2-3.
 *   p               problem description (host memory, read only)
 *   num_cus         compute units of the device the run will use (the total, as the device
 *                   reports it); <= 0 queries the current HIP device (the only HIP call this
 *                   function makes).  Passing the count keeps the plan a pure host function.
 *   plan            output (host memory)
 *   workspace_bytes output: device bytes that sparse_mla_decode_run needs (0 when none)
 * Depends only on shapes and num_cus, never on data; no device memory is touched.
 * Errors: NULL_ARG, BAD_SHAPE, UNSUPPORTED, HIP (device query failed). */
smla_status sparse_mla_decode_plan(const smla_problem* p, int32_t num_cus, smla_plan* plan,
                                   size_t* workspace_bytes);

/* Number of splits S chosen by a plan (>= 1), or -1 for an invalid plan. */
int32_t sparse_mla_plan_num_splits(const smla_plan* plan);

/* Run the decode on `stream`: the sparse-MLA attention call of the serving engine's
 * forward_mqa, which consumes each token's top-k index list and writes the output of shape
 * [tokens, heads, kv_lora_rank] in q's dtype (prhub vllm#43477 "DSv4 and GLM-5.1 on Blackwell
 * SM120", key code excerpts: FlashInferMLASparseSM120Impl.forward_mqa), computing the
 * gather + dequant, tiled online softmax, sink and split merge of prhub sglang#24692
 * implementation breakdown items 2-3 as defined at the top of this header.  All pointers
 * are device pointers.
 *   q           bf16 [R][H][576]; 16-byte aligned
 *   kv_cache    num_pages pages in the layout above; 16-byte aligned
 *   indices     int32 [R][K]; -1 = empty; 16-byte aligned (K is a multiple of 4)
 *   row_req     int32 [R] request of each row (LOGICAL mode; may be NULL in GLOBAL mode)
 *   page_table  int32 [B][max_pages_per_req] page ids (LOGICAL mode; may be NULL in GLOBAL mode)
 *   sinks       fp32 [H] per-head sink logits, or NULL for no sink (-inf sinks are allowed)
 *   out         bf16 [R][H][512]                  (not written with SMLA_F_PARTIALS_ONLY)
 *   lse         fp32 [R][H] or NULL               (not written with SMLA_F_PARTIALS_ONLY)
 *   partial_o   fp32 [R][S][H][512]  only with SMLA_F_PARTIALS_ONLY, else NULL
 *   partial_lse fp32 [R][S][H]       only with SMLA_F_PARTIALS_ONLY, else NULL
 *   workspace   device scratch of at least the planned size (may be NULL when it is 0);
 *               256-byte aligned; its contents need not be initialised
 * R == 0 returns SMLA_OK without launching or checking pointers (empty tensors may
 * pass NULL).  No device-to-host traffic and no
 * allocation: the call can be captured in a HIP graph.
 * Errors: BAD_PLAN, NULL_ARG, MISALIGNED, WORKSPACE_TOO_SMALL, HIP. */
smla_status sparse_mla_decode_run(const smla_plan* plan, const void* q, const void* kv_cache,
                                  const int32_t* indices, const int32_t* row_req,
                                  const int32_t* page_table, const float* sinks, void* out,
                                  float* lse, float* partial_o, float* partial_lse,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* The same decode as sparse_mla_decode_run, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): it
 * takes no workspace.  A split plan's fp32 partials (and a balanced plan's row counts and
 * order, SMLA_F_BALANCE_ROWS) go to scratch the library holds, one
 * SMLA_NOALLOC_SCRATCH_BYTES array per GPU in the library's own device memory, reserved
 * when the library is loaded and kept until the process ends; no call allocates or frees
 * anything.  Arguments as for sparse_mla_decode_run, without partial_o, partial_lse and
 * the workspace.
 *   - Plans whose workspace exceeds SMLA_NOALLOC_SCRATCH_BYTES return
 *     SMLA_ERR_WORKSPACE_TOO_SMALL before anything else happens (raise the split count's
 *     ceiling differently: force fewer splits, or call sparse_mla_decode_run).
 *   - Plans with SMLA_F_PARTIALS_ONLY or SMLA_F_CHECK_INDICES return SMLA_ERR_UNSUPPORTED.
 *   - Every call on one GPU uses that GPU's one scratch array: calls that may overlap on a
 *     GPU (other streams, other host threads) race on it and give wrong results; calls in
 *     one stream are ordered and safe.  The scratch keeps the last call's contents; nothing
 *     in it needs to start at zero.
 * Errors: BAD_PLAN, UNSUPPORTED, WORKSPACE_TOO_SMALL, NULL_ARG, MISALIGNED, HIP. */
smla_status sparse_mla_decode_run_noalloc(const smla_plan* plan, const void* q, const void* kv_cache,
                                          const int32_t* indices, const int32_t* row_req,
                                          const int32_t* page_table, const float* sinks, void* out,
                                          float* lse, void* stream);

/* LSE-merge S sink-free partials and apply the sink once (the merge and sink steps that
 * follow the split decode on prhub sglang#24692, key files: flash_mla_sm120_triton.py).
 *   partial_o   fp32 [R][S][H][512], partial_lse fp32 [R][S][H] (natural log, -inf = empty)
 *   sinks       fp32 [H] or NULL;  out bf16 [R][H][512];  lse fp32 [R][H] or NULL
 * num_rows == 0 returns SMLA_OK without launching.  H need not be a multiple of 16 here
 * (1..1024); S in [1, SMLA_MAX_SPLITS].
 * Errors: NULL_ARG, BAD_SHAPE, MISALIGNED, HIP. */
smla_status sparse_mla_merge_partials(const float* partial_o, const float* partial_lse,
                                      int32_t num_rows, int32_t num_splits, int32_t num_heads,
                                      const float* sinks, void* out, float* lse, void* stream);

/* Write new tokens into the paged cache (the step before the decode path: the FP8 paged
 * cache with UE8M0 scales per 64 latent elements and a bf16 rope part of prhub vllm#43827,
 * motivation and key code excerpts; in-page addressing as on prhub sglang#24692,
 * implementation breakdown 2).
 *   latent    bf16 [num_tokens][512], rope bf16 [num_tokens][64]   (device, 16-byte aligned)
 *   slots     int32 [num_tokens]: the global slot (page * page_size + row) of each token;
 *             negative or >= num_pages * page_size: the token is skipped.  Slots must be
 *             distinct: for a repeated slot it is unspecified which token's bytes remain.
 *   kv_cache  the cache of the layout above, updated in place (caller-owned)
 * FP8: each 64-element group gets the scale byte e (value 2^(e-127)) of the smallest power
 * of two with 448 * 2^(e-127) >= the group's largest magnitude (e = 127 for an all-zero
 * group; clamped to [0, 254]) and codes = e4m3fn(x / 2^(e-127)) rounded to nearest, ties to
 * even; the rope is copied.  BF16: the 576 values are copied.  Non-finite inputs give
 * unspecified codes.  num_tokens == 0 returns SMLA_OK without launching.  No allocation;
 * asynchronous on `stream`.
 * Errors: NULL_ARG, BAD_SHAPE, UNSUPPORTED (format; FP8 with page_size < 2), MISALIGNED, HIP. */
smla_status sparse_mla_cache_store(const void* latent, const void* rope, const int32_t* slots,
                                   int32_t num_tokens, int32_t kv_format, int32_t page_size,
                                   int32_t num_pages, void* kv_cache, void* stream);

/* Indexer, the step that produces the index lists: FP8 paged MQA logits of every query
 * row over its context (the indexer's fp8_paged_mqa_logits on prhub sglang#24692,
 * implementation breakdown item 5; next_n rows of a request served natively, so each key
 * page is read once for all of them, per-row context lengths: prhub vllm#52164,
 * implementation breakdown items 1-5).  With e = e4m3fn decode:
 *   logits[r][t] = sum_h weights[r][h] * max(0, scale_t * sum_d e(q[r][h][d]) * e(code_t[d]))
 * for 0 <= t < min(row_len[r], width); positions t >= min(row_len[r], width) are not
 * written.  Positions are request-local and translated through page_table as on the decode
 * path; a position whose page id is outside [0, num_pages) gets -inf.
 *   q_codes   e4m3fn [R][64][128], R = num_requests * next_n rows, request-major (row
 *             b*next_n + i is row i of request b)                    (device, 16 B aligned)
 *   weights   fp32 [R][64] (any query scale folded in)                (device, 16 B aligned)
 *   key_cache num_pages pages of 132*page_size bytes: codes e4m3fn [page_size][128], then
 *             fp32 scales [page_size]; scales must be >= 0 (quantization scales)
 *   row_len   int32 [R]; page_table int32 [num_requests][max_pages]
 *   logits    fp32 [R][width] (caller-owned, 16 B aligned); width a multiple of 64,
 *             at most 2^28 (a row's bytes stay below 2^31), and max_pages * 64 >= width
 * Supported: num_heads = 64, page_size = 64, next_n 1..4.  No allocation; asynchronous.
 * Errors: UNSUPPORTED, BAD_SHAPE, NULL_ARG, MISALIGNED, HIP. */
smla_status sparse_mla_indexer_logits(const void* q_codes, const float* weights, const void* key_cache,
                                      const int32_t* row_len, const int32_t* page_table,
                                      int32_t num_requests, int32_t next_n, int32_t num_heads,
                                      int32_t page_size, int32_t num_pages, int32_t max_pages,
                                      int32_t width, float* logits, void* stream);

/* Top-k of the indexer logits (the selection that yields the decode path's index lists,
 * same passages as above): for each row r, with n = min(row_len[r], width), the topk
 * positions t < n of largest logits[r][t], a tie at the boundary going to the smaller
 * position, written to indices[r][0..topk) in ascending position order; with n <= topk,
 * positions 0..n-1 and then -1.  NaN logits give an unspecified selection.
 *   logits fp32 [rows][width] (16 B aligned, width a multiple of 4); row_len int32 [rows];
 *   indices int32 [rows][topk]
 * No allocation; asynchronous.  Errors: BAD_SHAPE, NULL_ARG, MISALIGNED, HIP. */
smla_status sparse_mla_indexer_topk(const float* logits, const int32_t* row_len, int32_t rows,
                                    int32_t width, int32_t topk, int32_t* indices, void* stream);

/* Once-per-step global index build: translate request-local top-k positions into global
 * cache slots, so that the decode calls of every layer in the step read them in
 * SMLA_IDX_GLOBAL mode without the block-table lookups (the once-per-step sparse index
 * build reused across layers: prhub vllm#43827, implementation breakdown 3; the translation
 * itself is vllm#43477's block-table conversion, key code excerpts: forward_mqa).
 *   slots[r][j] = page_table[row_req[r]][t / page_size] * page_size + t % page_size,
 *   t = indices[r][j]; -1 where the decode path would mask the entry (t < 0, the page
 *   index >= max_pages, a page id outside [0, num_pages), row_req outside [0, num_requests)).
 *   indices, slots int32 [rows][topk]; row_req int32 [rows];
 *   page_table int32 [num_requests][max_pages]  (device, caller-owned)
 * page_size a power of two <= 1024.  No allocation; asynchronous.
 * Errors: BAD_SHAPE, NULL_ARG, MISALIGNED, HIP. */
smla_status sparse_mla_translate_indices(const int32_t* indices, const int32_t* row_req,
                                        const int32_t* page_table, int32_t rows, int32_t topk,
                                        int32_t num_requests, int32_t max_pages, int32_t page_size,
                                        int32_t num_pages, int32_t* slots, void* stream);

/* Test helper: decode n cache slots (global slot numbers, device int32 [n]) into bf16
 * rows out[n][576] with a plain per-element reference decoder on the GPU (one thread per
 * 8 dims, direct loads).  It is NOT the decode kernel's gather: that one copies entries into
 * LDS with its own addressing and dequantizes them there, and is checked bit for bit
 * through sparse_mla_decode_run itself.  Slots outside [0, num_pages*page_size) give a zero
 * row.  The cache layout is the one at the top of this header.  For
 * SMLA_KV_FP8_TENSOR the row holds the code values e4m3fn(code[d]): the decode applies
 * kv_scale as two scalar factors, not per element.
 * Errors: NULL_ARG, BAD_SHAPE, UNSUPPORTED, MISALIGNED, HIP. */
smla_status sparse_mla_gather_debug(const void* kv_cache, int32_t kv_format, int32_t page_size,
                                    int32_t num_pages, const int32_t* slots, int32_t n, void* out,
                                    void* stream);

/* With SMLA_F_CHECK_INDICES: copy the two int32 words (row, position) of the first
 * out-of-range index recorded in `workspace` by the last run into host memory
 * `row_pos` (-1, -1 when none).  Synchronises `stream`; for tests and debugging only.
 * Errors: BAD_PLAN, NULL_ARG, HIP. */
smla_status sparse_mla_read_index_error(const smla_plan* plan, const void* workspace,
                                        int32_t* row_pos, void* stream);

/* Static text for a status code (never NULL).  Takes any int32: a value that is not an
 * smla_status gives "unknown status". */
const char* sparse_mla_status_string(int32_t status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t sparse_mla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_MLA_H_ */
