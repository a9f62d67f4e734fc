/*
 * libsparsemla - sparse MLA decode with an index-driven KV gather, for
 * AMD Instinct MI355X (gfx950).  C ABI: plain pointers, sizes and HIP
 * streams; no C++ or framework types cross this boundary.
 *
 * The operation (FlashInfer "trtllm_batch_decode_sparse_mla_dsv4",
 * introduction and parameters): every query token t carries H heads of 512
 * dims (448 NoPE then 64 RoPE, per the "q" parameter of FlashInfer
 * "cake_sparse_mla_sm120_dsv4_nvfp4_decode").  It attends only to the KV
 * rows named by row t of an int32 table: columns 0..127 index the SWA pool,
 * the other columns index the compressed pool, -1 masks a slot, and
 * topk_lens[t] (which counts the 128 SWA columns) truncates the row.  Each
 * KV row is one 512-d latent vector shared by every head as both key and
 * value.  For head h, with s_c = bmm1_scale * <q[t,h,:], row_c> over the
 * active slots c:
 *
 *   Z          = sum_c e^{s_c} + e^{sinks[h]}          (sink term if given)
 *   out[t,h,:] = bf16( bmm2_scale * sum_c e^{s_c} row_c / Z )
 *   out_lse    = lse_scale * log2(Z)
 *
 * Readings where the pages are silent: log2(e) is applied inside the
 * library (bmm1_scale is the plain softmax scale times any FP8 scales, as
 * the vLLM DeepseekV4FlashInferMLAAttention listing builds it); the sink is
 * a natural-log logit that bmm1_scale does not multiply; out_lse includes
 * the sink term; a token with no active slot gets out = 0 and
 * out_lse = -inf (or lse_scale * sink * log2(e) with a sink); seq_lens and
 * cum_seq_lens_q do not change the result (the table is authoritative).
 *
 * Conventions for every entry point:
 *  - Ownership: the caller owns every buffer.  The library keeps no
 *    per-call state, allocates no device memory and never synchronises
 *    (except sparse_mla_get_device_error, which says so).
 *  - Errors: each call returns an int status, SMLA_OK (0) on success.
 *    Argument checks happen on the host before anything is launched; a
 *    rejected call launches nothing.  Nothing is ever copied to fix a
 *    layout: a wrong layout is an error (FlashInfer
 *    "msa_sparse_decode_attention", parameter "out").
 *  - Device pointers must point to memory of the device that is current
 *    on the calling thread, and "stream" must belong to that device.
 */
#ifndef SPARSEMLA_H_
#define SPARSEMLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t without including HIP headers; pass a hipStream_t (or 0 for
 * the null stream). */
typedef struct ihipStream_t* smla_stream_t;

/* ---- status codes --------------------------------------------------- */
#define SMLA_OK                      0
#define SMLA_ERR_INVALID_ARG         1  /* null pointer, bad size or stride */
#define SMLA_ERR_UNSUPPORTED_DTYPE   2  /* dtype pair (q/kv) not BF16/BF16, FP8/FP8,
                                           BF16/FP8 or BF16/PACKED_FP8_584 */
#define SMLA_ERR_UNSUPPORTED_SHAPE   3  /* H not 64 or 128 */
#define SMLA_ERR_WORKSPACE_TOO_SMALL 4
#define SMLA_ERR_MISALIGNED          5  /* see the alignment rules below */
#define SMLA_ERR_BAD_PLAN            6  /* plan fields inconsistent with the call */
#define SMLA_ERR_HIP                 7  /* a HIP runtime call or launch failed */
#define SMLA_ERR_TOO_LARGE           8  /* sparse_mla_decode_noalloc: the call needs
                                           more than SMLA_NOALLOC_SCRATCH_BYTES */

/* ---- element types -------------------------------------------------- */
#define SMLA_DTYPE_BF16       0   /* bfloat16 */
#define SMLA_DTYPE_FP8_E4M3FN 1   /* OCP FP8 E4M3FN, per-tensor scaled */
/* KV pools only, with BF16 q: packed block-scaled FP8 rows of 584 bytes
 * (FlashInfer trtllm_batch_decode_sparse_mla_dsv4, introduction,
 * packed-backend paragraph and parameter "swa_kv_cache": 584 bytes per token
 * of uint8; vLLM DeepseekV4FlashInferMLAAttention, class comment on
 * use_flashmla_fp8_layout: UE8M0 block-scaled FP8).  The byte order is this
 * library's reading, the pages giving only size and family:
 *   bytes [0, 448)   NoPE dims 0..447 as OCP E4M3FN codes,
 *   bytes [448, 576) RoPE dims 448..511 as BF16, little-endian,
 *   bytes [576, 584) 8 UE8M0 scale bytes e_j (2^(e_j - 127)), byte j
 *                    scaling NoPE dims [56 j, 56 j + 56).
 * Scale bytes 1..254 with every scaled NoPE value in BF16's normal range
 * are decoded exactly; 0 (2^-127) and 255 (NaN) are accepted as their UE8M0
 * values but lie outside the tested range.  The row stride
 * (pool_row_stride) is counted in bytes, 0 meaning 584, and must be a
 * multiple of 8. */
#define SMLA_DTYPE_PACKED_FP8_584 2
#define SMLA_PACKED_ROW_BYTES 584

/* ---- flags ---------------------------------------------------------- */
/* Check every active index on the device and record the first violation
 * (an index outside [0, rows) of its pool other than -1, or a topk_len
 * outside [0, K]) in the workspace's error block; read it back with
 * sparse_mla_get_device_error.  Violating slots are skipped either way:
 * an out-of-range index is never dereferenced, with or without the flag. */
#define SMLA_FLAG_VALIDATE_INDICES 1u
/* A check for races in the kernels' tile pipeline, not a production path:
 * every step of the pipeline (the row loads of a tile, the S^T products, the
 * O^T products and softmax) completes, and all waves of the workgroup meet,
 * before the next step starts.  The arithmetic is unchanged, so the results
 * must be bitwise identical to the same call without the flag; a difference
 * means that overlapping steps disturbed each other.  Slower.  Combined-table
 * calls only (sparse_mla_decode, sparse_mla_decode_noalloc); with the
 * two-segment or page-table forms, or sparse_mla_gather_only, the call
 * returns SMLA_ERR_INVALID_ARG.  Any flag bit not defined here is
 * SMLA_ERR_INVALID_ARG too. */
#define SMLA_FLAG_SERIAL_PIPELINE 2u

/* Device-side error codes reported by sparse_mla_get_device_error. */
#define SMLA_DEVERR_NONE          0
#define SMLA_DEVERR_INDEX_RANGE   1
#define SMLA_DEVERR_TOPK_LEN      2

#define SMLA_HEAD_DIM     512
#define SMLA_SWA_COLUMNS  128
#define SMLA_MAX_SPLITS   64   /* hard cap of any plan (the planner's default cap is 16) */

/* Split-K plan (FlashInfer "cake_sparse_mla_sm120_dsv4_nvfp4_decode":
 * the resolved plan {head_tiles, num_splits, chunks_per_block}).  Table
 * columns are cut into chunks of chunk_cols; split s covers columns
 * [s*chunks_per_split*chunk_cols, (s+1)*chunks_per_split*chunk_cols).  A
 * split whose columns are all inactive yields an empty partial.  A plan
 * passed to a decode call must have 1 <= num_splits <= SMLA_MAX_SPLITS,
 * chunk_cols and chunks_per_split >= 1, K equal to the call's K, span
 * num_splits * chunks_per_split * chunk_cols columns with
 * K <= span <= SMLA_MAX_PLAN_COLUMNS, and head_tiles 1, or 2 at H=128;
 * otherwise the call returns SMLA_ERR_BAD_PLAN. */
#define SMLA_MAX_PLAN_COLUMNS (1 << 30)
typedef struct smla_plan {
  int32_t num_splits;        /* S >= 1; S == 1 writes out/out_lse directly */
  int32_t head_tiles;        /* 1: one workgroup covers all heads; 2 (H=128
                                only): each token runs as two 64-head
                                halves, each gathering the token's rows
                                (the second read mostly from L2); same
                                workspace, same outputs up to rounding */
  int32_t chunk_cols;        /* columns per chunk */
  int32_t chunks_per_split;  /* consecutive chunks per split */
  int32_t num_chunks;        /* ceil(K / chunk_cols) */
  int32_t K;                 /* table width the plan was made for */
  int32_t reserved[2];
} smla_plan;

/* Arguments of sparse_mla_decode.  Field names follow the pages' statement
 * of the problem (FlashInfer trtllm_batch_decode_sparse_mla_dsv4
 * parameters).  All pointers are device pointers unless noted. */
typedef struct smla_decode_args {
  int32_t T;                   /* query tokens (flattened over requests); 0 = no-op */
  int32_t H;                   /* heads per token: 64 or 128 (callers zero-pad,
                                  vLLM get_padded_num_q_heads) */
  int32_t K;                   /* table width (columns) >= 1 */
  int32_t q_dtype;             /* SMLA_DTYPE_BF16 or SMLA_DTYPE_FP8_E4M3FN */
  const void* q;               /* [T, H, 512] contiguous, 16-B aligned */
  const void* swa_pool;        /* [swa_rows, row_stride] rows of 512 elements */
  int64_t swa_rows;
  const void* compressed_pool; /* [compressed_rows, row_stride]; may be NULL
                                  only if K <= 128 */
  int64_t compressed_rows;
  int32_t kv_dtype;            /* dtype of both pools (SMLA_DTYPE_*) */
  int32_t flags;               /* SMLA_FLAG_* */
  int64_t pool_row_stride;     /* elements between rows of both pools; 0 means
                                  512 (bytes, and 0 means 584, for
                                  SMLA_DTYPE_PACKED_FP8_584 rows).  A pool of one KV head is the same
                                  bytes in HND and NHD layouts, so a paged
                                  [pages, page_size, 512] pool is passed as
                                  flat rows row = page * page_size + offset */
  const int32_t* indices;      /* [T, index_row_stride], first K columns used */
  int64_t index_row_stride;    /* 0 means K */
  const int32_t* topk_lens;    /* [T] active column count (<= K) or NULL = K */
  const int32_t* seq_lens;     /* [num_requests] or NULL; accepted, unused by the math */
  const int32_t* cum_seq_lens_q; /* [num_requests + 1] or NULL; accepted, unused by the math */
  int32_t num_requests;
  int32_t reserved0;
  const float* sinks;          /* [H] fp32 or NULL */
  float bmm1_scale;            /* QK scale: sm_scale (* q_scale * kv_scale for FP8);
                                  must be finite and > 0 (a softmax scale), and
                                  bmm1_scale * log2(e) must be a finite float */
  float bmm2_scale;            /* VO scale: 1 (or kv_scale for FP8 pools); finite */
  float lse_scale;             /* multiplier of the base-2 LSE, 1 by default; finite */
  int32_t reserved1;
  void* out;                   /* [T, H, 512] BF16 contiguous, 16-B aligned */
  float* out_lse;              /* [T, H] fp32 or NULL */
  void* workspace;             /* device scratch, 256-B aligned; may be NULL
                                  when sparse_mla_workspace_size() is 0 */
  size_t workspace_bytes;
} smla_decode_args;

/* Choose the split-K plan from shapes only (host-only, deterministic, no
 * device work; FlashInfer cake_* "num_splits"/"max_splits" and the adaptive
 * chunking of msa_sparse_decode_attention "force_fused": one chunk per
 * block at low batch, a single chunk at high batch).
 *   max_splits <= 0 selects the default cap 16; num_splits_override > 0
 *   forces S = clamp(override, 1, min(num_chunks, SMLA_MAX_SPLITS));
 *   num_cus <= 0 queries the current device's compute-unit count once and
 *   caches it per device.
 *   Every row format is widened and multiplied on the BF16 MFMA, so a
 *   split's time follows its row count, not its bytes.  The row format
 *   changes the plan only at H=64, where BF16 rows (gathered straight into
 *   LDS) cost half as much as rows staged through registers (FP8, packed).  At H=128 the planner also weighs head tiles
 *   (head_tiles = 2, with its own split count) against one workgroup per
 *   token and split: they pay at small and mid T, where the grid is short
 *   of workgroups; an override of num_splits keeps head_tiles = 1.
 * Returns SMLA_ERR_INVALID_ARG for T < 0, K < 1, K > SMLA_MAX_PLAN_COLUMNS
 * or a NULL out_plan,
 * SMLA_ERR_UNSUPPORTED_SHAPE for H not in {64,128},
 * SMLA_ERR_UNSUPPORTED_DTYPE for a (q, kv) pair the decode does not take,
 * SMLA_ERR_HIP if the device query fails. */
int sparse_mla_plan_splits(int T, int H, int K, int q_dtype, int kv_dtype,
                           int max_splits, int num_splits_override,
                           int num_cus, smla_plan* out_plan);

/* Workspace bytes sparse_mla_decode needs for this plan: a 256-B error
 * block, then (when S > 1) mid_lse [T, H, S] fp32 and mid_out
 * [T, H, S, 512] BF16 (FlashInfer cake_* "mid_out"/"mid_lse").  Returns 0
 * when S == 1 and validation is off (pass flags), or (size_t)-1 on bad
 * arguments. */
size_t sparse_mla_workspace_size(const smla_plan* plan, int T, int H,
                                 int flags);

/* Byte offsets of mid_lse and mid_out inside a workspace laid out for
 * (plan, T, H); for callers that want to inspect the partials. */
int sparse_mla_workspace_layout(const smla_plan* plan, int T, int H,
                                size_t* mid_lse_offset,
                                size_t* mid_out_offset);

/* Run the decode asynchronously on "stream": the split kernel, then the
 * combine kernel when plan->num_splits > 1.  plan == NULL plans
 * internally (defaults, current device).  No allocation and no
 * synchronisation, so the call can be captured into a HIP graph (FlashInfer
 * msa_sparse_decode_attention "workspace": host arithmetic only before the
 * launches).  Alignment rules (SMLA_ERR_MISALIGNED): q, out, both pools
 * and pool_row_stride * element size are multiples of 16 bytes; the
 * workspace is 256-B aligned.  Indices at columns >= topk_lens[t] are
 * never read as rows.  A bmm1_scale that is not a positive finite number,
 * or a non-finite bmm2_scale or lse_scale, gives SMLA_ERR_INVALID_ARG. */
int sparse_mla_decode(const smla_decode_args* args, const smla_plan* plan,
                      smla_stream_t stream);

/* Scratch bytes of sparse_mla_decode_noalloc, per GPU. */
#define SMLA_NOALLOC_SCRATCH_BYTES (64u << 20)

/* sparse_mla_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, plan, kernels and results as
 * sparse_mla_decode, except that the caller passes no workspace
 * (args->workspace must be NULL and args->workspace_bytes 0) and
 * SMLA_FLAG_VALIDATE_INDICES is not offered (SMLA_ERR_INVALID_ARG
 * otherwise).  When the plan splits, the split partials (the layout
 * sparse_mla_workspace_size/_layout describe) go to a static device array of
 * SMLA_NOALLOC_SCRATCH_BYTES inside the library instead; a call needing more
 * than that returns SMLA_ERR_TOO_LARGE and launches nothing.  Each GPU the
 * library runs on holds its own copy of that array, from the library's
 * first use on that GPU until the process ends.  Nothing is allocated: no
 * hipMalloc, hipFree or allocating library routine is called.  All calls on
 * one GPU share its array, so calls that overlap in time on one GPU (on
 * different streams, or from different threads) race and give undefined
 * results; calls ordered on one stream are safe.  The first call on a
 * device looks up the array's address (not a stream operation); make that
 * first call outside graph capture.  Asynchronous on "stream". */
int sparse_mla_decode_noalloc(const smla_decode_args* args, const smla_plan* plan,
                              smla_stream_t stream);

/* The two-segment form of the token tables (FlashInfer
 * "trtllm_batch_decode_sparse_mla_dsv4", introduction (packed-backend
 * paragraph) and parameters "swa_topk_lens", "extra_sparse_indices",
 * "extra_sparse_topk_lens"; FlashInfer "cake_sparse_mla_sm120_dsv4_nvfp4_decode",
 * parameters "indices"/"topk_length" and "extra_indices"/"extra_topk_length"):
 * token t's SWA rows are named by an SWA table with its own active length,
 * its compressed rows by an extra table with its own length, and the
 * softmax runs over the active slots of both.  -1 masks a slot in either
 * table; columns at or past a table's length are never read as rows.
 * Device pointers; the caller owns them. */
typedef struct smla_segments {
  const int32_t* swa_indices;     /* [T, swa_row_stride] rows of swa_pool; NULL iff
                                     swa_width == 0 */
  int64_t swa_row_stride;         /* elements; 0 means swa_width */
  const int32_t* swa_topk_lens;   /* [T] active SWA columns in [0, swa_width], or
                                     NULL = swa_width */
  const int32_t* extra_indices;   /* [T, extra_row_stride] rows of compressed_pool;
                                     NULL iff extra_width == 0 */
  int64_t extra_row_stride;       /* elements; 0 means extra_width */
  const int32_t* extra_topk_lens; /* [T] active extra columns in [0, extra_width],
                                     or NULL = extra_width */
  int32_t swa_width;              /* >= 0 */
  int32_t extra_width;            /* >= 0; swa_width + extra_width == args->K */
} smla_segments;

/* sparse_mla_decode with the tables in two segments.  args->K is the total
 * width swa_width + extra_width: the split plan and the split partials cut
 * that row, SWA column c being column c and extra column j being column
 * swa_width + j (also the column a validation error reports).
 * args->indices and args->topk_lens must be NULL and args->index_row_stride
 * is ignored; every other field, the plan, the workspace and the outputs
 * are exactly as for sparse_mla_decode.  swa_pool is required when
 * swa_width > 0, compressed_pool when extra_width > 0.  A length outside its
 * range is clamped (and reported in validate mode as
 * SMLA_DEVERR_TOPK_LEN).  Returns SMLA_ERR_INVALID_ARG for a NULL seg,
 * widths that do not add up to K, a table missing for a non-zero width, a
 * row stride below its width, or non-NULL args->indices / topk_lens;
 * otherwise as sparse_mla_decode.  Asynchronous, no allocation, graph
 * capturable. */
int sparse_mla_decode_segments(const smla_decode_args* args,
                               const smla_segments* seg, const smla_plan* plan,
                               smla_stream_t stream);

/* The page-table form (FlashInfer "trtllm_batch_decode_sparse_mla_dsv4",
 * introduction (HCA paragraph: the SWA stream takes physical token rows,
 * the compressed stream physical page IDs) and parameters
 * "hca_swa_indices", "swa_topk_lens", "hca_compressed_block_tables",
 * "sparse_topk_lens", "hca_seq_lens" and "hca_sparse_indices_format" (the
 * canonical expansion page_id * page_size + page_offset)): token t attends
 * to the first swa_topk_lens[t] rows of its window row and to the first
 * args->topk_lens[t] - swa_topk_lens[t] slots of the page expansion of its
 * block-table row, compressed slot j being row
 * block_tables[t][j / page_size] * page_size + j % page_size of
 * compressed_pool.  A -1 window entry masks its slot; a page whose rows
 * fall outside the pool is skipped (reported in validate mode).  Device
 * pointers; the caller owns them. */
typedef struct smla_paged {
  const int32_t* swa_indices;     /* [T, swa_row_stride] window rows of swa_pool
                                     (NULL iff swa_width == 0) */
  int64_t swa_row_stride;         /* elements; 0 means swa_width */
  const int32_t* swa_topk_lens;   /* [T] visible window rows in [0, swa_width], or
                                     NULL = swa_width */
  const int32_t* block_tables;    /* [T, block_table_stride] page IDs of
                                     compressed_pool (NULL iff max_pages == 0) */
  int64_t block_table_stride;     /* elements; 0 means max_pages */
  const int32_t* hca_seq_lens;    /* [num_requests] or NULL; accepted, unused by the
                                     math (a scheduling hint on the pages) */
  int32_t swa_width;              /* >= 0 (128 on the pages) */
  int32_t max_pages;              /* >= 0 */
  int32_t page_size;              /* rows per compressed page, >= 1 */
  int32_t reserved;
} smla_paged;

/* sparse_mla_decode with the page-table form.  args->K must be
 * swa_width + max_pages * page_size (window columns first, then compressed
 * slots: the row the split plan cuts and validation errors report);
 * args->indices must be NULL; args->topk_lens is the visible window +
 * compressed slot count (NULL = every slot; a count below the window or
 * beyond the table is clamped and, in validate mode, reported as
 * SMLA_DEVERR_TOPK_LEN, as is a window length outside [0, swa_width]).
 * Everything else as sparse_mla_decode.  Returns SMLA_ERR_INVALID_ARG for a
 * NULL pg, a bad width, page count or page size, a K that does not match,
 * a missing table or pool for a non-zero width, a row stride below its
 * width, or a non-NULL args->indices.  Asynchronous, no allocation, graph
 * capturable. */
int sparse_mla_decode_paged(const smla_decode_args* args, const smla_paged* pg,
                            const smla_plan* plan, smla_stream_t stream);

/* Combined index table from decode metadata: the step before the decode in
 * vLLM's DeepSeek-V4 FlashInfer attention
 * ("DeepseekV4FlashInferMLAAttention._build_sparse_index_metadata"), whose
 * result is the "sparse_indices" / "sparse_topk_lens" pair of FlashInfer
 * "trtllm_batch_decode_sparse_mla_dsv4".  Row t of out_indices is the
 * token's SWA row followed by its compressed entries:
 *   out[t][c]             = swa_indices[t][c]         for c < swa_width,
 *   out[t][swa_width + j] = compressed entry j, translated, for j < n2(t),
 *                           and -1 for n2(t) <= j < comp_width,
 * with n2(t) = comp_topk_lens[t] clamped to [0, comp_width] (comp_width when
 * NULL) and out_topk_lens[t] = swa_width + n2(t).  A negative entry gives
 * -1.  With comp_local != 0 an entry is a position p within the token's
 * request (the ratio-4 top-k positions) and becomes, by the canonical page
 * expansion of the FlashInfer page ("hca_sparse_indices_format"),
 *   block_tables[req][p / page_size] * page_size + p % page_size,
 * page_size being the compressed rows per block (the KV block size divided
 * by the compress ratio, as vLLM computes compressed_block_size) and req =
 * token_to_req[t] (NULL: t); otherwise it is a global row and is copied
 * (ratio 128, with "c128a_decode_topk_lens" as comp_topk_lens).  A position
 * whose page index is >= max_blocks, whose page ID is negative or whose row
 * exceeds INT32_MAX gives -1.  A token with valid_tokens[t] == 0, or (local
 * form) a request index outside [0, num_requests), gets an all -1 row and
 * length 0.  If err is not NULL it is cleared by the call and receives the
 * first untranslatable entry (SMLA_DEVERR_INDEX_RANGE, token, column; column
 * -1 for a bad request index); read it with sparse_mla_get_device_error.
 * Device pointers; the caller owns them. */
typedef struct smla_build_args {
  int32_t T;                       /* tokens, >= 0 */
  int32_t swa_width;               /* >= 0 (128 on the pages) */
  int32_t comp_width;              /* >= 0; swa_width + comp_width >= 1 */
  int32_t comp_local;              /* 1: request-local positions, 0: global rows */
  const int32_t* swa_indices;      /* [T, swa_row_stride] (NULL iff swa_width == 0) */
  int64_t swa_row_stride;          /* elements; 0 means swa_width */
  const int32_t* comp_indices;     /* [T, comp_row_stride] (NULL iff comp_width == 0) */
  int64_t comp_row_stride;         /* elements; 0 means comp_width */
  const int32_t* comp_topk_lens;   /* [T] or NULL */
  const int32_t* block_tables;     /* [num_requests, block_table_stride] page IDs
                                      (local form only) */
  int64_t block_table_stride;      /* elements; 0 means max_blocks */
  int32_t max_blocks;              /* >= 1 (local form) */
  int32_t page_size;               /* compressed rows per block, >= 1 (local form) */
  int32_t num_requests;            /* >= 1 (local form) */
  int32_t reserved;
  const int32_t* token_to_req;     /* [T] or NULL */
  const int32_t* valid_tokens;     /* [T] (0 = padding token) or NULL */
  int32_t* out_indices;            /* [T, out_row_stride] */
  int64_t out_row_stride;          /* elements; 0 means swa_width + comp_width */
  int32_t* out_topk_lens;          /* [T] */
  int32_t* err;                    /* 16-byte device error block, or NULL */
} smla_build_args;

/* Build the combined table (see smla_build_args).  Returns
 * SMLA_ERR_INVALID_ARG for a NULL args, negative sizes, a zero total width,
 * a missing table for a non-zero width, a missing output, a row stride below
 * its width, or (local form) a missing block table or max_blocks, page_size
 * or num_requests below 1; SMLA_ERR_MISALIGNED for a pointer that is not
 * 4-byte aligned.  T = 0 does nothing.  Asynchronous on "stream", no
 * allocation, graph capturable (the error block is cleared by a kernel). */
int sparse_mla_build_indices(const smla_build_args* args, smla_stream_t stream);

/* Measurement aid (not part of the method): run only the table compaction
 * and the row gather of sparse_mla_decode on the same arguments and plan,
 * with no arithmetic and no output, to give the attainable gathered-row
 * bandwidth on these exact tables (a companion pure-gather benchmark).
 * Same argument checks as sparse_mla_decode except that out, out_lse and
 * the workspace are not used, and the plan's head_tiles is ignored (the
 * gather has no heads; each token's rows are gathered once); only H = 128
 * with BF16 q and rows is supported (else SMLA_ERR_UNSUPPORTED_SHAPE /
 * _DTYPE).  Asynchronous on "stream"; no allocation. */
int sparse_mla_gather_only(const smla_decode_args* args, const smla_plan* plan,
                           smla_stream_t stream);

/* Merge split partials (FlashInfer cake_* "mid_out"/"mid_lse" and the
 * combine of msa_sparse_decode_attention "force_fused"; a non-finite
 * lse_scale gives SMLA_ERR_INVALID_ARG):
 *   mid_out [T, H, split_stride, 512] BF16 and mid_lse [T, H, split_stride]
 *   fp32 hold, for splits s < S, a normalised partial output (bmm2 already
 *   applied) and its base-2 LSE without sink or lse_scale (-inf = empty).
 *   out [T, H, 512] BF16 and out_lse [T, H] (or NULL) receive the merge,
 *   with the sink (if sinks != NULL) added once.
 * 1 <= S <= split_stride, S <= SMLA_MAX_SPLITS, H in {64,128}. */
int sparse_mla_combine(const void* mid_out, const float* mid_lse, int T,
                       int H, int S, int split_stride, const float* sinks,
                       float lse_scale, void* out, float* out_lse,
                       smla_stream_t stream);

/* Read the device error block of a workspace used with
 * SMLA_FLAG_VALIDATE_INDICES.  SYNCHRONISES "stream".  *code receives an
 * SMLA_DEVERR_* value, *token and *column the first violation found (or
 * -1).  Any of the output pointers may be NULL. */
int sparse_mla_get_device_error(const void* workspace, smla_stream_t stream,
                                int32_t* code, int32_t* token,
                                int32_t* column);

/* Static description of a status code. */
const char* sparse_mla_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPARSEMLA_H_ */
