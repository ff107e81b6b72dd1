/*
 * sfmla.h — C ABI of the MI355X (gfx950) shared-KV sparse flash MLA attention
 * library (libsfmla.so).
 *
 * The operation (sparse_flash_mla API page, 功能说明): for every query row,
 *
 *     O   = softmax(Q . K~^T . softmax_scale) . V~          (K~ = V~)
 *     LSE = log sum exp(S - max S) + max S,   S = Q . K~^T . softmax_scale
 *
 * where K~ is the concatenation of (a) rows of the original KV `ori_kv` picked
 * by a mask rule (no mask / right-down causal / sliding band) or by a TopK
 * index list, and (b) rows of the compressed KV `cmp_kv` picked by a TopK
 * index list (CSA) or all causally visible ones (HCA).  An optional per-head
 * sink adds one logit with zero value to each head's softmax normaliser.  The
 * token-wise TopK form over one KV with a 64-dim rope tail and a separate or
 * aliased V (SparseFlashAttention page) and the INT8 / FP8-E4M3 per-128-tile
 * packed rows (kv_quant_sparse_flash_attention blog, packed Key layout) are
 * the original-KV side with a TopK list.
 *
 * Call pattern (sparse_flash_mla API page, 功能说明 typical flow): build the
 * split plan with sfmla_metadata() from the same parameters, then call
 * sfmla_forward() with that plan.  The forward merges the partial results of
 * the KV splits it plans itself (the FLASH_DECODE split); sfmla_combine() is
 * the same LSE merge for partial results a caller produced over disjoint
 * parts of a row set (e.g. KV shards held by different devices).  A plan built
 * from other parameters is rejected on the device (outputs become NaN and
 * *status is set), because the host never reads device memory.
 *
 * Conventions for every entry point:
 *   - All pointers in sfmla_lengths / sfmla_tensors and the metadata and
 *     workspace buffers are DEVICE pointers owned by the caller; the library
 *     allocates no device memory and keeps no state besides a thread-local
 *     error string.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*); nothing
 *     synchronises, so calls can be captured in a HIP graph.
 *   - Every rule decidable from the parameters is checked on the host before
 *     anything is launched; on failure the function returns a nonzero status
 *     and sfmla_last_error() describes the rule.  Tensor *values* (lengths,
 *     indices, block-table entries) are the caller's responsibility, as on the
 *     pages (约束说明: values are user-guaranteed); gathered rows are
 *     nevertheless bounds-checked against the pool sizes given here, and an
 *     out-of-range row is skipped and reported through `status`.
 *   - Size limits of this implementation, also checked on the host: a query
 *     row's list (as bounded by the parameters) holds at most 4096 x 2048
 *     rows, and one query row's split partials stay below 2^31 bytes.
 *   - bf16 tensors hold IEEE bfloat16 values; fp32 is IEEE binary32.
 */
#ifndef SFMLA_H
#define SFMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SFMLA_VERSION "0.1.0"

typedef enum sfmla_status {
  SFMLA_OK = 0,
  SFMLA_ERR_INVALID_ARGUMENT = 1, /* a shape / attribute rule is violated      */
  SFMLA_ERR_UNSUPPORTED = 2,      /* valid on the pages, not built here        */
  SFMLA_ERR_BUFFER_TOO_SMALL = 3, /* metadata or workspace smaller than needed */
  SFMLA_ERR_LAUNCH = 4,           /* the HIP runtime refused a launch          */
  SFMLA_ERR_METADATA = 5          /* device status: plan built from other params */
} sfmla_status;

/* device status word bits (sfmla_tensors.status) */
#define SFMLA_STATUS_METADATA_MISMATCH 1
#define SFMLA_STATUS_ROW_OUT_OF_RANGE 2
#define SFMLA_STATUS_LIST_TOO_LONG 4   /* a row's list exceeds what max_seqlen_* / topk allow */

/* layouts (API page 参数说明 layout_q / layout_kv; PA_BBND, PA_ND and PA_BSND
 * on the different pages name the same paged layout) */
#define SFMLA_LAYOUT_BSND 0
#define SFMLA_LAYOUT_TND 1
#define SFMLA_LAYOUT_PA_BSND 2

/* KV storage formats */
#define SFMLA_KV_BF16 0
#define SFMLA_KV_INT8_PACKED 1     /* 512 int8 codes, rope bf16, 4 fp32 scales */
#define SFMLA_KV_FP8_E4M3_PACKED 2 /* 512 OCP E4M3FN codes, rope bf16, 4 scales */
#define SFMLA_KV_FP16 3            /* IEEE float16 q, kv (and V) and attention_out:
                                      the pages' other 16-bit type, shared by
                                      q and kv (SparseFlashAttention README,
                                      约束说明; API page 参数说明 ori_kv)  */

/* mask modes (API page 参数说明 ori_mask_mode / cmp_mask_mode) */
#define SFMLA_MASK_NONE 0
#define SFMLA_MASK_CAUSAL 3 /* right-down causal */
#define SFMLA_MASK_BAND 4   /* sliding window [p - win_left, p + win_right]  */

/*
 * Operator parameters.  No field has a default: the caller fills every one
 * (the pages' two entry points have different defaults for the mask fields,
 * API page 函数原型 note, so nothing is inferred).
 */
typedef struct sfmla_params {
  int32_t num_heads_q;   /* 1..128                                            */
  int32_t num_heads_kv;  /* must be 1                                         */
  int32_t head_dim;      /* must be 512 (nope width; also the output width)   */
  int32_t rope_head_dim; /* 0 or 64: extra q/k dims (q last dim = 512 + rope) */
  int32_t batch_size;    /* b > 0                                             */
  int32_t layout_q;      /* SFMLA_LAYOUT_BSND or _TND                         */
  int32_t layout_kv;     /* SFMLA_LAYOUT_BSND, _TND or _PA_BSND; non-paged
                            layouts must equal layout_q                       */
  int32_t q_s;           /* BSND: q sequence dim; TND: 0                      */
  int32_t q_t;           /* query rows: b*q_s (BSND) or total tokens (TND)    */
  int32_t ori_kv_s;      /* BSND: ori_kv sequence dim; else 0                 */
  int32_t cmp_kv_s;      /* BSND: cmp_kv sequence dim; else 0                 */
  int32_t ori_block_size;   /* PA: tokens per ori block (1..1024); else 0     */
  int32_t cmp_block_size;   /* PA: tokens per cmp block (1..1024); else 0     */
  int32_t ori_block_table_cols; /* PA: entries per ori block-table row        */
  int32_t cmp_block_table_cols; /* PA: entries per cmp block-table row        */
  int64_t ori_kv_rows;   /* physical rows in the ori pool (all blocks),
                            < 2^31 - 1 (row ids are 31-bit on the device)   */
  int64_t cmp_kv_rows;   /* physical rows in the cmp pool (0 if none),
                            < 2^31 - 1                                       */
  int32_t max_seqlen_q;      /* > 0                                           */
  int32_t max_seqlen_ori_kv; /* > 0: longest ori length of any batch          */
  int32_t max_seqlen_cmp_kv; /* longest cmp length (0 without cmp_kv)         */
  int32_t ori_topk;      /* 0: window rule; > 0: TopK list over ori_kv        */
  int32_t cmp_topk;      /* 0: all visible cmp rows (HCA); > 0: CSA list      */
  int32_t ori_sparse_block_size; /* tokens per ori TopK entry: 1 token-wise;
                            2..128 (power of two) block-wise, entry v selecting
                            tokens v*s .. v*s+s-1 (SparseFlashAttention README,
                            参数说明 sparseBlockSize); must divide ori_block_size
                            under PA; 1 when ori_topk is 0                    */
  int32_t cmp_ratio;     /* >= 1 (1 without cmp_kv)                           */
  int32_t ori_mask_mode; /* 0, 3 or 4 (TopK lists: 0 or 3)                    */
  int32_t cmp_mask_mode; /* 0 or 3                                            */
  int32_t ori_win_left;  /* -1 (unbounded) or >= 0                            */
  int32_t ori_win_right; /* -1 (unbounded) or >= 0                            */
  int32_t has_ori_kv;    /* must be 1                                         */
  int32_t has_cmp_kv;    /* 0 or 1                                            */
  int32_t kv_dtype;      /* SFMLA_KV_*                                        */
  int32_t has_separate_v;      /* ori side: V read from ori_v (16-bit rows, or
                                  packed KV's value codes)                     */
  int32_t has_sinks;           /* sinks pointer present                       */
  int32_t return_softmax_lse;  /* softmax_lse pointer present                 */
  int32_t has_seqused_q;       /* which optional length tensors are passed    */
  int32_t has_seqused_ori_kv;
  int32_t has_seqused_cmp_kv;
  int32_t has_cmp_residual_kv;
  /* Work-split overrides (0 = the library's rule, which depends on the
   * parameters only).  They enter the plan fingerprint and the workspace
   * size, so a plan and a workspace always match the split they were built
   * for; nothing is read from the environment.
   *   split_rows            list rows per KV split of a short-query row:
   *                         0, or a multiple of 32 in 32..2048.  Changes the
   *                         rounding order of the split merge (results stay
   *                         within the stated tolerances).
   *   head_blocks_per_group 16-head blocks that share one gathered KV row
   *                         set: 0, or 1, 2, 4, 8 (at most the kernel's
   *                         waves).  Results are bitwise the same for every
   *                         value.                                           */
  int32_t split_rows;
  int32_t head_blocks_per_group;
  /* How the partials of a split row are merged inside sfmla_forward
   * (0 = the library's rule): -1 = the last split to arrive merges them; a
   * positive value = the split that owns a block of heads waits at most that
   * many microseconds (1..10000) for the others and merges them itself
   * (used only when every workgroup of the launch is resident at once; on
   * time-out the last to arrive merges).  Every setting gives the same bits. */
  int32_t merge_wait_us;
  /* Query tiles (0 = the library's rule).  Consecutive query rows of one
   * sequence share a workgroup: their lists are merged into one union list
   * that is gathered once, and each row masks the union positions that its
   * own list does not hold (SparseAttnSharedkv README, 调用说明: prefill with
   * s1 query tokens per sequence).  Tiles are used where every list is a
   * rule (window and / or every visible compressed row: ori_topk = cmp_topk
   * = 0), KV is bf16 or float16, at most 64 heads, and the parameters bound
   * a tile's union to one split of 2048 rows (window: win_left + win_right +
   * rows per tile, else max_seqlen_ori_kv; plus max_seqlen_cmp_kv).
   * The rule tiles 8 / (16-head blocks rounded up to a power of two) rows,
   * i.e. 2 rows at 64 heads, 8 at 16, when max_seqlen_q >= 16 and the rows
   * carry rope or a separate V (rope-free rows whose V is the K nope go to
   * a four-wave kernel with two workgroups per CU instead, which was
   * measured faster than tiles on every prefill shape).
   *   1        never tile;
   *   2, 4, 8  that many rows per tile (refused where the parameters do not
   *            allow tiles of that size).
   * Tiles start at each sequence's first query row, so a row's tile depends
   * on its own sequence only.  Tiling changes the rounding order (results
   * stay within the stated tolerances); split_rows, head_blocks_per_group
   * and merge_wait_us have no effect on a tiled call, which needs no
   * workspace. */
  int32_t query_tile;
  /* Wave pairs (0 = the library's rule) for calls without query tiles: two
   * waves share 16 heads, each computes the scores of half of every 32-row
   * KV tile and accumulates half of the 512 value columns, so each wave's
   * chain of products per tile is half as long.  Results are bitwise the
   * same either way.
   *   1  never;
   *   2  always (refused where the parameters do not allow pairs).
   * The rule takes pairs where the call has fewer than 256 (query row,
   * split) units, i.e. where a row's heads are spread over several
   * workgroups and each walks its chain of tiles alone.  head_blocks_per_group
   * then counts pairs (at most 4 per group). */
  int32_t wave_pairs;
} sfmla_params;

/*
 * Length tensors (API page 参数说明 cu_seqlens_*, seqused_*, cmp_residual_kv).
 * int32 device arrays; NULL when absent.  cu_seqlens_* have b+1 entries
 * (start 0, non-decreasing), the others b entries.
 *   cu_seqlens_q        required iff layout_q is TND
 *   cu_seqlens_ori_kv   required iff layout_kv is TND
 *   cu_seqlens_cmp_kv   required iff layout_kv is TND and has_cmp_kv
 *   seqused_q           optional: valid query rows per batch (rows past it
 *                       are written as O = 0, LSE = -inf)
 *   seqused_ori_kv      required for PA; optional otherwise (overrides)
 *   seqused_cmp_kv      required for PA with cmp_kv; optional otherwise
 *   cmp_residual_kv     required with cmp_kv and cmp_mask_mode 3; values in
 *                       [0, cmp_ratio) with cmp_len*ratio + residual = ori_len
 */
typedef struct sfmla_lengths {
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_ori_kv;
  const int32_t* cu_seqlens_cmp_kv;
  const int32_t* seqused_q;
  const int32_t* seqused_ori_kv;
  const int32_t* seqused_cmp_kv;
  const int32_t* cmp_residual_kv;
} sfmla_lengths;

/*
 * Tensors of one forward call (device pointers; strides in BYTES between
 * consecutive physical rows, which may include padding — API page 约束说明:
 * non-contiguous rows with inter-row padding are allowed).
 *
 *   q            bf16 (float16 for SFMLA_KV_FP16), contiguous
 *                (q_t, num_heads_q, 512 + rope), or (q_t, num_heads_q, 512)
 *                when q_rope is given; "bf16" below reads float16 for that
 *                format
 *   q_rope       the query's rope part stored apart (SparseFlashAttention
 *                README, 参数说明 query_rope): bf16, contiguous
 *                (q_t, num_heads_q, 64), rope_head_dim 64 only; else NULL
 *   ori_kv       bf16 rows: 512 nope values, then (if rope_head_dim = 64 and
 *                ori_rope is NULL) 64 rope values; packed rows: 512 codes,
 *                2*rope bytes of bf16 rope, 16 bytes of fp32 scales
 *   ori_rope     bf16 rope rows (64 values) when stored apart; else NULL
 *   ori_v        when has_separate_v (else NULL), rows indexed like ori_kv's
 *                (at least ori_kv_rows of them): bf16 / fp16 value rows of
 *                512 values; with packed KV, 512 value codes per row in the
 *                key's format, each 128-column tile scaled by the key row's
 *                scale of that tile (KV quant blog, 参数说明 value: a 512-wide
 *                NoPE value tensor whose own dequant scale is reserved)
 *   cmp_kv / cmp_rope   as ori_kv / ori_rope (no separate V)
 *   ori_block_table / cmp_block_table   int32 (b, *_block_table_cols), PA only
 *   ori_sparse_indices  int32 (q_t, 1, ori_topk) when ori_topk > 0
 *   cmp_sparse_indices  int32 (q_t, 1, cmp_topk) when cmp_topk > 0;
 *                       -1 marks an empty slot
 *   sinks        fp32 (num_heads_q) when has_sinks
 *   attention_out  bf16 (q_t, num_heads_q, 512)  [written]
 *   softmax_lse    fp32 (q_t, num_heads_q), i.e. (b, 1, q_s, q_n) for BSND and
 *                  (1, q_t, q_n) for TND, when return_softmax_lse  [written]
 *   status       optional int32 word: bits SFMLA_STATUS_* are OR-ed in
 */
typedef struct sfmla_tensors {
  const void* q;
  const void* ori_kv;   int64_t ori_kv_stride;
  const void* ori_rope; int64_t ori_rope_stride;
  const void* ori_v;    int64_t ori_v_stride;
  const void* cmp_kv;   int64_t cmp_kv_stride;
  const void* cmp_rope; int64_t cmp_rope_stride;
  const int32_t* ori_block_table;
  const int32_t* cmp_block_table;
  const int32_t* ori_sparse_indices;
  const int32_t* cmp_sparse_indices;
  const float* sinks;
  void* attention_out;
  float* softmax_lse;
  int32_t* status;
  const void* q_rope;
} sfmla_tensors;

/* Number of int32 the plan of these parameters occupies (host only). */
sfmla_status sfmla_metadata_size(const sfmla_params* params, size_t* n_ints);

/*
 * Build the split plan (sparse_flash_mla_metadata on the API page): per query
 * row its batch, position, resolved window / list extents and split count,
 * plus a fingerprint of `params`; with query tiles (sfmla_params.query_tile)
 * also the tiles, numbered sequence by sequence with no gaps, each as its
 * first query row and row count.  Reads the length tensors on the device
 * (cu_seqlens_q must start at 0, be non-decreasing and end at q_t).
 * `metadata` holds at least sfmla_metadata_size() int32, 16-byte aligned.
 */
sfmla_status sfmla_metadata(const sfmla_params* params, const sfmla_lengths* lengths,
                            int32_t* metadata, size_t n_ints, void* stream);

/* Bytes of scratch sfmla_forward needs for split partials (host only). */
sfmla_status sfmla_workspace_size(const sfmla_params* params, size_t* bytes);

/*
 * Attention forward (sparse_flash_mla on the API page): writes attention_out
 * (and softmax_lse).  softmax_scale must be finite.  `workspace` holds at
 * least sfmla_workspace_size() bytes, 256-byte aligned (NULL when that size
 * is 0).  Rows whose list the plan splits are merged inside this call (the
 * last split of a row to finish merges the others' partials, which pass
 * through `workspace` as bf16), so attention_out and softmax_lse are final
 * when the call's work completes.  The plan buffer doubles as the arrival counters of that in-call merge: the
 * call leaves them as it found them (zero), so the same plan serves any
 * number of calls, but two calls that share one plan must not overlap.
 */
sfmla_status sfmla_forward(const sfmla_params* params, const sfmla_tensors* tensors,
                           int32_t* metadata, size_t n_ints, float softmax_scale,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * For callers that cannot allocate device memory: code under HIP graph
 * capture that must not call hipMalloc, tight serving loops, harnesses that
 * forbid allocation.  The same as sfmla_forward(), except that the split
 * workspace is a buffer the library owns: one static device array of
 * SFMLA_STATIC_WORKSPACE_BYTES on each GPU the library runs on, held from the
 * time the library's code is loaded on that GPU until the process ends.  The
 * call allocates and frees nothing.  A call whose parameters need a larger
 * workspace (sfmla_workspace_size()) is refused with
 * SFMLA_ERR_BUFFER_TOO_SMALL before anything is launched.  The stream must
 * belong to the current device.  Every call on one GPU shares that GPU's
 * array, and its contents from the last call stay there (nothing in it has
 * to start at zero: every byte a call reads was written earlier in the same
 * call).  Calls that overlap in time on one GPU (e.g. on two streams) race on
 * it and give undefined results.
 */
#define SFMLA_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)
sfmla_status sfmla_forward_static_workspace(const sfmla_params* params,
                                            const sfmla_tensors* tensors, int32_t* metadata,
                                            size_t n_ints, float softmax_scale, void* stream);

/*
 * LSE merge of partial results over disjoint parts of each row set (the
 * FLASH_DECODE split of the kv_quant_sparse_flash_attention blog's kernel
 * structure; its usage notes name the max / sum outputs as what merges
 * KV-sharded (DCP) partial results).  For r in [0, rows), h in [0, heads):
 *   part_o[(k*rows + r)*heads + h][0..dv)  fp32, part k's output normalised
 *                                           without the sink
 *   part_lse[(k*rows + r)*heads + h]        fp32, part k's LSE (-inf = empty)
 *   out  bf16 (rows, heads, dv) = sum_k e^{lse_k} O_k / (sum_k e^{lse_k} + e^{sink_h})
 *   lse_out fp32 (rows, heads) = log sum_k e^{lse_k}  (may be NULL)
 * The sink (sinks: fp32 (heads), NULL = no sink) is applied once, here.  A
 * (row, head) whose parts are all empty gives O = 0, LSE = -inf.  part_o is
 * 16-byte aligned, out 8-byte aligned; dv is a multiple of 4 in 4..4096,
 * heads <= 65535.  sfmla_forward() needs no call of this: it merges the
 * splits it plans itself.
 */
sfmla_status sfmla_combine(int32_t n_parts, const float* part_o, const float* part_lse,
                           const float* sinks, void* out, float* lse_out, int32_t rows,
                           int32_t heads, int32_t dv, void* stream);

/*
 * Debug view of the resolver: writes each query row's resolved physical rows
 * in canonical order (original-KV rows first — ascending for mask rules, slot
 * order for TopK lists — then compressed rows, ascending for HCA and slot
 * order for CSA), dropping -1 and masked slots.  rows_out is int64
 * (q_t, max_rows), compressed rows tagged with bit 62, unused entries -1;
 * counts_out is int32 (q_t) and may exceed max_rows (then the list is cut).
 */
sfmla_status sfmla_debug_resolve(const sfmla_params* params, const sfmla_tensors* tensors,
                                 const int32_t* metadata, size_t n_ints, int64_t* rows_out,
                                 int32_t max_rows, int32_t* counts_out, void* stream);

/*
 * Measurement hook: the next sfmla_forward() call on this thread launches its
 * kernel with these HIP events (hipEvent_t, either may be NULL) stamped by
 * the dispatch itself at the kernel's start and end, so that
 * hipEventElapsedTime() of the pair is that kernel's duration with no event
 * packets queued around it.  The events must exist (created or recorded once
 * before); the library keeps no reference after that call, which uses them
 * whether or not it succeeds.  Always SFMLA_OK.
 */
sfmla_status sfmla_time_next_forward(void* start_event, void* stop_event);

/* Thread-local description of the last failed call ("" after success). */
const char* sfmla_last_error(void);
const char* sfmla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SFMLA_H */
