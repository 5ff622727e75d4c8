/*
 * cascade_attn.h -- C ABI of the MI355X (gfx950) shared-prefix ("cascade")
 * attention library.
 *
 * The method ("vLLM Cascade Attention：用法、场景与原理解析", beaiera.top,
 * section 1 and section 8 Step 5): for a batch of requests whose paged KV
 * caches begin with the same physical pages,
 *   (1) all requests' query tokens, packed as one sequence, attend
 *       non-causally and once to the shared-prefix KV pages;
 *   (2) each request attends causally to its own remaining ("suffix") pages;
 *   (3) the two partial results are merged by log-sum-exp rescaling.
 * The result equals ordinary causal attention of every request over its
 * whole KV sequence; the saving is that the shared pages are read once
 * instead of once per request (same page, section 5).
 *
 * Host side (same page, section 8 Steps 1-3): count the leading KV pages
 * common to every request of the batch, cap that prefix at the smallest
 * num_computed_tokens and floor it to a page, decide whether cascade pays,
 * and derive the per-phase metadata. That is cascade_attn_plan(); it touches
 * no device memory and may run while the GPU is busy with the previous step.
 * cascade_attn_run() launches the kernels on the caller's stream.
 *
 * Conventions for every entry point:
 *   - Plain C, no allocation visible to the caller other than the plan
 *     handle; the caller owns every tensor (device memory from any allocator).
 *   - Dtypes: Q and output are bf16; the K/V caches bf16 or fp8 e4m3
 *     (ca_kv_dtype_t); LSE fp32; workspace partial states bf16 or fp32
 *     (partials_fp32) with fp32 LSEs; metadata int32.
 *   - seq_lens[r] counts all KV positions of request r including this
 *     step's q_len_r query tokens, which are its last q_len_r positions;
 *     num_computed_tokens[r] = seq_lens[r] - q_len_r.
 *   - Causal rule: query i (0-based within request r) sees KV positions
 *     t <= num_computed_tokens[r] + i.
 *   - GQA: query head h reads KV head h / (num_q_heads / num_kv_heads).
 *   - LSE values are natural logs of the softmax normaliser of the scaled
 *     scores.
 *   - Every function returns a ca_status_t; on a non-OK status,
 *     cascade_attn_last_error() returns a message for the calling thread.
 *     No function aborts the process on bad input.
 */
#ifndef CASCADE_ATTN_H_
#define CASCADE_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CA_OK = 0,
  CA_EINVAL = 1,        /* null pointer, bad handle, bad size argument */
  CA_EUNSUPPORTED = 2,  /* head_dim not 64/128 (fp8: not 128), page_size not 16, Hq % Hkv != 0 */
  CA_EMETA = 3,         /* inconsistent batch metadata (lengths, page ids, strides) */
  CA_EWORKSPACE = 4,    /* workspace smaller than the plan requires */
  CA_EHIP = 5           /* a HIP runtime call or kernel launch failed */
} ca_status_t;

/* User switch over the planner's decision ([p1] "Diary - vLLM's cascade
 * attention": the disable_cascade_attn option; [p2] section 3: cascade is
 * only used when the heuristic says it pays). */
typedef enum {
  CA_MODE_AUTO = 0,       /* prefix and request gates + cost model decide */
  CA_MODE_FORCE_ON = 1,   /* cascade whenever the capped shared prefix is > 0 */
  CA_MODE_FORCE_OFF = 2   /* always the non-cascade path */
} ca_mode_t;

/* Element type of the paged K/V caches. FlashInfer's cascade path was turned
 * off for FP8 caches ([p2] section 6); here both run every phase. */
typedef enum {
  CA_KV_BF16 = 0,        /* bf16 */
  CA_KV_FP8_E4M3 = 1     /* fp8 e4m3 (OCP: bias 7, max 448, NaN 0x7f / 0xff, no infinity), one byte per
                            element, dequantised as value * k_scale (K) and value * v_scale (V); head_dim 128 */
} ca_kv_dtype_t;

typedef struct {
  int32_t num_reqs;            /* N >= 1 */
  int32_t num_q_heads;         /* Hq */
  int32_t num_kv_heads;        /* Hkv, Hq % Hkv == 0 */
  int32_t head_dim;            /* d: 64 or 128 */
  int32_t page_size;           /* tokens per KV page: 16 */
  int32_t block_table_stride;  /* int32 entries per block-table row */
  int32_t num_pages;           /* pages in the KV pool (bounds check of page ids) */
  int32_t separate_phases;     /* cascade path only: 0 = prefix and suffix work-groups share one
                                  launch; 1 = two launches (prefix, then suffix) doing the same
                                  work with identical results, e.g. to time each phase */
  /* K/V cache element strides (elements of kv_dtype). The cache is indexed
   * [page][slot][kv_head][d] with d contiguous; NHD layout
   * [num_pages, page_size, Hkv, d] has (page_size*Hkv*d, Hkv*d, d), HND
   * layout [num_pages, Hkv, page_size, d] has (Hkv*page_size*d, d, page_size*d).
   * All three must be multiples of 8 for bf16 and of 16 for fp8 (16-byte
   * aligned rows), and
   * kv_stride_token at most 2^26 (byte offsets within one page fit 32 bits). */
  int64_t kv_stride_page;
  int64_t kv_stride_token;
  int64_t kv_stride_head;
  float softmax_scale;         /* <= 0 selects 1/sqrt(head_dim) */
  int32_t mode;                /* ca_mode_t */
  int32_t num_cus;             /* compute units to plan for; 0 = query the current device */
  int32_t heads_per_item;      /* KV heads one decode-shaped suffix item runs back to back
                                  (0 = planner's choice; else must divide num_kv_heads;
                                  ignored for items of more than 16 rows) */
  int32_t max_levels;          /* shared levels of the cascade path, 0..4: 0 = planner default (4);
                                  1 = the batch-wide prefix only; L >= 2 = also nested groups of
                                  requests (any, not only consecutive) that share more pages, up to
                                  L - 1 levels below the prefix (see cascade_attn_plan_groups) */
  int32_t kv_dtype;            /* ca_kv_dtype_t */
  float k_scale;               /* fp8: K dequantisation factor (<= 0 selects 1); ignored for bf16 */
  float v_scale;               /* fp8: V dequantisation factor (<= 0 selects 1); ignored for bf16 */
  int32_t sliding_window;      /* 0 = none; W >= 1: a query at position p sees p - W < t <= p. Cascade
                                  is not used when the window binds ([p2] section 3 lists sliding
                                  window among the features cascade does not support): AUTO then
                                  runs the non-cascade path and FORCE_ON fails with CA_EUNSUPPORTED */
  int32_t prefix_splits;       /* 0 = planner's choice; else KV splits of the prefix phase (raised if an
                                  item would exceed 8192 keys, lowered to the prefix's 64-key tiles) */
  int32_t suffix_order;        /* 0 = per-request work items start longest key range first (batches of
                                  at most 512 requests; results are identical, only the dispatch
                                  order changes); 1 = batch order */
  int32_t partials_fp32;       /* partial outputs of the phases before the merge: 0 = bf16 (the
                                  attention dtype, as [p2] section 8 Step 5 merges the two phases'
                                  outputs), 1 = fp32; partial LSEs are fp32 either way */
  int32_t merge_mode;          /* where the partial states are merged: 0 (default) = the planner's
                                  choice by cost; 1 = a separate merge launch (as always with
                                  separate_phases); 2 = inside the attention launch, by the work item
                                  that completes each row block (one launch per step; plans with
                                  nested levels merge separately). All merge in the same order:
                                  same bits */
  int32_t use_tuned;           /* 0 (default) = AUTO is a pure function of the batch and these
                                  params; 1 = an AUTO plan whose batch shape has a choice recorded
                                  by cascade_attn_autotune / cascade_attn_autotune_record takes
                                  that choice. Off by default so that a request's output bits never
                                  depend on what the process tuned before ([p1]: output that
                                  changes with batch composition is the failure to avoid) */
} ca_params_t;

typedef struct {
  int32_t use_cascade;                 /* 1 if run() takes the three-phase path */
  int32_t num_common_prefix_blocks;    /* pages shared by every request */
  int32_t common_prefix_len;           /* capped, page-floored shared prefix (tokens) */
  int32_t gates_pass;                  /* the pages' gates: prefix >= 256 tokens and >= 8 requests
                                          (reported; AUTO's own gate is prefix >= 256 tokens and
                                          >= 2 requests, see cascade_attn_plan) */
  int32_t prefix_splits;               /* KV splits of the prefix phase */
  int32_t prefix_row_tile;             /* packed query rows per prefix work-group */
  int32_t suffix_chunks;               /* KV chunks per request of the suffix (or only) phase */
  int32_t suffix_chunk_tokens;         /* tokens per chunk */
  int32_t suffix_kernel;               /* 0 = tiled kernel, 1 = decode kernel */
  int32_t num_partial_slots;           /* partial states per (token, head) */
  int32_t prefix_stages;               /* LDS pipeline depth of the prefix kernel */
  int32_t suffix_stages;               /* LDS pipeline depth of the suffix / only kernel */
  int32_t merge_in_launch;             /* 1 if the partial states are merged inside the attention launch */
  int32_t suffix_heads_per_item;       /* consecutive KV heads one suffix (or only) work item runs */
  int32_t separate_phases;             /* 1 if the cascade phases run as separate launches */
  int32_t num_level1_groups;           /* request groups of the nested shared levels (0 = none) */
  int32_t level1_splits;               /* KV splits of every group of the first nested level */
  int32_t kv_dtype;                    /* ca_kv_dtype_t of the plan */
  int32_t sliding_window;              /* window applied by the plan (0: none, or it never binds) */
  int32_t suffix_longest_first;        /* 1 if per-request items start longest key range first */
  int64_t total_q;                     /* T = query_start_loc[N] */
  int64_t workspace_bytes;             /* bytes run() needs (0 = none) */
  int64_t kv_tokens_cascade;           /* prefix + sum of suffixes (positions read by cascade) */
  int64_t kv_tokens_noncascade;        /* sum of seq_lens (positions read without cascade) */
  float est_us_cascade;                /* cost-model estimates used by AUTO */
  float est_us_noncascade;
  int32_t partials_fp32;               /* 1 if partial outputs are fp32, 0 if bf16 */
  int32_t shared_levels;               /* shared levels the cascade path runs (1 = the batch-wide
                                          prefix only; 0 = non-cascade) */
} ca_plan_info_t;

typedef struct ca_plan* ca_plan_t;

/*
 * Number of leading KV pages shared by every request of the batch
 * ([p2] section 8 Step 1: count the physical blocks shared by all running
 * requests, matching contiguously from block 0; [p3] "resolve async KV
 * transfer bug in cascade attention #23485": only the running requests --
 * here, the rows passed in -- are counted).
 *
 * block_table_h: host int32 [num_reqs][stride]; seq_lens_h: host int32
 * [num_reqs]. Column j is compared only if j < ceil(seq_lens[r]/page_size)
 * for every r, so block-table padding never counts. Result in *out_blocks.
 * Errors: CA_EINVAL for null pointers or non-positive sizes, CA_EMETA if a
 * request needs more pages than stride.
 */
ca_status_t cascade_attn_num_common_prefix_blocks(const int32_t* block_table_h, int32_t num_reqs,
                                                  int32_t stride, const int32_t* seq_lens_h,
                                                  int32_t page_size, int32_t* out_blocks);

/*
 * Host-only planner ([p2] section 8 Steps 1-3; the decision of section 3).
 * Reads host copies of the batch metadata:
 *   block_table_h        int32 [num_reqs][block_table_stride]
 *   query_start_loc_h    int32 [num_reqs + 1], [0] == 0, q_len_r >= 1
 *   seq_lens_h           int32 [num_reqs]
 *   num_computed_tokens_h int32 [num_reqs] (may be NULL: derived as
 *                        seq_lens - q_len; if given it must equal that)
 * and computes: the shared-page count, the capped/floored prefix length,
 * the pages' gates (prefix >= 256 tokens, >= 8 requests; [p2] section 3,
 * reported in gates_pass), the cascade/non-cascade decision (mode; in AUTO,
 * a prefix of >= 256 tokens shared by >= 2 requests, the request gate
 * re-derived for these kernels, then a cost model of this library's kernels
 * on params->num_cus compute units), the work partition of each
 * phase and the workspace size. Copies nothing but derived scalars; the
 * plan is valid for every layer of the step (same metadata, any Q/KV).
 * Device is touched only when params->num_cus == 0 (to read the CU count).
 * Errors: CA_EINVAL (null pointers), CA_EUNSUPPORTED (head_dim, page_size,
 * head ratio, strides), CA_EMETA (inconsistent lengths, a request needing
 * more than stride pages, a referenced page id outside [0, num_pages)).
 */
ca_status_t cascade_attn_plan(const ca_params_t* params, const int32_t* block_table_h,
                              const int32_t* query_start_loc_h, const int32_t* seq_lens_h,
                              const int32_t* num_computed_tokens_h, ca_plan_t* out_plan);

/* Copies the plan's decisions and sizes (the quantities of [p2] section 8
 * Steps 1-3: shared pages, capped prefix length, gates and decision, and
 * the per-phase partition) into *out. Errors: CA_EINVAL for a null plan or
 * output. */
ca_status_t cascade_attn_plan_info(ca_plan_t plan, ca_plan_info_t* out);

/*
 * Nested shared levels of the plan. FlashInfer's cascade takes any number of
 * levels ([p2] section 7) and the workloads of [p2] section 3 nest (system
 * prompt -> document -> chapter -> request). When the cascade path is taken
 * and params->max_levels != 1, the planner applies the batch-wide rule of
 * [p2] section 8 Steps 1-2 (leading pages shared by the members, capped at
 * their smallest num_computed_tokens, floored to a page) at every node of
 * the prefix tree of the requests' page-id sequences: members that share
 * every page up to some column are split by their page at that column; a
 * part of >= 2 requests whose shared length exceeds the enclosing level's by
 * >= 256 tokens (the pages' prefix-length gate, [p2] section 3) becomes a
 * group one level deeper. Members need not be consecutive in the batch.
 * Levels below the prefix: at most max_levels - 1 (default 3); groups: at
 * most 64, kept level by level by the KV reads they save; batches of more
 * than 512 requests get none. A group's queries, packed, attend non-causally
 * once to its positions [key_begin, key_end) (key_begin: the enclosing
 * level's shared length); each request's own phase starts at the key_end of
 * its innermost group. Writes min(n, capacity) rows (level >= 1, parent
 * group index or -1 for the batch-wide prefix, key_begin, key_end) to
 * groups_out [capacity][4], parents before children; if deepest_out is not
 * NULL, each request's innermost group (or -1) to deepest_out [num_reqs];
 * and n to *n_out. Errors: CA_EINVAL (null plan / n_out, capacity < 0, null
 * groups_out with capacity > 0).
 */
ca_status_t cascade_attn_plan_groups(ca_plan_t plan, int32_t capacity, int32_t* groups_out, int32_t* deepest_out,
                                     int32_t* n_out);

/*
 * Runs one attention step of the plan on `stream` (a hipStream_t; NULL =
 * the null stream). Asynchronous: no host synchronisation, no allocation,
 * no host-to-device copy; inputs must stay alive until the stream passes
 * this call.
 *   q                [T][num_q_heads][head_dim] bf16, contiguous
 *   k_cache, v_cache paged caches of the plan's kv_dtype and strides
 *   block_table_d, query_start_loc_d, seq_lens_d: device copies of the
 *                    same metadata given to cascade_attn_plan
 *   sinks_d          [num_q_heads] fp32 attention-sink logits, or NULL. [p2]
 *                    section 9: every backend receives an optional sinks
 *                    parameter. Reading: one logit z_h per query head joins
 *                    the softmax normaliser with no value, out = sum_t
 *                    exp(s_t) v_t / (sum_t exp(s_t) + exp(z_h)), and lse
 *                    includes it. May change between runs of one plan.
 *   out              [T][num_q_heads][head_dim] bf16 (written)
 *   lse_out          [T][num_q_heads] fp32, natural log (written; may be NULL)
 *   workspace        device scratch of >= info.workspace_bytes bytes (may be
 *                    NULL when that is 0); 256-byte aligned. Its first
 *                    CA_WORKSPACE_COUNTER_BYTES hold the arrival counters of
 *                    the merge inside the attention launch: they must be zero
 *                    before the workspace's first run (allocate it zeroed, or
 *                    call cascade_attn_workspace_init once), and every run
 *                    leaves them zero, so one workspace serves any sequence
 *                    of plans. The rest needs no initialisation. Nothing else
 *                    may write the workspace between runs; two runs that
 *                    overlap in time must not share it.
 * Cascade path: the prefix phase, the group level (if the plan has one) and
 * the suffix phase in one launch, then the LSE merge ([p2] section 8 Step
 * 5); the merge runs as its own launch or inside the attention launch
 * (merge_mode; info.merge_in_launch). Non-cascade path: one attention over each request's full
 * block table (Step 4), merging its KV chunks the same way when the plan
 * splits the KV range.
 * Errors: CA_EINVAL (null pointers/handle), CA_EWORKSPACE (too small),
 * CA_EHIP (launch failure).
 */
ca_status_t cascade_attn_run(ca_plan_t plan, const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table_d, const int32_t* query_start_loc_d,
                             const int32_t* seq_lens_d, const float* sinks_d, void* out, float* lse_out,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Zeroes the merge counters at the start of a workspace (the first
 * min(workspace_bytes, CA_WORKSPACE_COUNTER_BYTES) bytes) with a kernel on
 * `stream` (graph-capturable; no memset). Needed once per workspace before
 * its first run unless it was allocated zeroed.
 * Errors: CA_EINVAL (null workspace with a size, misaligned), CA_EHIP.
 */
#define CA_WORKSPACE_COUNTER_BYTES (256u << 10)
ca_status_t cascade_attn_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * cascade_attn_run without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). The partial states live in a
 * library-owned device array of CA_NOALLOC_WORKSPACE_BYTES (32 MiB), one
 * copy per GPU, taken when the library first runs this entry point on that
 * GPU and held until the process ends. This call allocates nothing (no
 * hipMalloc / hipFree, no allocating library routine); on its first call on
 * a device it looks up that device's copy of the array.
 * Arguments as for cascade_attn_run. Every call on one GPU shares that GPU's
 * array and it keeps the last call's contents: calls that overlap in time on
 * one GPU (two streams, two threads) race and must not be issued; calls on
 * one stream are ordered and safe. No part of the array needs to start at
 * zero (each call writes every partial state it reads back).
 * Errors: as cascade_attn_run; CA_EWORKSPACE when the plan's workspace_bytes
 * exceed CA_NOALLOC_WORKSPACE_BYTES (e.g. very large prefill batches, or
 * partials_fp32); CA_EHIP if the array's device address cannot be found.
 */
#define CA_NOALLOC_WORKSPACE_BYTES (32u << 20)
ca_status_t cascade_attn_run_noalloc(ca_plan_t plan, const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_table_d, const int32_t* query_start_loc_d,
                                     const int32_t* seq_lens_d, const float* sinks_d, void* out,
                                     float* lse_out, void* stream);

/*
 * Per-shape autotuning ([p4] "Update Cascade Attention Heuristics for FA3":
 * the heuristic has to be re-derived for each kernel family; [p2] section 9:
 * cascade only when it beats the plain path). Plans the batch as AUTO would,
 * then times candidate plans on the device with the caller's data: the
 * non-cascade path and, when a prefix is shared and no window binds, the
 * cascade path with the planner's prefix split count, half and twice it,
 * one, two or the planner's KV heads per decode item, and (if the batch has
 * nested groups) every shared level the detector finds, the batch-wide prefix
 * only, and two levels when it finds more. Each candidate runs twice untimed and
 * `iters` times between two HIP events on `stream`; candidates needing more
 * than workspace_bytes are skipped. Returns the fastest plan in *out_plan
 * (the caller destroys it) and its mean time per run in *out_us (may be
 * NULL), and records the choice for this batch shape: later AUTO plans with
 * params->use_tuned = 1, no explicit overrides (prefix_splits,
 * heads_per_item, max_levels all 0) and the same shape apply it. A shape is (num_reqs, head counts, head_dim,
 * kv_dtype, window, and the power-of-two buckets of the shared prefix, total
 * queries, longest query, mean remaining length and nested-group count).
 * Synchronises the stream; not for graph capture. out, lse_out and
 * workspace are overwritten (out / lse_out hold this batch's result).
 * Errors: as cascade_attn_plan and cascade_attn_run; CA_EINVAL for iters
 * outside [1, 1000]; CA_EWORKSPACE if no candidate fits the workspace.
 */
ca_status_t cascade_attn_autotune(const ca_params_t* params, const int32_t* block_table_h,
                                  const int32_t* query_start_loc_h, const int32_t* seq_lens_h,
                                  const int32_t* num_computed_tokens_h, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_table_d,
                                  const int32_t* query_start_loc_d, const int32_t* seq_lens_d,
                                  const float* sinks_d, void* out, float* lse_out, void* workspace,
                                  size_t workspace_bytes, void* stream, int32_t iters, ca_plan_t* out_plan,
                                  float* out_us);

/*
 * Records a choice for the batch's shape without timing anything (host only;
 * e.g. to restore choices a previous process tuned). The shape is that of
 * the AUTO plan of (params, metadata), as cascade_attn_autotune records it;
 * the choice is the mode (CA_MODE_FORCE_ON or CA_MODE_FORCE_OFF) and the
 * ca_params_t settings prefix_splits, heads_per_item and max_levels (0 =
 * planner's choice). Only plans made with params->use_tuned = 1 consult it.
 * Errors: as cascade_attn_plan; CA_EINVAL for a mode other than FORCE_ON /
 * FORCE_OFF or a negative setting.
 */
ca_status_t cascade_attn_autotune_record(const ca_params_t* params, const int32_t* block_table_h,
                                         const int32_t* query_start_loc_h, const int32_t* seq_lens_h,
                                         const int32_t* num_computed_tokens_h, int32_t mode,
                                         int32_t prefix_splits, int32_t heads_per_item, int32_t max_levels);

/* Forgets every shape recorded by cascade_attn_autotune or
 * cascade_attn_autotune_record. */
void cascade_attn_autotune_reset(void);

/* Frees a plan (NULL is accepted). */
void cascade_attn_plan_destroy(ca_plan_t plan);

/* Message for the last non-OK status returned on the calling thread. */
const char* cascade_attn_last_error(void);

/*
 * Kernel timing for measurement. cascade_attn_profile_enable(capacity)
 * creates a pool of 2 * capacity HIP events (call it outside any timed
 * region; 0 disables timing and frees the pool). While enabled, each kernel
 * run() launches takes the next start / stop pair of the pool, recorded on
 * the launch stream right before and right after that kernel (no event is
 * created during run()); launches past the pool's capacity run untimed. cascade_attn_profile_read() waits for the
 * recorded events, writes the summed milliseconds and launch counts per
 * kernel kind into ms[CA_PROFILE_KINDS] and counts[CA_PROFILE_KINDS], and
 * makes the whole pool available again.
 * Kinds: 0 = cascade phases (prefix and suffix work-groups of the cascade
 * path in one launch), 1 = tiled attention of the non-cascade path,
 * 2 = merge, 3 = decode attention of the non-cascade path, 4 = prefix phase,
 * 5 = suffix phase and 6 = group level when a plan runs the phases as
 * separate launches.
 * Errors: CA_EINVAL (capacity outside [0, 2^20], null outputs), CA_EHIP if
 * an event call fails.
 */
#define CA_PROFILE_KINDS 7
ca_status_t cascade_attn_profile_enable(int32_t capacity);
ca_status_t cascade_attn_profile_read(double* ms, int64_t* counts);

#ifdef __cplusplus
}
#endif

#endif /* CASCADE_ATTN_H_ */
