/*
 * hsab.h - C ABI of libhsab.so, a two-level (block, then token) sparse
 * attention decode operator for AMD Instinct MI355X (gfx950).
 *
 * Method: AsyncTLS, "Efficient Generative LLM Inference with Asynchronous
 * Two-level Sparse Attention". Citations name the page and its section:
 *   [abstract]  mlsanity.com index page of the paper, "Abstract (arXiv)"
 *   [de 2.A]    gist.science/de explainer, section 2 "Methodik", part A
 *   [de 2.B]    gist.science/de explainer, section 2 "Methodik", part B
 *   [es 2.A]    gist.science/es explainer, section 2 "Metodologia", part A
 *   [es 2.B]    gist.science/es explainer, section 2 "Metodologia", part B
 *
 * Vocabulary
 *   B        batch size; Hq query heads; Hkv KV heads; G = Hq / Hkv.
 *            Query head h reads KV head h / G.
 *   unit     one (batch b, KV head g) pair; units are independent.
 *   n        ctx_len[b]: valid tokens of every KV head of batch row b.
 *   block    tokens per KV block; block j holds tokens [j*block, (j+1)*block)
 *            clipped to n; nb = ceil(n / block); nb_cap = ceil(max_ctx / block).
 *   r        label channels per KV head (Double-Sparsity style token index).
 *   K_b, K_t kept blocks / kept tokens per unit.
 *
 * Data layout (all bf16 values are raw uint16 bit patterns; every pointer
 * argument except `dims` is DEVICE memory owned by the caller; the library
 * never allocates, frees or synchronises):
 *   q        [B][Hq][d_k]                         bf16
 *   K        [B][Hkv][max_ctx][d_k]               bf16 key cache
 *   V        [B][Hkv][max_ctx][d_v]               bf16 value cache; when
 *            dims.v_alias_k != 0 there is no V array: the value of a token
 *            is the first d_v entries of its key row (absorbed MLA latent).
 *   meta     [B][Hkv][nb_cap][2][d_k]             per block, the
 *            channelwise key max row followed by the key min row; bf16
 *            values, or with dims.meta_format == HSAB_META_FP8 one byte
 *            per value in fp8 e4m3 (OCP "fn": bias 7, no infinities, max
 *            448), the max rounded up and the min rounded down to that
 *            grid so every block bound stays >= the true block maximum
 *            (keys with |k| > 448 saturate and lose that guarantee). The
 *            pointer type stays uint16_t*; the array then holds
 *            B*Hkv*nb_cap*2*d_k bytes. Quantised index data: AsyncTLS
 *            (gist.science/de explainer, section 2.A "Stufe 2") names
 *            quantisation as a way to cut the indexing cost without giving
 *            a scheme; outward rounding is this library's reading.
 *   klabel   [B][Hkv][max_ctx][r]                 bf16: K restricted to the
 *            label channels, klabel[..][t][c] = K[..][t][label_ch[g][c]];
 *            with dims.label_format == HSAB_LABEL_FP8 one byte per value,
 *            that key value rounded to the nearest fp8 e4m3 value (ties to
 *            the even mantissa, saturating at +-448); the pointer type stays
 *            uint16_t* and the array then holds B*Hkv*max_ctx*r bytes.
 *   label_ch [Hkv][r]                             int32 channel indices.
 *   ctx_len  [B]                                  int32, 1 <= n <= max_ctx.
 *   blk_idx  [B][Hkv][K_b]                        int32 ascending, -1 padded
 *            ([B][Hq][K_b] with per-head selection, HSAB_AGG_HEAD).
 *   tok_idx  [B][Hkv][K_t]                        int32 token positions,
 *            ascending, -1 padded ([B][Hq][K_t] with HSAB_AGG_HEAD).
 *   out      [B][Hq][d_v]                         fp32 attention output.
 *   lse      [B][Hq]                              fp32 natural-log
 *            logsumexp of the logits sm_scale*q.k over the kept tokens.
 *
 * Inputs must be finite (no inf/NaN in q, K, V or the new token).
 *
 * Selection rules (the pages leave them open; fixed here):
 *   - query heads sharing a KV head are combined by the maximum over the
 *     group, for block scores and token scores; one selection per unit
 *     (by default; dims.group_agg selects the sum, or one selection per
 *     query head);
 *   - top-k ties go to the lower index; index lists are ascending;
 *   - K_b and K_t clamp to what exists; unused slots are -1.
 *
 * Errors: every call returns HSAB_OK (0) or a negative code. Arguments are
 * checked on the host before anything is launched; on an error no kernel
 * runs and no output is written. HSAB_EHIP reports a failed launch (the
 * HIP error is readable with hsab_last_hip_error). Conditions only the
 * device can see (ctx_len out of [1, max_ctx]) are clamped on the device.
 * All work is enqueued on `stream` (NULL = the null stream) in order.
 */
#ifndef HSAB_H
#define HSAB_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSAB_OK            0
#define HSAB_EINVAL       -1   /* bad argument: null pointer, shape, budget, workspace too small */
#define HSAB_EHIP         -2   /* a HIP launch or runtime call failed */
#define HSAB_EUNSUPPORTED -3   /* valid shape with no kernel instantiation (see limits below) */
#define HSAB_ESCRATCH     -4   /* hsab_decode_step_noalloc: workspace beyond HSAB_SCRATCH_BYTES */

/* Shape and budget of one decode layer.
 * Limits: 1 <= G <= 32; d_k % 16 == 0, 16 <= d_k <= 1024 (d_k % 32 == 0
 * with fp8 metadata); d_v % 8 == 0;
 * r in {16, 32, 64, 128}, r <= d_k; 1 <= K_b <= 2048;
 * K_b * block <= 8192; nb_cap <= 8192; K_t >= 1.
 * Attention kernels exist for d_k == d_v in {64, 128, 256} with G in
 * {1, 2, 4, 8} (GQA/MQA/MHA, separate V), and for the absorbed latent
 * layout (v_alias_k, G == 32, d_k % 32 == 0, d_v % 64 == 0, d_v <= 512);
 * other shapes return HSAB_EUNSUPPORTED from hsab_sparse_attend and
 * hsab_decode_step. */
typedef struct hsab_dims {
    int32_t batch;        /* B */
    int32_t n_q_heads;    /* Hq */
    int32_t n_kv_heads;   /* Hkv, Hq % Hkv == 0 */
    int32_t d_k;          /* key / query head dim */
    int32_t d_v;          /* value head dim */
    int32_t v_alias_k;    /* nonzero: value = first d_v dims of the key row */
    int32_t block;        /* tokens per block */
    int32_t r;            /* label channels per KV head */
    int32_t k_blocks;     /* K_b */
    int32_t k_tokens;     /* K_t */
    int32_t max_ctx;      /* cache capacity (tokens) per unit */
    float   sm_scale;     /* logit scale, typically 1/sqrt(d_k) */
    int32_t meta_format;  /* HSAB_META_BF16 (0) or HSAB_META_FP8 (1) */
    int32_t group_agg;    /* HSAB_AGG_MAX (0), HSAB_AGG_SUM (1) or HSAB_AGG_HEAD (2): how the
                             query heads of a group combine block and token scores */
    int32_t sink_blocks;  /* the first sink_blocks blocks are always kept */
    int32_t local_blocks; /* the last local_blocks blocks (newest) are always kept;
                             sink_blocks + local_blocks <= k_blocks */
    int32_t label_format; /* HSAB_LABEL_BF16 (0) or HSAB_LABEL_FP8 (1): label rows in bf16 or
                             in nearest-rounded fp8 e4m3 */
} hsab_dims;

/* Selection variants (opt-in; zero-initialised dims select the default).
 * The pages combine no query-head scores and force no blocks; their
 * related-work list names StreamingLLM (AsyncTLS index page, "Builds on").
 * HSAB_AGG_SUM scores a block (token) by the sum of the group's bounds
 * (label scores) instead of their maximum. Forced blocks occupy K_b slots;
 * the remaining slots take the best other blocks; hsab_select_blocks and
 * the block stage of hsab_decode_step and the offload engine apply them. */
#define HSAB_AGG_MAX 0
#define HSAB_AGG_SUM 1
/* HSAB_AGG_HEAD: per-query-head selection (Quest, which the pages build on,
 * selects per head; the pages do not say how heads that share a KV head
 * combine). Every query head runs both stages on its own bound and label
 * score, as a group of one: block scores are [B][Hq][nb_cap], blk_idx
 * [B][Hq][K_b], tok_score [B][Hq][K_b*block], tok_idx [B][Hq][K_t], and
 * head h attends over its own tokens. The attention reads each row of the
 * union of a KV head's token sets once (hsab_sparse_attend and
 * hsab_decode_step build that union in the workspace). The block metadata
 * is read once per KV head: one product scores every head. Supported for
 * the separate-V attention shapes (not the absorbed latent layout) and not
 * by the offload engine (HSAB_EUNSUPPORTED). */
#define HSAB_AGG_HEAD 2

#define HSAB_META_BF16 0   /* block metadata in bf16 (exact key max/min) */
#define HSAB_META_FP8  1   /* fp8 e4m3, max rounded up, min rounded down */

/* Label rows (the fine stage's compressed keys): Double Sparsity keeps its
 * label cache in few bits and the pages name quantisation of the index data
 * (gist.science/de explainer, section 2.A "Stufe 2"). With HSAB_LABEL_FP8
 * the rows are e4m3 bytes rounded to nearest (the label score is an
 * estimate, so no rounding direction is needed); queries stay bf16 and the
 * label products are exact in fp32. */
#define HSAB_LABEL_BF16 0
#define HSAB_LABEL_FP8  1

/* Bytes of device workspace the calls below need for these dims (the same
 * size serves every call). The workspace holds block scores, token scores,
 * split-attention partials and the keys and arrival counters of a token
 * selection spread over several workgroups per (batch, KV head); it needs
 * no initialisation (the calls that use the counters set them first).
 * Calls that overlap on one workspace race. */
size_t hsab_workspace_bytes(const hsab_dims* dims);

/* Static text for a status code. */
const char* hsab_status_string(int status);

/* hipError_t of the most recent HSAB_EHIP on the calling thread (0 if none). */
int hsab_last_hip_error(void);

/* Block metadata and label cache from a prefilled key cache
 * [de 2.A Stufe 1: blocks summarised by key max/min; de 2.A Stufe 2 and
 * es 2.A item 2: label channels of the keys].
 * Reads K rows [0, n) of every unit; writes meta blocks [0, nb) and klabel
 * rows [0, n). The last block is summarised over its valid tokens only. */
int hsab_build_meta(const hsab_dims* dims, const uint16_t* K, const int32_t* ctx_len,
                    const int32_t* label_ch, uint16_t* meta, uint16_t* klabel,
                    hipStream_t stream);

/* Block scores alone [es 2.A item 1, the Quest-based score recast as a
 * dense product; de 2.A "Optimierung"]:
 *   blk_score[b][g][j] = max_{h in group g} ( q_h+ . Kmax_j + q_h- . Kmin_j )
 * with q+ = max(q, 0), q- = min(q, 0), accumulated in fp32 on the matrix
 * cores (the sum over the group with HSAB_AGG_SUM). Writes j in [0, nb)
 * of each unit; entries [nb, nb_cap) untouched.
 * blk_score: [B][Hkv][nb_cap] fp32; with HSAB_AGG_HEAD [B][Hq][nb_cap],
 * every head's own bound. */
int hsab_score_blocks(const hsab_dims* dims, const uint16_t* q, const uint16_t* meta,
                      const int32_t* ctx_len, float* blk_score, hipStream_t stream);

/* Coarse stage [es 2.A item 1]: block scores as above, then the K_b best
 * blocks per unit (ties to the lower index), ascending, -1 padded.
 * blk_score may be NULL; if given it receives the scores as in
 * hsab_score_blocks. */
int hsab_select_blocks(const hsab_dims* dims, const uint16_t* q, const uint16_t* meta,
                       const int32_t* ctx_len, int32_t* blk_idx, float* blk_score,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* Fine stage [de 2.A Stufe 2; es 2.A item 2]: for every valid token of the
 * blocks listed in blk_idx (ascending, -1 entries ignored) the label score
 *   s_t = max_{h in group} sum_c q_h[label_ch[g][c]] * klabel[t][c]
 * then the K_t best tokens (ties to the lower position), ascending.
 * tok_score may be NULL; if given ([B][Hkv][K_b*block] fp32) it receives
 * the score of candidate i = (slot of the block in blk_idx)*block + offset,
 * -inf for slots that hold no valid token. */
int hsab_select_tokens(const hsab_dims* dims, const uint16_t* q, const uint16_t* klabel,
                       const int32_t* label_ch, const int32_t* blk_idx, const int32_t* ctx_len,
                       int32_t* tok_idx, float* tok_score, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* Exact attention over the kept tokens [es 2.A item 2, final attention]:
 *   out[b][h] = sum_t softmax_t(sm_scale * q_h . K_t) V_t,  t in tok_idx[b][h/G]
 * computed as split partials (max, sum, weighted values) merged by
 * log-sum-exp. -1 entries of tok_idx, and entries at or past ctx_len[b],
 * are skipped (a list with no entry left gives out 0 and lse -inf).
 * slot_of == NULL: K and V are the dense caches above. Otherwise K is the
 * offload engine's block cache [B][Hkv][n_slots][slot] (a slot is block
 * key rows of d_k followed, unless v_alias_k, by block value rows of d_v),
 * V is ignored, and slot_of [B][Hkv][nb_cap] int32 gives the cache slot of
 * block j; a token whose block has a slot outside [0, n_slots) is skipped. */
int hsab_sparse_attend(const hsab_dims* dims, const uint16_t* q, const uint16_t* K,
                       const uint16_t* V, const int32_t* tok_idx, const int32_t* ctx_len,
                       const int32_t* slot_of, int32_t n_slots, float* out, float* lse,
                       void* ws, size_t ws_bytes, hipStream_t stream);

/* One whole decode step on an HBM-resident cache [abstract; de 2.A; es 2.A]:
 * appends the new token at position n-1 (n = ctx_len[b] already counts it):
 * writes its key/value rows, widens the tail block's max/min (or starts
 * the block), writes its label row; then block scores, top-K_b, label
 * scores over the kept blocks, top-K_t and exact attention.
 * k_new [B][Hkv][d_k], v_new [B][Hkv][d_v] (v_new ignored when aliased).
 * Re-running a step with the same inputs is idempotent. */
int hsab_decode_step(const hsab_dims* dims, const uint16_t* q, const uint16_t* k_new,
                     const uint16_t* v_new, uint16_t* K, uint16_t* V, uint16_t* meta,
                     uint16_t* klabel, const int32_t* label_ch, const int32_t* ctx_len,
                     int32_t* blk_idx, int32_t* tok_idx, float* out, float* lse,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* hsab_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under graph capture, serving loops or
 * harnesses that forbid allocation): the same kernels run on a static
 * array of HSAB_SCRATCH_BYTES held by the library on each GPU it runs on
 * (from its first use there until the process ends). The array of the
 * calling thread's current device is used, so `stream` must belong to that
 * device. Nothing is allocated or freed. Returns HSAB_ESCRATCH, before any
 * launch, when hsab_workspace_bytes(dims) > HSAB_SCRATCH_BYTES (every
 * workload of this library's benchmarks fits; per-query-head selection at
 * 96k context does not); otherwise as hsab_decode_step. All calls on one
 * GPU share its array: calls that overlap in time on one GPU (concurrent
 * streams, or several threads) race and give undefined results. */
#define HSAB_SCRATCH_BYTES ((size_t)16 << 20)
int hsab_decode_step_noalloc(const hsab_dims* dims, const uint16_t* q, const uint16_t* k_new,
                             const uint16_t* v_new, uint16_t* K, uint16_t* V, uint16_t* meta,
                             uint16_t* klabel, const int32_t* label_ch, const int32_t* ctx_len,
                             int32_t* blk_idx, int32_t* tok_idx, float* out, float* lse, hipStream_t stream);

/* ------------------------------------------------- label-channel calibration
 * The offline step that chooses the label channels the fine stage scores
 * tokens on (Double Sparsity; AsyncTLS, gist.science/de explainer section
 * 2.A "Stufe 2", gist.science/es explainer section 2.A item 2; the pages do
 * not define "important", this library reads it as below):
 *   importance[g][c] = sum_{s < n_samples} sum_{h in group g} |q_s[h][c] * k_s[g][c]|
 *   label_ch[g]      = the r channels of largest importance (ties to the
 *                      lower channel), ascending
 * q_samples [n_samples][Hq][d_k] bf16 and k_samples [n_samples][Hkv][d_k]
 * bf16 are sampled query / key rows (device); importance [Hkv][d_k] fp32 and
 * label_ch [Hkv][r] int32 are written (device). The sums are fp32 in a fixed
 * order (deterministic). Only batch-independent dims fields are used (Hq,
 * Hkv, d_k, r). HSAB_EINVAL for null pointers or n_samples < 1. */
int hsab_calibrate_labels(const hsab_dims* dims, const uint16_t* q_samples, const uint16_t* k_samples,
                          int32_t n_samples, float* importance, int32_t* label_ch, hipStream_t stream);

/* ------------------------------------------------------------ dense reference
 * Full attention over every token, the operator the sparse step replaces
 * (the pages report the sparse operator's speedup over full attention
 * [abstract; de 4; es 4]):
 *   out[b][h] = sum_{t < n} softmax_t(sm_scale * q_h . K_t) V_t, n = ctx_len[b]
 * with lse as for hsab_sparse_attend. K and V are the dense caches (V NULL
 * when values alias keys); k_blocks, k_tokens, block and r are ignored.
 * Supported for the shapes hsab_sparse_attend supports (HSAB_EUNSUPPORTED
 * otherwise). */
size_t hsab_dense_workspace_bytes(const hsab_dims* dims);   /* 0 if dims invalid or unsupported */
int hsab_dense_attend(const hsab_dims* dims, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                      const int32_t* ctx_len, float* out, float* lse, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* ------------------------------------------------------------------ offload
 * Asynchronous offload engine [de 2.B; es 2.B]: the whole KV cache lives in
 * pinned host memory; a GPU block cache holds the blocks the attention reads.
 * Step t selects S_b(t) on the GPU (metadata and label rows stay on the GPU),
 * attends over R(t) = S_b(t-1) through the block cache, and meanwhile copies
 * only the blocks of S_b(t) not already on the GPU, on a side stream, so
 * they are resident for step t+1. Step 0 attends over S_b(0) after a
 * synchronous fill.
 *
 * Block layout (pool and cache): a block is block*d_k key values followed by
 * block*d_v value values (no values when v_alias_k), bf16.
 *   host_pool  pinned host [B][Hkv][nb_cap][block elements]
 *   cache      device      [B][Hkv][n_slots][block elements]
 *   slot_of    device      [B][Hkv][nb_cap] int32: cache slot of a resident
 *              block; read by hsab_sparse_attend (pass cache as K; V is
 *              ignored in that mode).
 * Slots 0 .. n_slots-3 hold selected blocks; slots n_slots-2 and n_slots-1
 * are tail slots: block j is appended to in slot n_slots-2 + (j & 1), so the
 * block being appended to and the one completed just before it stay on the
 * GPU and never cross the host link. n_slots >= 2*K_b + 2.
 */

/* Append the token at position ctx_len[b]-1 (k_new [B][Hkv][d_k], v_new
 * [B][Hkv][d_v]) into its block's tail slot, widen that block's key max/min
 * (or start it) and write its label row. The caller writes the same rows
 * into host_pool. */
int hsab_offload_append(const hsab_dims* dims, int32_t n_slots, const uint16_t* k_new,
                        const uint16_t* v_new, uint16_t* cache, uint16_t* meta, uint16_t* klabel,
                        const int32_t* label_ch, const int32_t* ctx_len, hipStream_t stream);

/* Host-only planner of one step (no GPU call). All arrays are host memory.
 *   resident  [B][Hkv][K_b] blocks the current step's attention reads, -1 pad
 *   selected  [B][Hkv][K_b] blocks the next step reads, -1 pad
 *   tail      [B][Hkv][2]   block held by tail slot parity p at the next
 *                           step, -1 if none
 *   slot_map  [B][Hkv][nb_cap] in/out host mirror of slot_of
 *   plan      [B][Hkv][K_b][3] out: (block, slot, copy?) for every selected
 *                           block, ascending by block, -1 padded
 *   delta_bytes             out (nullable): bytes to copy
 * A selected block held in a tail slot maps there; one resident in a block
 * slot keeps it; any other is copied into the lowest block slot no resident
 * block uses. Returns HSAB_EINVAL if n_slots is too small. */
int hsab_offload_plan(const hsab_dims* dims, int32_t n_slots, const int32_t* resident,
                      const int32_t* selected, const int32_t* tail, int32_t* slot_map, int32_t* plan,
                      int64_t* delta_bytes);

/* How the delta crosses the host link:
 *   HSAB_OFFLOAD_COPY_KERNEL  a GPU kernel reads the blocks from the pinned
 *       pool (hipHostMalloc memory, mapped into the GPU address space) and
 *       writes them to their slots, then a second kernel patches slot_of
 *       (a reader of slot_of finds a block's old slot or a finished copy);
 *   HSAB_OFFLOAD_COPY_DMA     the DMA engines copy each run of consecutive
 *       blocks into consecutive slots (one hipMemcpyAsync per run), then a
 *       kernel patches slot_of. */
#define HSAB_OFFLOAD_COPY_KERNEL 0
#define HSAB_OFFLOAD_COPY_DMA    1
/* Engine only: kernel copies whose plan the copy stream makes on the GPU
 * (the same rules as hsab_offload_plan), so hsab_offload_step never waits
 * on the host; the step's delta bytes come from hsab_offload_step_delta. */
#define HSAB_OFFLOAD_COPY_KERNEL_GPU_PLAN 2

/* Enqueue a plan on copy_stream: the block copies as copy_mode says, the
 * upload of the plan (plan must be pinned host memory; plan_dev is device
 * [B][Hkv][K_b][3] int32), slot_of written for every planned block, then
 * `done` (nullable) is recorded. host_pool (pinned) and cache must be
 * 16-byte aligned. n_copies (nullable) receives the blocks gathered
 * (kernel) or the copies issued (DMA). */
int hsab_offload_copy(const hsab_dims* dims, int32_t n_slots, const uint16_t* host_pool, uint16_t* cache,
                      const int32_t* plan, int32_t* plan_dev, int32_t* slot_of, int32_t copy_mode,
                      hipStream_t copy_stream, hipEvent_t done, int32_t* n_copies);

/* Offload engine object: the lagged schedule above driven step by step.
 * It owns only small buffers (in coherent pinned memory S_b, the plans,
 * copy lists and per-step copy counts; on the GPU the selections, plans,
 * copy lists and slot map of the device planner) and events, allocated by
 * hsab_offload_create and freed by hsab_offload_destroy; the caller owns
 * the pool, the block cache, metadata, label rows and outputs. Unlike the
 * rest of the library, hsab_offload_step waits on the host (for S_b(t),
 * which the selection kernel writes into the engine's mapped pinned
 * buffer) once per step, except with HSAB_OFFLOAD_COPY_KERNEL_GPU_PLAN,
 * where the copy stream plans the delta on the GPU (the same rules as
 * hsab_offload_plan) and the host does not wait. One engine serves one
 * caller thread. */
typedef struct hsab_offload_engine hsab_offload_engine;

/* With GPU planning the plan is made after the call returns:
 * delta_bytes, cold_bytes, delta_blocks and n_copies are then -1, and
 * hsab_offload_step_delta gives the bytes once the step's copies ran. */
typedef struct hsab_offload_stats {
    int64_t step;          /* index of the step just enqueued (0 = cold start) */
    int64_t delta_bytes;   /* host-to-device bytes of the step's delta */
    int64_t cold_bytes;    /* bytes of the synchronous fill of S_b(0); step 0 only */
    int32_t delta_blocks;  /* blocks in the delta */
    int32_t n_copies;      /* blocks gathered (kernel copy) or copies issued (DMA copy) */
    float host_wait_ms;    /* host wait for S_b(t) */
    float host_plan_ms;    /* planning and enqueue of the copies */
} hsab_offload_stats;

/* n_slots >= 2*K_b + 2; copy_mode is HSAB_OFFLOAD_COPY_KERNEL, _DMA or
 * _KERNEL_GPU_PLAN (HSAB_EINVAL for the last when n_slots is beyond what
 * the device planner holds in LDS: 2*ceil((n_slots-2)/32) + K_b > 15360);
 * HSAB_EUNSUPPORTED for per-query-head selection (HSAB_AGG_HEAD: blocks
 * move per KV head) and for shapes the attention does not take; HSAB_EHIP
 * if an allocation fails. */
int hsab_offload_create(const hsab_dims* dims, int32_t n_slots, int32_t copy_mode, hsab_offload_engine** engine);
void hsab_offload_destroy(hsab_offload_engine* engine);

/* After prefill (host_pool holds n_prefill[b] tokens of every sequence,
 * meta/klabel built on the GPU, e.g. by hsab_build_meta): copies each
 * unit's last prefill block into its tail slot, resets slot_of and the
 * engine's step counter. n_prefill is host memory, 0 <= n_prefill[b] <
 * max_ctx. Synchronous. */
int hsab_offload_begin(hsab_offload_engine* engine, const int32_t* n_prefill, const uint16_t* host_pool,
                       uint16_t* cache, int32_t* slot_of, hipStream_t stream);

/* Decode step t [de 2.B; es 2.B]: appends k_new/v_new (device, written to
 * the tail slot, meta, klabel, and by the same kernel to host_pool through
 * its device mapping; host_pool must be pinned, hipHostMalloc memory),
 * selects S_b(t), runs the token stage and attention over R(t) = S_b(t-1) through
 * the block cache (R(0) = S_b(0) after a synchronous fill), and enqueues
 * the delta for step t+1 on copy_stream. ctx_len (device) and ctx_len_host
 * hold the same lengths, one more than at the previous step; only work on
 * compute_stream reads ctx_len (the copy stream plans from a copy the step
 * takes), so the caller may update it in place by work it enqueues on
 * compute_stream after this call. The step's inputs (q, k_new, v_new) are
 * read by compute_stream only. tok_idx, out
 * and lse are as for hsab_decode_step; ws is a workspace of
 * hsab_workspace_bytes. stats is nullable. Steps may be enqueued
 * back to back without synchronising in between: each step's attention
 * waits on the GPU for the previous step's copies. */
int hsab_offload_step(hsab_offload_engine* engine, const uint16_t* q, const uint16_t* k_new,
                      const uint16_t* v_new, uint16_t* host_pool, uint16_t* cache, uint16_t* meta,
                      uint16_t* klabel, const int32_t* label_ch, const int32_t* ctx_len,
                      const int32_t* ctx_len_host, int32_t* slot_of, int32_t* tok_idx, float* out, float* lse,
                      void* ws, size_t ws_bytes, hipStream_t compute_stream, hipStream_t copy_stream,
                      hsab_offload_stats* stats);

/* Per-step GPU timestamps for hsab_offload_timing, for the steps enqueued
 * after this call while enable is nonzero. Off by default: the six timed
 * event records of a step are markers the GPU processes in stream order,
 * and cost the step several microseconds. HSAB_EINVAL for a null engine. */
int hsab_offload_set_timing(hsab_offload_engine* engine, int32_t enable);

/* GPU times (ms) of a step among the last 32 that was enqueued with timing
 * on, waiting for them (ms has 5 entries): ms[0] compute stream span of the
 * step, ms[1] span of the step's copies on the copy stream, ms[2] and ms[3]
 * their start and end relative to the step's compute start, ms[4] how long
 * the compute stream waited for the previous step's copies (the cold fill
 * at step 0) before its attention. HSAB_EINVAL for a step outside that
 * window or enqueued without timing. */
int hsab_offload_timing(hsab_offload_engine* engine, int64_t step, float* ms);

/* Host copy of the last step's S_b [B][Hkv][K_b] (ascending, -1 padded);
 * waits for that step's block selection. */
int hsab_offload_selection(const hsab_offload_engine* engine, int32_t* blk_idx_host);

/* Host copy of S_b [B][Hkv][K_b] of a step among the last 32 enqueued
 * (ascending, -1 padded), waiting for that step's selection (with GPU
 * planning, for that step's copies). Lets a caller that enqueues several
 * steps without synchronising read every step's selection afterwards.
 * HSAB_EINVAL for a null pointer or a step outside that window; HSAB_EHIP
 * if the wait fails. */
int hsab_offload_step_selection(hsab_offload_engine* engine, int64_t step, int32_t* blk_idx_host);

/* Delta bytes (and, for step 0, the cold-fill bytes; else 0) of a step
 * among the last 32 enqueued, waiting for that step's copies when the GPU
 * planned them. HSAB_EINVAL for a null pointer or a step outside that
 * window; HSAB_EHIP if the wait fails. */
int hsab_offload_step_delta(hsab_offload_engine* engine, int64_t step, int64_t* delta_bytes, int64_t* cold_bytes);

#ifdef __cplusplus
}
#endif
#endif /* HSAB_H */
