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
 *   meta     [B][Hkv][nb_cap][2][d_k]             bf16: per block, the
 *            channelwise key max row followed by the key min row.
 *   klabel   [B][Hkv][max_ctx][r]                 bf16: K restricted to the
 *            label channels, klabel[..][t][c] = K[..][t][label_ch[g][c]].
 *   label_ch [Hkv][r]                             int32 channel indices.
 *   ctx_len  [B]                                  int32, 1 <= n <= max_ctx.
 *   blk_idx  [B][Hkv][K_b]                        int32 ascending, -1 padded.
 *   tok_idx  [B][Hkv][K_t]                        int32 token positions,
 *            ascending, -1 padded.
 *   out      [B][Hq][d_v]                         fp32 attention output.
 *   lse      [B][Hq]                              fp32 natural-log
 *            logsumexp of the logits sm_scale*q.k over the kept tokens.
 *
 * Inputs must be finite (no inf/NaN in q, K, V or the new token).
 *
 * Selection rules (the pages leave them open; fixed here):
 *   - query heads sharing a KV head are combined by the maximum over the
 *     group, for block scores and token scores; one selection per unit;
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

/* Shape and budget of one decode layer.
 * Limits: 1 <= G <= 32; d_k % 16 == 0, 16 <= d_k <= 1024; d_v % 8 == 0;
 * r in {16, 32, 64, 128}, r <= d_k; 1 <= K_b <= 2048;
 * K_b * block <= 8192; nb_cap <= 8192; K_t >= 1.
 * Attention kernels exist for d_k == d_v in {64, 128, 256} with G in
 * {1, 2, 4, 8} (GQA/MQA/MHA); other shapes return HSAB_EUNSUPPORTED from
 * hsab_sparse_attend and hsab_decode_step. */
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
} hsab_dims;

/* Bytes of device workspace the calls below need for these dims (the same
 * size serves every call). The workspace holds block scores, token scores
 * and split-attention partials; it needs no initialisation. */
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
 * cores. Writes j in [0, nb) of each unit; entries [nb, nb_cap) untouched.
 * blk_score: [B][Hkv][nb_cap] fp32. */
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
 * log-sum-exp. -1 entries of tok_idx are skipped.
 * slot_of == NULL: K and V are the dense caches above. Otherwise K and V
 * are block caches [B][Hkv][n_slots][block][d] (same row layout) and
 * slot_of [B][Hkv][nb_cap] int32 gives the cache slot of block j
 * (used by the offload engine; a token whose block has slot < 0 is skipped). */
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

#ifdef __cplusplus
}
#endif
#endif /* HSAB_H */
