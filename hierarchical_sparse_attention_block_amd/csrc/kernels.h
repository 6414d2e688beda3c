// Internal launchers of libhsab (host side). Each returns hipError_t of
// the launch; shapes were validated by the C-ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include "../../include/hsab.h"

namespace hsab {

// Limits enforced by the C-ABI validation and assumed by the kernels.
constexpr int MAX_NB = 8192;         // blocks per unit (block-score top-k keys)
constexpr int MAX_CAND = 8192;       // K_b * block (token-score top-k keys)
constexpr int MAX_KB = 2048;         // K_b
constexpr int MAX_G = 32;            // query heads per KV head
constexpr int MAX_R = 128;           // label channels
constexpr int ATT_TOK_PER_SPLIT = 64;    // tokens per attention workgroup (GQA path)
constexpr int ATT_TOK_PER_SPLIT_LONG = 128;   // GQA path when 64-token splits need more than one round
constexpr int ATT_ROUND_WGS = 1024;      // GQA attention workgroups resident at once (four per CU)
constexpr int MLA_TOK_PER_SPLIT = 64;    // tokens per attention workgroup (MLA path)

// group score modes (dims.group_agg)
constexpr int AGG_MAX = HSAB_AGG_MAX;
constexpr int AGG_SUM = HSAB_AGG_SUM;
constexpr int AGG_HEAD = HSAB_AGG_HEAD;

struct Shape {
    int B, Hq, Hkv, G, dk, dv, valias, bs, r, kb, kt, max_ctx, nb_cap;
    float sm_scale;
    int meta8;   // block metadata in fp8 e4m3 (outward rounded) instead of bf16
    int lab8;    // label rows in fp8 e4m3 (nearest) instead of bf16
    int agg;     // AGG_MAX, AGG_SUM or AGG_HEAD (every query head selects on its own)
    int agg_sum; // agg == AGG_SUM
    int heads;   // selections per unit: G with AGG_HEAD, else 1
    int sink, local;   // always-kept first / last blocks
};

Shape make_shape(const hsab_dims& d);
int attn_splits(const Shape& s);
// list entries per attention workgroup (one split)
int attn_tok_per_split(const Shape& s);
// entries of a unit's attention token list: K_t, or G * K_t (the union of
// the heads' token sets) with per-head selection
int attn_list_len(const Shape& s);

// workspace carve-up (byte offsets, 256-aligned)
struct WsLayout {
    size_t blk_score, part_ml, part_acc, sel_keys, sel_cnt, union_idx, union_mask, total;
};
WsLayout ws_layout(const Shape& s);

hipError_t launch_build_meta(const Shape& s, const uint16_t* K, const int32_t* ctx_len,
                             const int32_t* label_ch, uint16_t* meta, uint16_t* klabel,
                             hipStream_t st);
// A split token selection's shared state in the workspace: one arrival
// counter per selection ([U * heads]) and the candidate keys the parts
// publish ([U * heads][K_b * block]). The block-score launch of the same
// step sets every counter to zero and every key to KEY_PENDING, a value no
// key takes (0 marks an empty candidate; f32_key maps every number to
// 0x007fffff or more), so the part that arrives last can tell a key not yet
// visible to it from a stored one.
struct Handoff {
    int32_t* cnt;
    uint32_t* keys;
    int keys_per_sel;
};
constexpr uint32_t KEY_PENDING = 1u;
// Block scores ([U][nb_cap], or [U][G][nb_cap] with per-head selection);
// with k_new non-null the decode-step append runs first. ho (nullable): the
// shared state of a following split token selection, reset here.
hipError_t launch_block_score(const Shape& s, const uint16_t* q, uint16_t* meta, const int32_t* ctx_len,
                              float* score, const uint16_t* k_new, const uint16_t* v_new, uint16_t* K,
                              uint16_t* V, uint16_t* klabel, const int32_t* label_ch, const Handoff* ho,
                              hipStream_t st);
// mode bit 1: select blocks from block scores; bit 2: score + select tokens.
// With sel_keys and sel_cnt non-null (counters zero and keys KEY_PENDING on
// entry: the block-score launch of the step resets them, see Handoff) the
// token stage of each selection is spread over several workgroups. Per-head selection runs U * G selections, each of one query
// head (block lists [U][G][K_b], token lists [U][G][K_t]). blk_copy
// (nullable): a second buffer that receives the same block lists (e.g.
// host memory mapped into the GPU).
hipError_t launch_select(const Shape& s, int mode, const uint16_t* q, const float* blk_score,
                         const uint16_t* klabel, const int32_t* label_ch, const int32_t* ctx_len,
                         int32_t* blk_idx, int32_t* tok_idx, float* tok_score, uint32_t* sel_keys,
                         int32_t* sel_cnt, hipStream_t st, int32_t* blk_copy = nullptr);
bool attend_supported(const Shape& s);
// Per-head selection: the ascending union of the G token lists of each
// unit ([U][G][K_t] -> [U][G*K_t], -1 padded) and, per entry, the bit mask
// of the heads that selected it.
hipError_t launch_union(const Shape& s, const int32_t* tok_idx, const int32_t* ctx_len, int32_t* union_idx,
                        uint32_t* union_mask, hipStream_t st);
// Split attention over the kept tokens, then the merge of the partials.
// tok_idx: [U][list_len]; tok_mask (nullable): per entry the query heads
// of the group that attend it (all when null); entries at or past
// ctx_len[b] are skipped.
hipError_t launch_attend(const Shape& s, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                         const int32_t* tok_idx, const uint32_t* tok_mask, int list_len, const int32_t* ctx_len,
                         const int32_t* slot_of, int n_slots, float* part_ml, float* part_acc, float* out,
                         float* lse, hipStream_t st);

// Merge of per-split (max, sum, weighted values) partials into out / lse.
hipError_t launch_combine(const Shape& s, const float* part_ml, const float* part_acc, float* out, float* lse,
                          int n_splits, hipStream_t st);

// Dense decode attention over every token of the context (dense.hip): the
// full-attention reference the sparse operator is measured against.
constexpr int DENSE_CHUNK = 1024;     // tokens per workgroup
bool dense_supported(const Shape& s);
size_t dense_workspace_bytes(const Shape& s);
hipError_t launch_dense(const Shape& s, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                        const int32_t* ctx_len, float* out, float* lse, void* ws, hipStream_t st);

// Label-channel calibration from n_samples sampled (query, key) pairs (calib.hip).
hipError_t launch_calibrate(const Shape& s, const uint16_t* q_samples, const uint16_t* k_samples, int n_samples,
                            float* importance, int32_t* label_ch, hipStream_t st);

// offload engine (offload.hip); per-step timing events kept for this many steps
constexpr int TIMING_RING = 32;
hipError_t launch_append_slot(const Shape& s, int n_slots, const uint16_t* k_new, const uint16_t* v_new,
                              uint16_t* cache, uint16_t* meta, uint16_t* klabel, const int32_t* label_ch,
                              const int32_t* ctx_len, hipStream_t st, uint16_t* pool_dev = nullptr,
                              int32_t* ctx_copy = nullptr);
int offload_plan(const Shape& s, int n_slots, const int32_t* resident, const int32_t* selected,
                 const int32_t* tail, int32_t* slot_map, int32_t* plan, int64_t* delta_bytes);
constexpr int OFFLOAD_COPY_KERNEL = HSAB_OFFLOAD_COPY_KERNEL;
constexpr int OFFLOAD_COPY_DMA = HSAB_OFFLOAD_COPY_DMA;
constexpr int OFFLOAD_COPY_KERNEL_GPU_PLAN = HSAB_OFFLOAD_COPY_KERNEL_GPU_PLAN;
// The offload engine's plan buffers in coherent pinned memory: the copy
// lists ([U][K_b] pairs) and counts ([U]) the host fills, and the device
// addresses of those, of the plan and of the pool.
struct MappedPlan {
    int32_t* list_h = nullptr;
    int32_t* cnt_h = nullptr;
    const int32_t* plan_dev = nullptr;
    const int32_t* list_dev = nullptr;
    const int32_t* cnt_dev = nullptr;
    const uint16_t* pool_dev = nullptr;
};
hipError_t offload_copy(const Shape& s, int n_slots, const uint16_t* host_pool, uint16_t* cache,
                        const int32_t* plan, int32_t* plan_dev, int32_t* slot_of, hipStream_t cs,
                        hipEvent_t done, int* n_copies, int mode, const MappedPlan* mp);
hipError_t offload_create(const Shape& s, int n_slots, int copy_mode, hsab_offload_engine** out);
void offload_destroy(hsab_offload_engine* e);
hipError_t offload_begin(hsab_offload_engine* e, const int32_t* n_prefill, const uint16_t* host_pool,
                         uint16_t* cache, int32_t* slot_of, hipStream_t st);
// *einval is set when the context lengths or the slot count do not fit.
hipError_t offload_step(hsab_offload_engine* e, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                        uint16_t* host_pool, uint16_t* cache, uint16_t* meta, uint16_t* klabel,
                        const int32_t* label_ch, const int32_t* ctx_len, const int32_t* ctx_len_host,
                        int32_t* slot_of, int32_t* tok_idx, float* out, float* lse, void* ws, hipStream_t cs,
                        hipStream_t xs, hsab_offload_stats* st, int* einval);
hipError_t offload_timing(hsab_offload_engine* e, int64_t step, float* ms4);
void offload_set_timing(hsab_offload_engine* e, bool on);
bool offload_step_timed(const hsab_offload_engine* e, int64_t step);
const int32_t* offload_last_selection(hsab_offload_engine* e);
const int32_t* offload_step_selection(hsab_offload_engine* e, int64_t step);
hipError_t offload_step_delta(hsab_offload_engine* e, int64_t step, int64_t* delta_bytes, int64_t* cold_bytes);
int64_t offload_steps(const hsab_offload_engine* e);
const Shape& offload_shape(const hsab_offload_engine* e);

}  // namespace hsab
