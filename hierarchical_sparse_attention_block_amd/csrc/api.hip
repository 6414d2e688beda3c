// C ABI of libhsab: argument checks, workspace layout and kernel sequencing.
// Apart from the offload engine object (hsab_offload_create/_begin/_step),
// the library never allocates, frees or synchronises; every call enqueues
// its kernels on the caller's stream.
#include <math.h>
#include <string.h>

#include <mutex>

#include "kernels.h"

namespace hsab {

static thread_local int g_last_hip = 0;

Shape make_shape(const hsab_dims& d) {
    Shape s;
    s.B = d.batch; s.Hq = d.n_q_heads; s.Hkv = d.n_kv_heads;
    s.G = d.n_kv_heads > 0 ? d.n_q_heads / d.n_kv_heads : 0;
    s.dk = d.d_k; s.dv = d.d_v; s.valias = d.v_alias_k != 0;
    s.bs = d.block; s.r = d.r; s.kb = d.k_blocks; s.kt = d.k_tokens; s.max_ctx = d.max_ctx;
    s.nb_cap = d.block > 0 ? (d.max_ctx + d.block - 1) / d.block : 0;
    s.sm_scale = d.sm_scale;
    s.meta8 = d.meta_format == HSAB_META_FP8;
    s.lab8 = d.label_format == HSAB_LABEL_FP8;
    s.agg = d.group_agg;
    s.agg_sum = d.group_agg == HSAB_AGG_SUM;
    s.heads = d.group_agg == HSAB_AGG_HEAD ? s.G : 1;
    s.sink = d.sink_blocks;
    s.local = d.local_blocks;
    return s;
}

int attn_list_len(const Shape& s) { return s.kt * s.heads; }

int attn_tok_per_split(const Shape& s) {
    if (s.valias) return MLA_TOK_PER_SPLIT;
    // GQA: 64-token splits while they fit one round of resident workgroups;
    // beyond that, 128-token splits (for d <= 128) halve the workgroups
    // instead of running a second round
    const long wgs = (long)s.B * s.Hkv * ((attn_list_len(s) + ATT_TOK_PER_SPLIT - 1) / ATT_TOK_PER_SPLIT);
    return wgs > ATT_ROUND_WGS && s.dk <= 128 ? ATT_TOK_PER_SPLIT_LONG : ATT_TOK_PER_SPLIT;
}

int attn_splits(const Shape& s) {
    const int tps = attn_tok_per_split(s);
    return (attn_list_len(s) + tps - 1) / tps;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(const Shape& s) {
    WsLayout w;
    size_t off = 0;
    const size_t sels = (size_t)s.B * s.Hkv * s.heads;   // selections
    w.blk_score = off; off = align256(off + sels * s.nb_cap * sizeof(float));
    w.part_ml = off;   off = align256(off + (size_t)s.B * s.Hq * attn_splits(s) * 2 * sizeof(float));
    w.part_acc = off;  off = align256(off + (size_t)s.B * s.Hq * attn_splits(s) * s.dv * sizeof(float));
    w.sel_keys = off;  off = align256(off + sels * s.kb * s.bs * sizeof(uint32_t));
    w.sel_cnt = off;   off = align256(off + sels * sizeof(int32_t));
    const size_t ulen = s.heads > 1 ? (size_t)s.B * s.Hkv * attn_list_len(s) : 0;
    w.union_idx = off;  off = align256(off + ulen * sizeof(int32_t));
    w.union_mask = off; off = align256(off + ulen * sizeof(uint32_t));
    w.total = off;
    return w;
}

// Shape checks shared by every entry point.
static int check_dims(const hsab_dims* d) {
    if (!d) return HSAB_EINVAL;
    if (d->batch < 1 || d->n_kv_heads < 1 || d->n_q_heads < 1) return HSAB_EINVAL;
    if (d->n_q_heads % d->n_kv_heads != 0) return HSAB_EINVAL;
    const int G = d->n_q_heads / d->n_kv_heads;
    if (G > MAX_G) return HSAB_EINVAL;
    if (d->d_k < 16 || d->d_k > 1024 || d->d_k % 16 != 0) return HSAB_EINVAL;
    if (d->d_v < 8 || d->d_v % 8 != 0) return HSAB_EINVAL;
    if (d->v_alias_k && d->d_v > d->d_k) return HSAB_EINVAL;
    if (d->block < 1 || d->max_ctx < 1) return HSAB_EINVAL;
    if ((d->r != 16 && d->r != 32 && d->r != 64 && d->r != 128) || d->r > d->d_k) return HSAB_EINVAL;
    if (d->k_blocks < 1 || d->k_blocks > MAX_KB) return HSAB_EINVAL;
    if ((long)d->k_blocks * d->block > MAX_CAND) return HSAB_EINVAL;
    if (d->k_tokens < 1) return HSAB_EINVAL;
    if ((d->max_ctx + d->block - 1) / d->block > MAX_NB) return HSAB_EINVAL;
    if (!isfinite(d->sm_scale)) return HSAB_EINVAL;
    if (d->meta_format != HSAB_META_BF16 && d->meta_format != HSAB_META_FP8) return HSAB_EINVAL;
    if (d->meta_format == HSAB_META_FP8 && d->d_k % 32 != 0) return HSAB_EINVAL;   // whole 64-byte row loads
    if (d->label_format != HSAB_LABEL_BF16 && d->label_format != HSAB_LABEL_FP8) return HSAB_EINVAL;
    if (d->group_agg != HSAB_AGG_MAX && d->group_agg != HSAB_AGG_SUM && d->group_agg != HSAB_AGG_HEAD)
        return HSAB_EINVAL;
    if (d->sink_blocks < 0 || d->local_blocks < 0 || d->sink_blocks + d->local_blocks > d->k_blocks)
        return HSAB_EINVAL;
    return HSAB_OK;
}

static int hip_status(hipError_t e) {
    if (e == hipSuccess) return HSAB_OK;
    g_last_hip = (int)e;
    return HSAB_EHIP;
}

// Attention over the kept tokens: with per-head selection the heads' lists
// are merged into their union (with head masks) in the workspace first
// (with one head per group the list is already its own union).
static int attend_step(const Shape& s, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                       const int32_t* tok_idx, const int32_t* ctx_len, const int32_t* slot_of, int n_slots, char* w,
                       const WsLayout& L, float* out, float* lse, hipStream_t stream) {
    const int32_t* list = tok_idx;
    const uint32_t* mask = nullptr;
    if (s.heads > 1) {
        int32_t* uidx = reinterpret_cast<int32_t*>(w + L.union_idx);
        uint32_t* umask = reinterpret_cast<uint32_t*>(w + L.union_mask);
        const int rc = hip_status(launch_union(s, tok_idx, ctx_len, uidx, umask, stream));
        if (rc) return rc;
        list = uidx;
        mask = umask;
    }
    return hip_status(launch_attend(s, q, K, V, list, mask, attn_list_len(s), ctx_len, slot_of, n_slots,
                                    reinterpret_cast<float*>(w + L.part_ml),
                                    reinterpret_cast<float*>(w + L.part_acc), out, lse, stream));
}

static int decode_step_ws(const hsab_dims* dims, const uint16_t* q, const uint16_t* k_new,
                          const uint16_t* v_new, uint16_t* K, uint16_t* V, uint16_t* meta,
                          uint16_t* klabel, const int32_t* label_ch, const int32_t* ctx_len,
                          int32_t* blk_idx, int32_t* tok_idx, float* out, float* lse, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    const Shape s = make_shape(*dims);
    if (!q || !k_new || !K || !meta || !klabel || !label_ch || !ctx_len || !blk_idx || !tok_idx ||
        !out || !lse)
        return HSAB_EINVAL;
    if (!s.valias && (!V || !v_new)) return HSAB_EINVAL;
    const WsLayout L = ws_layout(s);
    if (!ws || ws_bytes < L.total) return HSAB_EINVAL;
    if (!attend_supported(s)) return HSAB_EUNSUPPORTED;
    char* w = static_cast<char*>(ws);
    float* scores = reinterpret_cast<float*>(w + L.blk_score);
    uint32_t* sel_keys = reinterpret_cast<uint32_t*>(w + L.sel_keys);
    int32_t* sel_cnt = reinterpret_cast<int32_t*>(w + L.sel_cnt);
    // 1) append + block scores (and zeroed selection counters); 2) top-K_b,
    // label scores, top-K_t; 3) split attention and the merge of its partials
    const Handoff ho{sel_cnt, sel_keys, s.kb * s.bs};
    rc = hip_status(launch_block_score(s, q, meta, ctx_len, scores, k_new, v_new, K, V, klabel, label_ch, &ho,
                                       stream));
    if (rc) return rc;
    rc = hip_status(launch_select(s, 3, q, scores, klabel, label_ch, ctx_len, blk_idx, tok_idx, nullptr,
                                  sel_keys, sel_cnt, stream));
    if (rc) return rc;
    return attend_step(s, q, K, s.valias ? K : V, tok_idx, ctx_len, nullptr, 0, w, L, out, lse, stream);
}

// The allocation-free step's workspace: one fixed array per GPU, held from
// the library's first use on that GPU until the process ends. Host code
// never passes `scratch` itself (its host-side name is no device address);
// it passes the address hipGetSymbolAddress gives for the current device.
static __device__ __align__(256) unsigned char scratch[HSAB_SCRATCH_BYTES];
constexpr int SCRATCH_DEVICES = 64;
static void* g_scratch_ptr[SCRATCH_DEVICES];
static hipError_t g_scratch_err[SCRATCH_DEVICES];
static std::once_flag g_scratch_once[SCRATCH_DEVICES];

// Device address of the current device's scratch array, looked up once per
// device (with that device current).
static hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= SCRATCH_DEVICES) return hipErrorInvalidDevice;
    std::call_once(g_scratch_once[dev], [dev] {
        g_scratch_err[dev] = hipGetSymbolAddress(&g_scratch_ptr[dev], HIP_SYMBOL(scratch));
    });
    if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace hsab

using namespace hsab;

extern "C" {

size_t hsab_workspace_bytes(const hsab_dims* dims) {
    if (check_dims(dims) != HSAB_OK) return 0;
    return ws_layout(make_shape(*dims)).total;
}

const char* hsab_status_string(int status) {
    switch (status) {
        case HSAB_OK: return "ok";
        case HSAB_EINVAL: return "invalid argument";
        case HSAB_EHIP: return "HIP launch or runtime error";
        case HSAB_EUNSUPPORTED: return "shape not supported by the available kernels";
        case HSAB_ESCRATCH: return "workspace larger than the static scratch of hsab_decode_step_noalloc";
        default: return "unknown status";
    }
}

int hsab_last_hip_error(void) { return g_last_hip; }

int hsab_build_meta(const hsab_dims* dims, const uint16_t* K, const int32_t* ctx_len,
                    const int32_t* label_ch, uint16_t* meta, uint16_t* klabel, hipStream_t stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (!K || !ctx_len || !label_ch || !meta || !klabel) return HSAB_EINVAL;
    return hip_status(launch_build_meta(make_shape(*dims), K, ctx_len, label_ch, meta, klabel, stream));
}

int hsab_score_blocks(const hsab_dims* dims, const uint16_t* q, const uint16_t* meta,
                      const int32_t* ctx_len, float* blk_score, hipStream_t stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (!q || !meta || !ctx_len || !blk_score) return HSAB_EINVAL;
    return hip_status(launch_block_score(make_shape(*dims), q, const_cast<uint16_t*>(meta), ctx_len,
                                         blk_score, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                         nullptr, stream));
}

int hsab_select_blocks(const hsab_dims* dims, const uint16_t* q, const uint16_t* meta,
                       const int32_t* ctx_len, int32_t* blk_idx, float* blk_score, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (!q || !meta || !ctx_len || !blk_idx) return HSAB_EINVAL;
    const Shape s = make_shape(*dims);
    const WsLayout L = ws_layout(s);
    float* scores = blk_score;
    if (!scores) {
        if (!ws || ws_bytes < L.total) return HSAB_EINVAL;
        scores = reinterpret_cast<float*>(static_cast<char*>(ws) + L.blk_score);
    }
    rc = hip_status(launch_block_score(s, q, const_cast<uint16_t*>(meta), ctx_len, scores, nullptr,
                                       nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, stream));
    if (rc) return rc;
    return hip_status(launch_select(s, 1, q, scores, nullptr, nullptr, ctx_len, blk_idx, nullptr,
                                    nullptr, nullptr, nullptr, stream));
}

int hsab_select_tokens(const hsab_dims* dims, const uint16_t* q, const uint16_t* klabel,
                       const int32_t* label_ch, const int32_t* blk_idx, const int32_t* ctx_len,
                       int32_t* tok_idx, float* tok_score, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
    (void)ws; (void)ws_bytes;
    int rc = check_dims(dims);
    if (rc) return rc;
    if (!q || !klabel || !label_ch || !blk_idx || !ctx_len || !tok_idx) return HSAB_EINVAL;
    return hip_status(launch_select(make_shape(*dims), 2, q, nullptr, klabel, label_ch, ctx_len,
                                    const_cast<int32_t*>(blk_idx), tok_idx, tok_score, nullptr, nullptr,
                                    stream));
}

int hsab_sparse_attend(const hsab_dims* dims, const uint16_t* q, const uint16_t* K,
                       const uint16_t* V, const int32_t* tok_idx, const int32_t* ctx_len,
                       const int32_t* slot_of, int32_t n_slots, float* out, float* lse, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    const Shape s = make_shape(*dims);
    if (!q || !K || !tok_idx || !ctx_len || !out || !lse) return HSAB_EINVAL;
    if (!s.valias && !V && !slot_of) return HSAB_EINVAL;   // a block cache carries its values
    if (slot_of && n_slots < 1) return HSAB_EINVAL;
    const WsLayout L = ws_layout(s);
    if (!ws || ws_bytes < L.total) return HSAB_EINVAL;
    if (!attend_supported(s)) return HSAB_EUNSUPPORTED;
    char* w = static_cast<char*>(ws);
    return attend_step(s, q, K, s.valias ? K : V, tok_idx, ctx_len, slot_of, n_slots, w, L, out, lse, stream);
}


int hsab_decode_step(const hsab_dims* dims, const uint16_t* q, const uint16_t* k_new,
                     const uint16_t* v_new, uint16_t* K, uint16_t* V, uint16_t* meta,
                     uint16_t* klabel, const int32_t* label_ch, const int32_t* ctx_len,
                     int32_t* blk_idx, int32_t* tok_idx, float* out, float* lse, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
    return decode_step_ws(dims, q, k_new, v_new, K, V, meta, klabel, label_ch, ctx_len, blk_idx, tok_idx, out,
                          lse, ws, ws_bytes, stream);
}

int hsab_decode_step_noalloc(const hsab_dims* dims, const uint16_t* q, const uint16_t* k_new,
                             const uint16_t* v_new, uint16_t* K, uint16_t* V, uint16_t* meta,
                             uint16_t* klabel, const int32_t* label_ch, const int32_t* ctx_len,
                             int32_t* blk_idx, int32_t* tok_idx, float* out, float* lse, hipStream_t stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    const size_t need = ws_layout(make_shape(*dims)).total;
    if (need > HSAB_SCRATCH_BYTES) return HSAB_ESCRATCH;
    void* ws = nullptr;
    rc = hip_status(scratch_address(&ws));
    if (rc) return rc;
    // the workspace needs no clearing: the selection counters in it are set
    // to zero by the step's first kernel, everything else is written before
    // it is read
    return decode_step_ws(dims, q, k_new, v_new, K, V, meta, klabel, label_ch, ctx_len, blk_idx, tok_idx, out,
                          lse, ws, HSAB_SCRATCH_BYTES, stream);
}

int hsab_calibrate_labels(const hsab_dims* dims, const uint16_t* q_samples, const uint16_t* k_samples,
                          int32_t n_samples, float* importance, int32_t* label_ch, hipStream_t stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (!q_samples || !k_samples || !importance || !label_ch || n_samples < 1) return HSAB_EINVAL;
    return hip_status(launch_calibrate(make_shape(*dims), q_samples, k_samples, n_samples, importance, label_ch,
                                       stream));
}

size_t hsab_dense_workspace_bytes(const hsab_dims* dims) {
    if (check_dims(dims) != HSAB_OK) return 0;
    const Shape s = make_shape(*dims);
    return dense_supported(s) ? dense_workspace_bytes(s) : 0;
}

int hsab_dense_attend(const hsab_dims* dims, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                      const int32_t* ctx_len, float* out, float* lse, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (!q || !K || !ctx_len || !out || !lse) return HSAB_EINVAL;
    const Shape s = make_shape(*dims);
    if (!s.valias && !V) return HSAB_EINVAL;
    if (!dense_supported(s)) return HSAB_EUNSUPPORTED;
    if (!ws || ws_bytes < dense_workspace_bytes(s)) return HSAB_EINVAL;
    return hip_status(launch_dense(s, q, K, V, ctx_len, out, lse, ws, stream));
}

int hsab_offload_append(const hsab_dims* dims, int32_t n_slots, const uint16_t* k_new,
                        const uint16_t* v_new, uint16_t* cache, uint16_t* meta, uint16_t* klabel,
                        const int32_t* label_ch, const int32_t* ctx_len, hipStream_t stream) {
    int rc = check_dims(dims);
    if (rc) return rc;
    const Shape s = make_shape(*dims);
    if (n_slots < 2 * s.kb + 2) return HSAB_EINVAL;
    if (!k_new || !cache || !meta || !klabel || !label_ch || !ctx_len) return HSAB_EINVAL;
    if (!s.valias && !v_new) return HSAB_EINVAL;
    return hip_status(launch_append_slot(s, n_slots, k_new, v_new, cache, meta, klabel, label_ch, ctx_len, stream));
}

int hsab_offload_plan(const hsab_dims* dims, int32_t n_slots, const int32_t* resident,
                      const int32_t* selected, const int32_t* tail, int32_t* slot_map, int32_t* plan,
                      int64_t* delta_bytes) {
    int rc = check_dims(dims);
    if (rc) return rc;
    const Shape s = make_shape(*dims);
    if (n_slots < 2 * s.kb + 2) return HSAB_EINVAL;
    if (!resident || !selected || !tail || !slot_map || !plan) return HSAB_EINVAL;
    return offload_plan(s, n_slots, resident, selected, tail, slot_map, plan, delta_bytes);
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int hsab_offload_copy(const hsab_dims* dims, int32_t n_slots, const uint16_t* host_pool, uint16_t* cache,
                      const int32_t* plan, int32_t* plan_dev, int32_t* slot_of, int32_t copy_mode,
                      hipStream_t copy_stream, hipEvent_t done, int32_t* n_copies) {
    int rc = check_dims(dims);
    if (rc) return rc;
    const Shape s = make_shape(*dims);
    if (n_slots < 2 * s.kb + 2) return HSAB_EINVAL;
    if (!host_pool || !cache || !plan || !plan_dev || !slot_of) return HSAB_EINVAL;
    if (copy_mode != HSAB_OFFLOAD_COPY_KERNEL && copy_mode != HSAB_OFFLOAD_COPY_DMA) return HSAB_EINVAL;
    if (!aligned16(host_pool) || !aligned16(cache)) return HSAB_EINVAL;
    int calls = 0;
    rc = hip_status(offload_copy(s, n_slots, host_pool, cache, plan, plan_dev, slot_of, copy_stream, done, &calls,
                                 copy_mode, nullptr));
    if (n_copies) *n_copies = calls;
    return rc;
}

int hsab_offload_create(const hsab_dims* dims, int32_t n_slots, int32_t copy_mode, hsab_offload_engine** engine) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (!engine) return HSAB_EINVAL;
    *engine = nullptr;
    const Shape s = make_shape(*dims);
    if (n_slots < 2 * s.kb + 2) return HSAB_EINVAL;
    if (copy_mode != HSAB_OFFLOAD_COPY_KERNEL && copy_mode != HSAB_OFFLOAD_COPY_DMA &&
        copy_mode != HSAB_OFFLOAD_COPY_KERNEL_GPU_PLAN)
        return HSAB_EINVAL;
    if (copy_mode == HSAB_OFFLOAD_COPY_KERNEL_GPU_PLAN && 2 * ((n_slots - 2 + 31) / 32) + s.kb > 15360)
        return HSAB_EINVAL;   // the device planner's LDS
    if (!attend_supported(s) || s.agg == AGG_HEAD) return HSAB_EUNSUPPORTED;   // blocks move per KV head
    return hip_status(offload_create(s, n_slots, copy_mode, engine));
}

void hsab_offload_destroy(hsab_offload_engine* engine) { offload_destroy(engine); }

int hsab_offload_begin(hsab_offload_engine* engine, const int32_t* n_prefill, const uint16_t* host_pool,
                       uint16_t* cache, int32_t* slot_of, hipStream_t stream) {
    if (!engine || !n_prefill || !host_pool || !cache || !slot_of) return HSAB_EINVAL;
    if (!aligned16(host_pool) || !aligned16(cache)) return HSAB_EINVAL;
    const Shape& s = offload_shape(engine);
    for (int b = 0; b < s.B; ++b)
        if (n_prefill[b] < 0 || n_prefill[b] >= s.max_ctx) return HSAB_EINVAL;
    return hip_status(offload_begin(engine, n_prefill, host_pool, cache, slot_of, stream));
}

int hsab_offload_step(hsab_offload_engine* engine, const uint16_t* q, const uint16_t* k_new,
                      const uint16_t* v_new, uint16_t* host_pool, uint16_t* cache, uint16_t* meta,
                      uint16_t* klabel, const int32_t* label_ch, const int32_t* ctx_len,
                      const int32_t* ctx_len_host, int32_t* slot_of, int32_t* tok_idx, float* out, float* lse,
                      void* ws, size_t ws_bytes, hipStream_t compute_stream, hipStream_t copy_stream,
                      hsab_offload_stats* stats) {
    if (!engine || offload_steps(engine) < 0) return HSAB_EINVAL;   // hsab_offload_begin first
    const Shape& s = offload_shape(engine);
    if (!q || !k_new || !host_pool || !cache || !meta || !klabel || !label_ch || !ctx_len || !ctx_len_host ||
        !slot_of || !tok_idx || !out || !lse)
        return HSAB_EINVAL;
    if (!s.valias && !v_new) return HSAB_EINVAL;
    if (!aligned16(host_pool) || !aligned16(cache)) return HSAB_EINVAL;
    if (!ws || ws_bytes < ws_layout(s).total) return HSAB_EINVAL;
    int einval = 0;
    const int rc = hip_status(offload_step(engine, q, k_new, v_new, host_pool, cache, meta, klabel, label_ch,
                                           ctx_len, ctx_len_host, slot_of, tok_idx, out, lse, ws, compute_stream,
                                           copy_stream, stats, &einval));
    return rc ? rc : (einval ? HSAB_EINVAL : HSAB_OK);
}

int hsab_offload_set_timing(hsab_offload_engine* engine, int32_t enable) {
    if (!engine) return HSAB_EINVAL;
    offload_set_timing(engine, enable != 0);
    return HSAB_OK;
}

int hsab_offload_timing(hsab_offload_engine* engine, int64_t step, float* ms) {
    if (!engine || !ms || step < 0 || step >= offload_steps(engine) || step < offload_steps(engine) - TIMING_RING ||
        !offload_step_timed(engine, step))
        return HSAB_EINVAL;
    return hip_status(offload_timing(engine, step, ms));
}

int hsab_offload_selection(const hsab_offload_engine* engine, int32_t* blk_idx_host) {
    if (!engine || !blk_idx_host || offload_steps(engine) < 1) return HSAB_EINVAL;
    const Shape& s = offload_shape(engine);
    const int32_t* sel = offload_last_selection(const_cast<hsab_offload_engine*>(engine));
    if (!sel) return HSAB_EHIP;
    memcpy(blk_idx_host, sel, (size_t)s.B * s.Hkv * s.kb * sizeof(int32_t));
    return HSAB_OK;
}

int hsab_offload_step_selection(hsab_offload_engine* engine, int64_t step, int32_t* blk_idx_host) {
    if (!engine || !blk_idx_host || step < 0 || step >= offload_steps(engine) ||
        step < offload_steps(engine) - TIMING_RING)
        return HSAB_EINVAL;
    const Shape& s = offload_shape(engine);
    const int32_t* sel = offload_step_selection(engine, step);
    if (!sel) return HSAB_EHIP;
    memcpy(blk_idx_host, sel, (size_t)s.B * s.Hkv * s.kb * sizeof(int32_t));
    return HSAB_OK;
}

int hsab_offload_step_delta(hsab_offload_engine* engine, int64_t step, int64_t* delta_bytes, int64_t* cold_bytes) {
    if (!engine || !delta_bytes || !cold_bytes || step < 0 || step >= offload_steps(engine) ||
        step < offload_steps(engine) - TIMING_RING)
        return HSAB_EINVAL;
    return hip_status(offload_step_delta(engine, step, delta_bytes, cold_bytes));
}

}  // extern "C"
