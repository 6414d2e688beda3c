// Offload engine: the full KV cache lives in pinned host memory and a GPU
// block cache holds the blocks the attention reads. At step t the token
// stage and attention run over the blocks selected at step t-1 while the
// blocks newly selected at step t are copied in on a side stream; only the
// difference between consecutive selections crosses the host link
// (AsyncTLS, gist.science/de explainer section 2.B; gist.science/es
// explainer section 2.B).
//
// Slot layout of a unit's cache: n_slots slots of block*(d_k+d_v) elements
// (block*d_k when values alias keys), key rows first then value rows.
// Slots 0 .. n_slots-3 are "normal" slots; the last two are tail slots,
// slot n_slots-2 + (j & 1) holds block j while it is being appended to, so
// a block that has just been completed stays readable while the next one
// fills. The host pool has the same block layout, [U][nb_cap][slot].
#include <algorithm>
#include <chrono>
#include <cstring>
#include <vector>

#include "common.h"
#include "kernels.h"

namespace hsab {

namespace {

// grid: (B*Hkv), one workgroup per unit. Appends the token at position
// ctx_len[b]-1 into the tail slot of its block, widens that block's
// max/min and writes its label row.
__global__ __launch_bounds__(256) void append_slot_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, uint16_t* __restrict__ cache,
    uint16_t* __restrict__ meta, uint16_t* __restrict__ klabel, const int32_t* __restrict__ label_ch,
    const int32_t* __restrict__ ctx_len, uint16_t* __restrict__ pool, int Hkv, int dk, int dv, int valias, int bs,
    int r, int max_ctx, int nb_cap, int n_slots, int meta8, int lab8) {
    const int unit = blockIdx.x, b = unit / Hkv, g = unit % Hkv;
    const int pos = ctx_len[b] - 1;
    if (pos < 0 || pos >= max_ctx) return;
    const int j = pos / bs, off = pos - j * bs;
    const bool first = off == 0;
    const size_t slot_elems = (size_t)bs * (valias ? dk : dk + dv);
    const uint16_t* kn = k_new + (size_t)unit * dk;
    uint16_t* slot = cache + ((size_t)unit * n_slots + (n_slots - 2 + (j & 1))) * slot_elems;
    uint8_t* M = meta_block(meta, (size_t)unit * nb_cap + j, dk, meta8);
    // the same rows go to the pool block (pinned host memory through its
    // device mapping) when pool is given
    uint16_t* pb = pool ? pool + ((size_t)unit * nb_cap + j) * slot_elems : nullptr;
    for (int c = threadIdx.x; c < dk; c += blockDim.x) {
        const uint16_t kb = kn[c];
        slot[(size_t)off * dk + c] = kb;
        if (pb) pb[(size_t)off * dk + c] = kb;
        meta_widen(M, dk, c, kb, first, meta8);
    }
    if (!valias) {
        const uint16_t* vn = v_new + (size_t)unit * dv;
        for (int c = threadIdx.x; c < dv; c += blockDim.x) {
            slot[(size_t)bs * dk + (size_t)off * dv + c] = vn[c];
            if (pb) pb[(size_t)bs * dk + (size_t)off * dv + c] = vn[c];
        }
    }
    const size_t lrow = ((size_t)unit * max_ctx + pos) * r;
    for (int c = threadIdx.x; c < r; c += blockDim.x)
        label_put(klabel, lrow + c, kn[clamp_ch(label_ch[g * r + c], dk)], lab8);
}

// grid: (U). slot_of[unit][block] = slot for every (block, slot, copy) entry.
__global__ __launch_bounds__(256) void slot_patch_kernel(const int32_t* __restrict__ plan, int32_t* __restrict__ slot_of,
                                                         int kb, int nb_cap) {
    const int unit = blockIdx.x;
    for (int i = threadIdx.x; i < kb; i += blockDim.x) {
        const int32_t* e = plan + ((size_t)unit * kb + i) * 3;
        const int blk = e[0], slot = e[1];
        if (blk >= 0 && blk < nb_cap) slot_of[(size_t)unit * nb_cap + blk] = slot;
    }
}

// Copy one block (blk_elems bf16, 16-byte aligned) per pair of sources and
// destinations, both blocks in flight at once: eight 16-byte loads per lane
// and block for 8 KiB, unconditional (clamped) so none waits for another.
__device__ __forceinline__ void copy_two_blocks(const uint4* src0, const uint4* src1, uint4* dst0, uint4* dst1,
                                                int n16, int lane) {
    for (int c0 = 0; c0 < n16; c0 += 8 * 64) {
        uint4 v0[8], v1[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int c = c0 + k * 64 + lane;
            const int cc = c < n16 ? c : n16 - 1;
            v0[k] = src0[cc];
            v1[k] = src1[cc];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int c = c0 + k * 64 + lane;
            if (c < n16) {
                dst0[c] = v0[k];
                dst1[c] = v1[k];
            }
        }
    }
}

// The waves copy the blocks marked for copying from the pinned host pool
// (mapped into the GPU's address space) into their cache slots, two blocks
// in flight per wave; the slot table is patched by the next launch, once
// every copy has landed (the step's attention may read slot_of meanwhile
// and must find either a block's old slot, still intact, or a finished
// copy). With a copy list (pairs of pool
// block index and cache slot index, built by the host) wave v takes copies
// 2v, 2v+1, then 2v + 2*waves, ... (balanced over the waves, the list
// entries of all its rounds read in one load); without one, wave v takes
// the marked entries among plan entries [32v, 32v + 32) (one ballot). A few
// dozen workgroups keep the host link busy (a probe of scattered 8 KiB
// reads from pinned memory peaked at 16-32 four-wave workgroups) and leave
// the compute units to the next step's kernels. plan and copy_list are
// device memory or coherent pinned memory through its device mapping.
constexpr int GATHER_EPW = 32;
__global__ __launch_bounds__(256) void gather_kernel(const int32_t* __restrict__ plan,
                                                     const int32_t* __restrict__ copy_list, int n_copies,
                                                     const uint16_t* __restrict__ pool, uint16_t* __restrict__ cache,
                                                     int kb, int nb_cap, int n_slots, int blk_elems, int n_entries) {
    const int lane = threadIdx.x & 63;
    const int wv = (blockIdx.x * blockDim.x + threadIdx.x) >> 6, n_waves = (gridDim.x * blockDim.x) >> 6;
    const int n16 = blk_elems / 8;   // 16-byte chunks per block
    const uint4* P4 = reinterpret_cast<const uint4*>(pool);
    uint4* C4 = reinterpret_cast<uint4*>(cache);
    if (copy_list) {
        // copies of this wave, round k: list entries 2(v + k*waves) and the next
        int src = -1, dst = -1;
        {
            const int li = 2 * (wv + (lane >> 1) * n_waves) + (lane & 1);
            if (li < n_copies) {
                src = copy_list[2 * (size_t)li];
                dst = copy_list[2 * (size_t)li + 1];
            }
        }
        for (int k = 0; 2 * (wv + k * n_waves) < n_copies; ++k) {
            if (k == 32) break;   // more than 32 rounds: not reached (checked on the host)
            const int a = 2 * k, bl = 2 * (wv + k * n_waves) + 1 < n_copies ? 2 * k + 1 : 2 * k;
            const int s0 = __builtin_amdgcn_readlane(src, a), d0 = __builtin_amdgcn_readlane(dst, a);
            const int s1 = __builtin_amdgcn_readlane(src, bl), d1 = __builtin_amdgcn_readlane(dst, bl);
            copy_two_blocks(P4 + (size_t)s0 * n16, P4 + (size_t)s1 * n16, C4 + (size_t)d0 * n16, C4 + (size_t)d1 * n16,
                            n16, lane);
        }
    } else {
        const int e0 = wv * GATHER_EPW, e = e0 + lane;
        int blk = -1, slot = -1, cp = 0;
        if (lane < GATHER_EPW && e < n_entries) {
            blk = plan[(size_t)e * 3];
            slot = plan[(size_t)e * 3 + 1];
            cp = plan[(size_t)e * 3 + 2];
        }
        const bool ok = lane < GATHER_EPW && e < n_entries && blk >= 0 && blk < nb_cap && slot >= 0 && slot < n_slots;
        uint64_t todo = __ballot(ok && cp != 0);
        while (todo) {
            const int i0 = __ffsll((unsigned long long)todo) - 1;
            todo &= todo - 1;
            const int i1 = todo ? __ffsll((unsigned long long)todo) - 1 : i0;   // i1 == i0: one block left
            if (todo) todo &= todo - 1;
            const int u0 = (e0 + i0) / kb, u1 = (e0 + i1) / kb;
            const size_t s0 = (size_t)u0 * nb_cap + __builtin_amdgcn_readlane(blk, i0);
            const size_t s1 = (size_t)u1 * nb_cap + __builtin_amdgcn_readlane(blk, i1);
            const size_t d0 = (size_t)u0 * n_slots + __builtin_amdgcn_readlane(slot, i0);
            const size_t d1 = (size_t)u1 * n_slots + __builtin_amdgcn_readlane(slot, i1);
            copy_two_blocks(P4 + s0 * n16, P4 + s1 * n16, C4 + d0 * n16, C4 + d1 * n16, n16, lane);
        }
    }
}

}  // namespace

hipError_t launch_append_slot(const Shape& s, int n_slots, const uint16_t* k_new, const uint16_t* v_new,
                              uint16_t* cache, uint16_t* meta, uint16_t* klabel, const int32_t* label_ch,
                              const int32_t* ctx_len, hipStream_t st, uint16_t* pool_dev) {
    hipLaunchKernelGGL(append_slot_kernel, dim3(s.B * s.Hkv), dim3(256), 0, st, k_new, v_new, cache, meta, klabel,
                       label_ch, ctx_len, pool_dev, s.Hkv, s.dk, s.dv, s.valias, s.bs, s.r, s.max_ctx, s.nb_cap,
                       n_slots, s.meta8, s.lab8);
    return hipGetLastError();
}

// Host planner for one step. resident: blocks the current step's attention
// reads (R(t)); selected: blocks the next step reads (S_b(t)); tail: per
// unit the blocks held by the two tail slots at the next step. For every
// selected block: if it sits in a tail slot, map it there; if it is
// resident in a normal slot, keep that slot; otherwise copy it into a
// normal slot that no resident block uses (lowest first).
int offload_plan(const Shape& s, int n_slots, const int32_t* resident, const int32_t* selected,
                 const int32_t* tail, int32_t* slot_map, int32_t* plan, int64_t* delta_bytes) {
    const int U = s.B * s.Hkv, kb = s.kb, n_norm = n_slots - 2;
    const int64_t blk_bytes = (int64_t)s.bs * (s.valias ? s.dk : s.dk + s.dv) * 2;
    int64_t bytes = 0;
    std::vector<char> used(n_norm);
    std::vector<char> is_res(s.nb_cap, 0);   // R of the current unit, cleared after it
    std::vector<int> sel;
    for (int u = 0; u < U; ++u) {
        const int32_t* R = resident + (size_t)u * kb;
        const int32_t* S = selected + (size_t)u * kb;
        int32_t* map = slot_map + (size_t)u * s.nb_cap;
        int32_t* P = plan + (size_t)u * kb * 3;
        const int32_t* tl = tail + 2 * u;   // tl[p]: block in tail slot of parity p
        std::fill(used.begin(), used.end(), 0);
        for (int i = 0; i < kb; ++i) {
            const int blk = R[i];
            if (blk < 0 || blk >= s.nb_cap) continue;
            is_res[blk] = 1;
            const int sl = map[blk];
            if (sl >= 0 && sl < n_norm) used[sl] = 1;
        }
        // ascending, -1 entries last (unsigned order); the selection kernel's
        // lists already are, other callers' are sorted here
        sel.assign(S, S + kb);
        const auto asc = [](int32_t x, int32_t y) { return (uint32_t)x < (uint32_t)y; };
        if (!std::is_sorted(sel.begin(), sel.end(), asc)) std::sort(sel.begin(), sel.end(), asc);
        int np = 0, next_free = 0, rc = HSAB_OK;
        for (int blk : sel) {
            if (blk < 0 || blk >= s.nb_cap) continue;
            int slot;
            int copy = 0;
            if (blk == tl[blk & 1]) {
                slot = n_slots - 2 + (blk & 1);
            } else if (is_res[blk] && map[blk] >= 0 && map[blk] < n_norm) {
                slot = map[blk];
            } else {
                while (next_free < n_norm && used[next_free]) ++next_free;
                if (next_free >= n_norm) {   // n_slots too small
                    rc = HSAB_EINVAL;
                    break;
                }
                slot = next_free;
                used[next_free] = 1;
                copy = 1;
                bytes += blk_bytes;
            }
            map[blk] = slot;
            P[3 * np + 0] = blk;
            P[3 * np + 1] = slot;
            P[3 * np + 2] = copy;
            ++np;
        }
        for (int i = 0; i < kb; ++i)
            if (R[i] >= 0 && R[i] < s.nb_cap) is_res[R[i]] = 0;
        if (rc != HSAB_OK) return rc;
        for (int i = np; i < kb; ++i) P[3 * i] = P[3 * i + 1] = P[3 * i + 2] = -1;
    }
    if (delta_bytes) *delta_bytes = bytes;
    return HSAB_OK;
}

// Enqueue a plan on copy stream cs, then record `done`.
//  OFFLOAD_COPY_KERNEL: gather_kernel pulls the blocks from the mapped pool,
//    then slot_patch_kernel patches the slot table; with copy_list (coherent
//    pinned, U*K_b pairs) the plan (then also coherent pinned) and the
//    list the host fills here are read in place, else the plan is
//    uploaded to plan_dev;
//  OFFLOAD_COPY_DMA: contiguous runs of blocks into contiguous slots
//    become one hipMemcpyAsync each (DMA engines), then the plan upload
//    and the slot-table patch.
// *n_copies: blocks gathered (kernel) or copies issued (DMA).
hipError_t offload_copy(const Shape& s, int n_slots, const uint16_t* host_pool, uint16_t* cache,
                        const int32_t* plan, int32_t* plan_dev, int32_t* slot_of, hipStream_t cs,
                        hipEvent_t done, int* n_copies, int mode, int32_t* copy_list) {
    const int U = s.B * s.Hkv, kb = s.kb;
    const size_t blk_elems = (size_t)s.bs * (s.valias ? s.dk : s.dk + s.dv);
    int calls = 0;
    hipError_t e = hipSuccess;
    if (mode == OFFLOAD_COPY_KERNEL) {
        const int n_entries = U * kb, waves = (n_entries + GATHER_EPW - 1) / GATHER_EPW;
        const int n_wg = (waves + 3) / 4;
        // a copy list (pool block, cache slot) lets the waves share the
        // copies evenly; it holds at most 32 rounds of two per wave
        int32_t* list = copy_list;
        for (int i = 0; i < n_entries; ++i) {
            const int blk = plan[3 * i], slot = plan[3 * i + 1];
            if (blk < 0 || blk >= s.nb_cap || slot < 0 || slot >= n_slots || plan[3 * i + 2] <= 0) continue;
            if (list) {
                const int u = i / kb;
                list[2 * calls] = u * s.nb_cap + plan[3 * i];
                list[2 * calls + 1] = u * n_slots + plan[3 * i + 1];
            }
            ++calls;
        }
        if (calls > 2 * 32 * n_wg * 4) list = nullptr;
        const uint16_t* pool_dev = nullptr;
        e = hipHostGetDevicePointer((void**)&pool_dev, const_cast<uint16_t*>(host_pool), 0);
        if (e != hipSuccess) return e;
        const int32_t* plan_src = plan_dev;
        const int32_t* list_dev = nullptr;
        if (copy_list) {   // the engine's plan and list: coherent pinned memory, read in place
            e = hipHostGetDevicePointer((void**)&plan_src, const_cast<int32_t*>(plan), 0);
            if (e == hipSuccess && list) e = hipHostGetDevicePointer((void**)&list_dev, list, 0);
        } else {
            e = hipMemcpyAsync(plan_dev, plan, (size_t)n_entries * 3 * sizeof(int32_t), hipMemcpyHostToDevice, cs);
        }
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(gather_kernel, dim3(n_wg), dim3(256), 0, cs, plan_src, list_dev, calls, pool_dev, cache,
                           kb, s.nb_cap, n_slots, (int)blk_elems, n_entries);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(slot_patch_kernel, dim3(U), dim3(256), 0, cs, plan_src, slot_of, kb, s.nb_cap);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    } else {
        std::vector<void*> dsts, srcs;
        std::vector<size_t> sizes;
        for (int u = 0; u < U; ++u) {
            const int32_t* P = plan + (size_t)u * kb * 3;
            int i = 0;
            while (i < kb && P[3 * i] >= 0) {
                if (!P[3 * i + 2]) { ++i; continue; }
                int j = i + 1;
                while (j < kb && P[3 * j] >= 0 && P[3 * j + 2] && P[3 * j] == P[3 * (j - 1)] + 1 &&
                       P[3 * j + 1] == P[3 * (j - 1) + 1] + 1)
                    ++j;
                const int blk = P[3 * i], slot = P[3 * i + 1], run = j - i;
                dsts.push_back(cache + ((size_t)u * n_slots + slot) * blk_elems);
                srcs.push_back(const_cast<uint16_t*>(host_pool) + ((size_t)u * s.nb_cap + blk) * blk_elems);
                sizes.push_back((size_t)run * blk_elems * sizeof(uint16_t));
                i = j;
            }
        }
        calls = (int)dsts.size();
        for (int c = 0; c < calls; ++c) {
            e = hipMemcpyAsync(dsts[c], srcs[c], sizes[c], hipMemcpyHostToDevice, cs);
            if (e != hipSuccess) return e;
        }
        e = hipMemcpyAsync(plan_dev, plan, (size_t)U * kb * 3 * sizeof(int32_t), hipMemcpyHostToDevice, cs);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(slot_patch_kernel, dim3(U), dim3(256), 0, cs, plan_dev, slot_of, kb, s.nb_cap);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (n_copies) *n_copies = calls;
    return done ? hipEventRecord(done, cs) : hipSuccess;
}

// Blocks the two tail slots hold once the context has n tokens: block
// j = (n-1)/bs, and j-1 if it was appended to during decoding (j-1 >= the
// last prefill block jp); -1 where a parity holds none.
static void tail_blocks(int n, int jp, int bs, int32_t out[2]) {
    out[0] = out[1] = -1;
    if (n < 1) return;
    const int j = (n - 1) / bs;
    out[j & 1] = j;
    if (j - 1 >= jp) out[(j - 1) & 1] = j - 1;
}

}  // namespace hsab

// Engine state; every buffer here is allocated by offload_create.
struct hsab_offload_engine {
    hsab::Shape s;
    int n_slots = 0, U = 0, copy_mode = 0;
    size_t blk_elems = 0;
    int64_t step = -1;                        // next step index; -1 before offload_begin
    std::vector<int32_t> n_ctx, jp;           // [B] tokens so far, last prefill block
    std::vector<int32_t> prev_sel, cur_sel;   // [U][K_b] S_b(t-1), S_b(t)
    std::vector<int32_t> none, slot_map, tail;
    int32_t* sel_h = nullptr;                 // pinned [U][K_b]
    int32_t* plan_h[2] = {nullptr, nullptr};  // pinned coherent [U][K_b][3]
    int32_t* copy_h[2] = {nullptr, nullptr};  // pinned coherent [U*K_b][2]: the step's copies
    int32_t* sel_d[2] = {nullptr, nullptr};   // device [U][K_b]
    int32_t* plan_d[2] = {nullptr, nullptr};  // device [U][K_b][3]
    hipEvent_t ev_sel = nullptr, ev_copy[2] = {nullptr, nullptr};
    // per step % TIMING_RING: compute begin, compute end, copy begin, copy
    // end, and the compute stream before and after its wait for the copies
    hipEvent_t tm[hsab::TIMING_RING][6] = {};
};

namespace hsab {

void offload_destroy(hsab_offload_engine* e) {
    if (!e) return;
    if (e->sel_h) (void)hipHostFree(e->sel_h);
    for (int i = 0; i < 2; ++i) {
        if (e->plan_h[i]) (void)hipHostFree(e->plan_h[i]);
        if (e->copy_h[i]) (void)hipHostFree(e->copy_h[i]);
        if (e->sel_d[i]) (void)hipFree(e->sel_d[i]);
        if (e->plan_d[i]) (void)hipFree(e->plan_d[i]);
        if (e->ev_copy[i]) (void)hipEventDestroy(e->ev_copy[i]);
    }
    if (e->ev_sel) (void)hipEventDestroy(e->ev_sel);
    for (auto& row : e->tm)
        for (auto& ev : row)
            if (ev) (void)hipEventDestroy(ev);
    delete e;
}

hipError_t offload_create(const Shape& s, int n_slots, int copy_mode, hsab_offload_engine** out) {
    auto* e = new hsab_offload_engine();
    e->s = s;
    e->n_slots = n_slots;
    e->copy_mode = copy_mode;
    e->U = s.B * s.Hkv;
    e->blk_elems = (size_t)s.bs * (s.valias ? s.dk : s.dk + s.dv);
    const size_t nsel = (size_t)e->U * s.kb;
    e->n_ctx.assign(s.B, 0);
    e->jp.assign(s.B, 0);
    e->prev_sel.assign(nsel, -1);
    e->cur_sel.assign(nsel, -1);
    e->none.assign(nsel, -1);
    e->slot_map.assign((size_t)e->U * s.nb_cap, -1);
    e->tail.assign((size_t)e->U * 2, -1);
    hipError_t r = hipSuccess;
    auto ok = [&](hipError_t x) { if (r == hipSuccess) r = x; };
    // coherent: the selection kernel writes S_b(t) here through the mapping
    ok(hipHostMalloc((void**)&e->sel_h, nsel * sizeof(int32_t), hipHostMallocMapped | hipHostMallocCoherent));
    for (int i = 0; i < 2; ++i) {
        // coherent: the gather kernel reads the plan in place while the host
        // writes the other parity's
        ok(hipHostMalloc((void**)&e->plan_h[i], nsel * 3 * sizeof(int32_t),
                         hipHostMallocMapped | hipHostMallocCoherent));
        ok(hipHostMalloc((void**)&e->copy_h[i], nsel * 2 * sizeof(int32_t),
                         hipHostMallocMapped | hipHostMallocCoherent));
        ok(hipMalloc((void**)&e->sel_d[i], nsel * sizeof(int32_t)));
        ok(hipMalloc((void**)&e->plan_d[i], nsel * 3 * sizeof(int32_t)));
        ok(hipEventCreate(&e->ev_copy[i]));
    }
    ok(hipEventCreateWithFlags(&e->ev_sel, hipEventDisableTiming));
    for (auto& row : e->tm)
        for (auto& ev : row) ok(hipEventCreate(&ev));
    if (r != hipSuccess) {
        offload_destroy(e);
        return r;
    }
    *out = e;
    return hipSuccess;
}

// After prefill: each unit's last prefill block goes to its tail slot and
// the slot table is reset. Synchronous on st.
hipError_t offload_begin(hsab_offload_engine* e, const int32_t* n_prefill, const uint16_t* host_pool,
                         uint16_t* cache, int32_t* slot_of, hipStream_t st) {
    const Shape& s = e->s;
    std::fill(e->slot_map.begin(), e->slot_map.end(), -1);
    for (int b = 0; b < s.B; ++b) {
        const int np = n_prefill[b];
        e->n_ctx[b] = np;
        e->jp[b] = np > 0 ? (np - 1) / s.bs : 0;
        if (np == 0) continue;
        const int j = e->jp[b], slot = e->n_slots - 2 + (j & 1);
        for (int g = 0; g < s.Hkv; ++g) {
            const int u = b * s.Hkv + g;
            hipError_t r = hipMemcpyAsync(cache + ((size_t)u * e->n_slots + slot) * e->blk_elems,
                                          host_pool + ((size_t)u * s.nb_cap + j) * e->blk_elems,
                                          e->blk_elems * sizeof(uint16_t), hipMemcpyHostToDevice, st);
            if (r != hipSuccess) return r;
            e->slot_map[(size_t)u * s.nb_cap + j] = slot;
        }
    }
    hipError_t r = hipMemcpyAsync(slot_of, e->slot_map.data(), e->slot_map.size() * sizeof(int32_t),
                                  hipMemcpyHostToDevice, st);
    if (r != hipSuccess) return r;
    r = hipStreamSynchronize(st);
    if (r != hipSuccess) return r;
    std::fill(e->prev_sel.begin(), e->prev_sel.end(), -1);
    e->step = 0;
    return hipSuccess;
}

#define HSAB_TRY(x)                            \
    do {                                       \
        const hipError_t _e = (x);             \
        if (_e != hipSuccess) return _e;       \
    } while (0)

// One decode step under the lagged schedule. Compute stream: append into
// the tail slot, block scores and S_b(t), its copy to the host, the token
// stage over R(t), then (after the copies of the previous step) attention
// through the slot table. Host: wait for S_b(t) only, write the new token
// into the pool, plan, and enqueue the copies on the copy stream; the
// copies run while the GPU finishes step t and starts step t+1.
hipError_t offload_step(hsab_offload_engine* e, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                        uint16_t* host_pool, uint16_t* cache, uint16_t* meta, uint16_t* klabel,
                        const int32_t* label_ch, const int32_t* ctx_len, const int32_t* ctx_len_host,
                        int32_t* slot_of, int32_t* tok_idx, float* out, float* lse, void* ws, hipStream_t cs,
                        hipStream_t xs, hsab_offload_stats* st, int* einval) {
    using clk = std::chrono::steady_clock;
    const Shape& s = e->s;
    *einval = 0;
    for (int b = 0; b < s.B; ++b)   // one token per sequence per step
        if (ctx_len_host[b] != e->n_ctx[b] + 1 || ctx_len_host[b] > s.max_ctx) {
            *einval = 1;
            return hipSuccess;
        }
    const int U = e->U, kb = s.kb, t = (int)(e->step & 0x7fffffff);
    const size_t nsel = (size_t)U * kb;
    const WsLayout L = ws_layout(s);
    char* w = static_cast<char*>(ws);
    float* blk_score = reinterpret_cast<float*>(w + L.blk_score);
    float* part_ml = reinterpret_cast<float*>(w + L.part_ml);
    float* part_acc = reinterpret_cast<float*>(w + L.part_acc);
    uint32_t* sel_keys = reinterpret_cast<uint32_t*>(w + L.sel_keys);
    int32_t* sel_cnt = reinterpret_cast<int32_t*>(w + L.sel_cnt);
    hipEvent_t* tm = e->tm[e->step % TIMING_RING];
    int32_t* sel_now = e->sel_d[t & 1];
    const int32_t* resident = e->step == 0 ? sel_now : e->sel_d[(t - 1) & 1];

    // ---- compute stream, up to the token stage
    HSAB_TRY(hipEventRecord(tm[0], cs));
    // the append also writes the new rows into the pool, and the block
    // selection writes S_b(t) into mapped pinned memory as well: no copy
    // engine round trip sits between the step's start and the host's plan
    uint16_t* pool_dev = nullptr;
    int32_t* sel_map = nullptr;
    HSAB_TRY(hipHostGetDevicePointer((void**)&pool_dev, host_pool, 0));
    HSAB_TRY(hipHostGetDevicePointer((void**)&sel_map, e->sel_h, 0));
    HSAB_TRY(launch_append_slot(s, e->n_slots, k_new, v_new, cache, meta, klabel, label_ch, ctx_len, cs, pool_dev));
    HSAB_TRY(launch_block_score(s, q, meta, ctx_len, blk_score, nullptr, nullptr, nullptr, nullptr, nullptr,
                                nullptr, sel_cnt, cs));
    HSAB_TRY(launch_select(s, 1, q, blk_score, nullptr, nullptr, ctx_len, sel_now, nullptr, nullptr, nullptr,
                           nullptr, cs, sel_map));
    HSAB_TRY(hipEventRecord(e->ev_sel, cs));
    HSAB_TRY(launch_select(s, 2, q, nullptr, klabel, label_ch, ctx_len, const_cast<int32_t*>(resident), tok_idx,
                           nullptr, sel_keys, sel_cnt, cs));
    if (e->step > 0) {
        HSAB_TRY(hipEventRecord(tm[4], cs));
        HSAB_TRY(hipStreamWaitEvent(cs, e->ev_copy[(t - 1) & 1], 0));
        HSAB_TRY(hipEventRecord(tm[5], cs));
        HSAB_TRY(launch_attend(s, q, cache, cache, tok_idx, nullptr, s.kt, slot_of, e->n_slots, part_ml, part_acc,
                               out, lse, cs));
        HSAB_TRY(hipEventRecord(tm[1], cs));
    }

    // ---- host: S_b(t), the new rows into the pool, plans
    const auto t0 = clk::now();
    HSAB_TRY(hipEventSynchronize(e->ev_sel));
    const auto t1 = clk::now();
    std::memcpy(e->cur_sel.data(), e->sel_h, nsel * sizeof(int32_t));
    for (int b = 0; b < s.B; ++b) e->n_ctx[b] += 1;
    int64_t cold_bytes = 0, delta_bytes = 0;
    int copies = 0, calls = 0;
    if (e->step == 0) {   // cold start: fill S_b(0) synchronously
        for (int u = 0; u < U; ++u) tail_blocks(e->n_ctx[u / s.Hkv], e->jp[u / s.Hkv], s.bs, &e->tail[2 * u]);
        if (offload_plan(s, e->n_slots, e->none.data(), e->cur_sel.data(), e->tail.data(), e->slot_map.data(),
                         e->plan_h[1], &cold_bytes) != HSAB_OK) {
            *einval = 1;
            return hipSuccess;
        }
        HSAB_TRY(offload_copy(s, e->n_slots, host_pool, cache, e->plan_h[1], e->plan_d[1], slot_of, xs,
                              e->ev_copy[1], &calls, e->copy_mode, e->copy_h[1]));
        copies += calls;
        HSAB_TRY(hipEventRecord(tm[4], cs));
        HSAB_TRY(hipStreamWaitEvent(cs, e->ev_copy[1], 0));
        HSAB_TRY(hipEventRecord(tm[5], cs));
        HSAB_TRY(launch_attend(s, q, cache, cache, tok_idx, nullptr, s.kt, slot_of, e->n_slots, part_ml, part_acc,
                               out, lse, cs));
        HSAB_TRY(hipEventRecord(tm[1], cs));
    }
    for (int u = 0; u < U; ++u) tail_blocks(e->n_ctx[u / s.Hkv] + 1, e->jp[u / s.Hkv], s.bs, &e->tail[2 * u]);
    const int32_t* R = e->step == 0 ? e->cur_sel.data() : e->prev_sel.data();
    if (offload_plan(s, e->n_slots, R, e->cur_sel.data(), e->tail.data(), e->slot_map.data(), e->plan_h[t & 1],
                     &delta_bytes) != HSAB_OK) {
        *einval = 1;
        return hipSuccess;
    }
    HSAB_TRY(hipEventRecord(tm[2], xs));
    HSAB_TRY(offload_copy(s, e->n_slots, host_pool, cache, e->plan_h[t & 1], e->plan_d[t & 1], slot_of, xs,
                          e->ev_copy[t & 1], &calls, e->copy_mode, e->copy_h[t & 1]));
    copies += calls;
    HSAB_TRY(hipEventRecord(tm[3], xs));
    const auto t2 = clk::now();
    e->prev_sel.swap(e->cur_sel);
    if (st) {
        const int64_t blk_bytes = (int64_t)e->blk_elems * 2;
        st->step = e->step;
        st->delta_bytes = delta_bytes;
        st->delta_blocks = (int32_t)(delta_bytes / blk_bytes);
        st->cold_bytes = cold_bytes;
        st->n_copies = copies;
        st->host_wait_ms = std::chrono::duration<float, std::milli>(t1 - t0).count();
        st->host_plan_ms = std::chrono::duration<float, std::milli>(t2 - t1).count();
    }
    e->step += 1;
    return hipSuccess;
}

// GPU times of a finished step (within the last four), see
// hsab_offload_timing. Waits for that step's events.
hipError_t offload_timing(hsab_offload_engine* e, int64_t step, float* ms) {
    hipEvent_t* tm = e->tm[step % TIMING_RING];
    HSAB_TRY(hipEventSynchronize(tm[3]));
    HSAB_TRY(hipEventSynchronize(tm[1]));
    HSAB_TRY(hipEventElapsedTime(&ms[0], tm[0], tm[1]));
    HSAB_TRY(hipEventElapsedTime(&ms[1], tm[2], tm[3]));
    HSAB_TRY(hipEventElapsedTime(&ms[2], tm[0], tm[2]));
    HSAB_TRY(hipEventElapsedTime(&ms[3], tm[0], tm[3]));
    HSAB_TRY(hipEventElapsedTime(&ms[4], tm[4], tm[5]));
    return hipSuccess;
}

const int32_t* offload_last_selection(const hsab_offload_engine* e) { return e->prev_sel.data(); }
int64_t offload_steps(const hsab_offload_engine* e) { return e->step; }
const Shape& offload_shape(const hsab_offload_engine* e) { return e->s; }

}  // namespace hsab
