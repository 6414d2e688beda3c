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
// max/min and writes its label row. ctx_copy (nullable) receives ctx_len:
// the copy stream's planner reads that snapshot, never the caller's
// buffer, which the caller may change once the compute stream is past it.
__global__ __launch_bounds__(256) void append_slot_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new, uint16_t* __restrict__ cache,
    uint16_t* __restrict__ meta, uint16_t* __restrict__ klabel, const int32_t* __restrict__ label_ch,
    const int32_t* __restrict__ ctx_len, uint16_t* __restrict__ pool, int32_t* __restrict__ ctx_copy, int Hkv,
    int dk, int dv, int valias, int bs, int r, int max_ctx, int nb_cap, int n_slots, int meta8, int lab8) {
    const int unit = blockIdx.x, b = unit / Hkv, g = unit % Hkv;
    const int pos = ctx_len[b] - 1;
    if (ctx_copy && g == 0 && threadIdx.x == 0) ctx_copy[b] = pos + 1;
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

// grid: (U). slot_of[unit][block] = slot for every (block, slot, copy)
// entry; with cnt and rec (nullable) the unit's copy count is also
// recorded into rec[unit] (mapped pinned memory read by the host later).
__global__ __launch_bounds__(256) void slot_patch_kernel(const int32_t* __restrict__ plan, int32_t* __restrict__ slot_of,
                                                         int kb, int nb_cap, const int32_t* __restrict__ cnt,
                                                         int32_t* __restrict__ rec) {
    const int unit = blockIdx.x;
    if (rec && threadIdx.x == 0) rec[unit] = cnt[unit];
    for (int i = threadIdx.x; i < kb; i += blockDim.x) {
        const int32_t* e = plan + ((size_t)unit * kb + i) * 3;
        const int blk = e[0], slot = e[1];
        if (blk >= 0 && blk < nb_cap) slot_of[(size_t)unit * nb_cap + blk] = slot;
    }
}

// Exclusive prefix sum over a 256-thread workgroup (v per thread, in thread
// order); *total receives the sum. Uses s_w[4] of LDS.
__device__ __forceinline__ uint32_t wg_excl_scan256(uint32_t v, uint32_t* s_w, uint32_t* total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t incl = wave_scan_dpp(v);
    if (lane == 63) s_w[w] = incl;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        before += i < w ? s_w[i] : 0u;
        tot += s_w[i];
    }
    __syncthreads();   // s_w is reused by the next scan
    *total = tot;
    return before + incl - v;
}

// Binary search of blk among the resident blocks (ascending, -1 last:
// unsigned order); true when present.
__device__ __forceinline__ bool is_resident(const int32_t* sR, int kb, int blk) {
    int lo = 0, hi = kb;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((uint32_t)sR[mid] < (uint32_t)blk) lo = mid + 1; else hi = mid;
    }
    return lo < kb && sR[lo] == blk;
}

// The host planner's rules (offload_plan) on the device, one 256-thread
// workgroup per unit, so the copy stream plans a step's delta without a
// host round trip. Slots held by the resident blocks R are marked used; a
// selected block (S ascending, -1 last) that sits in a tail slot at the
// step the plan serves maps there, one resident in a block slot keeps it,
// and every other takes the lowest unused block slot in ascending block
// order (the k-th block to copy takes the k-th free slot: two prefix sums
// replace the host's sequential scan). Writes the plan entries, the unit's
// copy list (pool block index, cache slot index) and count, and the slot
// map the next plan reads. next: 1 when the plan serves the next step (its
// tail holds one more token), 0 for the cold fill. K_b <= 2048.
constexpr int PLAN_THREADS = 256;
constexpr int PLAN_EPT = MAX_KB / PLAN_THREADS;   // entries per thread at most
__global__ __launch_bounds__(PLAN_THREADS) void plan_kernel(
    const int32_t* __restrict__ R, const int32_t* __restrict__ S, const int32_t* __restrict__ ctx_len,
    const int32_t* __restrict__ jp, int32_t* __restrict__ map, int32_t* __restrict__ plan,
    int32_t* __restrict__ list, int32_t* __restrict__ cnt, int Hkv, int kb, int nb_cap, int n_slots, int bs,
    int max_ctx, int next) {
    extern __shared__ uint32_t sm[];   // used bitmap [nw], free-slot prefix [nw], resident blocks [kb]
    __shared__ uint32_t s_w[4];
    __shared__ int s_tl[2];
    const int u = blockIdx.x, b = u / Hkv, tid = threadIdx.x;
    const int n_norm = n_slots - 2, nw = (n_norm + 31) / 32;
    uint32_t* used = sm;
    uint32_t* zpre = sm + nw;
    int32_t* sR = reinterpret_cast<int32_t*>(sm + 2 * nw);
    int32_t* mu = map + (size_t)u * nb_cap;
    if (tid == 0) {   // blocks in the tail slots at the step the plan serves
        int n = ctx_len[b];
        n = (n < 1 ? 1 : (n > max_ctx ? max_ctx : n)) + next;
        const int j = (n - 1) / bs;
        s_tl[0] = s_tl[1] = -1;
        s_tl[j & 1] = j;
        if (j - 1 >= jp[b]) s_tl[(j - 1) & 1] = j - 1;
    }
    for (int w = tid; w < nw; w += PLAN_THREADS) used[w] = 0u;
    for (int i = tid; i < kb; i += PLAN_THREADS) sR[i] = R ? R[(size_t)u * kb + i] : -1;
    __syncthreads();
    for (int i = tid; i < kb; i += PLAN_THREADS) {
        const int blk = sR[i];
        if (blk >= 0 && blk < nb_cap) {
            const int sl = mu[blk];
            if (sl >= 0 && sl < n_norm) atomicOr(&used[sl >> 5], 1u << (sl & 31));
        }
    }
    __syncthreads();
    // free block slots per word, and their prefix over the words (each
    // thread takes consecutive words)
    auto word_free = [&](int w) {
        const int valid = n_norm - 32 * w < 32 ? n_norm - 32 * w : 32;
        return ~used[w] & (valid == 32 ? ~0u : ((1u << valid) - 1u));
    };
    const int wpt = (nw + PLAN_THREADS - 1) / PLAN_THREADS;
    uint32_t zl = 0;
    for (int w = tid * wpt; w < nw && w < (tid + 1) * wpt; ++w) zl += __popc(word_free(w));
    uint32_t free_total;
    uint32_t zb = wg_excl_scan256(zl, s_w, &free_total);
    for (int w = tid * wpt; w < nw && w < (tid + 1) * wpt; ++w) {
        zpre[w] = zb;
        zb += __popc(word_free(w));
    }
    __syncthreads();
    // this thread's consecutive entries of S; the blocks to copy are ranked
    // in entry order
    const int ept = (kb + PLAN_THREADS - 1) / PLAN_THREADS;
    const int i0 = tid * ept;
    int kind[PLAN_EPT];   // -1 none, 0 tail, 1 kept, 2 copy
    uint32_t ncp = 0;
#pragma unroll
    for (int k = 0; k < PLAN_EPT; ++k) {
        kind[k] = -1;
        const int i = i0 + k;
        if (k >= ept || i >= kb) continue;
        const int blk = S[(size_t)u * kb + i];
        if (blk < 0 || blk >= nb_cap) continue;
        if (blk == s_tl[blk & 1]) {
            kind[k] = 0;
        } else {
            const int sl = mu[blk];
            kind[k] = is_resident(sR, kb, blk) && sl >= 0 && sl < n_norm ? 1 : 2;
            ncp += kind[k] == 2;
        }
    }
    uint32_t n_copy;
    uint32_t rank = wg_excl_scan256(ncp, s_w, &n_copy);
    int slots[PLAN_EPT];
#pragma unroll
    for (int k = 0; k < PLAN_EPT; ++k) {
        slots[k] = -1;
        const int i = i0 + k;
        if (k >= ept || i >= kb) continue;
        const int blk = S[(size_t)u * kb + i];
        int copy = 0;
        if (kind[k] == 0) {
            slots[k] = n_slots - 2 + (blk & 1);
        } else if (kind[k] == 1) {
            slots[k] = mu[blk];
        } else if (kind[k] == 2 && rank < free_total) {   // the rank-th free slot
            int wl = 0, wh = nw - 1;                        // last word whose prefix <= rank
            while (wl < wh) {
                const int mid = (wl + wh + 1) >> 1;
                if (zpre[mid] <= rank) wl = mid; else wh = mid - 1;
            }
            uint32_t z = word_free(wl);
            for (uint32_t r = zpre[wl]; r < rank; ++r) z &= z - 1;   // drop the lower free slots
            slots[k] = 32 * wl + __ffs(z) - 1;
            copy = 1;
            int32_t* L = list + ((size_t)u * kb + rank) * 2;
            L[0] = u * nb_cap + blk;
            L[1] = u * n_slots + slots[k];
            ++rank;
        }
        int32_t* P = plan + ((size_t)u * kb + i) * 3;
        P[0] = slots[k] >= 0 ? blk : -1;
        P[1] = slots[k];
        P[2] = slots[k] >= 0 ? copy : -1;
    }
    __syncthreads();   // every read of the slot map is done
#pragma unroll
    for (int k = 0; k < PLAN_EPT; ++k) {
        const int i = i0 + k;
        if (k < ept && i < kb && slots[k] >= 0) mu[S[(size_t)u * kb + i]] = slots[k];
    }
    if (tid == 0) cnt[u] = (int32_t)(n_copy < free_total ? n_copy : free_total);
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
// copy). With per-unit copy lists (list [U][K_b] pairs of pool block index
// and cache slot index, cnt [U] filled entries each, written by
// plan_kernel or by the host) wave v takes items v, v + waves, v + 2 waves, ... of the
// entry-major item order (item x: entry x / U of unit x % U; 32 per wave),
// so the filled entries, which sit at the front of every list, spread
// evenly over the waves, and copies them two at a time; without lists
// (plan from the host), wave v takes the marked entries among plan entries
// [32v, 32v + 32) (one ballot). A few dozen workgroups keep the host link
// busy (a probe of scattered 8 KiB reads from pinned memory peaked at 16-32
// four-wave workgroups) and leave the compute units to the next step's
// kernels.
constexpr int GATHER_EPW = 32;
__global__ __launch_bounds__(256) void gather_kernel(const int32_t* __restrict__ plan,
                                                     const int32_t* __restrict__ list, const int32_t* __restrict__ cnt,
                                                     const uint16_t* __restrict__ pool, uint16_t* __restrict__ cache,
                                                     int kb, int nb_cap, int n_slots, int blk_elems, int n_entries) {
    const int lane = threadIdx.x & 63;
    const int wv = (blockIdx.x * blockDim.x + threadIdx.x) >> 6, n_waves = (gridDim.x * blockDim.x) >> 6;
    const int n16 = blk_elems / 8;   // 16-byte chunks per block
    const uint4* P4 = reinterpret_cast<const uint4*>(pool);
    uint4* C4 = reinterpret_cast<uint4*>(cache);
    if (list) {
        int src = -1, dst = -1;
        bool has = false;
        const int x = wv + n_waves * lane;   // this lane's list item, entry-major: unit x % U, entry x / U
        const int U = n_entries / kb;
        if (lane < GATHER_EPW && x < n_entries) {
            const int i = x / U, u = x - i * U;
            if (i < cnt[u]) {
                const size_t li = (size_t)u * kb + i;
                src = list[2 * li];
                dst = list[2 * li + 1];
                has = true;
            }
        }
        uint64_t todo = __ballot(has);
        while (todo) {
            const int i0 = __ffsll((unsigned long long)todo) - 1;
            todo &= todo - 1;
            const int i1 = todo ? __ffsll((unsigned long long)todo) - 1 : i0;   // i1 == i0: one block left
            if (todo) todo &= todo - 1;
            const size_t s0 = (size_t)__builtin_amdgcn_readlane(src, i0), d0 = (size_t)__builtin_amdgcn_readlane(dst, i0);
            const size_t s1 = (size_t)__builtin_amdgcn_readlane(src, i1), d1 = (size_t)__builtin_amdgcn_readlane(dst, i1);
            copy_two_blocks(P4 + s0 * n16, P4 + s1 * n16, C4 + d0 * n16, C4 + d1 * n16, n16, lane);
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
                              const int32_t* ctx_len, hipStream_t st, uint16_t* pool_dev, int32_t* ctx_copy) {
    hipLaunchKernelGGL(append_slot_kernel, dim3(s.B * s.Hkv), dim3(256), 0, st, k_new, v_new, cache, meta, klabel,
                       label_ch, ctx_len, pool_dev, ctx_copy, s.Hkv, s.dk, s.dv, s.valias, s.bs, s.r, s.max_ctx,
                       s.nb_cap, n_slots, s.meta8, s.lab8);
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

// Enqueue a host plan on copy stream cs, then record `done`.
//  OFFLOAD_COPY_KERNEL: gather_kernel pulls the blocks from the mapped pool
//    then slot_patch_kernel patches the slot table; with mp (the plan in
//    coherent pinned memory, list and count buffers there too, and the
//    device addresses of all of them and of the pool) the plan and the
//    per-unit copy lists filled here are read in place, else the plan is
//    uploaded to plan_dev and each wave takes the marked entries among 32
//    plan entries;
//  OFFLOAD_COPY_DMA: contiguous runs of blocks into contiguous slots
//    become one hipMemcpyAsync each (DMA engines), then the plan upload
//    and the slot-table patch.
// *n_copies: blocks gathered (kernel) or copies issued (DMA).
hipError_t offload_copy(const Shape& s, int n_slots, const uint16_t* host_pool, uint16_t* cache,
                        const int32_t* plan, int32_t* plan_dev, int32_t* slot_of, hipStream_t cs,
                        hipEvent_t done, int* n_copies, int mode, const MappedPlan* mp) {
    const int U = s.B * s.Hkv, kb = s.kb;
    const size_t blk_elems = (size_t)s.bs * (s.valias ? s.dk : s.dk + s.dv);
    int calls = 0;
    hipError_t e = hipSuccess;
    if (mode == OFFLOAD_COPY_KERNEL) {
        const int n_entries = U * kb, waves = (n_entries + GATHER_EPW - 1) / GATHER_EPW;
        // with the engine's coherent pinned list and count buffers, the
        // copies go into per-unit lists (the entries the plan marks, in
        // order) that the gather spreads evenly over its waves
        for (int u = 0; u < U; ++u) {
            int c = 0;
            for (int i = 0; i < kb; ++i) {
                const int32_t* P = plan + ((size_t)u * kb + i) * 3;
                if (P[0] < 0 || P[0] >= s.nb_cap || P[1] < 0 || P[1] >= n_slots || P[2] <= 0) continue;
                if (mp) {
                    mp->list_h[((size_t)u * kb + c) * 2] = u * s.nb_cap + P[0];
                    mp->list_h[((size_t)u * kb + c) * 2 + 1] = u * n_slots + P[1];
                }
                ++c;
            }
            if (mp) mp->cnt_h[u] = c;
            calls += c;
        }
        const uint16_t* pool_dev = mp ? mp->pool_dev : nullptr;
        const int32_t* plan_src = mp ? mp->plan_dev : plan_dev;
        const int32_t* list_dev = mp ? mp->list_dev : nullptr;
        const int32_t* cnt_dev = mp ? mp->cnt_dev : nullptr;
        if (!mp) {
            e = hipHostGetDevicePointer((void**)&pool_dev, const_cast<uint16_t*>(host_pool), 0);
            if (e == hipSuccess)
                e = hipMemcpyAsync(plan_dev, plan, (size_t)n_entries * 3 * sizeof(int32_t), hipMemcpyHostToDevice,
                                   cs);
            if (e != hipSuccess) return e;
        }
        hipLaunchKernelGGL(gather_kernel, dim3((waves + 3) / 4), dim3(256), 0, cs, plan_src, list_dev, cnt_dev,
                           pool_dev, cache, kb, s.nb_cap, n_slots, (int)blk_elems, n_entries);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(slot_patch_kernel, dim3(U), dim3(256), 0, cs, plan_src, slot_of, kb, s.nb_cap, nullptr,
                           nullptr);
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
        hipLaunchKernelGGL(slot_patch_kernel, dim3(U), dim3(256), 0, cs, plan_dev, slot_of, kb, s.nb_cap, nullptr,
                           nullptr);
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
    // pinned coherent [TIMING_RING][U][K_b]: S_b of each of the last steps,
    // written by the selection kernel through the mapping (sel_map)
    int32_t* sel_h = nullptr;
    int32_t* sel_map = nullptr;
    const uint16_t* pool_h = nullptr;         // the last pool seen, and its device address
    uint16_t* pool_dev = nullptr;
    int32_t* plan_h[2] = {nullptr, nullptr};  // pinned coherent [U][K_b][3]
    int32_t* list_h[2] = {nullptr, nullptr};  // pinned coherent [U][K_b][2]: host-planned copy lists
    int32_t* cnt_h[2] = {nullptr, nullptr};   // pinned coherent [U]
    hsab::MappedPlan mp[2];                   // the above with their device addresses
    // device [U][K_b] selections, a ring of three: step t writes sel_d[t % 3]
    // while the copy stream may still plan step t-1 from sel_d[(t-2) % 3]
    // (its R) and sel_d[(t-1) % 3]; step t's attention waits for step t-1's
    // copies, so step t+1 reuses sel_d[(t-2) % 3] only after that plan ran
    int32_t* sel_d[3] = {nullptr, nullptr, nullptr};
    int32_t* ctx_d[2] = {nullptr, nullptr};   // device [B]: ctx_len of the step's parity, for the planner
    int32_t* plan_d[2] = {nullptr, nullptr};  // device [U][K_b][3]
    // planning on the GPU (kernel copies): the slot map, the last prefill
    // block per sequence, per-unit copy lists and counts, and per step the
    // units' copy counts (delta, cold fill) for the host to read later
    bool gpu_plan = false;
    int32_t* map_d = nullptr;                 // device [U][nb_cap]
    int32_t* jp_d = nullptr;                  // device [B]
    int32_t* list_d[2] = {nullptr, nullptr};  // device [U][K_b][2]
    int32_t* cnt_d[2] = {nullptr, nullptr};   // device [U]
    int32_t* rec_h = nullptr;                 // pinned coherent [TIMING_RING][2][U]
    int64_t ring_delta[hsab::TIMING_RING] = {}, ring_cold[hsab::TIMING_RING] = {};   // host-planned steps
    hipEvent_t ev_sel = nullptr, ev_copy[2] = {nullptr, nullptr};
    // per step % TIMING_RING, recorded only while timing is on (each timed
    // record is a marker the GPU processes, ~1-3 us per step and record):
    // compute begin, compute end, copy begin, copy end, and the compute
    // stream before and after its wait for the copies
    hipEvent_t tm[hsab::TIMING_RING][6] = {};
    bool timing = false;
    bool ring_timed[hsab::TIMING_RING] = {};
    // per step % TIMING_RING, GPU planning only: the step's copies are done
    hipEvent_t done[hsab::TIMING_RING] = {};
};

namespace hsab {

void offload_destroy(hsab_offload_engine* e) {
    if (!e) return;
    if (e->sel_h) (void)hipHostFree(e->sel_h);
    if (e->rec_h) (void)hipHostFree(e->rec_h);
    if (e->map_d) (void)hipFree(e->map_d);
    if (e->jp_d) (void)hipFree(e->jp_d);
    for (int i = 0; i < 3; ++i)
        if (e->sel_d[i]) (void)hipFree(e->sel_d[i]);
    for (int i = 0; i < 2; ++i) {
        if (e->ctx_d[i]) (void)hipFree(e->ctx_d[i]);
        if (e->plan_h[i]) (void)hipHostFree(e->plan_h[i]);
        if (e->list_h[i]) (void)hipHostFree(e->list_h[i]);
        if (e->cnt_h[i]) (void)hipHostFree(e->cnt_h[i]);
        if (e->plan_d[i]) (void)hipFree(e->plan_d[i]);
        if (e->list_d[i]) (void)hipFree(e->list_d[i]);
        if (e->cnt_d[i]) (void)hipFree(e->cnt_d[i]);
        if (e->ev_copy[i]) (void)hipEventDestroy(e->ev_copy[i]);
    }
    if (e->ev_sel) (void)hipEventDestroy(e->ev_sel);
    for (auto& row : e->tm)
        for (auto& ev : row)
            if (ev) (void)hipEventDestroy(ev);
    for (auto& ev : e->done)
        if (ev) (void)hipEventDestroy(ev);
    delete e;
}

hipError_t offload_create(const Shape& s, int n_slots, int copy_mode, hsab_offload_engine** out) {
    auto* e = new hsab_offload_engine();
    e->s = s;
    e->n_slots = n_slots;
    e->gpu_plan = copy_mode == OFFLOAD_COPY_KERNEL_GPU_PLAN;
    e->copy_mode = e->gpu_plan ? OFFLOAD_COPY_KERNEL : copy_mode;   // how the host path copies
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
    ok(hipHostMalloc((void**)&e->sel_h, (size_t)TIMING_RING * nsel * sizeof(int32_t),
                     hipHostMallocMapped | hipHostMallocCoherent));
    if (r == hipSuccess) ok(hipHostGetDevicePointer((void**)&e->sel_map, e->sel_h, 0));
    for (int i = 0; i < 3; ++i) ok(hipMalloc((void**)&e->sel_d[i], nsel * sizeof(int32_t)));
    for (int i = 0; i < 2; ++i) {
        // coherent: the gather kernel reads the plan in place while the host
        // writes the other parity's
        ok(hipHostMalloc((void**)&e->plan_h[i], nsel * 3 * sizeof(int32_t),
                         hipHostMallocMapped | hipHostMallocCoherent));
        ok(hipHostMalloc((void**)&e->list_h[i], nsel * 2 * sizeof(int32_t),
                         hipHostMallocMapped | hipHostMallocCoherent));
        ok(hipHostMalloc((void**)&e->cnt_h[i], (size_t)e->U * sizeof(int32_t),
                         hipHostMallocMapped | hipHostMallocCoherent));
        MappedPlan& m = e->mp[i];
        m.list_h = e->list_h[i];
        m.cnt_h = e->cnt_h[i];
        ok(hipHostGetDevicePointer((void**)&m.plan_dev, e->plan_h[i], 0));
        ok(hipHostGetDevicePointer((void**)&m.list_dev, e->list_h[i], 0));
        ok(hipHostGetDevicePointer((void**)&m.cnt_dev, e->cnt_h[i], 0));
        ok(hipMalloc((void**)&e->ctx_d[i], (size_t)s.B * sizeof(int32_t)));
        ok(hipMalloc((void**)&e->plan_d[i], nsel * 3 * sizeof(int32_t)));
        ok(hipMalloc((void**)&e->list_d[i], nsel * 2 * sizeof(int32_t)));
        ok(hipMalloc((void**)&e->cnt_d[i], (size_t)e->U * sizeof(int32_t)));
        ok(hipEventCreateWithFlags(&e->ev_copy[i], hipEventDisableTiming));
    }
    ok(hipEventCreateWithFlags(&e->ev_sel, hipEventDisableTiming));
    ok(hipMalloc((void**)&e->map_d, (size_t)e->U * s.nb_cap * sizeof(int32_t)));
    ok(hipMalloc((void**)&e->jp_d, (size_t)s.B * sizeof(int32_t)));
    ok(hipHostMalloc((void**)&e->rec_h, (size_t)TIMING_RING * 2 * e->U * sizeof(int32_t),
                     hipHostMallocMapped | hipHostMallocCoherent));

    for (auto& row : e->tm)
        for (auto& ev : row) ok(hipEventCreate(&ev));
    for (auto& ev : e->done) ok(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
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
    r = hipMemcpyAsync(e->map_d, e->slot_map.data(), e->slot_map.size() * sizeof(int32_t), hipMemcpyHostToDevice, st);
    if (r != hipSuccess) return r;
    r = hipMemcpyAsync(e->jp_d, e->jp.data(), e->jp.size() * sizeof(int32_t), hipMemcpyHostToDevice, st);
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

// Plan and copy of one step's delta on the copy stream, all on the GPU:
// plan_kernel (slot map, plan entries, per-unit copy lists), gather_kernel
// (the copies), slot_patch_kernel (slot_of, and the units' copy counts into
// rec). par selects the plan / list buffers of the step's parity.
static hipError_t gpu_plan_copy(hsab_offload_engine* e, int par, const int32_t* R, const int32_t* S,
                                const int32_t* ctx_len, int next, const uint16_t* pool_dev, uint16_t* cache,
                                int32_t* slot_of, int32_t* rec, hipStream_t xs) {
    const Shape& s = e->s;
    const int nw = (e->n_slots - 2 + 31) / 32, n_entries = e->U * s.kb;
    hipLaunchKernelGGL(plan_kernel, dim3(e->U), dim3(PLAN_THREADS), (2 * nw + s.kb) * sizeof(int32_t), xs, R, S,
                       ctx_len, e->jp_d, e->map_d, e->plan_d[par], e->list_d[par], e->cnt_d[par], s.Hkv, s.kb,
                       s.nb_cap, e->n_slots, s.bs, s.max_ctx, next);
    HSAB_TRY(hipGetLastError());
    const int waves = (n_entries + GATHER_EPW - 1) / GATHER_EPW;
    // twice the host path's workgroups: with the host planning, the host's
    // calls pace the steps and more copy waves only slow the compute
    // kernels; here the copies are the step's longest chain
    hipLaunchKernelGGL(gather_kernel, dim3((waves + 1) / 2), dim3(256), 0, xs, e->plan_d[par], e->list_d[par],
                       e->cnt_d[par], pool_dev, cache, s.kb, s.nb_cap, e->n_slots, (int)e->blk_elems, n_entries);
    HSAB_TRY(hipGetLastError());
    hipLaunchKernelGGL(slot_patch_kernel, dim3(e->U), dim3(256), 0, xs, e->plan_d[par], slot_of, s.kb, s.nb_cap,
                       e->cnt_d[par], rec);
    return hipGetLastError();
}

// One decode step under the lagged schedule. Compute stream: append into
// the tail slot (and the pool), block scores and S_b(t), the token stage
// over R(t), then (after the copies of the previous step) attention
// through the slot table. Kernel copies: the copy stream waits for S_b(t)
// and plans, copies and patches the delta for step t+1 on the GPU; the host
// only enqueues. DMA copies: the host waits for S_b(t), plans and enqueues
// one copy per run of blocks. The copies run while the GPU finishes step t
// and starts step t+1.
hipError_t offload_step(hsab_offload_engine* e, const uint16_t* q, const uint16_t* k_new, const uint16_t* v_new,
                        uint16_t* host_pool, uint16_t* cache, uint16_t* meta, uint16_t* klabel,
                        const int32_t* label_ch, const int32_t* ctx_len, const int32_t* ctx_len_host,
                        int32_t* slot_of, int32_t* tok_idx, float* out, float* lse, void* ws, hipStream_t cs,
                        hipStream_t xs, hsab_offload_stats* st, int* einval) {
    using clk = std::chrono::steady_clock;
    const auto t_in = clk::now();
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
    const int ring = (int)(e->step % TIMING_RING);
    hipEvent_t* tm = e->tm[ring];
    const bool timed = e->timing;
    e->ring_timed[ring] = timed;
    auto mark = [&](int i, hipStream_t s) { return timed ? hipEventRecord(tm[i], s) : hipSuccess; };
    int32_t* sel_now = e->sel_d[e->step % 3];
    const int32_t* resident = e->step == 0 ? sel_now : e->sel_d[(e->step - 1) % 3];
    int32_t* ctx_snap = e->ctx_d[t & 1];

    // ---- compute stream, up to the token stage. The append also writes the
    // new rows into the pool, and the block selection writes S_b(t) into
    // mapped pinned memory as well: no copy-engine round trip before the plan
    if (host_pool != e->pool_h) {
        HSAB_TRY(hipHostGetDevicePointer((void**)&e->pool_dev, host_pool, 0));
        e->pool_h = host_pool;
        e->mp[0].pool_dev = e->mp[1].pool_dev = e->pool_dev;
    }
    uint16_t* pool_dev = e->pool_dev;
    int32_t* sel_map = e->sel_map + (size_t)ring * nsel;
    HSAB_TRY(mark(0, cs));
    HSAB_TRY(launch_append_slot(s, e->n_slots, k_new, v_new, cache, meta, klabel, label_ch, ctx_len, cs, pool_dev,
                                ctx_snap));
    const Handoff ho{sel_cnt, sel_keys, s.kb * s.bs};
    HSAB_TRY(launch_block_score(s, q, meta, ctx_len, blk_score, nullptr, nullptr, nullptr, nullptr, nullptr,
                                nullptr, &ho, cs));
    HSAB_TRY(launch_select(s, 1, q, blk_score, nullptr, nullptr, ctx_len, sel_now, nullptr, nullptr, nullptr,
                           nullptr, cs, sel_map));
    HSAB_TRY(hipEventRecord(e->ev_sel, cs));
    HSAB_TRY(launch_select(s, 2, q, nullptr, klabel, label_ch, ctx_len, const_cast<int32_t*>(resident), tok_idx,
                           nullptr, sel_keys, sel_cnt, cs));
    auto attend_after = [&](hipEvent_t copies) -> hipError_t {
        HSAB_TRY(mark(4, cs));
        HSAB_TRY(hipStreamWaitEvent(cs, copies, 0));
        HSAB_TRY(mark(5, cs));
        HSAB_TRY(launch_attend(s, q, cache, cache, tok_idx, nullptr, s.kt, ctx_len, slot_of, e->n_slots, part_ml, part_acc,
                               out, lse, cs));
        return mark(1, cs);
    };
    if (e->step > 0) {   // the previous step's copies: its done event (GPU planning) or its parity's copy event
        const int prev_ring = (int)((e->step - 1) % TIMING_RING);
        HSAB_TRY(attend_after(e->gpu_plan ? e->done[prev_ring] : e->ev_copy[(t - 1) & 1]));
    }

    int64_t cold_bytes = 0, delta_bytes = 0;
    int copies = 0, calls = 0;
    auto t0 = clk::now(), t1 = t0;
    if (e->gpu_plan) {
        // ---- copy stream: plan, copy, patch on the GPU after S_b(t)
        int32_t* rec = e->rec_h + (size_t)ring * 2 * U;
        HSAB_TRY(hipStreamWaitEvent(xs, e->ev_sel, 0));
        if (e->step == 0) {   // cold start: S_b(0) is also R(0)
            HSAB_TRY(gpu_plan_copy(e, 1, nullptr, sel_now, ctx_snap, 0, pool_dev, cache, slot_of, rec + U, xs));
            HSAB_TRY(hipEventRecord(e->ev_copy[1], xs));
            HSAB_TRY(attend_after(e->ev_copy[1]));
        }
        HSAB_TRY(mark(2, xs));
        HSAB_TRY(gpu_plan_copy(e, t & 1, resident, sel_now, ctx_snap, 1, pool_dev, cache, slot_of, rec, xs));
        HSAB_TRY(mark(3, xs));
        HSAB_TRY(hipEventRecord(e->done[ring], xs));
        for (int b = 0; b < s.B; ++b) e->n_ctx[b] += 1;
        e->ring_delta[ring] = e->ring_cold[ring] = -1;   // known once the copy stream gets there
        delta_bytes = cold_bytes = -1;
        copies = -1;
        t0 = t1 = clk::now();
    } else {
        // ---- host: S_b(t), plans, one copy per run of blocks
        t0 = clk::now();
        HSAB_TRY(hipEventSynchronize(e->ev_sel));
        t1 = clk::now();
        std::memcpy(e->cur_sel.data(), e->sel_h + (size_t)ring * nsel, nsel * sizeof(int32_t));
        for (int b = 0; b < s.B; ++b) e->n_ctx[b] += 1;
        if (e->step == 0) {   // cold start: fill S_b(0) synchronously
            for (int u = 0; u < U; ++u) tail_blocks(e->n_ctx[u / s.Hkv], e->jp[u / s.Hkv], s.bs, &e->tail[2 * u]);
            if (offload_plan(s, e->n_slots, e->none.data(), e->cur_sel.data(), e->tail.data(), e->slot_map.data(),
                             e->plan_h[1], &cold_bytes) != HSAB_OK) {
                *einval = 1;
                return hipSuccess;
            }
            HSAB_TRY(offload_copy(s, e->n_slots, host_pool, cache, e->plan_h[1], e->plan_d[1], slot_of, xs,
                                  e->ev_copy[1], &calls, e->copy_mode, &e->mp[1]));
            copies += calls;
            HSAB_TRY(attend_after(e->ev_copy[1]));
        }
        for (int u = 0; u < U; ++u) tail_blocks(e->n_ctx[u / s.Hkv] + 1, e->jp[u / s.Hkv], s.bs, &e->tail[2 * u]);
        const int32_t* R = e->step == 0 ? e->cur_sel.data() : e->prev_sel.data();
        if (offload_plan(s, e->n_slots, R, e->cur_sel.data(), e->tail.data(), e->slot_map.data(), e->plan_h[t & 1],
                         &delta_bytes) != HSAB_OK) {
            *einval = 1;
            return hipSuccess;
        }
        HSAB_TRY(mark(2, xs));
        HSAB_TRY(offload_copy(s, e->n_slots, host_pool, cache, e->plan_h[t & 1], e->plan_d[t & 1], slot_of, xs,
                              e->ev_copy[t & 1], &calls, e->copy_mode, &e->mp[t & 1]));
        copies += calls;
        HSAB_TRY(mark(3, xs));
        e->prev_sel.swap(e->cur_sel);
        e->ring_delta[ring] = delta_bytes;
        e->ring_cold[ring] = cold_bytes;
    }
    const auto t2 = clk::now();
    if (st) {
        const int64_t blk_bytes = (int64_t)e->blk_elems * 2;
        st->step = e->step;
        st->delta_bytes = delta_bytes;
        st->delta_blocks = delta_bytes < 0 ? -1 : (int32_t)(delta_bytes / blk_bytes);
        st->cold_bytes = cold_bytes;
        st->n_copies = copies;
        st->host_wait_ms = std::chrono::duration<float, std::milli>(t1 - t0).count();
        st->host_plan_ms = std::chrono::duration<float, std::milli>(t2 - t1).count() +
                           (e->gpu_plan ? std::chrono::duration<float, std::milli>(t0 - t_in).count() : 0.f);
    }
    e->step += 1;
    return hipSuccess;
}

// Delta and cold-fill bytes of a step among the last TIMING_RING (waits for
// that step's copies when the GPU planned them).
hipError_t offload_step_delta(hsab_offload_engine* e, int64_t step, int64_t* delta_bytes, int64_t* cold_bytes) {
    const int ring = (int)(step % TIMING_RING);
    if (e->ring_delta[ring] < 0) {
        HSAB_TRY(hipEventSynchronize(e->done[ring]));
        const int32_t* rec = e->rec_h + (size_t)ring * 2 * e->U;
        int64_t d = 0, c = 0;
        for (int u = 0; u < e->U; ++u) {
            d += rec[u];
            if (step == 0) c += rec[e->U + u];
        }
        const int64_t blk_bytes = (int64_t)e->blk_elems * 2;
        e->ring_delta[ring] = d * blk_bytes;
        e->ring_cold[ring] = c * blk_bytes;
    }
    *delta_bytes = e->ring_delta[ring];
    *cold_bytes = e->ring_cold[ring];
    return hipSuccess;
}

// Timestamps for the steps enqueued from now on (off by default).
void offload_set_timing(hsab_offload_engine* e, bool on) { e->timing = on; }
bool offload_step_timed(const hsab_offload_engine* e, int64_t step) { return e->ring_timed[step % TIMING_RING]; }

// GPU times of a finished step enqueued with timing on (within the last
// TIMING_RING), see hsab_offload_timing. Waits for that step's events.
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

// S_b of the last step: the host's copy (host planning), or the mapped
// buffer the selection kernel wrote (after that kernel).
const int32_t* offload_last_selection(hsab_offload_engine* e) {
    if (!e->gpu_plan) return e->prev_sel.data();
    if (hipEventSynchronize(e->ev_sel) != hipSuccess) return nullptr;
    return e->sel_h + (size_t)((e->step - 1) % TIMING_RING) * e->U * e->s.kb;
}

// S_b of a step among the last TIMING_RING. With host planning the host
// waited for it when the step was enqueued; with GPU planning the step's
// copies (planned from it) are waited for.
const int32_t* offload_step_selection(hsab_offload_engine* e, int64_t step) {
    const int ring = (int)(step % TIMING_RING);
    if (e->gpu_plan && hipEventSynchronize(e->done[ring]) != hipSuccess) return nullptr;
    return e->sel_h + (size_t)ring * e->U * e->s.kb;
}
int64_t offload_steps(const hsab_offload_engine* e) { return e->step; }
const Shape& offload_shape(const hsab_offload_engine* e) { return e->s; }

}  // namespace hsab
