// Union of the token sets of the query heads of one KV head, for
// per-query-head selection: each head keeps its own tokens (Quest-style
// selection per head, the mode the pages' one-product block scoring for
// shared-KV heads leaves open), and the attention reads every row the
// group needs once, masking per head.
//
// One 1024-thread workgroup per unit. The heads' lists are ascending token
// positions (-1 padded); a window of positions gets one LDS bit set per
// head (bit t of head h: head h kept token t), the words of the window are
// OR-ed over the heads, counted and prefix-summed over the workgroup into
// per-word entry offsets, and every set bit becomes one union entry (its
// position, and the bits of the heads that hold it as the mask). Entries
// are emitted by entry, not by word: thread e finds the word holding entry
// e by binary search over the offsets and writes slot e, so the stores are
// coalesced and the dense words (the kept tokens cluster in kept blocks)
// are not left to a few lanes. Each window starts at the smallest listed
// position past the previous window (the first at the smallest of all, or
// at 0 when one window covers the context), so windows holding no entry
// are never visited and the union comes out ascending; positions at or
// past the unit's context length are dropped.
// The LDS per window is fixed (60 KiB).
#include <climits>
#include "common.h"
#include "kernels.h"

namespace hsab {

namespace {

constexpr int UNION_THREADS = 1024;
constexpr int UNION_LDS_WORDS = 15360;   // 60 KiB per window: head bitmaps [G][wph], word offsets [wph]

// G: heads per group (compile time); (G + 1) * wph <= UNION_LDS_WORDS.
template <int G>
__global__ __launch_bounds__(UNION_THREADS) void union_kernel(const int32_t* __restrict__ tok_idx,
                                                              const int32_t* __restrict__ ctx_len,
                                                              int32_t* __restrict__ union_idx,
                                                              uint32_t* __restrict__ union_mask, int Hkv, int kt,
                                                              int max_ctx, int wph) {
    __shared__ uint32_t bits[UNION_LDS_WORDS];   // [G][wph] head bitmaps, then [wph] word offsets
    uint32_t* off = bits + G * wph;
    __shared__ uint32_t s_wsum[UNION_THREADS / 64];
    __shared__ int s_next;                        // smallest listed position past the window
    const int unit = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int E = G * kt;
    const int32_t* L = tok_idx + (size_t)unit * E;
    int32_t* U = union_idx + (size_t)unit * E;
    uint32_t* M = union_mask + (size_t)unit * E;
    int n = ctx_len[unit / Hkv];
    n = n < 0 ? 0 : (n > max_ctx ? max_ctx : n);
    const int span = wph * 32;                        // positions per window
    const int per = (wph + UNION_THREADS - 1) / UNION_THREADS;   // words per thread
    int base = 0;                                     // entries written so far
    int w0 = 0;   // one window from 0 covers a context no longer than a window
    if (n > span) {
        if (tid == 0) s_next = INT_MAX;
        __syncthreads();
        // the smallest listed position: a minimum per thread, then per wave
        // (same-address LDS atomics serialise, one per wave is cheap)
        uint32_t lmin = INT_MAX;
        for (int e = tid; e < E; e += UNION_THREADS) {
            const int t = L[e];
            if (t >= 0 && t < n) lmin = (uint32_t)t < lmin ? (uint32_t)t : lmin;
        }
        lmin = wave_minmax<false>(lmin);
        if (lane == 0 && lmin != (uint32_t)INT_MAX) atomicMin(&s_next, (int)lmin);
        __syncthreads();
        w0 = s_next;   // INT_MAX: no entry at all
    }
    while (w0 < n) {
        __syncthreads();                              // every thread has read s_next
        if (tid == 0) s_next = INT_MAX;
        for (int i = tid; i < G * wph; i += UNION_THREADS) bits[i] = 0u;
        __syncthreads();
        const int w1 = n - w0 > span ? w0 + span : n;  // this window: positions [w0, w1)
        uint32_t nmin = INT_MAX;   // smallest listed position past this window
        for (int e = tid; e < E; e += UNION_THREADS) {
            const int t = L[e];
            if (t >= w0 && t < w1) {
                const int h = e / kt, o = t - w0;
                atomicOr(&bits[h * wph + (o >> 5)], 1u << (o & 31));
            } else if (t >= w1 && t < n) {
                nmin = (uint32_t)t < nmin ? (uint32_t)t : nmin;
            }
        }
        nmin = wave_minmax<false>(nmin);
        if (lane == 0 && nmin != (uint32_t)INT_MAX) atomicMin(&s_next, (int)nmin);
        __syncthreads();
        // this thread's words: [k0, k1) of the window
        const int k0 = tid * per, k1 = min(k0 + per, wph);
        uint32_t cnt = 0;
        for (int k = k0; k < k1; ++k) {
            uint32_t u = 0;
#pragma unroll
            for (int h = 0; h < G; ++h) u |= bits[h * wph + k];
            cnt += __popc(u);
        }
        const uint32_t incl = wave_scan_dpp(cnt);
        if (lane == 63) s_wsum[w] = incl;
        __syncthreads();
        uint32_t before = 0, total = 0;
        for (int i = 0; i < UNION_THREADS / 64; ++i) {
            const uint32_t x = s_wsum[i];
            before += i < w ? x : 0u;
            total += x;
        }
        // entries before each of this thread's words
        uint32_t run = before + incl - cnt;
        for (int k = k0; k < k1; ++k) {
            off[k] = run;
            uint32_t u = 0;
#pragma unroll
            for (int h = 0; h < G; ++h) u |= bits[h * wph + k];
            run += __popc(u);
        }
        __syncthreads();
        for (int e = tid; e < (int)total; e += UNION_THREADS) {
            // the last word whose offset is <= e holds entry e (words past
            // it start later; an empty word shares the next one's offset)
            int lo = 0, hi = wph - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (off[mid] <= (uint32_t)e) lo = mid; else hi = mid - 1;
            }
            uint32_t hw[G], u = 0;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                hw[h] = bits[h * wph + lo];
                u |= hw[h];
            }
            for (uint32_t r = (uint32_t)e - off[lo]; r > 0; --r) u &= u - 1;   // drop the lower entries
            const int bit = __ffs(u) - 1;
            uint32_t m = 0;
#pragma unroll
            for (int h = 0; h < G; ++h) m |= ((hw[h] >> bit) & 1u) << h;
            U[base + e] = w0 + lo * 32 + bit;
            M[base + e] = m;
        }
        base += (int)total;
        __syncthreads();   // the next window reuses bits and s_wsum
        w0 = s_next;
    }
    for (int e = base + tid; e < E; e += UNION_THREADS) {
        U[e] = -1;
        M[e] = 0u;
    }
}

}  // namespace

hipError_t launch_union(const Shape& s, const int32_t* tok_idx, const int32_t* ctx_len, int32_t* union_idx,
                        uint32_t* union_mask, hipStream_t st) {
    const int words = (s.max_ctx + 31) / 32;
    const int cap = UNION_LDS_WORDS / (s.G + 1);
    const int wph = words < cap ? words : cap;
    const dim3 grid(s.B * s.Hkv), block(UNION_THREADS);
    switch (s.G) {   // the group sizes the masked attention takes
        case 1: hipLaunchKernelGGL(union_kernel<1>, grid, block, 0, st, tok_idx, ctx_len, union_idx, union_mask,
                                   s.Hkv, s.kt, s.max_ctx, wph); break;
        case 2: hipLaunchKernelGGL(union_kernel<2>, grid, block, 0, st, tok_idx, ctx_len, union_idx, union_mask,
                                   s.Hkv, s.kt, s.max_ctx, wph); break;
        case 4: hipLaunchKernelGGL(union_kernel<4>, grid, block, 0, st, tok_idx, ctx_len, union_idx, union_mask,
                                   s.Hkv, s.kt, s.max_ctx, wph); break;
        case 8: hipLaunchKernelGGL(union_kernel<8>, grid, block, 0, st, tok_idx, ctx_len, union_idx, union_mask,
                                   s.Hkv, s.kt, s.max_ctx, wph); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace hsab
