// Device helpers shared by the gfx950 kernels of libhsab.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hsab {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int WAVE = 64;

__device__ __forceinline__ float bf16_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Low and high bf16 of a packed 32-bit word, widened exactly.
__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Keep the bf16 lanes of w whose sign bit is clear (q+) or set (q-); the
// other lanes become +0. Exact: the kept values are unchanged.
__device__ __forceinline__ uint32_t bf16x2_pos(uint32_t w) {
    uint32_t m = ((w & 0x80008000u) >> 15) * 0xffffu;   // 0xffff per negative lane
    return w & ~m;
}
__device__ __forceinline__ uint32_t bf16x2_neg(uint32_t w) {
    uint32_t m = ((w & 0x80008000u) >> 15) * 0xffffu;
    return w & m;
}

// Order-preserving map of fp32 onto uint32 (a > b  <=>  key(a) > key(b) for
// non-NaN values; -0 and +0 share one key). Every non-NaN float maps to a
// key >= 0x007fffff, so 0 is free to mark "no entry".
__device__ __forceinline__ uint32_t f32_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_f32(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Label channel indices come from the caller; keep them inside the row.
__device__ __forceinline__ int clamp_ch(int c, int dk) { return c < 0 ? 0 : (c >= dk ? dk - 1 : c); }

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ldg8(const void* p) { return *reinterpret_cast<const uint2*>(p); }

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ i16x4_t as_i16x4(uint2 v) { return __builtin_bit_cast(i16x4_t, v); }

// ---------------------------------------------------------------------------
// Exact block-wide top-k selection with stable ties.
//
// NW waves hold up to NW*64*PT keys in registers; with pt <= PT slots in
// use, key j of lane `lane` in wave w is entry i = (w*pt + j)*64 + lane.
// Keys are uint32 from f32_key with 0 = empty. select() keeps the
// k_eff = min(k, #nonempty) largest keys, preferring the lower entry among
// equal keys, and calls emit(pos, i) for each kept entry i with pos its rank
// in entry order (0..k_eff-1). Returns k_eff.
//
// Method: a 2048-bin histogram of the key values over their [min, max]
// range. The bin map is monotone (non-decreasing) in the key, so every key
// in a higher bin is strictly larger than every key in a lower one: the bins
// above the bin holding the k-th largest key are kept whole, the bins below
// are dropped, and only that one bin's entries are ranked exactly. If that
// bin holds more than CMAX entries (or the range is not finite) the k-th
// largest key is found instead by bit-serial refinement over all keys, two
// bits per round.
template <int NW, int PT>
struct TopK {
    static constexpr int NT = NW * 64;
    static constexpr int NBIN = 2048;
    static constexpr int CMAX = 1024;
    static constexpr int BPT = NBIN / NT;     // bins per thread in the scan
    static_assert(NBIN % NT == 0, "bins must split evenly");
    // red layout: [0,8NW) round counts (two parity slots of 4NW),
    // [8NW,10NW) fallback tie counts, [10NW,11NW) compaction counts,
    // [11NW,12NW) scan wave sums, then 4 words of results.
    struct Smem {
        uint32_t hist[NBIN];
        uint32_t ckey[CMAX];
        int32_t cidx[CMAX];
        uint32_t red[12 * NW + 4];
    };

    __device__ static uint32_t wave_sum(uint32_t v) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
        return v;
    }
    __device__ static uint32_t wave_min(uint32_t v) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor(v, o));
        return v;
    }
    __device__ static uint32_t wave_max(uint32_t v) {
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor(v, o));
        return v;
    }

    template <typename Emit>
    __device__ static int select(const uint32_t (&key)[PT], int pt, int k, Smem& sm, Emit emit) {
        const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
        uint32_t* red = sm.red;
        uint32_t* res = red + 12 * NW;   // [0] pivot bin, [1] needed from it, [2] candidate count
        // 1) clear the histogram; range and count of the nonempty keys
        for (int i = tid; i < NBIN; i += NT) sm.hist[i] = 0u;
        uint32_t lmin = 0xffffffffu, lmax = 0u, lcnt = 0u;
#pragma unroll
        for (int j = 0; j < PT; ++j)
            if (j < pt && key[j] != 0u) { lmin = min(lmin, key[j]); lmax = max(lmax, key[j]); ++lcnt; }
        lmin = wave_min(lmin);
        lmax = wave_max(lmax);
        lcnt = wave_sum(lcnt);
        if (lane == 0) { red[w] = lmin; red[NW + w] = lmax; red[2 * NW + w] = lcnt; }
        if (tid == 0) res[2] = 0u;
        __syncthreads();
        uint32_t kmin = 0xffffffffu, kmax = 0u, nval = 0u;
#pragma unroll
        for (int i = 0; i < NW; ++i) { kmin = min(kmin, red[i]); kmax = max(kmax, red[NW + i]); nval += red[2 * NW + i]; }
        const int k_eff = k < (int)nval ? k : (int)nval;
        if (k_eff <= 0) { __syncthreads(); return 0; }
        if (k_eff == (int)nval) {   // every nonempty key is kept
            compact(key, pt, [&](int j) { return key[j] != 0u; }, red, emit);
            return k_eff;
        }
        const float vmin = key_f32(kmin), vmax = key_f32(kmax);
        const float range = vmax - vmin;
        const float scale = (float)NBIN / range;
        const bool binned = isfinite(range) && range > 0.f && isfinite(scale);
        auto bin = [&](uint32_t kk) {
            const int b = (int)((key_f32(kk) - vmin) * scale);
            return b < 0 ? 0 : (b >= NBIN ? NBIN - 1 : b);
        };
        int bstar = -1, need = 0;
        uint32_t m = 0;
        if (binned) {
            // 2) histogram
#pragma unroll
            for (int j = 0; j < PT; ++j)
                if (j < pt && key[j] != 0u) atomicAdd(&sm.hist[bin(key[j])], 1u);
            __syncthreads();
            // 3) thread t owns bins NBIN-1-(t*BPT+e), e < BPT (from the top);
            //    an exclusive scan in thread order gives the count above them
            uint32_t hv[BPT], loc = 0;
#pragma unroll
            for (int e = 0; e < BPT; ++e) { hv[e] = sm.hist[NBIN - 1 - (tid * BPT + e)]; loc += hv[e]; }
            uint32_t inc = loc;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t y = __shfl_up(inc, o);
                if (lane >= o) inc += y;
            }
            uint32_t* wsum = red + 11 * NW;
            if (lane == 63) wsum[w] = inc;
            __syncthreads();
            uint32_t above = inc - loc;
            for (int i = 0; i < w; ++i) above += wsum[i];
#pragma unroll
            for (int e = 0; e < BPT; ++e) {
                if (above < (uint32_t)k_eff && above + hv[e] >= (uint32_t)k_eff) {
                    res[0] = (uint32_t)(NBIN - 1 - (tid * BPT + e));
                    res[1] = (uint32_t)k_eff - above;
                }
                above += hv[e];
            }
            __syncthreads();
            bstar = (int)res[0];
            need = (int)res[1];
            m = sm.hist[bstar];
        }
        if (binned && m <= (uint32_t)CMAX) {
            // 4) gather the pivot bin's entries, rank them by (key desc, entry asc)
#pragma unroll
            for (int j = 0; j < PT; ++j) {
                if (j < pt && key[j] != 0u && bin(key[j]) == bstar) {
                    const uint32_t slot = atomicAdd(&res[2], 1u);
                    sm.ckey[slot] = key[j];
                    sm.cidx[slot] = (w * pt + j) * 64 + lane;
                }
            }
            __syncthreads();
            bool keep[PT];
#pragma unroll
            for (int j = 0; j < PT; ++j) {
                keep[j] = false;
                if (j < pt && key[j] != 0u) {
                    const int bj = bin(key[j]);
                    if (bj > bstar) {
                        keep[j] = true;
                    } else if (bj == bstar) {
                        const int me = (w * pt + j) * 64 + lane;
                        int rank = 0;
                        for (uint32_t c = 0; c < m; ++c) {
                            const uint32_t ck = sm.ckey[c];
                            rank += (ck > key[j]) || (ck == key[j] && sm.cidx[c] < me);
                        }
                        keep[j] = rank < need;
                    }
                }
            }
            compact(key, pt, [&](int j) { return keep[j]; }, red, emit);
            return k_eff;
        }
        // fallback: bit-serial search for the k-th largest key T
        uint32_t prefix = 0;
        int round = 1;
        for (int bit = 30; bit >= 0; bit -= 2, ++round) {
            const uint32_t c1 = prefix | (1u << bit), c2 = prefix | (2u << bit), c3 = prefix | (3u << bit);
            uint32_t n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
            for (int j = 0; j < PT; ++j) {
                if (j < pt) {
                    n1 += __popcll(__ballot(key[j] >= c1));
                    n2 += __popcll(__ballot(key[j] >= c2));
                    n3 += __popcll(__ballot(key[j] >= c3));
                }
            }
            uint32_t* slot = red + (round & 1) * 4 * NW;
            if (lane == 0) { slot[w] = n1; slot[NW + w] = n2; slot[2 * NW + w] = n3; }
            __syncthreads();
            uint32_t t1 = 0, t2 = 0, t3 = 0;
#pragma unroll
            for (int i = 0; i < NW; ++i) { t1 += slot[i]; t2 += slot[NW + i]; t3 += slot[2 * NW + i]; }
            if (t3 >= (uint32_t)k_eff) prefix = c3;
            else if (t2 >= (uint32_t)k_eff) prefix = c2;
            else if (t1 >= (uint32_t)k_eff) prefix = c1;
        }
        const uint32_t T = prefix;
        // keys > T are kept; among keys == T the first (k_eff - #{> T}) in entry order
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int j = 0; j < PT; ++j)
            if (j < pt) { gt += __popcll(__ballot(key[j] > T)); eq += __popcll(__ballot(key[j] == T)); }
        uint32_t* cnt = red + 8 * NW;
        if (lane == 0) { cnt[w] = gt; cnt[NW + w] = eq; }
        __syncthreads();
        uint32_t gt_tot = 0, eq_before = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i) { gt_tot += cnt[i]; if (i < w) eq_before += cnt[NW + i]; }
        const uint32_t need_eq = (uint32_t)k_eff - gt_tot;
        const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        bool keep[PT];
        uint32_t eq_run = eq_before;
#pragma unroll
        for (int j = 0; j < PT; ++j) {
            keep[j] = false;
            if (j < pt) {
                const uint64_t meq = __ballot(key[j] == T);
                keep[j] = key[j] > T || (key[j] == T && eq_run + __popcll(meq & lt) < need_eq);
                eq_run += __popcll(meq);
            }
        }
        compact(key, pt, [&](int j) { return keep[j]; }, red, emit);
        return k_eff;
    }

    // Emit the entries whose predicate holds, ranked in entry order.
    template <typename Pred, typename Emit>
    __device__ static void compact(const uint32_t (&key)[PT], int pt, Pred pred, uint32_t* red, Emit emit) {
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        uint32_t cntw = 0;
#pragma unroll
        for (int j = 0; j < PT; ++j)
            if (j < pt) cntw += __popcll(__ballot(pred(j)));
        uint32_t* c = red + 10 * NW;
        if (lane == 0) c[w] = cntw;
        __syncthreads();
        uint32_t run = 0;
        for (int i = 0; i < w; ++i) run += c[i];
#pragma unroll
        for (int j = 0; j < PT; ++j) {
            if (j < pt) {
                const bool p = pred(j);
                const uint64_t mk = __ballot(p);
                if (p) emit((int)(run + __popcll(mk & lt)), (w * pt + j) * 64 + lane);
                run += __popcll(mk);
            }
        }
        __syncthreads();   // shared scratch free for the caller again
    }
};

}  // namespace hsab
