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
// non-NaN values). Every non-NaN float maps to a key >= 0x007fffff, so 0 is
// free to mark "no entry".
__device__ __forceinline__ uint32_t f32_key(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Label channel indices come from the caller; keep them inside the row.
__device__ __forceinline__ int clamp_ch(int c, int dk) { return c < 0 ? 0 : (c >= dk ? dk - 1 : c); }

__device__ __forceinline__ uint4 ldg16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 ldg8(const void* p) { return *reinterpret_cast<const uint2*>(p); }

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ i16x4_t as_i16x4(uint2 v) { return __builtin_bit_cast(i16x4_t, v); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// ---------------------------------------------------------------------------
// Exact block-wide top-k selection with stable ties.
//
// NW waves hold up to NW*64*PT keys in registers; with pt <= PT slots in
// use, key j of lane `lane` in wave w is entry i = (w*pt + j)*64 + lane.
// Keys are uint32 with 0 = empty.
// select() finds the k-th largest key T by bit-serial refinement (two bits
// per round, one barrier per round), then keeps every key > T and the first
// (k - #{key > T}) keys == T in entry order, and calls emit(pos, i) with
// pos = rank of entry i among the kept ones in entry order (0..k_eff-1).
// Returns k_eff = min(k, number of nonzero keys).
//
// lds must hold 2*4*NW + 2*NW uint32 (counts are double buffered by round
// parity, so one barrier per round suffices).
template <int NW, int PT>
struct TopK {
    static constexpr int LDS_WORDS = 2 * 4 * NW + 2 * NW;

    template <typename Emit>
    __device__ static int select(const uint32_t (&key)[PT], int pt, int k, uint32_t* lds, Emit emit) {
        const int lane = threadIdx.x & 63;
        const int w = threadIdx.x >> 6;
        const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

        // number of nonzero keys
        uint32_t nz = 0;
#pragma unroll
        for (int j = 0; j < PT; ++j)
            if (j < pt) nz += __popcll(__ballot(key[j] != 0u));
        uint32_t n_valid = block_sum<0>(nz, lds);
        int k_eff = k < (int)n_valid ? k : (int)n_valid;
        if (k_eff <= 0) return 0;

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
            uint32_t* slot = lds + (round & 1) * 4 * NW;
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

        // per-wave counts of keys > T and == T
        uint32_t gt = 0, eq = 0;
#pragma unroll
        for (int j = 0; j < PT; ++j) {
            if (j < pt) {
                gt += __popcll(__ballot(key[j] > T));
                eq += __popcll(__ballot(key[j] == T));
            }
        }
        uint32_t* cnt = lds + 8 * NW;
        if (lane == 0) { cnt[w] = gt; cnt[NW + w] = eq; }
        __syncthreads();
        uint32_t gt_tot = 0, gt_before = 0, eq_before = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            gt_tot += cnt[i];
            if (i < w) { gt_before += cnt[i]; eq_before += cnt[NW + i]; }
        }
        const uint32_t need_eq = (uint32_t)k_eff - gt_tot;
        uint32_t sel_run = gt_before + (eq_before < need_eq ? eq_before : need_eq);
        uint32_t eq_run = eq_before;
#pragma unroll
        for (int j = 0; j < PT; ++j) {
            if (j < pt) {
                const bool is_gt = key[j] > T, is_eq = key[j] == T;
                const uint64_t meq = __ballot(is_eq);
                const uint32_t eq_rank = eq_run + __popcll(meq & lt);
                const bool sel = is_gt || (is_eq && eq_rank < need_eq);
                const uint64_t msel = __ballot(sel);
                if (sel) emit((int)(sel_run + __popcll(msel & lt)), (w * pt + j) * 64 + lane);
                eq_run += __popcll(meq);
                sel_run += __popcll(msel);
            }
        }
        __syncthreads();   // lds free for the caller again
        return k_eff;
    }

    // Sum of one value per wave (taken from lane 0's argument) over the block.
    template <int TAG>
    __device__ static uint32_t block_sum(uint32_t v, uint32_t* lds) {
        const int w = threadIdx.x >> 6;
        uint32_t* s = lds + 8 * NW;
        if ((threadIdx.x & 63) == 0) s[w] = v;
        __syncthreads();
        uint32_t t = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i) t += s[i];
        __syncthreads();
        return t;
    }
};

}  // namespace hsab
