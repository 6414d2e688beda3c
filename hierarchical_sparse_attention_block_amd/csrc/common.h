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
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Low and high bf16 of a packed 32-bit word, widened exactly.
__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Sign split of a packed bf16 pair. As signed 16-bit integers the halves
// whose sign bit is clear are exactly the non-negative ones, so a packed
// integer max with 0 leaves q+ (the others become +0), and w ^ q+ leaves
// q- (the halves with the sign bit set). neg = ~0 selects q-, 0 selects q+.
// Exact: kept values are unchanged.
typedef short s16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_split(uint32_t w, uint32_t neg) {
    const s16x2_t h = __builtin_bit_cast(s16x2_t, w);
    const uint32_t pos = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(h, s16x2_t{0, 0}));
    return pos ^ (w & neg);
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
__device__ __forceinline__ uint32_t ldg4(const void* p) { return *reinterpret_cast<const uint32_t*>(p); }
// Non-temporal forms, for rows a step reads once (the nontemporal hint on
// the load: the line is not kept in the caches for reuse).
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ldg16_nt(const void* p) {
    const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 ldg8_nt(const void* p) {
    const u32x2v v = __builtin_nontemporal_load(reinterpret_cast<const u32x2v*>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t ldg4_nt(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// a.lo*b.lo + a.hi*b.hi + c for packed bf16 pairs, fp32 accumulate
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Eight packed bf16 widened to fp32, exactly.
__device__ __forceinline__ void widen8(uint4 v, float (&f)[8]) {
    f[0] = lo_f32(v.x); f[1] = hi_f32(v.x); f[2] = lo_f32(v.y); f[3] = hi_f32(v.y);
    f[4] = lo_f32(v.z); f[5] = hi_f32(v.z); f[6] = lo_f32(v.w); f[7] = hi_f32(v.w);
}

// Cross-row partners on gfx950 without LDS: v_permlane16_swap pairs row 2i
// with row 2i+1 (lane ^ 16), v_permlane32_swap pairs the two wave halves
// (lane ^ 32). Both results of the swap hold the two partners' values.
__device__ __forceinline__ float max_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Inclusive prefix sum over the 64 lanes: DPP row shifts by 1, 2, 4, 8
// within each 16-lane row, then the row broadcasts of lanes 15 and 31.
__device__ __forceinline__ uint32_t wave_scan_dpp(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);
    return v;
}

// Wave-wide min / max of a uint32 through DPP lane permutations (quad
// swaps, half-row and row mirrors) and four readlanes; result is uniform.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_minmax(uint32_t v) {
    auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // lane ^ 1
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // lane ^ 2
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // half-row mirror
    v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
    const uint32_t a = __builtin_amdgcn_readlane((int)v, 0), b = __builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = __builtin_amdgcn_readlane((int)v, 32), d = __builtin_amdgcn_readlane((int)v, 48);
    return op(op(a, b), op(c, d));
}

// Sum over aligned groups of N lanes (N = 8, 16 or 32); every lane of a
// group gets the group's total. Within a 16-lane row the partners come from
// DPP lane swaps (lane ^ 1, lane ^ 2, half-row mirror, row mirror); the
// step across two rows is a permlane16 swap.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N == 8 || N == 16 || N == 32, "group size");
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));
    if (N >= 16) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));
    if (N == 32) v = sum_xor16(v);
    return v;
}

// Maximum over aligned groups of N lanes (N = 8 or 16), same lane swaps.
template <int N>
__device__ __forceinline__ float group_max(float v) {
    static_assert(N == 8 || N == 16, "group size");
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false)));
    if (N == 16) v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false)));
    return v;
}


__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Two floats as a packed bf16 pair (a in the low half), rounded to nearest
// even by the gfx950 packed conversion.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}
// a = hi + lo with hi, lo bf16 pairs: hi holds a's leading 8 mantissa
// bits, lo the next 8 (the product of either with a bf16 value is exact in
// fp32 accumulation)
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = pk_bf16(a, b);
    lo = pk_bf16(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// fp8 e4m3 (OCP "fn": sign, 4 exponent bits with bias 7, 3 mantissa bits,
// exponent 0 subnormal with step 2^-9, 0x7f/0xff NaN, largest finite 448)
// from a bf16 value, rounded outward: up (toward +inf) or down (toward
// -inf) to the nearest grid value, saturating at +-448. The magnitude is
// first truncated; an inexact result then steps one code away from zero
// when that is the rounding direction (codes are monotone in magnitude).
__device__ __forceinline__ uint32_t f8_outward(uint32_t b, bool up) {
    const uint32_t sgn = (b >> 15) & 1u, E = (b >> 7) & 0xffu, M = b & 0x7fu;
    uint32_t code;
    bool inexact;
    if (E == 0) {                       // bf16 zero or subnormal: below every nonzero e4m3 value
        code = 0;
        inexact = M != 0;
    } else {
        const int e = (int)E - 120;     // e4m3 exponent field (unbiased + 7)
        if (e >= 1) {
            code = ((uint32_t)e << 3) | (M >> 4);
            inexact = (M & 0xfu) != 0;
            if (code > 0x7eu) {         // beyond 448
                code = 0x7eu;
                inexact = true;
            }
        } else {                        // e4m3 subnormal range: |x| / 2^-9 = (128 + M) * 2^(e - 5)
            const int sh = 5 - e;       // >= 5
            const uint32_t F = 128u + M;
            code = sh >= 9 ? 0u : (F >> sh);
            inexact = sh >= 9 ? true : (F & ((1u << sh) - 1u)) != 0;
        }
    }
    if (inexact && (up != (sgn != 0u))) code = code + 1u > 0x7eu ? 0x7eu : code + 1u;
    return (sgn << 7) | code;
}
// bf16 value b (bit pattern) rounded to the nearest e4m3 value, a value
// halfway between two codes going to the even code, saturating at +-448:
// the magnitude's truncated code plus one when the dropped bits exceed half
// a step (or equal it and the code is odd); codes are monotone in
// magnitude, so a carry into the exponent field is the next value up.
__device__ __forceinline__ uint32_t f8_nearest(uint32_t b) {
    const uint32_t sgn = (b >> 15) & 1u, E = (b >> 7) & 0xffu, M = b & 0x7fu;
    uint32_t code = 0, rem = 0, half = 1;
    if (E != 0) {                       // bf16 zeros and subnormals round to zero
        const int e = (int)E - 120;     // e4m3 exponent field (unbiased + 7)
        if (e >= 1) {
            code = ((uint32_t)e << 3) | (M >> 4);
            rem = M & 0xfu;
            half = 8u;
        } else {                        // e4m3 subnormal range: |x| / 2^-9 = (128 + M) * 2^(e - 5)
            const int sh = 5 - e;       // >= 5
            const uint32_t F = 128u + M;
            if (sh < 9) {
                code = F >> sh;
                rem = F & ((1u << sh) - 1u);
                half = 1u << (sh - 1);
            }                           // sh >= 9: below a quarter of the smallest step
        }
    }
    if (code >= 0x7eu) {
        code = 0x7eu;                   // 448 and beyond: saturate
    } else if (rem > half || (rem == half && (code & 1u))) {
        code += 1u;
    }
    return (sgn << 7) | (code > 0x7eu ? 0x7eu : code);
}
// value of an e4m3 code (finite codes only)
__device__ __forceinline__ float f8_value(uint32_t code) {
    return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}
// eight e4m3 values (bytes of w, lowest first) as eight bf16 (exact)
__device__ __forceinline__ uint4 f8x8_bf16(uint2 w) {
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, false), b = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, true);
    const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, false), d = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, true);
    return make_uint4(pk_bf16(a[0], a[1]), pk_bf16(b[0], b[1]), pk_bf16(c[0], c[1]), pk_bf16(d[0], d[1]));
}

// four e4m3 values (bytes of w, lowest first) as four bf16 (exact)
__device__ __forceinline__ uint2 f8x4_bf16(uint32_t w) {
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(w, false), b = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
    return make_uint2(pk_bf16(a[0], a[1]), pk_bf16(b[0], b[1]));
}

// Label row entry idx: bf16 bits, or (lab8) the nearest e4m3 byte.
__device__ __forceinline__ void label_put(uint16_t* klabel, size_t idx, uint16_t kb, bool lab8) {
    if (lab8)
        reinterpret_cast<uint8_t*>(klabel)[idx] = (uint8_t)f8_nearest(kb);
    else
        klabel[idx] = kb;
}

// Metadata of block blk: its max row then its min row, d_k values each,
// bf16 or (meta8) e4m3 bytes.
__device__ __forceinline__ uint8_t* meta_block(uint16_t* meta, size_t blk, int dk, bool meta8) {
    return reinterpret_cast<uint8_t*>(meta) + blk * (size_t)(2 * dk) * (meta8 ? 1u : 2u);
}
// Channel c of a block's metadata widened to include key value kb (bf16
// bits), or started from it when the block opens. In e4m3 the max rounds
// up and the min down; rounding is monotone, so widening rounded bounds
// equals rounding the widened ones.
__device__ __forceinline__ void meta_widen(uint8_t* M, int dk, int c, uint16_t kb, bool first, bool meta8) {
    if (meta8) {
        const uint32_t up = f8_outward(kb, true), dn = f8_outward(kb, false);
        if (first || f8_value(up) > f8_value(M[c])) M[c] = (uint8_t)up;
        if (first || f8_value(dn) < f8_value(M[dk + c])) M[dk + c] = (uint8_t)dn;
    } else {
        uint16_t* M16 = reinterpret_cast<uint16_t*>(M);
        const float kf = __uint_as_float((uint32_t)kb << 16);
        if (first || kf > __uint_as_float((uint32_t)M16[c] << 16)) M16[c] = kb;
        if (first || kf < __uint_as_float((uint32_t)M16[dk + c] << 16)) M16[dk + c] = kb;
    }
}

// Operand of the gfx950 transposing LDS read of four 16-bit elements.
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __attribute__((address_space(3))) s16x4_t* lds_s16x4(const uint16_t* p) {
    return (__attribute__((address_space(3))) s16x4_t*)(p);
}
__device__ __forceinline__ i16x4_t as_i16x4(uint2 v) { return __builtin_bit_cast(i16x4_t, v); }

}  // namespace hsab
