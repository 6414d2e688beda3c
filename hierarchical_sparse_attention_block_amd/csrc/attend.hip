// Exact attention over the kept tokens (AsyncTLS, gist.science/es
// explainer, section 2.A item 2: the final attention runs on the K_t
// selected tokens only), split over workgroups and merged by log-sum-exp.
//
// GQA path (d_k == d_v == D, G query heads per KV head): one workgroup of
// four waves takes 64 consecutive entries of the unit's token list; D/8
// lanes share a token (8 channels = 16 bytes each), so one wave load
// gathers 64/(D/8) whole key rows. Logits are fp32 (bf16 products are
// exact in fp32), kept in base-2 units (q pre-scaled by sm_scale*log2 e).
// Each wave keeps (max, sum, weighted values) per head; the workgroup
// merges its four waves and writes one partial per head; the combine
// kernel merges the partials of all splits.
//
// MLA path (values are the first d_v dims of the d_k-dim latent key rows,
// 32 query heads on one KV head): a workgroup takes 32 kept tokens; the
// 32x32 logit tile (tokens x heads) is four 16x16 tiles of
// v_mfma_f32_16x16x32_bf16, one per wave, with key rows and queries read
// straight from memory as A and B fragments; softmax runs in LDS; P.V runs
// in fp32 on the VALU from the value rows staged in LDS (each thread: one
// head, d_v/8 interleaved channels).
//
// Workgroup numbering: the dispatcher hands consecutive workgroups to the
// eight XCDs in turn, so workgroup L runs on XCD L % 8. All splits of a unit
// are given the same L % 8, which keeps a unit's rows and partials in one L2.
#include "common.h"
#include "kernels.h"

namespace hsab {

namespace {

// Row index (in rows of d_k elements from the K base) of token t of unit,
// or -1. Dense caches: unit*max_ctx + t. Block cache: slot s of the unit
// spans slot_rows rows (key rows first, then value rows), found through
// slot_of.
__device__ __forceinline__ long row_of(int t, int unit, int bs, int max_ctx, int nb_cap,
                                       const int32_t* __restrict__ slot_of, int n_slots, int slot_rows) {
    if (t < 0) return -1;
    if (!slot_of) return (t < max_ctx) ? (long)unit * max_ctx + t : -1;
    const int blk = t / bs;
    if (blk >= nb_cap) return -1;
    const int slot = slot_of[(size_t)unit * nb_cap + blk];
    if (slot < 0 || slot >= n_slots) return -1;
    return ((long)unit * n_slots + slot) * slot_rows + (t - blk * bs);
}

template <int D, int G>
__global__ __launch_bounds__(256) void attend_gqa_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const int32_t* __restrict__ tok_idx, const int32_t* __restrict__ slot_of, int n_slots,
    float* __restrict__ part_ml, float* __restrict__ part_acc, int Hkv, int bs, int kt,
    int max_ctx, int nb_cap, int n_splits, int units, float scale2, int slot_rows) {
    constexpr int LPT = D / 8;                         // lanes per token (8 channels each)
    constexpr int TPI = 64 / LPT;                      // tokens per wave load = lane groups per wave
    constexpr int TPW = ATT_TOK_PER_SPLIT / 4;         // tokens per wave
    constexpr int IT = TPW / TPI;                      // tokens per lane group
    constexpr int NP = 4 * TPI;                        // partial softmax states per workgroup
    static_assert(IT >= 1 && TPW % TPI == 0, "bad D");
    __shared__ float s_m[NP][G], s_l[NP][G];
    __shared__ float s_acc[NP][G][D];

    const int xcd = blockIdx.x & 7, y = blockIdx.x >> 3;
    const int unit = (y / n_splits) * 8 + xcd, split = y % n_splits;
    if (unit >= units) return;
    const int b = unit / Hkv, g = unit % Hkv;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cc = lane % LPT, ts = lane / LPT;

    float qf[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const uint4 v = ldg16(q + ((size_t)(b * Hkv + g) * G + h) * D + cc * 8);
        widen8(v, qf[h]);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[h][e] *= scale2;
    }

    // Three dependent rounds, each with all its loads in flight: token
    // positions, block slots (block cache only), then the K and V rows.
    // Loads are unconditional (invalid entries read row 0 and are masked)
    // so no round waits on a previous one's stragglers.
    uint4 kr[IT], vr[IT];
    bool ok[IT];
    long rows[IT];
    const int32_t* tl = tok_idx + (size_t)unit * kt;
    int tv[IT];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int ti = split * ATT_TOK_PER_SPLIT + wave * TPW + it * TPI + ts;
        const int t = tl[ti < kt ? ti : kt - 1];
        tv[it] = ti < kt ? t : -1;
    }
    if (slot_of) {
        int sl[IT];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int blk = tv[it] >= 0 ? tv[it] / bs : 0;
            sl[it] = slot_of[(size_t)unit * nb_cap + (blk < nb_cap ? blk : 0)];
        }
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int t = tv[it], blk = t >= 0 ? t / bs : 0;
            const bool v = t >= 0 && blk < nb_cap && sl[it] >= 0 && sl[it] < n_slots;
            rows[it] = v ? ((long)unit * n_slots + sl[it]) * slot_rows + (t - blk * bs) : -1;
        }
    } else {
#pragma unroll
        for (int it = 0; it < IT; ++it)
            rows[it] = (tv[it] >= 0 && tv[it] < max_ctx) ? (long)unit * max_ctx + tv[it] : -1;
    }
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        ok[it] = rows[it] >= 0;
        const long r = ok[it] ? rows[it] : 0;
        kr[it] = ldg16(K + r * D + cc * 8);
        vr[it] = ldg16(V + r * D + cc * 8);
    }
    // keep the value loads here, in flight with the key loads; left alone
    // the scheduler sinks them to their use after the logits
    __builtin_amdgcn_sched_barrier(0);

    // logits: 8-channel partial dots, summed over the token's lane group
    float z[IT][G];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        float kf[8];
        widen8(kr[it], kf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float p = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) p = fmaf(qf[h][e], kf[e], p);
            p = group_sum<LPT>(p);
            z[it][h] = ok[it] ? p : -INFINITY;
        }
    }

    // softmax state of this lane group's IT tokens; the groups of the
    // workgroup are merged once through LDS, no cross-group shuffles
    const int slot = wave * TPI + ts;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float m = z[0][h];
#pragma unroll
        for (int it = 1; it < IT; ++it) m = fmaxf(m, z[it][h]);
        float l = 0.f, acc[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        if (m != -INFINITY) {
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                float vf[8];
                widen8(vr[it], vf);
                const float p = ok[it] ? exp2f(z[it][h] - m) : 0.f;
                l += p;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = fmaf(p, vf[e], acc[e]);
            }
        }
        float4* dst = reinterpret_cast<float4*>(&s_acc[slot][h][cc * 8]);
        dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
        if (cc == 0) {
            s_m[slot][h] = m;
            s_l[slot][h] = l;
        }
    }
    __syncthreads();

    for (int p = threadIdx.x; p < G * D; p += blockDim.x) {
        const int h = p / D, c = p - h * D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NP; ++w) M = fmaxf(M, s_m[w][h]);
        float L = 0.f, A = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < NP; ++w) {
                const float mw = s_m[w][h];
                const float wt = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
                L = fmaf(s_l[w][h], wt, L);
                A = fmaf(s_acc[w][h][c], wt, A);
            }
        }
        const size_t bh = (size_t)(b * Hkv + g) * G + h;
        part_acc[(bh * n_splits + split) * D + c] = A;
        if (c == 0) {
            part_ml[(bh * n_splits + split) * 2 + 0] = M;
            part_ml[(bh * n_splits + split) * 2 + 1] = L;
        }
    }
}

// grid: as the GQA kernel; block 256 (4 waves). Hq = 32 * Hkv, d_k % 32 ==
// 0, d_k <= DKMAX, d_v % 64 == 0, d_v <= 512, values alias the first d_v
// key dims (absorbed latent). One workgroup takes T = 32 kept tokens:
//  1. the group's query fragments are requested first (registers), the
//     token rows and slots next; the 32 key rows (which hold the values)
//     are staged in LDS with every load in flight;
//  2. logits on v_mfma_f32_16x16x32_bf16: wave w multiplies token tile
//     w & 1 by head tile w >> 1 over the d_k / 32 steps;
//  3. softmax per head over the 32 tokens (8 lanes per head, DPP);
//  4. P.V on the same instruction with M = heads, N = 16 value channels,
//     K = the 32 tokens. P enters as two bf16 terms (hi + lo) so the
//     weights keep ~16 mantissa bits; V is exact in bf16.
// Operands of steps past d_k are zeros: the matrix instructions run for
// every step.
template <int DKMAX>
__global__ __launch_bounds__(256) void attend_mla_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ K, const int32_t* __restrict__ tok_idx,
    const int32_t* __restrict__ slot_of, int n_slots, float* __restrict__ part_ml,
    float* __restrict__ part_acc, int Hkv, int dk, int dv, int bs, int kt, int max_ctx, int nb_cap,
    int n_splits, int units, float scale2, int slot_rows) {
    constexpr int T = MLA_TOK_PER_SPLIT;   // 32 tokens
    constexpr int H = 32;                  // query heads per KV head
    constexpr int KSMAX = DKMAX / 32;      // logit steps
    constexpr int RS = DKMAX + 8;          // LDS row stride (elements): spreads rows over banks
    __shared__ __align__(16) uint16_t sK[T * RS];
    __shared__ float sS[T][H + 1];
    __shared__ float sm[H], sl[H];
    __shared__ long s_row[T];

    const int xcd = blockIdx.x & 7, y = blockIdx.x >> 3;
    const int unit = (y / n_splits) * 8 + xcd, split = y % n_splits;
    if (unit >= units) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int KS = dk / 32;
    const int mt = wave & 1, nt = wave >> 1;   // logit tile: tokens 16*mt.., heads 16*nt..

    // 1. query fragments (B operand: head nt*16 + lane%16, channels
    //    32*s + 8*(lane/16)..), then token rows
    uint4 qb[KSMAX];
    {
        const uint16_t* qr = q + ((size_t)unit * H + nt * 16 + (lane & 15)) * dk + (lane >> 4) * 8;
#pragma unroll
        for (int u = 0; u < KSMAX; ++u) qb[u] = u < KS ? ldg16(qr + u * 32) : make_uint4(0u, 0u, 0u, 0u);
    }
    if (tid < T) {
        const int ti = split * T + tid;
        const int t = ti < kt ? tok_idx[(size_t)unit * kt + ti] : -1;
        long row = -1;
        if (!slot_of) {
            row = (t >= 0 && t < max_ctx) ? (long)unit * max_ctx + t : -1;
        } else if (t >= 0) {
            const int blk = t / bs;
            const int sl_ = blk < nb_cap ? slot_of[(size_t)unit * nb_cap + blk] : -1;
            row = (sl_ >= 0 && sl_ < n_slots) ? ((long)unit * n_slots + sl_) * slot_rows + (t - blk * bs) : -1;
        }
        s_row[tid] = row;
    }
    __syncthreads();

    // key rows into LDS: chunk c of token r at sK[r * RS + 8c]; every load
    // of the thread is issued before the first store
    {
        const int cpr = dk / 8;
        constexpr int PER = (T * DKMAX / 8 + 255) / 256;
        uint4 v[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = tid + i * 256;
            const int r = c / cpr, ch = c - r * cpr;
            const long row = c < T * cpr ? s_row[r] : -1;
            v[i] = row >= 0 ? ldg16(K + row * dk + ch * 8) : make_uint4(0u, 0u, 0u, 0u);
        }
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = tid + i * 256;
            if (c < T * cpr) {
                const int r = c / cpr, ch = c - r * cpr;
                *reinterpret_cast<uint4*>(&sK[r * RS + ch * 8]) = v[i];
            }
        }
    }
    __syncthreads();

    // 2. logits: A = key rows of tile mt from LDS, B = query fragments
    {
        const uint16_t* ar = &sK[(mt * 16 + (lane & 15)) * RS + (lane >> 4) * 8];
        f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < KSMAX; u += 2) {
            const uint4 a0 = u < KS ? *reinterpret_cast<const uint4*>(ar + u * 32) : make_uint4(0u, 0u, 0u, 0u);
            acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(qb[u]), acc0, 0, 0, 0);
            if (u + 1 < KSMAX) {
                const uint4 a1 =
                    u + 1 < KS ? *reinterpret_cast<const uint4*>(ar + (u + 1) * 32) : make_uint4(0u, 0u, 0u, 0u);
                acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(qb[u + 1]), acc1, 0, 0, 0);
            }
        }
        const f32x4_t acc = acc0 + acc1;
        // lane: head nt*16 + lane%16, tokens mt*16 + 4*(lane/16) + i
        const int h = nt * 16 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tok = mt * 16 + (lane >> 4) * 4 + i;
            sS[tok][h] = s_row[tok] >= 0 ? acc[i] * scale2 : -INFINITY;
        }
    }
    __syncthreads();

    // 3. softmax per head: 8 lanes per head, 4 tokens each
    {
        const int h = tid >> 3, part = tid & 7;
        float z[4], m = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z[i] = sS[part * 4 + i][h];
            m = fmaxf(m, z[i]);
        }
        m = group_max<8>(m);
        float l = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = (z[i] == -INFINITY) ? 0.f : exp2f(z[i] - m);
            sS[part * 4 + i][h] = p;
            l += p;
        }
        l = group_sum<8>(l);
        if (part == 0) {
            sm[h] = m;
            sl[h] = l;
        }
    }
    __syncthreads();

    // 4. P.V: wave w takes value channels [dv/4 * w, dv/4 * (w+1)) in
    //    16-channel tiles, both head tiles. A = P (head lane%16, tokens
    //    8*(lane/16)..+8), B = V (channel lane%16, same tokens).
    const int NT = dv / 16;            // channel tiles (<= 32)
    bf16x8_t pa_hi[2], pa_lo[2];
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2) {
        const int h = m2 * 16 + (lane & 15);
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float p0 = sS[(lane >> 4) * 8 + 2 * j][h], p1 = sS[(lane >> 4) * 8 + 2 * j + 1][h];
            const uint32_t h0 = f32_bf16_rne(p0), h1 = f32_bf16_rne(p1);
            const uint32_t l0 = f32_bf16_rne(p0 - bf16_f32(h0)), l1 = f32_bf16_rne(p1 - bf16_f32(h1));
            hi[j] = h0 | (h1 << 16);
            lo[j] = l0 | (l1 << 16);
        }
        pa_hi[m2] = as_bf16x8(make_uint4(hi[0], hi[1], hi[2], hi[3]));
        pa_lo[m2] = as_bf16x8(make_uint4(lo[0], lo[1], lo[2], lo[3]));
    }
    const size_t bh0 = (size_t)unit * H;
    for (int n = wave; n < NT; n += 4) {
        // B fragment: 8 tokens of channel n*16 + lane%16
        const int c = n * 16 + (lane & 15);
        uint32_t w4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int t0 = (lane >> 4) * 8 + 2 * j;
            w4[j] = (uint32_t)sK[t0 * RS + c] | ((uint32_t)sK[(t0 + 1) * RS + c] << 16);
        }
        const bf16x8_t vb = as_bf16x8(make_uint4(w4[0], w4[1], w4[2], w4[3]));
#pragma unroll
        for (int m2 = 0; m2 < 2; ++m2) {
            f32x4_t o = {0.f, 0.f, 0.f, 0.f};
            o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_hi[m2], vb, o, 0, 0, 0);
            o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa_lo[m2], vb, o, 0, 0, 0);
            // lane: channel c, heads m2*16 + 4*(lane/16) + i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int h = m2 * 16 + (lane >> 4) * 4 + i;
                part_acc[((bh0 + h) * n_splits + split) * dv + c] = o[i];
            }
        }
    }
    if (tid < H) {
        part_ml[((bh0 + tid) * n_splits + split) * 2 + 0] = sm[tid];
        part_ml[((bh0 + tid) * n_splits + split) * 2 + 1] = sl[tid];
    }
}

// grid: (B*Hq). Merges the split partials of one query head. The (max,
// sum) pairs and the accumulator rows of a chunk of eight splits are all
// loaded before any arithmetic, so a chunk costs one memory round trip.
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ part_ml, const float* __restrict__ part_acc, float* __restrict__ out,
    float* __restrict__ lse, int dv, int n_splits) {
    constexpr int CH = 8;
    const size_t bh = blockIdx.x;
    const float* ml = part_ml + bh * n_splits * 2;
    const float* pa = part_acc + bh * n_splits * dv;
    const int c0 = threadIdx.x, c1 = threadIdx.x + blockDim.x;   // dv <= 2 * blockDim.x
    float M = -INFINITY, L = 0.f, A0 = 0.f, A1 = 0.f;
    for (int s0 = 0; s0 < n_splits; s0 += CH) {
        float2 mlv[CH];
        float a0[CH], a1[CH];
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            const int sj = s0 + j < n_splits ? s0 + j : n_splits - 1;
            mlv[j] = *reinterpret_cast<const float2*>(ml + 2 * sj);
            a0[j] = c0 < dv ? pa[(size_t)sj * dv + c0] : 0.f;
            a1[j] = c1 < dv ? pa[(size_t)sj * dv + c1] : 0.f;
        }
        float Mc = M;
#pragma unroll
        for (int j = 0; j < CH; ++j)
            if (s0 + j < n_splits) Mc = fmaxf(Mc, mlv[j].x);
        if (Mc == -INFINITY) continue;
        const float r = M == -INFINITY ? 0.f : exp2f(M - Mc);   // rescale what is merged so far
        L *= r;
        A0 *= r;
        A1 *= r;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
            if (s0 + j < n_splits && mlv[j].x != -INFINITY) {
                const float wt = exp2f(mlv[j].x - Mc);
                L = fmaf(mlv[j].y, wt, L);
                A0 = fmaf(a0[j], wt, A0);
                A1 = fmaf(a1[j], wt, A1);
            }
        }
        M = Mc;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    if (c0 < dv) out[bh * dv + c0] = A0 * inv;
    if (c1 < dv) out[bh * dv + c1] = A1 * inv;
    if (threadIdx.x == 0) lse[bh] = L > 0.f ? (M + log2f(L)) * LN2 : -INFINITY;
}

template <int D, int G>
hipError_t launch_gqa(const Shape& s, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                      const int32_t* tok_idx, const int32_t* slot_of, int n_slots, float* part_ml,
                      float* part_acc, hipStream_t st) {
    const int ns = attn_splits(s);
    const int units = s.B * s.Hkv;
    hipLaunchKernelGGL((attend_gqa_kernel<D, G>), dim3(((units + 7) / 8) * 8 * ns), dim3(256), 0, st, q, K, V,
                       tok_idx, slot_of, n_slots, part_ml, part_acc, s.Hkv, s.bs, s.kt, s.max_ctx, s.nb_cap, ns,
                       units, s.sm_scale * LOG2E, 2 * s.bs);
    return hipGetLastError();
}

template <int D>
hipError_t launch_gqa_d(const Shape& s, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                        const int32_t* tok_idx, const int32_t* slot_of, int n_slots, float* part_ml,
                        float* part_acc, hipStream_t st) {
    switch (s.G) {
        case 1: return launch_gqa<D, 1>(s, q, K, V, tok_idx, slot_of, n_slots, part_ml, part_acc, st);
        case 2: return launch_gqa<D, 2>(s, q, K, V, tok_idx, slot_of, n_slots, part_ml, part_acc, st);
        case 4: return launch_gqa<D, 4>(s, q, K, V, tok_idx, slot_of, n_slots, part_ml, part_acc, st);
        case 8: return launch_gqa<D, 8>(s, q, K, V, tok_idx, slot_of, n_slots, part_ml, part_acc, st);
        default: return hipErrorInvalidValue;
    }
}

bool mla_shape(const Shape& s) {
    return s.valias && s.G == 32 && s.dk % 32 == 0 && s.dv % 64 == 0 && s.dv <= 512 && s.dv <= s.dk;
}

}  // namespace

hipError_t launch_combine(const Shape& s, const float* part_ml, const float* part_acc, float* out, float* lse,
                          int n_splits, hipStream_t st) {
    hipLaunchKernelGGL(combine_kernel, dim3(s.B * s.Hq), dim3(s.dv < 256 ? 128 : 256), 0, st, part_ml, part_acc,
                       out, lse, s.dv, n_splits);
    return hipGetLastError();
}

bool attend_supported(const Shape& s) {
    if (mla_shape(s)) return true;
    return !s.valias && s.dk == s.dv && (s.dk == 64 || s.dk == 128 || s.dk == 256) &&
           (s.G == 1 || s.G == 2 || s.G == 4 || s.G == 8);
}

hipError_t launch_attend(const Shape& s, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                         const int32_t* tok_idx, const int32_t* slot_of, int n_slots,
                         float* part_ml, float* part_acc, int32_t* arrivals, float* out, float* lse,
                         hipStream_t st) {
    (void)arrivals;
    if (!attend_supported(s)) return hipErrorInvalidValue;
    if (slot_of && !s.valias) V = K + (size_t)s.bs * s.dk;   // value rows follow the key rows in a slot
    const int ns = attn_splits(s);
    hipError_t e = hipSuccess;
    if (mla_shape(s)) {
        const int units = s.B * s.Hkv;
        const dim3 grid(((units + 7) / 8) * 8 * ns);
        if (s.dk <= 576)
            hipLaunchKernelGGL(attend_mla_kernel<576>, grid, dim3(256), 0, st, q, K, tok_idx, slot_of, n_slots,
                               part_ml, part_acc, s.Hkv, s.dk, s.dv, s.bs, s.kt, s.max_ctx, s.nb_cap, ns, units,
                               s.sm_scale * LOG2E, s.bs);
        else
            hipLaunchKernelGGL(attend_mla_kernel<1024>, grid, dim3(256), 0, st, q, K, tok_idx, slot_of, n_slots,
                               part_ml, part_acc, s.Hkv, s.dk, s.dv, s.bs, s.kt, s.max_ctx, s.nb_cap, ns, units,
                               s.sm_scale * LOG2E, s.bs);
        e = hipGetLastError();
    } else {
        switch (s.dk) {
            case 64: e = launch_gqa_d<64>(s, q, K, V, tok_idx, slot_of, n_slots, part_ml, part_acc, st); break;
            case 128: e = launch_gqa_d<128>(s, q, K, V, tok_idx, slot_of, n_slots, part_ml, part_acc, st); break;
            case 256: e = launch_gqa_d<256>(s, q, K, V, tok_idx, slot_of, n_slots, part_ml, part_acc, st); break;
            default: return hipErrorInvalidValue;
        }
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(combine_kernel, dim3(s.B * s.Hq), dim3(s.dv < 256 ? 128 : 256), 0, st, part_ml,
                       part_acc, out, lse, s.dv, ns);
    return hipGetLastError();
}

}  // namespace hsab
