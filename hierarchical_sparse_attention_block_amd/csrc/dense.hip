// Dense decode attention: every query head attends over all n tokens of its
// KV head. This is the full-attention operator the sparse path replaces and
// is measured against (the pages report the sparse operator's speedup over
// full attention: AsyncTLS abstract; gist.science/de explainer section 4;
// gist.science/es explainer section 4).
//
// Flash-decoding layout: one workgroup per (unit, chunk of DENSE_CHUNK
// consecutive tokens); four waves stream the chunk 64 tokens at a time
// (16 per wave, d/8 lanes per token), the next 64 tokens' K and V rows in
// flight while the current ones are used; each lane group keeps an online
// softmax state (running max, sum, weighted values), the groups are merged
// once in LDS, and the split merge kernel combines the chunks.
#include "common.h"
#include "kernels.h"

namespace hsab {

namespace {

template <int D, int G>
__global__ __launch_bounds__(256) void dense_gqa_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const int32_t* __restrict__ ctx_len, float* __restrict__ part_ml, float* __restrict__ part_acc, int Hkv,
    int max_ctx, int n_splits, int units, float scale2) {
    constexpr int LPT = D / 8;        // lanes per token
    constexpr int TPI = 64 / LPT;     // tokens per wave load = lane groups per wave
    constexpr int TPW = 16;           // tokens per wave per round
    constexpr int IT = TPW / TPI;     // tokens per lane group per round
    constexpr int NP = 4 * TPI;       // softmax states per workgroup
    static_assert(IT >= 1 && TPW % TPI == 0, "bad D");
    __shared__ float s_m[NP][G], s_l[NP][G];
    __shared__ float s_acc[NP][G][D];

    const int xcd = blockIdx.x & 7, y = blockIdx.x >> 3;
    const int unit = (y / n_splits) * 8 + xcd, split = y % n_splits;
    if (unit >= units) return;
    const int b = unit / Hkv, g = unit % Hkv;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int cc = lane % LPT, ts = lane / LPT;
    int n = ctx_len[b];
    n = n < 1 ? 1 : (n > max_ctx ? max_ctx : n);
    const int t_begin = split * DENSE_CHUNK;
    const int t_end = t_begin + DENSE_CHUNK < n ? t_begin + DENSE_CHUNK : n;

    float qf[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const uint4 v = ldg16(q + ((size_t)(b * Hkv + g) * G + h) * D + cc * 8);
        widen8(v, qf[h]);
#pragma unroll
        for (int e = 0; e < 8; ++e) qf[h][e] *= scale2;
    }

    const uint16_t* Ku = K + (size_t)unit * max_ctx * D + cc * 8;
    const uint16_t* Vu = V + (size_t)unit * max_ctx * D + cc * 8;
    // token of lane group ts, slot it, in the round starting at t0
    auto tok = [&](int t0, int it) { return t0 + wave * TPW + it * TPI + ts; };
    uint4 kr[IT], vr[IT], kn[IT], vn[IT];
    if (t_begin < t_end) {
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            const int t = tok(t_begin, it);
            const size_t r = (size_t)(t < t_end ? t : t_end - 1);
            kr[it] = ldg16(Ku + r * D);
            vr[it] = ldg16(Vu + r * D);
        }
    }

    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }
    for (int t0 = t_begin; t0 < t_end; t0 += 4 * TPW) {
        const bool more = t0 + 4 * TPW < t_end;
        if (more) {
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                const int t = tok(t0 + 4 * TPW, it);
                const size_t r = (size_t)(t < t_end ? t : t_end - 1);
                kn[it] = ldg16(Ku + r * D);
                vn[it] = ldg16(Vu + r * D);
            }
        }
        float z[IT][G];
#pragma unroll
        for (int it = 0; it < IT; ++it) {
            float kf[8];
            widen8(kr[it], kf);
            const bool ok = tok(t0, it) < t_end;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float p = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) p = fmaf(qf[h][e], kf[e], p);
                p = group_sum<LPT>(p);
                z[it][h] = ok ? p : -INFINITY;
            }
        }
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mr = m[h];
#pragma unroll
            for (int it = 0; it < IT; ++it) mr = fmaxf(mr, z[it][h]);
            if (mr == -INFINITY) continue;   // nothing valid yet for this group
            const float r = m[h] == -INFINITY ? 0.f : exp2f(m[h] - mr);
            l[h] *= r;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] *= r;
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                float vf[8];
                widen8(vr[it], vf);
                const float p = z[it][h] == -INFINITY ? 0.f : exp2f(z[it][h] - mr);
                l[h] += p;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
            }
            m[h] = mr;
        }
        if (more) {
#pragma unroll
            for (int it = 0; it < IT; ++it) {
                kr[it] = kn[it];
                vr[it] = vn[it];
            }
        }
    }

    const int slot = wave * TPI + ts;
#pragma unroll
    for (int h = 0; h < G; ++h) {
        float4* dst = reinterpret_cast<float4*>(&s_acc[slot][h][cc * 8]);
        dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
        dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
        if (cc == 0) {
            s_m[slot][h] = m[h];
            s_l[slot][h] = l[h];
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

// Absorbed latent layout (32 query heads on one latent key, values = its
// first d_v dims): per workgroup a chunk of DENSE_CHUNK tokens in rounds of
// 32. A round's 32 latent rows are staged in LDS beside the unit's query
// rows while the next round's rows are loaded into registers. Wave w owns
// head tile w & 1 and every other 16-channel value tile from w >> 1: it
// computes the logits of its heads and token tile w >> 1 on
// v_mfma_f32_16x16x32_bf16, swaps them through LDS with the wave that has
// the other token tile, and keeps its heads' running max and sum itself, so
// a round has three barriers. The weighted values are accumulated
// transposed, O^T += V^T P^T: the logit accumulators already hold P^T in
// the B-operand layout (tokens permuted alike on both operands), each
// accumulator lane's rescale factor is its own head's, and the V^T operand
// comes from LDS through the gfx950 transposing 16-bit read (within each
// 16-lane group, lane i receives element i % 4 of the 8 bytes that lane
// 4j + i / 4 addressed, j = 0..3). P enters as hi + lo bf16.
template <int DKMAX>
__global__ __launch_bounds__(256, DKMAX <= 576 ? 2 : 1) void dense_mla_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ K, const int32_t* __restrict__ ctx_len,
    float* __restrict__ part_ml, float* __restrict__ part_acc, int Hkv, int dk, int dv, int max_ctx, int n_splits,
    int units, float scale2) {
    constexpr int T = 32;                  // tokens per round
    constexpr int H = 32;                  // query heads per KV head
    constexpr int KSMAX = DKMAX / 32;      // logit steps
    constexpr int RS = DKMAX + 8;          // LDS row stride (elements)
    constexpr int PER = (T * DKMAX / 8 + 255) / 256;
    constexpr int NTW = 16;                // value tiles of 16 channels per wave (d_v <= 512)
    __shared__ __align__(16) uint16_t sK[T * RS];
    __shared__ __align__(16) uint16_t sQ[H * RS];
    __shared__ __align__(16) float sZ[4][64][4];   // logit tile of each wave

    const int xcd = blockIdx.x & 7, y = blockIdx.x >> 3;
    const int unit = (y / n_splits) * 8 + xcd, split = y % n_splits;
    if (unit >= units) return;
    const int b = unit / Hkv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15, nt = wave & 1, half = wave >> 1;
    const int cpr = dk / 8, NT = dv / 16, nchunk = T * cpr;
    int n = ctx_len[b];
    n = n < 1 ? 1 : (n > max_ctx ? max_ctx : n);
    const int t_begin = split * DENSE_CHUNK;
    const int t_end = t_begin + DENSE_CHUNK < n ? t_begin + DENSE_CHUNK : n;

    // query rows (zero past d_k); key columns past d_k stay zero (row
    // stores never touch them)
    for (int c = tid; c < H * (DKMAX / 8); c += 256) {
        const int h = c / (DKMAX / 8), ch = c - h * (DKMAX / 8);
        *reinterpret_cast<uint4*>(&sQ[h * RS + ch * 8]) =
            ch < cpr ? ldg16(q + ((size_t)unit * H + h) * dk + ch * 8) : make_uint4(0u, 0u, 0u, 0u);
        *reinterpret_cast<uint4*>(&sK[h * RS + ch * 8]) = make_uint4(0u, 0u, 0u, 0u);
    }
    // chunk c of a round is 16 bytes at element 8c of the round's rows (row
    // c / cpr in LDS); chunks past the row count repeat the last one and
    // chunks past the end of the context read its last chunk (finite
    // values, masked out of the softmax)
    const uint16_t* Ku = K + (size_t)unit * max_ctx * dk;
    int soff[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        int c = tid + i * 256;
        c = c < nchunk ? c : nchunk - 1;
        const int r = c / cpr;
        soff[i] = r * RS + (c - r * cpr) * 8;
    }
    const size_t lim = (size_t)t_end * dk - 8;
    auto load_rows = [&](int t0, uint4 (&v)[PER]) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int c = tid + i * 256 < nchunk ? tid + i * 256 : nchunk - 1;
            const size_t o = (size_t)t0 * dk + (size_t)c * 8;
            v[i] = ldg16(Ku + (o < lim ? o : lim));
        }
    };
    uint4 v[PER];
    if (t_begin < t_end) load_rows(t_begin, v);

    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t acc[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const uint16_t* ka = &sK[(half * 16 + c16) * RS + g * 8];
    const uint16_t* qa = &sQ[(nt * 16 + c16) * RS + g * 8];
    // transposed-read address: token 4g + c16 / 4, channels 4 (c16 % 4) ..
    const uint16_t* va = &sK[(g * 4 + (c16 >> 2)) * RS + (c16 & 3) * 4];
    for (int t0 = t_begin; t0 < t_end; t0 += T) {
        __syncthreads();   // every wave is done with the previous round's rows
#pragma unroll
        for (int i = 0; i < PER; ++i) *reinterpret_cast<uint4*>(&sK[soff[i]]) = v[i];
        __syncthreads();
        if (t0 + T < t_end) load_rows(t0 + T, v);   // next round in flight

        // this wave's logit tile: tokens half*16 + 4g + i, head nt*16 + c16;
        // the partner wave (same heads) holds the other 16 tokens
        f32x4_t za = {0.f, 0.f, 0.f, 0.f}, zb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < KSMAX; u += 2) {
            za = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(*reinterpret_cast<const uint4*>(ka + u * 32)),
                                                         as_bf16x8(*reinterpret_cast<const uint4*>(qa + u * 32)),
                                                         za, 0, 0, 0);
            if (u + 1 < KSMAX)
                zb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(*reinterpret_cast<const uint4*>(ka + (u + 1) * 32)),
                    as_bf16x8(*reinterpret_cast<const uint4*>(qa + (u + 1) * 32)), zb, 0, 0, 0);
        }
        *reinterpret_cast<f32x4_t*>(sZ[wave][lane]) = za + zb;
        __syncthreads();
        const f32x4_t z0 = *reinterpret_cast<const f32x4_t*>(sZ[nt][lane]);
        const f32x4_t z1 = *reinterpret_cast<const f32x4_t*>(sZ[2 + nt][lane]);

        // online softmax of head nt*16 + c16 over the round's 32 tokens
        float p[8], mc = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = t0 + g * 4 + i < t_end ? z0[i] * scale2 : -INFINITY;
            p[4 + i] = t0 + 16 + g * 4 + i < t_end ? z1[i] * scale2 : -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) mc = fmaxf(mc, p[i]);
        mc = max_xor32(max_xor16(mc));   // finite: the round holds a valid token
        const float mn = fmaxf(m_run, mc);
        const float rs = exp2f(m_run - mn);   // 0 on the first round
        float ls = 0.f;
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float p0 = exp2f(p[2 * k] - mn), p1 = exp2f(p[2 * k + 1] - mn);
            ls += p0 + p1;
            split_bf16x2(p0, p1, hi[k], lo[k]);
        }
        ls = sum_xor32(sum_xor16(ls));
        l_run = l_run * rs + ls;
        m_run = mn;
        const bf16x8_t pb_hi = as_bf16x8(make_uint4(hi[0], hi[1], hi[2], hi[3]));
        const bf16x8_t pb_lo = as_bf16x8(make_uint4(lo[0], lo[1], lo[2], lo[3]));

        // O^T tile (channels nn*16.., heads nt*16..) += V^T P^T; the k index
        // 8g + j stands for token 4g + j (j < 4) or 16 + 4g + j - 4
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
            const int nn = half + 2 * j;
            if (nn < NT) {
                const s16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_s16x4(va + nn * 16));
                const s16x4_t v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_s16x4(va + 16 * RS + nn * 16));
                const uint2 w0 = __builtin_bit_cast(uint2, v0), w1 = __builtin_bit_cast(uint2, v1);
                const bf16x8_t vt = as_bf16x8(make_uint4(w0.x, w0.y, w1.x, w1.y));
                f32x4_t o = acc[j] * rs;
                o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pb_hi, o, 0, 0, 0);
                o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pb_lo, o, 0, 0, 0);
                acc[j] = o;
            }
        }
    }

    // partials: channel nn*16 + 4g + i, head nt*16 + c16
    const size_t bh = (size_t)unit * H + nt * 16 + c16;
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
        const int nn = half + 2 * j;
        if (nn < NT)
            *reinterpret_cast<float4*>(&part_acc[(bh * n_splits + split) * dv + nn * 16 + g * 4]) =
                make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
    }
    if (half == 0 && g == 0) {
        part_ml[(bh * n_splits + split) * 2] = m_run;
        part_ml[(bh * n_splits + split) * 2 + 1] = l_run;
    }
}

struct DenseLayout {
    size_t ml, acc, total;
};

DenseLayout dense_layout(const Shape& s) {
    const size_t ns = (size_t)(s.max_ctx + DENSE_CHUNK - 1) / DENSE_CHUNK;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    DenseLayout L;
    L.ml = 0;
    L.acc = al((size_t)s.B * s.Hq * ns * 2 * sizeof(float));
    L.total = L.acc + al((size_t)s.B * s.Hq * ns * s.dv * sizeof(float));
    return L;
}

template <int D, int G>
hipError_t launch_d(const Shape& s, const uint16_t* q, const uint16_t* K, const uint16_t* V, const int32_t* ctx_len,
                    float* ml, float* acc, int ns, hipStream_t st) {
    const int units = s.B * s.Hkv;
    hipLaunchKernelGGL((dense_gqa_kernel<D, G>), dim3(((units + 7) / 8) * 8 * ns), dim3(256), 0, st, q, K, V,
                       ctx_len, ml, acc, s.Hkv, s.max_ctx, ns, units, s.sm_scale * LOG2E);
    return hipGetLastError();
}

template <int D>
hipError_t launch_dg(const Shape& s, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                     const int32_t* ctx_len, float* ml, float* acc, int ns, hipStream_t st) {
    switch (s.G) {
        case 1: return launch_d<D, 1>(s, q, K, V, ctx_len, ml, acc, ns, st);
        case 2: return launch_d<D, 2>(s, q, K, V, ctx_len, ml, acc, ns, st);
        case 4: return launch_d<D, 4>(s, q, K, V, ctx_len, ml, acc, ns, st);
        case 8: return launch_d<D, 8>(s, q, K, V, ctx_len, ml, acc, ns, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

static bool dense_latent(const Shape& s) {
    return s.valias && s.G == 32 && s.dk % 32 == 0 && s.dv % 64 == 0 && s.dv <= 512 && s.dv <= s.dk;
}

bool dense_supported(const Shape& s) {
    if (dense_latent(s)) return true;
    return !s.valias && s.dk == s.dv && (s.dk == 64 || s.dk == 128 || s.dk == 256) &&
           (s.G == 1 || s.G == 2 || s.G == 4 || s.G == 8);
}

size_t dense_workspace_bytes(const Shape& s) { return dense_layout(s).total; }

hipError_t launch_dense(const Shape& s, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                        const int32_t* ctx_len, float* out, float* lse, void* ws, hipStream_t st) {
    if (!dense_supported(s)) return hipErrorInvalidValue;
    const DenseLayout L = dense_layout(s);
    const int ns = (s.max_ctx + DENSE_CHUNK - 1) / DENSE_CHUNK;
    char* w = static_cast<char*>(ws);
    float* ml = reinterpret_cast<float*>(w + L.ml);
    float* acc = reinterpret_cast<float*>(w + L.acc);
    hipError_t e;
    if (dense_latent(s)) {
        const int units = s.B * s.Hkv;
        const dim3 grid(((units + 7) / 8) * 8 * ns);
        if (s.dk <= 576)
            hipLaunchKernelGGL(dense_mla_kernel<576>, grid, dim3(256), 0, st, q, K, ctx_len, ml, acc, s.Hkv, s.dk,
                               s.dv, s.max_ctx, ns, units, s.sm_scale * LOG2E);
        else
            hipLaunchKernelGGL(dense_mla_kernel<1024>, grid, dim3(256), 0, st, q, K, ctx_len, ml, acc, s.Hkv, s.dk,
                               s.dv, s.max_ctx, ns, units, s.sm_scale * LOG2E);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_combine(s, ml, acc, out, lse, ns, st);
    }
    switch (s.dk) {
        case 64: e = launch_dg<64>(s, q, K, V, ctx_len, ml, acc, ns, st); break;
        case 128: e = launch_dg<128>(s, q, K, V, ctx_len, ml, acc, ns, st); break;
        case 256: e = launch_dg<256>(s, q, K, V, ctx_len, ml, acc, ns, st); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    return launch_combine(s, ml, acc, out, lse, ns, st);
}

}  // namespace hsab
