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

bool dense_supported(const Shape& s) {
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
