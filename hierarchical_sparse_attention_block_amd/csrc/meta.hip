// Block metadata: channelwise key max/min per block and the label-channel
// key copy. Blocks summarised by key max/min follow the AsyncTLS coarse
// stage (gist.science/de explainer, section 2.A "Stufe 1"); the label copy
// is the compressed key of the fine stage (gist.science/es explainer,
// section 2.A item 2). Both are exact bf16 copies / comparisons.
#include "common.h"
#include "kernels.h"

namespace hsab {

namespace {

constexpr int META_BLOCKS_PER_WG = 16;

__device__ __forceinline__ uint32_t bmax2(uint32_t a, uint32_t b) {
    float lo = fmaxf(lo_f32(a), lo_f32(b)), hi = fmaxf(hi_f32(a), hi_f32(b));
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}
__device__ __forceinline__ uint32_t bmin2(uint32_t a, uint32_t b) {
    float lo = fminf(lo_f32(a), lo_f32(b)), hi = fminf(hi_f32(a), hi_f32(b));
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}
__device__ __forceinline__ uint4 vmax(uint4 a, uint4 b) { return {bmax2(a.x, b.x), bmax2(a.y, b.y), bmax2(a.z, b.z), bmax2(a.w, b.w)}; }
__device__ __forceinline__ uint4 vmin(uint4 a, uint4 b) { return {bmin2(a.x, b.x), bmin2(a.y, b.y), bmin2(a.z, b.z), bmin2(a.w, b.w)}; }

// grid: (ceil(nb_cap / 16), units). Each workgroup summarises 16 blocks.
__global__ __launch_bounds__(256) void build_meta_kernel(
    const uint16_t* __restrict__ K, const int32_t* __restrict__ ctx_len,
    const int32_t* __restrict__ label_ch, uint16_t* __restrict__ meta, uint16_t* __restrict__ klabel,
    int Hkv, int dk, int bs, int r, int max_ctx, int nb_cap) {
    const int unit = blockIdx.y, b = unit / Hkv, g = unit % Hkv;
    int n = ctx_len[b];
    n = n < 0 ? 0 : (n > max_ctx ? max_ctx : n);
    const int nb = (n + bs - 1) / bs;
    const int j0 = blockIdx.x * META_BLOCKS_PER_WG;
    if (j0 >= nb) return;
    const uint16_t* Ku = K + (size_t)unit * max_ctx * dk;
    uint16_t* Mu = meta + (size_t)unit * nb_cap * 2 * dk;

    const int cpb = dk / 8;   // 16-byte chunks per key row
    for (int p = threadIdx.x; p < META_BLOCKS_PER_WG * cpb; p += blockDim.x) {
        const int j = j0 + p / cpb, c = p % cpb;
        if (j >= nb) continue;
        const int t0 = j * bs, t1 = min(t0 + bs, n);
        uint4 mx = ldg16(Ku + (size_t)t0 * dk + c * 8), mn = mx;
        for (int t = t0 + 1; t < t1; ++t) {
            uint4 v = ldg16(Ku + (size_t)t * dk + c * 8);
            mx = vmax(mx, v);
            mn = vmin(mn, v);
        }
        *reinterpret_cast<uint4*>(Mu + (size_t)j * 2 * dk + c * 8) = mx;
        *reinterpret_cast<uint4*>(Mu + (size_t)j * 2 * dk + dk + c * 8) = mn;
    }
    const int32_t* lab = label_ch + g * r;
    uint16_t* Lu = klabel + (size_t)unit * max_ctx * r;
    const int tb = j0 * bs, te = min((j0 + META_BLOCKS_PER_WG) * bs, n);
    for (int p = threadIdx.x; p < (te - tb) * r; p += blockDim.x) {
        const int t = tb + p / r, c = p % r;
        Lu[(size_t)t * r + c] = Ku[(size_t)t * dk + clamp_ch(lab[c], dk)];
    }
}

// grid: (B). Appends the token at position ctx_len[b]-1 of every KV head.
__global__ __launch_bounds__(256) void append_kernel(
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    uint16_t* __restrict__ K, uint16_t* __restrict__ V, uint16_t* __restrict__ meta,
    uint16_t* __restrict__ klabel, const int32_t* __restrict__ label_ch,
    const int32_t* __restrict__ ctx_len, int Hkv, int dk, int dv, int valias, int bs, int r,
    int max_ctx, int nb_cap) {
    const int b = blockIdx.x;
    const int pos = ctx_len[b] - 1;
    if (pos < 0 || pos >= max_ctx) return;
    const int j = pos / bs;
    const bool first = (pos % bs) == 0;
    for (int g = 0; g < Hkv; ++g) {
        const int unit = b * Hkv + g;
        const uint16_t* kn = k_new + (size_t)unit * dk;
        uint16_t* Krow = K + ((size_t)unit * max_ctx + pos) * dk;
        uint16_t* M = meta + ((size_t)unit * nb_cap + j) * 2 * dk;
        for (int c = threadIdx.x; c < dk; c += blockDim.x) {
            const uint16_t kb = kn[c];
            Krow[c] = kb;
            if (first) {
                M[c] = kb;
                M[dk + c] = kb;
            } else {
                const float kf = bf16_f32(kb);
                if (kf > bf16_f32(M[c])) M[c] = kb;
                if (kf < bf16_f32(M[dk + c])) M[dk + c] = kb;
            }
        }
        if (!valias) {
            const uint16_t* vn = v_new + (size_t)unit * dv;
            uint16_t* Vrow = V + ((size_t)unit * max_ctx + pos) * dv;
            for (int c = threadIdx.x; c < dv; c += blockDim.x) Vrow[c] = vn[c];
        }
        uint16_t* Lrow = klabel + ((size_t)unit * max_ctx + pos) * r;
        for (int c = threadIdx.x; c < r; c += blockDim.x) Lrow[c] = kn[clamp_ch(label_ch[g * r + c], dk)];
    }
}

}  // namespace

hipError_t launch_build_meta(const Shape& s, const uint16_t* K, const int32_t* ctx_len,
                             const int32_t* label_ch, uint16_t* meta, uint16_t* klabel,
                             hipStream_t st) {
    dim3 grid((s.nb_cap + META_BLOCKS_PER_WG - 1) / META_BLOCKS_PER_WG, s.B * s.Hkv);
    hipLaunchKernelGGL(build_meta_kernel, grid, dim3(256), 0, st, K, ctx_len, label_ch, meta, klabel,
                       s.Hkv, s.dk, s.bs, s.r, s.max_ctx, s.nb_cap);
    return hipGetLastError();
}

hipError_t launch_append(const Shape& s, const uint16_t* k_new, const uint16_t* v_new,
                         uint16_t* K, uint16_t* V, uint16_t* meta, uint16_t* klabel,
                         const int32_t* label_ch, const int32_t* ctx_len, hipStream_t st) {
    hipLaunchKernelGGL(append_kernel, dim3(s.B), dim3(256), 0, st, k_new, v_new, K, V, meta, klabel,
                       label_ch, ctx_len, s.Hkv, s.dk, s.dv, s.valias, s.bs, s.r, s.max_ctx, s.nb_cap);
    return hipGetLastError();
}

}  // namespace hsab
