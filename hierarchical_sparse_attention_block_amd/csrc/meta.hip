// Block metadata from a prefilled cache: channelwise key max/min per block
// and the label-channel key copy (the per-step append lives with the block
// scoring kernel). Blocks summarised by key max/min follow the AsyncTLS coarse
// stage (gist.science/de explainer, section 2.A "Stufe 1"); the label copy
// is the compressed key of the fine stage (gist.science/es explainer,
// section 2.A item 2). Both are exact bf16 copies / comparisons; with fp8
// metadata the max and min are then rounded outward to e4m3.
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
    int Hkv, int dk, int bs, int r, int max_ctx, int nb_cap, int meta8, int lab8) {
    const int unit = blockIdx.y, b = unit / Hkv, g = unit % Hkv;
    int n = ctx_len[b];
    n = n < 0 ? 0 : (n > max_ctx ? max_ctx : n);
    const int nb = (n + bs - 1) / bs;
    const int j0 = blockIdx.x * META_BLOCKS_PER_WG;
    if (j0 >= nb) return;
    const uint16_t* Ku = K + (size_t)unit * max_ctx * dk;

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
        uint8_t* M = meta_block(meta, (size_t)unit * nb_cap + j, dk, meta8);
        if (meta8) {
            const uint32_t hx[4] = {mx.x, mx.y, mx.z, mx.w}, hn[4] = {mn.x, mn.y, mn.z, mn.w};
            uint32_t ux[2] = {0u, 0u}, dn[2] = {0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t bx = (hx[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                const uint32_t bn = (hn[e >> 1] >> (16 * (e & 1))) & 0xffffu;
                ux[e >> 2] |= f8_outward(bx, true) << (8 * (e & 3));
                dn[e >> 2] |= f8_outward(bn, false) << (8 * (e & 3));
            }
            *reinterpret_cast<uint2*>(M + c * 8) = make_uint2(ux[0], ux[1]);
            *reinterpret_cast<uint2*>(M + dk + c * 8) = make_uint2(dn[0], dn[1]);
        } else {
            *reinterpret_cast<uint4*>(M + c * 16) = mx;
            *reinterpret_cast<uint4*>(M + 2 * dk + c * 16) = mn;
        }
    }
    const int32_t* lab = label_ch + g * r;
    const size_t lu = (size_t)unit * max_ctx * r;
    const int tb = j0 * bs, te = min((j0 + META_BLOCKS_PER_WG) * bs, n);
    for (int p = threadIdx.x; p < (te - tb) * r; p += blockDim.x) {
        const int t = tb + p / r, c = p % r;
        label_put(klabel, lu + (size_t)t * r + c, Ku[(size_t)t * dk + clamp_ch(lab[c], dk)], lab8);
    }
}

}  // namespace

hipError_t launch_build_meta(const Shape& s, const uint16_t* K, const int32_t* ctx_len,
                             const int32_t* label_ch, uint16_t* meta, uint16_t* klabel,
                             hipStream_t st) {
    dim3 grid((s.nb_cap + META_BLOCKS_PER_WG - 1) / META_BLOCKS_PER_WG, s.B * s.Hkv);
    hipLaunchKernelGGL(build_meta_kernel, grid, dim3(256), 0, st, K, ctx_len, label_ch, meta, klabel,
                       s.Hkv, s.dk, s.bs, s.r, s.max_ctx, s.nb_cap, s.meta8, s.lab8);
    return hipGetLastError();
}

}  // namespace hsab
