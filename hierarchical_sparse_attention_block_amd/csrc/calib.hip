// Label-channel calibration from sampled activations: the offline step that
// picks the few channels the fine stage scores tokens on (Double Sparsity;
// AsyncTLS, gist.science/de explainer section 2.A "Stufe 2",
// gist.science/es explainer section 2.A item 2). Channel c of KV head g
// weighs sum over samples s and the group's query heads h of
// |q[s][h][c] * k[s][g][c]|; the r heaviest channels (ties to the lower
// channel) form the label set, ascending.
#include "common.h"
#include "kernels.h"

namespace hsab {

namespace {

constexpr int CAL_WAVES = 16;   // waves splitting the samples of a 64-channel chunk

// grid: (Hkv, ceil(d_k / 64)); block CAL_WAVES * 64. Lane l of every wave
// owns channel 64*chunk + l; wave w takes samples w, w + CAL_WAVES, ...;
// the waves' partial sums meet in LDS and are added in wave order, so the
// result does not depend on scheduling.
__global__ __launch_bounds__(CAL_WAVES * 64) void channel_weight_kernel(
    const uint16_t* __restrict__ qs, const uint16_t* __restrict__ ks, float* __restrict__ imp, int n_samples,
    int Hq, int Hkv, int G, int dk) {
    __shared__ float part[CAL_WAVES][64];
    const int g = blockIdx.x, c = blockIdx.y * 64 + (threadIdx.x & 63), w = threadIdx.x >> 6;
    const int cc = c < dk ? c : dk - 1;   // lanes past d_k read a valid channel and drop it
    // each product of two bf16 values is exact in fp32; the group's heads
    // are read four at a time so their loads are in flight together
    float acc = 0.f;
    for (int s = w; s < n_samples; s += CAL_WAVES) {
        const float kv = bf16_f32(ks[((size_t)s * Hkv + g) * dk + cc]);
        const uint16_t* qr = qs + ((size_t)s * Hq + (size_t)g * G) * dk + cc;
        int h = 0;
        for (; h + 4 <= G; h += 4) {
            const float q0 = bf16_f32(qr[(size_t)h * dk]), q1 = bf16_f32(qr[(size_t)(h + 1) * dk]);
            const float q2 = bf16_f32(qr[(size_t)(h + 2) * dk]), q3 = bf16_f32(qr[(size_t)(h + 3) * dk]);
            acc += fabsf(q0 * kv);
            acc += fabsf(q1 * kv);
            acc += fabsf(q2 * kv);
            acc += fabsf(q3 * kv);
        }
        for (; h < G; ++h) acc += fabsf(bf16_f32(qr[(size_t)h * dk]) * kv);
    }
    part[w][threadIdx.x & 63] = acc;
    __syncthreads();
    if (w == 0 && c < dk) {
        float t = 0.f;
#pragma unroll
        for (int i = 0; i < CAL_WAVES; ++i) t += part[i][threadIdx.x];
        imp[(size_t)g * dk + c] = t;
    }
}

// grid: (Hkv); block 256. Rank of channel c = #{c' : w[c'] > w[c], or equal
// with c' < c}; the channels ranked below r are kept and written in channel
// order.
__global__ __launch_bounds__(256) void label_rank_kernel(const float* __restrict__ imp, int32_t* __restrict__ label_ch,
                                                        int dk, int r) {
    __shared__ float s_w[1024];
    __shared__ uint8_t s_keep[1024];
    const int g = blockIdx.x;
    for (int c = threadIdx.x; c < dk; c += blockDim.x) s_w[c] = imp[(size_t)g * dk + c];
    __syncthreads();
    for (int c = threadIdx.x; c < dk; c += blockDim.x) {
        const float v = s_w[c];
        int rank = 0;
        for (int c2 = 0; c2 < dk; ++c2) {
            const float u = s_w[c2];
            rank += (u > v) || (u == v && c2 < c);
        }
        s_keep[c] = rank < r;
    }
    __syncthreads();
    for (int c = threadIdx.x; c < dk; c += blockDim.x) {
        if (!s_keep[c]) continue;
        int pos = 0;
        for (int c2 = 0; c2 < c; ++c2) pos += s_keep[c2];
        label_ch[(size_t)g * r + pos] = c;
    }
}

}  // namespace

hipError_t launch_calibrate(const Shape& s, const uint16_t* q_samples, const uint16_t* k_samples, int n_samples,
                            float* importance, int32_t* label_ch, hipStream_t st) {
    hipLaunchKernelGGL(channel_weight_kernel, dim3(s.Hkv, (s.dk + 63) / 64), dim3(CAL_WAVES * 64), 0, st,
                       q_samples, k_samples, importance, n_samples, s.Hq, s.Hkv, s.G, s.dk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(label_rank_kernel, dim3(s.Hkv), dim3(256), 0, st, importance, label_ch, s.dk, s.r);
    return hipGetLastError();
}

}  // namespace hsab
