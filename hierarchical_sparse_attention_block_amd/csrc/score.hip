// Block scoring on the matrix cores.
//
// The Quest-style upper bound of q.k over a block, sum_c max(q_c*Kmax_c,
// q_c*Kmin_c), equals q+ . Kmax + q- . Kmin with q+ = max(q,0) and
// q- = min(q,0). Stacking [Kmax | Kmin] per block (the metadata row) and
// [q+ | q-] per query head turns the bound of every (head, block) pair into
// one dense product, so query heads that share a KV head (GQA groups, MLA)
// score all blocks in a single GEMM (AsyncTLS, gist.science/de explainer
// section 2.A "Optimierung"; gist.science/es explainer section 2.A item 1).
// The block score is the maximum of the bound over the group.
//
// Mapping onto v_mfma_f32_16x16x32_bf16: A = [q+ | q-] (16 head rows per
// tile, padded with zeros), B = metadata rows (16 blocks per tile), K = the
// 2*d_k stacked channels in steps of 32. Lane l supplies block (l % 16) and
// the 8-channel chunk 4*s + l/16 of step s, i.e. one 16-byte load per step;
// the 16 lanes of a chunk read 16 different 64-byte row segments, and four
// consecutive steps cover each row's cache lines fully. A fragments are
// built once per workgroup in LDS. The result tile holds block (l % 16) in
// lane l for head rows 4*(l/16)..+3; a max over valid heads and two lane
// swaps leave the block score in lanes 0..15.
#include "common.h"
#include "kernels.h"

namespace hsab {

namespace {

constexpr int SCORE_WAVES = 4;

template <int MT, int KSMAX>
__global__ __launch_bounds__(256) void block_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ meta,
    const int32_t* __restrict__ ctx_len, float* __restrict__ score,
    int Hkv, int G, int dk, int bs, int max_ctx, int nb_cap, int tiles_per_wave) {
    __shared__ uint4 qa[MT * KSMAX * 64];   // A fragments [mt][step][lane]

    const int unit = blockIdx.y, b = unit / Hkv, g = unit % Hkv;
    int n = ctx_len[b];
    n = n < 1 ? 1 : (n > max_ctx ? max_ctx : n);
    const int nb = (n + bs - 1) / bs;
    const int j_wg = blockIdx.x * (SCORE_WAVES * tiles_per_wave * 16);
    if (j_wg >= nb) return;

    const int KS = dk / 16;        // steps of 32 over 2*dk stacked channels
    const int CH = dk / 8;         // 8-channel chunks in one half
    const uint16_t* qg = q + ((size_t)b * Hkv * G + (size_t)g * G) * dk;
    for (int e = threadIdx.x; e < MT * KS * 64; e += blockDim.x) {
        const int lane = e & 63, s = (e >> 6) % KS, mt = e / (64 * KS);
        const int m = mt * 16 + (lane & 15);
        const int c = s * 4 + (lane >> 4);
        uint4 v = {0u, 0u, 0u, 0u};
        if (m < G) {
            const bool lower = c >= CH;
            const uint4 raw = ldg16(qg + (size_t)m * dk + (lower ? c - CH : c) * 8);
            if (lower) v = {bf16x2_neg(raw.x), bf16x2_neg(raw.y), bf16x2_neg(raw.z), bf16x2_neg(raw.w)};
            else v = {bf16x2_pos(raw.x), bf16x2_pos(raw.y), bf16x2_pos(raw.z), bf16x2_pos(raw.w)};
        }
        qa[(mt * KSMAX + s) * 64 + lane] = v;
    }
    __syncthreads();

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint16_t* Mu = meta + (size_t)unit * nb_cap * 2 * dk;
    float* Su = score + (size_t)unit * nb_cap;
    for (int t = 0; t < tiles_per_wave; ++t) {
        const int j0 = j_wg + (t * SCORE_WAVES + wave) * 16;
        if (j0 >= nb) break;
        const int jl = j0 + (lane & 15);
        const int jc = jl < nb ? jl : nb - 1;          // keep loads inside the unit's blocks
        const uint16_t* row = Mu + (size_t)jc * 2 * dk + (lane >> 4) * 8;
        f32x4_t acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int s0 = 0; s0 < KS; s0 += 8) {
            uint4 bf[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s0 + u < KS) bf[u] = ldg16(row + (s0 + u) * 32);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (s0 + u < KS) {
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            as_bf16x8(qa[(mt * KSMAX + s0 + u) * 64 + lane]), as_bf16x8(bf[u]), acc[mt], 0, 0, 0);
                }
            }
        }
        float v = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (mt * 16 + (lane >> 4) * 4 + i < G) v = fmaxf(v, acc[mt][i]);
        v = fmaxf(v, __shfl_xor(v, 16));
        v = fmaxf(v, __shfl_xor(v, 32));
        if (lane < 16 && jl < nb) Su[jl] = v;
    }
}

template <int MT, int KSMAX>
hipError_t launch_t(const Shape& s, const uint16_t* q, const uint16_t* meta, const int32_t* ctx_len,
                    float* score, hipStream_t st) {
    const int tiles_per_unit = (s.nb_cap + 15) / 16;
    const long total_wave_tiles = (long)tiles_per_unit * s.B * s.Hkv / SCORE_WAVES;
    // aim for ~2048 workgroups (8 per CU) before giving a wave more tiles
    int tpw = (int)((total_wave_tiles + 2047) / 2048);
    tpw = tpw < 1 ? 1 : (tpw > 8 ? 8 : tpw);
    const int per_wg = SCORE_WAVES * tpw * 16;
    dim3 grid((s.nb_cap + per_wg - 1) / per_wg, s.B * s.Hkv);
    hipLaunchKernelGGL((block_score_kernel<MT, KSMAX>), grid, dim3(64 * SCORE_WAVES), 0, st, q, meta,
                       ctx_len, score, s.Hkv, s.G, s.dk, s.bs, s.max_ctx, s.nb_cap, tpw);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_block_score(const Shape& s, const uint16_t* q, const uint16_t* meta,
                              const int32_t* ctx_len, float* score, hipStream_t st) {
    const int ks = s.dk / 16;
    if (s.G <= 16) {
        if (ks <= 8) return launch_t<1, 8>(s, q, meta, ctx_len, score, st);
        if (ks <= 16) return launch_t<1, 16>(s, q, meta, ctx_len, score, st);
        if (ks <= 36) return launch_t<1, 36>(s, q, meta, ctx_len, score, st);
        return launch_t<1, 64>(s, q, meta, ctx_len, score, st);
    }
    if (ks <= 8) return launch_t<2, 8>(s, q, meta, ctx_len, score, st);
    if (ks <= 16) return launch_t<2, 16>(s, q, meta, ctx_len, score, st);
    if (ks <= 36) return launch_t<2, 36>(s, q, meta, ctx_len, score, st);
    return launch_t<2, 64>(s, q, meta, ctx_len, score, st);
}

}  // namespace hsab
