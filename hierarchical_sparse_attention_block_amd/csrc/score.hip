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

// Token append of a decode step (optional): the new key/value rows land at
// position n-1, the tail block's max/min widen to include the key (or start
// from it when it opens a new block), and the label row is copied.
struct Append {
    const uint16_t* k_new;    // [B][Hkv][dk], null: no append
    const uint16_t* v_new;    // [B][Hkv][dv]
    uint16_t* K;
    uint16_t* V;              // null when values alias keys
    uint16_t* klabel;
    const int32_t* label_ch;
    int dv, r;
};

template <int MT, int KSMAX>
__global__ __launch_bounds__(256) void block_score_kernel(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ meta,
    const int32_t* __restrict__ ctx_len, float* __restrict__ score,
    int Hkv, int G, int dk, int bs, int max_ctx, int nb_cap, int tiles_per_wave, Append ap) {
    __shared__ uint4 qa[MT * KSMAX * 64];   // A fragments [mt][step][lane]

    const int unit = blockIdx.y, b = unit / Hkv, g = unit % Hkv;
    int n = ctx_len[b];
    n = n < 1 ? 1 : (n > max_ctx ? max_ctx : n);
    const int nb = (n + bs - 1) / bs;
    const int per_wg = SCORE_WAVES * tiles_per_wave * 16;
    const int j_wg = blockIdx.x * per_wg;
    if (j_wg >= nb) return;

    if (ap.k_new && nb - 1 < j_wg + per_wg) {
        // this workgroup owns the tail block: append before scoring it
        const int pos = n - 1, jt = pos / bs;
        const bool first = (pos % bs) == 0;
        const uint16_t* kn = ap.k_new + (size_t)unit * dk;
        uint16_t* Mt = meta + ((size_t)unit * nb_cap + jt) * 2 * dk;
        uint16_t* Krow = ap.K + ((size_t)unit * max_ctx + pos) * dk;
        for (int c = threadIdx.x; c < dk; c += blockDim.x) {
            const uint16_t kb = kn[c];
            Krow[c] = kb;
            if (first) {
                Mt[c] = kb;
                Mt[dk + c] = kb;
            } else {
                const float kf = bf16_f32(kb);
                if (kf > bf16_f32(Mt[c])) Mt[c] = kb;
                if (kf < bf16_f32(Mt[dk + c])) Mt[dk + c] = kb;
            }
        }
        if (ap.V) {
            const uint16_t* vn = ap.v_new + (size_t)unit * ap.dv;
            uint16_t* Vrow = ap.V + ((size_t)unit * max_ctx + pos) * ap.dv;
            for (int c = threadIdx.x; c < ap.dv; c += blockDim.x) Vrow[c] = vn[c];
        }
        uint16_t* Lrow = ap.klabel + ((size_t)unit * max_ctx + pos) * ap.r;
        for (int c = threadIdx.x; c < ap.r; c += blockDim.x)
            Lrow[c] = kn[clamp_ch(ap.label_ch[g * ap.r + c], dk)];
        __syncthreads();   // the tail block's new bounds are read below
    }

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
        if (G > 4) {   // heads 4.. sit in the other 16-lane rows
            v = fmaxf(v, __shfl_xor(v, 16));
            v = fmaxf(v, __shfl_xor(v, 32));
        }
        if (lane < 16 && jl < nb) Su[jl] = v;
    }
}

template <int MT, int KSMAX>
hipError_t launch_t(const Shape& s, const uint16_t* q, uint16_t* meta, const int32_t* ctx_len,
                    float* score, const Append& ap, hipStream_t st) {
    const int tiles_per_unit = (s.nb_cap + 15) / 16;
    const long total_wave_tiles = (long)tiles_per_unit * s.B * s.Hkv / SCORE_WAVES;
    // aim for ~2048 workgroups (8 per CU) before giving a wave more tiles
    int tpw = (int)((total_wave_tiles + 2047) / 2048);
    tpw = tpw < 1 ? 1 : (tpw > 8 ? 8 : tpw);
    const int per_wg = SCORE_WAVES * tpw * 16;
    dim3 grid((s.nb_cap + per_wg - 1) / per_wg, s.B * s.Hkv);
    hipLaunchKernelGGL((block_score_kernel<MT, KSMAX>), grid, dim3(64 * SCORE_WAVES), 0, st, q, meta,
                       ctx_len, score, s.Hkv, s.G, s.dk, s.bs, s.max_ctx, s.nb_cap, tpw, ap);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_block_score(const Shape& s, const uint16_t* q, uint16_t* meta, const int32_t* ctx_len,
                              float* score, const uint16_t* k_new, const uint16_t* v_new, uint16_t* K,
                              uint16_t* V, uint16_t* klabel, const int32_t* label_ch, hipStream_t st) {
    const Append ap{k_new, v_new, K, s.valias ? nullptr : V, klabel, label_ch, s.dv, s.r};
    const int ks = s.dk / 16;
    if (s.G <= 16) {
        if (ks <= 8) return launch_t<1, 8>(s, q, meta, ctx_len, score, ap, st);
        if (ks <= 16) return launch_t<1, 16>(s, q, meta, ctx_len, score, ap, st);
        if (ks <= 36) return launch_t<1, 36>(s, q, meta, ctx_len, score, ap, st);
        return launch_t<1, 64>(s, q, meta, ctx_len, score, ap, st);
    }
    if (ks <= 8) return launch_t<2, 8>(s, q, meta, ctx_len, score, ap, st);
    if (ks <= 16) return launch_t<2, 16>(s, q, meta, ctx_len, score, ap, st);
    if (ks <= 36) return launch_t<2, 36>(s, q, meta, ctx_len, score, ap, st);
    return launch_t<2, 64>(s, q, meta, ctx_len, score, ap, st);
}

}  // namespace hsab
