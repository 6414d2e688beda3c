// Exact attention over the kept tokens (AsyncTLS, gist.science/es
// explainer, section 2.A item 2: the final attention runs on the K_t
// selected tokens only), split over workgroups and merged by log-sum-exp.
//
// GQA path (d_k == d_v == D, G query heads per KV head): one workgroup of
// four waves takes 64 consecutive entries of the unit's token list (128
// for D <= 128 when 64-entry splits would need more workgroups than one
// resident round holds); D/8 lanes share a token (8 channels = 16 bytes
// each), so one wave load gathers 64/(D/8) whole key rows. Logits are
// v_dot2_f32_bf16 sums of the packed bf16 pairs (fp32 accumulation),
// added over the token's lane group and then scaled by sm_scale*log2 e
// (base-2 units). Rows are addressed from the unit's first row by 32-bit
// byte offsets, one register per entry for its key and value loads. With
// 128 entries per workgroup each lane keeps 8 key and 8 value rows in
// flight; at G <= 4 the kernel is held to 128 registers so that four
// workgroups share a CU and one resident round takes the whole grid.
// Each wave keeps (max, sum, weighted values) per head; the workgroup
// merges its four waves and writes one partial per head; the combine
// kernel merges the partials of all splits.
//
// MLA path (values are the first d_v dims of the d_k-dim latent key rows,
// 32 query heads on one KV head): a workgroup takes rounds of 32 kept
// tokens; logits and P.V run on v_mfma_f32_16x16x32_bf16 from key rows and
// queries staged in LDS, with an online softmax across the rounds; the
// rows are loaded non-temporally, as in the GQA path.
//
// Workgroup numbering: the dispatcher hands consecutive workgroups to the
// eight XCDs in turn, so workgroup L runs on XCD L % 8 (measured on MI355X:
// every workgroup of 1-D and 2-D grids of 1,024 to 6,272 workgroups read
// L % 8 from its XCC_ID hardware register). All splits of a unit are given
// the same L % 8, which keeps a unit's rows and partials in one L2. The key
// and value rows are loaded non-temporally: a step reads each one once.
#include "common.h"
#include "kernels.h"

namespace hsab {

namespace {

// MASKED: the token list is the union of the heads' own token sets (per-head
// selection) and tok_mask gives, per entry, the heads that attend it.
// NSC: the split count fixed at compile time (the list then holds exactly
// NSC * TPS entries); 0: from the arguments
template <int D, int G, bool MASKED, int TPS, int NSC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(TPS == 128 && G <= 4 ? 4 : 1)))
void attend_gqa_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const int32_t* __restrict__ tok_idx, const uint32_t* __restrict__ tok_mask,
    const int32_t* __restrict__ ctx_len, const int32_t* __restrict__ slot_of, int n_slots,
    float* __restrict__ part_ml, float* __restrict__ part_acc, int Hkv, int bs, int kt_arg,
    int max_ctx, int nb_cap, int n_splits_arg, int units, float scale2, int slot_rows) {
    const int n_splits = NSC ? NSC : n_splits_arg, kt = NSC ? NSC * TPS : kt_arg;
    constexpr int LPT = D / 8;                         // lanes per token (8 channels each)
    constexpr int TPI = 64 / LPT;                      // tokens per wave load = lane groups per wave
    constexpr int TPW = TPS / 4;                       // tokens per wave
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
    // entries at or past the context length are skipped
    int n = ctx_len[b];
    n = n < 0 ? 0 : (n > max_ctx ? max_ctx : n);

    uint4 qp[G];   // this lane's 8 query channels of each head, bf16 pairs
#pragma unroll
    for (int h = 0; h < G; ++h) qp[h] = ldg16(q + ((size_t)(b * Hkv + g) * G + h) * D + cc * 8);

    // Three dependent rounds, each with all its loads in flight: token
    // positions, block slots (block cache only), then the K and V rows.
    // Loads are unconditional (invalid entries read the unit's row 0 and are masked)
    // so no round waits on a previous one's stragglers.
    uint4 kr[IT], vr[IT];
    bool ok[IT];
    const int32_t* tl = tok_idx + (size_t)unit * kt;
    int tv[IT];
    uint32_t mk[IT];   // heads that attend the entry
    // all heads, as a value the compiler cannot see through: with a
    // constant here the unmasked kernel schedules differently and spills
    // under the 128-register limit (the masked one does not)
    uint32_t all_heads = ~0u;
    asm volatile("" : "+s"(all_heads));
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        const int ti = split * TPS + wave * TPW + it * TPI + ts;
        const int tc = ti < kt ? ti : kt - 1;
        const int t = (int)ldg4_nt(tl + tc);
        tv[it] = ti < kt && t < n ? t : -1;
        mk[it] = MASKED ? tok_mask[(size_t)unit * kt + tc] : all_heads;
    }
    // rows are addressed within the unit (a uniform base and a 32-bit
    // byte offset per lane, one register shared by the key and value loads)
    int rin[IT];   // row of the entry inside the unit's rows, -1: none
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
            rin[it] = v ? sl[it] * slot_rows + (t - blk * bs) : -1;
        }
    } else {
#pragma unroll
        for (int it = 0; it < IT; ++it) rin[it] = tv[it];
    }
    const size_t urows = slot_of ? (size_t)unit * n_slots * slot_rows : (size_t)unit * max_ctx;
    const char* Ku = reinterpret_cast<const char*>(K + urows * D);
    const char* Vu = reinterpret_cast<const char*>(V + urows * D);
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        ok[it] = rin[it] >= 0;
        const uint32_t off = (uint32_t)(ok[it] ? rin[it] : 0) * (uint32_t)(D * 2) + (uint32_t)(cc * 16);
        kr[it] = ldg16_nt(Ku + off);
        vr[it] = ldg16_nt(Vu + off);
    }
    // keep the value loads here, in flight with the key loads; left alone
    // the scheduler sinks them to their use after the logits
    __builtin_amdgcn_sched_barrier(0);

    // logits: 8-channel partial dots, summed over the token's lane group
    float z[IT][G];
#pragma unroll
    for (int it = 0; it < IT; ++it) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const uint4 k = kr[it], qv = qp[h];
            const float p = dot2_bf16(qv.w, k.w, dot2_bf16(qv.z, k.z, dot2_bf16(qv.y, k.y, dot2_bf16(qv.x, k.x, 0.f))));
            const float zl = group_sum<LPT>(p) * scale2;
            z[it][h] = ok[it] && ((mk[it] >> h) & 1u) ? zl : -INFINITY;
        }
    }

    // softmax state of this lane group's IT tokens; the groups of the
    // workgroup are merged once through LDS, no cross-group shuffles
    const int slot = wave * TPI + ts;
    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = z[0][h];
#pragma unroll
        for (int it = 1; it < IT; ++it) m[h] = fmaxf(m[h], z[it][h]);
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }
    // tokens outermost, so each value row is widened once for all heads
    // (heads outermost, the widened rows of every token stay live across
    // the head loop and cost a wave per SIMD at G = 4, 128 entries)
#pragma unroll
    for (int it = 0; it < IT; ++it) {
        float vf[8];
        widen8(vr[it], vf);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            // -inf logits (an absent token, or a head that does not attend
            // it) weigh 0; a finite logit implies a finite head maximum
            const float p = z[it][h] == -INFINITY ? 0.f : exp2f(z[it][h] - m[h]);
            l[h] += p;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
        }
    }
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

// grid: as the GQA kernel; block 256 (4 waves). Hq = 32 * Hkv, d_k % 32 ==
// 0, d_k <= DKMAX, d_v % 64 == 0, d_v <= 512, values alias the first d_v
// key dims (absorbed latent). A split of 32 * rounds consecutive entries of
// the unit's token list (32 per round) is shared by vsplit workgroups, each
// owning a range of value channels (all of them gather the split's rows and
// compute its logits; the splits of a unit share an XCD):
//  * the round's 32 key rows (which hold the values) are staged in LDS; the
//    next round's rows are gathered into registers meanwhile; absent
//    tokens (-1) are zero rows;
//  * wave w owns head tile w & 1 (query fragments in registers): it
//    multiplies token tile w >> 1 of the round by its heads on
//    v_mfma_f32_16x16x32_bf16, swaps that tile
//    through LDS with the wave holding the other token tile, and keeps its
//    heads' running max and sum over the rounds itself;
//  * P.V is accumulated transposed, O^T += V^T P^T, over value tiles
//    w >> 1, w >> 1 + 2, ...: the logit accumulators already hold P^T in
//    the B-operand layout (tokens permuted alike on both operands), each
//    accumulator lane's rescale factor is its own head's, and the V^T
//    operand comes from LDS through the gfx950 transposing 16-bit read
//    (within each 16-lane group, lane i receives element i % 4 of the 8
//    bytes that lane 4j + i / 4 addressed). P enters as two bf16 terms
//    (hi + lo) so the weights keep ~16 mantissa bits; V is exact in bf16.
// DKC, DVC: d_k and d_v fixed at compile time (0: taken from the arguments),
// which turns the row-chunk divisions into multiplications
template <int DKMAX, int DKC, int DVC, int VS>
__global__ __launch_bounds__(256, 1) void attend_mla_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ K, const int32_t* __restrict__ tok_idx,
    const int32_t* __restrict__ ctx_len, const int32_t* __restrict__ slot_of, int n_slots, float* __restrict__ part_ml,
    float* __restrict__ part_acc, int Hkv, int dk_arg, int dv_arg, int bs, int kt, int max_ctx, int nb_cap,
    int n_splits, int units, float scale2, int slot_rows, int rounds_arg, int vsplit_arg) {
    static_assert(DKC == 0 || (DKC <= DKMAX && DKC % 32 == 0), "d_k");
    const int dk = DKC ? DKC : dk_arg, dv = DVC ? DVC : dv_arg;
    // VS: workgroups per split fixed at compile time (0: from the argument);
    // the rounds per split are always MLA_TOK_PER_SPLIT / 32
    const int vsplit = VS ? VS : vsplit_arg;
    constexpr int rounds = MLA_TOK_PER_SPLIT / 32;
    (void)rounds_arg;
    constexpr int T = 32;                  // tokens per round
    constexpr int H = 32;                  // query heads per KV head
    constexpr int KSMAX = DKMAX / 32;      // logit steps
    constexpr int RS = DKMAX + 8;          // LDS row stride (elements): spreads rows over banks
    constexpr int PER = (T * DKMAX / 8 + 255) / 256;
    constexpr int NTW = 16;                // value tiles of 16 channels per wave (d_v <= 512)
    constexpr int RMAX = MLA_TOK_PER_SPLIT / T;
    __shared__ __align__(16) uint16_t sK[T * RS];
    __shared__ __align__(16) float sZ[4][64][4];   // logit tile of each wave
    __shared__ long s_row[RMAX * T];
    __shared__ uint32_t s_vm[RMAX];                // valid-token mask of each round

    const int xcd = blockIdx.x & 7, y = blockIdx.x >> 3;
    const int per_unit = n_splits * vsplit;
    const int unit = (y / per_unit) * 8 + xcd, split = (y % per_unit) / vsplit, vpart = y % vsplit;
    if (unit >= units) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, c16 = lane & 15, nt = wave & 1, half = wave >> 1;
    const int cpr = dk / 8, nchunk = T * cpr;
    const int TS = rounds * T;
    // value tiles [nt_lo, nt_hi) of this workgroup
    const int NTall = dv / 16, nt_lo = vpart * NTall / vsplit, nt_hi = (vpart + 1) * NTall / vsplit;

    // the token list is requested before the query fragments (loads
    // complete in order, so the rows wait for no fragment)
    const int ti = split * TS + tid;
    const int t_raw = (int)ldg4_nt(tok_idx + (size_t)unit * kt + (ti < kt ? ti : kt - 1));   // unconditional load
    int n = ctx_len[unit / Hkv];   // entries at or past the context length are skipped
    n = n < 0 ? 0 : (n > max_ctx ? max_ctx : n);
    const int t = tid < TS && ti < kt && t_raw < n ? t_raw : -1;
    // query fragments of head nt*16 + c16 (B operand, zero past d_k)
    uint4 qb[KSMAX];
    {
        const uint16_t* qr = q + ((size_t)unit * H + nt * 16 + c16) * dk + g * 8;
#pragma unroll
        for (int u = 0; u < KSMAX; ++u) qb[u] = u < dk / 32 ? ldg16(qr + u * 32) : make_uint4(0u, 0u, 0u, 0u);
    }

    // token rows of the split and each round's valid mask
    if (tid < RMAX * T) {
        long row = -1;
        if (tid < TS) {
            if (!slot_of) {
                row = t >= 0 ? (long)unit * max_ctx + t : -1;
            } else if (t >= 0) {
                const int blk = t / bs;
                const int sl_ = blk < nb_cap ? slot_of[(size_t)unit * nb_cap + blk] : -1;
                row = (sl_ >= 0 && sl_ < n_slots) ? ((long)unit * n_slots + sl_) * slot_rows + (t - blk * bs) : -1;
            }
        }
        s_row[tid] = row;
        const uint64_t bal = __ballot(row >= 0);
        if ((tid & 63) == 0) {
            s_vm[tid >> 5] = (uint32_t)bal;
            if ((tid >> 5) + 1 < RMAX) s_vm[(tid >> 5) + 1] = (uint32_t)(bal >> 32);
        }
    }
    // key columns past d_k stay zero (row stores never touch them)
    for (int c = tid; c < T * (DKMAX / 8); c += 256)
        *reinterpret_cast<uint4*>(&sK[(c / (DKMAX / 8)) * RS + (c % (DKMAX / 8)) * 8]) = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();

    // chunk c of a round: 16 bytes at column 8 (c % cpr) of row c / cpr;
    // chunks past the row count repeat the last one
    int soff[PER], rsel[PER], coff[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        int c = tid + i * 256;
        c = c < nchunk ? c : nchunk - 1;
        rsel[i] = c / cpr;
        coff[i] = (c - rsel[i] * cpr) * 8;
        soff[i] = rsel[i] * RS + coff[i];
    }
    auto load_rows = [&](int rd, uint4 (&v)[PER]) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const long row = s_row[rd * T + rsel[i]];
            v[i] = row >= 0 ? ldg16_nt(K + row * dk + coff[i]) : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    uint4 v[PER];
    load_rows(0, v);

    float m_run = -INFINITY, l_run = 0.f;
    f32x4_t acc[NTW];
#pragma unroll
    for (int j = 0; j < NTW; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const uint16_t* ka = &sK[(half * 16 + c16) * RS + g * 8];
    // transposed-read address: token 4g + c16 / 4, channels 4 (c16 % 4) ..
    const uint16_t* va = &sK[(g * 4 + (c16 >> 2)) * RS + (c16 & 3) * 4];
    for (int rd = 0; rd < rounds; ++rd) {
        if (rd > 0) __syncthreads();   // every wave is done with the previous round's rows
#pragma unroll
        for (int i = 0; i < PER; ++i) *reinterpret_cast<uint4*>(&sK[soff[i]]) = v[i];
        __syncthreads();
        if (rd + 1 < rounds) load_rows(rd + 1, v);   // next round in flight
        const uint32_t vm = s_vm[rd];

        // this wave's logit tile: tokens half*16 + 4g + i, head nt*16 + c16
        f32x4_t za = {0.f, 0.f, 0.f, 0.f}, zb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < KSMAX; u += 2) {
            za = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(*reinterpret_cast<const uint4*>(ka + u * 32)),
                                                         as_bf16x8(qb[u]), za, 0, 0, 0);
            if (u + 1 < KSMAX)
                zb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(*reinterpret_cast<const uint4*>(ka + (u + 1) * 32)), as_bf16x8(qb[u + 1]), zb, 0, 0,
                    0);
        }
        *reinterpret_cast<f32x4_t*>(sZ[wave][lane]) = za + zb;
        __syncthreads();
        const f32x4_t z0 = *reinterpret_cast<const f32x4_t*>(sZ[nt][lane]);
        const f32x4_t z1 = *reinterpret_cast<const f32x4_t*>(sZ[2 + nt][lane]);

        // online softmax of head nt*16 + c16 over the round's tokens
        float p[8], mc = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = (vm >> (g * 4 + i)) & 1u ? z0[i] * scale2 : -INFINITY;
            p[4 + i] = (vm >> (16 + g * 4 + i)) & 1u ? z1[i] * scale2 : -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) mc = fmaxf(mc, p[i]);
        mc = max_xor32(max_xor16(mc));
        const float mn = fmaxf(m_run, mc);
        // -inf only while no valid token has been seen: nothing to rescale
        const float rs = m_run == -INFINITY ? 0.f : exp2f(m_run - mn);
        float ls = 0.f;
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float p0 = p[2 * k] == -INFINITY ? 0.f : exp2f(p[2 * k] - mn);
            const float p1 = p[2 * k + 1] == -INFINITY ? 0.f : exp2f(p[2 * k + 1] - mn);
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
            const int nn = nt_lo + half + 2 * j;
            if (nn < nt_hi) {
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
        const int nn = nt_lo + half + 2 * j;
        if (nn < nt_hi)
            *reinterpret_cast<float4*>(&part_acc[(bh * n_splits + split) * dv + nn * 16 + g * 4]) =
                make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
    }
    if (vpart == 0 && half == 0 && g == 0) {
        part_ml[(bh * n_splits + split) * 2] = m_run;
        part_ml[(bh * n_splits + split) * 2 + 1] = l_run;
    }
}

// grid: (B*Hq). Merges the split partials of one query head. The (max,
// sum) pairs and the accumulator rows of a chunk of eight splits are all
// loaded before any arithmetic, so a chunk costs one memory round trip.
// DVC, NSC: d_v and the split count fixed at compile time (0: from the
// arguments)
template <int DVC, int NSC>
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ part_ml, const float* __restrict__ part_acc, float* __restrict__ out,
    float* __restrict__ lse, int dv_arg, int n_splits_arg) {
    const int dv = DVC ? DVC : dv_arg, n_splits = NSC ? NSC : n_splits_arg;
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
            { const uint2 t2 = ldg8_nt(ml + 2 * sj); mlv[j] = make_float2(__uint_as_float(t2.x), __uint_as_float(t2.y)); }
            a0[j] = c0 < dv ? __uint_as_float(ldg4_nt(pa + (size_t)sj * dv + c0)) : 0.f;
            a1[j] = c1 < dv ? __uint_as_float(ldg4_nt(pa + (size_t)sj * dv + c1)) : 0.f;
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

template <int D, int G, int TPS>
hipError_t launch_gqa_tps(const Shape& s, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                          const int32_t* tok_idx, const uint32_t* tok_mask, int list_len, int ns,
                          const int32_t* ctx_len, const int32_t* slot_of, int n_slots, float* part_ml,
                          float* part_acc, hipStream_t st) {
    const int units = s.B * s.Hkv;
    // a unit's rows are addressed by 32-bit byte offsets (always within
    // range under the shape limits: nb_cap <= 8192, d_k <= 256 here)
    const size_t unit_rows = slot_of ? (size_t)n_slots * 2 * s.bs : (size_t)s.max_ctx;
    if (unit_rows * D * 2 > 0xffffffffull) return hipErrorInvalidValue;
    const dim3 grid(((units + 7) / 8) * 8 * ns);
    if (tok_mask)
        hipLaunchKernelGGL((attend_gqa_kernel<D, G, true, TPS, 0>), grid, dim3(256), 0, st, q, K, V, tok_idx, tok_mask,
                           ctx_len, slot_of, n_slots, part_ml, part_acc, s.Hkv, s.bs, list_len, s.max_ctx, s.nb_cap,
                           ns, units, s.sm_scale * LOG2E, 2 * s.bs);
    else if (ns == 8 && list_len == 8 * TPS)   // the 48k and 96k layers: 8 splits
        hipLaunchKernelGGL((attend_gqa_kernel<D, G, false, TPS, 8>), grid, dim3(256), 0, st, q, K, V, tok_idx, tok_mask,
                           ctx_len, slot_of, n_slots, part_ml, part_acc, s.Hkv, s.bs, list_len, s.max_ctx, s.nb_cap,
                           ns, units, s.sm_scale * LOG2E, 2 * s.bs);
    else
        hipLaunchKernelGGL((attend_gqa_kernel<D, G, false, TPS, 0>), grid, dim3(256), 0, st, q, K, V, tok_idx, tok_mask,
                           ctx_len, slot_of, n_slots, part_ml, part_acc, s.Hkv, s.bs, list_len, s.max_ctx, s.nb_cap,
                           ns, units, s.sm_scale * LOG2E, 2 * s.bs);
    return hipGetLastError();
}

template <int D, int G>
hipError_t launch_gqa(const Shape& s, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                      const int32_t* tok_idx, const uint32_t* tok_mask, int list_len, int ns, const int32_t* ctx_len,
                      const int32_t* slot_of, int n_slots, float* part_ml, float* part_acc, hipStream_t st) {
    if constexpr (D <= 128) {
        if (attn_tok_per_split(s) == ATT_TOK_PER_SPLIT_LONG)
            return launch_gqa_tps<D, G, ATT_TOK_PER_SPLIT_LONG>(s, q, K, V, tok_idx, tok_mask, list_len, ns, ctx_len,
                                                                slot_of, n_slots, part_ml, part_acc, st);
    }
    return launch_gqa_tps<D, G, ATT_TOK_PER_SPLIT>(s, q, K, V, tok_idx, tok_mask, list_len, ns, ctx_len, slot_of,
                                                   n_slots, part_ml, part_acc, st);
}

template <int D>
hipError_t launch_gqa_d(const Shape& s, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                        const int32_t* tok_idx, const uint32_t* tok_mask, int list_len, int ns, const int32_t* ctx_len,
                        const int32_t* slot_of, int n_slots, float* part_ml, float* part_acc, hipStream_t st) {
    switch (s.G) {
        case 1: return launch_gqa<D, 1>(s, q, K, V, tok_idx, tok_mask, list_len, ns, ctx_len, slot_of, n_slots, part_ml, part_acc, st);
        case 2: return launch_gqa<D, 2>(s, q, K, V, tok_idx, tok_mask, list_len, ns, ctx_len, slot_of, n_slots, part_ml, part_acc, st);
        case 4: return launch_gqa<D, 4>(s, q, K, V, tok_idx, tok_mask, list_len, ns, ctx_len, slot_of, n_slots, part_ml, part_acc, st);
        case 8: return launch_gqa<D, 8>(s, q, K, V, tok_idx, tok_mask, list_len, ns, ctx_len, slot_of, n_slots, part_ml, part_acc, st);
        default: return hipErrorInvalidValue;
    }
}

bool mla_shape(const Shape& s) {
    return s.valias && s.G == 32 && s.dk % 32 == 0 && s.dv % 64 == 0 && s.dv <= 512 && s.dv <= s.dk;
}

}  // namespace

hipError_t launch_combine(const Shape& s, const float* part_ml, const float* part_acc, float* out, float* lse,
                          int n_splits, hipStream_t st) {
    // the benchmark layers' merges: 8 splits of 128 values, 16 of 512
    if (s.dv == 128 && n_splits == 8) {
        hipLaunchKernelGGL((combine_kernel<128, 8>), dim3(s.B * s.Hq), dim3(128), 0, st, part_ml, part_acc, out, lse,
                           s.dv, n_splits);
        return hipGetLastError();
    }
    if (s.dv == 512 && n_splits == 16) {
        hipLaunchKernelGGL((combine_kernel<512, 16>), dim3(s.B * s.Hq), dim3(256), 0, st, part_ml, part_acc, out, lse,
                           s.dv, n_splits);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((combine_kernel<0, 0>), dim3(s.B * s.Hq), dim3(s.dv < 256 ? 128 : 256), 0, st, part_ml, part_acc,
                       out, lse, s.dv, n_splits);
    return hipGetLastError();
}

bool attend_supported(const Shape& s) {
    if (mla_shape(s)) return s.agg != AGG_HEAD;
    return !s.valias && s.dk == s.dv && (s.dk == 64 || s.dk == 128 || s.dk == 256) &&
           (s.G == 1 || s.G == 2 || s.G == 4 || s.G == 8);
}

hipError_t launch_attend(const Shape& s, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                         const int32_t* tok_idx, const uint32_t* tok_mask, int list_len, const int32_t* ctx_len,
                         const int32_t* slot_of, int n_slots, float* part_ml, float* part_acc, float* out,
                         float* lse, hipStream_t st) {
    if (!attend_supported(s)) return hipErrorInvalidValue;
    if (slot_of && !s.valias) V = K + (size_t)s.bs * s.dk;   // value rows follow the key rows in a slot
    const int tps = mla_shape(s) ? MLA_TOK_PER_SPLIT : attn_tok_per_split(s);
    const int ns = (list_len + tps - 1) / tps;
    hipError_t e = hipSuccess;
    if (mla_shape(s)) {
        const int units = s.B * s.Hkv;
        // value channels are split over two workgroups while the splits
        // alone would leave CUs idle
        const int vs = (long)units * ns < 256 && s.dv >= 128 ? 2 : 1;
        const dim3 grid(((units + 7) / 8) * 8 * ns * vs);
        if (s.dk == 576 && s.dv == 512 && vs == 2)   // the 512 + 64 latent layout
            hipLaunchKernelGGL((attend_mla_kernel<576, 576, 512, 2>), grid, dim3(256), 0, st, q, K, tok_idx, ctx_len,
                               slot_of, n_slots, part_ml, part_acc, s.Hkv, s.dk, s.dv, s.bs, s.kt, s.max_ctx, s.nb_cap,
                               ns, units, s.sm_scale * LOG2E, s.bs, MLA_TOK_PER_SPLIT / 32, vs);
        else if (s.dk == 576 && s.dv == 512)
            hipLaunchKernelGGL((attend_mla_kernel<576, 576, 512, 0>), grid, dim3(256), 0, st, q, K, tok_idx, ctx_len,
                               slot_of, n_slots, part_ml, part_acc, s.Hkv, s.dk, s.dv, s.bs, s.kt, s.max_ctx, s.nb_cap,
                               ns, units, s.sm_scale * LOG2E, s.bs, MLA_TOK_PER_SPLIT / 32, vs);
        else if (s.dk <= 576)
            hipLaunchKernelGGL((attend_mla_kernel<576, 0, 0, 0>), grid, dim3(256), 0, st, q, K, tok_idx, ctx_len, slot_of, n_slots,
                               part_ml, part_acc, s.Hkv, s.dk, s.dv, s.bs, s.kt, s.max_ctx, s.nb_cap, ns, units,
                               s.sm_scale * LOG2E, s.bs, MLA_TOK_PER_SPLIT / 32, vs);
        else
            hipLaunchKernelGGL((attend_mla_kernel<1024, 0, 0, 0>), grid, dim3(256), 0, st, q, K, tok_idx, ctx_len, slot_of, n_slots,
                               part_ml, part_acc, s.Hkv, s.dk, s.dv, s.bs, s.kt, s.max_ctx, s.nb_cap, ns, units,
                               s.sm_scale * LOG2E, s.bs, MLA_TOK_PER_SPLIT / 32, vs);
        e = hipGetLastError();
    } else {
        switch (s.dk) {
            case 64: e = launch_gqa_d<64>(s, q, K, V, tok_idx, tok_mask, list_len, ns, ctx_len, slot_of, n_slots, part_ml, part_acc, st); break;
            case 128: e = launch_gqa_d<128>(s, q, K, V, tok_idx, tok_mask, list_len, ns, ctx_len, slot_of, n_slots, part_ml, part_acc, st); break;
            case 256: e = launch_gqa_d<256>(s, q, K, V, tok_idx, tok_mask, list_len, ns, ctx_len, slot_of, n_slots, part_ml, part_acc, st); break;
            default: return hipErrorInvalidValue;
        }
    }
    if (e != hipSuccess) return e;
    return launch_combine(s, part_ml, part_acc, out, lse, ns, st);
}

}  // namespace hsab
