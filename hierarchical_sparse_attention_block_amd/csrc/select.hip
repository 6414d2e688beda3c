// Selection stages of one unit (batch b, KV head g) in one workgroup:
//   * top-K_b over the block scores (coarse stage; AsyncTLS,
//     gist.science/es explainer, section 2.A item 1);
//   * label-channel scores of every valid token of the kept blocks, then
//     top-K_t (fine stage, Double-Sparsity style; gist.science/de explainer
//     section 2.A "Stufe 2", gist.science/es section 2.A item 2).
// With per-head selection every query head is a selection of its own (a
// group of one head: its own block scores, label scores and lists), run by
// its own workgroups; the label rows are still those of its KV head.
// Label score of token t: max over the group's query heads of
// sum_c q_h[label_ch[c]] * klabel[t][c] on the matrix cores with 16
// candidate tokens per tile and the group's label-channel queries as A.
// With 16 label channels a step is v_mfma_f32_16x16x16_bf16 (lane l: token
// l % 16, channels 4*(l/16)..+3, an 8-byte load); with 32 or more it is
// v_mfma_f32_16x16x32_bf16 (channels 32*s + 8*(l/16)..+7, a 16-byte load),
// which halves the load round trips of long label rows. Each wave issues
// eight label-row loads before its MFMAs. Selection keeps all scores in
// registers and LDS (TopK in topk.h).
//
// Split token stage: the label-row gather of one unit is bound by how many
// misses one CU keeps in flight, so with few units each unit gets `parts`
// workgroups (on one XCD). Every part selects the blocks itself (part 0
// writes them), scores its share of the candidate tiles and publishes the
// keys with agent-scope stores; after its stores have completed, each part
// bumps the unit's arrival counter, and the part that arrives last reads
// all keys back (agent-scope loads), runs top-K_t and resets the counter.
#include <type_traits>
#include "common.h"
#include "kernels.h"
#include "topk.h"

namespace hsab {

namespace {

constexpr int SEL_WAVES = 16;
constexpr int SEL_THREADS = SEL_WAVES * 64;

// KK: channels per matrix step (16, or 32 when r >= 32); L8: label rows in
// e4m3 bytes (half the bytes per load), widened exactly to bf16 at the
// matrix step so the loads stay back to back
template <int PT, int KK, bool L8>
__global__ __launch_bounds__(SEL_THREADS) void select_kernel(
    int mode, const uint16_t* __restrict__ q, const float* __restrict__ blk_score,
    const uint16_t* __restrict__ klabel, const int32_t* __restrict__ label_ch,
    const int32_t* __restrict__ ctx_len, int32_t* __restrict__ blk_idx, int32_t* __restrict__ tok_idx,
    float* __restrict__ tok_score, uint32_t* __restrict__ gkeys, int32_t* __restrict__ cnt,
    int32_t* __restrict__ blk_copy, int parts,
    int units, int heads, int Hkv, int G, int dk, int bs, int r, int kb, int kt, int max_ctx, int nb_cap,
    int bs_shift, int agg_sum, int sink, int local) {
    using Sel = TopK<SEL_WAVES, PT>;
    // candidate i sits in slot i / bs of the block list (a shift when bs is a power of two)
    auto slot_of = [&](int i) { return bs_shift >= 0 ? (i >> bs_shift) : i / bs; };
    __shared__ uint32_t s_key[MAX_CAND];
    __shared__ int32_t s_blk[MAX_KB];
    // A fragments [head tile][step][lane]: uint2 per lane for KK = 16,
    // uint4 for KK = 32 (same bytes)
    __shared__ uint4 s_qa4[2 * (MAX_R / 32) * 64];
    uint2* s_qa = reinterpret_cast<uint2*>(s_qa4);
    __shared__ typename Sel::Smem s_sel;
    __shared__ int s_last;

    // selection sel (of `units`) belongs to KV unit sel / heads and, with
    // per-head selection (heads == G), to query head sel % heads of it; the
    // parts of a selection share an XCD (workgroup L runs on XCD L % 8)
    const int xcd = blockIdx.x & 7, y = blockIdx.x >> 3;
    const int sel = (y / parts) * 8 + xcd, part = y % parts;
    if (sel >= units) return;
    const int unit = sel / heads, hsel = sel - unit * heads;
    const int b = unit / Hkv, g = unit % Hkv;
    const int Ge = heads > 1 ? 1 : G;   // query heads scored together
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    // block scores are loaded over the whole capacity in the same round trip
    // as ctx_len and masked once n is known; the entry layout of the block
    // selection uses the capacity's slot count
    const int pt_b = (nb_cap + SEL_THREADS - 1) / SEL_THREADS;
    float sraw[PT];
    if (mode & 1) {
        const float* S = blk_score + (size_t)sel * nb_cap;
#pragma unroll
        for (int j = 0; j < PT; ++j) {
            const int i = (w * pt_b + j) * 64 + lane;
            sraw[j] = (j < pt_b && i < nb_cap) ? S[i] : 0.f;
        }
    }
    int n = ctx_len[b];
    n = n < 1 ? 1 : (n > max_ctx ? max_ctx : n);
    const int nb = (n + bs - 1) / bs;
    const uint16_t* qg = q + ((size_t)unit * G + hsel) * dk;

    // label-channel A fragments (independent of the block selection)
    const int MT = (Ge + 15) / 16;
    const int KSr = r / KK;               // matrix steps per label row
    constexpr int CPL = KK / 4;           // channels per lane per step
    constexpr int SMAX = MAX_R / KK;      // step stride of the fragment table
    if (mode & 2) {
        const int32_t* lab = label_ch + g * r;
        for (int e = threadIdx.x; e < MT * KSr * 64; e += SEL_THREADS) {
            const int l = e & 63, s = (e >> 6) % KSr, mt = e / (64 * KSr);
            const int m = mt * 16 + (l & 15);
            const int c0 = s * KK + (l >> 4) * CPL;
            uint32_t x[CPL / 2];
#pragma unroll
            for (int j = 0; j < CPL / 2; ++j) x[j] = 0u;
            if (m < Ge) {
                const uint16_t* qh = qg + (size_t)m * dk;
#pragma unroll
                for (int j = 0; j < CPL / 2; ++j)
                    x[j] = (uint32_t)qh[clamp_ch(lab[c0 + 2 * j], dk)] |
                           ((uint32_t)qh[clamp_ch(lab[c0 + 2 * j + 1], dk)] << 16);
            }
            if constexpr (KK == 32)
                s_qa4[(mt * SMAX + s) * 64 + l] = make_uint4(x[0], x[1], x[2], x[3]);
            else
                s_qa[(mt * SMAX + s) * 64 + l] = make_uint2(x[0], x[1]);
        }
    }

    // ------------------------------------------------------------ blocks
    if (mode & 1) {
        // forced blocks [0, s1) and [l0, nb) stay out of the ranking; the
        // list is [0, s1), the top kb - forced of the rest, [l0, nb)
        const int s1 = sink < nb ? sink : nb;
        const int l0 = nb - local > s1 ? nb - local : s1;
        const int nforced = s1 + (nb - l0);
        uint32_t bkey[PT];
#pragma unroll
        for (int j = 0; j < PT; ++j) {
            const int i = (w * pt_b + j) * 64 + lane;
            bkey[j] = (j < pt_b && i < nb && i >= s1 && i < l0) ? f32_key(sraw[j]) : 0u;
        }
        int32_t* bo = blk_idx + (size_t)sel * kb;
        int32_t* bc = blk_copy ? blk_copy + (size_t)sel * kb : nullptr;   // second copy of the list (nullable)
        const int keff = Sel::select(bkey, pt_b, kb - nforced, s_sel, [&](int pos, int i) {
            s_blk[s1 + pos] = i;
            if (part == 0) {
                bo[s1 + pos] = i;
                if (bc) bc[s1 + pos] = i;
            }
        });
        for (int p = threadIdx.x; p < nforced; p += SEL_THREADS) {
            const int at = p < s1 ? p : keff + p, blk = p < s1 ? p : l0 + (p - s1);
            s_blk[at] = blk;
            if (part == 0) {
                bo[at] = blk;
                if (bc) bc[at] = blk;
            }
        }
        for (int p = nforced + keff + threadIdx.x; p < kb; p += SEL_THREADS) {
            s_blk[p] = -1;
            if (part == 0) {
                bo[p] = -1;
                if (bc) bc[p] = -1;
            }
        }
    } else {
        for (int p = threadIdx.x; p < kb; p += SEL_THREADS) s_blk[p] = blk_idx[(size_t)sel * kb + p];
    }
    if (!(mode & 2)) return;
    __syncthreads();   // s_blk, s_qa and the selector's scratch settled

    // -------------------------------------------------- token label scores
    const int ncand = kb * bs;
    const size_t lu = (size_t)unit * max_ctx * r;   // first label entry of the unit
    float* TS = tok_score ? tok_score + (size_t)sel * ncand : nullptr;
    const int n_tiles = (ncand + 15) / 16;
    const int t_lo = part * n_tiles / parts, t_hi = (part + 1) * n_tiles / parts;   // this part's tiles
    // eight label loads in flight per lane: load u feeds step u % KSr of
    // tile u / KSr of the batch (KSr is a power of two <= 8)
    const int lg = KSr == 1 ? 0 : KSr == 2 ? 1 : KSr == 4 ? 2 : 3;
    const int tb = 8 >> lg;                         // tiles per batch
    using Frag = typename std::conditional<KK == 32, uint4, uint2>::type;
    using Raw = typename std::conditional<L8, typename std::conditional<KK == 32, uint2, uint32_t>::type, Frag>::type;
    for (int t0 = t_lo + w; t0 < t_hi; t0 += SEL_WAVES * tb) {
        Raw bf[8];
        uint32_t vmask = 0;   // bit u: the token this lane loads for load u is valid
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int tile = t0 + (u >> lg) * SEL_WAVES, st = u & (KSr - 1);
            const int i = tile * 16 + (lane & 15);
            const int slot = slot_of(i), off = i - slot * bs;
            const int blk = (tile < t_hi && i < ncand) ? s_blk[slot] : -1;
            const int pos = blk * bs + off;
            const bool valid = blk >= 0 && blk < nb && pos < n;
            vmask |= (valid ? 1u : 0u) << u;
            const size_t e = lu + (size_t)(valid ? pos : 0) * r + (lane >> 4) * CPL + st * KK;
            if constexpr (L8) {
                const uint8_t* src = reinterpret_cast<const uint8_t*>(klabel) + e;
                if constexpr (KK == 32)
                    bf[u] = ldg8(src);
                else
                    bf[u] = ldg4(src);
            } else {
                if constexpr (KK == 32)
                    bf[u] = ldg16(klabel + e);
                else
                    bf[u] = ldg8(klabel + e);
            }
        }
        f32x4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int tile = t0 + (u >> lg) * SEL_WAVES, st = u & (KSr - 1);
            if (st == 0) acc0 = acc1 = f32x4_t{0.f, 0.f, 0.f, 0.f};
            Frag fr;
            if constexpr (!L8)
                fr = bf[u];
            else if constexpr (KK == 32)
                fr = f8x8_bf16(bf[u]);
            else
                fr = f8x4_bf16(bf[u]);
            if constexpr (KK == 32) {
                const bf16x8_t bfrag = as_bf16x8(fr);
                acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(s_qa4[st * 64 + lane]), bfrag, acc0, 0, 0, 0);
                if (MT > 1)
                    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(s_qa4[(SMAX + st) * 64 + lane]), bfrag,
                                                                   acc1, 0, 0, 0);
            } else {
                const i16x4_t bfrag = as_i16x4(fr);
                acc0 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_i16x4(s_qa[st * 64 + lane]), bfrag, acc0, 0, 0, 0);
                if (MT > 1)
                    acc1 = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_i16x4(s_qa[(SMAX + st) * 64 + lane]), bfrag,
                                                                     acc1, 0, 0, 0);
            }
            if (st == KSr - 1 && tile < t_hi) {
                float v = agg_sum ? 0.f : -INFINITY;   // group max (or sum) of the label scores
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int h = (lane >> 4) * 4 + e;
                    if (h < Ge) v = agg_sum ? v + acc0[e] : fmaxf(v, acc0[e]);
                    if (16 + h < Ge) v = agg_sum ? v + acc1[e] : fmaxf(v, acc1[e]);
                }
                if (Ge > 4) {   // heads 4.. sit in the other 16-lane rows
                    v = agg_sum ? sum_xor32(sum_xor16(v)) : max_xor32(max_xor16(v));
                }
                const int i = tile * 16 + (lane & 15);
                if (lane < 16 && i < ncand) {
                    const bool valid = (vmask >> u) & 1u;
                    const uint32_t kv = valid ? f32_key(v) : 0u;
                    if (parts > 1)
                        __hip_atomic_store(&gkeys[(size_t)sel * ncand + i], kv, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                    else
                        s_key[i] = kv;
                    if (TS) TS[i] = valid ? v : -INFINITY;
                }
            }
        }
    }
    if (parts > 1) {
        // this part's key stores are complete before the arrival is counted
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
        __syncthreads();
        if (threadIdx.x == 0)
            s_last = __hip_atomic_fetch_add(&cnt[sel], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == parts - 1;
        __syncthreads();
        if (!s_last) return;
    } else {
        __syncthreads();
    }

    // ----------------------------------------------------------- top-K_t
    const int pt = (ncand + SEL_THREADS - 1) / SEL_THREADS;
    uint32_t key[PT];
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        const int i = (w * pt + j) * 64 + lane;
        const bool in = j < pt && i < ncand;
        if (parts > 1)
            key[j] = in ? __hip_atomic_load(&gkeys[(size_t)sel * ncand + i], __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT)
                        : 0u;
        else
            key[j] = in ? s_key[i] : 0u;
    }
    int32_t* to = tok_idx + (size_t)sel * kt;
    const int keff_t = Sel::select(key, pt, kt, s_sel, [&](int p, int i) {
        const int slot = slot_of(i);
        to[p] = s_blk[slot] * bs + (i - slot * bs);
    });
    for (int p = keff_t + threadIdx.x; p < kt; p += SEL_THREADS) to[p] = -1;
    if (parts > 1 && threadIdx.x == 0)   // ready for the next call
        __hip_atomic_store(&cnt[sel], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int PT, int KK, bool L8>
hipError_t launch_k(const Shape& s, dim3 grid, int mode, const uint16_t* q, const float* blk_score,
                    const uint16_t* klabel, const int32_t* label_ch, const int32_t* ctx_len, int32_t* blk_idx,
                    int32_t* tok_idx, float* tok_score, uint32_t* gkeys, int32_t* cnt, int32_t* blk_copy, int parts,
                    int units, int shift, hipStream_t st) {
    hipLaunchKernelGGL((select_kernel<PT, KK, L8>), grid, dim3(SEL_THREADS), 0, st, mode, q, blk_score, klabel,
                       label_ch, ctx_len, blk_idx, tok_idx, tok_score, gkeys, cnt, blk_copy, parts, units, s.heads, s.Hkv, s.G,
                       s.dk, s.bs, s.r, s.kb, s.kt, s.max_ctx, s.nb_cap, shift, s.agg_sum, s.sink, s.local);
    return hipGetLastError();
}

template <int PT>
hipError_t launch_t(const Shape& s, int mode, const uint16_t* q, const float* blk_score,
                    const uint16_t* klabel, const int32_t* label_ch, const int32_t* ctx_len,
                    int32_t* blk_idx, int32_t* tok_idx, float* tok_score, uint32_t* gkeys, int32_t* cnt,
                    int32_t* blk_copy, hipStream_t st) {
    const int shift = (s.bs & (s.bs - 1)) ? -1 : __builtin_ctz(s.bs);
    const int units = s.B * s.Hkv * s.heads;   // selections
    // parts per selection: enough workgroups to cover the CUs, at least eight
    // candidate tiles (half a tile per wave) each
    int parts = 1;
    if ((mode & 2) && gkeys && cnt) {
        const int n_tiles = (s.kb * s.bs + 15) / 16;
        while (parts < 32 && (long)parts * 2 * units <= 256 && parts * 2 * 8 <= n_tiles) parts *= 2;
    }
    const dim3 grid(((units + 7) / 8) * 8 * parts);
    if (s.r >= 32)
        return s.lab8 ? launch_k<PT, 32, true>(s, grid, mode, q, blk_score, klabel, label_ch, ctx_len, blk_idx, tok_idx,
                                               tok_score, gkeys, cnt, blk_copy, parts, units, shift, st)
                      : launch_k<PT, 32, false>(s, grid, mode, q, blk_score, klabel, label_ch, ctx_len, blk_idx,
                                                tok_idx, tok_score, gkeys, cnt, blk_copy, parts, units, shift, st);
    return s.lab8 ? launch_k<PT, 16, true>(s, grid, mode, q, blk_score, klabel, label_ch, ctx_len, blk_idx, tok_idx,
                                           tok_score, gkeys, cnt, blk_copy, parts, units, shift, st)
                  : launch_k<PT, 16, false>(s, grid, mode, q, blk_score, klabel, label_ch, ctx_len, blk_idx, tok_idx,
                                            tok_score, gkeys, cnt, blk_copy, parts, units, shift, st);
}

}  // namespace

hipError_t launch_select(const Shape& s, int mode, const uint16_t* q, const float* blk_score,
                         const uint16_t* klabel, const int32_t* label_ch, const int32_t* ctx_len,
                         int32_t* blk_idx, int32_t* tok_idx, float* tok_score, uint32_t* sel_keys,
                         int32_t* sel_cnt, hipStream_t st, int32_t* blk_copy) {
    int need = 1;
    if (mode & 1) need = (s.nb_cap + SEL_THREADS - 1) / SEL_THREADS;
    if (mode & 2) {
        const int t = (s.kb * s.bs + SEL_THREADS - 1) / SEL_THREADS;
        need = t > need ? t : need;
    }
    if (need <= 1) return launch_t<1>(s, mode, q, blk_score, klabel, label_ch, ctx_len, blk_idx, tok_idx, tok_score, sel_keys, sel_cnt, blk_copy, st);
    if (need <= 2) return launch_t<2>(s, mode, q, blk_score, klabel, label_ch, ctx_len, blk_idx, tok_idx, tok_score, sel_keys, sel_cnt, blk_copy, st);
    if (need <= 4) return launch_t<4>(s, mode, q, blk_score, klabel, label_ch, ctx_len, blk_idx, tok_idx, tok_score, sel_keys, sel_cnt, blk_copy, st);
    return launch_t<8>(s, mode, q, blk_score, klabel, label_ch, ctx_len, blk_idx, tok_idx, tok_score, sel_keys, sel_cnt, blk_copy, st);
}

}  // namespace hsab
