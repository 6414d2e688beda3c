// Exact block-wide top-k selection with stable ties (used by the selection
// kernel for the K_b best blocks and the K_t best tokens of a unit).
#pragma once
#include "common.h"

namespace hsab {

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) { return wave_scan_dpp(v); }

// NW waves hold up to NW*64*PT keys in registers; with pt <= PT slots in
// use, key j of lane `lane` in wave w is entry i = (w*pt + j)*64 + lane.
// Keys are uint32 from f32_key with 0 = empty. select() keeps the
// k_eff = min(k, #nonempty) largest keys, preferring the lower entry among
// equal keys, and calls emit(pos, i) for each kept entry i with pos its rank
// in entry order (0..k_eff-1). Returns k_eff. The caller must pass a
// barrier before it reads what emit wrote to LDS or reuses the scratch.
//
// Method: a 2048-bin histogram of the key values over their [min, max]
// range. The bin map is monotone (non-decreasing) in the key, so every key
// in a higher bin is strictly larger than every key in a lower one: the bins
// above the bin holding the k-th largest key are kept whole, the bins below
// are dropped, and only that one bin's entries are ranked exactly. If that
// bin holds more than CMAX entries (or the value range is not a finite
// positive fp32 number) the k-th largest key is found instead by bit-serial
// refinement over all keys, two bits per round.
// Scratch of a top-k selection by NW waves (independent of the keys per
// thread, so selections of different sizes can share it).
template <int NW>
struct TopKSmem {
    static constexpr int NBIN = 2048, CMAX = 1024;
    uint32_t hist[NBIN];
    uint32_t ckey[CMAX];
    int32_t cidx[CMAX];
    uint32_t red[15 * NW + 4];
};

template <int NW, int PT>
struct TopK {
    static constexpr int NT = NW * 64;
    static constexpr int NBIN = 2048;
    static constexpr int CMAX = 1024;
    static constexpr int BPW = NBIN / NW;     // bins per wave in the scan
    static constexpr int BPT = BPW / 64;      // bins per thread
    static_assert(NBIN % NT == 0, "bins must split evenly");
    // red: [0,8NW) round counts (two parity slots of 4NW), [8NW,10NW)
    // fallback tie counts, [10NW,11NW) compaction counts, [11NW,12NW) wave
    // bin totals, [12NW,15NW) wave min/max/count, then the candidate count.
    using Smem = TopKSmem<NW>;
    static_assert(Smem::NBIN == NBIN && Smem::CMAX == CMAX, "scratch layout");

    template <typename Emit>
    __device__ static int select(const uint32_t (&key)[PT], int pt, int k, Smem& sm, Emit emit) {
        const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
        uint32_t* red = sm.red;
        uint32_t* ccount = red + 15 * NW;
        // 1) clear the histogram; range and count of the nonempty keys
        for (int i = tid; i < NBIN; i += NT) sm.hist[i] = 0u;
        uint32_t lmin = 0xffffffffu, lmax = 0u, cnt = 0u;
#pragma unroll
        for (int j = 0; j < PT; ++j) {
            if (j < pt) {
                const bool v = key[j] != 0u;
                if (v) { lmin = min(lmin, key[j]); lmax = max(lmax, key[j]); }
                cnt += __popcll(__ballot(v));
            }
        }
        lmin = wave_minmax<false>(lmin);
        lmax = wave_minmax<true>(lmax);
        if (lane == 0) { red[12 * NW + w] = lmin; red[13 * NW + w] = lmax; red[14 * NW + w] = cnt; }
        if (tid == 0) *ccount = 0u;
        __syncthreads();
        // over the waves: lane i reads wave i's entries
        const uint32_t kmin = wave_minmax<false>(lane < NW ? red[12 * NW + lane] : 0xffffffffu);
        const uint32_t kmax = wave_minmax<true>(lane < NW ? red[13 * NW + lane] : 0u);
        const uint32_t nval =
            (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_dpp(lane < NW ? red[14 * NW + lane] : 0u), 63);
        const int k_eff = k < (int)nval ? k : (int)nval;
        if (k_eff <= 0) return 0;

        bool keep[PT];
#pragma unroll
        for (int j = 0; j < PT; ++j) keep[j] = key[j] != 0u;   // right when every key is kept
        if (k_eff < (int)nval) {
            const float vmin = key_f32(kmin), vmax = key_f32(kmax);
            const float range = vmax - vmin;
            const float scale = (float)NBIN / range;
            auto bin = [&](uint32_t kk) {
                const int b = (int)((key_f32(kk) - vmin) * scale);
                return b < 0 ? 0 : (b >= NBIN ? NBIN - 1 : b);
            };
            bool done = false;
            if (isfinite(range) && range > 0.f && isfinite(scale)) {
                // 2) histogram
#pragma unroll
                for (int j = 0; j < PT; ++j)
                    if (j < pt && key[j] != 0u) atomicAdd(&sm.hist[bin(key[j])], 1u);
                __syncthreads();
                // 3) wave v owns the bins NBIN-1-(v*BPW + i), i < BPW (top down);
                //    per-wave totals locate the wave whose range holds the k-th
                //    key, then every wave rescans that range itself
                uint32_t loc = 0;
#pragma unroll
                for (int e = 0; e < BPT; ++e) loc += sm.hist[NBIN - 1 - (w * BPW + lane * BPT + e)];
                const uint32_t tot = (uint32_t)__builtin_amdgcn_readlane((int)wave_scan_dpp(loc), 63);
                if (lane == 0) red[11 * NW + w] = tot;
                __syncthreads();
                // the first wave whose running total reaches k_eff, from one
                // lane-parallel read and a scan (the totals cover nval keys)
                const uint32_t tw = lane < NW ? red[11 * NW + lane] : 0u;
                const uint32_t incl = wave_scan_dpp(tw);
                int wp = __ffsll((unsigned long long)__ballot(lane < NW && incl >= (uint32_t)k_eff)) - 1;
                wp = wp < 0 ? NW - 1 : wp;   // unreachable: the totals reach nval >= k_eff
                const uint32_t above = (uint32_t)__builtin_amdgcn_readlane((int)(incl - tw), wp);
                uint32_t hv[BPT], ploc = 0;
#pragma unroll
                for (int e = 0; e < BPT; ++e) { hv[e] = sm.hist[NBIN - 1 - (wp * BPW + lane * BPT + e)]; ploc += hv[e]; }
                uint32_t run = above + wave_incl_scan(ploc) - ploc;
                int bstar = -1;
                uint32_t need = 0;
#pragma unroll
                for (int e = 0; e < BPT; ++e) {
                    if (run < (uint32_t)k_eff && run + hv[e] >= (uint32_t)k_eff) {
                        bstar = NBIN - 1 - (wp * BPW + lane * BPT + e);
                        need = (uint32_t)k_eff - run;
                    }
                    run += hv[e];
                }
                // exactly one lane found it; make it wave-uniform
                const int src = __ffsll((unsigned long long)__ballot(bstar >= 0)) - 1;
                bstar = __builtin_amdgcn_readlane(bstar, src);
                need = __builtin_amdgcn_readlane((int)need, src);
                const uint32_t m = sm.hist[bstar];
                if (m <= (uint32_t)CMAX) {
                    // 4) gather the pivot bin, rank its entries by (key desc, entry asc)
#pragma unroll
                    for (int j = 0; j < PT; ++j) {
                        if (j < pt && key[j] != 0u && bin(key[j]) == bstar) {
                            const uint32_t slot = atomicAdd(ccount, 1u);
                            sm.ckey[slot] = key[j];
                            sm.cidx[slot] = (w * pt + j) * 64 + lane;
                        }
                    }
                    __syncthreads();
#pragma unroll
                    for (int j = 0; j < PT; ++j) {
                        if (j < pt && key[j] != 0u) {
                            const int bj = bin(key[j]);
                            if (bj == bstar) {
                                const int me = (w * pt + j) * 64 + lane;
                                uint32_t rank = 0, c = 0;
                                for (; c + 4 <= m; c += 4) {   // four candidates per LDS read
                                    const uint4 ck = *reinterpret_cast<const uint4*>(&sm.ckey[c]);
                                    const int4 ci = *reinterpret_cast<const int4*>(&sm.cidx[c]);
                                    rank += (ck.x > key[j]) || (ck.x == key[j] && ci.x < me);
                                    rank += (ck.y > key[j]) || (ck.y == key[j] && ci.y < me);
                                    rank += (ck.z > key[j]) || (ck.z == key[j] && ci.z < me);
                                    rank += (ck.w > key[j]) || (ck.w == key[j] && ci.w < me);
                                }
                                for (; c < m; ++c) {
                                    const uint32_t ck = sm.ckey[c];
                                    rank += (ck > key[j]) || (ck == key[j] && sm.cidx[c] < me);
                                }
                                keep[j] = rank < need;
                            } else {
                                keep[j] = bj > bstar;
                            }
                        }
                    }
                    done = true;
                }
            }
            if (!done) {
                // fallback: bit-serial search for the k-th largest key T
                uint32_t prefix = 0;
                int round = 1;
                for (int bit = 30; bit >= 0; bit -= 2, ++round) {
                    const uint32_t c1 = prefix | (1u << bit), c2 = prefix | (2u << bit), c3 = prefix | (3u << bit);
                    uint32_t n1 = 0, n2 = 0, n3 = 0;
#pragma unroll
                    for (int j = 0; j < PT; ++j) {
                        if (j < pt) {
                            n1 += __popcll(__ballot(key[j] >= c1));
                            n2 += __popcll(__ballot(key[j] >= c2));
                            n3 += __popcll(__ballot(key[j] >= c3));
                        }
                    }
                    uint32_t* slot = red + (round & 1) * 4 * NW;
                    if (lane == 0) { slot[w] = n1; slot[NW + w] = n2; slot[2 * NW + w] = n3; }
                    __syncthreads();
                    uint32_t t1 = 0, t2 = 0, t3 = 0;
#pragma unroll
                    for (int i = 0; i < NW; ++i) { t1 += slot[i]; t2 += slot[NW + i]; t3 += slot[2 * NW + i]; }
                    if (t3 >= (uint32_t)k_eff) prefix = c3;
                    else if (t2 >= (uint32_t)k_eff) prefix = c2;
                    else if (t1 >= (uint32_t)k_eff) prefix = c1;
                }
                const uint32_t T = prefix;
                // keys > T are kept; among keys == T the first (k_eff - #{> T}) in entry order
                uint32_t gt = 0, eq = 0;
#pragma unroll
                for (int j = 0; j < PT; ++j)
                    if (j < pt) { gt += __popcll(__ballot(key[j] > T)); eq += __popcll(__ballot(key[j] == T)); }
                uint32_t* cnt2 = red + 8 * NW;
                if (lane == 0) { cnt2[w] = gt; cnt2[NW + w] = eq; }
                __syncthreads();
                uint32_t gt_tot = 0, eq_before = 0;
#pragma unroll
                for (int i = 0; i < NW; ++i) { gt_tot += cnt2[i]; if (i < w) eq_before += cnt2[NW + i]; }
                const uint32_t need_eq = (uint32_t)k_eff - gt_tot;
                const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
                uint32_t eq_run = eq_before;
#pragma unroll
                for (int j = 0; j < PT; ++j) {
                    if (j < pt) {
                        const uint64_t meq = __ballot(key[j] == T);
                        keep[j] = key[j] > T || (key[j] == T && eq_run + __popcll(meq & lt) < need_eq);
                        eq_run += __popcll(meq);
                    }
                }
            }
        }
        compact(key, pt, keep, red, emit);
        return k_eff;
    }

    // Emit the entries with keep[j] set, ranked in entry order.
    template <typename Emit>
    __device__ static void compact(const uint32_t (&key)[PT], int pt, const bool (&keep)[PT], uint32_t* red,
                                   Emit emit) {
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        uint32_t cntw = 0;
#pragma unroll
        for (int j = 0; j < PT; ++j)
            if (j < pt) cntw += __popcll(__ballot(keep[j]));
        uint32_t* c = red + 10 * NW;
        if (lane == 0) c[w] = cntw;
        __syncthreads();
        // entries kept by the waves before this one: lane-parallel read + scan
        const uint32_t cv = lane < NW ? c[lane] : 0u;
        uint32_t run = (uint32_t)__builtin_amdgcn_readlane((int)(wave_scan_dpp(cv) - cv), w);
#pragma unroll
        for (int j = 0; j < PT; ++j) {
            if (j < pt) {
                const uint64_t mk = __ballot(keep[j]);
                if (keep[j]) emit((int)(run + __popcll(mk & lt)), (w * pt + j) * 64 + lane);
                run += __popcll(mk);
            }
        }
    }
};

}  // namespace hsab
