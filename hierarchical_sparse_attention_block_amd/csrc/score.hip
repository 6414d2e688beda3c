// Block scoring on the matrix cores.
//
// The Quest-style upper bound of q.k over a block, sum_c max(q_c*Kmax_c,
// q_c*Kmin_c), equals q+ . Kmax + q- . Kmin with q+ = max(q,0) and
// q- = min(q,0). Stacking [Kmax | Kmin] per block (the metadata row) and
// [q+ | q-] per query head turns the bound of every (head, block) pair into
// one dense product, so query heads that share a KV head (GQA groups, MLA)
// score all blocks in a single GEMM (AsyncTLS, gist.science/de explainer
// section 2.A "Optimierung"; gist.science/es explainer section 2.A item 1).
// The block score is the maximum of the bound over the group (or the sum,
// or, with per-head selection, every head's own bound).
//
// Mapping onto v_mfma_f32_16x16x32_bf16: A = [q+ | q-] (16 head rows per
// tile; rows past the group repeat head 0 and are never read back), B =
// metadata rows (16 blocks per tile), K = the
// 2*d_k stacked channels in steps of 32. Lane l supplies block (l % 16) and
// the 8-channel chunk 4*s + l/16 of step s, i.e. one 16-byte load per step;
// the 16 lanes of a chunk read 16 different 64-byte row segments, and four
// consecutive steps cover each row's cache lines fully. Each wave holds its
// A fragments in registers (loaded once; the queries stay in L2), so no
// workgroup barrier precedes the metadata stream. Long rows (more than 16
// steps, e.g. 576-dim latent keys) split their steps over the four waves of
// a workgroup, which add their partial tiles through LDS. The result tile
// holds block (l % 16) in lane l for head rows 4*(l/16)..+3; a max over
// valid heads and two lane swaps leave the block score in lanes 0..15.
//
// Metadata in fp8 e4m3 (max rounded up, min rounded down, so the bound
// still holds; quantised index data, gist.science/de explainer section 2.A
// "Stufe 2"): a 16-byte load then carries 16 channels, which
// v_cvt_pk_f32_fp8 and v_cvt_pk_bf16_f32 widen exactly to the B fragments
// of two consecutive steps; the A fragments follow the same channel order.
#include "common.h"
#include "kernels.h"

namespace hsab {

namespace {

constexpr int SCORE_WAVES = 4;
constexpr int SPLIT_TILES = 4;   // tiles of a split-row workgroup

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
    int lab8;                 // label rows in e4m3 bytes
};

// MT: 16-row head tiles (G <= 16 or <= 32); KSW: max row loads (16 bytes
// per lane) per wave and tile; KSPLIT: waves sharing one block tile (1: each
// wave scores its own tiles); F8: metadata in e4m3 bytes, widened to bf16 in
// registers (one load then feeds two matrix steps).
template <int MT, int KSW, int KSPLIT, bool F8>
__global__ __launch_bounds__(256) void block_score_kernel(
    const uint16_t* __restrict__ q, uint16_t* __restrict__ meta,
    const int32_t* __restrict__ ctx_len, float* __restrict__ score,
    int Hkv, int G, int dk, int bs, int max_ctx, int nb_cap, int tiles_per_wave, Append ap,
    Handoff ho, int agg) {
    __shared__ f32x4_t red[KSPLIT > 1 ? SPLIT_TILES * KSPLIT * MT * 64 : 1];

    const int unit = blockIdx.y, b = unit / Hkv, g = unit % Hkv;
    int n = ctx_len[b];
    n = n < 1 ? 1 : (n > max_ctx ? max_ctx : n);
    const int nb = (n + bs - 1) / bs;
    constexpr int TILES_WG = SCORE_WAVES / KSPLIT;     // block tiles side by side in a workgroup
    const int per_wg = TILES_WG * tiles_per_wave * 16;
    const int j_wg = blockIdx.x * per_wg;
    // With an append and one tile per wave, an extra last column of
    // workgroups appends the token and then scores the tile holding the tail
    // block, which the workgroup covering that tile skips: the append then
    // delays no streaming workgroup, and the tile is scored by the same code
    // either way. Split-row workgroups (one per CU, a grid of about one
    // round) append in the workgroup that owns the tail block instead, as an
    // extra workgroup there would run in a second round.
    constexpr bool SEP = KSPLIT == 1;
    const bool app_wg = SEP && ap.k_new && blockIdx.x == gridDim.x - 1;
    const int tail_j0 = SEP && ap.k_new ? ((nb - 1) & ~15) : -1;
    // shared state of the split token selection that follows in the step:
    // arrival counters (one per unit, or one per query head with per-head
    // selection) to zero, the unit's candidate keys to KEY_PENDING, spread
    // over the unit's workgroups
    const int heads = agg == AGG_HEAD ? G : 1;
    if (ho.cnt) {
        if (blockIdx.x == 0 && threadIdx.x < heads) ho.cnt[unit * heads + threadIdx.x] = 0;
        const int nk = heads * ho.keys_per_sel;
        uint32_t* ku = ho.keys + (size_t)unit * nk;
        for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < nk; i += gridDim.x * blockDim.x) ku[i] = KEY_PENDING;
    }
    if (!app_wg && j_wg >= nb) return;

    if (app_wg) {
        const int pos = n - 1, jt = pos / bs;
        const bool first = (pos % bs) == 0;
        const uint16_t* kn = ap.k_new + (size_t)unit * dk;
        uint8_t* Mt = meta_block(meta, (size_t)unit * nb_cap + jt, dk, F8);
        uint16_t* Krow = ap.K + ((size_t)unit * max_ctx + pos) * dk;
        for (int c = threadIdx.x; c < dk; c += blockDim.x) {
            const uint16_t kb = kn[c];
            Krow[c] = kb;
            meta_widen(Mt, dk, c, kb, first, F8);
        }
        if (ap.V) {
            const uint16_t* vn = ap.v_new + (size_t)unit * ap.dv;
            uint16_t* Vrow = ap.V + ((size_t)unit * max_ctx + pos) * ap.dv;
            for (int c = threadIdx.x; c < ap.dv; c += blockDim.x) Vrow[c] = vn[c];
        }
        const size_t lrow = ((size_t)unit * max_ctx + pos) * ap.r;
        for (int c = threadIdx.x; c < ap.r; c += blockDim.x)
            label_put(ap.klabel, lrow + c, kn[clamp_ch(ap.label_ch[g * ap.r + c], dk)], ap.lab8);
        __syncthreads();   // the tail block's new bounds are read below
    }

    // Split-row append: the workgroup owning the tail block requests the
    // tail block's current bounds, the new key (and value) and the label
    // channels before its A fragments and tile rows, widens the bounds in
    // LDS once those arrive (its rows still in flight), publishes the
    // widened row, the key, value and label rows, and multiplies its copy
    // of the tail block's rows from LDS; no tile row waits for the append.
    constexpr int RV = KSPLIT > 1 ? 256 : 1;    // 16-byte words of the longest metadata row (2 x 1024 bf16)
    __shared__ uint4 s_tail[RV];
    __shared__ uint16_t s_kn[KSPLIT > 1 ? 1024 : 1];
    const bool app_split = KSPLIT > 1 && ap.k_new && nb - 1 < j_wg + per_wg;
    const int jt = (n - 1) / bs;                 // the tail block
    const int row_vec = 2 * dk * (F8 ? 1 : 2) / 16;
    uint4 orow = make_uint4(0u, 0u, 0u, 0u);
    uint16_t kv[4] = {0, 0, 0, 0}, vv[4] = {0, 0, 0, 0};
    int lab = 0;
    if constexpr (KSPLIT > 1) {
        if (app_split) {   // every load unconditional (clamped), so the wait counts stay exact
            const int tid = threadIdx.x;
            const uint8_t* Mo = meta_block(meta, (size_t)unit * nb_cap + jt, dk, F8);
            orow = ldg16(Mo + (size_t)(tid < row_vec ? tid : row_vec - 1) * 16);
            const uint16_t* kn = ap.k_new + (size_t)unit * dk;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = tid + 256 * i;
                kv[i] = kn[c < dk ? c : dk - 1];
            }
            const uint16_t* vn = ap.V ? ap.v_new + (size_t)unit * ap.dv : kn;
            const int vlim = ap.V ? ap.dv : dk;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = tid + 256 * i;
                vv[i] = vn[c < vlim ? c : vlim - 1];
            }
            lab = ap.label_ch[g * ap.r + (tid < ap.r ? tid : ap.r - 1)];
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // row loads of 64 bytes per 16 lanes over the 2*dk stacked channels:
    // 32 channels of bf16 (one matrix step) or 64 of e4m3 (two steps)
    constexpr int LS = F8 ? 2 : 1;             // matrix steps per load
    const int KS = F8 ? dk / 32 : dk / 16;     // loads per metadata row
    const int CH = dk / 8;                     // 8-channel chunks in one half
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int part = KSPLIT > 1 ? wave : 0;              // step range of this wave
    const int tslot = KSPLIT > 1 ? 0 : wave;             // tile column of this wave
    const int s_lo = part * KS / KSPLIT, s_hi = (part + 1) * KS / KSPLIT;
    float* Su = score + (size_t)unit * heads * nb_cap;
    // first block of tile t of this wave (nb or more: no such tile)
    auto tile_j0 = [&](int t) {
        return app_wg ? (t == 0 && tslot == 0 ? tail_j0 : nb) : j_wg + (t * TILES_WG + tslot) * 16;
    };
    auto tile_row = [&](int t) {
        const int jl = tile_j0(t) + (lane & 15);
        const int jc = jl < nb ? jl : nb - 1;          // keep loads inside the unit's blocks
        return meta_block(meta, (size_t)unit * nb_cap + jc, dk, F8) + (lane >> 4) * 16;
    };
    // 8-channel chunk of the stacked row that matrix step w of load st feeds
    // to this lane (the A fragments follow the same order)
    auto chunk = [&](int st, int w) { return F8 ? 2 * (st * 4 + (lane >> 4)) + w : st * 4 + (lane >> 4); };

    // A fragments are requested first (they come from L2), then the tile
    // rows, so converting the fragments waits for none of the rows. Every
    // load is unconditional: steps past this wave's range re-read its last
    // step and meet zero A fragments (the matrix instructions run for every
    // step, so their products must vanish rather than depend on stale
    // registers), and tiles past the workgroup's range re-read its last
    // tile, which keeps each wait count exact.
    const uint16_t* qg = q + ((size_t)b * Hkv * G + (size_t)g * G) * dk;
    uint4 af[MT][KSW * LS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + (lane & 15);
        const uint16_t* qm = qg + (size_t)(m < G ? m : 0) * dk;
#pragma unroll
        for (int u = 0; u < KSW; ++u) {
            const int st = s_lo + u < s_hi ? s_lo + u : s_hi - 1;
#pragma unroll
            for (int w = 0; w < LS; ++w) {
                const int c = chunk(st, w);
                af[mt][u * LS + w] = ldg16(qm + (c >= CH ? c - CH : c) * 8);
            }
        }
    }
    // split-row (latent) rows are loaded non-temporally: the stream then
    // leaves the caches to the selection and attention that follow it
    auto load_tile = [&](int t, uint4 (&dst)[KSW]) {
        const uint8_t* row = tile_row(t < tiles_per_wave ? t : tiles_per_wave - 1);
#pragma unroll
        for (int u = 0; u < KSW; ++u) {
            const uint8_t* p = row + (s_lo + u < s_hi ? s_lo + u : s_hi - 1) * 64;
            dst[u] = KSPLIT > 1 ? ldg16_nt(p) : ldg16(p);
        }
    };
    // split-row workgroups take SPLIT_TILES tiles, all requested at once:
    // tile 0 first, then the sign split of the fragments (it runs while
    // tile 0's rows are in flight), then the other tiles. The scheduling
    // barriers pin that order and keep every load ahead of the first row
    // wait, so the waits count the loads down in issue order; left to
    // itself the scheduler moves loads behind earlier tiles' products. A
    // wave cannot issue past a full memory queue, so whatever follows the
    // last load waits for the queue to drain.
    constexpr int NBUF = KSPLIT > 1 ? SPLIT_TILES : 1;
    uint4 tl[NBUF][KSW];
    load_tile(0, tl[0]);
    if constexpr (KSPLIT > 1) __builtin_amdgcn_sched_barrier(0);
    // sign split without branches (a branch here lets the compiler sink a
    // fragment load into it, behind the rows). Rows of heads >= G are never
    // read back, so they need no clearing; steps past this wave's range
    // re-read its last step and are cleared below, as the matrix
    // instructions run for every step.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int u = 0; u < KSW * LS; ++u) {
            const uint4 r = af[mt][u];
            const uint32_t neg = chunk(s_lo + u / LS, u % LS) >= CH ? ~0u : 0u;
            af[mt][u] = make_uint4(bf16x2_split(r.x, neg), bf16x2_split(r.y, neg), bf16x2_split(r.z, neg),
                                   bf16x2_split(r.w, neg));
        }
    }
    if (s_hi - s_lo < KSW) {   // uniform: this wave has fewer steps than loads
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int u = 0; u < KSW * LS; ++u)
                if (s_lo + u / LS >= s_hi) af[mt][u] = make_uint4(0u, 0u, 0u, 0u);
    }
    if constexpr (KSPLIT > 1) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 1; d < NBUF; ++d) load_tile(d, tl[d]);
        __builtin_amdgcn_sched_barrier(0);
    }
    int tail_tile = -1;   // split-row append: this workgroup's tile holding the tail block
    if constexpr (KSPLIT > 1) {
        if (app_split) {
            const int tid = threadIdx.x, pos = n - 1;
            const bool first = (pos % bs) == 0;
            if (tid < row_vec) s_tail[tid] = orow;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (tid + 256 * i < dk) s_kn[tid + 256 * i] = kv[i];
            __syncthreads();
            uint16_t* Krow = ap.K + ((size_t)unit * max_ctx + pos) * dk;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = tid + 256 * i;
                if (c < dk) {
                    meta_widen(reinterpret_cast<uint8_t*>(s_tail), dk, c, kv[i], first, F8);
                    Krow[c] = kv[i];
                }
            }
            if (ap.V) {
                uint16_t* Vrow = ap.V + ((size_t)unit * max_ctx + pos) * ap.dv;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (tid + 256 * i < ap.dv) Vrow[tid + 256 * i] = vv[i];
                const uint16_t* vn = ap.v_new + (size_t)unit * ap.dv;
                for (int c = tid + 1024; c < ap.dv; c += 256) Vrow[c] = vn[c];   // values past 1024
            }
            __syncthreads();
            uint8_t* Mt = meta_block(meta, (size_t)unit * nb_cap + jt, dk, F8);
            if (tid < row_vec) *reinterpret_cast<uint4*>(Mt + (size_t)tid * 16) = s_tail[tid];
            if (tid < ap.r)
                label_put(ap.klabel, ((size_t)unit * max_ctx + pos) * ap.r + tid, s_kn[clamp_ch(lab, dk)], ap.lab8);
            tail_tile = (jt - j_wg) / 16;
        }
    }

    // partial bound tile of this wave's steps
    // take: this lane holds the tail block of a split-row append, whose
    // widened rows are read from LDS instead of the rows loaded before
    auto mul_tile = [&](const uint4 (&rows)[KSW], f32x4_t (&tot)[MT], bool take = false) {
        // two accumulators per head tile shorten the dependent MFMA chain
        f32x4_t acc[MT][2];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt][0] = acc[mt][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < KSW; ++u) {
            uint4 rw = rows[u];
            if constexpr (KSPLIT > 1) {
                const int st = s_lo + u < s_hi ? s_lo + u : s_hi - 1;
                const uint4 pv = s_tail[st * 4 + (lane >> 4)];
                // per component: a select of the whole vector goes through memory
                rw.x = take ? pv.x : rw.x;
                rw.y = take ? pv.y : rw.y;
                rw.z = take ? pv.z : rw.z;
                rw.w = take ? pv.w : rw.w;
            }
#pragma unroll
            for (int w = 0; w < LS; ++w) {
                // e4m3 bytes 8w..8w+7 of the load widened to bf16 (exact)
                const uint4 bv = F8 ? f8x8_bf16(w == 0 ? make_uint2(rw.x, rw.y) : make_uint2(rw.z, rw.w)) : rw;
                const int k = u * LS + w;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[mt][k & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(af[mt][k]), as_bf16x8(bv),
                                                                           acc[mt][k & 1], 0, 0, 0);
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) tot[mt] = acc[mt][0] + acc[mt][1];
    };
    // group maximum (or sum) of the bound of tile t's blocks, stored; with
    // per-head selection every head's bound is stored in its own row
    auto emit = [&](int t, const f32x4_t (&tot)[MT]) {
        if (agg == AGG_HEAD) {
            const int j0 = tile_j0(t), jl = j0 + (lane & 15);
            if (jl < nb && (app_wg || j0 != tail_j0)) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int h = mt * 16 + (lane >> 4) * 4 + i;
                        if (h < G) Su[(size_t)h * nb_cap + jl] = tot[mt][i];
                    }
            }
            return;
        }
        // group maximum and sum side by side, without branches; heads past
        // G are left out by selects
        float vs = 0.f, vm = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = mt * 16 + (lane >> 4) * 4 + i < G;
                const float x = tot[mt][i];
                vs = ok ? vs + x : vs;
                vm = ok ? fmaxf(vm, x) : vm;
            }
        if (G > 4) {   // heads 4.. sit in the other 16-lane rows
            vs = sum_xor32(sum_xor16(vs));
            vm = max_xor32(max_xor16(vm));
        }
        const float v = agg == AGG_SUM ? vs : vm;
        const int j0 = tile_j0(t), jl = j0 + (lane & 15);
        if (lane < 16 && jl < nb && (app_wg || j0 != tail_j0)) Su[jl] = v;
    };

    if constexpr (KSPLIT > 1) {
        // every wave multiplies its steps of each tile as the rows land, the
        // partial tiles meet in LDS once, and wave d adds up and emits tile d
#pragma unroll
        for (int d = 0; d < NBUF; ++d) {
            f32x4_t tot[MT];
            mul_tile(tl[d], tot, d == tail_tile && tile_j0(d) + (lane & 15) == jt);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) red[((d * KSPLIT + wave) * MT + mt) * 64 + lane] = tot[mt];
        }
        __syncthreads();
        static_assert(NBUF <= SCORE_WAVES, "one emitting wave per tile");
        if (wave < NBUF && tile_j0(wave) < nb) {
            f32x4_t tot[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                tot[mt] = red[((wave * KSPLIT) * MT + mt) * 64 + lane];
#pragma unroll
                for (int w = 1; w < KSPLIT; ++w) tot[mt] += red[((wave * KSPLIT + w) * MT + mt) * 64 + lane];
            }
            emit(wave, tot);
        }
    } else {
        // one tile in flight per wave: the next tile's rows are requested
        // once the current one is multiplied (with this many waves per CU
        // the memory system is kept busy; prefetching one or more tiles
        // ahead measured no faster with bf16 rows and slower with e4m3)
        for (int t = 0; t < tiles_per_wave; ++t) {
            if (tile_j0(t) >= nb) break;
            f32x4_t tot[MT];
            mul_tile(tl[0], tot);
            emit(t, tot);
            if (t + 1 < tiles_per_wave && tile_j0(t + 1) < nb) load_tile(t + 1, tl[0]);
        }
    }
}

template <int MT, int KSW, int KSPLIT, bool F8>
hipError_t launch_t(const Shape& s, const uint16_t* q, uint16_t* meta, const int32_t* ctx_len,
                    float* score, const Append& ap, const Handoff& ho, hipStream_t st) {
    constexpr int TILES_WG = SCORE_WAVES / KSPLIT;
    // Tiles per wave, chosen by timing the step: bf16 rows take one, so the
    // grid is many short workgroups that keep every CU fed to the end of the
    // launch (against ~2048 workgroups of 2-6 tiles per wave: gqa48k step
    // 52.8 -> 52.0 us, gqa96k 133.8 -> 125.2 us); e4m3 rows carry half the
    // bytes per tile and take two (one: gqa48k 44.7 -> 46.7 us; ~2048
    // workgroups: gqa96k 95.1 -> 97.5 us); split-row workgroups take
    // SPLIT_TILES tiles each, all in flight at once
    const int tpw = KSPLIT > 1 ? SPLIT_TILES : (F8 ? 2 : 1);
    const int per_wg = TILES_WG * tpw * 16;
    dim3 grid((s.nb_cap + per_wg - 1) / per_wg + (KSPLIT == 1 && ap.k_new ? 1 : 0), s.B * s.Hkv);
    hipLaunchKernelGGL((block_score_kernel<MT, KSW, KSPLIT, F8>), grid, dim3(64 * SCORE_WAVES), 0, st, q, meta,
                       ctx_len, score, s.Hkv, s.G, s.dk, s.bs, s.max_ctx, s.nb_cap, tpw, ap, ho, s.agg);
    return hipGetLastError();
}

template <int MT>
hipError_t launch_mt(const Shape& s, const uint16_t* q, uint16_t* meta, const int32_t* ctx_len, float* score,
                     const Append& ap, const Handoff& ho, hipStream_t st) {
    if (s.meta8) {   // e4m3 rows: d_k / 32 loads of 64 channels, two matrix steps each
        const int kl = s.dk / 32;
        if (kl <= 2) return launch_t<MT, 2, 1, true>(s, q, meta, ctx_len, score, ap, ho, st);
        if (kl <= 4) return launch_t<MT, 4, 1, true>(s, q, meta, ctx_len, score, ap, ho, st);
        if (kl <= 8) return launch_t<MT, 8, 1, true>(s, q, meta, ctx_len, score, ap, ho, st);
        if (kl <= 16) return launch_t<MT, 4, 4, true>(s, q, meta, ctx_len, score, ap, ho, st);
        if (kl <= 20) return launch_t<MT, 5, 4, true>(s, q, meta, ctx_len, score, ap, ho, st);
        return launch_t<MT, 8, 4, true>(s, q, meta, ctx_len, score, ap, ho, st);   // d_k <= 1024
    }
    const int ks = s.dk / 16;
    if (ks <= 4) return launch_t<MT, 4, 1, false>(s, q, meta, ctx_len, score, ap, ho, st);
    if (ks <= 8) return launch_t<MT, 8, 1, false>(s, q, meta, ctx_len, score, ap, ho, st);
    if (ks <= 16) return launch_t<MT, 16, 1, false>(s, q, meta, ctx_len, score, ap, ho, st);
    if (ks <= 32) return launch_t<MT, 8, 4, false>(s, q, meta, ctx_len, score, ap, ho, st);
    if (ks <= 36) return launch_t<MT, 9, 4, false>(s, q, meta, ctx_len, score, ap, ho, st);    // 576-dim latent keys
    if (ks <= 40) return launch_t<MT, 10, 4, false>(s, q, meta, ctx_len, score, ap, ho, st);
    return launch_t<MT, 16, 4, false>(s, q, meta, ctx_len, score, ap, ho, st);   // d_k <= 1024: <= 64 steps
}

}  // namespace

hipError_t launch_block_score(const Shape& s, const uint16_t* q, uint16_t* meta, const int32_t* ctx_len,
                              float* score, const uint16_t* k_new, const uint16_t* v_new, uint16_t* K,
                              uint16_t* V, uint16_t* klabel, const int32_t* label_ch, const Handoff* ho,
                              hipStream_t st) {
    const Append ap{k_new, v_new, K, s.valias ? nullptr : V, klabel, label_ch, s.dv, s.r, s.lab8};
    const Handoff h = ho ? *ho : Handoff{nullptr, nullptr, 0};
    return s.G <= 16 ? launch_mt<1>(s, q, meta, ctx_len, score, ap, h, st)
                     : launch_mt<2>(s, q, meta, ctx_len, score, ap, h, st);
}

}  // namespace hsab
