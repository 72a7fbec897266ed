// upper.hip -- the coarse-to-fine walk above the leaf level (gfx950).
//
// Reading note "Block Sparse Attention with Log-Linear Complexity", section
// 3.2 and "Scoring: LogSumExp": from the root down to level 2, the candidates
// of a level are the children of the previous survivors; a level with at most
// K candidates keeps them all, otherwise each candidate scores the LSE of the
// query's logits against its (at most two) children's summaries, summed over
// the query heads of the GQA group (section 4.1), and the K best survive. The
// kernel stops at level 2 and writes, per walk, the children of the level-2
// survivors: the leaf-block candidates, ascending, -1 padded.
//
// Layout and arithmetic:
//   * The fp32 summaries are pre-multiplied by log2(e)/sqrt(64) and split
//     into two bf16 planes (hi = rne(x), lo = rne(x - hi); a 17-bit mantissa),
//     so one bf16 MFMA chain v_mfma_f32_16x16x32_bf16 (hi and lo, two k-steps)
//     yields base-2 logits directly. fp32 inputs use fp32 summaries on
//     v_mfma_f32_16x16x4_f32 instead (exact products).
//   * bf16 inputs (walk_upper_delta_kernel): a wavefront walks 64/SLOTS
//     queries at once, SLOTS = 16, 32 or 64 lanes per walk (2K <= SLOTS), lane
//     i of a segment holding candidate slot i. A candidate is scored from ONE
//     row, delta(c) = s(2c) - s(c), and the head-summed logit P(c) of its own
//     summary carried down the walk (the "delta form" in walk_math.h). Each
//     16-column MFMA tile takes the group's query heads as its A operand and 16
//     candidates' delta rows as its B operand, so a lane holds four heads of
//     one candidate: the head sums are in-lane adds plus permlane16/32 swaps.
//   * fp32 inputs (walk_upper_f32_kernel) score both children rows of each
//     candidate on v_mfma_f32_16x16x4_f32 (exact products), children as tile
//     rows and heads as columns.
//   * The coarsest levels are staged in LDS once per workgroup (their delta
//     rows, plus the summary rows of the level where most walks start
//     scoring); finer levels are gathered from global memory (L2), their delta
//     rows stored quarter-major (the 64 bytes one MFMA lane quarter reads of a
//     node together, see delta_planes_kernel). The two kinds of level run in
//     separate loops.
//   * Top-K: bitonic network on each walk's slots over 64-bit (score, node)
//     keys; when 2K equals the slot count, a partial network keeps the top
//     half as a set.
#include "walk_math.h"

namespace pisa {

// planes[0] = rne(x * s), planes[1] = rne(x * s - hi), elementwise over the whole pyramid.
__global__ __launch_bounds__(256) void split_planes_kernel(const float* __restrict__ pyr,
                                                           uint16_t* __restrict__ planes,
                                                           int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        uint32_t hi, lo;
        split_scaled(pyr[i], hi, lo);
        planes[i] = (uint16_t)hi;
        planes[n + i] = (uint16_t)lo;
    }
}

// ------------------------------------------------------------ upper scoring --

template <typename KT>
struct UpperQ;

// bf16 queries: B operand of the bf16 MFMA, dims {8g..8g+7} and {32+8g..32+8g+7}.
template <>
struct UpperQ<uint16_t> {
    bf16x8 k0, k1;
    __device__ void load(const uint16_t* row, bool valid, int gq) {
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (valid) {
            a = *reinterpret_cast<const u32x4*>(row + 8 * gq);
            b = *reinterpret_cast<const u32x4*>(row + 32 + 8 * gq);
        }
        k0 = __builtin_bit_cast(bf16x8, a);
        k1 = __builtin_bit_cast(bf16x8, b);
    }
};

template <>
struct UpperQ<float> {
    float f[16];
    __device__ void load(const float* row, bool valid, int gq) {
#pragma unroll
        for (int i = 0; i < 16; ++i) f[i] = 0.f;
        if (valid) {
            load8_f32(row + 8 * gq, f);
            load8_f32(row + 32 + 8 * gq, f + 8);
        }
    }
};

__device__ inline f32x4 child_tile_f32(const UpperQ<float>& q, const float* __restrict__ pyr_row, int gq) {
    float a[16];
    load8_f32(pyr_row + 8 * gq, a);
    load8_f32(pyr_row + 32 + 8 * gq, a + 8);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 16; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], q.f[s], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] *= kScale2;
    return acc;
}

// ------------------------------------------------------------- tile layout --
// Candidate slot m (0 <= m < SLOTS) of walk w of a wavefront lives in lane
//   16 * g + (SLOTS/4) * w + 2 * tau + p,   with m = 8 * tau + 2 * g + p.
// A 16-row MFMA tile tau of walk w holds children 2m, 2m+1 of slots m = 8 tau .. 8 tau + 7
// in rows 2(m - 8 tau) and 2(m - 8 tau) + 1; the result lane (g, n) holds rows 4g .. 4g+3,
// i.e. both children of slots 8 tau + 2g and 8 tau + 2g + 1: the slots whose home lanes
// are in the same 16-lane row g. After the sum over the head columns a candidate's
// score is present in its home row, so it is taken by a select, without a lane move.
// Flipping bit J of the slot index moves between lanes lane ^ slot_bit_lane(J).
template <int SLOTS>
__device__ constexpr int slot_lane(int w, int m) {
    return 16 * ((m >> 1) & 3) + (SLOTS / 4) * w + 2 * (m >> 3) + (m & 1);
}
constexpr int slot_bit_lane(int J) { return J == 1 ? 1 : J == 2 ? 16 : J == 4 ? 32 : J == 8 ? 2 : J == 16 ? 4 : 8; }

// Children rows of one bf16 tile: hi and lo planes, two k-steps each.
struct TileRows {
    u32x4 h0, h1, l0, l1;
};

__device__ inline TileRows rows_lds(const lds_char_t* lds, int lds_node, int gq) {
    // 24-bit multiply (a full-rate VALU op): LDS slots number fewer than 2^24
    const lds_char_t* p = lds + __umul24((uint32_t)lds_node, (uint32_t)kLdsNodeBytes);
    TileRows r;
    r.h0 = *reinterpret_cast<const lds_u32x4_t*>(p + 16 * gq);
    r.h1 = *reinterpret_cast<const lds_u32x4_t*>(p + 64 + 16 * gq);
    r.l0 = *reinterpret_cast<const lds_u32x4_t*>(p + 128 + 16 * gq);
    r.l1 = *reinterpret_cast<const lds_u32x4_t*>(p + 192 + 16 * gq);
    return r;
}

// Row `row` of a level's hi and lo planes through buffer resources based at the level's
// first row (64 bf16 = 128 bytes per row): one 32-bit offset per lane.
__device__ inline TileRows rows_buffer(buf_rsrc_t hi, buf_rsrc_t lo, int row, int gq) {
    const uint32_t off = ((uint32_t)row << 7) + ((uint32_t)gq << 4);
    TileRows r;
    r.h0 = load_b128(hi, off);
    r.h1 = load_b128(hi, off + 64);
    r.l0 = load_b128(lo, off);
    r.l1 = load_b128(lo, off + 64);
    return r;
}

// The delta row of node `row` of a level of M nodes in the quarter-major layout of the delta
// planes (see delta_planes_kernel): lane quarter gq reads the 64 bytes of (gq, row), hi chunks
// gq and 4 + gq then lo chunks gq and 4 + gq, through a buffer resource based at the level.
__device__ inline TileRows rows_quarter_major(buf_rsrc_t lvl, int row, uint32_t M, int gq) {
    const uint32_t o = (__umul24((uint32_t)gq, M) + (uint32_t)row) << 6;   // M < 2^24
    TileRows r;
    r.h0 = load_b128(lvl, o);
    r.h1 = load_b128(lvl, o + 16);
    r.l0 = load_b128(lvl, o + 32);
    r.l1 = load_b128(lvl, o + 48);
    return r;
}

__device__ inline TileRows rows_global(const uint16_t* __restrict__ plane, int64_t plane_stride, int gq) {
    TileRows r;
    r.h0 = *reinterpret_cast<const u32x4*>(plane + 8 * gq);
    r.h1 = *reinterpret_cast<const u32x4*>(plane + 32 + 8 * gq);
    r.l0 = *reinterpret_cast<const u32x4*>(plane + plane_stride + 8 * gq);
    r.l1 = *reinterpret_cast<const u32x4*>(plane + plane_stride + 32 + 8 * gq);
    return r;
}

// Slot bit J of the tile layout is lane bit slot_bit_lane(J).
struct TileLanes {
    static constexpr int of(int J) { return slot_bit_lane(J); }
};

// fp32 inputs: walks for positions t0 + ti, ti in [0, NT), of every batch element and KV
// head, scoring each candidate from its two children rows of the fp32 pyramid on
// v_mfma_f32_16x16x4_f32. Output per walk (index (b*NT + ti)*Hkv + kvh): cand_out[2K]
// ascending leaf candidates (-1 padded) and ncand_out = their count.
template <int SLOTS, int S>
__global__ __launch_bounds__(kUpperThreads) void walk_upper_f32_kernel(const float* __restrict__ q,
                                                             const float* __restrict__ pyr, Geom G, int64_t t0,
                                                             int64_t NT, int32_t* __restrict__ cand_out,
                                                             int32_t* __restrict__ ncand_out) {
    using KT = float;
    constexpr int WPW = 64 / SLOTS, QW = SLOTS / 4;
    // XCD-aware placement: workgroup i runs on XCD i % 8; when B*Hkv divides 8, every
    // XCD serves a single (batch, KV head), so its L2 holds that head's finer levels only.
    const int BH = G.B * G.Hkv;
    const int id = blockIdx.x, nwg = gridDim.x;
    int bh, peer, npeers;
    if (BH <= 8 && 8 % BH == 0 && nwg % 8 == 0) {
        bh = (id % 8) % BH;
        peer = (id / 8) * (8 / BH) + (id % 8) / BH;
        npeers = nwg / BH;
    } else {
        bh = id % BH;
        peer = id / BH;
        npeers = (nwg - bh + BH - 1) / BH;
    }
    const int b = bh / G.Hkv, kvh = bh % G.Hkv;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    const int gq = lane >> 4, n = lane & 15;
    const int wl = n / QW, ql = n % QW;                       // this lane's walk and position in its row
    const int ml = 8 * (ql >> 1) + 2 * gq + (ql & 1);         // this lane's candidate slot
    const int K = G.topk;
    const int64_t bh_row0 = (int64_t)bh * G.P;

    // lanes of walk w: bits of a wavefront mask
    uint64_t wmask[WPW];
#pragma unroll
    for (int w = 0; w < WPW; ++w) {
        uint64_t mk = 0;
        for (int m = 0; m < SLOTS; ++m) mk |= 1ull << slot_lane<SLOTS>(w, m);
        wmask[w] = mk;
    }

    const int64_t ngroups = (NT + WPW - 1) / WPW;
    for (int64_t grp = (int64_t)peer * nwaves + wave; grp < ngroups; grp += (int64_t)npeers * nwaves) {
        // queries of the WPW walks of this wavefront
        UpperQ<KT> qf[WPW];
        int64_t tw[WPW];
#pragma unroll
        for (int w = 0; w < WPW; ++w) {
            const int64_t ti = grp * WPW + w;
            tw[w] = t0 + ti;
            const bool ok = ti < NT && n < G.GQ;
            const KT* qrow = q + (((int64_t)b * NT + (ti < NT ? ti : 0)) * G.Hq + (int64_t)kvh * G.GQ + n) * kD;
            qf[w].load(qrow, ok, gq);
        }
        const int64_t my_ti = grp * WPW + wl;
        const int64_t my_t = t0 + my_ti;
        const bool my_ok = my_ti < NT;

        int surv = (ml == 0 && my_ok) ? 0 : -1;   // survivors of the level above, slots 0..K-1
        for (int l = G.L; l >= 2; --l) {
            int cand;
            if (l == G.L) {
                cand = surv;
            } else {
                const int par = shfl_i(surv, slot_lane<SLOTS>(wl, ml >> 1));
                const int child = 2 * par + (ml & 1);
                const bool ok = ml < 2 * K && par >= 0 && child < G.M[l] && child <= (int)(my_t >> (kLog2C + l - 1));
                cand = ok ? child : -1;
            }
            // does any walk of this wavefront have more than K candidates here?
            const uint64_t vm = ballot(cand >= 0);
            bool need = false;
#pragma unroll
            for (int w = 0; w < WPW; ++w) need |= __popcll(vm & wmask[w]) > K;
            float my = (cand >= 0) ? 0.0f : -INFINITY;
            if (need) {
                const int lc = l - 1;
                const int Mc = G.M[lc];
                const int sh = kLog2C + lc - 1;              // first key of node i at level lc: i << sh
                const float* pyr_lvl = pyr + (bh_row0 + G.off[lc]) * kD;
#pragma unroll
                for (int w = 0; w < WPW; ++w) {
                    const int tl = (int)(tw[w] >> sh);         // children <= tl are eligible
#pragma unroll
                    for (int tau = 0; tau < SLOTS / 8; ++tau) {
                        // MFMA row n: child (n & 1) of slot 8 tau + n/2
                        const int par = shfl_i(cand, slot_lane<SLOTS>(w, 8 * tau + (n >> 1)));
                        const int child = 2 * par + (n & 1);
                        const bool valid = par >= 0 && child < Mc && child <= tl;
                        const int row = valid ? child : 0;      // invalid rows read row 0; their results are unused
                        const uint32_t rows_ok = (uint32_t)ballot(valid);   // bit r: row r valid
                        const f32x4 acc = child_tile_f32(qf[w], pyr_lvl + (int64_t)row * kD, gq);
                        float sc[2];
                        pair_scores<S>(acc, rows_ok, gq, n, G.GQ, sc);
                        if (wl == w && (ql >> 1) == tau) my = (ql & 1) ? sc[1] : sc[0];
                    }
                }
                if (cand < 0) my = -INFINITY;
            }
            // the survivors are the K best as a set; with 2K = SLOTS a partial network finds them
            const int cidx = (cand >= 0) ? cand : INT_MAX;
            const int nd = (2 * K == SLOTS) ? select_top_half<SLOTS, TileLanes>(my, cidx, ml)
                                            : select_sort<SLOTS, TileLanes>(my, cidx, ml);
            surv = (ml < K && nd != INT_MAX) ? nd : -1;
        }
        // leaf candidates: children of the level-2 survivors (or the root if it is a leaf)
        int leaf;
        if (G.L == 1) {
            leaf = surv;
        } else {
            const int par = shfl_i(surv, slot_lane<SLOTS>(wl, ml >> 1));
            const int child = 2 * par + (ml & 1);
            const bool ok = ml < 2 * K && par >= 0 && child < G.M[1] && child <= (int)(my_t >> kLog2C);
            leaf = ok ? child : -1;
        }
        // ascending order, -1 last
        const int nd = index_sort<SLOTS, TileLanes>((leaf >= 0) ? leaf : INT_MAX, ml);
        leaf = (nd != INT_MAX && ml < 2 * K) ? nd : -1;
        const uint64_t lm = ballot(leaf >= 0);
        uint64_t mine = 0;
#pragma unroll
        for (int w = 0; w < WPW; ++w) mine = (wl == w) ? wmask[w] : mine;
        if (my_ok && ml < 2 * K) {
            const int64_t wid = ((int64_t)b * NT + my_ti) * G.Hkv + kvh;
            cand_out[wid * (2 * K) + ml] = leaf;
            if (ml == 0) ncand_out[wid] = __popcll(lm & mine);
        }
    }
}

// ------------------------------------------------------ delta-form bf16 walk --
// The bf16 walk scores a candidate from ONE summary row, delta(c) = s(2c) - s(c), and a
// carried head-summed logit P(c) (walk_math.h, "delta form"): half the rows, MFMAs and
// gather traffic of scoring from both children. The candidate's own summary is read
// only at the first scored level of a walk (to start P), and the children of the one
// ragged node of a level (a partial right child) are read directly.

// delta planes: node c of level l >= 2 holds the hi/lo bf16 split of
// 2 (s_{l-1}(2c) - s_l(c)) * log2(e)/8 (the doubled delta), rounded like the summary
// planes, 256 bytes per node (both planes). Quarter-major inside each level of a sequence:
// the level's M nodes take M * 256 bytes from twice its first row's summary offset, and
// the 64 bytes that MFMA lane quarter q needs of node c (hi chunks q and 4 + q, lo chunks q
// and 4 + q; chunk g = dims 8g .. 8g+7, 16 bytes) sit together at byte (q * M + c) * 64. A
// walk's 16 candidates come as sibling pairs, which this puts in one 128-byte line, so a
// quarter-wavefront's four loads of a tile touch at most 8 cache lines (the row-major
// planes took 32: the lookups, not the bytes, bound those gathers).
// Grid: (chunks, B * Hkv); with a pack (pk.cu non-null), (D * Hkv, chunks), one row of
// workgroups per (document, KV head).
__global__ __launch_bounds__(256) void delta_planes_kernel(const float* __restrict__ pyr,
                                                           uint16_t* __restrict__ dplanes, Geom G, Pack pk) {
    int64_t row0;
    Seg sg;
    int chunk, nchunks;
    if (pk.cu) {
        const int d = blockIdx.x / G.Hkv;
        sg = pack_seg(pk, d);
        row0 = (int64_t)(blockIdx.x % G.Hkv) * G.P;
        chunk = blockIdx.y;
        nchunks = gridDim.y;
        if (sg.N == 0) return;
    } else {
        sg = batch_seg(G.N, 0);
        row0 = (int64_t)blockIdx.y * G.P;
        chunk = blockIdx.x;
        nchunks = gridDim.x;
    }
    int64_t total = 0;
    for (int l = 2; l <= sg.L; ++l) total += (int64_t)sg.M(l) * kD;
    const float* base = pyr + row0 * kD;
    for (int64_t i = (int64_t)chunk * 256 + threadIdx.x; i < total; i += (int64_t)nchunks * 256) {
        const int e = (int)(i & (kD - 1));
        int64_t r = i >> 6;
        int l = 2;
        while (r >= sg.M(l)) { r -= sg.M(l); ++l; }
        const int64_t lrow = G.off[l] + sg.shift(l), prow = lrow + r, crow = G.off[l - 1] + sg.shift(l - 1) + 2 * r;
        uint32_t hi, lo;
        split_scaled(2.0f * (base[crow * kD + e] - base[prow * kD + e]), hi, lo);
        const int g = e >> 3;
        const int64_t o = (row0 + lrow) * (2 * kD) + (((int64_t)(g & 3) * sg.M(l) + r) * 4 + (g >> 2)) * 8 + (e & 7);
        dplanes[o] = (uint16_t)hi;
        dplanes[o + 16] = (uint16_t)lo;   // the lo chunk two 16-byte pieces on
    }
}

// Slot layout: slot m of walk w (SLOTS = 16 * TPW slots per walk) lives in lane
// w * SLOTS + m. Tile i (lanes 16i .. 16i+15) puts the candidates of its 16 slots in its
// MFMA columns, and the head sums of column n reach every lane of that column, so lane
// 16i + n takes tile i's sums of column n.
template <int SLOTS>
__device__ constexpr int dslot_lane(int w, int m) { return w * SLOTS + m; }

// XCD-aware placement of the walk workgroups: workgroup i runs on XCD i % 8; when B*Hkv
// divides 8, every XCD serves a single (batch, KV head), so its L2 holds that head's finer
// levels only.
__device__ inline void upper_placement(int BH, int& bh, int& peer, int& npeers) {
    const int id = blockIdx.x, nwg = gridDim.x;
    if (BH <= 8 && 8 % BH == 0 && nwg % 8 == 0) {
        bh = (id % 8) % BH;
        peer = (id / 8) * (8 / BH) + (id % 8) / BH;
        npeers = nwg / BH;
    } else {
        bh = id % BH;
        peer = id / BH;
        npeers = (nwg - bh + BH - 1) / BH;
    }
}

// Stage one sequence's rows (U) in LDS, node i of level j -> LDS slot lds_first[j] + i,
// planes hi|lo; the caller synchronises.
__device__ inline void stage_upper_lds(lds_char_t* lds, const uint16_t* __restrict__ splanes,
                                       const uint16_t* __restrict__ dplanes, const Geom& G, const UpperCfg& U,
                                       const Seg& sg, int64_t bh_row0, int64_t plane_stride) {
    for (int j = U.j_lo; j <= U.j_hi; ++j) {
        const int mj = sg.M(j);
        const int64_t r0 = bh_row0 + G.off[j] + sg.shift(j);
        for (int c = threadIdx.x; c < mj * 16; c += blockDim.x) {
            // 16-byte pieces in memory order: quarter q, node, piece p (hi q, hi 4 + q, lo q, lo 4 + q)
            const int qq = c / (4 * mj), r2 = c - qq * 4 * mj, node = r2 >> 2, pp = r2 & 3;
            const uint16_t* src = dplanes + r0 * (2 * kD) + (int64_t)c * 8;
            *reinterpret_cast<lds_u32x4_t*>(lds + (U.lds_first[j] + node) * kLdsNodeBytes + (pp >> 1) * 128 +
                                            (qq + 4 * (pp & 1)) * 16) = *reinterpret_cast<const u32x4*>(src);
        }
    }
    if (U.s_level >= 2) {
        const int ms = sg.M(U.s_level);
        const int64_t r0 = bh_row0 + G.off[U.s_level] + sg.shift(U.s_level);
        for (int c = threadIdx.x; c < ms * 16; c += blockDim.x) {
            const int node = c >> 4, part = c & 15;
            const uint16_t* src = splanes + (part >> 3) * plane_stride + (r0 + node) * kD + (part & 7) * 8;
            *reinterpret_cast<lds_u32x4_t*>(lds + (U.s_first + node) * kLdsNodeBytes + (part >> 3) * 128 +
                                            (part & 7) * 16) = *reinterpret_cast<const u32x4*>(src);
        }
    }
}

// The walks of one wavefront: positions t0 + grp * WPW + w (w < WPW, grp * WPW + w < NT) of
// sequence sg, whose queries (and walk records) are rows qrow0 + grp * WPW + w.
template <int SLOTS, int S>
__device__ inline void upper_delta_group(const uint16_t* __restrict__ q, const uint16_t* __restrict__ splanes,
                                         const uint16_t* __restrict__ dplanes, const Geom& G, const UpperCfg& U,
                                         const Seg& sg, const lds_char_t* lds, int64_t bh_row0,
                                         int64_t plane_stride, int kvh, int64_t qrow0, int64_t t0, int64_t NT,
                                         int64_t grp, int32_t* __restrict__ cand_out,
                                         int32_t* __restrict__ ncand_out) {
    constexpr int WPW = 64 / SLOTS, TPW = SLOTS / 16, NTILE = WPW * TPW;
    static_assert(NTILE == 4, "four 16-row tiles per wavefront");
    const int lane = threadIdx.x & 63;
    const int gq = lane >> 4, n = lane & 15;
    const int u = gq;                                        // tile whose results land in this lane
    const int wl = lane / SLOTS;                             // this lane's walk
    const int ml = lane % SLOTS;                             // this lane's slot
    const int K = G.topk;
    uint64_t wmask[WPW];
#pragma unroll
    for (int w = 0; w < WPW; ++w) {
        uint64_t mk = 0;
        for (int m = 0; m < SLOTS; ++m) mk |= 1ull << dslot_lane<SLOTS>(w, m);
        wmask[w] = mk;
    }

    UpperQ<uint16_t> qf[WPW];
    int tw[WPW];   // positions of the wavefront's walks (wave-uniform; positions fit 31 bits)
    // query rows of consecutive walks are Hq * 64 elements apart; rows past NT are not read
    const uint16_t* qrow0p = q + ((qrow0 + grp * WPW) * G.Hq + (int64_t)kvh * G.GQ + n) * kD;
#pragma unroll
    for (int w = 0; w < WPW; ++w) {
        const int64_t ti = grp * WPW + w;
        tw[w] = __builtin_amdgcn_readfirstlane((int)(t0 + ti));
        const bool ok = ti < NT && n < G.GQ;
        qf[w].load(qrow0p + (int64_t)w * G.Hq * kD, ok, gq);
    }
    const int64_t my_ti = grp * WPW + wl;
    const int my_t = (int)(t0 + my_ti);
    const bool my_ok = my_ti < NT;

    // Levels of at most K nodes keep every eligible node unscored, so the walk starts at the
    // highest level with more than K nodes (at most 2K, since the level above has at most K):
    // its candidates are its eligible nodes, node m in slot m. Without such a level it starts at
    // the root.
    int ls = sg.L;
    for (int j = sg.L; j >= 2; --j) {
        if (sg.M(j) > K) {
            ls = j;
            break;
        }
    }
    uint32_t surv_low = 0;     // sorted key low word in slots < K: the survivors
    float Pa = 0.0f, Pb = 0.0f;  // head-summed logits of this slot's candidate's children
    uint32_t pk = 0;           // walks whose candidates' P is known (scored at the level above)
    // one level of the walk; kInLds: the level's delta rows are staged in LDS (else gathered)
    auto level = [&](int l, auto in_lds_const) {
        constexpr bool in_lds = decltype(in_lds_const)::value;
        // the serial chain from the survivors to the level's row loads runs at a raised wave
        // priority, so that a wavefront's next loads issue ahead of the other wavefronts'
        // scoring arithmetic; the scoring and the sort run at the normal priority
        __builtin_amdgcn_s_setprio(2);
        int cand;
        float P = 0.0f;
        if (l == ls) {
            cand = (my_ok && ml < sg.M(l) && ml <= (my_t >> (kLog2C + l - 1))) ? ml : -1;
        } else {
            const uint32_t lowk = (uint32_t)shfl_i((int)surv_low, dslot_lane<SLOTS>(wl, ml >> 1));
            const int pnode = key_node(lowk);
            const int child = 2 * pnode + (ml & 1);
            const bool ok = (ml < 2 * K) & (pnode >= 0) & (child < sg.M(l)) & (child <= (my_t >> (kLog2C + l - 1)));
            cand = ok ? child : -1;
            const int src = dslot_lane<SLOTS>(wl, key_slot(lowk));
            const float pa = shfl_f(Pa, src), pb = shfl_f(Pb, src);
            P = (ml & 1) ? pb : pa;
        }
        const uint64_t vm = ballot(cand >= 0);
        uint32_t scored = 0;
#pragma unroll
        for (int w = 0; w < WPW; ++w) scored |= (__popcll(vm & wmask[w]) > K) ? (1u << w) : 0u;
        float score = 0.0f;
        Pa = 0.0f;
        Pb = 0.0f;
        if (scored) {
            const int lc = l - 1;
            const int shc = kLog2C + lc - 1;            // first key of a level-lc node i: i << shc
            const int Mc = sg.M(lc);
            const int64_t row_l = bh_row0 + G.off[l] + sg.shift(l);
            const int64_t row_lc = bh_row0 + G.off[lc] + sg.shift(lc);
            const uint32_t lvl_bytes = (uint32_t)sg.M(l) * (kD * 2);
            // level-lc nodes up to tw[w] >> shc are eligible for walk w, so a right child 2c + 1
            // is eligible when it is at most rlim[w] = min(Mc - 1, tw[w] >> shc): one unsigned
            // compare, which c = -1 (2c + 1 = 0xffffffff) fails
            uint32_t rlim[WPW];
#pragma unroll
            for (int w = 0; w < WPW; ++w) {
                const int tl = tw[w] >> shc;
                rlim[w] = (uint32_t)(Mc - 1 < tl ? Mc - 1 : tl);
            }
            // candidate of MFMA column n of tile i (lane 16i + n)
            auto row_cand = [&](int i) -> int { return shfl_i(cand, 16 * i + n); };
            // (1) P of the candidates of walks that were not scored at the level above:
            // head sums of the logits of the candidates' own summaries
            const uint32_t need_p = scored & ~pk;
            if (need_p) {
                const bool s_lds = l == U.s_level;
                const buf_rsrc_t shi = make_rsrc(splanes + row_l * kD, lvl_bytes);
                const buf_rsrc_t slo = make_rsrc(splanes + plane_stride + row_l * kD, lvl_bytes);
#pragma unroll
                for (int i = 0; i < NTILE; ++i) {
                    const int c = row_cand(i);
                    const int cc = (c >= 0) ? c : 0;
                    const TileRows r = s_lds ? rows_lds(lds, U.s_first + cc, gq) : rows_buffer(shi, slo, cc, gq);
                    const f32x4 acc = summary_tile_mfma(qf[i / TPW].k0, qf[i / TPW].k1, r.h0, r.h1, r.l0, r.l1);
                    const float ps = tile_head_sums(acc);
                    if (u == i && ((need_p >> wl) & 1)) P = ps;
                }
            }
            // (2) the delta tiles, the next tile's row in flight
            const int lds_lvl = in_lds ? U.lds_first[l] : 0;
            const buf_rsrc_t dlvl = make_rsrc(dplanes + row_l * (2 * kD), 2 * lvl_bytes);
            auto pick = [&](int i, int& row) -> bool {   // column n's candidate has an eligible right child
                const int c = row_cand(i);
                row = c > 0 ? c : 0;
                return (uint32_t)(2 * c + 1) <= rlim[i / TPW];
            };
            const uint32_t Ml = (uint32_t)sg.M(l);
            auto fetch = [&](int row) -> TileRows {
                if constexpr (in_lds) return rows_lds(lds, lds_lvl + row, gq);
                else return rows_quarter_major(dlvl, row, Ml, gq);
            };
            // each tile's in-lane head parts, then one exchange pattern leaves lane (gq, n)
            // with the sums of tile gq, column n
            float fp[NTILE], xp[NTILE];
            int row0;
            bool rv = pick(0, row0);
            TileRows cur = fetch(row0);
#pragma unroll
            for (int i = 0; i < NTILE; ++i) {
                TileRows nxt = cur;
                bool rv_next = false;
                if (i + 1 < NTILE) {
                    int rown;
                    rv_next = pick(i + 1, rown);
                    nxt = fetch(rown);
                }
                if (i == 0) __builtin_amdgcn_s_setprio(0);
                const f32x4 acc = summary_tile_mfma(qf[i / TPW].k0, qf[i / TPW].k1, cur.h0, cur.h1, cur.l0, cur.l1);
                delta_tile_parts<S>(acc, rv, gq, G.GQ, fp[i], xp[i]);
                cur = nxt;
                rv = rv_next;
            }
            float F, D;
            delta_sums4(fp, xp, F, D);
            score = P + F;
            Pa = P + D;
            Pb = P - D;
            // (3) the ragged node of level l (a partial right child): its two children are
            // read directly when a walk has it as a candidate with an eligible right child
            const int crag = sg.M(l) - 1, brag = 2 * crag + 1;
            if (brag < Mc && covered(lc, brag, sg.N) < span_of(lc)) {
                const bool is_rag = cand == crag && brag <= (my_t >> shc);
                const uint64_t rm = ballot(is_rag);
#pragma unroll
                for (int w = 0; w < WPW; ++w) {
                    if (rm & wmask[w]) {
                        const int crow = (n == 1) ? brag : brag - 1;   // column 0: left child, 1: right
                        const TileRows r = rows_global(splanes + (row_lc + crow) * kD, plane_stride, gq);
                        const f32x4 acc = summary_tile_mfma(qf[w].k0, qf[w].k1, r.h0, r.h1, r.l0, r.l1);
                        float xf, xp;
                        ragged_sums<S>(acc, gq, G.GQ, xf, xp);
                        const float f_fix = readlane_f(xf, 0), pa_fix = readlane_f(xp, 0), pb_fix = readlane_f(xp, 1);
                        if (is_rag && wl == w) {
                            score = f_fix;
                            Pa = pa_fix;
                            Pb = pb_fix;
                        }
                    }
                }
            }
        }
        pk = scored;
        if (scored) {
            // walks with at most K candidates keep them all whatever their scores
            const uint64_t key = slot_key((cand >= 0) ? score : -INFINITY, cand, ml);
            // the survivors are the K best as a set; with 2K = SLOTS a partial network finds them
            uint64_t sorted;
            if constexpr (SLOTS <= 16)
                sorted = (2 * K == SLOTS) ? top_half_mirror<SLOTS>(key, ml) : bitonic_desc<SLOTS, SegmentLanes>(key, ml);
            else
                sorted = (2 * K == SLOTS) ? bitonic_top_half<SLOTS, SegmentLanes>(key, ml)
                                          : bitonic_desc<SLOTS, SegmentLanes>(key, ml);
            surv_low = (ml < K) ? (uint32_t)sorted : 0u;
        } else {
            // no walk of the wavefront has more than K candidates here: all survive. Each walk's
            // candidates move to its first slots (the survivors are a set: order is free), the
            // empty slots after them, by one lane permutation instead of the sorting network.
            const int base = wl * SLOTS;
            const uint64_t seg = (SLOTS == 64) ? ~0ull : (((1ull << SLOTS) - 1ull) << base);
            const int below_c = lanes_below(vm & seg), below_e = lanes_below(~vm & seg);
            const int dst = base + ((cand >= 0) ? below_c : __popcll(vm & seg) + below_e);
            const uint32_t moved = (uint32_t)push_to_lane(dst, (int)(uint32_t)slot_key(0.0f, cand, ml));
            surv_low = (ml < K) ? moved : 0u;
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // the levels down to the last one staged in LDS (the levels above it are not scored), then
    // the gathered ones: each phase without a per-tile choice of source
    int l = ls;
    if (U.j_lo <= U.j_hi)
        for (; l >= 2 && l >= U.j_lo; --l) level(l, std::true_type{});
    for (; l >= 2; --l) level(l, std::false_type{});
    // leaf candidates: children of the level-2 survivors (or the root if it is a leaf)
    int leaf;
    if (sg.L == 1) {
        leaf = (ml == 0 && my_ok) ? 0 : -1;
    } else {
        const uint32_t lowk = (uint32_t)shfl_i((int)surv_low, dslot_lane<SLOTS>(wl, ml >> 1));
        const int pnode = key_node(lowk);
        const int child = 2 * pnode + (ml & 1);
        const bool ok = (ml < 2 * K) & (pnode >= 0) & (child < sg.M(1)) & (child <= (my_t >> kLog2C));
        leaf = ok ? child : -1;
    }
    // ascending order, -1 last
    const int nd = index_sort<SLOTS, SegmentLanes>((leaf >= 0) ? leaf : INT_MAX, ml);
    leaf = (nd != INT_MAX && ml < 2 * K) ? nd : -1;
    const uint64_t lm = ballot(leaf >= 0);
    uint64_t mine = 0;
#pragma unroll
    for (int w = 0; w < WPW; ++w) mine = (wl == w) ? wmask[w] : mine;
    if (my_ok && ml < 2 * K) {
        const int64_t wid = (qrow0 + my_ti) * G.Hkv + kvh;
        cand_out[wid * (2 * K) + ml] = leaf;
        if (ml == 0) ncand_out[wid] = __popcll(lm & mine);
    }
}

// bf16 walks of every batch element: positions t0 + ti, ti in [0, NT), query rows b*NT + ti.
template <int SLOTS, int S>
__global__ __launch_bounds__(kUpperThreads) void walk_upper_delta_kernel(const uint16_t* __restrict__ q,
                                                                         const uint16_t* __restrict__ splanes,
                                                                         const uint16_t* __restrict__ dplanes,
                                                                         Geom G, UpperCfg U, int64_t t0, int64_t NT,
                                                                         int32_t* __restrict__ cand_out,
                                                                         int32_t* __restrict__ ncand_out) {
    constexpr int WPW = 64 / SLOTS;
    extern __shared__ u32x4 lds_u4[];
    lds_char_t* lds = (lds_char_t*)lds_u4;
    int bh, peer, npeers;
    upper_placement(G.B * G.Hkv, bh, peer, npeers);
    const int b = bh / G.Hkv, kvh = bh % G.Hkv;
    const int wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    const int64_t plane_stride = (int64_t)G.B * G.Hkv * G.P * kD;
    const int64_t bh_row0 = (int64_t)bh * G.P;
    const Seg sg = batch_seg(G.N, 0);
    stage_upper_lds(lds, splanes, dplanes, G, U, sg, bh_row0, plane_stride);
    __syncthreads();
    const int64_t ngroups = (NT + WPW - 1) / WPW;
    for (int64_t grp = (int64_t)peer * nwaves + wave; grp < ngroups; grp += (int64_t)npeers * nwaves)
        upper_delta_group<SLOTS, S>(q, splanes, dplanes, G, U, sg, lds, bh_row0, plane_stride, kvh, (int64_t)b * NT,
                                    t0, NT, grp, cand_out, ncand_out);
}

// bf16 walks of a pack of documents (G: the packed layout, B = 1, N = T). The tokens are
// cut into pieces of 2^plog2 (512, or fewer for small packs); the workgroups of a KV head take every npeers-th piece (so
// each holds early and late positions of long documents alike), and walk the document
// parts of a piece with that document's rows staged in LDS (restaged only when the
// document changes).
template <int SLOTS, int S>
__global__ __launch_bounds__(kUpperThreads) void walk_upper_delta_pack_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ splanes, const uint16_t* __restrict__ dplanes,
    Geom G, Pack pk, int plog2, int32_t* __restrict__ cand_out, int32_t* __restrict__ ncand_out) {
    constexpr int WPW = 64 / SLOTS;
    extern __shared__ u32x4 lds_u4[];
    lds_char_t* lds = (lds_char_t*)lds_u4;
    __shared__ UpperCfg s_U;
    int kvh, peer, npeers;
    upper_placement(G.Hkv, kvh, peer, npeers);
    const int wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
    const int64_t plane_stride = (int64_t)G.Hkv * G.P * kD;
    const int64_t bh_row0 = (int64_t)kvh * G.P;
    const int64_t piece = (int64_t)1 << plog2;
    const int64_t npieces = (pk.T + piece - 1) >> plog2;
    int staged = -1;
    for (int64_t p = peer; p < npieces; p += npeers) {
        const int64_t a = p << plog2, e = (a + piece < pk.T) ? a + piece : pk.T;
        for (int d = pack_find_token(pk, a); d < pk.D; ++d) {
            const Seg sg = pack_seg(pk, d);
            const int64_t da = sg.lsh, db = da + sg.N;
            if (da >= e) break;
            if (sg.N == 0 || db <= a) continue;
            if (d != staged) {
                __syncthreads();   // every wavefront is done with the previous document's rows
                if (threadIdx.x == 0) upper_cfg_for(sg, G.topk, s_U);
                __syncthreads();
                stage_upper_lds(lds, splanes, dplanes, G, s_U, sg, bh_row0, plane_stride);
                __syncthreads();
                staged = d;
            }
            const int64_t lo = (a > da ? a : da) - da, hi = (e < db ? e : db) - da;
            const int64_t NT = hi - lo, ngroups = (NT + WPW - 1) / WPW;
            for (int64_t grp = wave; grp < ngroups; grp += nwaves)
                upper_delta_group<SLOTS, S>(q, splanes, dplanes, G, s_U, sg, lds, bh_row0, plane_stride, kvh,
                                            da + lo, lo, NT, grp, cand_out, ncand_out);
        }
    }
}

template __global__ void walk_upper_delta_kernel<16, kScoreLse>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, UpperCfg, int64_t, int64_t, int32_t*, int32_t*);
template __global__ void walk_upper_delta_kernel<16, kScoreMean>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, UpperCfg, int64_t, int64_t, int32_t*, int32_t*);
template __global__ void walk_upper_delta_kernel<16, kScoreMeanHalfVar>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, UpperCfg, int64_t, int64_t, int32_t*, int32_t*);
template __global__ void walk_upper_delta_kernel<32, kScoreLse>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, UpperCfg, int64_t, int64_t, int32_t*, int32_t*);
template __global__ void walk_upper_delta_kernel<32, kScoreMean>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, UpperCfg, int64_t, int64_t, int32_t*, int32_t*);
template __global__ void walk_upper_delta_kernel<32, kScoreMeanHalfVar>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, UpperCfg, int64_t, int64_t, int32_t*, int32_t*);
template __global__ void walk_upper_delta_kernel<64, kScoreLse>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, UpperCfg, int64_t, int64_t, int32_t*, int32_t*);
template __global__ void walk_upper_delta_kernel<64, kScoreMean>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, UpperCfg, int64_t, int64_t, int32_t*, int32_t*);
template __global__ void walk_upper_delta_kernel<64, kScoreMeanHalfVar>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, UpperCfg, int64_t, int64_t, int32_t*, int32_t*);
template __global__ void walk_upper_delta_pack_kernel<16, kScoreLse>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, Pack, int, int32_t*, int32_t*);
template __global__ void walk_upper_delta_pack_kernel<16, kScoreMean>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, Pack, int, int32_t*, int32_t*);
template __global__ void walk_upper_delta_pack_kernel<16, kScoreMeanHalfVar>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, Pack, int, int32_t*, int32_t*);
template __global__ void walk_upper_delta_pack_kernel<32, kScoreLse>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, Pack, int, int32_t*, int32_t*);
template __global__ void walk_upper_delta_pack_kernel<32, kScoreMean>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, Pack, int, int32_t*, int32_t*);
template __global__ void walk_upper_delta_pack_kernel<32, kScoreMeanHalfVar>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, Pack, int, int32_t*, int32_t*);
template __global__ void walk_upper_delta_pack_kernel<64, kScoreLse>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, Pack, int, int32_t*, int32_t*);
template __global__ void walk_upper_delta_pack_kernel<64, kScoreMean>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, Pack, int, int32_t*, int32_t*);
template __global__ void walk_upper_delta_pack_kernel<64, kScoreMeanHalfVar>(const uint16_t*, const uint16_t*, const uint16_t*, Geom, Pack, int, int32_t*, int32_t*);
template __global__ void walk_upper_f32_kernel<16, kScoreLse>(const float*, const float*, Geom, int64_t, int64_t, int32_t*, int32_t*);
template __global__ void walk_upper_f32_kernel<16, kScoreMean>(const float*, const float*, Geom, int64_t, int64_t, int32_t*, int32_t*);
template __global__ void walk_upper_f32_kernel<16, kScoreMeanHalfVar>(const float*, const float*, Geom, int64_t, int64_t, int32_t*, int32_t*);
template __global__ void walk_upper_f32_kernel<32, kScoreLse>(const float*, const float*, Geom, int64_t, int64_t, int32_t*, int32_t*);
template __global__ void walk_upper_f32_kernel<32, kScoreMean>(const float*, const float*, Geom, int64_t, int64_t, int32_t*, int32_t*);
template __global__ void walk_upper_f32_kernel<32, kScoreMeanHalfVar>(const float*, const float*, Geom, int64_t, int64_t, int32_t*, int32_t*);
template __global__ void walk_upper_f32_kernel<64, kScoreLse>(const float*, const float*, Geom, int64_t, int64_t, int32_t*, int32_t*);
template __global__ void walk_upper_f32_kernel<64, kScoreMean>(const float*, const float*, Geom, int64_t, int64_t, int32_t*, int32_t*);
template __global__ void walk_upper_f32_kernel<64, kScoreMeanHalfVar>(const float*, const float*, Geom, int64_t, int64_t, int32_t*, int32_t*);

}  // namespace pisa
