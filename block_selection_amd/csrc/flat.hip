// flat.hip -- flat stage-one selection (gfx950): every query position against every
// eligible leaf summary, top K per (position, KV head).
//
// Reading note "Block Sparse Attention with Log-Linear Complexity", "Background: two
// stages, and the bottleneck in the first" (and the ai4snews summary's first paragraph):
// the conventional stage one gives every key block a mean-pooled summary and scores each
// query against all of them, keeping the K best -- the scan the pyramid walk replaces.
// Score of block b for (position t, KV head j): the sum over the group's query heads h of
// q_{t,h} . kbar_b / sqrt(64), which equals (sum_h q_{t,h}) . kbar_b / 8, so one summed
// query row per (t, j) enters the product. Block b is eligible iff b * 64 <= t; equal
// scores rank the lower block first; the output lists the K best in ascending order, -1
// padded.
//
// Layout and arithmetic:
//   * flat_planes_kernel: the fp32 leaf means (pyramid level 1) as two bf16 planes,
//     hi = rne(x) and lo = rne(x - hi) (a 17-bit mantissa).
//   * flat_select_kernel: one wavefront per 32 consecutive positions of one (batch, KV
//     head); they share one causal bound (blocks 0 .. T0/64). The summed query rows (fp32
//     sums of the group's heads, split into hi and lo the same way) are the B operand of
//     v_mfma_f32_16x16x32_bf16 (2 column tiles of 16 positions), 16 blocks' summary planes
//     the A operand; hi*hi + hi*lo + lo*hi over two k-steps give fp32 scores within about
//     2^-16 of the exact product. Lane (gq, n) of column tile c receives blocks
//     16 bt + 4 gq + r (r < 4) of position T0 + 16 c + n.
//   * Top K per position: a candidate list in LDS of 64-bit selection keys (score, then
//     lower index) and a threshold, the score of the K-th best key kept so far -- a block
//     scoring below it cannot enter the top K. Scores at or above it are appended; a list
//     that could overflow on the next tile is cut back to its K best by a bitonic sort,
//     which raises the threshold. At the end each list's K best are sorted by block index.
#include "walk_math.h"

namespace pisa {

// hi/lo bf16 planes of the leaf means of every (batch, KV head): planes[(bh * M1 + i) * 64 + e]
// and the lo plane plane_stride elements later.
__global__ __launch_bounds__(256) void flat_planes_kernel(const float* __restrict__ pyr, Geom G,
                                                          uint16_t* __restrict__ planes) {
    const int64_t M1 = G.M[1];
    const int64_t n = (int64_t)G.B * G.Hkv * M1 * kD;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const int64_t bh = i / (M1 * kD), rem = i % (M1 * kD);
        const float x = pyr[(bh * G.P + G.off[1]) * kD + rem];
        const uint32_t hi = rne_bf16_bits(x);
        const uint32_t lo = rne_bf16_bits(x - __uint_as_float(hi << 16));
        planes[i] = (uint16_t)hi;
        planes[n + i] = (uint16_t)lo;
    }
}

// The float score a selection key was made from (inverse of select_key's mapping).
__device__ inline float key_score(uint64_t key) {
    const uint32_t o = (uint32_t)(key >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// Eight dims of the group-summed query row: dims e0 .. e0 + 7 of heads h0 .. h0 + GQ - 1.
template <typename KT>
__device__ inline void sum_heads8(const KT* __restrict__ row, int GQ, int e0, float s[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = 0.0f;
    for (int h = 0; h < GQ; ++h) {
        float v[8];
        load8_f32(row + (int64_t)h * kD + e0, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) s[i] += v[i];
    }
}

// hi and lo bf16 fragments of eight fp32 values.
__device__ inline void split_hi_lo8(const float s[8], bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t h0 = rne_bf16_bits(s[2 * i]), h1 = rne_bf16_bits(s[2 * i + 1]);
        const uint32_t l0 = rne_bf16_bits(s[2 * i] - __uint_as_float(h0 << 16));
        const uint32_t l1 = rne_bf16_bits(s[2 * i + 1] - __uint_as_float(h1 << 16));
        h[i] = h0 | (h1 << 16);
        l[i] = l0 | (l1 << 16);
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

// Column tiles of 16 positions per wavefront: 2 (32 positions) measured fastest at 256K keys
// on an MI355X (64 positions: fewer waves fit a CU; 16: each summary tile serves too few).
constexpr int kFlatCols = 2;
constexpr int kFlatPositions = 16 * kFlatCols;

// Cut the lists of the positions in `mask` (bit p: position p of the wavefront) back to their
// K best and set their thresholds; CAP lanes sort one list, 64 / CAP lists per pass.
template <int CAP>
__device__ inline void flat_compact(uint64_t mask, uint64_t* s_buf, uint32_t* s_cnt, float* s_thr, int K) {
    constexpr int PER = 64 / CAP;
    const int lane = threadIdx.x & 63, seg = lane / CAP, slot = lane % CAP;
    while (mask) {
        int p = -1;
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int q = mask ? __builtin_ctzll(mask) : -1;
            if (q >= 0) mask &= mask - 1;
            if (s == seg) p = q;
        }
        const uint32_t cnt = (p >= 0) ? s_cnt[p] : 0u;
        uint64_t key = (p >= 0 && (uint32_t)slot < cnt) ? s_buf[p * CAP + slot] : 0ull;
        key = bitonic_desc<CAP, SegmentLanes>(key, slot);
        if (p >= 0 && slot < K) s_buf[p * CAP + slot] = key;
        if (p >= 0 && slot == K - 1) s_thr[p] = key_score(key);
        if (p >= 0 && slot == 0) s_cnt[p] = (cnt < (uint32_t)K) ? cnt : (uint32_t)K;
    }
}

// One wavefront per workgroup: positions T0 .. T0 + kFlatPositions - 1 of (batch, KV head) bh,
// where the workgroups of the longest causal spans run first.
template <typename KT, int CAP>
__global__ __launch_bounds__(64) void flat_select_kernel(const KT* __restrict__ q,
                                                         const uint16_t* __restrict__ planes, Geom G,
                                                         int32_t* __restrict__ out) {
    static_assert(CAP == 32 || CAP == 64, "a list is sorted by 32 or 64 lanes");
    __shared__ uint64_t s_buf[kFlatPositions * CAP];
    __shared__ uint32_t s_cnt[kFlatPositions];
    __shared__ float s_thr[kFlatPositions];
    const int lane = threadIdx.x & 63, gq = lane >> 4, n = lane & 15;
    const int BH = G.B * G.Hkv;
    const int64_t M1 = G.M[1];
    const int bh = (int)(blockIdx.x % BH);
    const int64_t ngrp = (G.N + kFlatPositions - 1) / kFlatPositions;
    const int64_t grp = ngrp - 1 - (int64_t)(blockIdx.x / BH);
    const int b = bh / G.Hkv, kvh = bh % G.Hkv;
    const int K = G.topk;
    const int64_t T0 = grp * kFlatPositions;
    const int64_t n_elig = (T0 >> 6) + 1;    // blocks 0 .. T0/64, the same for all the wavefront's positions
    const int64_t plane_stride = (int64_t)BH * M1 * kD;
    const uint16_t* pl = planes + (int64_t)bh * M1 * kD;

    // B operand: the group-summed query rows of the wavefront's positions, hi and lo
    bf16x8 qh[kFlatCols][2], ql[kFlatCols][2];
#pragma unroll
    for (int c = 0; c < kFlatCols; ++c) {
        const int64_t p = T0 + 16 * c + n;
        float s0[8], s1[8];
        if (p < G.N) {
            const KT* row = q + (((int64_t)b * G.N + p) * G.Hq + (int64_t)kvh * G.GQ) * kD;
            sum_heads8(row, G.GQ, 8 * gq, s0);
            sum_heads8(row, G.GQ, 32 + 8 * gq, s1);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) s0[i] = s1[i] = 0.0f;
        }
        split_hi_lo8(s0, qh[c][0], ql[c][0]);
        split_hi_lo8(s1, qh[c][1], ql[c][1]);
    }
    if (lane < kFlatPositions) {
        s_cnt[lane] = 0u;
        s_thr[lane] = -INFINITY;
    }
    // each position's threshold in units of the raw product (8 x the score; the 1/8 scale is
    // exact, so comparing products is comparing scores)
    float thr[kFlatCols];
#pragma unroll
    for (int c = 0; c < kFlatCols; ++c) thr[c] = -INFINITY;
    __syncthreads();

    // A operand of block tile bt: row 16 bt + n; rows past the causal bound lie outside the
    // buffer range (read as zero) and are masked in the last tile
    const uint32_t range = (uint32_t)(n_elig * kD * 2);
    const buf_rsrc_t ahi = make_rsrc(pl, range), alo = make_rsrc(pl + plane_stride, range);
    auto load_a = [&](int64_t bt, u32x4 (&a)[4]) {
        const uint32_t off = ((uint32_t)(bt * 16 + n) << 7) + ((uint32_t)gq << 4);
        a[0] = load_b128(ahi, off);
        a[1] = load_b128(ahi, off + 64);
        a[2] = load_b128(alo, off);
        a[3] = load_b128(alo, off + 64);
    };
    const int64_t nbt = (n_elig + 15) / 16;
    u32x4 a_cur[4], a_nxt[4];
    load_a(0, a_cur);
    for (int64_t bt = 0; bt < nbt; ++bt) {
        if (bt + 1 < nbt) load_a(bt + 1, a_nxt);
        const bf16x8 ah0 = __builtin_bit_cast(bf16x8, a_cur[0]), ah1 = __builtin_bit_cast(bf16x8, a_cur[1]);
        const bf16x8 al0 = __builtin_bit_cast(bf16x8, a_cur[2]), al1 = __builtin_bit_cast(bf16x8, a_cur[3]);
        const int64_t blk0 = bt * 16 + 4 * gq;
        const bool last = bt + 1 == nbt;     // wave-uniform: the only tile that can hold blocks past the bound
        f32x4 acc[kFlatCols];
        bool any = false;
#pragma unroll
        for (int c = 0; c < kFlatCols; ++c) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah0, qh[c][0], a, 0, 0, 0);
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah1, qh[c][1], a, 0, 0, 0);
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah0, ql[c][0], a, 0, 0, 0);
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah1, ql[c][1], a, 0, 0, 0);
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al0, qh[c][0], a, 0, 0, 0);
            a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al1, qh[c][1], a, 0, 0, 0);
            if (last) {
#pragma unroll
                for (int r = 0; r < 4; ++r) a[r] = (blk0 + r < n_elig) ? a[r] : -INFINITY;
            }
            acc[c] = a;
            any = any || fmaxf(fmaxf(a[0], a[1]), fmaxf(a[2], a[3])) >= thr[c];
        }
        if (ballot(any)) {
            // append every eligible score at or above its position's threshold
#pragma unroll
            for (int c = 0; c < kFlatCols; ++c) {
                const int p = 16 * c + n;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if (acc[c][r] >= thr[c] && acc[c][r] > -INFINITY) {
                        const uint32_t i = atomicAdd(&s_cnt[p], 1u);
                        s_buf[p * CAP + i] = select_key(acc[c][r] * 0.125f, (int)(blk0 + r));
                    }
                }
            }
            __syncthreads();
            // lists that could overflow on the next tile (16 more entries) are cut back to K
            uint64_t mask = 0;
#pragma unroll
            for (int c = 0; c < kFlatCols; ++c) {
                const uint64_t m = ballot(gq == 0 && s_cnt[16 * c + n] > (uint32_t)(CAP - 16)) & 0xffffull;
                mask |= m << (16 * c);
            }
            if (mask) {
                flat_compact<CAP>(mask, s_buf, s_cnt, s_thr, K);
                __syncthreads();
#pragma unroll
                for (int c = 0; c < kFlatCols; ++c) thr[c] = 8.0f * s_thr[16 * c + n];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) a_cur[i] = a_nxt[i];
    }
    __syncthreads();

    // every list: its K best, then those blocks in ascending order
    constexpr int PER = 64 / CAP;
    const int seg = lane / CAP, slot = lane % CAP;
    for (int p0 = 0; p0 < kFlatPositions; p0 += PER) {
        const int p = p0 + seg;
        const uint32_t cnt = s_cnt[p];
        uint64_t key = ((uint32_t)slot < cnt) ? s_buf[p * CAP + slot] : 0ull;
        key = bitonic_desc<CAP, SegmentLanes>(key, slot);
        const int blk = (slot < K && (uint32_t)slot < cnt) ? key_index(key) : INT_MAX;
        const int sorted = index_sort<CAP, SegmentLanes>(blk, slot);
        const int64_t t = T0 + p;
        if (slot < K && t < G.N)
            out[(((int64_t)b * G.N + t) * G.Hkv + kvh) * K + slot] = (sorted != INT_MAX) ? sorted : -1;
    }
}

template __global__ void flat_select_kernel<uint16_t, 32>(const uint16_t*, const uint16_t*, Geom, int32_t*);
template __global__ void flat_select_kernel<uint16_t, 64>(const uint16_t*, const uint16_t*, Geom, int32_t*);
template __global__ void flat_select_kernel<float, 32>(const float*, const uint16_t*, Geom, int32_t*);
template __global__ void flat_select_kernel<float, 64>(const float*, const uint16_t*, Geom, int32_t*);

// Top K per (position, KV head) of the exact flat scores S (flat_exact_scores_kernel in
// cluster.hip): one wavefront per walk w = (b * N + t) * Hkv + kvh (the output's order), four
// per workgroup. The wavefront keeps the 64 best selection keys (score, then the lower block)
// sorted in descending order over its lanes; the keys of each next 64 eligible blocks are sorted
// ascending and merged in: slot i keeps the larger of kept key i and new key i, which leaves the
// 64 best as a bitonic sequence, and the descending merge (the last stage of a 64-slot sort)
// orders it again. The K best are then listed by block index, -1 padded.
__global__ __launch_bounds__(256) void flat_exact_topk_kernel(const float* __restrict__ S, Geom G,
                                                              int32_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= (int64_t)G.B * G.N * G.Hkv) return;   // wavefront-uniform
    const int kvh = (int)(w % G.Hkv);
    const int64_t bt = w / G.Hkv, b = bt / G.N, t = bt % G.N;
    const int64_t M1 = G.M[1];
    const int64_t n_el = (t / kC + 1 < M1) ? t / kC + 1 : M1;   // blocks 0 .. n_el - 1 are eligible
    const float* row = S + ((b * G.Hkv + kvh) * G.N + t) * M1;
    uint64_t best = 0ull;   // 0: an empty slot, below every key
    for (int64_t L0 = 0; L0 < n_el; L0 += 64) {
        const int64_t L = L0 + lane;
        uint64_t key = (L < n_el) ? select_key(row[L], (int)L) : 0ull;
        key = ~bitonic_desc<64, SegmentLanes>(~key, lane);   // ascending
        best = (best > key) ? best : key;
        key_step<32, 32>(best, lane, 64);
        key_step<16, 16>(best, lane, 64);
        key_step<8, 8>(best, lane, 64);
        key_step<4, 4>(best, lane, 64);
        key_step<2, 2>(best, lane, 64);
        key_step<1, 1>(best, lane, 64);
    }
    const int K = G.topk;
    const int nd = (lane < K && best != 0ull) ? key_index(best) : INT_MAX;
    const int srt = index_sort<64>(nd, lane);
    if (lane < K) out[w * K + lane] = (srt != INT_MAX) ? srt : -1;
}

}  // namespace pisa
