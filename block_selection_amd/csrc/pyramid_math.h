// pyramid_math.h -- leaf means and the decode path refresh, shared by the build,
// refresh and fused decode kernels (gfx950).
//
// Reading note "Block Sparse Attention with Log-Linear Complexity", section
// 3.1: a leaf summary is the mean of its 64 raw keys and a parent merges its
// children by their mean (count-weighted at the ragged right edge, so every
// node holds the mean of the raw keys it covers). ai4snews summary, second
// paragraph: decoding refreshes only the new token's leaf and its ancestors.
#pragma once

#include "pisa_device.h"

namespace pisa {

// Mean of leaf `leaf` over keys [64*leaf, n) for one (batch, KV head), computed by one
// wavefront. Lane = 8*r + c: lane c of each row group owns dims 8c..8c+7; row group r
// sums keys r, r+8, ..., then the 8 row groups are combined by a xor butterfly (all
// lanes end with identical sums). Row `alt_key`, if in range, is read from `alt_row`.
template <typename KT>
__device__ inline void leaf_mean_wave(const KT* kbase, int64_t row_stride, int64_t leaf,
                                      int64_t n, const KT* alt_row, int64_t alt_key,
                                      int lane, float mean[8]) {
    const int r = lane >> 3, c = lane & 7;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    const int64_t k0 = leaf * kC;
    // all eight rows are loaded unconditionally (rows past n read row n-1 and add 0), so
    // the loads are issued together; adding +0 leaves the sums bitwise unchanged
    float v[8][8];
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
        const int64_t key = k0 + rr * 8 + r;
        const int64_t kc = (key < n) ? key : n - 1;
        const KT* row = (kc == alt_key) ? alt_row : kbase + kc * row_stride;
        load8_f32(row + 8 * c, v[rr]);
    }
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
        const bool in = k0 + rr * 8 + r < n;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += in ? v[rr][e] : 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        acc[e] += xor_f(acc[e], 8);
        acc[e] += xor_f(acc[e], 16);
        acc[e] += xor_f(acc[e], 32);
    }
    const int64_t cnt64 = (n - k0 < kC) ? (n - k0) : kC;
    const float cnt = (float)cnt64;
#pragma unroll
    for (int e = 0; e < 8; ++e) mean[e] = __fdiv_rn(acc[e], cnt);
}

__device__ inline float* pyr_row(float* pyr, const Geom& G, int bh, int l, int64_t i) {
    return pyr + ((int64_t)bh * G.P + G.off[l] + i) * kD;
}
__device__ inline const float* pyr_row(const float* pyr, const Geom& G, int bh, int l, int64_t i) {
    return pyr + ((int64_t)bh * G.P + G.off[l] + i) * kD;
}

// Parent levels a refresh can touch: 2 .. kRefreshLevels + 1 (2^31 keys need 26).
constexpr int kRefreshLevels = 31;

// Decode refresh by one wavefront (lane = dimension) for one (batch, KV head): key
// row n = N-1 is written to the cache, leaf n/64 is recomputed over its keys, then
// each ancestor. The path node at every level is the last node of that level, so its
// only possible sibling is on its left, complete and unchanged by this step: all of
// them are loaded in one round before the path is recomputed. Uses the build's leaf
// sum order and parent formula, so the result is bitwise equal to a rebuild.
template <typename KT>
__device__ inline void refresh_wave(const KT* __restrict__ krow_new, KT* __restrict__ kbase, int64_t row_stride,
                                    const Geom& G, float* __restrict__ pyr_bh, int lane) {
    const int64_t n = G.N - 1;
    const int64_t leaf = n >> kLog2C;
    const KT knew = krow_new[lane];
    float sib[kRefreshLevels];   // levels above the root are not read (has = false)
#pragma unroll
    for (int i = 0; i < kRefreshLevels; ++i) {
        const int64_t child = leaf >> i;      // path node at level i + 1
        // unconditional load (row 0 of level 1 where there is no sibling) so all are in flight
        const bool has = i + 2 <= G.L && (child & 1);
        const float v = pyr_bh[(has ? G.off[i + 1] + (child ^ 1) : 0) * kD + lane];
        sib[i] = has ? v : 0.0f;
    }
    kbase[n * row_stride + lane] = knew;
    float mean[8];
    leaf_mean_wave<KT>(kbase, row_stride, leaf, G.N, krow_new, n, lane, mean);
    if (lane < 8) {
        float* dst = pyr_bh + (G.off[1] + leaf) * kD + 8 * lane;
#pragma unroll
        for (int e = 0; e < 8; ++e) dst[e] = mean[e];
    }
    // lane e takes dim e of the leaf mean (held by lanes with c = e/8)
    float own = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float v = shfl_f(mean[e], lane >> 3);
        if ((lane & 7) == e) own = v;
    }
#pragma unroll
    for (int i = 0; i < kRefreshLevels; ++i) {
        const int l = i + 2;
        if (l <= G.L) {
            const int64_t child = leaf >> i;
            const int64_t node = child >> 1;
            if (child & 1) {
                const float ca = (float)covered(l - 1, child - 1, G.N);
                const float cb = (float)covered(l - 1, child, G.N);
                own = parent_mean(sib[i], ca, own, cb);
            } else {
                own = parent_mean(own, (float)covered(l - 1, child, G.N), 0.0f, 0.0f);
            }
            pyr_bh[(G.off[l] + node) * kD + lane] = own;
        }
    }
}

}  // namespace pisa
