// pyramid.hip -- mean-pooled key pyramid: full build and decode refresh (gfx950).
//
// Reading note "Block Sparse Attention with Log-Linear Complexity", section
// 3.1: leaf summaries are means of C=64 raw keys; each level above merges two
// adjacent nodes by their mean, which equals the mean of all raw keys below.
// A right-edge node covering fewer keys holds the mean of the keys it covers:
// its parent is the count-weighted mean of its children. ai4snews summary,
// second paragraph: a decoding step refreshes only the new token's leaf and the
// leaf's ancestors.
//
// Both paths use the same leaf-sum order (leaf_mean_wave) and the same parent
// formula (parent_mean), so a refreshed pyramid is bitwise equal to a rebuild.
// HBM traffic of the build: one read of the keys (N*Hkv*64 elements) plus one
// fp32 write of every node (about 2*N/64*Hkv*64*4 bytes).
#include "pyramid_math.h"

namespace pisa {

constexpr int kSubLeaves = 16;   // leaves per workgroup subtree (levels 1..5)
constexpr int kSubLevels = 5;

// One workgroup (4 wavefronts) per (batch, KV head, 16-leaf subtree): the 16 leaf
// means, then levels 2..5 of the subtree from LDS. With a pack (pk.cu non-null) the
// workgroups run over (KV head, subtree slot) of the packed layout, a slot naming one
// document's subtree or nothing.
template <typename KT>
__global__ __launch_bounds__(256) void build_subtree_kernel(const KT* __restrict__ k, Geom G, Pack pk,
                                                            float* __restrict__ pyr) {
    __shared__ float s_lv[2][kSubLeaves * kD];
    Seg sg;
    int64_t row0;
    int sub, kvh;
    if (pk.cu) {
        const int64_t nss = (pk.T >> 10) + pk.D + 1;
        kvh = (int)(blockIdx.x / nss);
        const int64_t slot = blockIdx.x % nss;
        const int d = pack_find_slot(pk, 10, slot);
        sg = pack_seg(pk, d);
        const int64_t j = slot - ((sg.lsh >> 10) + d);
        if (sg.N == 0 || j < 0 || j >= (sg.N + kSubLeaves * kC - 1) / (kSubLeaves * kC)) return;
        sub = (int)j;
        row0 = (int64_t)kvh * G.P;
    } else {
        const int nsub = (G.M[1] + kSubLeaves - 1) / kSubLeaves;
        const int bh = blockIdx.x / nsub;          // b * Hkv + kvh
        sub = blockIdx.x % nsub;
        kvh = bh % G.Hkv;
        sg = batch_seg(G.N, (int64_t)(bh / G.Hkv) * G.cap);
        row0 = (int64_t)bh * G.P;
    }
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t row_stride = (int64_t)G.Hkv * kD;
    const KT* kbase = k + (sg.tk0 * G.Hkv + kvh) * kD;
    auto row = [&](int l, int64_t i) -> float* { return pyr + (row0 + G.off[l] + sg.shift(l) + i) * kD; };

    for (int j = 0; j < 4; ++j) {
        const int loc = wave * 4 + j;
        const int64_t leaf = (int64_t)sub * kSubLeaves + loc;
        if (leaf < sg.M(1)) {
            float mean[8];
            leaf_mean_wave<KT>(kbase, row_stride, leaf, sg.N, nullptr, -1, lane, mean);
            if (lane < 8) {
                float* dst = row(1, leaf) + 8 * lane;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    dst[e] = mean[e];
                    s_lv[0][loc * kD + 8 * lane + e] = mean[e];
                }
            }
        }
    }
    __syncthreads();
    int cur = 0;
    for (int l = 2; l <= kSubLevels && l <= sg.L; ++l) {
        const int nloc = kSubLeaves >> (l - 1);
        const int64_t base = (int64_t)sub * nloc;
        for (int idx = tid; idx < nloc * kD; idx += 256) {
            const int loc = idx / kD, e = idx % kD;
            const int64_t node = base + loc;
            if (node < sg.M(l)) {
                const float ca = (float)covered(l - 1, 2 * node, sg.N);
                const float cb = (float)covered(l - 1, 2 * node + 1, sg.N);
                const float a = s_lv[cur][(2 * loc) * kD + e];
                const float bv = (cb > 0.0f) ? s_lv[cur][(2 * loc + 1) * kD + e] : 0.0f;
                const float v = parent_mean(a, ca, bv, cb);
                s_lv[cur ^ 1][loc * kD + e] = v;
                row(l, node)[e] = v;
            }
        }
        __syncthreads();
        cur ^= 1;
    }
}

// Levels 6..L for one (batch, KV head), or with a pack for one (document, KV head): one
// workgroup, level by level. A level of at most kUpperLdsNodes nodes is also kept in LDS
// (two buffers, alternating), so the dependent chain of small levels near the root reads
// its children from LDS instead of memory. Same parent formula and operands either way.
constexpr int kUpperLdsNodes = 128;   // 32 KiB of fp32 rows per buffer
__global__ __launch_bounds__(1024) void build_upper_kernel(Geom G, Pack pk, float* __restrict__ pyr) {
    __shared__ float s_lv[2][kUpperLdsNodes * kD];
    Seg sg;
    int64_t row0;
    if (pk.cu) {
        sg = pack_seg(pk, blockIdx.x / G.Hkv);
        row0 = (int64_t)(blockIdx.x % G.Hkv) * G.P;
        if (sg.N == 0) return;
    } else {
        sg = batch_seg(G.N, 0);
        row0 = (int64_t)blockIdx.x * G.P;
    }
    auto row = [&](int l, int64_t i) -> float* { return pyr + (row0 + G.off[l] + sg.shift(l) + i) * kD; };
    bool in_lds = false;   // level l - 1 is in s_lv[cur]
    int cur = 0;
    for (int l = kSubLevels + 1; l <= sg.L; ++l) {
        const int64_t n = sg.M(l);
        const bool keep = n <= kUpperLdsNodes;   // then every level above fits as well
        for (int64_t idx = threadIdx.x; idx < n * kD; idx += 1024) {
            const int64_t node = idx / kD;
            const int e = (int)(idx % kD);
            const float ca = (float)covered(l - 1, 2 * node, sg.N);
            const float cb = (float)covered(l - 1, 2 * node + 1, sg.N);
            float a, bv;
            if (in_lds) {
                a = s_lv[cur][(2 * node) * kD + e];
                bv = (cb > 0.0f) ? s_lv[cur][(2 * node + 1) * kD + e] : 0.0f;
            } else {
                a = row(l - 1, 2 * node)[e];
                bv = (cb > 0.0f) ? row(l - 1, 2 * node + 1)[e] : 0.0f;
            }
            const float v = parent_mean(a, ca, bv, cb);
            row(l, node)[e] = v;
            if (keep) s_lv[cur ^ 1][idx] = v;
        }
        __syncthreads();   // level l complete (global and LDS) before level l + 1 reads it
        if (keep) {
            in_lds = true;
            cur ^= 1;
        }
    }
}

// Decode refresh for one (batch, KV head): writes k_new as key n (= G.N - 1), recomputes
// the mean of leaf n/64 and then every ancestor of that leaf up to the root of G.
// Decode refresh alone, one wavefront per (batch, KV head): key row N-1 appended,
// its leaf and every ancestor recomputed.
template <typename KT>
__global__ __launch_bounds__(64) void decode_refresh_kernel(const KT* __restrict__ k_new,
                                                            KT* __restrict__ k_cache, Geom G,
                                                            float* __restrict__ pyr) {
    const int bh = blockIdx.x;
    const int b = bh / G.Hkv, kvh = bh % G.Hkv;
    KT* kbase = k_cache + ((int64_t)b * G.cap * G.Hkv + kvh) * kD;
    refresh_wave<KT>(k_new + (int64_t)bh * kD, kbase, (int64_t)G.Hkv * kD, G, pyr + (int64_t)bh * G.P * kD,
                     threadIdx.x);
}

template __global__ void build_subtree_kernel<uint16_t>(const uint16_t*, Geom, Pack, float*);
template __global__ void build_subtree_kernel<float>(const float*, Geom, Pack, float*);
template __global__ void decode_refresh_kernel<uint16_t>(const uint16_t*, uint16_t*, Geom, float*);
template __global__ void decode_refresh_kernel<float>(const float*, float*, Geom, float*);

}  // namespace pisa
