// cluster.hip -- clustered leaf-level scoring for prefill (gfx950).
//
// The leaf level is where the walk spends its work: every candidate leaf needs
// the exact LSE over its 64 raw keys for each of the group's query heads
// (reading note "Block Sparse Attention with Log-Linear Complexity", "Scoring:
// LogSumExp" and section 4.1). The pages' prefill kernel clusters queries that
// need the same candidate key block so each loaded block is reused (ai4snews
// summary, second paragraph; reading note section 5.1). Here the cluster is a
// 16-leaf superblock (1024 keys, 128 KiB of bf16 per KV head, held in LDS) and
// its group of walks:
//   1. bucket_pass (count): one incidence per sibling pair of a walk's leaf
//      candidates inside a superblock, counted per bucket (batch, KV head,
//      superblock, range of query positions) in an LDS histogram;
//   2. scan_groups: bucket offsets and work items of at most kItemMax entries
//      of one (batch, KV head, superblock) group;
//   3. bucket_pass (fill): incidences written as entries at their offsets;
//   4. leaf_cluster: persistent workgroups take items from a counter; a workgroup stages the
//      superblock's keys in LDS once, then each wavefront takes entries (the
//      next entry's queries are prefetched while the current one is scored)
//      and scores every leaf of the entry's mask from LDS;
//   5. final_topk: per walk, the K best leaf candidates in ascending order.
// Per incidence the walk's queries (2 KiB) are read once; the keys of a
// superblock are read from memory once per work item.
#include "walk_math.h"

namespace pisa {

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

// Counting (fill = 0) or placing (fill = 1) the incidences of one range of kRangeT
// query positions of batch element blockIdx.y (range blockIdx.x). One incidence per
// sibling pair of a walk's leaf candidates (the children of one level-2 survivor); a
// walk with at most K candidates has none (its candidates are all kept). The workgroup owns the
// buckets (b, kvh, sb, r) of its range: an LDS histogram counts them, and in the fill
// pass the same bins, seeded with the bucket offsets, hand out entry positions.
// Entry = {walk, leaf mask | first slot << 16}: the mask holds the superblock offsets of
// one leaf or of a sibling pair.
template <int SL>
__global__ __launch_bounds__(1024) void bucket_pass_kernel(const int32_t* __restrict__ cand,
                                                          const int32_t* __restrict__ ncand, Geom G,
                                                          ClusterGeom CG, int64_t NT,
                                                          uint32_t* __restrict__ counts,
                                                          const uint32_t* __restrict__ offsets,
                                                          uint2* __restrict__ entries, int fill) {
    extern __shared__ uint32_t bins[];
    constexpr int WPW = 64 / SL;
    const int r = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, seg = lane / SL, i = lane % SL;
    const int K = G.topk, CS = 2 * G.topk;
    const int nbins = G.Hkv * CG.NSB;
    const int nthr = blockDim.x, nw = nthr >> 6;
    // bucket (range r, group g = (b, kvh, sb)) lives at r * ngroups + g
    for (int x = tid; x < nbins; x += nthr) {
        const int64_t bkt = (int64_t)r * CG.ngroups + (int64_t)b * nbins + x;
        bins[x] = fill ? offsets[bkt] : 0u;
    }
    __syncthreads();
    const int64_t t_lo = (int64_t)r * kRangeT;
    const int64_t t_hi = (t_lo + kRangeT < NT) ? t_lo + kRangeT : NT;
    const int64_t w_lo = ((int64_t)b * NT + t_lo) * G.Hkv, w_hi = ((int64_t)b * NT + t_hi) * G.Hkv;
    for (int64_t w0 = w_lo + (int64_t)(tid >> 6) * WPW; w0 < w_hi; w0 += (int64_t)nw * WPW) {
        const int64_t w = w0 + seg;
        const bool ok = w < w_hi;
        const int nc = ok ? ncand[w] : 0;
        const int leaf = (ok && i < CS && i < nc) ? cand[w * CS + i] : -1;
        const int kvh = (int)(w % G.Hkv);
        const int sbv = (leaf >= 0) ? leaf / kSbLeaves : -1;
        // candidates ascend and come as sibling pairs (2c, then 2c+1 if eligible): an entry
        // starts at an even leaf, or at an odd one whose sibling is not a candidate
        const int prv = shfl_i(leaf, lane > 0 ? lane - 1 : 0);
        const int nxt = shfl_i(leaf, lane < 63 ? lane + 1 : lane);
        const bool even = (leaf & 1) == 0;
        const bool start = nc > K && leaf >= 0 && (even || i == 0 || prv != leaf - 1);
        const bool pair = even && i + 1 < SL && nxt == leaf + 1;
        const uint32_t m = (leaf >= 0) ? ((pair ? 3u : 1u) << (leaf % kSbLeaves)) : 0u;
        if (start) {
            const uint32_t pos = atomicAdd(&bins[kvh * CG.NSB + sbv], 1u);
            if (fill) entries[pos] = make_uint2((uint32_t)w, m | ((uint32_t)i << 16));
        }
    }
    __syncthreads();
    if (!fill) {
        for (int x = tid; x < nbins; x += nthr) counts[(int64_t)r * CG.ngroups + (int64_t)b * nbins + x] = bins[x];
    }
}

// One workgroup: entry offsets of every bucket (groups (b, kvh, sb) in order, ranges
// inside a group consecutive) and work items of at most kItemMax entries of one group.
// Items holding kItemMax entries come first, the smaller remainders after them, so
// that the workgroups taking items in order finish together.
// meta[0] = number of items, meta[1] = number of entries, meta[2] = 0 (the counter the
// scoring workgroups take items from).
__global__ __launch_bounds__(1024) void scan_groups_kernel(const uint32_t* __restrict__ counts, ClusterGeom CG,
                                                           uint32_t* __restrict__ offsets,
                                                           int4* __restrict__ items,
                                                           uint32_t* __restrict__ meta) {
    __shared__ uint32_t s_e[1024], s_f[1024], s_p[1024];
    const int tid = threadIdx.x;
    const int per = (CG.ngroups + 1023) / 1024;
    const int lo = tid * per, hi = min(CG.ngroups, lo + per);
    uint32_t se = 0, sf = 0, sp = 0;
    for (int g = lo; g < hi; ++g) {
        uint32_t tot = 0;
        for (int r = 0; r < CG.NR; ++r) tot += counts[(int64_t)r * CG.ngroups + g];
        se += tot;
        sf += tot / kItemMax;              // full items
        sp += (tot % kItemMax) ? 1u : 0u;  // remainder item
    }
    s_e[tid] = se;
    s_f[tid] = sf;
    s_p[tid] = sp;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {       // inclusive Hillis-Steele scans
        const uint32_t ae = (tid >= d) ? s_e[tid - d] : 0u;
        const uint32_t af = (tid >= d) ? s_f[tid - d] : 0u;
        const uint32_t ap = (tid >= d) ? s_p[tid - d] : 0u;
        __syncthreads();
        s_e[tid] += ae;
        s_f[tid] += af;
        s_p[tid] += ap;
        __syncthreads();
    }
    const uint32_t nfull = s_f[1023];
    uint32_t eoff = s_e[tid] - se, foff = s_f[tid] - sf, poff = nfull + s_p[tid] - sp;
    for (int g = lo; g < hi; ++g) {
        const uint32_t g0 = eoff;
        for (int r = 0; r < CG.NR; ++r) {
            offsets[(int64_t)r * CG.ngroups + g] = eoff;
            eoff += counts[(int64_t)r * CG.ngroups + g];
        }
        const uint32_t tot = eoff - g0;
        for (uint32_t p = 0; p * kItemMax < tot; ++p) {
            const uint32_t len = min((uint32_t)kItemMax, tot - p * kItemMax);
            items[(len == kItemMax) ? foff++ : poff++] = make_int4(g, (int)(g0 + p * kItemMax), (int)len, 0);
        }
    }
    if (tid == 1023) {
        meta[0] = nfull + s_p[1023];
        meta[1] = s_e[1023];
        meta[2] = 0u;
    }
}

template __global__ void bucket_pass_kernel<16>(const int32_t*, const int32_t*, Geom, ClusterGeom, int64_t,
                                                uint32_t*, const uint32_t*, uint2*, int);
template __global__ void bucket_pass_kernel<32>(const int32_t*, const int32_t*, Geom, ClusterGeom, int64_t,
                                                uint32_t*, const uint32_t*, uint2*, int);
template __global__ void bucket_pass_kernel<64>(const int32_t*, const int32_t*, Geom, ClusterGeom, int64_t,
                                                uint32_t*, const uint32_t*, uint2*, int);

// LDS image of a superblock: key row r (0..1023) at r*128 bytes, its 16-byte chunk c
// stored at chunk position c ^ (r & 7) so that the MFMA A-fragment reads of 8
// consecutive rows hit distinct banks.
__device__ inline int sb_lds_offset(int r, int chunk) { return r * 128 + ((chunk ^ (r & 7)) << 4); }

// Scores of the leaves of one entry (mask: one leaf, or a sibling pair at bits b, b+1)
// for one walk: lane 0 writes the first leaf's score, lane 16 the second's, every other
// lane stores into the sink, so each entry issues exactly one store instruction (that
// keeps the wait counters exact and the next entries' query prefetches in flight).
// An empty mask (padding entry) scores nothing.
__device__ inline void score_entry(const lds_char_t* lds, int key_base, uint32_t mask, int t,
                                   const bf16x8 q0, const bf16x8 q1, int n, int gq, int lane, int GQ,
                                   float* __restrict__ score_row, float* __restrict__ sink) {
    float v = 0.0f;
    bool two = false;
    if (mask) {
        const int b0 = __builtin_ctz(mask);
        two = (mask >> (b0 + 1)) & 1u;
        const int bits[2] = {b0, two ? b0 + 1 : b0};
        f32x4 acc[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int tau = 0; tau < 4; ++tau) {
                const int r = bits[j] * kC + 16 * tau + n;
                const u32x4 a0 = *reinterpret_cast<const lds_u32x4_t*>(lds + sb_lds_offset(r, gq));
                const u32x4 a1 = *reinterpret_cast<const lds_u32x4_t*>(lds + sb_lds_offset(r, 4 + gq));
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0), q0, c, 0, 0, 0);
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a1), q1, c, 0, 0, 0);
                acc[j][tau] = c;
            }
        const int lim[2] = {min(t - (key_base + bits[0] * kC), kC - 1), min(t - (key_base + bits[1] * kC), kC - 1)};
        v = leaf_lse_pair(acc, lim, n, gq, GQ);
    }
    float* dst = (mask && lane == 0) ? score_row : ((two && lane == 16) ? score_row + 1 : sink + lane);
    *dst = v;
}

// B fragments of one walk's queries: head n of the group, dims {8gq..8gq+7} and
// {32+8gq..32+8gq+7}. Always loads (columns n >= GQ read head 0; their results are
// excluded from the group sum), so the number of loads per entry is fixed.
__device__ inline void load_q(const uint16_t* __restrict__ q, int64_t bt, int Hq, int kvh, int GQ, int n,
                              int gq, u32x4& qa, u32x4& qb) {
    const uint16_t* qrow = q + (bt * Hq + (int64_t)kvh * GQ + (n < GQ ? n : 0)) * kD;
    qa = *reinterpret_cast<const u32x4*>(qrow + 8 * gq);
    qb = *reinterpret_cast<const u32x4*>(qrow + 32 + 8 * gq);
}

__global__ __launch_bounds__(kClusterThreads) void leaf_cluster_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, Geom G, ClusterGeom CG, int64_t NT,
    const int4* __restrict__ items, const uint2* __restrict__ entries, uint32_t* __restrict__ meta,
    float* __restrict__ score, float* __restrict__ sink) {
    static_assert(kItemMax <= 64 * (kClusterThreads / 64), "a wavefront holds its entries in one VGPR pair");
    extern __shared__ u32x4 lds_u4[];
    lds_char_t* lds = (lds_char_t*)lds_u4;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = kClusterThreads / 64;
    const int n = lane & 15, gq = lane >> 4;
    const int CS = 2 * G.topk;
    __shared__ uint32_t s_item;
    const uint32_t n_items = meta[0];
    const int64_t row_stride = (int64_t)G.Hkv * kD;

    // items are taken from a counter, so a workgroup that finishes early takes the next one
    for (;;) {
        __syncthreads();   // the previous item's readers are done with LDS and s_item
        if (threadIdx.x == 0) s_item = atomicAdd(&meta[2], 1u);
        __syncthreads();
        const uint32_t it = s_item;
        if (it >= n_items) break;
        const int4 item = items[it];
        const int grp = item.x;
        const int sb = grp % CG.NSB;
        const int kvh = (grp / CG.NSB) % G.Hkv;
        const int b = grp / (CG.NSB * G.Hkv);
        const int key_base = sb * kSbKeys;
        const uint16_t* kb = k + ((int64_t)b * G.cap * G.Hkv + kvh) * kD;
        // this wavefront's entries item.y + wave + j*nwaves, j < cnt: lane j holds entry j
        const int first = item.y + wave;
        const int cnt = (item.z > wave) ? (item.z - wave + nwaves - 1) / nwaves : 0;
        const uint2 ev = (lane < cnt) ? entries[first + lane * nwaves] : make_uint2(0u, 0u);
        // queries of the first three entries, in flight during the key staging
        u32x4 qa0, qb0, qa1, qb1, qa2, qb2;
        // lanes j >= cnt of ev hold walk 0: prefetches past the end load a valid query row
        auto qload = [&](int j, u32x4& qa, u32x4& qb) {
            const uint32_t w = (uint32_t)__builtin_amdgcn_readlane((int)ev.x, j);
            load_q(q, (int64_t)(w / (uint32_t)G.Hkv), G.Hq, kvh, G.GQ, n, gq, qa, qb);
        };
        qload(0, qa0, qb0);
        qload(1, qa1, qb1);
        qload(2, qa2, qb2);
        for (int idx = tid; idx < kSbKeys * 8; idx += kClusterThreads) {
            const int r = idx >> 3, ch = idx & 7;
            const int key = key_base + r;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (key < G.N) v = *reinterpret_cast<const u32x4*>(kb + (int64_t)key * row_stride + ch * 8);
            *reinterpret_cast<lds_u32x4_t*>(lds + sb_lds_offset(r, ch)) = v;
        }
        __syncthreads();
        // j runs past cnt (up to cnt + 1 <= 65) in the last iteration: such entries get an
        // empty mask, so they score nothing and only store to the sink
        auto process = [&](int j, const u32x4& qa, const u32x4& qb) {
            const int jl = min(j, 63);
            const uint32_t w = (uint32_t)__builtin_amdgcn_readlane((int)ev.x, jl);
            const uint32_t y = (j < cnt) ? (uint32_t)__builtin_amdgcn_readlane((int)ev.y, jl) : 0u;
            const int t = (int)((w / (uint32_t)G.Hkv) % (uint32_t)NT);
            score_entry(lds, key_base, y & 0xffffu, t, __builtin_bit_cast(bf16x8, qa), __builtin_bit_cast(bf16x8, qb),
                        n, gq, lane, G.GQ, score + (int64_t)w * CS + (y >> 16), sink + wave * 64);
        };
        // steady state: a fixed sequence of memory operations per iteration (one store per
        // entry, two loads per prefetch), so wait counts stay exact across iterations
        for (int j = 0; j < cnt; j += 3) {
            process(j, qa0, qb0);
            qload(min(j + 3, 63), qa0, qb0);
            process(j + 1, qa1, qb1);
            qload(min(j + 4, 63), qa1, qb1);
            process(j + 2, qa2, qb2);
            qload(min(j + 5, 63), qa2, qb2);
        }
    }
}

// Per walk (SLOTS lanes each): at most K candidates are all kept; otherwise the K best
// by (score desc, index asc). Written in ascending leaf order, -1 padded.
template <int SLOTS>
__global__ __launch_bounds__(256) void final_topk_kernel(const int32_t* __restrict__ cand,
                                                         const int32_t* __restrict__ ncand,
                                                         const float* __restrict__ score, Geom G,
                                                         int64_t NT, int32_t* __restrict__ out) {
    constexpr int WPW = 64 / SLOTS;
    const int K = G.topk, CS = 2 * G.topk;
    const int lane = threadIdx.x & 63, seg = lane / SLOTS, i = lane % SLOTS;
    const int64_t walks = (int64_t)G.B * NT * G.Hkv;
    const int64_t groups = (walks + WPW - 1) / WPW;
    for (int64_t grp = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); grp < groups; grp += (int64_t)gridDim.x * 4) {
        const int64_t w = grp * WPW + seg;
        const bool ok = w < walks;
        const int nc = ok ? ncand[w] : 0;
        const int c = (ok && i < CS) ? cand[w * CS + i] : -1;
        float s = -INFINITY;
        if (c >= 0) s = (nc > K) ? score[w * CS + i] : 0.0f;
        const int nd = select_sort<SLOTS>(s, (c >= 0) ? c : INT_MAX, i);
        const int nd2 = index_sort<SLOTS>((i < K) ? nd : INT_MAX, i);
        if (ok && i < K) out[w * K + i] = (nd2 != INT_MAX) ? nd2 : -1;
    }
}

template __global__ void final_topk_kernel<16>(const int32_t*, const int32_t*, const float*, Geom, int64_t, int32_t*);
template __global__ void final_topk_kernel<32>(const int32_t*, const int32_t*, const float*, Geom, int64_t, int32_t*);
template __global__ void final_topk_kernel<64>(const int32_t*, const int32_t*, const float*, Geom, int64_t, int32_t*);

}  // namespace pisa
