// cluster.hip -- clustered leaf-level scoring for prefill (gfx950).
//
// The leaf level is where the walk spends its work: every candidate leaf needs
// the exact LSE over its 64 raw keys for each of the group's query heads
// (reading note "Block Sparse Attention with Log-Linear Complexity", "Scoring:
// LogSumExp" and section 4.1). The pages' prefill kernel clusters queries that
// need the same candidate key block so each loaded block is reused (ai4snews
// summary, second paragraph; reading note section 5.1). Here the cluster is a
// sibling pair of leaves (128 keys, 16 KiB of bf16 per KV head, held in one
// wavefront's registers) and the walks that score it:
//   1. bucket_pass (count): one incidence per sibling pair of a walk's leaf
//      candidates, counted per bucket (batch, KV head, pair, range of query
//      positions) in an LDS histogram;
//   2. plan_groups: per (batch, KV head, pair) group, the scan of its ranges'
//      counts (bucket offsets inside the group, group total), its place in the
//      entry array and its work items of at most L entries;
//   3. bucket_pass (fill): incidences written as entries at their offsets;
//   4. leaf_cluster: persistent wavefronts, each on its own, take items from
//      counters; a wavefront loads the item's pair of leaves into registers as
//      MFMA A fragments once, then scores the item's entries two walks at a time
//      (the queries of the next two such units are in flight while one is
//      scored, across the whole item);
//   5. final_topk: per walk, the K best leaf candidates in ascending order.
// Per incidence the walk's queries (2 KiB) are read once; the keys of a pair are
// read from memory once per work item.
#include <type_traits>

#include "walk_math.h"

namespace pisa {

// Counting (fill = 0) or placing (fill = 1) the incidences of one range of 2^RL
// query positions of batch element blockIdx.y (range blockIdx.x). One incidence per
// sibling pair of a walk's leaf candidates (the children of one level-2 survivor); a
// walk with at most K candidates has none (its candidates are all kept). The workgroup owns the
// buckets (b, kvh, pair, r) of its range: an LDS histogram counts them, and in the fill
// pass the same bins, seeded with the bucket offsets, hand out entry positions.
// Entry = {query position t, leaf mask | first slot << 16}: the mask holds the pair
// offsets of one leaf or of a sibling pair (batch element and KV head are the bucket's).
// Counts and offsets are range-major per sequence: bucket (range r, bin x) of batch element
// b at (b * NR + r) * nbins + x, so that a workgroup reads and writes one contiguous row;
// the fill pass starts bucket (r, x) at gbase[g] + offsets[...] (g: the bin's group). The
// bins live in LDS kBinSlice at a time (a sequence with more groups is counted slice by
// slice). The count pass also clears the counters in meta that the later kernels use.
// With a pack (pk.cu non-null) blockIdx.x is a range slot of the packed layout: range j of
// one document d (or nothing), positions t count from the document's start, and the
// workgroup's bins are the document's own groups, x = kvh * nsb_d + s (pair s of the
// document is pair slot (cu[d] >> 7) + d + s, group kvh * CG.NGP + that slot). Its counts
// sit in the document's block at cbase[d] + j * nbins_d + x.
template <int SL>
__global__ __launch_bounds__(1024) void bucket_pass_kernel(const int32_t* __restrict__ cand,
                                                          const int32_t* __restrict__ ncand, Geom G,
                                                          ClusterGeom CG, Pack pk, const int64_t* __restrict__ cbase,
                                                          int64_t NT, uint32_t* __restrict__ counts,
                                                          const uint32_t* __restrict__ offsets,
                                                          const uint32_t* __restrict__ gbase,
                                                          uint2* __restrict__ entries, uint32_t* __restrict__ meta,
                                                          int fill) {
    extern __shared__ uint32_t bins[];
    // the count pass clears the counters of the plan and of the leaf stage (before any exit)
    if (!fill && blockIdx.x == 0 && blockIdx.y == 0) {
        for (int i = threadIdx.x; i < kMetaWords; i += blockDim.x) meta[i] = 0u;
    }
    constexpr int WPW = 64 / SL;
    const int r = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, seg = lane / SL, i = lane % SL;
    const int K = G.topk, CS = 2 * G.topk;
    const int nthr = blockDim.x, nw = nthr >> 6;
    int64_t bt0, t_lo, t_hi;   // first query row of the sequence, positions [t_lo, t_hi)
    int nsb;                   // pair groups per KV head in the bins: x = kvh * nsb + s
    int64_t g_sb0, c0;         // bin x -> group (x / nsb) * CG.NGP + g_sb0 + x % nsb; count c0 + x
    if (pk.cu) {
        const int d = pack_find_slot(pk, CG.RL, r);
        const Seg sg = pack_seg(pk, d);
        const int64_t j = r - ((sg.lsh >> CG.RL) + d);
        const int64_t nr = sg.N ? ((sg.N - 1) >> CG.RL) + 1 : 0;
        if (sg.N == 0 || j < 0 || j >= nr) return;   // no positions, no buckets
        bt0 = sg.lsh;
        t_lo = j << CG.RL;
        t_hi = (t_lo + (1 << CG.RL) < sg.N) ? t_lo + (1 << CG.RL) : sg.N;
        nsb = (int)((sg.N + kGrpKeys - 1) / kGrpKeys);
        g_sb0 = (sg.lsh >> (kLog2GrpKeys)) + d;
        c0 = cbase[d] + j * (int64_t)(G.Hkv * nsb);
    } else {
        const int b = blockIdx.y;
        bt0 = (int64_t)b * NT;
        t_lo = (int64_t)r << CG.RL;
        t_hi = (t_lo + (1 << CG.RL) < NT) ? t_lo + (1 << CG.RL) : NT;
        nsb = CG.NGP;
        g_sb0 = (int64_t)b * G.Hkv * CG.NGP;
        c0 = ((int64_t)b * CG.NR + r) * (G.Hkv * CG.NGP);
    }
    // the bins are held in LDS kBinSlice at a time; a longer sequence's range is read once per slice
    const int nbins = G.Hkv * nsb;
    for (int x0 = 0; x0 < nbins; x0 += kBinSlice) {
    const int nx = min(kBinSlice, nbins - x0);
    if (x0) __syncthreads();   // the previous slice's counts are written out
    for (int x = tid; x < nx; x += nthr) {
        const int64_t g = (int64_t)((x0 + x) / nsb) * CG.NGP + g_sb0 + (x0 + x) % nsb;
        bins[x] = fill ? gbase[g] + offsets[c0 + x0 + x] : 0u;
    }
    __syncthreads();
    const int64_t w_lo = (bt0 + t_lo) * G.Hkv, w_hi = (bt0 + t_hi) * G.Hkv;
    // kBucketUnroll rounds of walks per loop trip, their loads issued together
    const int64_t step = (int64_t)nw * WPW;
    for (int64_t w0 = w_lo + (int64_t)(tid >> 6) * WPW; w0 < w_hi; w0 += kBucketUnroll * step) {
        int nc[kBucketUnroll], leafv[kBucketUnroll];
#pragma unroll
        for (int u = 0; u < kBucketUnroll; ++u) {
            const int64_t w = w0 + u * step + seg;
            const bool ok = w < w_hi;
            nc[u] = ok ? ncand[w] : 0;
            leafv[u] = (ok && i < CS) ? cand[w * CS + i] : -1;
        }
#pragma unroll
        for (int u = 0; u < kBucketUnroll; ++u) {
            const int64_t w = w0 + u * step + seg;
            const int leaf = (i < nc[u]) ? leafv[u] : -1;
            const int kvh = (int)(w % G.Hkv);
            const int sbv = (leaf >= 0) ? leaf / kGrpLeaves : -1;
            // candidates ascend and come as sibling pairs (2c, then 2c+1 if eligible): an entry
            // starts at an even leaf, or at an odd one whose sibling is not a candidate
            const int prv = shfl_i(leaf, lane > 0 ? lane - 1 : 0);
            const int nxt = shfl_i(leaf, lane < 63 ? lane + 1 : lane);
            const bool even = (leaf & 1) == 0;
            const bool start = nc[u] > K && leaf >= 0 && (even || i == 0 || prv != leaf - 1);
            const bool pair = even && i + 1 < SL && nxt == leaf + 1;
            const uint32_t m = (leaf >= 0) ? ((pair ? 3u : 1u) << (leaf % kGrpLeaves)) : 0u;
            const int bx = kvh * nsb + sbv - x0;
            if (start && bx >= 0 && bx < nx) {
                const uint32_t pos = atomicAdd(&bins[bx], 1u);
                if (fill) entries[pos] = make_uint2((uint32_t)(w / G.Hkv - bt0), m | ((uint32_t)i << 16));
            }
        }
    }
    __syncthreads();
    if (!fill) {
        for (int x = tid; x < nx; x += nthr) counts[c0 + x0 + x] = bins[x];
    }
    }
}

// Pack plan (one workgroup): cbase[d] = first count of document d's block (KV heads x its
// pairs x its ranges), an exclusive scan over the documents, cbase[D] = the total; and
// cbase[D + 1 + d] = the first 64-bin chunk of document d in the flat chunk space of the
// plan, cbase[2D + 1] = the number of chunks.
__global__ __launch_bounds__(1024) void pack_plan_kernel(Pack pk, int Hkv, int RL, int64_t* __restrict__ cbase) {
    __shared__ int64_t s_sum[1024], s_chk[1024];
    const int tid = threadIdx.x;
    const int per = (pk.D + 1023) / 1024;
    const int lo = tid * per, hi = min(pk.D, lo + per);
    auto size_of = [&](int d) -> int64_t {
        const Seg sg = pack_seg(pk, d);
        return sg.N ? (int64_t)Hkv * ((sg.N + kGrpKeys - 1) / kGrpKeys) * (((sg.N - 1) >> RL) + 1) : 0;
    };
    auto chunks_of = [&](int d) -> int64_t {
        const Seg sg = pack_seg(pk, d);
        return sg.N ? ((int64_t)Hkv * ((sg.N + kGrpKeys - 1) / kGrpKeys) + 63) / 64 : 0;
    };
    int64_t acc = 0, acc_c = 0;
    for (int d = lo; d < hi; ++d) {
        acc += size_of(d);
        acc_c += chunks_of(d);
    }
    s_sum[tid] = acc;
    s_chk[tid] = acc_c;
    __syncthreads();
    for (int st = 1; st < 1024; st <<= 1) {   // inclusive Hillis-Steele scans
        const int64_t add = (tid >= st) ? s_sum[tid - st] : 0;
        const int64_t add_c = (tid >= st) ? s_chk[tid - st] : 0;
        __syncthreads();
        s_sum[tid] += add;
        s_chk[tid] += add_c;
        __syncthreads();
    }
    int64_t run = s_sum[tid] - acc, run_c = s_chk[tid] - acc_c;
    for (int d = lo; d < hi; ++d) {
        cbase[d] = run;
        run += size_of(d);
        cbase[pk.D + 1 + d] = run_c;
        run_c += chunks_of(d);
    }
    if (tid == 1023) {
        cbase[pk.D] = s_sum[1023];
        cbase[2 * pk.D + 1] = s_chk[1023];
    }
}

// Plan of the leaf stage: a work unit is 64 consecutive bins x (groups) of one sequence (a
// batch element, or a document of a pack), one workgroup (4 wavefronts) per unit, the grid
// striding over the units. For each group: the exclusive scan
// of its ranges' counts (the offset of each bucket inside the group; wavefront w scans a
// quarter of the ranges), its total, its first entry gbase (wavefront 0 places its 64
// groups with one atomic on the entry counter), and its work items of at most L entries:
// the full ones at the front of the item array (from position meta[kMetaFront]), the
// remainder at the back (position item_cap - 1 - k, k from meta[kMetaBack]), so that the
// wavefronts taking items in order score the small remainders last.
__global__ __launch_bounds__(64 * kPlanWaves) void plan_groups_kernel(const uint32_t* __restrict__ counts, Geom G, ClusterGeom CG,
                                                          Pack pk, const int64_t* __restrict__ cbase, uint32_t L,
                                                          uint32_t item_cap, uint32_t* __restrict__ offsets,
                                                          uint32_t* __restrict__ gbase, int4* __restrict__ items,
                                                          uint32_t* __restrict__ meta) {
    __shared__ uint32_t s_part[kPlanWaves][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // work units: (sequence, chunk of 64 bins); a batch element has nchunks of them, a
    // document of a pack its own number (the flat chunk space of the pack plan)
    const int nchunks = (int)((G.Hkv * (int64_t)CG.NGP + 63) / 64);
    const int64_t nunits = pk.cu ? cbase[2 * pk.D + 1] : (int64_t)G.B * nchunks;
    for (int64_t unit = blockIdx.x; unit < nunits; unit += gridDim.x) {   // workgroup-uniform
        int nsb, nr, chunk;
        int64_t cb, g_sb0;   // the sequence's first count; bin x -> group (x / nsb) * CG.NGP + g_sb0 + x % nsb
        if (pk.cu) {
            const int64_t* cpre = cbase + pk.D + 1;
            int lo = 0, hi = pk.D - 1;   // the last document whose first chunk is <= unit
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (cpre[mid] <= unit) lo = mid;
                else hi = mid - 1;
            }
            const int q = lo;
            const Seg sg = pack_seg(pk, q);
            chunk = (int)(unit - cpre[q]);
            nsb = (int)((sg.N + kGrpKeys - 1) / kGrpKeys);
            nr = (int)(((sg.N - 1) >> CG.RL) + 1);
            cb = cbase[q];
            g_sb0 = (sg.lsh >> kLog2GrpKeys) + q;
        } else {
            const int q = (int)(unit / nchunks);
            chunk = (int)(unit % nchunks);
            nsb = CG.NGP;
            nr = CG.NR;
            cb = (int64_t)q * CG.NR * (G.Hkv * CG.NGP);
            g_sb0 = (int64_t)q * G.Hkv * CG.NGP;
        }
        const int nbins = G.Hkv * nsb;
        const int x = chunk * 64 + lane;
        const bool ok = x < nbins;
        const int r0 = (int)((int64_t)nr * wave / kPlanWaves), r1 = (int)((int64_t)nr * (wave + 1) / kPlanWaves);
        uint32_t part = 0;
        if (ok) {
            for (int r = r0; r < r1; ++r) part += counts[cb + (int64_t)r * nbins + x];
        }
        s_part[wave][lane] = part;
        __syncthreads();
        uint32_t run = 0, tot = 0;
#pragma unroll
        for (int w = 0; w < kPlanWaves; ++w) {
            const uint32_t pw = s_part[w][lane];
            run += (w < wave) ? pw : 0u;
            tot += pw;
        }
        __syncthreads();   // s_part is read by every wavefront before the next sequence writes it
        if (ok) {
            for (int r = r0; r < r1; ++r) {
                const int64_t c = cb + (int64_t)r * nbins + x;
                const uint32_t v = counts[c];
                offsets[c] = run;
                run += v;
            }
        }
        if (wave == 0) {
            // place the 64 groups' entries and items
            const uint32_t te = ok ? tot : 0u;
            const uint32_t nf = te / L, np = (te % L) ? 1u : 0u;
            uint32_t ie = te, i_f = nf, ip = np;   // inclusive scans over the wavefront
#pragma unroll
            for (int dd = 1; dd < 64; dd <<= 1) {
                const int src = lane >= dd ? lane - dd : lane;
                const uint32_t ye = (uint32_t)shfl_i((int)ie, src), yf = (uint32_t)shfl_i((int)i_f, src);
                const uint32_t yp = (uint32_t)shfl_i((int)ip, src);
                ie += (lane >= dd) ? ye : 0u;
                i_f += (lane >= dd) ? yf : 0u;
                ip += (lane >= dd) ? yp : 0u;
            }
            // the wavefront totals are read with every lane active (a cross-lane read inside the
            // lane-0 branch below would see lane 63 as it was before the branch)
            const uint32_t te_w = (uint32_t)__builtin_amdgcn_readlane((int)ie, 63);
            const uint32_t nf_w = (uint32_t)__builtin_amdgcn_readlane((int)i_f, 63);
            const uint32_t np_w = (uint32_t)__builtin_amdgcn_readlane((int)ip, 63);
            uint32_t eb = 0u, fb = 0u, pb = 0u;
            if (lane == 0) {
                eb = atomicAdd(&meta[kMetaEntries], te_w);
                fb = atomicAdd(&meta[kMetaFront], nf_w);
                pb = atomicAdd(&meta[kMetaBack], np_w);
            }
            eb = (uint32_t)__builtin_amdgcn_readlane((int)eb, 0);
            fb = (uint32_t)__builtin_amdgcn_readlane((int)fb, 0);
            pb = (uint32_t)__builtin_amdgcn_readlane((int)pb, 0);
            if (ok) {
                const int64_t g = (int64_t)(x / nsb) * CG.NGP + g_sb0 + x % nsb;
                const uint32_t g0 = eb + ie - te;
                gbase[g] = g0;
                const uint32_t f0 = fb + i_f - nf;
                for (uint32_t k = 0; k < nf; ++k) items[f0 + k] = make_int4((int)g, (int)(g0 + k * L), (int)L, 0);
                if (np)
                    items[item_cap - 1u - (pb + ip - np)] = make_int4((int)g, (int)(g0 + nf * L), (int)(te - nf * L), 0);
            }
        }
    }
}

template __global__ void bucket_pass_kernel<16>(const int32_t*, const int32_t*, Geom, ClusterGeom, Pack, const int64_t*, int64_t,
                                                uint32_t*, const uint32_t*, const uint32_t*, uint2*, uint32_t*, int);
template __global__ void bucket_pass_kernel<32>(const int32_t*, const int32_t*, Geom, ClusterGeom, Pack, const int64_t*, int64_t,
                                                uint32_t*, const uint32_t*, const uint32_t*, uint2*, uint32_t*, int);
template __global__ void bucket_pass_kernel<64>(const int32_t*, const int32_t*, Geom, ClusterGeom, Pack, const int64_t*, int64_t,
                                                uint32_t*, const uint32_t*, const uint32_t*, uint2*, uint32_t*, int);

// Key fragments of one sibling pair, held in registers for a whole work item: f[j][tau][h]
// is the MFMA A operand of leaf j's 16-key tile tau in lane (gq, n): key 16 tau + n of the
// leaf, dims 8 gq .. 8 gq + 7 (h = 0) or 32 + 8 gq .. 32 + 8 gq + 7 (h = 1). Keys at or
// past the sequence's end are zero.
struct PairKeys {
    u32x4 f[2][4][2];
};

__device__ inline void load_pair_keys(const uint16_t* __restrict__ kb, int64_t row_stride, int64_t key0,
                                      int64_t nkeys, int n, int gq, PairKeys& K) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
#pragma unroll
        for (int tau = 0; tau < 4; ++tau) {
            const int64_t key = key0 + j * kC + 16 * tau + n;
            u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
            if (key < nkeys) {
                const uint16_t* row = kb + key * row_stride;
                a = *reinterpret_cast<const u32x4*>(row + 8 * gq);
                b = *reinterpret_cast<const u32x4*>(row + 32 + 8 * gq);
            }
            K.f[j][tau][0] = a;
            K.f[j][tau][1] = b;
        }
    }
}

// MFMA logits of leaf J of the pair for one walk's query fragments: acc[tau] in lane
// (gq, n) holds keys 16 tau + 4 gq + r of head n.
template <int J>
__device__ inline void leaf_logits(const PairKeys& K, const bf16x8 q0, const bf16x8 q1, f32x4 acc[4]) {
#pragma unroll
    for (int tau = 0; tau < 4; ++tau) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, K.f[J][tau][0]), q0, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, K.f[J][tau][1]), q1, c, 0, 0, 0);
        acc[tau] = c;
    }
}

// This lane's exp sums of the four (walk, leaf) combinations of a unit (see score_unit),
// in row order r = (walk r >> 1, leaf r & 1), over the pair's eight 16-key tiles (leaf j,
// tile tau). Per tile each walk's four terms are added as (e0 + e1) + (e2 + e3), and the
// four tiles of a leaf as (t0 + t1) + (t2 + t3): the balanced-tree order of leaf_exp_sum.
// Without a second walk (kTwo false) walk b's rows repeat walk a's sums.
template <bool kFull, bool kTwo>
__device__ inline void unit_exp_sums(const PairKeys& K, const int (&lim)[4], const bf16x8 qa0, const bf16x8 qa1,
                                     const bf16x8 qb0, const bf16x8 qb1, int gq, float (&sum)[4]) {
    auto tile_sum = [&](const f32x4& c, int tau, int lm) -> float {
        float e[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float e2 = __builtin_amdgcn_exp2f(c[k] * kScale2);
            e[k] = (kFull || 16 * tau + 4 * gq + k <= lm) ? e2 : 0.0f;
        }
        return (e[0] + e[1]) + (e[2] + e[3]);
    };
    float ta[4], tb[4];
#pragma unroll
    for (int st = 0; st < 8; ++st) {
        const int j = st >> 2, tau = st & 3;
        const bf16x8 f0 = __builtin_bit_cast(bf16x8, K.f[j][tau][0]);
        const bf16x8 f1 = __builtin_bit_cast(bf16x8, K.f[j][tau][1]);
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f0, qa0, c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f1, qa1, c, 0, 0, 0);
        ta[tau] = tile_sum(c, tau, lim[j]);
        if (kTwo) {
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f0, qb0, d, 0, 0, 0);
            d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f1, qb1, d, 0, 0, 0);
            tb[tau] = tile_sum(d, tau, lim[2 + j]);
        }
        if (tau == 3) {
            sum[j] = (ta[0] + ta[1]) + (ta[2] + ta[3]);
            sum[2 + j] = kTwo ? (tb[0] + tb[1]) + (tb[2] + tb[3]) : sum[j];
        }
    }
}

// Scores of a unit: two walks a and b (b may repeat a) against both leaves of the pair.
// Each key fragment is used for both walks. The four (walk, leaf) sums are reduced in one
// vector; returns, in lanes of row group r, the score of (walk r >> 1, leaf r & 1),
// bitwise what leaf_lse_from_acc gives for the leaf alone. lim[] are per (walk, leaf) in
// that row order; an ineligible leaf (lim < 0) is computed with one key and its score
// discarded by the caller. two = false: the unit has walk a only (b repeats a), whose
// second copy is not computed.
__device__ inline float score_unit(const PairKeys& K, const int (&lim_in)[4], const bf16x8 qa0, const bf16x8 qa1,
                                   const bf16x8 qb0, const bf16x8 qb1, int n, int gq, int GQ, bool two) {
    int lim[4];
    bool full = true;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        lim[r] = max(lim_in[r], 0);
        full = full && lim[r] == kC - 1;
    }
    // one branch per unit: a unit with no masked key (the common case) runs straight-line code
    float sum[4];
    if (full && two)
        unit_exp_sums<true, true>(K, lim, qa0, qa1, qb0, qb1, gq, sum);
    else if (full)
        unit_exp_sums<true, false>(K, lim, qa0, qa1, qb0, qb1, gq, sum);
    else if (two)
        unit_exp_sums<false, true>(K, lim, qa0, qa1, qb0, qb1, gq, sum);
    else
        unit_exp_sums<false, false>(K, lim, qa0, qa1, qb0, qb1, gq, sum);
    // column totals of the four sums in one vector: row r = (walk r >> 1, leaf r & 1)
    const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(sum[0]), __float_as_uint(sum[1]), false, false);
    const float Sa = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(sum[2]), __float_as_uint(sum[3]), false, false);
    const float Sb = __uint_as_float(y[0]) + __uint_as_float(y[1]);
    const auto z = __builtin_amdgcn_permlane32_swap(__float_as_uint(Sa), __float_as_uint(Sb), false, false);
    float T = __uint_as_float(z[0]) + __uint_as_float(z[1]);
    float shift = 0.0f;
    const uint64_t bad = ballot(!(T < INFINITY && T > 0x1p-100f));
    if (bad) {
        // rare: the (walk, leaf) of a bad row group again, shifted by each column's maximum logit
        auto redo = [&](auto r_const, const bf16x8 q0, const bf16x8 q1) {
            constexpr int r = decltype(r_const)::value;
            if (bad & (0xffffull << (16 * r))) {
                f32x4 acc[4];
                leaf_logits<r & 1>(K, q0, q1, acc);
                const float moff = cols4_max(leaf_lane_max(acc, lim[r], gq)) * kScale2;
                const float v = leaf_exp_sum<false>(acc, lim[r], gq, moff);
                const float sr = cols4_sum(v);
                if (gq == r) {
                    T = sr;
                    shift = moff;
                }
            }
        };
        redo(std::integral_constant<int, 0>{}, qa0, qa1);
        redo(std::integral_constant<int, 1>{}, qa0, qa1);
        redo(std::integral_constant<int, 2>{}, qb0, qb1);
        redo(std::integral_constant<int, 3>{}, qb0, qb1);
    }
    const float lse2 = shift + __builtin_amdgcn_logf(T);
    return row16_sum((n < GQ) ? lse2 : 0.0f);
}

// Truncated scores of a unit (the layout and result convention of score_unit): the
// moments of the four (walk, leaf) combinations, each key fragment used for both walks
// (walk b skipped when two is false), reduced over the row groups in one packed exchange
// per moment (the order of cols4_sum), then mean (+ var/2) per head and the group sum: the
// bits leaf_trunc_from_acc gives for each leaf alone.
template <int S>
__device__ inline float score_unit_trunc(const PairKeys& K, const int (&lim_in)[4], const bf16x8 qa0,
                                         const bf16x8 qa1, const bf16x8 qb0, const bf16x8 qb1, int n, int gq, int GQ,
                                         bool two) {
    int lim[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lim[r] = max(lim_in[r], 0);
    float s1[4], s2[4];
    auto leaf = [&](auto j_const) {
        constexpr int j = decltype(j_const)::value;
        f32x4 acca[4], accb[4];
        leaf_logits<j>(K, qa0, qa1, acca);
        if (two) leaf_logits<j>(K, qb0, qb1, accb);
        if (lim[j] == kC - 1) leaf_moments<true>(acca, lim[j], gq, s1[j], s2[j]);
        else leaf_moments<false>(acca, lim[j], gq, s1[j], s2[j]);
        if (two) {
            if (lim[2 + j] == kC - 1) leaf_moments<true>(accb, lim[2 + j], gq, s1[2 + j], s2[2 + j]);
            else leaf_moments<false>(accb, lim[2 + j], gq, s1[2 + j], s2[2 + j]);
        } else {
            s1[2 + j] = s1[j];
            s2[2 + j] = s2[j];
        }
    };
    leaf(std::integral_constant<int, 0>{});
    leaf(std::integral_constant<int, 1>{});
    // column totals of the four combinations: row group r = (walk r >> 1, leaf r & 1)
    auto pack = [](const float (&v)[4]) -> float {
        const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[0]), __float_as_uint(v[1]), false, false);
        const float a = __uint_as_float(x[0]) + __uint_as_float(x[1]);
        const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[2]), __float_as_uint(v[3]), false, false);
        const float b = __uint_as_float(y[0]) + __uint_as_float(y[1]);
        const auto z = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        return __uint_as_float(z[0]) + __uint_as_float(z[1]);
    };
    const float T1 = pack(s1), T2 = pack(s2);
    const int my_lim = (gq == 0) ? lim[0] : (gq == 1) ? lim[1] : (gq == 2) ? lim[2] : lim[3];
    const float v = trunc_score2<S>(T1, T2, my_lim + 1);
    return row16_sum((n < GQ) ? v : 0.0f);
}

// B fragments of one walk's queries: head n of the group, dims {8gq..8gq+7} and
// {32+8gq..32+8gq+7}. Always loads (columns n >= GQ read head 0; their results are
// excluded from the group sum), so the number of loads per unit is fixed.
__device__ inline void load_q(const uint16_t* __restrict__ q, int64_t bt, int Hq, int kvh, int GQ, int n,
                              int gq, u32x4& qa, u32x4& qb) {
    const uint16_t* qrow = q + (bt * Hq + (int64_t)kvh * GQ + (n < GQ ? n : 0)) * kD;
    qa = *reinterpret_cast<const u32x4*>(qrow + 8 * gq);
    qb = *reinterpret_cast<const u32x4*>(qrow + 32 + 8 * gq);
}

// Persistent wavefronts, each on its own: a wavefront takes a work item from the counters,
// loads the item's sibling pair of leaves (128 keys) into registers as MFMA A fragments,
// and scores the item's entries two at a time (a unit: two walks, both leaves), the next
// two units' queries in flight while one is scored. No LDS and no barrier.
template <int S, bool kOneEach>
__device__ inline void leaf_cluster_body(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const Geom& G,
                                         const ClusterGeom& CG, const Pack& pk, int64_t NT,
                                         const int4* __restrict__ items, uint32_t item_cap,
                                         const uint2* __restrict__ entries, uint32_t* __restrict__ meta,
                                         float* __restrict__ score, float* __restrict__ sink) {
    // a unit is two walks (one walk per unit at four wavefronts per SIMD measured slower)
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, gq = lane >> 4;
    const int CS = 2 * G.topk;
    // items 0 .. n_front - 1 at the front of the array, then the remainders from its back
    const uint32_t n_front = meta[kMetaFront];
    const uint32_t n_items = n_front + meta[kMetaBack];
    const int64_t row_stride = (int64_t)G.Hkv * kD;
    float* const wsink = sink + wave * 64 + lane;

    // Items come in kItemStreams interleaved streams (stream s: items s, s + S, s + 2S, ...),
    // each with its own counter on its own 256-byte line, so that the atomics spread over S
    // addresses; a wavefront starts on its workgroup's stream and moves to the next one when
    // that is exhausted. kOneEach (chosen for short calls, which have about as many items as
    // wavefronts): wavefront w first takes item w without an atomic, and the streams then
    // hand out the items past the wavefront count. The ticket for a wavefront's next item is
    // taken when an item starts and read when it ends, so its round trip overlaps the scoring.
    const int s0 = (int)(blockIdx.x % kItemStreams);
    const uint32_t skip = kOneEach ? gridDim.x * (kLeafThreads / 64) : 0u;
    constexpr uint32_t kNone = 0xffffffffu;
    int si = 0;
    auto ticket = [&]() -> uint32_t {   // lane 0: a ticket of the current stream
        uint32_t got = 0u;
        if (lane == 0) got = atomicAdd(meta + kItemCounter0 + kItemCounterStride * ((s0 + si) % kItemStreams), 1u);
        return got;
    };
    auto resolve = [&](uint32_t got) -> uint32_t {   // the item of a ticket, else the next stream's
        for (;;) {
            const uint32_t it = skip + (uint32_t)__builtin_amdgcn_readlane((int)got, 0) * kItemStreams +
                                (uint32_t)((s0 + si) % kItemStreams);
            if (it < n_items) return it;
            if (++si == kItemStreams) return kNone;
            got = ticket();
        }
    };
    uint32_t it;
    if (kOneEach) {
        it = blockIdx.x * (kLeafThreads / 64) + wave;
        if (it >= n_items) return;
    } else {
        it = resolve(ticket());
    }
    while (it != kNone) {
        const int4 item = items[it < n_front ? it : item_cap - 1u - (it - n_front)];
        const int grp = item.x;
        const int gs = grp % CG.NGP;
        const int kvh = (grp / CG.NGP) % G.Hkv;
        // the group's sequence: its first query row, first key row and key count
        int64_t bt0, tk0, nkeys;
        int pg;
        if (pk.cu) {
            const int d = pack_find_slot(pk, kLog2GrpKeys, gs);
            const Seg sg = pack_seg(pk, d);
            pg = gs - (int)((sg.lsh >> kLog2GrpKeys) + d);
            bt0 = sg.lsh;
            tk0 = sg.tk0;
            nkeys = sg.N;
        } else {
            const int b = grp / (CG.NGP * G.Hkv);
            pg = gs;
            bt0 = (int64_t)b * NT;
            tk0 = (int64_t)b * G.cap;
            nkeys = G.N;
        }
        const int key0 = pg * kGrpKeys;
        PairKeys K;
        load_pair_keys(k + (tk0 * G.Hkv + kvh) * kD, row_stride, key0, nkeys, n, gq, K);
        // lane u holds unit u of the item (its entries 2u and 2u + 1; an item of kItemMax = 128
        // entries is 64 units): walk a's (position, slot word) in x, y and walk b's in z, w. A
        // unit without a second entry repeats walk a's position with a zero slot word; lanes past
        // the item hold zeros (position 0, a valid row, and no slot).
        static_assert(kItemMax == 2 * 64, "one unit per lane");
        const int m = item.z;
        const int nunits = (m + 1) >> 1;
        uint4 ev = make_uint4(0u, 0u, 0u, 0u);
        if (2 * lane < m) {
            const uint2 ea = entries[item.y + 2 * lane];
            const uint2 eb = (2 * lane + 1 < m) ? entries[item.y + 2 * lane + 1] : make_uint2(ea.x, 0u);
            ev = make_uint4(ea.x, ea.y, eb.x, eb.y);
        }
        const uint32_t next = ticket();
        // queries of unit u (u <= 63)
        auto qload = [&](int u, u32x4& a0, u32x4& a1, u32x4& b0, u32x4& b1) {
            const uint32_t ta = (uint32_t)__builtin_amdgcn_readlane((int)ev.x, u);
            const uint32_t tb = (uint32_t)__builtin_amdgcn_readlane((int)ev.z, u);
            load_q(q, bt0 + ta, G.Hq, kvh, G.GQ, n, gq, a0, a1);
            load_q(q, bt0 + tb, G.Hq, kvh, G.GQ, n, gq, b0, b1);
        };
        // one store instruction per unit: lanes 0 / 16 write walk a's two leaves, lanes 32 / 48
        // walk b's, every other lane (and every lane of a unit past the item) writes the sink
        auto process = [&](int u, const u32x4& a0, const u32x4& a1, const u32x4& b0, const u32x4& b1) {
            const bool real = u < nunits;
            const int lu = min(u, 63);
            const uint32_t tua = (uint32_t)__builtin_amdgcn_readlane((int)ev.x, lu);
            const uint32_t ya = real ? (uint32_t)__builtin_amdgcn_readlane((int)ev.y, lu) : 0u;
            const uint32_t tbr = (uint32_t)__builtin_amdgcn_readlane((int)ev.z, lu);
            const uint32_t yb = real ? (uint32_t)__builtin_amdgcn_readlane((int)ev.w, lu) : 0u;
            const uint32_t ma = ya & 3u, mb = yb & 3u;
            const uint32_t tub = mb ? tbr : tua;
            const int64_t wa = (bt0 + tua) * G.Hkv + kvh, wb = (bt0 + tub) * G.Hkv + kvh;
            float v = 0.0f;
            if (ma) {
                const int ta = (int)tua, tb = (int)tub;
                const int lim[4] = {min(ta - key0, kC - 1), min(ta - key0 - kC, kC - 1), min(tb - key0, kC - 1),
                                    min(tb - key0 - kC, kC - 1)};
                const bf16x8 fa0 = __builtin_bit_cast(bf16x8, a0), fa1 = __builtin_bit_cast(bf16x8, a1);
                const bf16x8 fb0 = __builtin_bit_cast(bf16x8, b0), fb1 = __builtin_bit_cast(bf16x8, b1);
                if constexpr (S == kScoreLse)
                    v = score_unit(K, lim, fa0, fa1, fb0, fb1, n, gq, G.GQ, mb != 0u);
                else
                    v = score_unit_trunc<S>(K, lim, fa0, fa1, fb0, fb1, n, gq, G.GQ, mb != 0u);
            }
            float* dst = wsink;
            if (lane == 0 && (ma & 1u)) dst = score + wa * CS + (ya >> 16);
            if (lane == 16 && (ma & 2u)) dst = score + wa * CS + (ya >> 16) + (ma & 1u);
            if (lane == 32 && (mb & 1u)) dst = score + wb * CS + (yb >> 16);
            if (lane == 48 && (mb & 2u)) dst = score + wb * CS + (yb >> 16) + (mb & 1u);
            *dst = v;
        };
        // the queries of the next two units are in flight while a unit is scored, over the
        // whole item; the steady state is a fixed sequence of memory operations per iteration
        // (one store per unit, four loads per prefetch), so wait counts stay exact across
        // iterations
        u32x4 qa0, qa1, qb0, qb1, ra0, ra1, rb0, rb1, sa0, sa1, sb0, sb1;
        qload(0, qa0, qa1, qb0, qb1);
        qload(1, ra0, ra1, rb0, rb1);
        qload(2, sa0, sa1, sb0, sb1);
        for (int u = 0; u < nunits; u += 3) {
            process(u, qa0, qa1, qb0, qb1);
            qload(min(u + 3, 63), qa0, qa1, qb0, qb1);
            process(u + 1, ra0, ra1, rb0, rb1);
            qload(min(u + 4, 63), ra0, ra1, rb0, rb1);
            process(u + 2, sa0, sa1, sb0, sb1);
            qload(min(u + 5, 63), sa0, sa1, sb0, sb1);
        }
        it = resolve(next);
    }
}

template <int S, bool kOneEach>
__global__ __launch_bounds__(kLeafThreads) void leaf_cluster_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, Geom G, ClusterGeom CG, Pack pk, int64_t NT,
    const int4* __restrict__ items, uint32_t item_cap, const uint2* __restrict__ entries,
    uint32_t* __restrict__ meta, float* __restrict__ score, float* __restrict__ sink) {
    leaf_cluster_body<S, kOneEach>(q, k, G, CG, pk, NT, items, item_cap, entries, meta, score, sink);
}
// The LSE kernel of long calls: held to three wavefronts per SIMD (166 VGPRs, no spill);
// the others take the occupancy their registers give.
template <>
__global__ __launch_bounds__(kLeafThreads) __attribute__((amdgpu_waves_per_eu(3))) void
leaf_cluster_kernel<kScoreLse, false>(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, Geom G,
                                      ClusterGeom CG, Pack pk, int64_t NT, const int4* __restrict__ items,
                                      uint32_t item_cap, const uint2* __restrict__ entries,
                                      uint32_t* __restrict__ meta, float* __restrict__ score,
                                      float* __restrict__ sink) {
    leaf_cluster_body<kScoreLse, false>(q, k, G, CG, pk, NT, items, item_cap, entries, meta, score, sink);
}

#define PISA_LEAF_CLUSTER_INST(S, O)                                                                      \
    template __global__ void leaf_cluster_kernel<S, O>(const uint16_t*, const uint16_t*, Geom, ClusterGeom, Pack, \
                                                       int64_t, const int4*, uint32_t, const uint2*, uint32_t*, float*, \
                                                       float*);
PISA_LEAF_CLUSTER_INST(kScoreMean, false)
PISA_LEAF_CLUSTER_INST(kScoreMeanHalfVar, false)
PISA_LEAF_CLUSTER_INST(kScoreLse, true)
PISA_LEAF_CLUSTER_INST(kScoreMean, true)
PISA_LEAF_CLUSTER_INST(kScoreMeanHalfVar, true)
#undef PISA_LEAF_CLUSTER_INST

// Per walk (SLOTS lanes each): at most K candidates are all kept; otherwise the K best
// by (score desc, index asc). Written in ascending leaf order, -1 padded. A wavefront
// takes kTopkBatch groups of walks per trip (grid stride) and issues all their loads
// before it selects, so one memory round trip serves several groups.
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
    const int64_t stride = (int64_t)gridDim.x * 4;
    for (int64_t g0 = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); g0 < groups; g0 += stride * kTopkBatch) {
        int nc[kTopkBatch], c[kTopkBatch];
        float sv[kTopkBatch];
#pragma unroll
        for (int j = 0; j < kTopkBatch; ++j) {
            const int64_t w = (g0 + j * stride) * WPW + seg;
            const bool ok = g0 + j * stride < groups && w < walks;
            nc[j] = ok ? ncand[w] : 0;
            c[j] = (ok && i < CS) ? cand[w * CS + i] : -1;
            sv[j] = (ok && i < CS) ? score[w * CS + i] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kTopkBatch; ++j) {
            if (g0 + j * stride >= groups) break;   // wavefront-uniform
            const int64_t w = (g0 + j * stride) * WPW + seg;
            float s = -INFINITY;
            if (c[j] >= 0) s = (nc[j] > K) ? sv[j] : 0.0f;
            const int cidx = (c[j] >= 0) ? c[j] : INT_MAX;
            const int nd = (2 * K == SLOTS) ? select_top_half<SLOTS>(s, cidx, i) : select_sort<SLOTS>(s, cidx, i);
            // the K kept indices sit in slots below K <= SLOTS / 2: sort the first half of the slots
            const int nd2 = index_sort<SLOTS / 2>((i < K) ? nd : INT_MAX, i % (SLOTS / 2));
            if (w < walks && i < K) out[w * K + i] = (nd2 != INT_MAX) ? nd2 : -1;
        }
    }
}

template __global__ void final_topk_kernel<16>(const int32_t*, const int32_t*, const float*, Geom, int64_t, int32_t*);
template __global__ void final_topk_kernel<32>(const int32_t*, const int32_t*, const float*, Geom, int64_t, int32_t*);
template __global__ void final_topk_kernel<64>(const int32_t*, const int32_t*, const float*, Geom, int64_t, int32_t*);

// Exact flat scores (pisa_select_flat_exact): S[(bh * N + t) * M1 + L] = the score the walk
// gives leaf L as a candidate of position t (score_unit: the group sum of the base-2 LSE over
// the leaf's raw keys up to t) for every eligible (t, L), i.e. L * 64 <= t; other entries are
// not written. The work is the lower triangle of (128-position chunk c, sibling pair p <= c)
// tiles, the pairs with a leaf eligible for some position of the chunk: tile c (c + 1) / 2 + p.
// One wavefront per tile, four per workgroup, grid (ceil(tiles / 4), B * Hkv): the wavefront
// holds the pair's keys in registers and scores the chunk's positions two at a time (a unit),
// the next unit's queries in flight while one is scored.
__global__ __launch_bounds__(256) void flat_exact_scores_kernel(const uint16_t* __restrict__ q,
                                                                const uint16_t* __restrict__ k, Geom G,
                                                                float* __restrict__ S) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, gq = lane >> 4;
    const int64_t N = G.N, M1 = G.M[1];
    const int64_t chunks = (N + kGrpKeys - 1) / kGrpKeys;
    const int64_t tile = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (tile >= chunks * (chunks + 1) / 2) return;   // wavefront-uniform
    int64_t c = (int64_t)((sqrt(8.0 * (double)tile + 1.0) - 1.0) * 0.5);
    while (c > 0 && c * (c + 1) / 2 > tile) --c;
    while ((c + 1) * (c + 2) / 2 <= tile) ++c;
    const int64_t p = tile - c * (c + 1) / 2;
    const int bh = blockIdx.y, b = bh / G.Hkv, kvh = bh % G.Hkv;
    const int64_t row_stride = (int64_t)G.Hkv * kD;
    const uint16_t* kb = k + ((int64_t)b * G.cap * G.Hkv + kvh) * kD;
    const int64_t qrow0 = (int64_t)b * N;   // query row of position 0 of batch element b
    float* Sb = S + (int64_t)bh * N * M1;
    // this lane's row group gq reports (position gq >> 1 of the unit, leaf gq & 1 of the pair)
    const int my_walk = gq >> 1, my_leaf = gq & 1;
    PairKeys K;
    load_pair_keys(kb, row_stride, p * kGrpKeys, N, n, gq, K);
    const int64_t t0 = c * kGrpKeys;
    const int64_t rest = N - t0;
    const int nu = (int)(rest >= kGrpKeys ? kGrpKeys / 2 : (rest + 1) / 2);
    auto unit_pos = [&](int u, int64_t& ta, int64_t& tb) {
        ta = t0 + 2 * u;
        tb = (ta + 1 < N) ? ta + 1 : ta;   // a unit of one position repeats it
    };
    u32x4 a0, a1, b0, b1;
    {
        int64_t ta, tb;
        unit_pos(0, ta, tb);
        load_q(q, qrow0 + ta, G.Hq, kvh, G.GQ, n, gq, a0, a1);
        load_q(q, qrow0 + tb, G.Hq, kvh, G.GQ, n, gq, b0, b1);
    }
    for (int u = 0; u < nu; ++u) {
        int64_t ta, tb;
        unit_pos(u, ta, tb);
        const bool two = tb != ta;
        u32x4 na0 = a0, na1 = a1, nb0 = b0, nb1 = b1;
        if (u + 1 < nu) {
            int64_t tan, tbn;
            unit_pos(u + 1, tan, tbn);
            load_q(q, qrow0 + tan, G.Hq, kvh, G.GQ, n, gq, na0, na1);
            load_q(q, qrow0 + tbn, G.Hq, kvh, G.GQ, n, gq, nb0, nb1);
        }
        int lim[4];   // per (walk r >> 1, leaf r & 1): the leaf's keys up to t are 0 .. lim
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t rel = ((r >> 1) ? tb : ta) - (2 * p + (r & 1)) * kC;
            lim[r] = rel < 0 ? -1 : (rel > kC - 1 ? kC - 1 : (int)rel);
        }
        const float sc = score_unit(K, lim, __builtin_bit_cast(bf16x8, a0), __builtin_bit_cast(bf16x8, a1),
                                    __builtin_bit_cast(bf16x8, b0), __builtin_bit_cast(bf16x8, b1), n, gq, G.GQ,
                                    two);
        const int64_t t = my_walk ? tb : ta, L = 2 * p + my_leaf;
        if (n == 0 && (two || my_walk == 0) && L < M1 && L * kC <= t) Sb[t * M1 + L] = sc;
        a0 = na0;
        a1 = na1;
        b0 = nb0;
        b1 = nb1;
    }
}

}  // namespace pisa
